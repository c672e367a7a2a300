"""Seeded synthetic workloads for Split-KV draft cross-attention.

This module only draws inputs: anchor positions, sequence lengths, context
chunk tables and N(0,1) tensors rounded to the storage dtype.  It holds none of
the method's arithmetic (no mask, no softmax, no cost model, no planner), so
both the fp64 oracle tests and the GPU path can consume the same arrays.

Workload shapes follow the pages' statement of the regime: a short draft-query
set (anchor blocks of 16 draft tokens) against a much longer context
("Split-KV: Efficient Context Parallelism for Training Diffusion Drafters",
abstract; rit.work blog, section on why a short query suffices for a long
context).  Real drafter training data is not available; these seeded inputs
stand in for it.

Seeds: ``numpy.random.default_rng(seed)`` draws the geometry (sequence
lengths, then anchors); each tensor comes from its own stream
``default_rng([seed, tag])`` and each context chunk of K and V from
``default_rng([seed, tag, chunk])``, so a shard can draw only its own rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK = 16  # draft tokens per anchor block


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    dtype: str                      # "f32" or "bf16"
    n_seq: int                      # packed sequences
    blocks_per_seq: int
    chunk: int                      # KV chunk length (unit of placement)
    tile_k: int = 64                # key tile of the cost model
    # single-sequence fields
    ctx: int = 0
    anchor_lo: int = 0
    anchor_hi: int = 0
    # varlen fields
    len_median: int = 0
    len_sigma: float = 1.0
    len_min: int = 0
    len_max: int = 0
    beta_a: float = 5.0
    beta_b: float = 1.0
    n_shards: int = 1               # simulated context-parallel ranks
    n_bins: int = 256               # CU bins for the in-GPU plan

    @property
    def nb(self) -> int:
        return self.n_seq * self.blocks_per_seq

    @property
    def nq(self) -> int:
        return self.nb * BLOCK


WORKLOADS = {
    # Tiny fp32 forward: 1K context, 4 anchor blocks, 2 heads, d=64, 8 chunks
    # of 128 over 4 simulated shards.
    "tiny_f32_ctx1k": Workload(
        name="tiny_f32_ctx1k", hq=2, hkv=2, d=64, dtype="f32", n_seq=1,
        blocks_per_seq=4, chunk=128, ctx=1024, anchor_lo=256, anchor_hi=1024,
        n_shards=4),
    # bf16 forward (+ backward on the same shapes): 32K context, 2048 draft
    # queries, GQA 32q/8kv, d=128, KV chunks of 256, 256 CU bins.
    "ctx32k_q2k": Workload(
        name="ctx32k_q2k", hq=32, hkv=8, d=128, dtype="bf16", n_seq=1,
        blocks_per_seq=128, chunk=256, ctx=32768, anchor_lo=8192,
        anchor_hi=32768),
    # One rank's share of a 64-way context-parallel split of a 512K context
    # with 4096 draft queries; chunks of 512.
    "cp64_rank0_ctx512k": Workload(
        name="cp64_rank0_ctx512k", hq=32, hkv=8, d=128, dtype="bf16",
        n_seq=1, blocks_per_seq=256, chunk=512, ctx=524288,
        anchor_lo=131072, anchor_hi=524288, n_shards=64),
    # Varlen fwd+bwd: 8 packed sequences, lognormal lengths (median 16K,
    # clipped to [4K, 64K]), 64 blocks per sequence, anchors skewed late.
    "varlen8_fwdbwd": Workload(
        name="varlen8_fwdbwd", hq=16, hkv=4, d=128, dtype="bf16", n_seq=8,
        blocks_per_seq=64, chunk=256, len_median=16384, len_sigma=1.0,
        len_min=4096, len_max=65536),
    # 1M-context stress: 8192 draft queries, 4096 chunks of 256, 64 shards,
    # 64-way merge.
    "ctx1m_merge64": Workload(
        name="ctx1m_merge64", hq=32, hkv=8, d=128, dtype="bf16", n_seq=1,
        blocks_per_seq=512, chunk=256, ctx=1048576, anchor_lo=262144,
        anchor_hi=1048576, n_shards=64),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 value (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are exactly representable in bf16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass
class Geometry:
    """Anchor blocks and the packed context they attend to."""
    seq_start: np.ndarray   # int64 [n_seq]
    seq_len: np.ndarray     # int64 [n_seq]
    anchors: np.ndarray     # int32 [nb]: exclusive bound of visible context
    lo: np.ndarray          # int32 [nb]: first visible context key
    ctx: int                # total packed context length
    chunk_pos: np.ndarray   # int32 [n_chunks] absolute first key
    chunk_len: np.ndarray   # int32 [n_chunks]


def draw_geometry(w: Workload, rng: np.random.Generator) -> Geometry:
    if w.n_seq == 1 and w.ctx:
        lens = np.array([w.ctx], np.int64)
    else:
        z = rng.standard_normal(w.n_seq)
        lens = np.rint(w.len_median * np.exp(w.len_sigma * z)).astype(np.int64)
        lens = np.clip(lens, w.len_min, w.len_max)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    anchors, lo = [], []
    for s in range(w.n_seq):
        if w.ctx:
            a = rng.choice(w.anchor_hi - w.anchor_lo, size=w.blocks_per_seq,
                           replace=False) + w.anchor_lo
        else:
            x = rng.beta(w.beta_a, w.beta_b, size=w.blocks_per_seq)
            a = np.floor(lens[s] * x).astype(np.int64)
            a = np.clip(a, 0, lens[s] - 1)
        a = np.sort(a) + starts[s]
        anchors.append(a)
        lo.append(np.full(w.blocks_per_seq, starts[s], np.int64))
    anchors = np.concatenate(anchors).astype(np.int32)
    lo = np.concatenate(lo).astype(np.int32)
    # Chunking restarts at every sequence start; the last chunk is ragged.
    cpos, clen = [], []
    for s in range(w.n_seq):
        for off in range(0, int(lens[s]), w.chunk):
            cpos.append(starts[s] + off)
            clen.append(min(w.chunk, int(lens[s]) - off))
    return Geometry(seq_start=starts, seq_len=lens, anchors=anchors, lo=lo,
                    ctx=int(lens.sum()),
                    chunk_pos=np.array(cpos, np.int32),
                    chunk_len=np.array(clen, np.int32))


def draw_normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) fp32 draw rounded to the storage dtype (kept as fp32 values)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(x) if dtype == "bf16" else x


# Stream tags: every tensor (and every context chunk of K and V) has its own
# counter-free numpy stream, so any subset of chunks can be drawn alone.
_TAG = {"Q": 0x51, "K": 0x4B, "V": 0x56, "Kd": 0x4B44, "Vd": 0x5644, "dO": 0x644F}


def _rng(seed: int, tag: str, *extra: int) -> np.random.Generator:
    return np.random.default_rng([seed, _TAG[tag], *extra])


@dataclasses.dataclass
class Tensors:
    Q: np.ndarray            # [Nq, Hq, d]
    K: np.ndarray            # [n_local, Hkv, d]: rows of the drawn chunks
    V: np.ndarray            # [n_local, Hkv, d]
    Kd: np.ndarray           # [Nq, Hkv, d] draft-block keys
    Vd: np.ndarray           # [Nq, Hkv, d]
    dO: Optional[np.ndarray]  # [Nq, Hq, d]
    chunk_ids: np.ndarray    # chunks whose rows K/V hold, in order


def draw_kv_chunks(w: Workload, g: Geometry, seed: int, chunk_ids, tag: str) -> np.ndarray:
    parts = [draw_normal(_rng(seed, tag, int(c)), (int(g.chunk_len[c]), w.hkv, w.d), w.dtype)
             for c in chunk_ids]
    if not parts:
        return np.zeros((0, w.hkv, w.d), np.float32)
    return np.concatenate(parts, axis=0)


def draw_tensors(w: Workload, g: Geometry, seed: int, with_grad: bool = False,
                 chunk_ids=None) -> Tensors:
    """Q, Kd, Vd (and dO) for all draft queries; K, V for the given chunks
    (default: every chunk, i.e. the whole packed context in order)."""
    if chunk_ids is None:
        chunk_ids = np.arange(len(g.chunk_pos))
    chunk_ids = np.asarray(chunk_ids, np.int64)
    Q = draw_normal(_rng(seed, "Q"), (w.nq, w.hq, w.d), w.dtype)
    K = draw_kv_chunks(w, g, seed, chunk_ids, "K")
    V = draw_kv_chunks(w, g, seed, chunk_ids, "V")
    Kd = draw_normal(_rng(seed, "Kd"), (w.nq, w.hkv, w.d), w.dtype)
    Vd = draw_normal(_rng(seed, "Vd"), (w.nq, w.hkv, w.d), w.dtype)
    dO = draw_normal(_rng(seed, "dO"), (w.nq, w.hq, w.d), w.dtype) if with_grad else None
    return Tensors(Q, K, V, Kd, Vd, dO, chunk_ids)


def make(name_or_w, seed: int, with_grad: bool = False, tensors: bool = True,
         chunk_ids=None):
    """Geometry (+ tensors) of a named workload for a given seed."""
    w = WORKLOADS[name_or_w] if isinstance(name_or_w, str) else name_or_w
    g = draw_geometry(w, np.random.default_rng(seed))
    t = draw_tensors(w, g, seed, with_grad, chunk_ids) if tensors else None
    return w, g, t


def scaled(w: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller test sizes)."""
    return dataclasses.replace(w, **over)


def softmax_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
