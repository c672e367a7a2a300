/*
 * libsplitkv — Split-KV draft cross-attention on one AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * The method (arXiv abstract of "Split-KV: Efficient Context Parallelism for
 * Training Diffusion Drafters"; rit.work blog post on Split-KV, sections
 * "A short query sufficed for a long context" and "Split-KV moves queries,
 * not keys and values"):
 *   - a short set of draft queries, built in blocks of 16 tokens around
 *     anchor positions sampled in the responses, attends to a much longer
 *     context through a block-sparse mask;
 *   - context keys/values stay on the participant that holds them; every
 *     participant sees the full query set, computes the attention of all
 *     queries over its local keys, and the per-participant results are
 *     combined exactly by reconciling the softmax normaliser;
 *   - the cost of each context chunk is known before the step, and chunks
 *     are placed longest-processing-time-first (LPT) on the least-loaded
 *     participant.
 *
 * Mask (the reading this library implements): anchor block i (draft query
 * rows 16i .. 16i+15) sees the context keys at absolute positions
 * lo[i] <= j < anchors[i] and the 16 draft keys of its own block (rows
 * 16i .. 16i+15 of Kd/Vd) in both directions.  Query head h reads kv head
 * h / (hq / hkv).
 *
 * Conventions
 *   - Every call returns an skv_status; SKV_OK is 0, errors are negative.
 *     skv_last_error() returns a description of the last failure on the
 *     calling thread.  No call aborts the process.
 *   - Device pointers are HIP device addresses.  The caller owns every
 *     buffer; the library allocates no device memory.  Scratch space is the
 *     caller's `workspace` of the size the schedule reports, except for
 *     skv_attn_fwd_partial_noalloc, whose scratch is a static array of the
 *     library's code object.
 *   - Device calls are asynchronous on the caller's stream (`stream` is a
 *     hipStream_t passed as void*; NULL is the default stream).  Launch
 *     errors are returned as SKV_ERR_HIP.  Host calls are synchronous.
 *   - Tensors are dense, row-major, 16-byte aligned (LSE arrays: 4-byte;
 *     the workspace: 16-byte).  A misaligned pointer is refused with
 *     SKV_ERR_INVALID_ARG before anything is launched:
 *       Q, O, dO, dQ   [Nq, hq, d]       (Nq = 16 * nb, token-major)
 *       LSE            [Nq, hq]          fp32, natural log
 *       K, V, dK, dV   [n_local, hkv, d] (local key rows of the shard)
 *       Kd, Vd, dKd... [Nq, hkv, d]      (draft-block keys/values)
 *   - dtypes: SKV_BF16 (bfloat16) or SKV_F32.  d is 64 or 128.  hq must be
 *     a multiple of hkv with hq / hkv in {1, 2, 4, 8, 16}.
 *   - The library keeps no state across calls except per-device caches of
 *     the compute-unit count and of the static scratch array's address; it is
 *     safe to call from several threads (skv_attn_fwd_partial_noalloc: see
 *     there).
 */
#ifndef SPLITKV_H
#define SPLITKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_ERR_INVALID_ARG = -1,   /* bad pointer, size, layout or value */
  SKV_ERR_UNSUPPORTED = -2,   /* valid but not implemented (d, dtype, G) */
  SKV_ERR_HIP = -3,           /* a HIP runtime call or launch failed */
  SKV_ERR_WORKSPACE = -4,     /* workspace or schedule buffer too small */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

/* Last error text on this thread ("" after a successful call). */
const char* skv_last_error(void);

/* ABI version of this header (bumped on incompatible changes; 2: four
 * words per workgroup in the clock-stamp buffer, skv_plan_lpt_split and
 * skv_dq_finalize added; 3: per-XCD queues, skv_schedule_info.xcd_mode,
 * clock stamps indexed by queue, skv_schedule_build_xcd added; 4: schedule
 * image version 3 (dQ sections of its own in xcd_mode) and the
 * skv_schedule_info.n_dq_* / dq_cost_* fields). */
int32_t skv_abi_version(void);
#define SKV_ABI_VERSION 4

/* ------------------------------------------------------------------------
 * Planner (host only, synchronous, deterministic).
 * ---------------------------------------------------------------------- */

/* Realised cost of each context chunk (arXiv abstract: chunks are balanced
 * by their realised attention cost, computable in advance from the global
 * query view; rit.work blog, section "Split-KV moves queries, not keys and
 * values").  Chunk c covers absolute keys [chunk_pos[c], chunk_pos[c] +
 * chunk_len[c]) and is cut into key tiles of tile_k keys from its first key
 * (the last tile may be short).  cost[c] counts the (anchor block, key tile)
 * pairs where the tile holds at least one key in [lo[i], anchors[i]).
 *   anchors, lo: host int32 [nb];  chunk_pos, chunk_len: host int32
 *   [n_chunks], chunk_len >= 1;  tile_k >= 1;  out_cost: host int64
 *   [n_chunks].  Errors: SKV_ERR_INVALID_ARG on NULL or bad sizes. */
skv_status skv_chunk_costs(const int32_t* anchors, const int32_t* lo,
                           int32_t nb, const int32_t* chunk_pos,
                           const int32_t* chunk_len, int32_t n_chunks,
                           int32_t tile_k, int64_t* out_cost);

/* LPT placement of n jobs with costs cost[n] >= 0 on n_bins bins (same
 * sources as above: most expensive first, each to the least-loaded bin).
 * Ties: equal costs in increasing job index, equal loads to the lowest bin.
 *   out_bin: host int32 [n];  out_load: host int64 [n_bins] or NULL.
 *   n may be 0.  Errors: SKV_ERR_INVALID_ARG on NULL, n_bins < 1 or a
 *   negative cost. */
skv_status skv_plan_lpt_costs(const int64_t* cost, int32_t n, int32_t n_bins,
                              int32_t* out_bin, int64_t* out_load);

/* skv_chunk_costs followed by skv_plan_lpt_costs: the chunk -> bin plan of
 * a context-parallel split (bins = participants) or of chunks over compute
 * units.  out_cost [n_chunks] and out_load [n_bins] may be NULL. */
skv_status skv_plan_lpt(const int32_t* anchors, const int32_t* lo, int32_t nb,
                        const int32_t* chunk_pos, const int32_t* chunk_len,
                        int32_t n_chunks, int32_t tile_k, int32_t n_bins,
                        int32_t* out_bin, int64_t* out_cost,
                        int64_t* out_load);

/* LPT with splitting: the placement the work schedule below uses for the
 * forward / dQ items of each XCD class (exported for tests and tools).
 * Same sources as above, plus the exact merge of partials (rit.work blog,
 * section "Split-KV moves queries, not keys and values"), which makes a
 * unit of work divisible.  Unit u is steps[u] >= 0 equal steps; a piece
 * [k0, k1) of it costs item_cost + step_cost * (k1 - k0), plus extra[u] on
 * the unit's first piece (k0 == 0).  Pending pieces are taken largest cost
 * first (ties: lower unit, then lower k0), each to the least-loaded bin
 * (ties: lower bin).  A piece that would lift that bin above `target` is
 * cut after the longest step prefix that fits when it has >= 2 steps and
 * the bin has room for its fixed part plus one step; the remainder returns
 * to the pending set and pays item_cost again.  Otherwise the bin takes
 * the piece whole.  A cut leaves its bin within one step of target, so no
 * bin is cut twice and there are at most n_units + n_bins pieces.
 *   target: 0 = chosen as the schedule does (ceil(total / n_bins), then
 *   reset to the mean load a pass produced plus item_cost / 2 until it
 *   repeats, at most four passes); INT64_MAX = never cut (plain LPT of the
 *   units, as skv_plan_lpt_costs).
 *   out_pieces: host int32 [capacity][4] = (unit, k0, k1, bin) in
 *   placement order; out_cost: host int64 [capacity]; *out_n: pieces;
 *   *out_target (may be NULL): the target used; out_load: host int64
 *   [n_bins] or NULL.  Costs are in the caller's units.
 * Errors: SKV_ERR_INVALID_ARG (NULL, negative values, total cost above
 * 2^60), SKV_ERR_WORKSPACE (capacity below *out_n, which is still set). */
skv_status skv_plan_lpt_split(const int64_t* extra, const int32_t* steps,
                              int32_t n_units, int64_t item_cost,
                              int64_t step_cost, int32_t n_bins,
                              int64_t target, int32_t capacity,
                              int32_t* out_pieces, int64_t* out_cost,
                              int32_t* out_n, int64_t* out_target,
                              int64_t* out_load);

/* ------------------------------------------------------------------------
 * Problem description and the in-GPU work schedule.
 * ---------------------------------------------------------------------- */

/* One participant's view: the full draft-query set and one local shard of
 * context chunks (rit.work blog, section "Split-KV moves queries, not keys
 * and values": every participant gathers all queries and keeps its own
 * keys/values).  All pointers are HOST pointers; the schedule builder copies
 * what the kernels need into the schedule image. */
typedef struct skv_problem {
  int32_t nb;              /* anchor blocks; Nq = 16 * nb                   */
  int32_t hq, hkv, d;      /* heads and head dim                            */
  float scale;             /* softmax scale on q.k, > 0                     */
  int32_t dtype;           /* skv_dtype of Q, K, V, Kd, Vd, O, dO           */
  const int32_t* anchors;  /* [nb] exclusive bound of block i's context     */
  const int32_t* lo;       /* [nb] first context key block i may see        */
  int32_t n_chunks;        /* chunks held by this shard (may be 0)          */
  const int32_t* chunk_pos;/* [n_chunks] absolute position of the first key */
  const int32_t* chunk_off;/* [n_chunks+1] local rows: chunk c is K rows    */
                           /*   chunk_off[c] .. chunk_off[c+1]-1; [0] == 0  */
  int32_t with_draft;      /* 1 if this shard adds the draft-block keys     */
} skv_problem;

/* Summary of a schedule image, filled by skv_schedule_build. */
typedef struct skv_schedule_info {
  int64_t words;               /* int32 words of the image                  */
  int32_t n_workgroups;        /* persistent workgroups (bins)              */
  int32_t n_tiles;             /* 64-key tiles of the shard                 */
  int32_t n_qtiles;            /* 256-row query tiles (all kv heads)        */
  int32_t n_items;             /* forward / dQ work items                   */
  int32_t n_split_qtiles;      /* query tiles cut into several items        */
  int32_t n_partial_slots;     /* partial (O, LSE) slots for those tiles    */
  int32_t n_kv_items;          /* backward dK/dV work items                 */
  int32_t xcd_mode;            /* 1: queues planned per XCD (skv_schedule_build_xcd) */
  int64_t fwd_workspace_bytes; /* workspace for skv_attn_fwd_partial        */
  int64_t bwd_workspace_bytes; /* workspace for skv_attn_bwd                */
  int64_t item_cost_total;     /* sum of forward item costs                 */
  int64_t item_cost_max_bin;   /* largest workgroup load (forward items)    */
  int64_t kv_cost_total;       /* same for the dK/dV items                  */
  int64_t kv_cost_max_bin;
  /* geometry the image was built for (checked by the device calls) */
  int32_t nb, hq, hkv, d, n_local, with_draft;
  /* dQ plan: the forward's items and queues, except in xcd_mode, where dQ
   * is planned on its own at the dQ kernel's XCD speeds */
  int32_t n_dq_items;          /* dQ work items                             */
  int32_t n_dq_split_qtiles;   /* query tiles cut into several dQ items     */
  int32_t n_dq_partial_slots;  /* fp32 dQ partial slots for those tiles     */
  int32_t reserved;
  int64_t dq_cost_total;       /* sum of dQ item costs                      */
  int64_t dq_cost_max_bin;     /* largest workgroup load (dQ items)         */
} skv_schedule_info;

/* Build the work schedule of one problem for n_workgroups persistent
 * workgroups (0 = the current device's compute-unit count; this call then
 * queries the device).  Forward / dQ work is cut into units (kv head,
 * 256-row query tile, run of consecutive 64-key tiles that some row of the
 * tile sees); the first unit of a query tile also takes its draft keys.
 * Item costs are in time units fitted to measured per-workgroup times, not
 * in the (anchor block, key tile) pairs of skv_chunk_costs: a key step
 * (64 keys) costs the same however many of the tile's anchor blocks see
 * it, and each item pays a fixed part.  Units are placed by
 * skv_plan_lpt_split (item_cost 44, step_cost 8, automatic target), so a
 * unit may be cut into several items whose partials are merged in the
 * forward call.  Work of one kv head is kept on the workgroups of one XCD
 * class (workgroup w runs on XCD w mod 8) so its keys/values share an L2.
 * Backward dK/dV items (kv head, two 64-key tiles) and draft groups (kv
 * head, 128 draft tokens) cost 13 plus 5 per 64-row tile of the anchor
 * blocks that see them, and are placed by plain LPT per XCD class; at run
 * time a workgroup that has finished its own queue takes the next items of
 * the queue with the most planned work left (every item still runs once,
 * and its outputs do not depend on where).
 *   image: host int32 buffer of capacity_words, or NULL to only fill
 *   `info` (size query).  The caller copies the image to device memory
 *   and passes that copy, with `info`, to the device calls below.  The
 *   schedule stays valid for every layer that shares the anchors and the
 *   shard (the mask does not change across layers).
 * Errors: SKV_ERR_INVALID_ARG, SKV_ERR_UNSUPPORTED, SKV_ERR_WORKSPACE
 * (image too small; info->words says how much is needed). */
skv_status skv_schedule_build(const skv_problem* p, int32_t n_workgroups,
                              int32_t* image, int64_t capacity_words,
                              skv_schedule_info* info);

/* The same schedule planned for XCDs of unequal speed (arXiv abstract of
 * the Split-KV paper: chunks are balanced by their realised cost; here the
 * realised speed of the hardware that runs them enters the cost).
 * xcd_speed[k * 8 + x] is the relative speed (work per unit time, any
 * positive scale) of XCD x in kernel k: 0 the forward, 1 dQ, 2 dK/dV, for
 * instance measured with skv_timing_wg_clock on a schedule without it
 * (dK/dV workgroups also run items of other queues, so their stamps do not
 * time their own queue alone: the dQ kernel's speeds can stand in).
 * Queue v is planned at the speed of XCD v % 8.  Each XCD class (the
 * workgroups that hold one kv head's work) first gets a share of the work
 * in proportion to its total speed: classes above their share pass whole
 * units (the largest that fit) and at most one unit's tail to the classes
 * below theirs.  Each class then places its units on its workgroups by
 * LPT with splitting at their speeds (each piece to the workgroup of least
 * time, load / speed), at the target of a small grid whose slowest
 * workgroup finishes first.  That plan is kept only if its slowest
 * workgroup finishes before the uniform plan's at the same speeds.  The
 * forward and dQ are planned separately at their own speeds (each with its
 * own cuts, queues and partial slots; info->n_dq_* and dq_cost_* describe
 * dQ's); dK/dV items are shared out the same way and placed by LPT at
 * their speeds, without cuts.  At run time each workgroup takes the next
 * unclaimed queue of the XCD it runs on (the next XCD's if those are
 * taken), so the plan holds whatever XCD the dispatcher starts a launch on.  The per-XCD counters
 * live in the last 256 bytes of each workspace (counted in the workspace
 * sizes); the device calls zero them before each launch.  info->xcd_mode
 * is set.  Requires n_workgroups divisible by 8.
 * cost_scale (NULL: none) corrects the cost model with measured costs:
 * cost_scale[(k * hkv + h) * qt + t], k = 0 (forward) or 1 (dQ), qt = the
 * query tiles per kv head (info->n_qtiles / hkv), multiplies the cost of
 * every unit of kv head h and 256-row query tile t in kernel k's plan (its
 * fixed part and each step alike; item costs, loads and the cost totals in
 * info are then the scaled, rounded ones).  Scales fitted to the clock
 * stamps of an earlier plan let the plan follow costs the model does not
 * see, such as a kv head whose keys and values the memory system serves
 * more slowly.
 * Errors: as skv_schedule_build; SKV_ERR_INVALID_ARG for a NULL, zero,
 * negative or non-finite speed or cost scale, or n_workgroups not divisible
 * by 8. */
skv_status skv_schedule_build_xcd(const skv_problem* p, int32_t n_workgroups,
                                  const float* xcd_speed, const float* cost_scale,
                                  int32_t* image, int64_t capacity_words,
                                  skv_schedule_info* info);

/* ------------------------------------------------------------------------
 * Device calls.
 * ---------------------------------------------------------------------- */

/* Forward partial attention of all draft queries over this shard's keys
 * (rit.work blog, section "Split-KV moves queries, not keys and values":
 * each participant computes the local parts of attention for the whole
 * query set).  Writes O [Nq, hq, d] (o_dtype, normalised by this shard's
 * own softmax sum) and LSE [Nq, hq] fp32, the natural-log normaliser of
 * this shard.  Rows that see no key of this shard get O = 0, LSE = -inf.
 * With with_draft = 0, Kd/Vd are ignored and may be NULL.
 *   schedule: device copy of the image built for exactly this problem.
 *   workspace: device buffer of >= info->fwd_workspace_bytes (may be NULL
 *   when that is 0).  Errors: SKV_ERR_INVALID_ARG (mismatch with info,
 *   NULL), SKV_ERR_WORKSPACE, SKV_ERR_UNSUPPORTED, SKV_ERR_HIP. */
skv_status skv_attn_fwd_partial(const skv_problem* p,
                                const skv_schedule_info* info,
                                const int32_t* schedule, const void* Q,
                                const void* K, const void* V, const void* Kd,
                                const void* Vd, void* O, int32_t o_dtype,
                                float* LSE, void* workspace,
                                int64_t workspace_bytes, void* stream);

/* skv_attn_fwd_partial without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial slots of split query tiles
 * live in a static device array of the library: 64 MiB on each GPU the
 * library runs on, held from the first call on that GPU until the process
 * ends.  A schedule whose info->fwd_workspace_bytes exceeds 64 MiB is refused
 * with SKV_ERR_WORKSPACE before anything is launched.  The call uses the
 * current device's copy (stream must belong to the current device); nothing
 * in it needs to start at zero.  Every call on one GPU shares that copy, so
 * calls that overlap on one GPU (from other threads or on other streams) race
 * on it and must be serialised by the caller.  Other arguments, results and
 * errors as skv_attn_fwd_partial; SKV_ERR_HIP if the array's address cannot
 * be looked up. */
skv_status skv_attn_fwd_partial_noalloc(const skv_problem* p,
                                        const skv_schedule_info* info,
                                        const int32_t* schedule, const void* Q,
                                        const void* K, const void* V,
                                        const void* Kd, const void* Vd, void* O,
                                        int32_t o_dtype, float* LSE, void* stream);

/* Exact merge of n_parts partial results (rit.work blog, section "Split-KV
 * moves queries, not keys and values": participants reconcile the
 * normalisation; the split reproduces single-device attention exactly).
 *   O_parts [n_parts, rows, d] (in_dtype), LSE_parts [n_parts, rows] fp32;
 *   O_out [rows, d] (out_dtype), LSE_out [rows] fp32.  rows = Nq * hq.
 *   LSE = M + ln sum_k exp(LSE_k - M), M = max_k LSE_k; O = sum_k
 *   exp(LSE_k - LSE) O_k.  Partials with LSE_k = -inf weigh zero; a row
 *   with no finite LSE_k gets O = 0, LSE = -inf.  O_out may not alias the
 *   inputs.  Errors: SKV_ERR_INVALID_ARG, SKV_ERR_UNSUPPORTED, SKV_ERR_HIP. */
skv_status skv_merge_lse(int32_t n_parts, int64_t rows, int32_t d,
                         const void* O_parts, int32_t in_dtype,
                         const float* LSE_parts, void* O_out,
                         int32_t out_dtype, float* LSE_out, void* stream);

/* Backward of this shard (rit.work blog, section "Split-KV moves queries,
 * not keys and values": only the queries and their gradients cross
 * participants; key/value gradients stay local).  With the FINAL merged
 * output O and normaliser LSE of the whole context:
 *   dQ  [Nq, hq, d] fp32: this shard's share of the query gradient
 *       (shares over shards sum to the full dQ); overwritten.
 *   dK, dV [n_local, hkv, d] (grad_dtype): gradients of the local keys.
 *   dKd, dVd [Nq, hkv, d] (grad_dtype): draft-key gradients, only with
 *       with_draft = 1 (else ignored, may be NULL).
 *   workspace: >= info->bwd_workspace_bytes.
 * The backward takes bf16 inputs only (problem dtype SKV_BF16); an fp32
 * problem returns SKV_ERR_UNSUPPORTED (the fp32 path is forward-only).
 * Errors as skv_attn_fwd_partial. */
skv_status skv_attn_bwd(const skv_problem* p, const skv_schedule_info* info,
                        const int32_t* schedule, const void* Q, const void* K,
                        const void* V, const void* Kd, const void* Vd,
                        const void* O, const void* dO, const float* LSE,
                        float* dQ, void* dK, void* dV, void* dKd, void* dVd,
                        int32_t grad_dtype, void* workspace,
                        int64_t workspace_bytes, void* stream);

/* dQ finalize: the sum of n_parts fp32 dQ shares, converted to out_dtype
 * (rit.work blog, section "Split-KV moves queries, not keys and values":
 * the participants return the query gradients to the query owner, who adds
 * them).  Share k is the `elems` floats at parts + k * part_stride (device,
 * 16-byte aligned; part_stride >= elems and a multiple of 4 when
 * n_parts > 1), e.g. the skv_attn_bwd dQ outputs of the shards, or what a
 * reduce-scatter delivered.  Shares are added in index order in fp32, so
 * the result does not depend on the launch; out_dtype SKV_BF16 rounds the
 * fp32 sum to nearest even once.  dq_out: device, 16-byte aligned, `elems`
 * values of out_dtype; it must not overlap the shares, except that an fp32
 * dq_out may be share 0 itself (in place).  elems = 0 launches nothing.
 * Async on `stream`.
 * Errors: SKV_ERR_INVALID_ARG, SKV_ERR_UNSUPPORTED (out_dtype),
 * SKV_ERR_HIP. */
skv_status skv_dq_finalize(int32_t n_parts, int64_t elems, const float* parts,
                           int64_t part_stride, void* dq_out, int32_t out_dtype,
                           void* stream);

/* ------------------------------------------------------------------------
 * Benchmark support: per-kernel timing with HIP events.
 * ---------------------------------------------------------------------- */

/* While enabled on the calling thread, every kernel a device call launches
 * is bracketed by a hipEventRecord pair on its launch stream.  Records are
 * per thread and kept until collected.  Disabled by default. */
skv_status skv_timing_enable(int32_t on);

/* Wait for the recorded events, fold them into per-kernel totals (launch
 * count and summed milliseconds) and clear the records; *n_kernels gets the
 * number of distinct kernels.  Errors: SKV_ERR_HIP if an event failed. */
skv_status skv_timing_collect(int32_t* n_kernels);

/* Kernel k of the last collect: its name (NUL-terminated, truncated to
 * name_cap), launch count and total milliseconds.  Errors:
 * SKV_ERR_INVALID_ARG for k out of range or a NULL/empty name buffer. */
skv_status skv_timing_result(int32_t k, char* name, int32_t name_cap, int64_t* launches,
                             double* total_ms);

/* Per-workgroup clock stamps, for measuring how evenly a plan's work lands
 * on the workgroups (the pages' load-balance claim, measured rather than
 * planned).  While `buffer` (device memory, 8-byte aligned, owned by the
 * caller) is set on the calling thread, the bf16 forward, dQ and dK/dV
 * kernels each write, per queue v (the queue a workgroup ran: v is the
 * workgroup index unless the schedule has per-XCD queues), four uint64 at
 * [4v, 4v + 3] of their region: start and end on the GPU's constant 100 MHz
 * clock, then the
 * hardware XCC_ID and HW_ID register values of the wave that wrote them
 * (XCC_ID's low bits give the XCD; HW_ID holds the wave, SIMD, CU and
 * shader-engine ids).  Regions: forward at 0, dQ at 4 n_wg, dK/dV at 8 n_wg (n_wg =
 * the schedule's workgroup count).  Each launch overwrites its region.
 * NULL turns it off (the default).  A device call whose n_wg needs more
 * than `bytes` (3 * n_wg * 32) fails with SKV_ERR_INVALID_ARG before
 * launching.  The buffer must stay allocated until it is cleared (NULL) or
 * replaced: the library keeps only the pointer.  Launches on other threads
 * do not see it.
 * Errors: SKV_ERR_INVALID_ARG for a misaligned buffer, negative bytes or a
 * pointer that is not device (or managed) memory. */
skv_status skv_timing_wg_clock(void* buffer, int64_t bytes);

#ifdef __cplusplus
}
#endif
#endif /* SPLITKV_H */
