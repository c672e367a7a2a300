// Layout of the schedule image shared by the host builder and the kernels.
//
// The image is a flat int32 array built once on the host for one
// (anchors, shard) pair and copied to device memory by the caller.  It holds
// everything the kernels need besides the tensors: per-block mask bounds,
// the shard's key tiles, the forward/dQ work items with their per-workgroup
// LPT queues, the list of query tiles whose key range is cut into several
// items (their partials are merged after the main kernel), and the dK/dV
// work items with their queues.  The dQ kernel reads its items, queues and
// split records through the H_OFF_DQ_* words: they point at the forward's
// sections, or at dQ's own when the schedule was planned per XCD (the two
// kernels' XCD speeds differ, so each gets its own cuts and queues).
//
// The dK/dV kernel takes its items from its queues at run time: a
// workgroup runs the next unclaimed position of its own queue, then of the
// queue with the most planned work left, read from H_OFF_KVSUF (per queue
// position, the summed cost of that position and the rest of its queue).
//
// Queues are indexed by a queue number v in [0, n_wg).  Normally workgroup
// v runs queue v.  When H_XCD is set, queue v was planned for XCD v % 8 at
// that XCD's measured speed, and each workgroup takes the next unclaimed
// queue of the XCD it runs on (per-XCD counters zeroed before the launch).
#pragma once
#include <stdint.h>

namespace skv {

constexpr int32_t kMagic = 0x314B5653;  // "SVK1"
constexpr int32_t kVersion = 4;
constexpr int kBlock = 16;      // draft tokens per anchor block
constexpr int kTileK = 64;      // keys per key tile
constexpr int kQTile = 256;     // query rows (token x head of one kv head) per tile
constexpr int kKvGroup = 128;   // keys per dK/dV item (two 64-key tiles)
constexpr int kStatPad = 64;    // padding rows after each kv head's row statistics
constexpr int kXcds = 8;        // XCDs of the device; queues of XCD x are v = x, x + 8, ...

// Header word indices.
enum Hdr : int {
  H_MAGIC = 0, H_VERSION, H_NB, H_HQ, H_HKV, H_D, H_G, H_NLOCAL, H_DRAFT,
  H_NTILES, H_QT_PER_HEAD, H_NITEMS, H_NWG, H_NSPLIT, H_NSLOTS, H_NKV,
  H_OFF_ANCHORS, H_OFF_LO, H_OFF_TILES, H_OFF_ITEMS, H_OFF_QOFF, H_OFF_QUEUE,
  H_OFF_SPLIT, H_OFF_KV, H_OFF_KVQOFF, H_OFF_KVQUEUE, H_NCLASS,
  H_XCD, H_OFF_DQ_ITEMS, H_OFF_DQ_QOFF, H_OFF_DQ_QUEUE, H_OFF_DQ_SPLIT,
  H_OFF_KVSUF,
  H_WORDS = 40
};
static_assert(H_OFF_DQ_SPLIT < H_WORDS, "header words overflow the header");

// Key tile: 4 words.
enum TileW : int { T_ROW = 0, T_POS, T_LEN, T_PAD, T_WORDS = 4 };

// Forward / dQ item: 8 words.  Tiles [t0, t1) of the sorted tile list;
// slot < 0 writes the final rows directly, else partial slot `slot`.
// I_WHOLE packs the item's steps [s0, s1) (s0 in the low 16 bits) that
// every row of the query tile sees whole: full 64-key tiles inside every
// row's visible interval, which need neither bounds nor masks.
enum ItemW : int {
  I_HEAD = 0, I_QT, I_T0, I_T1, I_SLOT, I_FLAGS, I_COST, I_WHOLE, I_WORDS = 8
};
constexpr int32_t kItemDraft = 1;  // the item also covers the draft keys

// Split query tile: 4 words.
enum SplitW : int { S_HEAD = 0, S_QT, S_SLOT0, S_NSLOT, S_WORDS = 4 };

// dK/dV item: 9 words.  Either context keys (tiles t0 .. t0+nt-1, nt in
// {1, 2}) or draft keys (draft tokens [dtok0, dtok0 + ndraft)).  Query
// blocks [b0, b1) may see the keys.
enum KvW : int {
  K_HEAD = 0, K_T0, K_NT, K_DTOK0, K_NDRAFT, K_B0, K_B1, K_COST, K_WHOLE, K_WORDS = 9
};

}  // namespace skv
