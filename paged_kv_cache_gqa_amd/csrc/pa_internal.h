// pa_internal.h -- work-list records and kernel arguments shared by the host
// planner (pa_api.hip) and the gfx950 kernels (pa_*.hip).  Library-internal.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

// One attention work item: a tile of query rows of one (sequence, KV head)
// against the key range [kv_lo, kv_hi) of that sequence.  The tile's rows are
// the query tokens [row0, row0 + nq) times the G query heads of the group,
// ordered row = token * G + head_in_group.  part < 0: the item covers every
// key its rows see and writes the final output; otherwise it writes partial
// results into partial slot `part`, merged later.
struct Item {
  int32_t seq;
  int32_t kvh;
  int32_t row0;   // global q row of the tile's first token
  int32_t pos0;   // absolute position of that token (hist + index in increment)
  int32_t nq;     // query tokens in the tile
  int32_t kv_lo;  // first key (multiple of the 64-key tile)
  int32_t kv_hi;  // one past the last key
  int32_t part;   // partial slot or -1
};
static_assert(sizeof(Item) == 32, "Item layout");

// One merge task: rows of one split tile, partial slots [part0, part0+nparts).
struct Merge {
  int32_t row0;
  int32_t nq;
  int32_t kvh;
  int32_t part0;
  int32_t nparts;
  int32_t rows_per_part;  // slot height: 128 (prefill tiles) or 16 (decode tiles)
  int32_t is_decode;      // which partial array the slots live in
  int32_t pad;
};
static_assert(sizeof(Merge) == 32, "Merge layout");

// Shared-prefix cascade ([Agentic] §2.1: sub-agents start from the main
// agent's context; §4.1: prefix reuse): the decode rows of up to
// kCascadeRows / G sequences whose first keys lie in the same physical
// blocks, against one key range of that shared prefix, as one tile.  Each
// member writes its rows' partial result to its own slot, merged by LSE with
// the partials of its own suffix.
struct CascadeItem {
  int32_t seq;    // a member: its block-table row names the shared blocks
  int32_t kvh;
  int32_t kv_lo;  // key range within the shared prefix
  int32_t kv_hi;
  int32_t mem0;   // this item's first entry in the member table
  int32_t nmem;   // members; member i's G rows are tile rows i*G .. i*G+G-1
  int32_t pad[2];
};
static_assert(sizeof(CascadeItem) == 32, "CascadeItem layout");
struct CascadeMember {
  int32_t row0;   // q row of the member's (single) new token
  int32_t part;   // decode partial slot for this item's key range
};
constexpr int kCascadeRows = 64;  // query rows per cascade tile (4 row blocks of 16)

// KV element formats (pa_kv_dtype)
enum KvFmt : int { kKvBf16 = 0, kKvE4m3 = 1, kKvMxfp4 = 2 };

struct CacheArgs {
  const void *k;
  const void *v;
  const void *ks;         // E4M3: fp32 [nb][hkv]; MXFP4: E8M0 bytes [nb][hkv][d/32][bs]
  const void *vs;
  int32_t num_blocks;
  int32_t hkv;
};

struct AttnArgs {
  const void *q;          // bf16 [total_q][hq][d]
  CacheArgs c;
  const int32_t *bt;      // [num_seqs][max_blocks]
  int32_t max_blocks;
  int32_t hq;
  int32_t group;          // G = hq / hkv (power of two)
  int32_t tile_rows;      // query rows per prefill tile (128 or 256)
  int32_t lg;             // log2(G)
  float scale_log2;       // softmax scale * log2(e)
  void *out;              // bf16 [total_q][hq][d]
  float *lse_out;         // optional fp32 [total_q][hq] (natural log)
  const Item *items;
  const int32_t *wg_first;  // persistent launch: work-group w runs items [wg_first[w], wg_first[w+1])
  float *part_o;          // [slots][rows_per_slot][d] fp32, normalised partial outputs
  float *part_lse;        // [slots][rows_per_slot], log2 units
};

struct MergeArgs {
  const Merge *merges;
  const float *part_o_prefill;
  const float *part_lse_prefill;
  const float *part_o_decode;
  const float *part_lse_decode;
  void *out;
  float *lse_out;
  int32_t hq;
  int32_t group;
  int32_t lg;
  int32_t d;
};

struct AppendArgs {
  const void *k_new;
  const void *v_new;
  const int64_t *slots;
  void *k_cache;
  void *v_cache;
  void *ks;               // E4M3: read; MXFP4: written
  void *vs;
  int64_t tok0;           // first token of this launch
  uint32_t nchunks;       // this launch's tokens * hkv * (d / 8), below 2^31
  int32_t hkv;
  int32_t bs;             // a power of two
  int32_t lbs;            // log2(bs)
  int32_t d;              // 64 or 128
  int32_t lcpr;           // log2(d / 8)
};

struct GatherArgs {
  const void *k;
  const void *v;
  const void *ks;         // MXFP4: scale bytes (the gather then writes bf16 values)
  const void *vs;
  const int32_t *bt_row;
  void *k_out;
  void *v_out;
  int64_t total_chunks;   // ctx * hkv * (row bytes / 16)
  int32_t hkv;
  int32_t bs;
  int32_t row_bytes;      // d * element bytes (MXFP4: d / 2)
  int32_t fmt;            // KvFmt
};

constexpr int kRegTileRows = 128;  // query rows (tokens x heads) per tile of prefill_kernel
constexpr int kW48TileRows = 384;  // query rows per tile of prefill_w48_kernel
constexpr int kDmaTileRows = kW48TileRows;  // the LDS-DMA prefill (head_dim 128)
constexpr int kPrefillRowsMax = 384;
constexpr int kMaxDecItemKeys = 32768;  // keys per decode item (block ids staged in LDS)
constexpr int kDecodeRows = 16;    // query rows per decode tile
constexpr int kKeyTile = 64;       // keys per inner-loop tile

// Launchers (defined next to their kernels).
// One launch per step: persistent work-groups claim tasks -- kv_append token
// chunks, prefill ranges (per-XCD queues), decode items -- by vector atomics
// on counters in the workspace; the last writer of a split tile's partials
// merges them.  Counters (uint32, zeroed by the work-list copy):
constexpr int kCtrAppendNext = 0;   // next append task
constexpr int kCtrAppendDone = 1;   // append tasks finished
constexpr int kCtrDecodeNext = 2;   // next decode item
constexpr int kCtrFlags = 3;        // bit 0: a bounded wait gave up (never expected)
constexpr int kCtrPrefillNext = 4;  // [kMaxXcds] next range of each XCD's prefill queue
constexpr int kMaxXcds = 8;
constexpr int kCtrRole = kCtrPrefillNext + kMaxXcds;  // [kMaxXcds] work-groups of each XCD past the append wait
constexpr int kCtrMerge = kCtrRole + kMaxXcds;        // [n_merges] partials written per merge record
constexpr int kStepThreads = 512;
constexpr int kStepAppendChunks = 8 * kStepThreads;  // 16-byte append chunks per append task

struct StepArgs {
  AttnArgs pre;                  // prefill items and partial arrays
  AttnArgs dec;                  // decode items and partial arrays
  AppendArgs app;                // the step's new tokens (tok0 = 0, nchunks = all)
  MergeArgs mg;                  // merge records over both partial arrays
  const int32_t *wg_first;       // prefill range r: items [wg_first[r], wg_first[r+1])
  const int32_t *pre_queue;      // range ids, XCD queue by XCD queue
  const int32_t *pre_queue_off;  // [kMaxXcds + 1]
  const int32_t *pre_part_merge; // merge record of each prefill partial slot
  const int32_t *dec_part_merge; // ... of each decode partial slot
  uint32_t *ctr;
  int32_t n_append_tasks;
  int32_t n_decode;
  int32_t xcds;                  // queues in use (1 .. kMaxXcds)
  int32_t decode_first;          // work-groups per XCD that take decode items before prefill ranges
};

hipError_t launch_step(const StepArgs &a, int n_groups, int bs, int fmt, hipStream_t s);
hipError_t launch_prefill(const AttnArgs &a, int n_items, int d, int bs, int fmt, hipStream_t s);
hipError_t launch_decode(const AttnArgs &a, int n_items, int d, int bs, int fmt, hipStream_t s);
// head_dim 128 decode launch (bf16 cascade items, if any, then decode items)
// whose items are claimed from *ctr (zero before the first of the launches
// that share it) by `groups` persistent work-groups
hipError_t launch_decode_claim(const AttnArgs &a, uint32_t *ctr, int n_decode, const CascadeItem *citems,
                               const CascadeMember *members, int n_cascade, int rows, int groups, int bs, int fmt,
                               hipStream_t s);
// bf16 head_dim 128 decode launch with shared-prefix cascade items first
// (rows: the largest member count times G among them, at most kCascadeRows)
hipError_t launch_decode_cascade(const AttnArgs &a, const CascadeItem *items, const CascadeMember *members,
                                 int n_cascade, int n_decode, int rows, int bs, hipStream_t s);
// merges [0, n_few) have at most kMergeSerialParts parts, [n_few, n_few +
// n_many) more, with at most many_rows rows each
hipError_t launch_merge(const MergeArgs &a, int n_few, int n_many, int many_rows, hipStream_t s);
constexpr int kMergeSerialParts = 16;
hipError_t launch_append(const AppendArgs &a, int fmt, int64_t num_tokens, hipStream_t s);
// measurement hooks (pa_peak.hip)
constexpr int kPeakMfmaGroups = 256;   // one 512-thread work-group per CU
constexpr int kPeakReadGroups = 256;   // streaming read: one 4-wave work-group per CU
hipError_t launch_peak_mfma(float *out, int iters, hipStream_t s);
hipError_t launch_peak_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);
hipError_t launch_xcc_ids(int32_t *out, int n, hipStream_t s);
hipError_t launch_stage(const void *src_host, void *dst, size_t bytes, hipStream_t s);

}  // namespace pa
