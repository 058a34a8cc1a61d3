// pa_api.hip -- the C ABI (include/pagedattn.h): host-side validation, the
// work planner, workspace layout, pinned staging of the work list, launches
// and per-kernel timing.
//
// Pages cited (title, then section):
//   [Agentic] "vLLM Agentic 推理｜面向 Agent 负载的推理优化"
//   [AMPD]    "ICML'26 | AMPD：PD 分离遇上多轮推理，incremental prefill 到底该在哪跑"
//   [V1Sched] "vLLM/V1 推理调度器"
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pagedattn.h"
#include "pa_internal.h"

using namespace pa;

// The no-allocation entry point's scratch (see scratch_address below).
static __device__ __attribute__((aligned(256))) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status hip_fail(hipError_t e, const char *what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

int log2_exact(int v) {
  int k = 0;
  while ((1 << k) < v) k++;
  return (1 << k) == v ? k : -1;
}

pa_status check_cache(const pa_kv_cache *c) {
  if (!c) return fail(PA_ERR_NULL_ARG, "cache is NULL");
  if (!c->k_cache || !c->v_cache) return fail(PA_ERR_NULL_ARG, "k_cache/v_cache is NULL");
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return fail(PA_ERR_BAD_SHAPE, "num_blocks (%d) and num_kv_heads (%d) must be positive",
                c->num_blocks, c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->block_size != 16 && c->block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (16 or 64)", c->block_size);
  if (c->dtype != PA_KV_BF16 && c->dtype != PA_KV_FP8_E4M3 && c->dtype != PA_KV_MXFP4)
    return fail(PA_ERR_UNSUPPORTED, "unknown KV dtype %d", (int)c->dtype);
  const bool scaled = c->dtype != PA_KV_BF16;
  if (scaled && (!c->k_scale || !c->v_scale))
    return fail(PA_ERR_NULL_ARG, "%s cache needs k_scale and v_scale",
                c->dtype == PA_KV_MXFP4 ? "MXFP4" : "E4M3");
  if (!scaled && (c->k_scale || c->v_scale))
    return fail(PA_ERR_BAD_SHAPE, "bf16 cache must not carry scales");
  if (c->dtype == PA_KV_MXFP4 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "MXFP4 KV needs head_dim 128 (got %d)", c->head_dim);
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Work planner.  Inputs are the scheduler's host-side lengths ([V1Sched]
// "实际实现": per request, the computed-token count and the tokens scheduled
// this step).  A sequence whose increment times the group size fits 16 rows
// is a decode-class tile (one tile per KV head); otherwise its increment is
// cut into 128-row prefill tiles.  Key ranges are split so that there are
// enough similar-sized items to fill every compute unit; split items write
// partials merged by LSE ([Agentic] §4.3.3).
constexpr int kDecodeItemsPerCU[] = {1, 2, 4};  // candidate decode cuts (decode_chunk)
constexpr int kDecodeMinChunk = 2048;
constexpr int kDecodeItemStartKeys = 512;  // an item's start-up, in keys streamed
constexpr int kPrefillItemsPerCU = 8;

// The machine the plan is cut for: compute units and XCDs (chiplets, each
// with its own L2) of the current device, queried once per device.  Without a
// device (the host-only planning hooks on a machine with no GPU) the MI355X's
// 256 CUs in 8 XCDs are assumed.  Work-group ids are dispatched round-robin
// over the XCDs (work-group w runs on XCD (w + k) mod num_xcds, k fixed per
// launch: 0 for a launch alone on the GPU, possibly not while another
// stream's launch is being dispatched); pa_debug_xcc_ids lets a test check
// that on the GPU.  The plans rely only on the work-groups of one residue
// class sharing an XCD.
struct MachineShape {
  int32_t cus = 256;
  int32_t xcds = 8;
};

MachineShape machine_shape() {
  static std::mutex mu;
  static std::vector<std::pair<int, MachineShape>> known;
  static bool no_device = false;
  std::lock_guard<std::mutex> lk(mu);
  if (no_device) return MachineShape{};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    no_device = true;
    return MachineShape{};
  }
  for (auto &k : known)
    if (k.first == dev) return k.second;
  MachineShape m;
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) m.cus = v;
  v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0 && m.cus % v == 0)
    m.xcds = v;
  else
    m.xcds = 1;
  (void)hipGetLastError();
  known.push_back({dev, m});
  return m;
}
constexpr int kPrefillMinChunk = 4096;
constexpr int kMinGroupKeyTiles = 16;  // persistent launch: at least 1024 keys per work-group

struct Plan {
  std::vector<Item> prefill, decode;
  std::vector<Merge> merges;
  std::vector<int32_t> wg_first;  // persistent prefill launch: items of work-group w are
                                  // prefill[wg_first[w] .. wg_first[w+1]); empty otherwise
  int64_t n_part_prefill = 0, n_part_decode = 0;
  // shared-prefix cascade: items and their member tables; the widest item's rows
  std::vector<CascadeItem> cascade;
  std::vector<CascadeMember> members;
  int32_t cascade_rows = 0;
  // one-launch step: prefill ranges per XCD queue, the merge record of
  // each partial slot, the task counters
  std::vector<int32_t> step_queue, step_queue_off, step_pre_merge, step_dec_merge;
  int32_t step_xcds = 1, step_ranges = 0;
  int32_t step_decode_cus = 0;  // one-launch step: CUs that take decode items first
  size_t n_ctr = 0;
  // co-scheduled mixed step: CUs that stream decode items beside the
  // persistent prefill launch (0: the launches run one after the other)
  int32_t overlap_cus = 0;
  size_t off_prefill = 0, off_decode = 0, off_merges = 0, off_wg = 0, off_cascade = 0, off_members = 0,
         off_sq = 0, off_sqo = 0, off_spm = 0, off_sdm = 0, off_ctr = 0, off_claim = 0, plan_bytes = 0;
  size_t off_po_pre = 0, off_pl_pre = 0, off_po_dec = 0, off_pl_dec = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Tile {
  int32_t seq, row0, pos0, nq, keys;  // keys = last row's position + 1
  bool decode;
  int32_t shared = 0;  // leading keys computed by a shared-prefix cascade item instead
};

// Prefix groups a caller declares (paged_attn_forward_cascade): group_of[s]
// (-1 = none) and the shared length of each group.
struct Groups {
  const int32_t *group_of = nullptr;
  const int32_t *group_len = nullptr;
  int32_t num_groups = 0;
};

// Prefill ranges per compute unit in the one-launch step's plan (more,
// shorter ranges let work-groups that finish early take more of them; with
// ranges of equal length that gained nothing: 4 per CU measured 12.6 ms
// against 12.3 ms for the mixed step, the extra partials and merges costing
// more than the balance won).
#ifndef PA_STEP_RANGES_PER_CU
#define PA_STEP_RANGES_PER_CU 1
#endif
constexpr int32_t kStepRangesPerCu = PA_STEP_RANGES_PER_CU;

// The step's new tokens for the one-launch step (paged_attn_step).
struct StepIn {
  const void *k_new = nullptr, *v_new = nullptr;
  const int64_t *slots = nullptr;
};

// Balanced cut of [0, keys) into n ranges whose inner boundaries are
// multiples of the 64-key tile.
void cut(int32_t keys, int32_t n, std::vector<std::pair<int32_t, int32_t>> &out) {
  out.clear();
  const int32_t ntile = (int32_t)cdiv64(keys, kKeyTile);
  n = std::max(1, std::min(n, ntile));
  for (int32_t i = 0; i < n; i++) {
    const int32_t lo = (int32_t)((int64_t)ntile * i / n) * kKeyTile;
    const int32_t hi = i + 1 == n ? keys : (int32_t)((int64_t)ntile * (i + 1) / n) * kKeyTile;
    if (hi > lo) out.push_back({lo, hi});
  }
}

// Query rows per prefill tile: the LDS-DMA kernel (head_dim 128, every KV
// format) takes 384, the register-staged kernel (head_dim 64) 128.
int32_t prefill_tile_rows(const pa_kv_cache *c) {
  return c->head_dim == 128 ? kDmaTileRows : kRegTileRows;
}

// Persistent split for the LDS-DMA prefill kernels.  The prefill work -- every tile
// times every KV head, measured in 64-key steps -- is laid out KV-head-major,
// then by key chunk, then by tile, and cut into nwg contiguous ranges of equal
// length (to within one step), one per work-group: every compute unit gets
// the same amount of work.  Key chunks are common to all tiles (chunk c is
// keys [c*C, (c+1)*C)), so the work-groups that walk one chunk of different
// tiles at the same time read the same K/V bytes and share them in L2.  A
// (tile, head) whose keys are spread over several chunks or ranges writes
// partials merged by LSE.  Range r goes to work-group w with r = (w % 8) *
// (nwg / 8) + w / 8 when nwg is a multiple of 8: work-group ids are dispatched
// round-robin over the eight XCDs, so each XCD (and its L2) holds one
// contiguous stretch of the work, i.e. mostly one KV head.
// Key chunks: with PA_GROUP_PIECES = k > 0 the chunk length is chosen so a
// work-group's share spans about k (tile, chunk) pieces; 0 (default) makes
// the whole key range one chunk: fewer split tiles (half the partial bytes
// at 48K), and the work-groups of an XCD still start together at key 0 (up
// to 7% faster at 48K, 3% at 131K, 1% at 1M than k = 2).
#ifndef PA_GROUP_PIECES
#define PA_GROUP_PIECES 0
#endif
constexpr int kGroupPieces = PA_GROUP_PIECES;
#ifndef PA_PLAN_LPT
#define PA_PLAN_LPT 1
#endif
constexpr bool kPlanLpt = PA_PLAN_LPT;

void plan_persistent(const std::vector<Tile> &tiles, int32_t hkv, int32_t tile_rows, const MachineShape &M,
                     Plan &P, int32_t ranges_per_cu = 1) {
  std::vector<int32_t> pre;  // prefill tiles
  int32_t max_steps = 0;
  int64_t W = 0;
  for (size_t i = 0; i < tiles.size(); i++) {
    if (tiles[i].decode) continue;
    pre.push_back((int32_t)i);
    const int32_t steps = (int32_t)cdiv64(tiles[i].keys, kKeyTile);
    max_steps = std::max(max_steps, steps);
    W += (int64_t)steps * hkv;
  }
  if (W == 0) return;
  const int32_t nwg =
      (int32_t)std::max<int64_t>(1, std::min<int64_t>((int64_t)M.cus * ranges_per_cu, W / kMinGroupKeyTiles));
  // chunk length (in steps) so that a work-group's range spans about
  // kGroupPieces (tile, chunk) pieces
  const int64_t units = (int64_t)pre.size() * hkv;
  const int64_t nchunk = kGroupPieces == 0 ? 1 : std::max<int64_t>(1, cdiv64((int64_t)kGroupPieces * nwg, units));
  const int32_t C = (int32_t)std::max<int64_t>(1, cdiv64(max_steps, nchunk));

  struct Piece {
    int32_t unit, lo, hi, range;  // unit = kvh * pre.size() + tile index; [lo, hi) in steps
  };
  std::vector<Piece> pieces;
  auto bound = [&](int64_t r) { return W * r / nwg; };  // first step of range r
  int64_t pos = 0;
  int32_t r = 0;
  // Many tiles per KV head (an initial prefill: tiles of every length up to
  // the context): whole (tile, head) units instead, longest first, each to
  // the least loaded range of the XCD that holds the head (greedy LPT: the
  // loads end within the shortest tiles' length of each other).  The XCD's
  // work-groups then start tiles of nearly equal length at key 0 together,
  // round after round, and share K/V in L2; no tile is split (no partials).
  const int32_t xcds = M.xcds;
  const int32_t per_xcd = nwg / xcds;
  const bool lpt = kPlanLpt && nwg % xcds == 0 && hkv % xcds == 0 &&
                   (int64_t)pre.size() * (hkv / xcds) >= 8 * per_xcd;
  if (lpt) {
    std::vector<int32_t> order(pre.size());
    for (size_t k = 0; k < pre.size(); k++) order[k] = (int32_t)k;
    auto steps_of = [&](int32_t k) { return (int32_t)cdiv64(tiles[pre[k]].keys, kKeyTile); };
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return steps_of(x) > steps_of(y); });
    for (int32_t x = 0; x < xcds; x++) {
      std::vector<int64_t> load(per_xcd, 0);
      for (int32_t kvh = x; kvh < hkv; kvh += xcds)
        for (int32_t k : order) {
          int32_t j = 0;
          for (int32_t q = 1; q < per_xcd; q++)
            if (load[q] < load[j]) j = q;
          const int32_t steps = steps_of(k);
          pieces.push_back({kvh * (int32_t)pre.size() + k, 0, steps, x * per_xcd + j});
          load[j] += steps;
        }
    }
  }
  for (int32_t kvh = 0; kvh < (lpt ? 0 : hkv); kvh++)
    for (int32_t c0 = 0; c0 < max_steps; c0 += C)
      for (size_t k = 0; k < pre.size(); k++) {
        const int32_t steps = (int32_t)cdiv64(tiles[pre[k]].keys, kKeyTile);
        if (c0 >= steps) continue;
        const int32_t c1 = std::min(steps, c0 + C);
        for (int32_t lo = c0; lo < c1;) {
          while (bound(r + 1) <= pos) r++;
          const int32_t hi = (int32_t)std::min<int64_t>((int64_t)c1, lo + bound(r + 1) - pos);
          pieces.push_back({kvh * (int32_t)pre.size() + (int32_t)k, lo, hi, r});
          pos += hi - lo;
          lo = hi;
        }
      }
  // partial slots: consecutive per (tile, head) unit, in key order.  A piece
  // is never cut for length: the kernel walks any key range in windows whose
  // block ids it restages, so a (tile, head) needs a partial slot per range
  // it spans -- at most units + work-groups slots, whatever the context.
  std::vector<int32_t> count(units, 0), part0(units, -1), seen(units, 0);
  for (const Piece &pc : pieces) count[pc.unit]++;
  for (int64_t u = 0; u < units; u++) {
    if (count[u] < 2) continue;
    const Tile &t = tiles[pre[u % pre.size()]];
    part0[u] = (int32_t)P.n_part_prefill;
    P.n_part_prefill += count[u];
    P.merges.push_back({t.row0, t.nq, (int32_t)(u / pre.size()), part0[u], count[u], tile_rows, 0, 0});
  }
  std::vector<std::vector<Item>> by_range(nwg);
  for (const Piece &pc : pieces) {
    const Tile &t = tiles[pre[pc.unit % pre.size()]];
    const int32_t part = part0[pc.unit] < 0 ? -1 : part0[pc.unit] + seen[pc.unit]++;
    by_range[pc.range].push_back({t.seq, pc.unit / (int32_t)pre.size(), t.row0, t.pos0, t.nq,
                                  pc.lo * kKeyTile, std::min(t.keys, pc.hi * kKeyTile), part});
  }
  // Within a range, pieces that start at a chunk boundary come first, in key
  // order: every work-group then starts at the start of a chunk at the same
  // moment, and the work-groups on one chunk walk it in step.
  for (auto &v : by_range)
    std::stable_partition(v.begin(), v.end(), [&](const Item &x) { return x.kv_lo % (C * kKeyTile) == 0; });
  P.wg_first.assign(nwg + 1, 0);
  for (int32_t w = 0; w < nwg; w++) {
    const int32_t rr = nwg % xcds == 0 ? (w % xcds) * (nwg / xcds) + w / xcds : w;
    P.wg_first[w] = (int32_t)P.prefill.size();
    P.prefill.insert(P.prefill.end(), by_range[rr].begin(), by_range[rr].end());
  }
  P.wg_first[nwg] = (int32_t)P.prefill.size();
}

// Key length of decode items.  Fewer, longer items pay an item's start-up
// (its block ids staged, the first loads in flight) less often; more, shorter
// ones balance better.  Among the cuts for 1, 2 and 4 items per CU (at least
// kDecodeMinChunk, at most kMaxDecItemKeys keys), the one with the shortest
// predicted makespan is taken: the items are dispatched longest first, each
// to the CU that frees first (one decode work-group per CU), and an item
// costs its keys plus kDecodeItemStartKeys.  (A single 1M-token sequence:
// 256 items of 32K keys instead of 1,024 of 8K, 6% faster for 4-bit KV.)
int64_t decode_chunk(const std::vector<Tile> &tiles, int32_t hkv, int32_t cus, int64_t wd) {
  int64_t best_chunk = kMaxDecItemKeys, best_span = -1;
  std::vector<std::pair<int32_t, int32_t>> ranges;
  std::vector<int64_t> cost;
  for (const int k : kDecodeItemsPerCU) {
    const int64_t chunk = std::min<int64_t>(
        kMaxDecItemKeys, std::max<int64_t>(kDecodeMinChunk, cdiv64(std::max<int64_t>(wd, 1), (int64_t)k * cus)));
    cost.clear();
    for (const Tile &t : tiles) {
      if (!t.decode) continue;
      cut(t.keys, (int32_t)std::min<int64_t>(cdiv64(t.keys, chunk), INT32_MAX), ranges);
      for (const auto &r : ranges)
        for (int32_t h = 0; h < hkv; h++) cost.push_back((int64_t)(r.second - r.first) + kDecodeItemStartKeys);
    }
    std::sort(cost.begin(), cost.end(), std::greater<int64_t>());
    // list scheduling: a min-heap of the CUs' finishing times
    std::vector<int64_t> cu(std::min<size_t>((size_t)cus, cost.size()), 0);
    int64_t span = 0;
    for (size_t i = 0; i < cost.size(); i++) {
      if (i < cu.size()) {
        cu[i] = cost[i];
        if (i + 1 == cu.size()) std::make_heap(cu.begin(), cu.end(), std::greater<int64_t>());
      } else {
        std::pop_heap(cu.begin(), cu.end(), std::greater<int64_t>());
        cu.back() += cost[i];
        std::push_heap(cu.begin(), cu.end(), std::greater<int64_t>());
      }
    }
    for (const int64_t f : cu) span = std::max(span, f);
    if (best_span < 0 || span < best_span) best_span = span, best_chunk = chunk;
  }
  return best_chunk;
}

// Co-scheduling a mixed step's decode with its prefill.  The 384-row prefill
// keeps every CU's matrix cores busy but draws little from HBM; the decode
// streams from HBM and computes little.  A CU streams more than its 1/256
// share of the chip's bandwidth when few CUs stream (measured with the
// LDS-filling read alone: 59 GB/s per CU with 32 CUs, 55 with 64, 48 with
// 128, 28 with all 256; the bf16 decode items beside the prefill: ~45 GB/s per CU
// with 8-wave work-groups), so a few CUs given to the decode while the others
// prefill stream most of it before the prefill ends.  The candidates are
// multiples of the XCD count (an equal number per XCD, so the prefill's
// ranges stay balanced per XCD) up to half the CUs; the time of each is
// predicted as the prefill on the remaining CUs plus the decode bytes those
// few CUs could not stream meanwhile, streamed afterwards by the whole chip;
// the shortest wins (0: no co-scheduling).  Each CU given to the decode
// also slows the prefill's other CUs a little (the decode's HBM streams and
// the chip's power draw are shared), a fraction per CU taken.  Unit costs,
// MI355X, per KV format (fitted to the mixed step below at n = 0 .. 56):
// the prefill time of a 384-row tile's 64-key step of one KV head on one CU;
// the decode's bytes per second per CU beside the prefill (the quantised
// formats spend more ALU per byte) and over the whole chip; the prefill's
// slow-down per CU taken.
// (The mixed step of 4 incremental prefills and 48 decodes, bf16, block 16:
// 12.4-12.6 ms one after the other; 11.0-11.1 ms with the 48 decode CUs the
// model picks, 11.3-11.5 with 40 or 56; the one-launch step likewise 12.1 ->
// 10.9 ms.  The same step with E4M3 KV, block 64, whose decode takes 1.9 ms
// on the whole chip: 10.6-10.7 ms one after the other, 10.5-10.6 with 8 to
// 32 CUs on one device and 10.8 with 32 on another, whose prefill slowed
// more beside the decode; with MXFP4 KV (decode 1.1 ms): 9.1 ms one after
// the other, 9.05 with 8 CUs, 9.2 with 16, 9.7 with 32.  The rates below
// sit between the devices' fits, so the model runs those two steps one
// launch after the other and co-schedules quantised steps whose decode
// share is larger.)
struct CoRates {
  double prefill_step_sec, decode_cu_bytes_per_sec, decode_chip_bytes_per_sec, prefill_slow_per_cu;
};
constexpr CoRates kCoRatesBf16 = {2.47e-6, 45e9, 6.5e12, 0.0009};
constexpr CoRates kCoRatesE4m3 = {2.49e-6, 30e9, 6.35e12, 0.0016};
constexpr CoRates kCoRatesMxfp4 = {2.26e-6, 28e9, 5.8e12, 0.002};
std::atomic<int32_t> g_overlap_force{-1};  // pa_debug_overlap_cus: < 0 the model's choice

// Returns the CUs taken from the prefill's share (-1: no co-scheduling).  A
// prefill too small to fill every CU (at least kMinGroupKeyTiles steps per
// work-group) leaves the rest to the decode at no cost.
// shared_keys: the keys the cascade items read once for all members of
// their groups (members' own keys count from the end of the shared prefix);
// key_bytes: K and V bytes of one key and KV head in the cache's format;
// R: that format's unit costs.
int32_t choose_overlap_cus(const std::vector<Tile> &tiles, int64_t shared_keys, int32_t hkv, int64_t key_bytes,
                           const CoRates &R, const MachineShape &M) {
  int64_t units = 0, dec_bytes = shared_keys * hkv * key_bytes;
  for (const Tile &t : tiles) {
    if (t.decode)
      dec_bytes += (int64_t)(t.keys - t.shared) * hkv * key_bytes;
    else
      units += cdiv64(t.keys, kKeyTile) * hkv;
  }
  if (units == 0 || dec_bytes == 0 || M.xcds <= 0 || M.cus % M.xcds != 0) return -1;
  const int32_t forced = g_overlap_force.load();
  if (forced == 0) return -1;
  if (forced > 0) return std::min(forced / M.xcds, M.cus / M.xcds / 2) * M.xcds;
  const int64_t pre_max = std::max<int64_t>(1, units / kMinGroupKeyTiles);
  int32_t best = 0;
  double best_t = -1.0;
  for (int32_t n = 0; n <= M.cus / 2; n += M.xcds) {
    const int64_t pre = std::min<int64_t>(M.cus - n, pre_max);
    const double tp = (double)units * R.prefill_step_sec / (double)pre * (1.0 + R.prefill_slow_per_cu * n);
    const double left = std::max(0.0, (double)dec_bytes - (double)(M.cus - pre) * R.decode_cu_bytes_per_sec * tp);
    const double t = tp + left / R.decode_chip_bytes_per_sec;
    if (best_t < 0.0 || t < best_t) best_t = t, best = n;
  }
  return best;
}

void make_plan(const int32_t *hist, const int32_t *incr, int32_t num_seqs, const pa_kv_cache *c,
               int32_t group, Plan &P, const Groups *groups = nullptr, bool step = false) {
  const int32_t hkv = c->num_kv_heads, d = c->head_dim, tile_rows = prefill_tile_rows(c);
  const MachineShape M = machine_shape();
  const int64_t prefill_target_items = (int64_t)kPrefillItemsPerCU * M.cus;
  const int32_t dec_tokens = kDecodeRows / group;  // >= 1 for group <= 16
  const int32_t pre_tokens = tile_rows / group;
  std::vector<Tile> tiles;
  int64_t row = 0;
  for (int32_t s = 0; s < num_seqs; s++) {
    const int32_t h = hist[s], n = incr[s];
    if (n > 0) {
      if (n <= dec_tokens) {
        tiles.push_back({s, (int32_t)row, h, n, h + n, true});
      } else {
        for (int32_t i = 0; i < n; i += pre_tokens) {
          const int32_t nq = std::min(pre_tokens, n - i);
          tiles.push_back({s, (int32_t)(row + i), h + i, nq, h + i + nq, false});
        }
      }
    }
    row += n;
  }
  // Shared-prefix cascade (bf16 KV, head_dim 128): a declared group's decode
  // members (one new token, history covering the shared prefix) leave the
  // prefix to cascade items; a group needs at least two such members.
  std::vector<std::vector<int32_t>> group_tiles;
  if (groups && groups->num_groups > 0 && c->dtype == PA_KV_BF16 && d == 128) {
    group_tiles.resize(groups->num_groups);
    for (size_t i = 0; i < tiles.size(); i++) {
      const Tile &t = tiles[i];
      const int32_t g = groups->group_of[t.seq];
      if (!t.decode || t.nq != 1 || g < 0) continue;
      const int32_t L = groups->group_len[g];
      if (L > 0 && hist[t.seq] >= L) group_tiles[g].push_back((int32_t)i);
    }
    for (auto &v : group_tiles)
      if (v.size() >= 2)
        for (int32_t i : v) tiles[i].shared = groups->group_len[groups->group_of[tiles[i].seq]];
      else
        v.clear();
  }
  int64_t wd = 0, wp = 0, np0 = 0;
  for (const Tile &t : tiles) {
    if (t.decode)
      wd += (int64_t)t.keys * hkv;
    else {
      wp += (int64_t)t.keys * hkv;
      np0 += hkv;
    }
  }
  const int64_t dchunk = decode_chunk(tiles, hkv, M.cus, wd);
  int64_t pchunk = INT32_MAX;
  if (np0 > 0 && np0 < prefill_target_items)
    pchunk = std::max<int64_t>(kPrefillMinChunk, cdiv64(wp, prefill_target_items));

  const bool persistent = tile_rows == kDmaTileRows;
  // co-scheduling: head_dim 128 (the LDS-DMA prefill and decode kernels);
  // in the one-launch step, some work-groups take decode items first
  int64_t shared_keys = 0;
  for (const auto &v : group_tiles)
    if (!v.empty()) shared_keys += tiles[v[0]].shared;
  const int64_t key_bytes = c->dtype == PA_KV_MXFP4 ? 2 * (d / 2 + d / 32) : c->dtype == PA_KV_FP8_E4M3 ? 2 * d : 4 * d;
  const CoRates &rates = c->dtype == PA_KV_MXFP4 ? kCoRatesMxfp4 : c->dtype == PA_KV_FP8_E4M3 ? kCoRatesE4m3 : kCoRatesBf16;
  const int32_t co = persistent ? choose_overlap_cus(tiles, shared_keys, hkv, key_bytes, rates, M) : -1;
  if (persistent) {
    MachineShape Mp = M;
    Mp.cus -= std::max(co, 0);
    plan_persistent(tiles, hkv, tile_rows, Mp, P, step ? kStepRangesPerCu : 1);
    if (step)
      P.step_decode_cus = std::max(co, 0);
    else if (co >= 0 && !P.wg_first.empty())  // the decode takes every CU the prefill launch does not hold
      P.overlap_cus = std::max(0, M.cus - ((int32_t)P.wg_first.size() - 1));
  }
  std::vector<std::vector<Item>> pre_by_head(hkv);
  std::vector<std::pair<int32_t, int32_t>> ranges;
  // cascade members: the first partial slot of tile i's KV head kvh (its
  // shared-prefix chunks come first, then its suffix items)
  std::vector<int32_t> member_part0;
  if (!group_tiles.empty()) member_part0.assign(tiles.size() * hkv, -1);
  for (size_t ti = 0; ti < tiles.size(); ti++) {
    const Tile &t = tiles[ti];
    if (persistent && !t.decode) continue;
    const int64_t chunk = t.decode ? dchunk : pchunk;
    int32_t nsh = 0;  // shared-prefix chunks (cascade items) ahead of this tile's own ranges
    if (t.shared > 0) {
      nsh = (int32_t)cdiv64(t.shared, chunk);
      cut(t.keys - t.shared, (int32_t)cdiv64(t.keys - t.shared, chunk), ranges);
      for (auto &r : ranges) r.first += t.shared, r.second += t.shared;
    } else {
      const int32_t nsplit = (int32_t)std::min<int64_t>(cdiv64(t.keys, chunk), INT32_MAX);
      cut(t.keys, nsplit, ranges);
    }
    for (int32_t kvh = 0; kvh < hkv; kvh++) {
      int32_t part0 = -1;
      const int32_t nparts = nsh + (int32_t)ranges.size();
      if (nparts > 1) {
        int64_t &np = t.decode ? P.n_part_decode : P.n_part_prefill;
        part0 = (int32_t)np;
        np += (int64_t)nparts;
        P.merges.push_back({t.row0, t.nq, kvh, part0, nparts,
                            t.decode ? kDecodeRows : tile_rows, t.decode ? 1 : 0, 0});
      }
      if (nsh > 0) member_part0[ti * hkv + kvh] = part0;
      for (size_t i = 0; i < ranges.size(); i++) {
        Item it{t.seq, kvh, t.row0, t.pos0, t.nq, ranges[i].first, ranges[i].second,
                part0 < 0 ? -1 : part0 + nsh + (int32_t)i};
        if (t.decode)
          P.decode.push_back(it);
        else
          pre_by_head[kvh].push_back(it);
      }
    }
  }
  // Longest items first; prefill items of one KV head are interleaved with
  // stride hkv so that consecutive work-group ids (dispatched round-robin
  // over the XCDs) keep one KV head's tiles on one XCD's L2 when hkv == 8.
  auto cost = [](const Item &x) { return (int64_t)(x.kv_hi - x.kv_lo) * (x.nq > 0 ? 1 : 0); };
  auto longer = [&](const Item &x, const Item &y) { return cost(x) > cost(y); };
  for (auto &v : pre_by_head) std::stable_sort(v.begin(), v.end(), longer);
  size_t maxlen = 0;
  for (auto &v : pre_by_head) maxlen = std::max(maxlen, v.size());
  for (size_t i = 0; i < maxlen; i++)
    for (int32_t k = 0; k < hkv; k++)
      if (i < pre_by_head[k].size()) P.prefill.push_back(pre_by_head[k][i]);
  std::stable_sort(P.decode.begin(), P.decode.end(), longer);

  // cascade items: per group, KV head, shared-prefix chunk and run of up to
  // kCascadeRows / G members
  const int32_t max_members = kCascadeRows / group;
  for (const auto &v : group_tiles) {
    if (v.empty()) continue;
    const Tile &t0 = tiles[v[0]];
    std::vector<std::pair<int32_t, int32_t>> sh;
    cut(t0.shared, (int32_t)cdiv64(t0.shared, dchunk), sh);
    for (int32_t kvh = 0; kvh < hkv; kvh++)
      for (size_t c = 0; c < sh.size(); c++)
        for (size_t m0 = 0; m0 < v.size(); m0 += max_members) {
          const int32_t nm = (int32_t)std::min<size_t>(max_members, v.size() - m0);
          P.cascade.push_back({t0.seq, kvh, sh[c].first, sh[c].second, (int32_t)P.members.size(), nm, {0, 0}});
          for (int32_t k = 0; k < nm; k++) {
            const int32_t ti = v[m0 + k];
            P.members.push_back({tiles[ti].row0, member_part0[ti * hkv + kvh] + (int32_t)c});
          }
          P.cascade_rows = std::max(P.cascade_rows, nm * group);
        }
  }

  // merges with many parts last (they take the one-row-per-work-group kernel)
  std::stable_partition(P.merges.begin(), P.merges.end(),
                        [](const Merge &m) { return m.nparts <= kMergeSerialParts; });

  if (step) {
    // prefill ranges: the persistent plan's work-group ranges (or one item
    // each); range w was cut for XCD w % xcds, so XCD x's queue holds the
    // ranges w = x, x + xcds, ...
    if (P.wg_first.empty() && !P.prefill.empty())
      for (int32_t i = 0; i <= (int32_t)P.prefill.size(); i++) P.wg_first.push_back(i);
    P.step_ranges = P.wg_first.empty() ? 0 : (int32_t)P.wg_first.size() - 1;
    const int32_t xq = std::min(M.xcds, kMaxXcds);
    P.step_xcds = P.step_ranges > 0 && P.step_ranges % xq == 0 ? xq : 1;
    P.step_queue_off.assign(kMaxXcds + 1, 0);
    for (int32_t x = 0; x < P.step_xcds; x++) {
      P.step_queue_off[x] = (int32_t)P.step_queue.size();
      for (int32_t w = x; w < P.step_ranges; w += P.step_xcds) P.step_queue.push_back(w);
    }
    for (int32_t x = P.step_xcds; x <= kMaxXcds; x++) P.step_queue_off[x] = (int32_t)P.step_queue.size();
    P.step_pre_merge.assign((size_t)P.n_part_prefill, -1);
    P.step_dec_merge.assign((size_t)P.n_part_decode, -1);
    for (size_t m = 0; m < P.merges.size(); m++) {
      auto &v = P.merges[m].is_decode ? P.step_dec_merge : P.step_pre_merge;
      for (int32_t i = 0; i < P.merges[m].nparts; i++) v[(size_t)P.merges[m].part0 + i] = (int32_t)m;
    }
    P.n_ctr = (size_t)kCtrMerge + P.merges.size();
  }

  size_t off = 0;
  P.off_prefill = off;
  off = align256(off + P.prefill.size() * sizeof(Item));
  P.off_decode = off;
  off = align256(off + P.decode.size() * sizeof(Item));
  P.off_merges = off;
  off = align256(off + P.merges.size() * sizeof(Merge));
  P.off_wg = off;
  off = align256(off + P.wg_first.size() * sizeof(int32_t));
  P.off_cascade = off;
  off = align256(off + P.cascade.size() * sizeof(CascadeItem));
  P.off_members = off;
  off = align256(off + P.members.size() * sizeof(CascadeMember));
  P.off_sq = off;
  off = align256(off + P.step_queue.size() * sizeof(int32_t));
  P.off_sqo = off;
  off = align256(off + P.step_queue_off.size() * sizeof(int32_t));
  P.off_spm = off;
  off = align256(off + P.step_pre_merge.size() * sizeof(int32_t));
  P.off_sdm = off;
  off = align256(off + P.step_dec_merge.size() * sizeof(int32_t));
  P.off_ctr = off;
  off = align256(off + P.n_ctr * sizeof(uint32_t));  // zeros in the staged copy
  P.off_claim = off;
  off = align256(off + (P.overlap_cus > 0 ? sizeof(uint32_t) : 0));  // decode claim counter, zero
  P.plan_bytes = off;
  P.off_po_pre = off;
  off = align256(off + (size_t)P.n_part_prefill * tile_rows * d * sizeof(float));
  P.off_pl_pre = off;
  off = align256(off + (size_t)P.n_part_prefill * tile_rows * sizeof(float));
  P.off_po_dec = off;
  off = align256(off + (size_t)P.n_part_decode * kDecodeRows * d * sizeof(float));
  P.off_pl_dec = off;
  off = align256(off + (size_t)P.n_part_decode * kDecodeRows * sizeof(float));
  P.total = off;
}

pa_status check_lengths(const int32_t *hist, const int32_t *incr, int32_t num_seqs,
                        int32_t num_q_heads, const pa_kv_cache *c, int32_t max_blocks,
                        bool check_table, int64_t *total_q_out) {
  if (num_seqs < 0) return fail(PA_ERR_BAD_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 0 && (!hist || !incr)) return fail(PA_ERR_NULL_ARG, "hist_lens/incr_lens is NULL");
  if (num_q_heads <= 0 || num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_BAD_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, c->num_kv_heads);
  const int group = num_q_heads / c->num_kv_heads;
  if (log2_exact(group) < 0 || group > 16)
    return fail(PA_ERR_UNSUPPORTED, "GQA group size %d not supported (1, 2, 4, 8, 16)", group);
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; s++) {
    if (hist[s] < 0 || incr[s] < 0)
      return fail(PA_ERR_BAD_SHAPE, "sequence %d: negative length (hist %d, incr %d)", s, hist[s],
                  incr[s]);
    const int64_t ctx = (int64_t)hist[s] + incr[s];
    if (ctx > INT32_MAX - kKeyTile) return fail(PA_ERR_BAD_SHAPE, "sequence %d: context too long", s);
    if (check_table && incr[s] > 0 && ctx > (int64_t)max_blocks * c->block_size)
      return fail(PA_ERR_BAD_SHAPE,
                  "sequence %d: context %lld exceeds its block table (%d blocks of %d)", s,
                  (long long)ctx, max_blocks, c->block_size);
    total += incr[s];
  }
  if (total >= INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "total query rows %lld too large", (long long)total);
  *total_q_out = total;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Pinned staging ring for work lists (one per device).  A slot is reused only
// after the kernel that last read it has completed.
struct StageSlot {
  void *host = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};
struct DeviceStage {
  int device = -1;
  std::vector<StageSlot> slots;
  size_t next = 0;
};
std::mutex g_stage_mu;
std::vector<DeviceStage> g_stages;

pa_status stage_copy(const void *src, size_t bytes, void *dst_dev, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_stage_mu);
  DeviceStage *ds = nullptr;
  for (auto &x : g_stages)
    if (x.device == dev) ds = &x;
  if (!ds) {
    g_stages.push_back(DeviceStage{});
    ds = &g_stages.back();
    ds->device = dev;
    ds->slots.resize(8);
  }
  StageSlot &sl = ds->slots[ds->next];
  ds->next = (ds->next + 1) % ds->slots.size();
  if (sl.pending) {
    e = hipEventSynchronize(sl.done);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    sl.pending = false;
  }
  if (!sl.done) {
    e = hipEventCreateWithFlags(&sl.done, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate(staging)");
  }
  if (sl.cap < bytes) {
    if (sl.host) (void)hipHostFree(sl.host);
    sl.host = nullptr;
    sl.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 1 << 20);
    e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail(e, "hipHostMalloc(staging)");
    sl.cap = cap;
  }
  memcpy(sl.host, src, bytes);
  // a kernel on the call's stream reads the pinned slot (no copy engine, so
  // no hand-off between engines before the attention kernels)
  void *src_dev = nullptr;
  e = hipHostGetDevicePointer(&src_dev, sl.host, 0);
  if (e != hipSuccess) return hip_fail(e, "hipHostGetDevicePointer(staging)");
  e = launch_stage(src_dev, dst_dev, bytes, stream);
  if (e != hipSuccess) return hip_fail(e, "work-list copy launch");
  e = hipEventRecord(sl.done, stream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(staging)");
  sl.pending = true;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Scratch of paged_attn_forward_noalloc: a static device array, one copy per
// device the library runs on, held until the process ends.  Host code never
// uses the array's name as an address (in host code it is only a stand-in for
// the symbol): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.  Its contents need no initialisation
// (the work list is copied in by each call; every partial result is written
// before it is read), and calls that overlap on one device share it and race.
// (the array itself: file scope, above)

struct DeviceScratch {
  int device;
  unsigned char *ptr;
};
std::mutex g_scratch_mu;
std::vector<DeviceScratch> g_scratch;

pa_status scratch_address(unsigned char **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  for (const auto &d : g_scratch)
    if (d.device == dev) {
      *out = d.ptr;
      return PA_OK;
    }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
  g_scratch.push_back({dev, (unsigned char *)p});
  *out = (unsigned char *)p;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// The second stream of a co-scheduled mixed step: one per device, created on
// first use (default priority, non-blocking), with the two events that fork
// it from the call's stream and join it back.  A call holds g_co_mu from the
// fork to the join, so calls from several host threads do not interleave on
// the shared events.
struct CoStream {
  int device;
  hipStream_t s2;
  hipEvent_t fork, join;
};
std::mutex g_co_mu;
std::vector<CoStream> g_co;

pa_status co_stream(CoStream *out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  for (const auto &c : g_co)
    if (c.device == dev) {
      *out = c;
      return PA_OK;
    }
  CoStream c{dev, nullptr, nullptr, nullptr};
  e = hipStreamCreateWithFlags(&c.s2, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c.fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c.join, hipEventDisableTiming);
  if (e != hipSuccess) {
    if (c.join) (void)hipEventDestroy(c.join);
    if (c.fork) (void)hipEventDestroy(c.fork);
    if (c.s2) (void)hipStreamDestroy(c.s2);
    return hip_fail(e, "co-scheduling stream");
  }
  g_co.push_back(c);
  *out = c;
  return PA_OK;
}

// ---------------------------------------------------------------------------
// Optional per-kernel timing with HIP events on the launch stream.
constexpr int kKinds = 5;
std::mutex g_time_mu;
bool g_timing = false;
struct TimedLaunch {
  hipEvent_t a, b;
};
std::vector<TimedLaunch> g_pending[kKinds];
std::vector<hipEvent_t> g_event_pool;

hipEvent_t get_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
hipError_t timed(int kind, hipStream_t s, F &&launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    on = g_timing;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    a = get_event();
    b = get_event();
  }
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_time_mu);
  g_pending[kind].push_back({a, b});
  return hipSuccess;
}

}  // namespace

// =============================================================================
extern "C" {

const char *pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_time_mu);
  g_timing = enable != 0;
  return PA_OK;
}

pa_status pa_timing_read(int kind, double *ms, int64_t *count) {
  if (kind < 0 || kind >= kKinds) return fail(PA_ERR_BAD_SHAPE, "timing kind %d", kind);
  if (!ms || !count) return fail(PA_ERR_NULL_ARG, "ms/count is NULL");
  std::vector<TimedLaunch> pend;
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    pend.swap(g_pending[kind]);
  }
  double sum = 0;
  for (auto &p : pend) {
    hipError_t e = hipEventSynchronize(p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(timing)");
    float t = 0;
    e = hipEventElapsedTime(&t, p.a, p.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sum += t;
  }
  {
    std::lock_guard<std::mutex> lk(g_time_mu);
    for (auto &p : pend) {
      g_event_pool.push_back(p.a);
      g_event_pool.push_back(p.b);
    }
  }
  *ms = sum;
  *count = (int64_t)pend.size();
  return PA_OK;
}

pa_status kv_append(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, int32_t num_tokens, void *stream) {
  pa_status st = check_cache(cache);
  if (st) return st;
  if (num_tokens < 0) return fail(PA_ERR_BAD_SHAPE, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_NULL_ARG, "k_new/v_new/slot_mapping is NULL");
  AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.ks = cache->k_scale;
  a.vs = cache->v_scale;
  a.hkv = cache->num_kv_heads;
  a.bs = cache->block_size;
  a.lbs = a.bs == 16 ? 4 : 6;
  a.d = cache->head_dim;
  a.lcpr = a.d == 64 ? 3 : 4;
  const int fmt = (int)cache->dtype;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed(0, s, [&] { return launch_append(a, fmt, num_tokens, s); });
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return PA_OK;
}

size_t pa_workspace_size(const int32_t *hist_lens, const int32_t *incr_lens, int32_t num_seqs,
                         int32_t num_q_heads, const pa_kv_cache *cache) {
  if (check_cache(cache)) return 0;
  int64_t total_q = 0;
  if (check_lengths(hist_lens, incr_lens, num_seqs, num_q_heads, cache, 0, false, &total_q))
    return 0;
  Plan P;
  make_plan(hist_lens, incr_lens, num_seqs, cache, num_q_heads / cache->num_kv_heads, P);
  return std::max<size_t>(P.total, 256);
}

}  // extern "C"

namespace {

// Validation, planning and launches shared by both forward entry points.
// workspace == nullptr: the static scratch (no allocation anywhere: the work
// list goes in by a stream-ordered copy from host memory instead of through
// the pinned staging ring, which is allocated on first use).
pa_status forward(const void *q, const pa_kv_cache *cache, const int32_t *block_tables,
                  int32_t max_blocks_per_seq, const int32_t *hist_lens, const int32_t *incr_lens,
                  int32_t num_seqs, int32_t num_q_heads, float scale, void *out, float *lse_out,
                  void *workspace, size_t workspace_bytes, void *stream, bool no_alloc,
                  const Groups *groups = nullptr, size_t *size_query = nullptr, const StepIn *step = nullptr) {
  pa_status st = check_cache(cache);
  if (st) return st;
  if (max_blocks_per_seq < 0) return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_seq < 0");
  int64_t total_q = 0;
  st = check_lengths(hist_lens, incr_lens, num_seqs, num_q_heads, cache, max_blocks_per_seq, true,
                     &total_q);
  if (st) return st;
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(PA_ERR_BAD_SHAPE, "scale must be finite and > 0 (got %g)", (double)scale);
  if (groups) {
    if (groups->num_groups < 0) return fail(PA_ERR_BAD_SHAPE, "num_groups %d < 0", groups->num_groups);
    if (groups->num_groups > 0 && (!groups->group_of || !groups->group_len))
      return fail(PA_ERR_NULL_ARG, "group_of/group_len is NULL");
    for (int32_t g = 0; g < groups->num_groups; g++)
      if (groups->group_len[g] < 0 || groups->group_len[g] % cache->block_size != 0)
        return fail(PA_ERR_BAD_SHAPE, "group %d: shared length %d is not a non-negative multiple of the block size %d",
                    g, groups->group_len[g], cache->block_size);
    for (int32_t s = 0; s < num_seqs && groups->num_groups > 0; s++)
      if (groups->group_of[s] < -1 || groups->group_of[s] >= groups->num_groups)
        return fail(PA_ERR_BAD_SHAPE, "sequence %d: group %d out of range", s, groups->group_of[s]);
  }
  if (step && cache->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "the one-launch step takes head_dim 128 (got %d)", cache->head_dim);
  const int32_t hkv = cache->num_kv_heads, group = num_q_heads / hkv, d = cache->head_dim;
  Plan P;
  const int32_t tile_rows = prefill_tile_rows(cache);
  if (size_query) {
    make_plan(hist_lens, incr_lens, num_seqs, cache, group, P, groups, step != nullptr);
    *size_query = std::max<size_t>(P.total, 256);
    return PA_OK;
  }
  if (total_q == 0) return PA_OK;
  if (!q || !out || !block_tables) return fail(PA_ERR_NULL_ARG, "q/out/block_tables is NULL");
  if (step && (!step->k_new || !step->v_new || !step->slots))
    return fail(PA_ERR_NULL_ARG, "k_new/v_new/slot_mapping is NULL");
  if (step && total_q * hkv * (d / 8) >= ((int64_t)1 << 31))
    return fail(PA_ERR_BAD_SHAPE, "too many new tokens for one step (%lld)", (long long)total_q);
  make_plan(hist_lens, incr_lens, num_seqs, cache, group, P, groups, step != nullptr);
  if (no_alloc) {
    if (P.total > (size_t)PA_NOALLOC_SCRATCH_BYTES)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                  "this step needs %zu bytes of scratch, more than the %zu of the no-allocation entry point "
                  "(use paged_attn_forward with a workspace)",
                  P.total, (size_t)PA_NOALLOC_SCRATCH_BYTES);
    unsigned char *sp = nullptr;
    st = scratch_address(&sp);
    if (st) return st;
    workspace = sp;
    workspace_bytes = PA_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace) return fail(PA_ERR_NULL_ARG, "workspace is NULL");
  if ((uintptr_t)workspace % 256 != 0) return fail(PA_ERR_BAD_SHAPE, "workspace not 256-byte aligned");
  if (workspace_bytes < P.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                P.total);

  std::vector<unsigned char> host(P.plan_bytes, 0);
  if (!P.prefill.empty()) memcpy(host.data() + P.off_prefill, P.prefill.data(), P.prefill.size() * sizeof(Item));
  if (!P.decode.empty()) memcpy(host.data() + P.off_decode, P.decode.data(), P.decode.size() * sizeof(Item));
  if (!P.merges.empty()) memcpy(host.data() + P.off_merges, P.merges.data(), P.merges.size() * sizeof(Merge));
  if (!P.wg_first.empty())
    memcpy(host.data() + P.off_wg, P.wg_first.data(), P.wg_first.size() * sizeof(int32_t));
  if (!P.cascade.empty()) {
    memcpy(host.data() + P.off_cascade, P.cascade.data(), P.cascade.size() * sizeof(CascadeItem));
    memcpy(host.data() + P.off_members, P.members.data(), P.members.size() * sizeof(CascadeMember));
  }
  auto put = [&](size_t off, const std::vector<int32_t> &v) {
    if (!v.empty()) memcpy(host.data() + off, v.data(), v.size() * sizeof(int32_t));
  };
  put(P.off_sq, P.step_queue);
  put(P.off_sqo, P.step_queue_off);
  put(P.off_spm, P.step_pre_merge);
  put(P.off_sdm, P.step_dec_merge);  // (the counters stay zero)
  hipStream_t s = (hipStream_t)stream;
  unsigned char *ws = (unsigned char *)workspace;
  // the co-scheduling stream is made (once per device) before anything is
  // enqueued, so a failure there leaves everything untouched
  const bool coschedule = P.overlap_cus > 0 && !no_alloc;
  CoStream co{};
  if (coschedule) {
    std::lock_guard<std::mutex> lk(g_co_mu);
    st = co_stream(&co);
    if (st) return st;
  }
  if (no_alloc) {
    hipError_t e = hipMemcpyAsync(ws, host.data(), P.plan_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "work-list copy");
  } else {
    st = stage_copy(host.data(), P.plan_bytes, ws, s);
    if (st) return st;
  }
  AttnArgs a{};
  a.q = q;
  a.c.k = cache->k_cache;
  a.c.v = cache->v_cache;
  a.c.ks = cache->k_scale;
  a.c.vs = cache->v_scale;
  a.c.num_blocks = cache->num_blocks;
  a.c.hkv = hkv;
  a.bt = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.hq = num_q_heads;
  a.group = group;
  a.tile_rows = tile_rows;
  a.lg = log2_exact(group);
  a.scale_log2 = scale * 1.44269504088896341f;
  a.out = out;
  a.lse_out = lse_out;
  const int fmt = (int)cache->dtype;
  const int bs = cache->block_size;
  hipError_t e;
  MergeArgs m{};
  m.merges = (const Merge *)(ws + P.off_merges);
  m.part_o_prefill = (const float *)(ws + P.off_po_pre);
  m.part_lse_prefill = (const float *)(ws + P.off_pl_pre);
  m.part_o_decode = (const float *)(ws + P.off_po_dec);
  m.part_lse_decode = (const float *)(ws + P.off_pl_dec);
  m.out = out;
  m.lse_out = lse_out;
  m.hq = num_q_heads;
  m.group = group;
  m.lg = a.lg;
  m.d = d;
  if (step) {
    StepArgs sa{};
    sa.pre = a;
    sa.pre.items = (const Item *)(ws + P.off_prefill);
    sa.pre.part_o = (float *)(ws + P.off_po_pre);
    sa.pre.part_lse = (float *)(ws + P.off_pl_pre);
    sa.dec = a;
    sa.dec.items = (const Item *)(ws + P.off_decode);
    sa.dec.part_o = (float *)(ws + P.off_po_dec);
    sa.dec.part_lse = (float *)(ws + P.off_pl_dec);
    sa.app.k_new = step->k_new;
    sa.app.v_new = step->v_new;
    sa.app.slots = step->slots;
    sa.app.k_cache = cache->k_cache;
    sa.app.v_cache = cache->v_cache;
    sa.app.ks = cache->k_scale;
    sa.app.vs = cache->v_scale;
    sa.app.hkv = hkv;
    sa.app.bs = bs;
    sa.app.lbs = bs == 16 ? 4 : 6;
    sa.app.d = d;
    sa.app.lcpr = d == 64 ? 3 : 4;
    sa.app.tok0 = 0;
    sa.app.nchunks = (uint32_t)(total_q * hkv * (d / 8));
    sa.mg = m;
    sa.wg_first = (const int32_t *)(ws + P.off_wg);
    sa.pre_queue = (const int32_t *)(ws + P.off_sq);
    sa.pre_queue_off = (const int32_t *)(ws + P.off_sqo);
    sa.pre_part_merge = (const int32_t *)(ws + P.off_spm);
    sa.dec_part_merge = (const int32_t *)(ws + P.off_sdm);
    sa.ctr = (uint32_t *)(ws + P.off_ctr);
    sa.n_append_tasks = (int32_t)((sa.app.nchunks + kStepAppendChunks - 1) / kStepAppendChunks);
    sa.n_decode = (int32_t)P.decode.size();
    sa.xcds = P.step_xcds;
    sa.decode_first = P.step_xcds > 1 ? P.step_decode_cus / P.step_xcds : P.step_decode_cus;
    const int64_t tasks = (int64_t)sa.n_append_tasks + P.step_ranges + sa.n_decode;
    const int groups_n = (int)std::max<int64_t>(1, std::min<int64_t>(machine_shape().cus, tasks));
    e = timed(4, s, [&] { return launch_step(sa, groups_n, bs, fmt, s); });
    if (e != hipSuccess) return hip_fail(e, "step launch");
    return PA_OK;
  }
  if (coschedule) {
    // Co-scheduled mixed step: the persistent prefill (its ranges cut for
    // the CUs it leaves to the decode) on the call's stream; beside it, on
    // the second stream, overlap_cus work-groups claim the decode launch's
    // items (shared-prefix cascade items first, if any) from the list; after
    // the prefill, work-groups on the CUs it frees claim the rest.  Each CU holds one work-group of either kernel (registers and
    // LDS), and work-groups are dispatched round-robin over the XCDs, so the
    // decode takes overlap_cus / xcds CUs of every XCD.  The merges follow
    // the join.  (The no-allocation entry point runs the same plan's
    // launches one after the other: same items, same results.)
    AttnArgs ap = a;
    ap.items = (const Item *)(ws + P.off_prefill);
    ap.part_o = (float *)(ws + P.off_po_pre);
    ap.part_lse = (float *)(ws + P.off_pl_pre);
    ap.wg_first = (const int32_t *)(ws + P.off_wg);
    const int n_pre = (int)P.wg_first.size() - 1;
    AttnArgs ad = a;
    ad.items = (const Item *)(ws + P.off_decode);
    ad.wg_first = nullptr;
    ad.part_o = (float *)(ws + P.off_po_dec);
    ad.part_lse = (float *)(ws + P.off_pl_dec);
    uint32_t *ctr = (uint32_t *)(ws + P.off_claim);
    const int n_dec = (int)P.decode.size();
    const CascadeItem *citems = (const CascadeItem *)(ws + P.off_cascade);
    const CascadeMember *members = (const CascadeMember *)(ws + P.off_members);
    const int n_casc = (int)P.cascade.size();
    const int tail = std::max(1, machine_shape().cus - P.overlap_cus);
    std::lock_guard<std::mutex> lk(g_co_mu);
    if ((e = hipEventRecord(co.fork, s)) != hipSuccess) return hip_fail(e, "fork event");
    if ((e = hipStreamWaitEvent(co.s2, co.fork, 0)) != hipSuccess) return hip_fail(e, "fork wait");
    e = timed(1, s, [&] { return launch_prefill(ap, n_pre, d, bs, fmt, s); });
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
    e = timed(2, co.s2, [&] {
      return launch_decode_claim(ad, ctr, n_dec, citems, members, n_casc, P.cascade_rows, P.overlap_cus, bs, fmt,
                                 co.s2);
    });
    if (e != hipSuccess) return hip_fail(e, "decode attention launch (beside the prefill)");
    e = timed(2, s, [&] {
      return launch_decode_claim(ad, ctr, n_dec, citems, members, n_casc, P.cascade_rows, tail, bs, fmt, s);
    });
    if (e != hipSuccess) return hip_fail(e, "decode attention launch (after the prefill)");
    if ((e = hipEventRecord(co.join, co.s2)) != hipSuccess) return hip_fail(e, "join event");
    if ((e = hipStreamWaitEvent(s, co.join, 0)) != hipSuccess) return hip_fail(e, "join wait");
  } else if (!P.prefill.empty()) {
    AttnArgs ap = a;
    ap.items = (const Item *)(ws + P.off_prefill);
    ap.part_o = (float *)(ws + P.off_po_pre);
    ap.part_lse = (float *)(ws + P.off_pl_pre);
    ap.wg_first = P.wg_first.empty() ? nullptr : (const int32_t *)(ws + P.off_wg);
    const int n = P.wg_first.empty() ? (int)P.prefill.size() : (int)P.wg_first.size() - 1;
    e = timed(1, s, [&] { return launch_prefill(ap, n, d, bs, fmt, s); });
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  }
  if (coschedule) {
    // (the decode ran above)
  } else if (!P.cascade.empty()) {  // one launch: the cascade items, then the decode items
    a.items = (const Item *)(ws + P.off_decode);
    a.wg_first = nullptr;
    a.part_o = (float *)(ws + P.off_po_dec);
    a.part_lse = (float *)(ws + P.off_pl_dec);
    e = timed(2, s, [&] {
      return launch_decode_cascade(a, (const CascadeItem *)(ws + P.off_cascade),
                                   (const CascadeMember *)(ws + P.off_members), (int)P.cascade.size(),
                                   (int)P.decode.size(), P.cascade_rows, bs, s);
    });
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  } else if (!P.decode.empty()) {
    a.items = (const Item *)(ws + P.off_decode);
    a.wg_first = nullptr;
    a.part_o = (float *)(ws + P.off_po_dec);
    a.part_lse = (float *)(ws + P.off_pl_dec);
    const int n = (int)P.decode.size();
    e = timed(2, s, [&] { return launch_decode(a, n, d, bs, fmt, s); });
    if (e != hipSuccess) return hip_fail(e, "decode attention launch");
  }
  if (!P.merges.empty()) {
    int n_few = 0, many_rows = 0;
    for (const Merge &mg : P.merges) {
      if (mg.nparts <= kMergeSerialParts) n_few++;
      else many_rows = std::max(many_rows, mg.nq * group);
    }
    const int n_many = (int)P.merges.size() - n_few;
    e = timed(3, s, [&] { return launch_merge(m, n_few, n_many, many_rows, s); });
    if (e != hipSuccess) return hip_fail(e, "merge launch");
  }
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status paged_attn_forward(const void *q, const pa_kv_cache *cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *hist_lens, const int32_t *incr_lens,
                             int32_t num_seqs, int32_t num_q_heads, float scale, void *out,
                             float *lse_out, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return forward(q, cache, block_tables, max_blocks_per_seq, hist_lens, incr_lens, num_seqs,
                 num_q_heads, scale, out, lse_out, workspace, workspace_bytes, stream, false);
}

pa_status paged_attn_forward_cascade(const void *q, const pa_kv_cache *cache,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *hist_lens, const int32_t *incr_lens,
                                     int32_t num_seqs, int32_t num_q_heads, float scale, void *out,
                                     float *lse_out, const int32_t *group_of, const int32_t *group_len,
                                     int32_t num_groups, void *workspace, size_t *workspace_bytes,
                                     void *stream) {
  if (!workspace_bytes) return fail(PA_ERR_NULL_ARG, "workspace_bytes is NULL");
  Groups g;
  g.group_of = group_of;
  g.group_len = group_len;
  g.num_groups = num_groups;
  return forward(q, cache, block_tables, max_blocks_per_seq, hist_lens, incr_lens, num_seqs,
                 num_q_heads, scale, out, lse_out, workspace, *workspace_bytes, stream, false, &g,
                 workspace ? nullptr : workspace_bytes);
}

pa_status paged_attn_step(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                          const int64_t *slot_mapping, const void *q, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *hist_lens, const int32_t *incr_lens,
                          int32_t num_seqs, int32_t num_q_heads, float scale, void *out, float *lse_out,
                          void *workspace, size_t *workspace_bytes, void *stream) {
  if (!workspace_bytes) return fail(PA_ERR_NULL_ARG, "workspace_bytes is NULL");
  StepIn in;
  in.k_new = k_new;
  in.v_new = v_new;
  in.slots = slot_mapping;
  return forward(q, cache, block_tables, max_blocks_per_seq, hist_lens, incr_lens, num_seqs, num_q_heads,
                 scale, out, lse_out, workspace, *workspace_bytes, stream, false, nullptr,
                 workspace ? nullptr : workspace_bytes, &in);
}

pa_status pa_debug_step_flags(const void *workspace, const pa_kv_cache *cache, const int32_t *hist_lens,
                              const int32_t *incr_lens, int32_t num_seqs, int32_t num_q_heads,
                              uint32_t *flags_out, void *stream) {
  pa_status st = check_cache(cache);
  if (st) return st;
  int64_t total_q = 0;
  st = check_lengths(hist_lens, incr_lens, num_seqs, num_q_heads, cache, 0, false, &total_q);
  if (st) return st;
  if (!workspace || !flags_out) return fail(PA_ERR_NULL_ARG, "workspace/flags_out is NULL");
  Plan P;
  make_plan(hist_lens, incr_lens, num_seqs, cache, num_q_heads / cache->num_kv_heads, P, nullptr, true);
  hipError_t e = hipMemcpyAsync(flags_out, (const unsigned char *)workspace + P.off_ctr + kCtrFlags * 4, 4,
                                hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "flags copy");
  return PA_OK;
}

pa_status paged_attn_forward_noalloc(const void *q, const pa_kv_cache *cache,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *hist_lens, const int32_t *incr_lens,
                                     int32_t num_seqs, int32_t num_q_heads, float scale, void *out,
                                     float *lse_out, void *stream) {
  return forward(q, cache, block_tables, max_blocks_per_seq, hist_lens, incr_lens, num_seqs,
                 num_q_heads, scale, out, lse_out, nullptr, 0, stream, true);
}

pa_status pa_device_shape(int32_t *num_cus, int32_t *num_xcds) {
  if (!num_cus || !num_xcds) return fail(PA_ERR_NULL_ARG, "num_cus/num_xcds is NULL");
  const MachineShape m = machine_shape();
  *num_cus = m.cus;
  *num_xcds = m.xcds;
  return PA_OK;
}

pa_status pa_debug_xcc_ids(int32_t *out, int32_t n, void *stream) {
  if (!out) return fail(PA_ERR_NULL_ARG, "out is NULL");
  if (n < 1) return fail(PA_ERR_BAD_SHAPE, "n %d < 1", n);
  hipError_t e = launch_xcc_ids(out, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "xcc id launch");
  return PA_OK;
}

pa_status pa_peak_mfma(float *out, int32_t iters, void *stream) {
  if (!out) return fail(PA_ERR_NULL_ARG, "out is NULL");
  if (iters < 1) return fail(PA_ERR_BAD_SHAPE, "iters %d < 1", iters);
  hipError_t e = launch_peak_mfma(out, iters, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "peak_mfma launch");
  return PA_OK;
}

pa_status pa_peak_read(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!buf || !out) return fail(PA_ERR_NULL_ARG, "buf/out is NULL");
  if (bytes < 4096 || bytes % 4096 != 0)
    return fail(PA_ERR_BAD_SHAPE, "bytes %zu: a positive multiple of 4096 required", bytes);
  hipError_t e = launch_peak_read(buf, (int64_t)bytes, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "peak_read launch");
  return PA_OK;
}

pa_status pa_debug_gather(const pa_kv_cache *cache, const int32_t *block_table_row, int32_t ctx,
                          void *k_out, void *v_out, void *stream) {
  pa_status st = check_cache(cache);
  if (st) return st;
  if (ctx < 0) return fail(PA_ERR_BAD_SHAPE, "ctx %d < 0", ctx);
  if (ctx == 0) return PA_OK;
  if (!block_table_row || !k_out || !v_out)
    return fail(PA_ERR_NULL_ARG, "block_table_row/k_out/v_out is NULL");
  GatherArgs g{};
  g.k = cache->k_cache;
  g.v = cache->v_cache;
  g.bt_row = block_table_row;
  g.k_out = k_out;
  g.v_out = v_out;
  g.hkv = cache->num_kv_heads;
  g.bs = cache->block_size;
  g.ks = cache->k_scale;
  g.vs = cache->v_scale;
  g.fmt = (int)cache->dtype;
  g.row_bytes = cache->dtype == PA_KV_MXFP4 ? cache->head_dim / 2
                                            : cache->head_dim * (cache->dtype == PA_KV_FP8_E4M3 ? 1 : 2);
  // (MXFP4: one thread per 8 elements, i.e. per 4 bytes of codes)
  g.total_chunks = (int64_t)ctx * g.hkv * (cache->dtype == PA_KV_MXFP4 ? cache->head_dim / 8 : g.row_bytes / 16);
  hipError_t e = launch_gather(g, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return PA_OK;
}

pa_status pa_debug_overlap_cus(int32_t n) {
  g_overlap_force.store(n < 0 ? -1 : n);
  return PA_OK;
}

pa_status pa_debug_plan(const int32_t *hist_lens, const int32_t *incr_lens, int32_t num_seqs,
                        int32_t num_q_heads, const pa_kv_cache *cache, int32_t *items_out,
                        int32_t items_cap, int32_t *counts_out) {
  pa_status st = check_cache(cache);
  if (st) return st;
  int64_t total_q = 0;
  st = check_lengths(hist_lens, incr_lens, num_seqs, num_q_heads, cache, 0, false, &total_q);
  if (st) return st;
  if (!counts_out || (items_cap > 0 && !items_out)) return fail(PA_ERR_NULL_ARG, "output is NULL");
  Plan P;
  make_plan(hist_lens, incr_lens, num_seqs, cache, num_q_heads / cache->num_kv_heads, P);
  counts_out[0] = (int32_t)P.prefill.size();
  counts_out[1] = (int32_t)P.decode.size();
  counts_out[2] = (int32_t)P.merges.size();
  counts_out[3] = (int32_t)(P.n_part_prefill + P.n_part_decode);
  const size_t n = P.prefill.size() + P.decode.size();
  if (n > (size_t)std::max(items_cap, 0))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "items_cap %d, need %zu", items_cap, n);
  if (!P.prefill.empty()) memcpy(items_out, P.prefill.data(), P.prefill.size() * sizeof(Item));
  if (!P.decode.empty())
    memcpy(items_out + 8 * P.prefill.size(), P.decode.data(), P.decode.size() * sizeof(Item));
  return PA_OK;
}

pa_status pa_debug_plan_groups(const int32_t *hist_lens, const int32_t *incr_lens,
                               int32_t num_seqs, int32_t num_q_heads, const pa_kv_cache *cache,
                               int32_t *first_out, int32_t cap, int32_t *num_groups_out) {
  pa_status st = check_cache(cache);
  if (st) return st;
  int64_t total_q = 0;
  st = check_lengths(hist_lens, incr_lens, num_seqs, num_q_heads, cache, 0, false, &total_q);
  if (st) return st;
  if (!num_groups_out || (cap > 0 && !first_out)) return fail(PA_ERR_NULL_ARG, "output is NULL");
  Plan P;
  make_plan(hist_lens, incr_lens, num_seqs, cache, num_q_heads / cache->num_kv_heads, P);
  const int32_t n = P.wg_first.empty() ? 0 : (int32_t)P.wg_first.size() - 1;
  *num_groups_out = n;
  if (n == 0) return PA_OK;
  if (n + 1 > cap) return fail(PA_ERR_WORKSPACE_TOO_SMALL, "cap %d, need %d", cap, n + 1);
  memcpy(first_out, P.wg_first.data(), (size_t)(n + 1) * sizeof(int32_t));
  return PA_OK;
}

}  // extern "C"
