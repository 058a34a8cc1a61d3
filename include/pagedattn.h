/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged-KV GQA attention library.
 *
 * One scheduler step of one attention layer is two calls, in this order:
 *   1. kv_append           scatter the step's new K/V tokens into their cache
 *                          slots;
 *   2. paged_attn_forward  every new query token attends to its sequence's
 *                          cached history plus, causally, the new tokens.
 *
 * Pages cited (title, then section):
 *   [Agentic] "vLLM Agentic 推理｜面向 Agent 负载的推理优化"
 *   [AMPD]    "ICML'26 | AMPD：PD 分离遇上多轮推理，incremental prefill 到底该在哪跑"
 *   [V1Sched] "vLLM/V1 推理调度器"
 *   [V41]     "vLLM 优化 DeepSeek-V4.1-Flash：智能体吞吐提升 5 倍"
 *
 * The pages state the problem, not the formula or the layout; the readings
 * taken here are: scaled dot-product softmax attention, causal mask with an
 * inclusive boundary (a query at absolute position p sees keys 0..p), query
 * head h reads KV head h / (num_q_heads / num_kv_heads), cache layout
 * [num_blocks][num_kv_heads][block_size][head_dim], OCP E4M3 ("e4m3fn") for
 * 8-bit KV with one fp32 scale per (physical block, KV head), OCP MXFP4 for
 * 4-bit KV (E2M1 codes, one E8M0 scale per 32 elements of a token and head).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless marked HOST.  All tensors are dense
 *     row-major.  The caller owns and allocates every buffer; the library
 *     keeps only a small pinned host staging ring for work lists.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are asynchronous and ordered on `stream`; host arrays may be
 *     reused as soon as a call returns.
 *   - Every argument is validated on the host before anything is enqueued.
 *     A non-OK status means nothing was enqueued and nothing was written;
 *     pa_last_error() describes why.  PA_ERR_HIP reports a failed HIP call
 *     (outputs are then undefined).
 *   - Device *contents* are trusted: block ids outside [0, num_blocks),
 *     duplicate slots, or tables shorter than cdiv(ctx, block_size) are
 *     caller bugs with undefined results.
 *   - The library never aborts the process.
 *
 * Supported domain: head_dim in {64, 128}; block_size in {16, 64};
 * num_q_heads % num_kv_heads == 0 with group size in {1, 2, 4, 8, 16};
 * q and out bf16; KV bf16, E4M3 or MXFP4 (MXFP4: head_dim 128 only).
 * Element offsets are 64-bit throughout.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_ARG = 1,
  PA_ERR_BAD_SHAPE = 2,
  PA_ERR_UNSUPPORTED = 3,
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_HIP = 5
} pa_status;

typedef enum { PA_KV_BF16 = 0, PA_KV_FP8_E4M3 = 1, PA_KV_MXFP4 = 2 } pa_kv_dtype;

/* The paged KV cache: a pool of physical blocks, each holding block_size
 * consecutive token positions of one sequence for every KV head
 * ([V1Sched] 源码片段 "KVCacheManager.allocate_slots — 块容量": a request
 * needs cdiv(tokens, block_size) blocks; "Scheduler.schedule — 记账与状态":
 * each request holds a list of block ids; blocks may be shared).
 *   k_cache, v_cache  [num_blocks][num_kv_heads][block_size][head_dim],
 *                     bf16 (2 bytes) or E4M3 codes (1 byte) per element;
 *                     MXFP4: [num_blocks][num_kv_heads][block_size][head_dim/2]
 *                     bytes, element 2i in the low and 2i+1 in the high 4 bits
 *                     of byte i (OCP MX E2M1 codes).
 *   k_scale, v_scale  E4M3: fp32 [num_blocks][num_kv_heads]; stored value =
 *                     decode(code) * scale; every scale a block in use has is
 *                     a positive, finite, normal fp32 number.
 *                     MXFP4: uint8 E8M0 [num_blocks][num_kv_heads][head_dim/32]
 *                     [block_size], the scale 2^(byte - 127) (255 = NaN) of 32
 *                     consecutive elements of one token and head; stored
 *                     value = E2M1(code) * scale.  kv_append writes them.
 *                     NULL iff dtype == PA_KV_BF16.
 * ([V41] "SWA 有界重放" and the kernels section keep KV in FP8, and in FP4
 * for the long-lived part, to cut its footprint; MXFP4 is OCP's 4-bit format
 * with power-of-two scales, which gfx950 widens to bf16 exactly in one
 * instruction per two elements.  MXFP4 needs head_dim 128.) */
typedef struct {
  void *k_cache;
  void *v_cache;
  void *k_scale;
  void *v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  pa_kv_dtype dtype;
} pa_kv_cache;

/*
 * kv_append -- write the step's new K/V tokens into their cache slots.
 *
 * [Agentic] §5.2: within a decode layer the KV write happens before the
 * attention reads the cache.  [AMPD] §7: the increment's KV is concatenated
 * onto the history already held locally; only the increment moves.
 *
 *   k_new, v_new   bf16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping   int64 [num_tokens]; slot = physical_block * block_size +
 *                  offset; a negative slot skips the token.
 * For token t with slot >= 0 and every KV head h:
 *   bf16:  cache[slot / bs][h][slot % bs][:] = new[t][h][:]   (bit copy)
 *   E4M3:  cache[...][e] = E4M3(new[t][h][e] / scale[slot / bs][h]) where the
 *          division is the correctly rounded fp32 quotient and E4M3() rounds
 *          to nearest-even, saturating to +-448 (NaN -> NaN).  The scales are
 *          inputs and never modified.
 *   MXFP4: per group of 32 elements e = 32j .. 32j+31 of new[t][h]: scale
 *          byte E = clamp(floor(log2(max |x|)) - 2 + 127, 0, 254) (0 when all
 *          are zero), code[e] = E2M1(x[e] / 2^(E - 127)) rounded to
 *          nearest-even and saturating to +-6, sign bit = x's sign bit; a
 *          group holding a NaN or an infinity gets E = 255 and zero codes.
 *          Codes and scale bytes of the slot are written.
 * Only the named slots are written.
 * num_tokens == 0 is a no-op.
 */
PA_API pa_status kv_append(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                    const int64_t *slot_mapping, int32_t num_tokens, void *stream);

/*
 * paged_attn_forward -- attention of the step's query tokens over the paged
 * cache: incremental prefill, initial prefill and decode in one call.
 *
 * [AMPD] §1 and §3: incremental prefill processes l_incr new tokens that must
 * read the l_hist tokens already cached; initial prefill is l_hist = 0; decode
 * produces one token at a time over the whole, growing cache.  [V1Sched]
 * "实际实现" / "Scheduler.schedule": per request the scheduler knows the
 * computed-token count (hist) and the tokens scheduled this step (incr).
 *
 *   q             bf16 [total_q][num_q_heads][head_dim], total_q = sum(incr);
 *                 the rows of sequence s are rows rowstart[s] .. +incr[s]-1
 *                 with rowstart the exclusive prefix sum of incr.
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]; entries beyond
 *                 cdiv(hist + incr, block_size) are never read.
 *   hist_lens     HOST int32 [num_seqs]: tokens cached before this step.
 *   incr_lens     HOST int32 [num_seqs]: new tokens this step (1 = decode,
 *                 0 = sequence idle).  Their K/V must already be appended.
 *   scale         softmax scale applied to q.k (1/sqrt(head_dim) usually);
 *                 must be finite and > 0.
 *   out           bf16 [total_q][num_q_heads][head_dim].
 *   lse_out       optional fp32 [total_q][num_q_heads]: ln(sum_j exp(scale *
 *                 q.k_j)) over the keys the row sees; NULL to skip.
 *   workspace     device scratch of at least pa_workspace_size(...) bytes,
 *                 256-byte aligned; contents need no initialisation.  It
 *                 holds the work list and the fp32 partial results of key
 *                 ranges split across work-groups; its size depends on the
 *                 number of tiles and of compute units, not on context
 *                 length (for the prefill: at most one 384-row partial per
 *                 (tile, KV head) and work-group boundary).
 * Row i of sequence s is at position p = hist[s] + i, and
 *   out[row][h] = sum_{j<=p} softmax_j(scale * q[row][h] . K[j][h/G]) V[j][h/G].
 * With an E4M3 cache, K[j] and V[j] are code * scale of their (block, head);
 * the codes widen to bf16 exactly and the scales act in fp32 (the key scale
 * on the score, the value scale on the probability before it is rounded to
 * bf16 for the value product), in prefill and decode alike.  With an MXFP4
 * cache, code * scale widens to bf16 exactly and the arithmetic is the bf16
 * path's.
 * Neither q nor the caches are written.
 * Streams: everything is ordered after the work already on `stream`, and
 * work enqueued on `stream` afterwards is ordered after all of it.  A step
 * that holds both prefill and decode rows (head_dim 128, any KV format) may run
 * its decode partly on a second, library-owned stream per device, forked
 * from `stream` by an event and joined back to it before the merges, so the
 * decode streams from HBM on a few CUs while the prefill occupies the others
 * ([Agentic] §5.1-5.2: the decode's tasks taken from a table by persistent
 * work-groups).  Calls from several host threads serialise that section.
 */
PA_API pa_status paged_attn_forward(const void *q, const pa_kv_cache *cache,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *hist_lens, const int32_t *incr_lens,
                             int32_t num_seqs, int32_t num_q_heads, float scale, void *out,
                             float *lse_out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * paged_attn_forward_cascade -- paged_attn_forward for a step in which groups
 * of sequences share a prefix: the same physical blocks hold their first
 * tokens ([Agentic] §2.1: sub-agents fan out from the main agent's context;
 * §4.1: prefix reuse).  Same computation and arguments as paged_attn_forward,
 * plus:
 *   group_of   HOST int32 [num_seqs]: each sequence's prefix group, -1 for
 *              none (NULL allowed when num_groups == 0).
 *   group_len  HOST int32 [num_groups]: tokens of the group's shared prefix,
 *              a multiple of block_size.  Caller promise: every member s of
 *              group g has the same block ids in block_tables[s][0 ..
 *              group_len[g] / block_size - 1] (results are undefined if not).
 *   workspace_bytes  in: the workspace's size; with workspace == NULL the
 *              call only writes the size it needs there and returns PA_OK.
 * With bf16 KV and head_dim 128, the members of a group that decode one token
 * over a history covering the shared prefix (at least two of them) read the
 * prefix once: their rows (up to 64 per tile) are computed against it as one
 * tile per KV head and key range, and each member's partial result is merged
 * by LSE with its own suffix's.  Other sequences, and other cache types, are
 * computed as paged_attn_forward computes them.  Results agree with
 * paged_attn_forward within rounding (the key ranges are split differently),
 * not bit for bit.
 */
PA_API pa_status paged_attn_forward_cascade(const void *q, const pa_kv_cache *cache,
                                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                                            const int32_t *hist_lens, const int32_t *incr_lens,
                                            int32_t num_seqs, int32_t num_q_heads, float scale,
                                            void *out, float *lse_out, const int32_t *group_of,
                                            const int32_t *group_len, int32_t num_groups,
                                            void *workspace, size_t *workspace_bytes, void *stream);

/* Maximum scratch of paged_attn_forward_noalloc, bytes per device. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * paged_attn_forward_noalloc -- paged_attn_forward for callers that cannot
 * allocate memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments and
 * error behaviour, without the workspace arguments.  Its scratch is a
 * static device array of PA_NOALLOC_SCRATCH_BYTES, one per device, that the
 * library holds until the process ends; the call allocates no device or
 * pinned host memory (the work list reaches the device by a stream-ordered
 * copy from host memory).  A step that needs more scratch than that fails
 * with PA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (use
 * paged_attn_forward with a workspace).  Calls that overlap on one device
 * share the array and race; calls ordered on one stream are safe.  The
 * scratch keeps the last call's contents; no call relies on them.  The work
 * list is copied from a host buffer that lives only for the call, so a call
 * recorded by stream capture must not be replayed as a graph (each eager
 * call, the intended use here, copies its own list).  A co-scheduled mixed
 * step (see paged_attn_forward) runs its launches one after the other here,
 * on `stream` alone, with the same results.
 */
PA_API pa_status paged_attn_forward_noalloc(const void *q, const pa_kv_cache *cache,
                                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                                            const int32_t *hist_lens, const int32_t *incr_lens,
                                            int32_t num_seqs, int32_t num_q_heads, float scale,
                                            void *out, float *lse_out, void *stream);

/* Bytes of workspace paged_attn_forward needs for these HOST lengths.
 * Returns 0 and sets pa_last_error() if the arguments are invalid. */
PA_API size_t pa_workspace_size(const int32_t *hist_lens, const int32_t *incr_lens, int32_t num_seqs,
                         int32_t num_q_heads, const pa_kv_cache *cache);

/* Text of the calling thread's most recent non-OK status ("" if none). */
PA_API const char *pa_last_error(void);

/* Test hook for block-table addressing: gathers one sequence's cached
 * tokens in logical order, raw (bf16 or E4M3 bytes, no scaling):
 *   k_out[p][h][:] = k_cache[block_table_row[p / bs]][h][p % bs][:]
 * for p < ctx; same for v_out.  block_table_row is a device pointer;
 * k_out, v_out are [ctx][num_kv_heads][head_dim] elements of the cache type.
 * MXFP4: k_out, v_out receive the values instead, bf16 [ctx][num_kv_heads]
 * [head_dim] (code * scale, exact), widened by the attention kernels' own
 * conversion. */
PA_API pa_status pa_debug_gather(const pa_kv_cache *cache, const int32_t *block_table_row, int32_t ctx,
                          void *k_out, void *v_out, void *stream);

/*
 * paged_attn_step -- kv_append and paged_attn_forward of one step in ONE
 * kernel launch (after the work-list copy).
 *
 * [Agentic] §5.1-§5.2: a decode layer runs as persistent kernels, one block
 * per SM, whose stages are task tables the blocks claim by index, and the KV
 * write precedes the attention that reads it.  Here one work-group per
 * compute unit claims, with device-scope atomics on counters in the
 * workspace: the append of the step's new tokens in chunks, then (once every
 * append chunk has finished) the prefill work of the persistent plan from
 * its own XCD's queue, then the decode items; a split tile's partials are
 * merged by the work-group that writes its last part (no merge launch).
 *
 * Arguments are those of kv_append followed by those of paged_attn_forward,
 * with num_tokens = total_q: k_new, v_new [total_q][num_kv_heads][head_dim]
 * and slot_mapping [total_q] are the new tokens of the query rows, in the
 * same order.  The cache after the step equals kv_append's bit for bit
 * (E4M3: codes from the caller's scales; MXFP4: codes and the scale bytes the
 * append computes); the outputs equal paged_attn_forward's within the
 * attention tolerance (the merge sums in another order, so the bits may
 * differ).
 *   workspace       NULL: *workspace_bytes is set to the bytes this step
 *                   needs (nothing else happens); otherwise at least that
 *                   many bytes, 256-byte aligned, contents need no
 *                   initialisation.
 * Supported: head_dim 128, bf16, E4M3 or MXFP4 KV (PA_ERR_UNSUPPORTED for
 * head_dim 64).
 */
PA_API pa_status paged_attn_step(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                                 const int64_t *slot_mapping, const void *q, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *hist_lens, const int32_t *incr_lens,
                                 int32_t num_seqs, int32_t num_q_heads, float scale, void *out, float *lse_out,
                                 void *workspace, size_t *workspace_bytes, void *stream);

/* Test hook: after a paged_attn_step on `workspace` (same lengths), copies
 * its flag word to HOST *flags_out and synchronises `stream`.  Bit 0 set
 * means a bounded device-side wait gave up (never expected; the step's
 * results are then not to be trusted). */
PA_API pa_status pa_debug_step_flags(const void *workspace, const pa_kv_cache *cache, const int32_t *hist_lens,
                                     const int32_t *incr_lens, int32_t num_seqs, int32_t num_q_heads,
                                     uint32_t *flags_out, void *stream);

/* Per-kernel timing for measurement.  When enabled (nonzero), each launch
 * records HIP events on the call's stream around the kernel; the durations
 * accumulate until read.  pa_timing_read(kind, &ms, &count) returns, for
 * kind 0 = kv_append, 1 = prefill attention, 2 = decode attention
 * (holding the shared-prefix cascade items of paged_attn_forward_cascade,
 * which run in the same launch), 3 = LSE merge, 4 = the one launch of
 * paged_attn_step, the summed
 * milliseconds and launch count since the last reset (it synchronises on the
 * recorded events), then resets that kind. */
PA_API pa_status pa_timing_enable(int enable);
PA_API pa_status pa_timing_read(int kind, double *ms, int64_t *count);

/* Test hook for the work planner: the work list paged_attn_forward would
 * build for these HOST lengths, written to HOST memory.  items_out receives
 * up to items_cap records of 8 int32 each, prefill items first, then decode
 * items: {seq, kv_head, first_row, first_pos, tokens, key_lo, key_hi,
 * partial_slot (-1 = final)}.  counts_out[0..3] = prefill items, decode items,
 * merge tasks, partial slots.  Returns PA_ERR_WORKSPACE_TOO_SMALL (with the
 * counts filled) if items_cap is too small. */
PA_API pa_status pa_debug_plan(const int32_t *hist_lens, const int32_t *incr_lens,
                               int32_t num_seqs, int32_t num_q_heads, const pa_kv_cache *cache,
                               int32_t *items_out, int32_t items_cap, int32_t *counts_out);

/* Test and measurement hook for the co-scheduled mixed step (see
 * paged_attn_forward): n < 0 (the default) lets the planner choose how many
 * CUs to take from the prefill for the decode; n > 0 forces that many
 * (rounded down to a multiple of the XCD count, at most half the CUs); n = 0
 * runs the launches one after the other.  A prefill too small to hold every
 * CU leaves the others to the decode whenever co-scheduling is on.  Applies
 * to every later plan that qualifies (pa_workspace_size and the debug plans
 * alike); process-wide. */
PA_API pa_status pa_debug_overlap_cus(int32_t n);

/* Test hook for the persistent prefill launch: when the plan for these HOST
 * lengths runs the persistent 384-row kernel (head_dim 128, any KV format)
 * with one work-group per balanced range of work, *num_groups_out receives the number
 * of work-groups n and first_out[0..n] the offsets into the prefill items
 * (as listed by pa_debug_plan) where each work-group's items begin, with
 * first_out[n] = the number of prefill items.  n = 0 (nothing written) for
 * plans without such a launch.  PA_ERR_WORKSPACE_TOO_SMALL if cap < n + 1. */
PA_API pa_status pa_debug_plan_groups(const int32_t *hist_lens, const int32_t *incr_lens,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      const pa_kv_cache *cache, int32_t *first_out, int32_t cap,
                                      int32_t *num_groups_out);

/* The machine shape the work planner cuts plans for: the current device's
 * compute units and XCDs (chiplets, each with its own L2), queried once per
 * device (MI355X: 256 and 8); without a device, the MI355X's shape.  The
 * planner assumes work-group w of a launch runs on XCD w mod num_xcds. */
PA_API pa_status pa_device_shape(int32_t *num_cus, int32_t *num_xcds);

/* Test hook for that assumption: enqueues n work-groups on `stream`;
 * work-group w writes the id of the XCD it ran on to out[w] (device int32[n]). */
PA_API pa_status pa_debug_xcc_ids(int32_t *out, int32_t n, void *stream);

/* Measurement hooks: the practical ceilings of the two resources the
 * attention kernels are bound by, measured with the same instructions
 * (MI355X: 256 compute units).  Both enqueue one kernel on `stream`; the
 * caller times it (e.g. with events on that stream).
 *   pa_peak_mfma: 256 work-groups of 8 waves each run iters x 8 independent
 *     v_mfma_f32_16x16x32_bf16 (16,384 flops each): 2^28 * iters flops in
 *     all.  out: device float[256 * 512], written with a checksum.
 *   pa_peak_read: streams `bytes` (a positive multiple of 4096) of the
 *     device buffer `buf` through LDS with the decode kernels' non-temporal
 *     LDS-filling 16-byte loads: one work-group of 4 waves per compute unit,
 *     each wave a 4-stage ring of 4 KB requests.  out: device
 *     uint32[256 * 256], written with a checksum.
 * Nothing else is read or written. */
PA_API pa_status pa_peak_mfma(float *out, int32_t iters, void *stream);
PA_API pa_status pa_peak_read(const void *buf, size_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_H */
