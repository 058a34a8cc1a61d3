// pa_attention.hip -- gfx950 attention kernels over the paged KV cache.
//
// Pages cited (title, then section):
//   [Agentic] "vLLM Agentic 推理｜面向 Agent 负载的推理优化"
//   [AMPD]    "ICML'26 | AMPD：PD 分离遇上多轮推理，incremental prefill 到底该在哪跑"
//
// What is computed ([AMPD] §1, §3): each new query token at absolute position
// p attends to keys 0..p of its sequence -- the cached history plus the new
// tokens up to itself -- with softmax(scale * q.k) weights over the values.
// Prefill tiles are compute-bound, decode tiles stream the growing cache
// ([AMPD] §1: prefill is compute-bound, decode memory-bound).
//
// Both kernels use the transposed product S^T = K * Q^T so that one lane owns
// one query row's scores and the softmax reductions stay inside a lane (plus
// one cross-half exchange), and O^T = V^T * P^T so that the probabilities
// leave the score accumulators already in the B-operand layout.  The GQA group
// of query heads that share a KV head is packed into the MFMA N dimension, so
// every K/V tile loaded is used by all G heads.  V^T operands come from LDS
// with ds_read_b64_tr_b16.  Online softmax runs in the log2 domain (scale
// folded with log2 e), max/sum per lane.  Items that cover only part of a
// row's keys write normalised partial outputs and their log-sum-exp for the
// merge kernel ([Agentic] §4.3.3: partial O_i with LSE merged the
// online-softmax way; §5.2: split attention, then combine).
//
// Kernels, in file order (FMT: the KV format, 0 bf16, 1 E4M3, 2 MXFP4):
//   prefill_kernel<D, BS, FP8>     register-staged, 128-row tiles (head_dim 64)
//   prefill_w48_kernel<BS, FMT>    persistent 384-row LDS-DMA prefill (head_dim 128)
//   decode_kernel<D, BS, FP8>      register-staged decode (head_dim 64)
//   decode_dma_kernel<BS, NW, NST> LDS-DMA decode, bf16 (head_dim 128)
//   decode_cascade_kernel<BS, NRB, NW, NST>
//                                  shared-prefix cascade items, then decode items
//   decode_dma_fp8_kernel<BS, NW, NST>, decode_dma_fp4_kernel<BS, NW, NST>
//                                  LDS-DMA decode, E4M3 and MXFP4 (head_dim 128)
//   decode_claim_kernel<BS, NRB, FMT>
//                                  the decode launch's items claimed by persistent
//                                  work-groups (co-scheduled mixed steps)
//   merge_kernel, merge_many_kernel  LSE merge of split items
//   step_kernel<BS, FMT>           the whole step in one persistent launch
// (the decode kernels' bodies are item functions -- decode_dma_item,
// cascade_item, decode_fp8_item, decode_fp4_item -- that the claiming and
// step kernels call too)
#include "pa_append.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// LDS row layout of a K or V tile: rows of D bf16 (D/8 16-byte chunks).  Rows
// are padded by kLdsPad bytes so that consecutive rows start in different
// banks: the 16-byte A-operand reads of eight rows and the transpose reads of
// four rows x 32 bytes then touch disjoint banks, while every address a lane
// uses stays a per-lane base plus a compile-time offset.  kLdsPad == 0 selects
// an XOR swizzle of the chunk index instead (no padding).
#ifndef PA_LDS_PAD
#define PA_LDS_PAD 32
#endif
constexpr int kLdsPad = PA_LDS_PAD;

template <int D>
struct LdsRow {
  static constexpr int bytes = D * 2 + kLdsPad;  // row stride
  static __device__ __forceinline__ int off(int row, int chunk) {
    if constexpr (kLdsPad == 0) {
      constexpr int MASK = D / 16 - 1;
      return row * bytes + ((chunk ^ ((row & MASK) << 1)) * 16);
    } else {
      return row * bytes + chunk * 16;
    }
  }
};

// =============================================================================
// Softmax bookkeeping shared by both kernels.  Scores are kept raw (q.k); the
// running maximum m is kept in log2 units (raw * sl, sl = scale * log2 e > 0),
// so a probability is one fused multiply-add and one exp2.  The maximum is
// updated lazily: only when some lane's tile maximum exceeds its m by more than
// kRescaleSlack does the wave move m up and rescale its sums; otherwise the
// stale m is kept and the probabilities may reach 2^kRescaleSlack, which bf16
// and fp32 hold exactly as well as values below 1.  The final O / l is the
// same quantity either way.
constexpr float kRescaleSlack = 8.0f;

using MaskedTile = std::true_type;
using FullTile = std::false_type;

// =============================================================================
// Prefill: one work-group (4 waves) per item; 128 query rows (tokens x heads),
// each wave owns 32 rows; 64-key tiles double-buffered through LDS.
template <int D, int BS, bool FP8>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnArgs a) {
  constexpr int CPR = D / 8;             // 16-byte bf16 chunks per LDS row
  typedef LdsRow<D> L;
  constexpr int TILEB = kKeyTile * L::bytes;  // one K or V tile in LDS
  constexpr int NCH = kKeyTile * CPR / 256;
  constexpr int NC = D / 16;             // k-steps of the score product
  constexpr int ND = D / 32;             // 32-wide d blocks of the output
  constexpr int NSC = FP8 ? (BS == 16 ? 4 : 1) : 1;  // K/V scales per tile
  constexpr int RPI = 64 / CPR;          // key rows one wave covers per load instruction

  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[4 * TILEB];
  lds_u8 *smem = (lds_u8 *)smem_raw;

  const Item it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int row = wave * 32 + col;
  const int tok = row >> a.lg, g = row & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;

  // Q as the B operand of K * Q^T: lane holds q[row][16c + 8hh .. +7].
  bf16x8 qf[NC];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < NC; c++) {
      uint4 v = active ? gload16(qrow + (c * 16 + hh * 8) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = as_bf16x8(v);
    }
  }

  float m = kNegBig, l = 0.f;
  f32x16 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x16{};

  const int32_t *bt = a.bt + (int64_t)it.seq * a.max_blocks;
  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const int t_begin = it.kv_lo / kKeyTile;
  const int t_end = (it.kv_hi + kKeyTile - 1) / kKeyTile;
  // tiles below t_full need no mask: every key is < kv_hi and <= every row's position
  const int t_full = max(t_begin, min(t_end, min(it.pos0 + 1, it.kv_hi) / kKeyTile));
  const int last_blk = (it.kv_hi - 1) / BS;
  const int lim = min(pos, it.kv_hi - 1);  // last key this lane's row may see

  // Staging registers for the next tile's K and V chunks.  Load instruction i
  // of this wave covers key rows rb .. rb + RPI - 1 of the tile, all in one
  // cache block, so the block id is a wave-uniform (scalar) load.
  typedef typename std::conditional<FP8, uint2, uint4>::type chunk_t;
  chunk_t kr[NCH], vr[NCH];
  float ksc_n[NSC], vsc_n[NSC], ksc[NSC], vsc[NSC];
  const int lrow = lane / CPR, lch = lane % CPR;

  auto load_tile = [&](auto partial, int t) {
    constexpr bool PART = decltype(partial)::value;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int rb = (256 * i + 64 * wave) / CPR;
      int bidx = (t * kKeyTile + rb) / BS;
      if (PART) bidx = min(bidx, last_blk);
      const int64_t blk = bt[bidx];
      const int p = t * kKeyTile + rb + lrow;
      const int64_t e = ((blk * hkv + it.kvh) * BS + (p % BS)) * D + lch * 8;
      if constexpr (FP8) {
        kr[i] = gload8(kc + e);
        vr[i] = gload8(vc + e);
      } else {
        kr[i] = gload16(kc + e * 2);
        vr[i] = gload16(vc + e * 2);
      }
      if (PART && p >= it.kv_hi) {
        kr[i] = chunk_t{};
        vr[i] = chunk_t{};
      }
    }
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NSC; j++) {
        const int bidx = min((t * kKeyTile + j * BS) / BS, last_blk);
        const int64_t blk = bt[bidx];
        ksc_n[j] = ((const float *)a.c.ks)[blk * hkv + it.kvh];
        vsc_n[j] = ((const float *)a.c.vs)[blk * hkv + it.kvh];
      }
    }
  };
  auto store_tile = [&](int buf) {
    lds_u8 *kb = smem + buf * 2 * TILEB;
    lds_u8 *vb = kb + TILEB;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int r = (256 * i + 64 * wave) / CPR + lrow;
      const int off = L::off(r, lch);
      if constexpr (FP8) {
        lds_store16(kb + off, e4m3x8_to_bf16x8(kr[i]));
        lds_store16(vb + off, e4m3x8_to_bf16x8(vr[i]));
      } else {
        lds_store16(kb + off, kr[i]);
        lds_store16(vb + off, vr[i]);
      }
    }
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NSC; j++) {
        ksc[j] = ksc_n[j];
        vsc[j] = vsc_n[j];
      }
    }
  };
  auto load_next = [&](int t) {
    if ((t + 1) * kKeyTile <= it.kv_hi)
      load_tile(FullTile{}, t);
    else
      load_tile(MaskedTile{}, t);
  };

  const int g16 = lane >> 4, j16 = lane & 15;

  auto compute = [&](auto masked, int t, const lds_u8 *Kb, const lds_u8 *Vb) {
    constexpr bool MASK = decltype(masked)::value;
    // ---- S^T = K * Q^T : two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      const int krow = kb * 32 + col;
      s[kb] = mfma32x32x16(as_bf16x8(lds_load16(Kb + L::off(krow, hh))), qf[0], f32x16{});
#pragma unroll
      for (int c = 1; c < NC; c++) {
        bf16x8 af = as_bf16x8(lds_load16(Kb + L::off(krow, 2 * c + hh)));
        s[kb] = mfma32x32x16(af, qf[c], s[kb]);
      }
    }
    // ---- mask, tile maximum (raw scores; element 4i+r of block kb is key
    //      kb*32 + 8i + 4hh + r)
    float sl[NSC];
#pragma unroll
    for (int j = 0; j < NSC; j++) sl[j] = FP8 ? a.scale_log2 * ksc[j] : a.scale_log2;
    const int kbase = t * kKeyTile;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        if (MASK) {
          const int key = kbase + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
          s[kb][e] = key <= lim ? s[kb][e] : -INFINITY;
        }
        if constexpr (NSC > 1) s[kb][e] *= sl[kb * 2 + (e >> 3)];
        mx = fmaxf(mx, s[kb][e]);
      }
    mx = xor32_max(mx);
    const float mxs = NSC > 1 ? mx : mx * sl[0];
    if (__any(mxs > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mxs);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++) o[db] *= alpha;
    }
    const float slp = NSC > 1 ? 1.0f : sl[0];
    const float nm = -m;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][e], slp, nm));
        s[kb][e] = p;
        psum += p;
      }
    l += psum;

    // ---- O^T += V^T * P^T : four 16-key steps
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int kb = ks >> 1, i0 = (ks & 1) * 2;
      bf16x8 pb;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        float p0 = s[kb][4 * i0 + r], p1 = s[kb][4 * (i0 + 1) + r];
        if constexpr (FP8) {
          const float v0 = vsc[(NSC == 1) ? 0 : (kb * 2 + (i0 >> 1))];
          p0 *= v0;
          p1 *= v0;
        }
        pb[r] = (__bf16)p0;
        pb[4 + r] = (__bf16)p1;
      }
#pragma unroll
      for (int db = 0; db < ND; db++) {
        const int d0 = db * 32 + (g16 & 1) * 16 + 4 * (j16 & 3);
        const int vr0 = ks * 16 + 4 * hh + (j16 >> 2);
        const int vr1 = vr0 + 8;
        const bf16x4 h0 = lds_read_tr(Vb + L::off(vr0, d0 >> 3) + (d0 & 7) * 2);
        const bf16x4 h1 = lds_read_tr(Vb + L::off(vr1, d0 >> 3) + (d0 & 7) * 2);
        bf16x8 af = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma32x32x16(af, pb, o[db]);
      }
    }
  };

  if (t_begin < t_end) {
    load_next(t_begin);
    store_tile(0);
  }
  __syncthreads();

  // unmasked tiles, then the tiles that cross the causal diagonal or the
  // range's end (separate loops keep each body branch-free)
  int t = t_begin;
  for (; t < t_full; t++) {
    const int buf = (t - t_begin) & 1;
    const lds_u8 *Kb = smem + buf * 2 * TILEB;
    if (t + 1 < t_end) load_next(t + 1);
    compute(FullTile{}, t, Kb, Kb + TILEB);
    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();
  }
  for (; t < t_end; t++) {
    const int buf = (t - t_begin) & 1;
    const lds_u8 *Kb = smem + buf * 2 * TILEB;
    if (t + 1 < t_end) load_tile(MaskedTile{}, t + 1);
    compute(MaskedTile{}, t, Kb, Kb + TILEB);
    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: combine the two key halves' sums, normalise, store
  const float lt = xor32_sum(l);
  if (!active) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = lt > 0.f ? m + __log2f(lt) : -INFINITY;
  if (it.part < 0) {
    unsigned char *orow =
        (unsigned char *)a.out + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = (__bf16)(o[db][4 * i + r] * inv);
        *(bf16x4 *)(orow + (db * 32 + 8 * i + 4 * hh) * 2) = v;
      }
    if (a.lse_out && hh == 0) a.lse_out[(int64_t)(it.row0 + tok) * a.hq + qh] = lse2 * kLn2;
  } else {
    float *prow = a.part_o + ((int64_t)it.part * kRegTileRows + row) * D;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = o[db][4 * i + r] * inv;
        *(f32x4 *)(prow + db * 32 + 8 * i + 4 * hh) = v;
      }
    if (hh == 0) a.part_lse[(int64_t)it.part * kRegTileRows + row] = lse2;
  }
}

// =============================================================================
// LDS-DMA prefill for head_dim 128 (prefill_w48_kernel below).  K/V steps
// live in a multi-stage LDS ring filled directly from HBM by buffer loads
// that write LDS (no register staging), issued as inline assembly with
// explicit vmcnt waits: the compiler neither reorders them nor inserts waits
// of its own for them.  Each load covers four key rows of one cache block;
// its buffer resource starts at those rows and ends at the range's last key,
// so rows past the end read as zeros without touching memory.
// (LDS-filling loads: dma_load16 / dma_load16_nt and PA_WAIT_VMCNT in pa_device.h)

// Work-group barrier without a memory fence: LDS hazards around it are
// handled by explicit waits; the compiler-only fences keep memory operations
// and the scheduling barriers keep all instructions on their side of it.
__device__ __forceinline__ void wg_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}


// =============================================================================
// 384-row prefill, head_dim 128 ("ping-pong"): one work-group of 8 waves per
// CU; waves 0-3 (group 0) and 4-7 (group 1) each own 48 query rows per wave
// (three 16-row blocks) on v_mfma_f32_16x16x32_bf16, in 32-key steps.  In
// each half-step one group issues its matrix-core work (O += V(t)^T P(t)^T,
// then S(t+1) = K(t+1) Q^T) while the other turns scores into probabilities
// on the vector ALUs, so each SIMD always has one wave feeding its matrix
// core and one wave doing softmax.  (An earlier 256-row design with 32 rows
// per wave on 32x32x16 MFMAs and 64-key steps brought 1.5x the bytes into the
// CU per flop and ran at a lower clock.)
//   Sᵀ = K Qᵀ per (16-key block kb, 16-row block rb): A = K (lane: key c16,
//   d 32c + 8g..+7, one 16-byte LDS read), B = Qᵀ (lane: row c16, same d, in
//   registers), D: lane holds row c16, keys 16kb + 4g + r.
//   Oᵀ += Vᵀ Pᵀ per (16-d block db, rb) over the step's 32 keys: B = Pᵀ is
//   (S[0][rb][0..3], S[1][rb][0..3]) converted in place, which orders the
//   contraction index as keys 4g..4g+3, 16+4g..16+4g+3 of lane group g; A =
//   Vᵀ is read in that order by two transposing LDS reads (lane: d = 16db +
//   c16).  D: lane holds row c16, d = 16db + 4g + r.
// A row's 32 scores of a step sit in the four lanes c16 + 16g, reduced with
// the permlane swaps.
// E4M3 KV ([V41] kernels section: 8-bit KV to cut its footprint): the codes
// reach LDS by the same LDS-filling loads (half the bytes of bf16), and each
// step's K and V codes are widened to bf16 once per work-group (8 exact
// conversions per lane and step, all eight waves sharing the work) into the
// same tile layout the bf16 path reads, so the matrix-core code is the same.
// The per-(block, head) scales stay in fp32: the key scale joins the score's
// fused multiply-add, and the value scale enters the probability's exponent
// (so P * s_v is what is rounded to bf16 for the value product); the row sum
// l, which the matrix cores accumulate from those same bf16 values, is kept
// in units of the current step's value scale and rescaled by s_v(t)/s_v(t-1)
// when the step changes (divided out at the end).
// MXFP4 KV ([V41] kernels section: a 4-bit KV cache): a step's K and V codes
// (64 bytes a key) and scale bytes reach a code ring the same way -- waves
// 0-3 request the codes (16 key rows each), waves 4-7 the scale bytes (16
// keys of K or V each) -- and the widening applies each 32-element group's
// E8M0 scale in the conversion itself: the tiles then hold the values
// exactly, and the rest is the bf16 path (no scale in the softmax).
constexpr int kW48Step = 32;                        // keys per step
// K (or V) of one 32-key step in LDS: 8 blocks of 4 key rows, each block
// 1,024 bytes of data and 32 of padding (the layout is described at the
// item function)
constexpr int kW48BlockBytes = 4 * 128 * 2 + 32;
constexpr int kW48TileBytes = 8 * kW48BlockBytes;
#ifndef PA_W48_STAGES
#define PA_W48_STAGES 4
#endif
constexpr int kW48Stages = PA_W48_STAGES;
constexpr int kW48CodeStages = 8;                // E4M3 and MXFP4: stages of the code ring (8 against 4: 57.3 -> 55.0 ms for the 1M-token E4M3 prefill)
constexpr int kW48CodeBytes = kW48Step * 128;    // E4M3 codes of one step's K (or V)
constexpr int kW48ScaleSlots = 8;                // E4M3: steps held by the scale ring
constexpr int kW48ScaleSlotBytes = 1024;         // K half 0, K half 1, V half 0, V half 1: 256 bytes each
constexpr int kW48Fp8Lds = 4 * kW48TileBytes + kW48CodeStages * 2 * kW48CodeBytes + kW48ScaleSlots * kW48ScaleSlotBytes;
constexpr int kW48Fp4CodeBytes = kW48Step * 64;  // MXFP4 codes of one step's K (or V)
constexpr int kW48Fp4ScaleBytes = kW48Step * 4;  // MXFP4 scale bytes of one step's K (or V)
// a code-ring stage: K codes, V codes, then the scale bytes as K keys 0-15,
// K keys 16-31, V keys 0-15, V keys 16-31, each [group][16 keys]
constexpr int kW48Fp4StageBytes = 2 * kW48Fp4CodeBytes + 2 * kW48Fp4ScaleBytes;
constexpr int kW48Fp4Lds = 4 * kW48TileBytes + kW48CodeStages * kW48Fp4StageBytes;

template <int BS, int FMT>
__device__ __forceinline__ void w48_item(const AttnArgs &a, const Item it, lds_u8 *smem) {
  constexpr bool FP8 = FMT == kKvE4m3;
  constexpr bool FP4 = FMT == kKvMxfp4;
  constexpr bool CODED = FP8 || FP4;  // the tiles are widened from a code ring
  constexpr int REQ = FP4 ? 1 : 2;    // requests per wave and step (E4M3: of the scale-loading waves)
  constexpr int D = 128;
  constexpr int NCQ = D / 32;  // k-steps of the score product
  constexpr int NDB = D / 16;  // d-blocks of the value product
  constexpr int RB = 3;        // 16-row blocks per wave
  constexpr int TILEB = kW48TileBytes;
  constexpr int STAGEB = 2 * TILEB;
  constexpr int NST = kW48Stages;
  constexpr int NCS = kW48CodeStages;
  constexpr int CB = kW48CodeBytes;
  // E4M3, block 16: a step's two 16-key halves lie in different blocks (two
  // scales per step, l kept per half); block 64: one block per step
  constexpr bool SPLIT = FP8 && BS == 16;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const float scale_log2 = a.scale_log2;
  const int kvh = it.kvh, hkv = a.c.hkv;
  const int nq = it.nq;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int c16 = lane & 15, g = lane >> 4;

  // Q as stored (bf16, exact): the score MFMAs produce raw q.k, and one
  // fused multiply-add per score applies scale * log2(e) (times the key scale
  // for E4M3) and the row's reference exponent in fp32.
  bf16x8 qf[RB][NCQ];
  f32x4 o[NDB + 1][RB];  // O^T accumulators; o[NDB] is the row sum l
  float negm[RB];        // -m per row block; m itself is not kept
  int all_live = 0;      // every row of the wave has weight (wave-uniform)
  float isv[2] = {0.f, 0.f};  // E4M3: 1 / value scale of the last step's two 16-key halves
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    const int row = wave * 48 + rb * 16 + c16;
    const int tok = row >> a.lg, gq = row & (a.group - 1);
    const bool act = tok < nq;
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + kvh * a.group + gq) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCQ; c++) {
      uint4 v = act ? gload16(qrow + (32 * c + 8 * g) * 2) : make_uint4(0, 0, 0, 0);
      qf[rb][c] = as_bf16x8(v);
    }
    negm[rb] = 0.f;
#pragma unroll
    for (int db = 0; db <= NDB; db++) o[db][rb] = f32x4{};
  }
  f32x4 S[2][RB];
  bf16x8 pb[RB];
  // the row-sum operand: all ones, or for E4M3 block 16 one half per 16-key
  // half (A rows 0-7 sum keys 0-15, rows 8-15 keys 16-31: lanes with g < 2
  // accumulate the first half's l, g >= 2 the second's)
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; e++) ones[e] = (__bf16)(SPLIT ? (((e < 4) == (c16 < 8)) ? 1.0f : 0.0f) : 1.0f);

  const int kv_hi = it.kv_hi;
  const int t_begin = it.kv_lo / kW48Step;
  const int t_end = (kv_hi + kW48Step - 1) / kW48Step;
  const int t_full = max(t_begin, min(t_end, min(it.pos0 + 1, kv_hi) / kW48Step));
  const int last_blk = (kv_hi - 1) / BS;
  // The block ids (and E4M3 scales) are read through the scalar cache with
  // wave-uniform loads, each well before it is used: a vector load would be
  // counted with the K/V stream by vmcnt, and staging them in LDS would bound
  // the length of an item (the planner never cuts an item for length).
  typedef const __attribute__((address_space(4))) int32_t cint;
  const cint *btr = (const cint *)(a.bt + (int64_t)it.seq * a.max_blocks);
  auto block_of = [&](int key) __attribute__((always_inline)) {
    return btr[(uint32_t)min((int)((uint32_t)key / BS), last_blk)];  // (key >= 0: an unsigned shift)
  };

  // LDS tile of one step (32 keys, 256 bytes each): key row k lies in block
  // k / 4 (blocks kW48BlockBytes apart: 1 KB of data + 32 bytes), and within
  // its block, 16-byte chunk q of row r = k % 4 sits at byte
  // 256 (q / 4) + 64 r + 16 (q % 4).  gfx950's LDS serves 256 bytes a cycle
  // (64 four-byte banks).  A 16-byte read is served 16 lanes at a time, lanes
  // equal in lane bit 5 and in the parity of lane bits 2..4; a transposing
  // 8-byte read, a half-wave at a time (both measured with
  // SQ_LDS_BANK_CONFLICT on patterns built for the purpose).  With the
  // 32-byte block padding, the K reads (lane (g, c) reads chunk 4j + g of row
  // c) and the V^T reads (lane (g, c): row 4g + c/4, chunk 2db + (c%4)/2,
  // half c%2) both hit distinct banks, and every read is one per-lane base
  // plus an immediate: j * 256 (K), (db / 2) * 256 + (db % 2) * 32 (V), and
  // 4 blocks for the second 16 keys.  Each quarter-wave of a DMA request
  // fetches 64 contiguous bytes of one row.
  constexpr int KB16 = 4 * kW48BlockBytes;  // keys 16..31 of the step
  const int kbase = (c16 >> 2) * kW48BlockBytes + (c16 & 3) * 64 + g * 16;
  const int vbase = g * kW48BlockBytes + (c16 >> 2) * 64 + ((c16 & 3) >> 1) * 16 + (c16 & 1) * 8;
  auto kofs = [&](int c) { return kbase + c * 256; };
  auto vofs = [&](int db) { return vbase + (db >> 1) * 256 + (db & 1) * 32; };
  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;

  // K/V requests walk the item's steps in order, so their positions are
  // running counters.  Items start on a step boundary (the planner cuts key
  // ranges in multiples of 64 keys), so rpos >= kv_lo.  A request's buffer
  // size is the bytes of the range's rows left from its first row on (no
  // upper clamp: its lanes never address past the request's own rows), so
  // rows past the range end read as zeros, and a request past the end has
  // size zero: it moves no data but keeps the per-step vmcnt accounting.
  constexpr int LGBS = BS == 16 ? 4 : 6;
  static_assert(BS == 16 || BS == 64, "block size");
  constexpr int KEYB = FP4 ? D / 2 : FP8 ? D : 2 * D;  // bytes of one key row (K or V)
  const uint32_t blk_bytes = (uint32_t)hkv * BS * KEYB;
  // bf16: this wave's requests fill block `wave` of the step's K and V tiles
  // (key rows 4*wave .. +3): lane l writes byte 16 l of the block, i.e. row
  // (l / 4) % 4, chunk 4 (l / 16) + l % 4.  E4M3: waves 0-3 request K codes,
  // waves 4-7 V codes, rows 8 (wave % 4) .. +7 of the step (1 KB, one block),
  // into the code ring, where row R's 16-byte chunk j sits at position
  // j ^ (4 ((R >> 1) & 1)) (so that the widening reads below are free of bank
  // conflicts): lane l fetches the chunk its LDS position holds.
  // MXFP4: waves 0-3 request the codes of key rows 16 (wave & 1) .. +15 of K
  // (waves 0, 1) or V (2, 3), 1 KB as stored; waves 4-7 the scale bytes of
  // those 16 keys of K (4, 5) or V (6, 7): lanes 0-15 fetch the dword of
  // group lane / 4, keys 4 (lane % 4) .. +3.
  const int voff = FP4 ? (wave < 4 ? 16 * lane : BS * (lane >> 2) + 4 * (lane & 3))
                 : FP8 ? (lane >> 3) * 128 + 16 * ((lane & 7) ^ (((lane >> 4) & 1) << 2))
                       : ((lane >> 2) & 3) * 256 + (4 * (lane >> 4) + (lane & 3)) * 16;
  const int qw = wave & 3;
  const bool fp4_v = ((wave >> 1) & 1) != 0;  // MXFP4: this wave requests V (codes or scales)
  const unsigned char *mine = FP4 ? (fp4_v ? vc : kc) : FP8 && wave >= 4 ? vc : kc;
  const uint64_t kc_head = (uint64_t)(kc + (int64_t)kvh * BS * KEYB);
  const uint64_t vc_head = (uint64_t)(vc + (int64_t)kvh * BS * KEYB);
  const uint64_t my_head = (uint64_t)(mine + (int64_t)kvh * BS * KEYB);
  // first key row of this wave's next request
  int rpos = t_begin * kW48Step + (FP4 ? 16 * (wave & 1) : FP8 ? 8 * qw : 4 * wave);
  uint32_t st_off = 0;                                        // its ring stage, in bytes
  int blk_next = block_of(rpos);
  constexpr int RING = CODED ? 4 * TILEB : 0;  // the code ring follows the four bf16 tiles
  constexpr int SCB = RING + NCS * 2 * CB;   // E4M3: then the scale ring
  // E4M3: with its codes, one wave per scale the step needs also requests
  // it into the step's slot of the scale ring: waves 0 (K) and 4 (V), and
  // for block 16, whose two 16-key halves lie in different blocks, waves 2
  // and 6 for the second half (the half of a wave's rows is (wave % 4) / 2);
  // every lane reads the same 4 bytes.  Those waves make two requests a
  // step, the others one.
  const uint64_t sc_head = (uint64_t)(FP8 && wave >= 4 ? a.c.vs : a.c.ks) + (uint64_t)kvh * 4;
  // MXFP4 scale bytes of this wave's KV head: [block][hkv][group][BS]
  const uint64_t sc4_head = (uint64_t)(fp4_v ? a.c.vs : a.c.ks) + (uint64_t)kvh * (D / 32) * BS;
  const uint32_t sc4_blk = (uint32_t)hkv * (D / 32) * BS;
  const uint32_t fp4_dst = wave < 4 ? (fp4_v ? kW48Fp4CodeBytes : 0) + (wave & 1) * 1024
                                    : 2 * kW48Fp4CodeBytes + (2 * (fp4_v ? 1 : 0) + (wave & 1)) * 64;
  const uint32_t sc_lane0 = SCB + (wave >= 4 ? 512 : 0) + (qw >> 1) * 256;
  const bool sc_loader = FP8 && (SPLIT ? (qw & 1) == 0 : qw == 0);
  uint32_t sc_off = 0;
  const int zero = 0;
  auto issue = [&]() __attribute__((always_inline)) {
    const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane(blk_next);
    const uint64_t off = (uint64_t)blk * blk_bytes + (uint32_t)((rpos & (BS - 1)) * KEYB);
    if constexpr (FP4) {
      const uint32_t dst = smem_addr + RING + st_off + fp4_dst;
      if (wave < 4) {
        const int nrec = __builtin_amdgcn_readfirstlane(max(kv_hi - rpos, 0) * KEYB);
        const uint64_t ga = my_head + off;
        const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)ga),
                           __builtin_amdgcn_readfirstlane((int)((ga >> 32) & 0xFFFF)), nrec, kRsrcFlags};
        dma_load16(r, voff, dst);
      } else {
        // the block's scale bytes from its first key of the request on (keys
        // past the range are made harmless by the widening)
        const uint64_t sa = sc4_head + (uint64_t)blk * sc4_blk + (uint32_t)(rpos & (BS - 1));
        const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)sa),
                           __builtin_amdgcn_readfirstlane((int)((sa >> 32) & 0xFFFF)),
                           (D / 32) * BS - (rpos & (BS - 1)), kRsrcFlags};
        if (lane < 16) dma_load4(r, voff, dst);
      }
      st_off = st_off + kW48Fp4StageBytes == NCS * kW48Fp4StageBytes ? 0 : st_off + kW48Fp4StageBytes;
    } else if constexpr (FP8) {
      const int nrec = __builtin_amdgcn_readfirstlane(max(kv_hi - rpos, 0) * D);
      const uint64_t ga = my_head + off;
      const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)ga),
                         __builtin_amdgcn_readfirstlane((int)((ga >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      dma_load16(r, voff, smem_addr + RING + st_off + (wave >= 4 ? CB : 0) + qw * 1024);
      st_off = st_off + 2 * CB == NCS * 2 * CB ? 0 : st_off + 2 * CB;
      if (sc_loader) {
        const uint64_t sa = sc_head + (uint64_t)blk * ((uint32_t)hkv * 4);
        const i32x4_t rs = {__builtin_amdgcn_readfirstlane((int)(uint32_t)sa),
                            __builtin_amdgcn_readfirstlane((int)((sa >> 32) & 0xFFFF)), 4, kRsrcFlags};
        dma_load4(rs, zero, smem_addr + sc_lane0 + sc_off);
      }
      sc_off = (sc_off + kW48ScaleSlotBytes) & (kW48ScaleSlots * kW48ScaleSlotBytes - 1);
    } else {
      const int nrec = __builtin_amdgcn_readfirstlane(max(kv_hi - rpos, 0) * (D * 2));
      const uint32_t st = smem_addr + st_off;
      const uint64_t ka = kc_head + off, va = vc_head + off;
      // (readfirstlane keeps the descriptor in SGPRs, as the asm operand needs)
      const i32x4_t rk = {__builtin_amdgcn_readfirstlane((int)(uint32_t)ka),
                          __builtin_amdgcn_readfirstlane((int)((ka >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      const i32x4_t rv = {__builtin_amdgcn_readfirstlane((int)(uint32_t)va),
                          __builtin_amdgcn_readfirstlane((int)((va >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      dma_load16(rk, voff, st + wave * kW48BlockBytes);
      dma_load16(rv, voff, st + TILEB + wave * kW48BlockBytes);
      st_off = st_off + STAGEB == NST * STAGEB ? 0 : st_off + STAGEB;
    }
    rpos += kW48Step;
    blk_next = block_of(rpos);
  };
  (void)my_head;
  static_assert((NST & (NST - 1)) == 0 && (NCS & (NCS - 1)) == 0, "ring stages: a power of two");
  // bf16 tiles of step t: the DMA ring (bf16) or the widened double buffers (E4M3)
  auto ktile = [&](int t) __attribute__((always_inline)) {
    if constexpr (CODED) return (const lds_u8 *)(smem + (t & 1) * TILEB);
    else return (const lds_u8 *)(smem + ((t - t_begin) % NST) * STAGEB);
  };
  auto vtile = [&](int t) __attribute__((always_inline)) {
    if constexpr (CODED) return (const lds_u8 *)(smem + 2 * TILEB + (t & 1) * TILEB);
    else return (const lds_u8 *)(smem + ((t - t_begin) % NST) * STAGEB + TILEB);
  };
  // E4M3 widening: wave w converts block w (key rows 4w .. 4w+3) of a step's
  // K or V tile; lane (Q, r, qq) = (lane / 16, lane / 4 % 4, lane % 4) reads
  // the 8 codes of chunk q = 4Q + qq of row 4w + r and writes them as one
  // 16-byte bf16 chunk.  Reads and writes each cover 64 banks per 16 lanes.
  const int wrow = 4 * wave + ((lane >> 2) & 3);
  const int wq = 4 * (lane >> 4) + (lane & 3);
  const int w_rd = wrow * 128 + 16 * ((wq >> 1) ^ (((wrow >> 1) & 1) << 2)) + 8 * (wq & 1);
  const int w_wr = wave * kW48BlockBytes + 256 * (lane >> 4) + 64 * ((lane >> 2) & 3) + 16 * (lane & 3);
  auto widen_src = [&](int t, bool v) __attribute__((always_inline)) {
    return (const lds_u8 *)(smem + RING + ((t - t_begin) & (NCS - 1)) * 2 * CB + (v ? CB : 0) + w_rd);
  };
  auto widen_dst = [&](int t, bool v) __attribute__((always_inline)) {
    return smem + (v ? 2 * TILEB : 0) + (t & 1) * TILEB + w_wr;
  };
  // MXFP4: the same lane takes the 4 code bytes of d 8q .. 8q+7 of row
  // wrow (4 rows of 64 bytes per wave: 256 contiguous bytes) and the scale
  // byte of group q / 4; a key past the range end (codes zero, its slot's
  // scale byte possibly anything, NaN included) widens with scale 2^-127 so
  // that its values are zeros.
  const int f4_rd = wrow * 64 + 4 * wq;
  const int f4_sc = 2 * kW48Fp4CodeBytes + (wrow >> 4) * 64 + (wq >> 2) * 16 + (wrow & 15);
  auto f4_stage = [&](int t) __attribute__((always_inline)) {
    return (const lds_u8 *)(smem + RING + ((t - t_begin) & (NCS - 1)) * kW48Fp4StageBytes);
  };
  auto f4_read = [&](int t, bool v, uint32_t &w, uint32_t &e) __attribute__((always_inline)) {
    const lds_u8 *stg = f4_stage(t);
    w = *(const __attribute__((address_space(3))) uint32_t *)(stg + (v ? kW48Fp4CodeBytes : 0) + f4_rd);
    e = *(stg + f4_sc + (v ? 128 : 0));
  };
  auto f4_convert = [&](int t, uint32_t w, uint32_t e) __attribute__((always_inline)) {
    const uint32_t es = t * kW48Step + wrow < kv_hi ? e : 0u;
    return __builtin_bit_cast(uint4, fp4x8_to_bf16x8(w, e8m0_operand(es)));
  };
  auto widen = [&](int t, bool v) __attribute__((always_inline)) {
    if constexpr (FP4) {
      uint32_t w, e;
      f4_read(t, v, w, e);
      lds_store16(widen_dst(t, v), f4_convert(t, w, e));
    } else {
      lds_store16(widen_dst(t, v), __builtin_bit_cast(uint4, e4m3x8_to_bf16x8_hw(lds_load8(widen_src(t, v)))));
    }
  };

  // Matrix-core phase: O += V(t)^T P(t)^T (24 MFMAs, 16 transposing reads),
  // then S(t+1) = K(t+1) Q^T (24 MFMAs, 8 reads): the first three V
  // fragments' reads; per three MFMAs (one fragment's worth) the reads of the
  // fragment three ahead -- V during the value product's first 15 MFMAs, K
  // during its last 9 and the score product's first 3, in the order the score
  // product uses them -- so about three fragments are in flight at any time.
  // bf16 and E4M3 pin that order with scheduling barriers between the groups
  // (left to the scheduler, K fragments were at times requested in the
  // reverse of their use, into the registers the value product frees last,
  // and the score product's first MFMAs waited for them: pinned, ~1%
  // faster); MXFP4 measured 7% slower pinned and leaves the placement of the
  // same groups to the scheduler.
  auto gemm = [&](auto with_qk_tag, const lds_u8 *Vb, const lds_u8 *Kb) __attribute__((always_inline)) {
    constexpr bool with_qk = decltype(with_qk_tag)::value;
    static_assert(NDB == 8 && NCQ == 4 && RB == 3, "the phase's read order is laid out for d 128, 48 rows");
    bf16x8 vf[NDB];
    bf16x8 kf[NCQ][2];
    auto read_v = [&](int db) __attribute__((always_inline)) {
      const bf16x4 h0 = lds_read_tr(Vb + vofs(db));
      const bf16x4 h1 = lds_read_tr(Vb + KB16 + vofs(db));
      vf[db] = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_k = [&](int i) __attribute__((always_inline)) {
      kf[i >> 1][i & 1] = as_bf16x8(lds_load16(Kb + (i & 1) * KB16 + kofs(i >> 1)));
    };
    if constexpr (FP4) {
#pragma unroll
      for (int db = 0; db < NDB; db++) read_v(db);
#pragma unroll
      for (int db = 0; db < NDB; db++)
#pragma unroll
        for (int rb = 0; rb < RB; rb++) o[db][rb] = mfma16x16x32(vf[db], pb[rb], o[db][rb]);
#pragma unroll
      for (int rb = 0; rb < RB; rb++) o[NDB][rb] = mfma16x16x32(ones, pb[rb], o[NDB][rb]);
      if constexpr (with_qk) {
#pragma unroll
        for (int i = 0; i < 2 * NCQ; i++) read_k(i);
#pragma unroll
        for (int c = 0; c < NCQ; c++)
#pragma unroll
          for (int kb = 0; kb < 2; kb++)
#pragma unroll
            for (int rb = 0; rb < RB; rb++)
              S[kb][rb] = mfma16x16x32(kf[c][kb], qf[rb][c], c == 0 ? f32x4{} : S[kb][rb]);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < (with_qk ? 8 : 5); i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      if constexpr (with_qk) {
#pragma unroll
        for (int i = 0; i < 2; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 21, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      }
    } else {
      read_v(0);
      read_v(1);
      read_v(2);
#pragma unroll
      for (int db = 0; db < NDB; db++) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < RB; rb++) o[db][rb] = mfma16x16x32(vf[db], pb[rb], o[db][rb]);
        if (db + 3 < NDB) {
          read_v(db + 3);
        } else if constexpr (with_qk) {
          read_k(2 * (db - 5));
          read_k(2 * (db - 5) + 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RB; rb++) o[NDB][rb] = mfma16x16x32(ones, pb[rb], o[NDB][rb]);
      if constexpr (with_qk) {
        read_k(6);
#pragma unroll
        for (int c = 0; c < NCQ; c++)
#pragma unroll
          for (int kb = 0; kb < 2; kb++) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rb = 0; rb < RB; rb++)
              S[kb][rb] = mfma16x16x32(kf[c][kb], qf[rb][c], c == 0 ? f32x4{} : S[kb][rb]);
            if (c == 0 && kb == 0) read_k(7);
          }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto qk_only = [&](const lds_u8 *Kb) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < NCQ; c++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
        const bf16x8 kf = as_bf16x8(lds_load16(Kb + kb * KB16 + kofs(c)));
#pragma unroll
        for (int rb = 0; rb < RB; rb++) S[kb][rb] = mfma16x16x32(kf, qf[rb][c], c == 0 ? f32x4{} : S[kb][rb]);
      }
  };
  // E4M3: each step's scales reach the scale ring with the step's code
  // requests (slot (s - t_begin) % kW48ScaleSlots, landed when the codes
  // have); the
  // softmax of step t reads those of step t + 1 for the next call.
  float sk_n[2] = {0.f, 0.f}, sv_n[2] = {1.f, 1.f};
  auto read_scales = [&](int t) __attribute__((always_inline)) {
    const lds_u8 *slot = smem + SCB + ((t - t_begin) & (kW48ScaleSlots - 1)) * kW48ScaleSlotBytes;
#pragma unroll
    for (int kb = 0; kb < (SPLIT ? 2 : 1); kb++) {
      sk_n[kb] = *(const __attribute__((address_space(3))) float *)(slot + 256 * kb);
      sv_n[kb] = *(const __attribute__((address_space(3))) float *)(slot + 512 + 256 * kb);
    }
  };
  // m[rb]: the row's reference exponent (base 2).  A score's exponent is
  // fma(q.k, scale * log2 e, -m) (E4M3: fma(q.k_code, scale * log2 e * s_k,
  // -m + log2 s_v)), so a probability is one exp2; m moves up only when a
  // step's maximum exceeds it by kRescaleSlack, and while the row has no
  // weight yet it follows the maximum.
  // E4M3, block 64 (both halves of a step in one block): the scales change
  // every other step, so they are applied per block -- negm then holds
  // -m + log2 s_v of the current block, and the slack test compares against
  // kRescaleSlack + log2 s_v.
  float mul_k = scale_log2, lsv_cur = 0.f, thr = kRescaleSlack;
  auto softmax = [&](auto masked_tag, int t) __attribute__((always_inline)) {
    float mul[2] = {scale_log2, scale_log2}, lsv[2] = {0.f, 0.f};
    if constexpr (FP8 && !SPLIT) {
      if (((t * kW48Step) & (BS - 1)) == 0) {  // a new block: its scales
        mul_k = scale_log2 * sk_n[0];
        const float l_new = __builtin_amdgcn_logf(sv_n[0]);
#pragma unroll
        for (int rb = 0; rb < RB; rb++) negm[rb] += l_new - lsv_cur;
        lsv_cur = l_new;
        thr = kRescaleSlack + l_new;
        const float rv = sv_n[0] * isv[0];  // l: from units of the last block's s_v to this one's
        isv[0] = __builtin_amdgcn_rcpf(sv_n[0]);
#pragma unroll
        for (int rb = 0; rb < RB; rb++) o[NDB][rb][0] *= rv;
      }
      // (every step, although only a block's first step uses them: read
      // conditionally, the values had to be copied out at the branch's join,
      // which made the phase wait for its outstanding LDS and scalar loads
      // right there instead of at its end)
      read_scales(t + 1);
      mul[0] = mul[1] = mul_k;
    } else if constexpr (FP8) {
      float rv[2];
#pragma unroll
      for (int kb = 0; kb < (SPLIT ? 2 : 1); kb++) {
        mul[kb] = scale_log2 * sk_n[kb];
        lsv[kb] = __builtin_amdgcn_logf(sv_n[kb]);
        rv[kb] = sv_n[kb] * isv[kb];  // l: from units of the last step's s_v to this step's
        isv[kb] = __builtin_amdgcn_rcpf(sv_n[kb]);
      }
      if constexpr (!SPLIT) {
        mul[1] = mul[0];
        lsv[1] = lsv[0];
        rv[1] = rv[0];
        isv[1] = isv[0];
      }
      const float rl = SPLIT && g >= 2 ? rv[1] : rv[0];
#pragma unroll
      for (int rb = 0; rb < RB; rb++) o[NDB][rb][0] *= rl;
      read_scales(t + 1);  // in flight during the rest of the phase
    }
#pragma unroll
    for (int rb = 0; rb < RB; rb++)
#pragma unroll
      for (int kb = 0; kb < 2; kb++) {
        const float add = SPLIT ? negm[rb] + lsv[kb] : negm[rb];
#pragma unroll
        for (int r = 0; r < 4; r++) S[kb][rb][r] = __builtin_fmaf(S[kb][rb][r], mul[kb], add);
      }
    if constexpr (decltype(masked_tag)::value) {
      const int key0 = t * kW48Step + 4 * g;
#pragma unroll
      for (int rb = 0; rb < RB; rb++) {
        const int lim = min(it.pos0 + ((wave * 48 + rb * 16 + c16) >> a.lg), kv_hi - 1);
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
#pragma unroll
          for (int r = 0; r < 4; r++) S[kb][rb][r] = key0 + kb * 16 + r <= lim ? S[kb][rb][r] : -INFINITY;
      }
    }
    // S holds s - m (E4M3: plus log2 s_v).  A row's maximum is needed only
    // when m has to move: test the lane's own maximum first, reduce across
    // the row's four lanes only if some lane exceeds the slack (rare once m
    // has settled) or some row has no weight yet (m then follows the row
    // maximum).
    auto rescale = [&]() __attribute__((always_inline)) {
      bool live = true;
#pragma unroll
      for (int rb = 0; rb < RB; rb++) {
        float lmx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
          float k = -INFINITY;
#pragma unroll
          for (int r = 0; r < 4; r++) k = fmaxf(k, S[kb][rb][r]);
          lmx = fmaxf(lmx, SPLIT ? k - lsv[kb] : k);
        }
        if constexpr (FP8 && !SPLIT) lmx -= lsv_cur;
        const float mx = xor32_max(xor16_max(lmx));
        const bool empty = (SPLIT ? xor32_sum(o[NDB][rb][0]) : o[NDB][rb][0]) == 0.f;
        const bool mv = mx > kRescaleSlack || (empty && mx > -INFINITY);
        live = live && (!empty || mx > -INFINITY);
        const float shift = mv ? mx : 0.f;
        const float alpha = fast_exp2(-shift);
        negm[rb] -= shift;
#pragma unroll
        for (int db = 0; db <= NDB; db++) o[db][rb] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; kb++) S[kb][rb] -= shift;
      }
      all_live = __builtin_amdgcn_readfirstlane(__all(live));
    };
    // the lane's maximum as a shallow tree (a serial chain of max3 would put
    // a dozen dependent instructions on the phase's critical path)
    float kmx[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      float r4[RB];
#pragma unroll
      for (int rb = 0; rb < RB; rb++)
        r4[rb] = fmaxf(fmaxf(S[kb][rb][0], S[kb][rb][1]), fmaxf(S[kb][rb][2], S[kb][rb][3]));
      kmx[kb] = fmaxf(fmaxf(r4[0], r4[1]), r4[2]);
      if constexpr (SPLIT) kmx[kb] -= lsv[kb];
    }
    const float mx = fmaxf(kmx[0], kmx[1]);
    if (__any(mx > (FP8 && !SPLIT ? thr : kRescaleSlack)) || !all_live) rescale();
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        pb[rb][r] = (__bf16)fast_exp2(S[0][rb][r]);
        pb[rb][4 + r] = (__bf16)fast_exp2(S[1][rb][r]);
      }
    }
    // the phase's scalar loads (block ids, scales) have landed: with none
    // outstanding, the compiler's LDS waits in the matrix-core phase that
    // follows count reads precisely instead of waiting for all of them
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };

  // prologue.  bf16: NST-1 steps requested, step t0 waited.  E4M3: NCS steps
  // requested, t0 and t0+1 waited, then K(t0), V(t0), K(t0+1) widened.
  if constexpr (CODED) {
#pragma unroll
    for (int k = 0; k < NCS; k++) issue();
    if (FP8 && !sc_loader)
      PA_WAIT_VMCNT(NCS - 2);
    else
      PA_WAIT_VMCNT(REQ * (NCS - 2));
    wg_barrier();
    widen(t_begin, false);
    widen(t_begin, true);
    widen(t_begin + 1, false);  // (past the range end: a tile nothing reads)
    if constexpr (FP8) read_scales(t_begin);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the widened tiles are written
    wg_barrier();
  } else {
#pragma unroll
    for (int k = 0; k < NST - 1; k++) issue();
    PA_WAIT_VMCNT(2 * (NST - 2));
    wg_barrier();
  }
  qk_only(ktile(t_begin));
  // Each step opens once this wave's share of what the step reads has landed:
  // bf16, step t+1 (steps t+2 .. t+NST-2 may be in flight; step t+NST-1 is
  // requested into the stage step t-1 left); E4M3, the codes of step t+2
  // (steps t+3 .. t+NCS-1 in flight; t+NCS requested into the stage of step
  // t, whose codes were widened before), and the work-group then widens
  // K(t+2) and V(t+1) during the step -- the tiles the next step reads.
  // With one barrier per step the groups stay half a step apart: the
  // barrier of step t finds group 0 about to start its matrix-core phase and
  // group 1 its vector phase.
  auto open_step = [&]() __attribute__((always_inline)) {
    if constexpr (CODED) {
      if (FP8 && !sc_loader)
        PA_WAIT_VMCNT(NCS - 3);
      else
        PA_WAIT_VMCNT(REQ * (NCS - 3));
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's widened chunks are written
    } else {
      PA_WAIT_VMCNT(2 * (NST - 3));
    }
    wg_barrier();
  };
  // E4M3 widening of K(t+2) and V(t+1) around a softmax: the code reads go
  // out first, the conversions and writes follow the softmax.  (Past the
  // range end these touch only tiles nothing reads: no branch needed.)
  uint2 wk = {}, wv = {};
  uint32_t ek = 0, ev = 0;
  auto widen_read = [&](int t) __attribute__((always_inline)) {
    if constexpr (FP4) {
      f4_read(t + 2, false, wk.x, ek);
      f4_read(t + 1, true, wv.x, ev);
    } else if constexpr (FP8) {
      wk = lds_load8(widen_src(t + 2, false));
      wv = lds_load8(widen_src(t + 1, true));
    }
  };
  auto widen_write = [&](int t) __attribute__((always_inline)) {
    if constexpr (FP4) {
      lds_store16(widen_dst(t + 2, false), f4_convert(t + 2, wk.x, ek));
      lds_store16(widen_dst(t + 1, true), f4_convert(t + 1, wv.x, ev));
    } else if constexpr (FP8) {
      lds_store16(widen_dst(t + 2, false), __builtin_bit_cast(uint4, e4m3x8_to_bf16x8_hw(wk)));
      lds_store16(widen_dst(t + 1, true), __builtin_bit_cast(uint4, e4m3x8_to_bf16x8_hw(wv)));
    }
  };
  auto prio_hi = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
  };
  auto prio_lo = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
  };
  // Steps before t_full need no causal mask: each group's loop runs in two
  // parts, the mask code only in the second, so the first has no branch.
  const std::false_type open{};
  const std::true_type masked{};
  auto softmax_rt = [&](int t) __attribute__((always_inline)) {
    if (t >= t_full) softmax(masked, t);
    else softmax(open, t);
  };
  if (grp == 0) {
    softmax_rt(t_begin);
    int t = t_begin;
    auto body = [&](auto mtag) __attribute__((always_inline)) {
      open_step();
      prio_hi();
      gemm(std::true_type{}, vtile(t), ktile(t + 1));  // phase A: matrix cores
      prio_lo();
      issue();                                          // phase B: loads, widening, vector ALUs
      widen_read(t);
      softmax(mtag, t + 1);
      widen_write(t);
    };
    for (const int t_open = min(t_full, t_end) - 1; t < t_open; t++) body(open);
    for (; t + 1 < t_end; t++) body(masked);
    open_step();
    gemm(std::false_type{}, vtile(t), nullptr);
    issue();
  } else {
    int t = t_begin;
    auto body = [&](auto mtag) __attribute__((always_inline)) {
      open_step();
      issue();
      widen_read(t);
      softmax(mtag, t);                                 // phase A: vector ALUs
      widen_write(t);
      prio_hi();
      gemm(std::true_type{}, vtile(t), ktile(t + 1));  // phase B: matrix cores
      prio_lo();
    };
    for (const int t_open = min(t_full, t_end - 1); t < t_open; t++) body(open);
    for (; t + 1 < t_end; t++) body(masked);
    open_step();
    issue();
    softmax_rt(t);
    gemm(std::false_type{}, vtile(t), nullptr);
  }
  PA_WAIT_VMCNT(0);  // the trailing (empty) step requests complete before exit

#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    const int row = wave * 48 + rb * 16 + c16;
    const int tok = row >> a.lg, gq = row & (a.group - 1);
    float lt = o[NDB][rb][0];
    if constexpr (FP8) {
      lt *= SPLIT && g >= 2 ? isv[1] : isv[0];  // back from units of the last step's s_v
      if constexpr (SPLIT) lt = xor32_sum(lt);
    }
    if (tok >= nq) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float mrow = -negm[rb] + (FP8 && !SPLIT ? lsv_cur : 0.f);
    const float lse2 = lt > 0.f ? mrow + __log2f(lt) : -INFINITY;
    if (it.part < 0) {
      const int64_t orow = (int64_t)(it.row0 + tok) * a.hq + kvh * a.group + gq;
      unsigned char *op = (unsigned char *)a.out + orow * D * 2;
#pragma unroll
      for (int db = 0; db < NDB; db++) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = (__bf16)(o[db][rb][r] * inv);
        *(bf16x4 *)(op + (16 * db + 4 * g) * 2) = v;
      }
      if (a.lse_out && g == 0) a.lse_out[orow] = lse2 * kLn2;
    } else {
      float *prow = a.part_o + ((int64_t)it.part * kW48TileRows + row) * D;
#pragma unroll
      for (int db = 0; db < NDB; db++) *(f32x4 *)(prow + 16 * db + 4 * g) = o[db][rb] * inv;
      if (g == 0) a.part_lse[(int64_t)it.part * kW48TileRows + row] = lse2;
    }
  }
}

template <int BS, int FMT>
__global__ __launch_bounds__(512, 1) void prefill_w48_kernel(AttnArgs a) {
  constexpr int RING = FMT == kKvE4m3 ? kW48Fp8Lds : FMT == kKvMxfp4 ? kW48Fp4Lds : kW48Stages * 2 * kW48TileBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[RING];
  const int first = a.wg_first ? a.wg_first[blockIdx.x] : (int)blockIdx.x;
  const int last = a.wg_first ? a.wg_first[blockIdx.x + 1] : (int)blockIdx.x + 1;
  for (int i = first; i < last; i++) {
    if (i > first) __syncthreads();  // LDS of the previous item no longer read or written
    w48_item<BS, FMT>(a, a.items[i], (lds_u8 *)smem_raw);
  }
}

// The four waves of a decode work-group hold softmax states (m in log2
// units, per-lane partial l, o[d-block]) over disjoint keys of one item's
// 16 rows; combine them through LDS and write the rows (or the item's partial).
// PAIRED (the MXFP4 kernel): o[2j] holds d = 32j + 2(4 q4 + r), o[2j + 1]
// the odd d next to it; otherwise o[db] holds d = 16 db + 4 q4 + r.
template <int D, int NW = 4, bool PAIRED = false>
__device__ __forceinline__ void decode_combine(const AttnArgs &a, const Item &it, unsigned char *smem_raw,
                                               float m, float l, const f32x4 (&o)[D / 16]) {
  constexpr int ND = D / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  l = xor16_sum(l);
  l = xor32_sum(l);
  __syncthreads();
  float *red_o = (float *)smem_raw;                  // [NW][16][D]
  float *red_m = red_o + NW * 16 * D;                // [NW][16]
  float *red_l = red_m + NW * 16;                    // [NW][16]
  if constexpr (PAIRED) {
#pragma unroll
    for (int j = 0; j < ND / 2; j++) {
      const f32x4 lo = o[2 * j], hi = o[2 * j + 1];
      float *dst = red_o + (wave * 16 + n) * D + 32 * j + 8 * q4;
      *(f32x4 *)dst = f32x4{lo[0], hi[0], lo[1], hi[1]};
      *(f32x4 *)(dst + 4) = f32x4{lo[2], hi[2], lo[3], hi[3]};
    }
  } else {
#pragma unroll
    for (int db = 0; db < ND; db++)
      *(f32x4 *)(red_o + (wave * 16 + n) * D + db * 16 + 4 * q4) = o[db];
  }
  if (q4 == 0) {
    red_m[wave * 16 + n] = m;
    red_l[wave * 16 + n] = l;
  }
  __syncthreads();
  const int rows = it.nq << a.lg;
  for (int idx = tid; idx < 16 * D; idx += 64 * NW) {
    const int cn = idx / D, e = idx % D;
    if (cn >= rows) continue;
    float M = red_m[cn];
#pragma unroll
    for (int w = 1; w < NW; w++) M = fmaxf(M, red_m[w * 16 + cn]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      const float sc = fast_exp2(red_m[w * 16 + cn] - M);
      L += sc * red_l[w * 16 + cn];
      O += sc * red_o[(w * 16 + cn) * D + e];
    }
    const float val = L > 0.f ? O / L : 0.f;
    const int ctok = cn >> a.lg, cg = cn & (a.group - 1);
    const int64_t orow = (int64_t)(it.row0 + ctok) * a.hq + it.kvh * a.group + cg;
    if (it.part < 0) {
      ((__bf16 *)a.out)[orow * D + e] = (__bf16)val;
      if (e == 0 && a.lse_out) a.lse_out[orow] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      a.part_o[((int64_t)it.part * kDecodeRows + cn) * D + e] = val;
      if (e == 0)
        a.part_lse[(int64_t)it.part * kDecodeRows + cn] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// =============================================================================
// Decode (and short increments, tokens x G <= 16): one work-group per item;
// its four waves stream disjoint 64-key tiles of the item's range, each with
// its own softmax state, and are combined through LDS at the end.  K goes
// straight from HBM into MFMA A-operand registers; V passes through a
// per-wave LDS tile for the transposed read.  The next tile's K and V are in
// flight while the current one is computed; block ids are wave-uniform scalar
// loads, so waiting for them never waits for the K/V stream.
template <int D, bool FP8>
struct DecodeRegs {
  static constexpr int NCK = D / 32;  // 16-byte (bf16) or 8-byte (E4M3) loads per row slice
  typedef typename std::conditional<FP8, uint2, uint4>::type chunk_t;
  chunk_t k[4][NCK];
  chunk_t v[4][NCK];
  float ksc[4], vsc[4];
};

template <int D, int BS, bool FP8>
__global__ __launch_bounds__(256, 1) void decode_kernel(AttnArgs a) {
  constexpr int NCK = D / 32;   // score MFMAs per 16-key block (k = 32 each)
  constexpr int ND = D / 16;    // 16-wide d blocks of the output
  typedef LdsRow<D> L;
  constexpr int WAVEB = kKeyTile * L::bytes;
  typedef DecodeRegs<D, FP8> Regs;

  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[4 * WAVEB];
  lds_u8 *smem = (lds_u8 *)smem_raw;

  const Item it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int tok = n >> a.lg, g = n & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;
  lds_u8 *Vw = smem + wave * WAVEB;

  // Q as the B operand of K * Q^T (16x16x32): for product c the lane holds
  // q[n][32c + 8*q4 .. +7], matching the K slice its A operand holds.
  bf16x8 qf[NCK];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCK; c++) {
      uint4 v = active ? gload16(qrow + (32 * c + 8 * q4) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = as_bf16x8(v);
    }
  }

  float m = kNegBig, l = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x4{};

  const int32_t *bt = a.bt + (int64_t)it.seq * a.max_blocks;
  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const int t_first = it.kv_lo / kKeyTile;
  const int ntiles = (it.kv_hi - it.kv_lo + kKeyTile - 1) / kKeyTile;
  const int last_blk = (it.kv_hi - 1) / BS;
  const int lim = min(pos, it.kv_hi - 1);
  // tiles below t_full need no mask
  const int t_full = min(it.pos0 + 1, it.kv_hi) / kKeyTile;

  // Issue the loads of tile t.  This lane: key row kb*16 + n, elements
  // 32c + 8*q4 .. +7 for c = 0..NCK-1, so that each load instruction reads a
  // contiguous 64-byte (bf16) slice of every key row of the block.
  auto load = [&](Regs &R, int t) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int bidx = min((t * kKeyTile + kb * 16) / BS, last_blk);  // wave-uniform
      const int64_t blk = bt[bidx];
      const int off = (BS == 16) ? n : kb * 16 + n;
      const int64_t e = ((blk * hkv + it.kvh) * BS + off) * D + 8 * q4;
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        if constexpr (FP8) {
          R.k[kb][c] = gload8(kc + e + 32 * c);
          R.v[kb][c] = gload8(vc + e + 32 * c);
        } else {
          R.k[kb][c] = gload16(kc + (e + 32 * c) * 2);
          R.v[kb][c] = gload16(vc + (e + 32 * c) * 2);
        }
      }
      if constexpr (FP8) {
        R.ksc[kb] = ((const float *)a.c.ks)[blk * hkv + it.kvh];
        R.vsc[kb] = ((const float *)a.c.vs)[blk * hkv + it.kvh];
      }
    }
  };

  auto compute = [&](auto masked, Regs &R, int t) {
    constexpr bool MASK = decltype(masked)::value;
    const int kbase = t * kKeyTile;
    // V tile -> this wave's LDS (rows beyond the range zeroed)
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int r = kb * 16 + n;
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        uint4 v;
        if constexpr (FP8)
          v = e4m3x8_to_bf16x8(R.v[kb][c]);
        else
          v = R.v[kb][c];
        if (MASK && kbase + r >= it.kv_hi) v = make_uint4(0, 0, 0, 0);
        lds_store16(Vw + L::off(r, 4 * c + q4), v);
      }
    }
    // S^T = K * Q^T per 16-key block; element r of block kb is key kb*16 + 4*q4 + r
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        bf16x8 kf;
        if constexpr (FP8)
          kf = as_bf16x8(e4m3x8_to_bf16x8(R.k[kb][c]));
        else
          kf = as_bf16x8(R.k[kb][c]);
        s[kb] = c == 0 ? mfma16x16x32(kf, qf[0], f32x4{}) : mfma16x16x32(kf, qf[c], s[kb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        if (MASK) {
          const int key = kbase + kb * 16 + 4 * q4 + r;
          s[kb][r] = key <= lim ? s[kb][r] : -INFINITY;
        }
        if constexpr (FP8) s[kb][r] *= R.ksc[kb];
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = xor16_max(mx);
    mx = xor32_max(mx);
    const float mxs = mx * a.scale_log2;
    if (__any(mxs > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mxs);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++) o[db] *= alpha;
    }
    const float nm = -m;
    float psum = 0.f;
    bf16x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, nm));
        psum += p;
        float pv = p;
        if constexpr (FP8) pv *= R.vsc[kb];
        pb[kb][r] = (__bf16)pv;
      }
    l += psum;

    // the wave's own LDS writes above must land before its transpose reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int vrow = kb * 16 + 4 * q4 + (n >> 2);
#pragma unroll
      for (int db = 0; db < ND; db++) {
        const int d0 = db * 16 + 4 * (n & 3);
        bf16x4 af = lds_read_tr(Vw + L::off(vrow, d0 >> 3) + (d0 & 7) * 2);
        o[db] = mfma16x16x16(af, pb[kb], o[db]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto step = [&](Regs &R, int t) {
    if (t < t_full)
      compute(FullTile{}, R, t);
    else
      compute(MaskedTile{}, R, t);
  };

  Regs A, B;
  int tw = wave;
  if (tw < ntiles) load(A, t_first + tw);
  while (tw < ntiles) {
    if (tw + 4 < ntiles) load(B, t_first + tw + 4);
    step(A, t_first + tw);
    tw += 4;
    if (tw >= ntiles) break;
    if (tw + 4 < ntiles) load(A, t_first + tw + 4);
    step(B, t_first + tw);
    tw += 4;
  }

  decode_combine<D>(a, it, smem_raw, m, l, o);
}

// =============================================================================
// Decode for bf16 KV, head_dim 128, streamed through LDS.  One work-group per
// item; wave w takes the 16-key slices w, w+4, w+8, ... of the item's range
// with its own softmax state, combined through LDS at the end as above.  A
// slice of K (and of V) is 4 KB contiguous in the cache (16 rows of one
// block; the item's block ids are staged in LDS, items span at most
// kMaxDecItemKeys keys), moved into the wave's own 4-stage LDS ring by four LDS-filling
// buffer loads with the non-temporal hint (each byte is read once): full 1 KB
// requests, which stream from HBM faster than register loads of 64-byte row
// slices.  No wave reads another wave's ring, so only vmcnt waits are needed.
// K is read back as the A operand of v_mfma_f32_16x16x32_bf16 (lane: key n,
// d 32c + 8*q4 .. +7), V with ds_read_b64_tr_b16 as the A operand of
// v_mfma_f32_16x16x16_bf16 (lane: d 16*db + n, keys 4*q4 .. +3); LDS rows
// of 256 bytes with 16-byte chunk q of row r at q ^ ((r&7)<<1 | (r>>3)&1).

constexpr int kDecSlice = 16;                      // keys per wave step
constexpr int kDecSliceBytes = kDecSlice * 128 * 2;  // K (or V) of one slice, 4 KB
// waves per work-group and ring stages per wave of the bf16 decode items (the
// decode launch and the claiming decode launch): 8 x 2 and 4 x 4 stream the
// same over the whole chip (64 sessions: 5.629 against 5.628 ms), but beside
// a prefill 8 x 2 streams more per CU (the co-scheduled mixed step: 11.02 ms
// with 48 decode CUs against 11.33 ms at best with 4 x 4; with prefix groups
// 11.16 against 11.65 ms).  The cascade launch (and the claiming launch with
// cascade items) takes the same shape, except for 64-row cascade tiles,
// whose member rows need the registers of four waves (eight spill)
#ifndef PA_DEC_WAVES
#define PA_DEC_WAVES 8
#endif
#ifndef PA_DEC_STAGES
#define PA_DEC_STAGES 2
#endif
constexpr int kDecWaves = PA_DEC_WAVES;
constexpr int kDecStages = PA_DEC_STAGES;
constexpr int cascade_waves(int nrb) { return nrb >= 4 ? 4 : kDecWaves; }
constexpr int cascade_stages(int nrb) { return nrb >= 4 ? 4 : kDecStages; }

template <int BS, int NW, int NST>
__device__ __forceinline__ void decode_dma_item(const AttnArgs &a, const Item it, unsigned char *smem_raw,
                                                int *bt_lds) {
  constexpr int D = 128;
  constexpr int NCK = D / 32;  // score MFMAs per slice
  constexpr int ND = D / 16;   // 16-wide d blocks of the output
  constexpr int SB = kDecSliceBytes;
  static_assert(NW * NST * 2 * SB >= NW * 16 * (D + 2) * 4, "combine scratch");
  lds_u8 *smem = (lds_u8 *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int tok = n >> a.lg, g = n & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;
  const int kv_lo = it.kv_lo, kv_hi = it.kv_hi;

  bf16x8 qf[NCK];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCK; c++) {
      uint4 v = active ? gload16(qrow + (32 * c + 8 * q4) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = as_bf16x8(v);
    }
  }

  float m = kNegBig, l = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x4{};

  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const int n_slices = (kv_hi - kv_lo + kDecSlice - 1) / kDecSlice;
  const int nw = n_slices > wave ? (n_slices - wave + NW - 1) / NW : 0;  // this wave's slices
  const int blk0 = kv_lo / BS;
  const int last_blk = (kv_hi - 1) / BS;
  const int lim = min(pos, kv_hi - 1);
  {  // stage the item's block ids in LDS: a global load inside the loop would
     // make the compiler wait for every outstanding load, the K/V stream too
    const int32_t *btr = a.bt + (int64_t)it.seq * a.max_blocks + blk0;
    for (int i = tid; i <= last_blk - blk0; i += 64 * NW) bt_lds[i] = btr[i];
  }
  // Q and the block ids have landed (stated explicitly: otherwise the
  // compiler, which does not see the stream's loads, places its wait for Q
  // inside the loop as a full vmcnt(0))
  PA_WAIT_VMCNT(0);
  __syncthreads();
  const int lim_min = min(it.pos0, kv_hi - 1);  // slices ending at or below it need no mask

  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; q++)
    voff[q] = (lane >> 4) * 256 + (((lane & 15) ^ swz(4 * q + (lane >> 4))) << 4);
  const uint32_t ring = smem_addr + wave * NST * 2 * SB;
  lds_u8 *ring_p = smem + wave * NST * 2 * SB;

  auto slice_key = [&](int k) { return kv_lo + kDecSlice * (wave + NW * k); };
  // slice k's 4 KB of K and of V into stage k % NST; slices past this wave's
  // share are requested with an empty buffer range (nothing is read), which
  // keeps the vmcnt accounting uniform
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int key0 = slice_key(min(k, max(nw - 1, 0)));
    const int64_t blk = __builtin_amdgcn_readfirstlane(bt_lds[min(key0 / BS, last_blk) - blk0]);
    const int64_t base = ((blk * hkv + it.kvh) * BS + key0 % BS) * (D * 2);
    const uint64_t ka = (uint64_t)(kc + base), va = (uint64_t)(vc + base);
    const uint32_t st = ring + (k % NST) * 2 * SB;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int nrec = __builtin_amdgcn_readfirstlane(k < nw ? min(max(kv_hi - (key0 + 4 * q), 0), 4) * (D * 2) : 0);
      const uint64_t kq = ka + q * 4 * D * 2, vq = va + q * 4 * D * 2;
      const i32x4_t rk = {__builtin_amdgcn_readfirstlane((int)(uint32_t)kq),
                          __builtin_amdgcn_readfirstlane((int)((kq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      const i32x4_t rv = {__builtin_amdgcn_readfirstlane((int)(uint32_t)vq),
                          __builtin_amdgcn_readfirstlane((int)((vq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      dma_load16_nt(rk, voff[q], st + q * 1024);
      dma_load16_nt(rv, voff[q], st + SB + q * 1024);
    }
  };

  const int vr = 4 * q4 + (n >> 2);
  const int vbase = vr * 256 + ((((n & 3) >> 1) ^ swz(vr)) << 4) + (n & 1) * 8;
  // Slice k is read from LDS into registers first; its stage is then free
  // and slice k + NST is requested into it before the arithmetic, so all NST
  // stages are in flight while the wave computes.
  auto compute = [&](int k) __attribute__((always_inline)) {
    const lds_u8 *Ks = ring_p + (k % NST) * 2 * SB;
    const lds_u8 *Vs = Ks + SB;
    const int key0 = slice_key(k);
    uint4 kraw[NCK];
    bf16x4 vraw[ND];
#pragma unroll
    for (int c = 0; c < NCK; c++) kraw[c] = lds_load16(Ks + n * 256 + (((4 * c + q4) ^ swz(n)) << 4));
#pragma unroll
    for (int db = 0; db < ND; db++) vraw[db] = lds_read_tr(Vs + (vbase ^ (db << 5)));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage's bytes are in registers
    __builtin_amdgcn_sched_barrier(0);
    issue(k + NST);
    f32x4 s;
#pragma unroll
    for (int c = 0; c < NCK; c++) s = mfma16x16x32(as_bf16x8(kraw[c]), qf[c], c == 0 ? f32x4{} : s);
    if (key0 + kDecSlice - 1 > lim_min) {
#pragma unroll
      for (int r = 0; r < 4; r++) s[r] = key0 + 4 * q4 + r <= lim ? s[r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = xor32_max(xor16_max(mx));
    const float mxs = mx * a.scale_log2;
    if (__any(mxs > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mxs);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++) o[db] *= alpha;
    }
    const float nm = -m;
    bf16x4 pb;
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const float p = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, nm));
      l += p;
      pb[r] = (__bf16)p;
    }
#pragma unroll
    for (int db = 0; db < ND; db++) o[db] = mfma16x16x16(vraw[db], pb, o[db]);
  };

#pragma unroll
  for (int k = 0; k < NST; k++) issue(k);
  for (int k = 0; k < nw; k++) {
    PA_WAIT_VMCNT(8 * (NST - 1));  // slice k has landed (slices k+1 .. k+NST-1 may be in flight)
    compute(k);                    // requests slice k + NST into slice k's stage
  }
  PA_WAIT_VMCNT(0);

  decode_combine<D, NW>(a, it, smem_raw, m, l, o);
}

template <int BS, int NW, int NST>
__global__ __launch_bounds__(64 * NW, 1) void decode_dma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[NW * NST * 2 * kDecSliceBytes];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  decode_dma_item<BS, NW, NST>(a, a.items[blockIdx.x], smem_raw, bt_lds);
}

// =============================================================================
// Shared-prefix cascade for bf16 KV, head_dim 128: the decode rows of the
// members of a prefix group (up to 64 rows: NRB blocks of 16, G rows per
// member) against one key range of their shared prefix.  The keys stream
// exactly as in decode_dma_kernel (per-wave LDS rings of 16-key slices,
// non-temporal LDS-filling loads), but each slice now feeds NRB score and
// value products instead of one: the prefix is read once for all members, and
// the work per byte grows NRB-fold.  No causal mask is needed (the shared
// prefix lies before every member's own token); keys past the range end are
// masked.  The four waves' states are combined per row block through LDS and
// each member's rows go to its partial slot (row g of the slot = its head g).
template <int BS, int NRB, int NW, int NST>
__device__ __forceinline__ void cascade_item(const AttnArgs &a, const CascadeItem it, const CascadeMember *members,
                                             unsigned char *smem_raw, int *bt_lds) {
  constexpr int D = 128;
  constexpr int NCK = D / 32;
  constexpr int ND = D / 16;
  constexpr int SB = kDecSliceBytes;
  static_assert(NW * NST * 2 * SB >= NW * 16 * (D + 2) * 4, "combine scratch");
  lds_u8 *smem = (lds_u8 *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int hkv = a.c.hkv;
  const int kv_lo = it.kv_lo, kv_hi = it.kv_hi;

  bf16x8 qf[NRB][NCK];
#pragma unroll
  for (int rb = 0; rb < NRB; rb++) {
    const int r = rb * 16 + n;
    const int mi = r >> a.lg, g = r & (a.group - 1);
    const bool active = mi < it.nmem;
    const int row0 = active ? members[it.mem0 + mi].row0 : 0;
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)row0 * a.hq + it.kvh * a.group + g) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCK; c++) {
      uint4 v = active ? gload16(qrow + (32 * c + 8 * q4) * 2) : make_uint4(0, 0, 0, 0);
      qf[rb][c] = as_bf16x8(v);
    }
  }
  float m[NRB], l[NRB];
  f32x4 o[NRB][ND];
#pragma unroll
  for (int rb = 0; rb < NRB; rb++) {
    m[rb] = kNegBig;
    l[rb] = 0.f;
#pragma unroll
    for (int i = 0; i < ND; i++) o[rb][i] = f32x4{};
  }

  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const int n_slices = (kv_hi - kv_lo + kDecSlice - 1) / kDecSlice;
  const int nw = n_slices > wave ? (n_slices - wave + NW - 1) / NW : 0;
  const int blk0 = kv_lo / BS;
  const int last_blk = (kv_hi - 1) / BS;
  {
    const int32_t *btr = a.bt + (int64_t)it.seq * a.max_blocks + blk0;
    for (int i = tid; i <= last_blk - blk0; i += 64 * NW) bt_lds[i] = btr[i];
  }
  PA_WAIT_VMCNT(0);
  __syncthreads();

  auto swz = [](int r) { return ((r & 7) << 1) | ((r >> 3) & 1); };
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; q++)
    voff[q] = (lane >> 4) * 256 + (((lane & 15) ^ swz(4 * q + (lane >> 4))) << 4);
  const uint32_t ring = smem_addr + wave * NST * 2 * SB;
  lds_u8 *ring_p = smem + wave * NST * 2 * SB;
  auto slice_key = [&](int k) { return kv_lo + kDecSlice * (wave + NW * k); };
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int key0 = slice_key(min(k, max(nw - 1, 0)));
    const int64_t blk = __builtin_amdgcn_readfirstlane(bt_lds[min(key0 / BS, last_blk) - blk0]);
    const int64_t base = ((blk * hkv + it.kvh) * BS + key0 % BS) * (D * 2);
    const uint64_t ka = (uint64_t)(kc + base), va = (uint64_t)(vc + base);
    const uint32_t st = ring + (k % NST) * 2 * SB;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int nrec = __builtin_amdgcn_readfirstlane(k < nw ? min(max(kv_hi - (key0 + 4 * q), 0), 4) * (D * 2) : 0);
      const uint64_t kq = ka + q * 4 * D * 2, vq = va + q * 4 * D * 2;
      const i32x4_t rk = {__builtin_amdgcn_readfirstlane((int)(uint32_t)kq),
                          __builtin_amdgcn_readfirstlane((int)((kq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      const i32x4_t rv = {__builtin_amdgcn_readfirstlane((int)(uint32_t)vq),
                          __builtin_amdgcn_readfirstlane((int)((vq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      dma_load16_nt(rk, voff[q], st + q * 1024);
      dma_load16_nt(rv, voff[q], st + SB + q * 1024);
    }
  };
  const int vr = 4 * q4 + (n >> 2);
  const int vbase = vr * 256 + ((((n & 3) >> 1) ^ swz(vr)) << 4) + (n & 1) * 8;
  auto compute = [&](int k) __attribute__((always_inline)) {
    const lds_u8 *Ks = ring_p + (k % NST) * 2 * SB;
    const lds_u8 *Vs = Ks + SB;
    const int key0 = slice_key(k);
    uint4 kraw[NCK];
    bf16x4 vraw[ND];
#pragma unroll
    for (int c = 0; c < NCK; c++) kraw[c] = lds_load16(Ks + n * 256 + (((4 * c + q4) ^ swz(n)) << 4));
#pragma unroll
    for (int db = 0; db < ND; db++) vraw[db] = lds_read_tr(Vs + (vbase ^ (db << 5)));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage's bytes are in registers
    __builtin_amdgcn_sched_barrier(0);
    issue(k + NST);
    const bool tail = key0 + kDecSlice > kv_hi;
#pragma unroll
    for (int rb = 0; rb < NRB; rb++) {
      f32x4 s;
#pragma unroll
      for (int c = 0; c < NCK; c++) s = mfma16x16x32(as_bf16x8(kraw[c]), qf[rb][c], c == 0 ? f32x4{} : s);
      if (tail) {
#pragma unroll
        for (int r = 0; r < 4; r++) s[r] = key0 + 4 * q4 + r < kv_hi ? s[r] : -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = xor32_max(xor16_max(mx));
      const float mxs = mx * a.scale_log2;
      if (__any(mxs > m[rb] + kRescaleSlack)) {
        const float m_new = fmaxf(m[rb], mxs);
        const float alpha = fast_exp2(m[rb] - m_new);
        m[rb] = m_new;
        l[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < ND; db++) o[rb][db] *= alpha;
      }
      const float nm = -m[rb];
      bf16x4 pb;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float p = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, nm));
        l[rb] += p;
        pb[r] = (__bf16)p;
      }
#pragma unroll
      for (int db = 0; db < ND; db++) o[rb][db] = mfma16x16x16(vraw[db], pb, o[rb][db]);
    }
  };
#pragma unroll
  for (int k = 0; k < NST; k++) issue(k);
  for (int k = 0; k < nw; k++) {
    PA_WAIT_VMCNT(8 * (NST - 1));
    compute(k);
  }
  PA_WAIT_VMCNT(0);

  // combine the four waves' states one row block at a time through LDS
  float *red_o = (float *)smem_raw;        // [NW][16][D]
  float *red_m = red_o + NW * 16 * D;      // [NW][16]
  float *red_l = red_m + NW * 16;          // [NW][16]
#pragma unroll
  for (int rb = 0; rb < NRB; rb++) {
    float lt = xor32_sum(xor16_sum(l[rb]));
    __syncthreads();
#pragma unroll
    for (int db = 0; db < ND; db++) *(f32x4 *)(red_o + (wave * 16 + n) * D + db * 16 + 4 * q4) = o[rb][db];
    if (q4 == 0) {
      red_m[wave * 16 + n] = m[rb];
      red_l[wave * 16 + n] = lt;
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * D; idx += 64 * NW) {
      const int cn = idx / D, e = idx % D;
      const int r = rb * 16 + cn;
      const int mi = r >> a.lg, g = r & (a.group - 1);
      if (mi >= it.nmem) continue;
      float M = red_m[cn];
#pragma unroll
      for (int w = 1; w < NW; w++) M = fmaxf(M, red_m[w * 16 + cn]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) {
        const float sc = fast_exp2(red_m[w * 16 + cn] - M);
        L += sc * red_l[w * 16 + cn];
        O += sc * red_o[(w * 16 + cn) * D + e];
      }
      const int slot = members[it.mem0 + mi].part;
      a.part_o[((int64_t)slot * kDecodeRows + g) * D + e] = L > 0.f ? O / L : 0.f;
      if (e == 0) a.part_lse[(int64_t)slot * kDecodeRows + g] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// The decode launch of a step with shared-prefix groups: work-groups
// [0, n_cascade) run the cascade items (first: each carries several members'
// rows), the rest the ordinary decode items, in one grid.
template <int BS, int NRB>
__global__ __launch_bounds__(64 * cascade_waves(NRB), 1) void decode_cascade_kernel(AttnArgs a, const CascadeItem *citems,
                                                                const CascadeMember *members, int n_cascade) {
  constexpr int NW = cascade_waves(NRB), NST = cascade_stages(NRB);
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[NW * NST * 2 * kDecSliceBytes];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  if ((int)blockIdx.x < n_cascade)
    cascade_item<BS, NRB, NW, NST>(a, citems[blockIdx.x], members, smem_raw, bt_lds);
  else
    decode_dma_item<BS, NW, NST>(a, a.items[blockIdx.x - n_cascade], smem_raw, bt_lds);
}

// =============================================================================
// Decode for E4M3 KV, head_dim 128, streamed through LDS like the bf16 one:
// wave w takes the 32-key slices w, w+4, ... of the item's range; a slice of
// K codes (and of V codes) is 4 KB, 32 rows of 128 bytes, moved into the
// wave's ring by four 1 KB LDS-filling loads of 8 rows each (rows of a load
// lie in one cache block for block sizes 16 and 64).  LDS row r holds its
// 16-byte chunk q at q ^ f(r), f(r) = (r >> 1) & 7.
//   Scores, per 16-key half h: S_h = K_h Q^T on v_mfma_f32_16x16x32_bf16, A =
//   K codes widened to bf16 (lane: key n, d 32c + 8*q4 .. +7, one 8-byte LDS
//   read); the half's K scale multiplies the scores (a half lies in one
//   block).  Lane (n, q4) then holds row n's keys 16h + 4*q4 .. +3.
//   Values: O^T += V^T P^T on the same MFMA over the slice's 32 keys, B = P^T
//   as (half 0 keys 4*q4.., half 1 keys 16 + 4*q4..) with each half's V
//   scale folded into its probabilities; A = V^T from one transposing 8-bit
//   read per d-block, its lane pairs addressing the key rows in that order.
constexpr int kDec8Slice = 32;                        // keys per wave step
constexpr int kDec8SliceBytes = kDec8Slice * 128;     // K (or V) codes of one slice, 4 KB

template <int BS, int NW, int NST>
__device__ __forceinline__ void decode_fp8_item(const AttnArgs &a, const Item it, unsigned char *smem_raw,
                                                int *bt_lds) {
  constexpr int D = 128;
  constexpr int NCK = D / 32;
  constexpr int ND = D / 16;
  constexpr int SB = kDec8SliceBytes;
  static_assert(BS == 16 || BS == 64, "block size");
  static_assert(NW * NST * 2 * SB >= NW * 16 * (D + 2) * 4, "combine scratch");
  lds_u8 *smem = (lds_u8 *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int tok = n >> a.lg, g = n & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;
  const int kv_lo = it.kv_lo, kv_hi = it.kv_hi;

  bf16x8 qf[NCK];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCK; c++) {
      uint4 v = active ? gload16(qrow + (32 * c + 8 * q4) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = as_bf16x8(v);
    }
  }

  float m = kNegBig, l = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x4{};

  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const int n_slices = (kv_hi - kv_lo + kDec8Slice - 1) / kDec8Slice;
  const int nw = n_slices > wave ? (n_slices - wave + NW - 1) / NW : 0;  // this wave's slices
  const int blk0 = kv_lo / BS;
  const int last_blk = (kv_hi - 1) / BS;
  const int lim = min(pos, kv_hi - 1);
  {  // the item's block ids into LDS (see the bf16 kernel)
    const int32_t *btr = a.bt + (int64_t)it.seq * a.max_blocks + blk0;
    for (int i = tid; i <= last_blk - blk0; i += 64 * NW) bt_lds[i] = btr[i];
  }
  PA_WAIT_VMCNT(0);
  __syncthreads();
  const int lim_min = min(it.pos0, kv_hi - 1);

  // LDS rows of 128 bytes, logical 16-byte chunk q of row r at position
  // q ^ f(r).  A transposing 8-byte read is served a half-wave at a time
  // (256 bytes: 64 four-byte banks, measured with SQ_LDS_BANK_CONFLICT); the
  // V^T reads of half-wave 0 touch rows 0..7 and 16..23 (half-wave 1: 8..15
  // and 24..31), so f flips chunk bit 2 for rows 16..31 and the two row sets
  // land on distinct banks (without it, a 2-way conflict).  The K reads stay
  // conflict-free: rows 2k and 2k+1 share f and sit 128 bytes apart.
  auto f = [](int r) { return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 2); };
  // load q of a slice: rows 8q .. 8q+7; lane i fills chunk position i & 7 of
  // row 8q + (i >> 3) with the row's chunk (i & 7) ^ f(row)
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; q++) voff[q] = (lane >> 3) * 128 + (((lane & 7) ^ f(8 * q + (lane >> 3))) << 4);
  const uint32_t ring = smem_addr + wave * NST * 2 * SB;
  lds_u8 *ring_p = smem + wave * NST * 2 * SB;

  auto slice_key = [&](int k) { return kv_lo + kDec8Slice * (wave + NW * k); };
  auto block_at = [&](int key) {
    return __builtin_amdgcn_readfirstlane(bt_lds[min(key / BS, last_blk) - blk0]);
  };
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int key0 = slice_key(min(k, max(nw - 1, 0)));
    const uint32_t st = ring + (k % NST) * 2 * SB;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int row0 = key0 + 8 * q;
      const int64_t blk = block_at(row0);
      const int64_t base = ((blk * hkv + it.kvh) * BS + row0 % BS) * D;
      const int nrec = __builtin_amdgcn_readfirstlane(k < nw ? min(max(kv_hi - row0, 0), 8) * D : 0);
      const uint64_t kq = (uint64_t)(kc + base), vq = (uint64_t)(vc + base);
      const i32x4_t rk = {__builtin_amdgcn_readfirstlane((int)(uint32_t)kq),
                          __builtin_amdgcn_readfirstlane((int)((kq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      const i32x4_t rv = {__builtin_amdgcn_readfirstlane((int)(uint32_t)vq),
                          __builtin_amdgcn_readfirstlane((int)((vq >> 32) & 0xFFFF)), nrec, kRsrcFlags};
      dma_load16_nt(rk, voff[q], st + q * 1024);
      dma_load16_nt(rv, voff[q], st + SB + q * 1024);
    }
  };

  // per-lane LDS offsets: K fragment c of half h at kofs(h) ^ (c << 5); V^T
  // fragment db at vofs ^ (db << 4)
  auto kofs = [&](int h) {
    const int r = 16 * h + n;
    return r * 128 + (((q4 >> 1) ^ f(r)) << 4) + (q4 & 1) * 8;
  };
  const int vrow = (n >> 1) < 4 ? 4 * q4 + (n >> 1) : 16 + 4 * q4 + (n >> 1) - 4;
  const int vofs = vrow * 128 + (f(vrow) << 4) + (n & 1) * 8;

  // Slice k is read from LDS into registers first; its stage is then free
  // and slice k + NST is requested into it before the arithmetic, so all NST
  // stages are in flight while the wave computes.
  auto compute = [&](int k) __attribute__((always_inline)) {
    const lds_u8 *Ks = ring_p + (k % NST) * 2 * SB;
    const lds_u8 *Vs = Ks + SB;
    const int key0 = slice_key(k);
    uint2 kraw[2][NCK], vraw[ND];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int c = 0; c < NCK; c++) kraw[h][c] = lds_load8(Ks + (kofs(h) ^ (c << 5)));
#pragma unroll
    for (int db = 0; db < ND; db++) vraw[db] = lds_read_tr8(Vs + (vofs ^ (db << 4)));
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage's bytes are in registers
    __builtin_amdgcn_sched_barrier(0);
    issue(k + NST);
    // the scales through the constant address space: uniform scalar loads
    // (a vector load would be counted with the K/V stream by vmcnt)
    typedef const __attribute__((address_space(4))) float cfloat;
    float ksc[2], vsc[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int64_t blk = block_at(key0 + 16 * h);
      ksc[h] = ((cfloat *)a.c.ks)[blk * hkv + it.kvh] * a.scale_log2;
      vsc[h] = ((cfloat *)a.c.vs)[blk * hkv + it.kvh];
    }
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        const bf16x8 kf = e4m3x8_to_bf16x8_hw(kraw[h][c]);
        s[h] = mfma16x16x32(kf, qf[c], c == 0 ? f32x4{} : s[h]);
      }
      s[h] *= ksc[h];  // base-2 logits
    }
    if (key0 + kDec8Slice - 1 > lim_min) {
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int r = 0; r < 4; r++) s[h][r] = key0 + 16 * h + 4 * q4 + r <= lim ? s[h][r] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = xor32_max(xor16_max(mx));
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++) o[db] *= alpha;
    }
    bf16x8 pb;
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float p = fast_exp2(s[h][r] - m);
        l += p;
        pb[4 * h + r] = (__bf16)(p * vsc[h]);
      }
#pragma unroll
    for (int db = 0; db < ND; db++) {
      const bf16x8 vf = e4m3x8_to_bf16x8_hw(vraw[db]);
      o[db] = mfma16x16x32(vf, pb, o[db]);
    }
  };

#pragma unroll
  for (int k = 0; k < NST; k++) issue(k);
  for (int k = 0; k < nw; k++) {
    PA_WAIT_VMCNT(8 * (NST - 1));  // slice k has landed (slices k+1 .. k+NST-1 may be in flight)
    compute(k);                    // requests slice k + NST into slice k's stage
  }
  PA_WAIT_VMCNT(0);
  decode_combine<D, NW>(a, it, smem_raw, m, l, o);
}

template <int BS, int NW, int NST>
__global__ __launch_bounds__(64 * NW, 1) void decode_dma_fp8_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[NW * NST * 2 * kDec8SliceBytes];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  decode_fp8_item<BS, NW, NST>(a, a.items[blockIdx.x], smem_raw, bt_lds);
}

// =============================================================================
// Decode for MXFP4 KV, head_dim 128 ([V41] kernels section: a 4-bit KV cache,
// about half the bytes of 8-bit): wave w takes the 64-key slices w, w+4, ...
// of the item's range.  A slice's K codes (and V codes) are 4 KB, 64 rows of
// 64 bytes, moved into the wave's ring by four 1 KB LDS-filling loads of 16
// rows (one cache block each for block sizes 16 and 64); its K (and V) scale
// bytes, 256 of them, follow by one-dword-per-lane loads (block 64: the
// block's [group][key] bytes as they are; block 16: four loads by lanes
// 0..15, one per block, giving [block][group][16 keys]).  LDS row r holds its
// logical 16-byte chunk q at position q ^ G(r), G(r) = x0 | ((x0 ^ x1 ^ r4)
// << 1) with x = (r >> 2) & 3 and r4 = bit 4 of r, which keeps both read
// patterns below free of bank conflicts.
//   Scores, per 16-key quarter h: S_h = K_h Q^T on v_mfma_f32_16x16x32_bf16.
//   The contraction over d is ordered so that lane (n, q4) reads one 16-byte
//   chunk -- d 32 q4 .. +31 of key 16h + n, a single scale group -- and MFMA
//   c takes d 32 q4 + 8c .. +7 from it (Q is loaded in the same order); the
//   codes widen to bf16 with the group's scale, exactly, 2 per instruction.
//   Values: O^T += V^T P^T over each 32-key half.  A transposing 8-bit read
//   gives lane (n, q4) byte n of chunk j for the half's keys in P's order;
//   that byte holds d 32j + 2n and 32j + 2n + 1 of one key, whose scale
//   group is j, so each key's pair widens with one instruction and the pairs
//   are regrouped into two A operands: one MFMA over the even d, one over
//   the odd.  Lane (n, q4) then holds d 32j + 8 q4 .. +7 of row n.
constexpr int kDec4Slice = 64;                       // keys per wave step
constexpr int kDec4CodeBytes = kDec4Slice * 64;      // K (or V) codes of one slice, 4 KB
constexpr int kDec4ScaleBytes = kDec4Slice * 4;      // K (or V) scale bytes of one slice
constexpr int kDec4StageBytes = 2 * kDec4CodeBytes + 2 * kDec4ScaleBytes;

template <int BS, int NW, int NST>
__device__ __forceinline__ void decode_fp4_item(const AttnArgs &a, const Item it, unsigned char *smem_raw,
                                                int *bt_lds, float *vsf_all) {
  constexpr int D = 128;
  constexpr int ND = D / 16;
  constexpr int SB = kDec4CodeBytes;
  constexpr int STB = kDec4StageBytes;
  constexpr int PER_SLICE = 8 + (BS == 64 ? 2 : 8);  // vector-memory instructions per slice
  static_assert(BS == 16 || BS == 64, "block size");
  static_assert(NW * NST * STB >= NW * 16 * (D + 2) * 4, "combine scratch");
  // (every request of the NST stages outstanding at once fits the 6-bit
  // vector-memory counter)
  static_assert(PER_SLICE * NST < 64, "vmcnt range");
  lds_u8 *smem = (lds_u8 *)smem_raw;
  const uint32_t smem_addr = (uint32_t)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q4 = lane >> 4;
  const int tok = n >> a.lg, g = n & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;
  const int kv_lo = it.kv_lo, kv_hi = it.kv_hi;
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  lds_f32 *vsf = (lds_f32 *)(vsf_all + wave * 4 * kDec4Slice);

  // Q in the contraction order of the score product: qf[c] = d 32 q4 + 8c ..
  bf16x8 qf[4];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint4 v = active ? gload16(qrow + (32 * q4 + 8 * c) * 2) : make_uint4(0, 0, 0, 0);
      qf[c] = as_bf16x8(v);
    }
  }

  float m = kNegBig, l = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int i = 0; i < ND; i++) o[i] = f32x4{};

  const unsigned char *kc = (const unsigned char *)a.c.k;
  const unsigned char *vc = (const unsigned char *)a.c.v;
  const unsigned char *ksc = (const unsigned char *)a.c.ks;
  const unsigned char *vsc = (const unsigned char *)a.c.vs;
  const int n_slices = (kv_hi - kv_lo + kDec4Slice - 1) / kDec4Slice;
  const int nw = n_slices > wave ? (n_slices - wave + NW - 1) / NW : 0;  // this wave's slices
  const int blk0 = kv_lo / BS;
  const int last_blk = (kv_hi - 1) / BS;
  const int lim = min(pos, kv_hi - 1);
  {  // the item's block ids into LDS (see the bf16 kernel)
    const int32_t *btr = a.bt + (int64_t)it.seq * a.max_blocks + blk0;
    for (int i = tid; i <= last_blk - blk0; i += 64 * NW) bt_lds[i] = btr[i];
  }
  PA_WAIT_VMCNT(0);
  __syncthreads();
  const int lim_min = min(it.pos0, kv_hi - 1);

  auto G = [](int r) {
    const int x = (r >> 2) & 3;
    return (x & 1) | ((((x ^ (x >> 1)) ^ (r >> 4)) & 1) << 1);
  };
  // code loads: load L fills rows 16L .. 16L+15; lane i writes position
  // i & 3 of row 16L + (i >> 2) and so fetches that row's chunk (i & 3) ^ G
  // (G depends on L only through its parity)
  int voff[2];
#pragma unroll
  for (int par = 0; par < 2; par++)
    voff[par] = (lane >> 2) * 64 + 16 * ((lane & 3) ^ G(16 * par + (lane >> 2)));
  const uint32_t ring = smem_addr + wave * NST * STB;
  lds_u8 *ring_p = smem + wave * NST * STB;

  auto slice_key = [&](int k) { return kv_lo + kDec4Slice * (wave + NW * k); };
  auto block_at = [&](int key) {
    return __builtin_amdgcn_readfirstlane(bt_lds[min(key / BS, last_blk) - blk0]);
  };
  auto desc = [](const unsigned char *p, int nrec) __attribute__((always_inline)) {
    const uint64_t q = (uint64_t)p;
    return i32x4_t{__builtin_amdgcn_readfirstlane((int)(uint32_t)q),
                   __builtin_amdgcn_readfirstlane((int)((q >> 32) & 0xFFFF)), nrec, kRsrcFlags};
  };
  // A request past the range end has a buffer size of zero: it moves no
  // data (zeros land in LDS) but keeps the per-slice vmcnt accounting.
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int key0 = slice_key(min(k, max(nw - 1, 0)));
    const bool live = k < nw;
    const uint32_t st = ring + (k % NST) * STB;
#pragma unroll
    for (int L = 0; L < 4; L++) {
      const int row0 = key0 + 16 * L;
      const int64_t blk = block_at(row0);
      const int64_t base = ((blk * hkv + it.kvh) * BS + row0 % BS) * (D / 2);
      const int nrec = __builtin_amdgcn_readfirstlane(live ? min(max(kv_hi - row0, 0), 16) * (D / 2) : 0);
      dma_load16_nt(desc(kc + base, nrec), voff[L & 1], st + L * 1024);
      dma_load16_nt(desc(vc + base, nrec), voff[L & 1], st + SB + L * 1024);
    }
    if constexpr (BS == 64) {  // the slice is one block: its [group][64 keys] bytes
      const int64_t blk = block_at(key0);
      const int64_t base = (blk * hkv + it.kvh) * (D / 32) * BS;
      const int nrec = __builtin_amdgcn_readfirstlane(live ? kDec4ScaleBytes : 0);
      dma_load4(desc(ksc + base, nrec), 4 * lane, st + 2 * SB);
      dma_load4(desc(vsc + base, nrec), 4 * lane, st + 2 * SB + kDec4ScaleBytes);
    } else {  // four blocks of [group][16 keys], 64 bytes each
      if (lane < 16) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int64_t blk = block_at(key0 + 16 * j);
          const int64_t base = (blk * hkv + it.kvh) * (D / 32) * BS;
          const int nrec = __builtin_amdgcn_readfirstlane(live && key0 + 16 * j < kv_hi ? 64 : 0);
          dma_load4(desc(ksc + base, nrec), 4 * lane, st + 2 * SB + 64 * j);
          dma_load4(desc(vsc + base, nrec), 4 * lane, st + 2 * SB + kDec4ScaleBytes + 64 * j);
        }
      }
    }
  };

  // per-lane LDS offsets.  K: row 16h + n, chunk q4 (position q4 ^ G), and
  // its scale byte (group q4).  V^T: lane pair (n >> 1) addresses key row vr
  // of the half (P's order: 4 q4 + i, then 16 + 4 q4 + i), half n & 1 of
  // chunk j at position j ^ G; the half's scale dwords of group j.
  auto kofs = [&](int h) { return (16 * h + n) * 64 + 16 * (q4 ^ G(16 * h + n)); };
  auto ksofs = [&](int h) { return BS == 64 ? 64 * q4 + 16 * h + n : 64 * h + 16 * q4 + n; };
  const int vr = (n >> 1) < 4 ? 4 * q4 + (n >> 1) : 16 + 4 * q4 + (n >> 1) - 4;
  auto vofs = [&](int hf) { return (32 * hf + vr) * 64 + 16 * G(32 * hf + vr) + 8 * (n & 1); };
  typedef const __attribute__((address_space(3))) uint32_t lds_u32;
  // The V scales are used once per key pair, 64 per lane and slice: each
  // lane first turns 4 of the slice's 256 scale bytes into fp32 operands in
  // the wave's [group][64 keys] table (a key past the range end gets 2^-127:
  // its codes are zero, its slot's scale byte may be anything, NaN
  // included), and the value product reads them 4 at a time.
  const int xg = BS == 64 ? lane >> 4 : (lane >> 2) & 3;                       // group of the lane's 4 bytes
  const int xk = BS == 64 ? 4 * (lane & 15) : 16 * (lane >> 4) + 4 * (lane & 3);  // their first key

  // Slice k is read from LDS into registers first; its stage is then free
  // and slice k + NST is requested into it before the arithmetic.
  auto compute = [&](int k) __attribute__((always_inline)) {
    const lds_u8 *Ks = ring_p + (k % NST) * STB;
    const lds_u8 *Vs = Ks + SB;
    const lds_u8 *KSs = Ks + 2 * SB;
    const lds_u8 *VSs = KSs + kDec4ScaleBytes;
    const int key0 = slice_key(k);
    {
      uint32_t raw = *(lds_u32 *)(VSs + 4 * lane);
      const int c = min(max(kv_hi - (key0 + xk), 0), 4);
      raw &= c >= 4 ? 0xFFFFFFFFu : (1u << (8 * c)) - 1u;
      *(lds_f32x4 *)(vsf + xg * kDec4Slice + xk) =
          f32x4{e8m0_operand(raw & 0xFFu), e8m0_operand((raw >> 8) & 0xFFu), e8m0_operand((raw >> 16) & 0xFFu),
                e8m0_operand(raw >> 24)};
    }
    uint4 kraw[4];
    uint32_t kse[4];
    uint2 vraw[2][4];
    f32x4 vsc[2][4][2];
#pragma unroll
    for (int h = 0; h < 4; h++) {
      kraw[h] = lds_load16(Ks + kofs(h));
      kse[h] = *(KSs + ksofs(h));
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        vraw[hf][j] = lds_read_tr8(Vs + (vofs(hf) ^ (j << 4)));
#pragma unroll
        for (int part = 0; part < 2; part++)  // keys 32 hf + 16 part + 4 q4 .. +3, group j
          vsc[hf][j][part] = *(const lds_f32x4 *)(vsf + j * kDec4Slice + 32 * hf + 16 * part + 4 * q4);
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage's bytes are in registers
    __builtin_amdgcn_sched_barrier(0);
    issue(k + NST);
    f32x4 s[4];
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const float sc = e8m0_operand(kse[h]);
      const uint32_t w[4] = {kraw[h].x, kraw[h].y, kraw[h].z, kraw[h].w};
#pragma unroll
      for (int c = 0; c < 4; c++) s[h] = mfma16x16x32(fp4x8_to_bf16x8(w[c], sc), qf[c], c == 0 ? f32x4{} : s[h]);
      s[h] *= a.scale_log2;  // base-2 logits
    }
    if (key0 + kDec4Slice - 1 > lim_min) {
#pragma unroll
      for (int h = 0; h < 4; h++)
#pragma unroll
        for (int r = 0; r < 4; r++) s[h][r] = key0 + 16 * h + 4 * q4 + r <= lim ? s[h][r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int h = 0; h < 4; h++) mx = fmaxf(mx, fmaxf(fmaxf(s[h][0], s[h][1]), fmaxf(s[h][2], s[h][3])));
    mx = xor32_max(xor16_max(mx));
    if (__any(mx > m + kRescaleSlack)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; db++) o[db] *= alpha;
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 pb;
#pragma unroll
      for (int part = 0; part < 2; part++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const float p = fast_exp2(s[2 * hf + part][r] - m);
          l += p;
          pb[4 * part + r] = (__bf16)p;
        }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        // key i of the half (P's order): byte i of vraw and scale byte i of
        // the part's dword; it widens to (d 32j + 2n, d 32j + 2n + 1)
        uint32_t pr[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const uint32_t w = i < 4 ? vraw[hf][j].x : vraw[hf][j].y;
          const float sc = vsc[hf][j][i >> 2][i & 3];
          if ((i & 3) == 0) pr[i] = fp4x2_to_bf16x2<0>(w, sc);
          if ((i & 3) == 1) pr[i] = fp4x2_to_bf16x2<1>(w, sc);
          if ((i & 3) == 2) pr[i] = fp4x2_to_bf16x2<2>(w, sc);
          if ((i & 3) == 3) pr[i] = fp4x2_to_bf16x2<3>(w, sc);
        }
        const uint4 ev = make_uint4(__builtin_amdgcn_perm(pr[1], pr[0], 0x05040100u),
                                    __builtin_amdgcn_perm(pr[3], pr[2], 0x05040100u),
                                    __builtin_amdgcn_perm(pr[5], pr[4], 0x05040100u),
                                    __builtin_amdgcn_perm(pr[7], pr[6], 0x05040100u));
        const uint4 od = make_uint4(__builtin_amdgcn_perm(pr[1], pr[0], 0x07060302u),
                                    __builtin_amdgcn_perm(pr[3], pr[2], 0x07060302u),
                                    __builtin_amdgcn_perm(pr[5], pr[4], 0x07060302u),
                                    __builtin_amdgcn_perm(pr[7], pr[6], 0x07060302u));
        o[2 * j] = mfma16x16x32(as_bf16x8(ev), pb, o[2 * j]);
        o[2 * j + 1] = mfma16x16x32(as_bf16x8(od), pb, o[2 * j + 1]);
      }
    }
  };

#pragma unroll
  for (int k = 0; k < NST; k++) issue(k);
  for (int k = 0; k < nw; k++) {
    PA_WAIT_VMCNT(PER_SLICE * (NST - 1));  // slice k has landed (slices k+1 .. k+NST-1 may be in flight)
    compute(k);                            // requests slice k + NST into slice k's stage
  }
  PA_WAIT_VMCNT(0);
  decode_combine<D, NW, true>(a, it, smem_raw, m, l, o);
}

template <int BS, int NW, int NST>
__global__ __launch_bounds__(64 * NW, 1) void decode_dma_fp4_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[NW * NST * kDec4StageBytes];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  __shared__ __attribute__((aligned(16))) float vsf_lds[NW * 4 * kDec4Slice];  // a slice's V scales, fp32
  decode_fp4_item<BS, NW, NST>(a, a.items[blockIdx.x], smem_raw, bt_lds, vsf_lds);
}

// E4M3 decode: waves per work-group and ring stages per wave
#ifndef PA_DEC8_WAVES
#define PA_DEC8_WAVES 8
#endif
#ifndef PA_DEC8_STAGES
#define PA_DEC8_STAGES 2
#endif
// MXFP4 decode: eight waves of two stages, two per SIMD, so that one converts
// and multiplies while the other waits (measured: 0.208 ms against 0.25 ms
// for four waves of four stages at 1M keys)
constexpr int kDec4Waves = 8, kDec4Stages = 2;

// The decode launch's items (the cascade items, if any, then the decode
// items) taken from a shared list instead of one per work-group: a
// persistent grid whose work-groups claim item indexes from a counter in the
// workspace (zeroed by the work-list copy; one vector atomic by one lane per
// claim) until the list is exhausted.  The forward call launches it twice
// over the same list and counter -- on a few CUs beside a prefill launch that
// holds the others, and after that prefill on the CUs it frees -- so a mixed
// step's decode streams from HBM while its prefill keeps the matrix cores
// busy ([Agentic] §5.1-5.2: persistent work-groups taking tasks from a table
// by index).  Items are listed longest first (cascade items first).  NRB = 0:
// no cascade items (the only case for E4M3 and MXFP4 KV).  Each item is
// computed by the same item function, in the same work-group shape, as in
// the launch that runs it one work-group per item (the cascade launch with
// cascade items, else the decode launch of its KV format).
template <int FMT>
constexpr int claim_waves(int nrb) {
  return FMT == kKvE4m3 ? PA_DEC8_WAVES : FMT == kKvMxfp4 ? kDec4Waves : cascade_waves(nrb);
}
template <int BS, int NRB, int FMT>
__global__ __launch_bounds__(64 * claim_waves<FMT>(NRB), 1) void decode_claim_kernel(
    AttnArgs a, uint32_t *ctr, int n_items, const CascadeItem *citems, const CascadeMember *members, int n_cascade) {
  constexpr int NW = claim_waves<FMT>(NRB);
  constexpr int NST = FMT == kKvE4m3 ? PA_DEC8_STAGES : FMT == kKvMxfp4 ? kDec4Stages : cascade_stages(NRB);
  constexpr int RING = FMT == kKvE4m3 ? NW * NST * 2 * kDec8SliceBytes
                     : FMT == kKvMxfp4 ? NW * NST * kDec4StageBytes
                                       : NW * NST * 2 * kDecSliceBytes;
  static_assert(NRB == 0 || FMT == kKvBf16, "cascade items are bf16");
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[RING];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  __shared__ __attribute__((aligned(16))) float vsf_lds[FMT == kKvMxfp4 ? NW * 4 * kDec4Slice : 1];
  __shared__ int claim_s;
  for (;;) {
    if (threadIdx.x == 0) claim_s = (int)atomicAdd(ctr, 1u);
    __syncthreads();
    const int i = claim_s;
    __syncthreads();  // (claim_s is rewritten by the next claim)
    if (i >= n_items) break;
    if constexpr (FMT == kKvE4m3) {
      decode_fp8_item<BS, NW, NST>(a, a.items[i], smem_raw, bt_lds);
    } else if constexpr (FMT == kKvMxfp4) {
      decode_fp4_item<BS, NW, NST>(a, a.items[i], smem_raw, bt_lds, vsf_lds);
    } else if constexpr (NRB > 0) {
      if (i < n_cascade)
        cascade_item<BS, NRB, NW, NST>(a, citems[i], members, smem_raw, bt_lds);
      else
        decode_dma_item<BS, NW, NST>(a, a.items[i - n_cascade], smem_raw, bt_lds);
    } else {
      decode_dma_item<BS, NW, NST>(a, a.items[i], smem_raw, bt_lds);
    }
    __syncthreads();  // the item's LDS (ring, block ids, combine scratch) is free again
  }
}

// =============================================================================
// LSE merge of split items ([Agentic] §4.3.3): for each row,
// out = sum_i w_i o_i / sum_i w_i with w_i = 2^(lse_i - M), M = max_i lse_i,
// lse = M + log2(sum_i w_i); parts without keys (lse = -inf) weigh nothing
// (their stored o is 0).  A work-group takes kMergeRows rows of one task:
// the part weights go to LDS first (one thread per row for a few parts, one
// wave per row with the lanes splitting the parts otherwise), then each
// thread reduces four consecutive d of one row over the parts with 16-byte
// loads that do not wait on each other.
constexpr int kMergeRows = 64;
constexpr int kMergeWeights = 8192;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const Merge mt = a.merges[blockIdx.x];
  const int rows = mt.nq << a.lg;
  const int rb = blockIdx.y * kMergeRows;
  if (rb >= rows) return;
  const int nr = min(kMergeRows, rows - rb);
  const float *po = mt.is_decode ? a.part_o_decode : a.part_o_prefill;
  const float *pl = mt.is_decode ? a.part_lse_decode : a.part_lse_prefill;
  const int rpp = mt.rows_per_part;
  const int np = mt.nparts;  // <= kMergeSerialParts
  __shared__ float sm_w[kMergeRows * kMergeSerialParts];
  __shared__ float sm_inv[kMergeRows];
  auto row_out = [&](int r) {
    const int rr = rb + r;
    return (int64_t)(mt.row0 + (rr >> a.lg)) * a.hq + mt.kvh * a.group + (rr & (a.group - 1));
  };
  {  // one thread per row weighs the parts
    const int r = threadIdx.x;
    if (r < nr) {
      const float *lrow = pl + (int64_t)mt.part0 * rpp + rb + r;
      float li[kMergeSerialParts];
      float M = -INFINITY;
      for (int i = 0; i < np; i++) {
        li[i] = lrow[(int64_t)i * rpp];
        M = fmaxf(M, li[i]);
      }
      float S = 0.f;
      for (int i = 0; i < np; i++) {
        const float w = (M > -INFINITY && li[i] > -INFINITY) ? fast_exp2(li[i] - M) : 0.f;
        S += w;
        sm_w[r * kMergeSerialParts + i] = w;
      }
      sm_inv[r] = S > 0.f ? 1.f / S : 0.f;
      if (a.lse_out) a.lse_out[row_out(r)] = S > 0.f ? (M + __log2f(S)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  // each thread: four consecutive d of a row, two such units at a time so
  // that their parts' loads are in flight together
  const int d = a.d, d4 = d / 4;
  const int n_units = nr * d4;
  auto unit = [&](int idx, f32x4 &O) {
    const int r = idx / d4, e = (idx % d4) * 4;
    const float *orow = po + ((int64_t)mt.part0 * rpp + rb + r) * d + e;
    const float *w = sm_w + r * kMergeSerialParts;
    O = f32x4{0.f, 0.f, 0.f, 0.f};
    int i = 0;
    for (; i + 4 <= np; i += 4) {
      f32x4 v[4];
#pragma unroll
      for (int k = 0; k < 4; k++) v[k] = *(const f32x4 *)(orow + (int64_t)(i + k) * rpp * d);
#pragma unroll
      for (int k = 0; k < 4; k++) O += w[i + k] * v[k];
    }
    for (; i < np; i++) O += w[i] * *(const f32x4 *)(orow + (int64_t)i * rpp * d);
  };
  auto store = [&](int idx, const f32x4 &O) {
    const int r = idx / d4, e = (idx % d4) * 4;
    const float inv = sm_inv[r];
    bf16x4 v;
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = (__bf16)(O[k] * inv);
    *(bf16x4 *)((__bf16 *)a.out + row_out(r) * d + e) = v;
  };
  for (int idx = threadIdx.x; idx < n_units; idx += 2 * blockDim.x) {
    const int idx2 = idx + blockDim.x;
    f32x4 O, O2;
    unit(idx, O);
    if (idx2 < n_units) unit(idx2, O2);
    store(idx, O);
    if (idx2 < n_units) store(idx2, O2);
  }
}

// Merges of many parts (more than kMergeSerialParts; long decodes split
// over many items): one work-group per (task, row).  The 256 threads weigh the
// parts together, then 8 groups of 32 threads each sum every eighth part over
// the row's d (4 consecutive d per thread), combined through LDS.
__global__ __launch_bounds__(256) void merge_many_kernel(MergeArgs a, int first) {
  const Merge mt = a.merges[first + blockIdx.x];
  const int rows = mt.nq << a.lg;
  const int r = blockIdx.y;
  if (r >= rows) return;
  const float *po = mt.is_decode ? a.part_o_decode : a.part_o_prefill;
  const float *pl = mt.is_decode ? a.part_lse_decode : a.part_lse_prefill;
  const int rpp = mt.rows_per_part;
  const int np = mt.nparts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float sm_w[kMergeWeights];
  __shared__ float red[4];
  __shared__ f32x4 ored[8][32];
  const float *lrow = pl + (int64_t)mt.part0 * rpp + r;
  float M = -INFINITY;
  for (int i = tid; i < np; i += 256) M = fmaxf(M, lrow[(int64_t)i * rpp]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  auto weight = [&](int i) {
    const float li = lrow[(int64_t)i * rpp];
    return (M > -INFINITY && li > -INFINITY) ? fast_exp2(li - M) : 0.f;
  };
  float S = 0.f;
  for (int i = tid; i < np; i += 256) {
    const float w = weight(i);
    S += w;
    if (i < kMergeWeights) sm_w[i] = w;
  }
  S = wave_sum(S);
  if (lane == 0) red[wave] = S;
  __syncthreads();
  S = red[0] + red[1] + red[2] + red[3];
  const int d = a.d, d4 = d / 4;
  const int u = tid & 31, pg = tid >> 5;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  if (u < d4) {
    const float *orow = po + ((int64_t)mt.part0 * rpp + r) * d + 4 * u;
    int i = pg;
    for (; i + 24 < np; i += 32) {
      f32x4 v[4];
      float w[4];
#pragma unroll
      for (int k = 0; k < 4; k++) v[k] = *(const f32x4 *)(orow + (int64_t)(i + 8 * k) * rpp * d);
#pragma unroll
      for (int k = 0; k < 4; k++) w[k] = i + 8 * k < kMergeWeights ? sm_w[i + 8 * k] : weight(i + 8 * k);
#pragma unroll
      for (int k = 0; k < 4; k++) O += w[k] * v[k];
    }
    for (; i < np; i += 8) O += (i < kMergeWeights ? sm_w[i] : weight(i)) * *(const f32x4 *)(orow + (int64_t)i * rpp * d);
  }
  ored[pg][u] = O;
  __syncthreads();
  const int64_t orow_out = (int64_t)(mt.row0 + (r >> a.lg)) * a.hq + mt.kvh * a.group + (r & (a.group - 1));
  if (tid < d4) {
    f32x4 T = ored[0][tid];
#pragma unroll
    for (int g = 1; g < 8; g++) T += ored[g][tid];
    const float inv = S > 0.f ? 1.f / S : 0.f;
    bf16x4 v;
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = (__bf16)(T[k] * inv);
    *(bf16x4 *)((__bf16 *)a.out + orow_out * d + 4 * tid) = v;
  }
  if (tid == 0 && a.lse_out) a.lse_out[orow_out] = S > 0.f ? (M + __log2f(S)) * kLn2 : -INFINITY;
}

// =============================================================================
// =============================================================================
// One launch per step ([Agentic] §5.1-§5.2: a decode layer runs as two
// persistent kernels, one block per SM, whose stages are task tables the
// blocks claim by index, and the KV write comes before the attention that
// reads it).  Here one grid of one 8-wave work-group per CU runs the whole
// step: each work-group claims tasks from counters in the workspace with
// vector atomics (one lane), in this order --
//   1. kv_append chunks of the step's new tokens;
//   2. (once) wait until every append task has finished: the attention below
//      reads those tokens, and append tasks wait on nothing, so the wait
//      ends (bounded all the same: past the bound a flag is set);
//   3. prefill ranges of the persistent plan from its own XCD's queue (the
//      planner puts one KV head's ranges on one XCD for L2 reuse), then the
//      other XCDs' queues;
//   4. decode items (eight waves, two stages).
// Co-scheduled (decode_first > 0): the first decode_first work-groups of
// each XCD past the wait take decode items before prefill ranges, so the
// decode streams from HBM on those CUs while the others' matrix cores run
// the prefill (the planner cuts the prefill ranges for the rest).
// A split tile's partials are merged by the work-group that writes its last
// part: after its partial stores, one lane releases them at device scope and
// counts the part in; the one that completes the count acquires and merges
// (so a step has no merge launch).  Memory ordering: every wave waits for
// its own stores (vmcnt 0) before the barrier, the counting lane then
// releases at device scope (its XCD's L2 written back), and the merging
// work-group's device-scope acquire (caches invalidated) precedes its reads
// of other work-groups' partials.

// The in-work-group LSE merge of one record: wave w takes rows w, w + 8, ...;
// the lanes hold the part weights (64 parts at a time) and d = lane, lane +
// 64 of the output.
__device__ __forceinline__ void step_merge(const MergeArgs &a, const Merge mt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rows = mt.nq << a.lg;
  const float *po = mt.is_decode ? a.part_o_decode : a.part_o_prefill;
  const float *pl = mt.is_decode ? a.part_lse_decode : a.part_lse_prefill;
  const int rpp = mt.rows_per_part, np = mt.nparts, d = a.d;
  for (int r = wave; r < rows; r += kStepThreads / 64) {
    float M = -INFINITY;
    for (int i0 = 0; i0 < np; i0 += 64)
      if (i0 + lane < np) M = fmaxf(M, pl[(int64_t)(mt.part0 + i0 + lane) * rpp + r]);
    M = wave_max(M);
    float S = 0.f, O0 = 0.f, O1 = 0.f;
    for (int i0 = 0; i0 < np; i0 += 64) {
      const float li = i0 + lane < np ? pl[(int64_t)(mt.part0 + i0 + lane) * rpp + r] : -INFINITY;
      const float w = (M > -INFINITY && li > -INFINITY) ? fast_exp2(li - M) : 0.f;
      S += wave_sum(w);
      const int nn = min(64, np - i0);
      // eight parts' loads in flight at a time (the merge of a long decode
      // runs at the end of the step, so its latency is the step's); the sum
      // still takes the parts in order
      int i = 0;
      for (; i + 8 <= nn; i += 8) {
        float v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const float *orow = po + ((int64_t)(mt.part0 + i0 + i + k) * rpp + r) * d;
          v0[k] = orow[lane];
          v1[k] = d > 64 ? orow[lane + 64] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
          const float wi = __shfl(w, i + k);
          O0 += wi * v0[k];
          if (d > 64) O1 += wi * v1[k];
        }
      }
      for (; i < nn; i++) {
        const float wi = __shfl(w, i);
        const float *orow = po + ((int64_t)(mt.part0 + i0 + i) * rpp + r) * d;
        O0 += wi * orow[lane];
        if (d > 64) O1 += wi * orow[lane + 64];
      }
    }
    const float inv = S > 0.f ? 1.f / S : 0.f;
    const int64_t orow = (int64_t)(mt.row0 + (r >> a.lg)) * a.hq + mt.kvh * a.group + (r & (a.group - 1));
    ((__bf16 *)a.out)[orow * d + lane] = (__bf16)(O0 * inv);
    if (d > 64) ((__bf16 *)a.out)[orow * d + lane + 64] = (__bf16)(O1 * inv);
    if (lane == 0 && a.lse_out) a.lse_out[orow] = S > 0.f ? (M + __log2f(S)) * kLn2 : -INFINITY;
  }
}

enum : int { kTaskAppend = 1, kTaskPrefill = 2, kTaskDecode = 3 };

// Thread 0's claim: the next task, encoded (kind << 28) | index, or -1.
// (Claiming decode items first on half the XCDs, so that fewer compute
// units stream the decode part while the rest compute prefill, measured
// slower: 12.5-12.6 ms against 12.3-12.4 ms for the mixed step.)
__device__ __forceinline__ int step_claim(const StepArgs &s, int &phase, uint32_t xcc, bool &waited,
                                          bool &dec_empty, bool &dec_first) {
  uint32_t *c = s.ctr;
  if (phase == 0) {
    const uint32_t i = atomicAdd(&c[kCtrAppendNext], 1u);
    if (i < (uint32_t)s.n_append_tasks) return (kTaskAppend << 28) | (int)i;
    phase = 1;
  }
  if (!waited) {
    for (int it = 0; __hip_atomic_load(&c[kCtrAppendDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                     (uint32_t)s.n_append_tasks;
         it++) {
      if (it > (1 << 24)) {  // never expected: give up rather than hang
        atomicOr(&c[kCtrFlags], 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    waited = true;
    dec_first = s.decode_first > 0 && atomicAdd(&c[kCtrRole + xcc], 1u) < (uint32_t)s.decode_first;
  }
  if (dec_first && !dec_empty) {
    const uint32_t i = atomicAdd(&c[kCtrDecodeNext], 1u);
    if (i < (uint32_t)s.n_decode) return (kTaskDecode << 28) | (int)i;
    dec_empty = true;
  }
  while (phase <= s.xcds) {  // phase p: the prefill queue of XCD (xcc + p - 1) % xcds
    const int q = (int)((xcc + (uint32_t)phase - 1) % (uint32_t)s.xcds);
    const int n = s.pre_queue_off[q + 1] - s.pre_queue_off[q];
    if (n > 0) {
      const uint32_t i = atomicAdd(&c[kCtrPrefillNext + q], 1u);
      if (i < (uint32_t)n) return (kTaskPrefill << 28) | s.pre_queue[s.pre_queue_off[q] + (int)i];
    }
    phase++;
  }
  if (dec_empty) return -1;
  const uint32_t i = atomicAdd(&c[kCtrDecodeNext], 1u);
  if (i < (uint32_t)s.n_decode) return (kTaskDecode << 28) | (int)i;
  dec_empty = true;
  return -1;
}

// One loop over the claimed tasks of every kind.  (A single 1M-token decode
// runs 9-11% slower through this kernel than through the append, decode and
// merge launches; the cause is not established.  A structure with one loop
// per task kind hung on its first test, cause not found, and is not used.)
template <int BS, int FMT>
__global__ __launch_bounds__(kStepThreads, 1) void step_kernel(StepArgs s) {
  // One LDS area for whichever item runs: the decode ring of the KV format
  // (8 waves x 2 stages; the combine scratch lies inside it) or the 384-row
  // prefill's (its K/V tiles and, for E4M3 and MXFP4, its code ring).
  constexpr int NW = kStepThreads / 64;
  constexpr int DEC_NST = FMT == kKvE4m3 ? PA_DEC8_STAGES : FMT == kKvMxfp4 ? kDec4Stages : kDecStages;
  constexpr int DEC_LDS = FMT == kKvE4m3   ? NW * DEC_NST * 2 * kDec8SliceBytes
                          : FMT == kKvMxfp4 ? NW * DEC_NST * kDec4StageBytes
                                            : NW * DEC_NST * 2 * kDecSliceBytes;
  constexpr int PRE_LDS = FMT == kKvE4m3 ? kW48Fp8Lds : FMT == kKvMxfp4 ? kW48Fp4Lds : kW48Stages * 2 * kW48TileBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[DEC_LDS > PRE_LDS ? DEC_LDS : PRE_LDS];
  __shared__ int bt_lds[kMaxDecItemKeys / BS + 2];
  __shared__ __attribute__((aligned(16))) float vsf_lds[FMT == kKvMxfp4 ? NW * 4 * kDec4Slice : 1];
  __shared__ int task_s, merge_s;
  const int tid = threadIdx.x;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  xcc %= (uint32_t)s.xcds;
  int phase = 0;
  bool waited = false, dec_empty = false, dec_first = false;
  // Each task reads its arguments through a fresh view of the kernel
  // argument segment (the pointer passed through an empty asm, so the
  // compiler cannot keep the fields loaded across tasks): with one view for
  // the whole kernel it held many fields in scalar registers throughout and
  // spilled them into vector lanes (300-640 lane reads in the step kernels,
  // some in the decode items' key-step loops).
  typedef const __attribute__((address_space(4))) StepArgs KStepArgs;
  auto fresh = [&]() __attribute__((always_inline)) {
    KStepArgs *p = (KStepArgs *)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return (const StepArgs *)p;
  };
  // after a task's partial stores: count the part in; the last one merges
  auto part_done = [&](int merge) __attribute__((always_inline)) {
    PA_WAIT_VMCNT(0);
    __syncthreads();
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t old = atomicAdd(&s.ctr[kCtrMerge + merge], 1u);
      const bool last = old + 1 == (uint32_t)s.mg.merges[merge].nparts;
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      merge_s = last ? merge : -1;
    }
    __syncthreads();
    if (merge_s >= 0) {
      const StepArgs *sp = fresh();
      step_merge(sp->mg, sp->mg.merges[merge_s]);
    }
  };
  for (;;) {
    if (tid == 0) task_s = step_claim(s, phase, xcc, waited, dec_empty, dec_first);
    __syncthreads();
    const int t = task_s;
    __syncthreads();  // (task_s is rewritten by the next claim)
    if (t < 0) break;
    const int kind = t >> 28, idx = t & 0x0FFFFFFF;
    if (kind == kTaskAppend) {
      // (chunk bounds are multiples of 4: an MXFP4 32-element group's four
      // lanes are active together)
      const uint32_t c0 = (uint32_t)idx * kStepAppendChunks;
      const StepArgs *sp = fresh();
#pragma unroll 1
      for (uint32_t gid = c0 + tid; gid < min(c0 + kStepAppendChunks, sp->app.nchunks); gid += kStepThreads)
        append_chunk<FMT>(sp->app, gid);
      PA_WAIT_VMCNT(0);
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        atomicAdd(&s.ctr[kCtrAppendDone], 1u);
      }
    } else if (kind == kTaskPrefill) {
      for (int i = s.wg_first[idx]; i < s.wg_first[idx + 1]; i++) {
        const StepArgs *sp = fresh();
        const Item it = sp->pre.items[i];
        w48_item<BS, FMT>(sp->pre, it, (lds_u8 *)smem_raw);
        if (it.part >= 0)
          part_done(s.pre_part_merge[it.part]);
        else
          __syncthreads();  // LDS of this item no longer read or written
      }
    } else {
      const StepArgs *sp = fresh();
      const Item it = sp->dec.items[idx];
      if constexpr (FMT == kKvE4m3)
        decode_fp8_item<BS, NW, DEC_NST>(sp->dec, it, smem_raw, bt_lds);
      else if constexpr (FMT == kKvMxfp4)
        decode_fp4_item<BS, NW, DEC_NST>(sp->dec, it, smem_raw, bt_lds, vsf_lds);
      else
        decode_dma_item<BS, NW, DEC_NST>(sp->dec, it, smem_raw, bt_lds);
      if (it.part >= 0) part_done(s.dec_part_merge[it.part]);
    }
  }
}

hipError_t launch_step(const StepArgs &a, int n_groups, int bs, int fmt, hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  if (bs != 16 && bs != 64) return hipErrorInvalidValue;
#define PA_STEP(B, F) hipLaunchKernelGGL((step_kernel<B, F>), dim3(n_groups), dim3(kStepThreads), 0, s, a)
  if (fmt == kKvE4m3) {
    if (bs == 16) PA_STEP(16, kKvE4m3);
    else PA_STEP(64, kKvE4m3);
  } else if (fmt == kKvMxfp4) {
    if (bs == 16) PA_STEP(16, kKvMxfp4);
    else PA_STEP(64, kKvMxfp4);
  } else {
    if (bs == 16) PA_STEP(16, kKvBf16);
    else PA_STEP(64, kKvBf16);
  }
#undef PA_STEP
  return hipGetLastError();
}

template <int D, int BS, bool FP8>
static hipError_t launch_prefill_t(const AttnArgs &a, int n, hipStream_t s) {
  if constexpr (D == 128) {
    if (a.tile_rows == kW48TileRows) {
      hipLaunchKernelGGL((prefill_w48_kernel<BS, FP8 ? kKvE4m3 : kKvBf16>), dim3(n), dim3(512), 0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<D, BS, FP8>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}
#ifndef PA_DECODE_DMA
#define PA_DECODE_DMA 1
#endif
template <int D, int BS, bool FP8>
static hipError_t launch_decode_t(const AttnArgs &a, int n, hipStream_t s) {
  if constexpr (!FP8 && D == 128 && PA_DECODE_DMA) {
    hipLaunchKernelGGL((decode_dma_kernel<BS, kDecWaves, kDecStages>), dim3(n), dim3(64 * kDecWaves), 0, s, a);
    return hipGetLastError();
  }
  if constexpr (FP8 && D == 128 && PA_DECODE_DMA) {
    hipLaunchKernelGGL((decode_dma_fp8_kernel<BS, PA_DEC8_WAVES, PA_DEC8_STAGES>), dim3(n), dim3(64 * PA_DEC8_WAVES), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_kernel<D, BS, FP8>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

#define PA_DISPATCH(FN, ...)                                                       \
  do {                                                                             \
    if (d == 128 && bs == 16 && !fp8) return FN<128, 16, false>(__VA_ARGS__);      \
    if (d == 128 && bs == 64 && !fp8) return FN<128, 64, false>(__VA_ARGS__);      \
    if (d == 128 && bs == 16 && fp8) return FN<128, 16, true>(__VA_ARGS__);        \
    if (d == 128 && bs == 64 && fp8) return FN<128, 64, true>(__VA_ARGS__);        \
    if (d == 64 && bs == 16 && !fp8) return FN<64, 16, false>(__VA_ARGS__);        \
    if (d == 64 && bs == 64 && !fp8) return FN<64, 64, false>(__VA_ARGS__);        \
    if (d == 64 && bs == 16 && fp8) return FN<64, 16, true>(__VA_ARGS__);          \
    if (d == 64 && bs == 64 && fp8) return FN<64, 64, true>(__VA_ARGS__);          \
    return hipErrorInvalidValue;                                                   \
  } while (0)

hipError_t launch_prefill(const AttnArgs &a, int n, int d, int bs, int fmt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (fmt == kKvMxfp4) {  // head_dim 128, the 384-row kernel only
    if (d != 128 || a.tile_rows != kW48TileRows) return hipErrorInvalidValue;
    if (bs == 16)
      hipLaunchKernelGGL((prefill_w48_kernel<16, kKvMxfp4>), dim3(n), dim3(512), 0, s, a);
    else if (bs == 64)
      hipLaunchKernelGGL((prefill_w48_kernel<64, kKvMxfp4>), dim3(n), dim3(512), 0, s, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const bool fp8 = fmt == kKvE4m3;
  PA_DISPATCH(launch_prefill_t, a, n, s);
}
hipError_t launch_decode(const AttnArgs &a, int n, int d, int bs, int fmt, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (fmt == kKvMxfp4) {
    if (d != 128) return hipErrorInvalidValue;
    if (bs == 16)
      hipLaunchKernelGGL((decode_dma_fp4_kernel<16, kDec4Waves, kDec4Stages>), dim3(n), dim3(64 * kDec4Waves), 0, s, a);
    else if (bs == 64)
      hipLaunchKernelGGL((decode_dma_fp4_kernel<64, kDec4Waves, kDec4Stages>), dim3(n), dim3(64 * kDec4Waves), 0, s, a);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  const bool fp8 = fmt == kKvE4m3;
  PA_DISPATCH(launch_decode_t, a, n, s);
}
hipError_t launch_decode_claim(const AttnArgs &a, uint32_t *ctr, int n_decode, const CascadeItem *citems,
                               const CascadeMember *members, int n_cascade, int rows, int groups, int bs, int fmt,
                               hipStream_t s) {
  const int n = n_cascade + n_decode;
  if (n <= 0 || groups <= 0) return hipSuccess;
  if ((n_cascade > 0 && (fmt != kKvBf16 || rows <= 0 || rows > kCascadeRows)) || (bs != 16 && bs != 64))
    return hipErrorInvalidValue;
#define PA_CLAIM(B, R, F)                                                                                     \
  hipLaunchKernelGGL((decode_claim_kernel<B, R, F>), dim3(groups), dim3(64 * claim_waves<F>(R)), 0, s, a, ctr, \
                     n, citems, members, n_cascade)
  if (fmt == kKvE4m3) {
    if (bs == 16) PA_CLAIM(16, 0, kKvE4m3);
    else PA_CLAIM(64, 0, kKvE4m3);
  } else if (fmt == kKvMxfp4) {
    if (bs == 16) PA_CLAIM(16, 0, kKvMxfp4);
    else PA_CLAIM(64, 0, kKvMxfp4);
  } else if (bs == 16) {
    if (n_cascade == 0) PA_CLAIM(16, 0, kKvBf16);
    else if (rows <= 16) PA_CLAIM(16, 1, kKvBf16);
    else if (rows <= 32) PA_CLAIM(16, 2, kKvBf16);
    else PA_CLAIM(16, 4, kKvBf16);
  } else {
    if (n_cascade == 0) PA_CLAIM(64, 0, kKvBf16);
    else if (rows <= 16) PA_CLAIM(64, 1, kKvBf16);
    else if (rows <= 32) PA_CLAIM(64, 2, kKvBf16);
    else PA_CLAIM(64, 4, kKvBf16);
  }
#undef PA_CLAIM
  return hipGetLastError();
}
hipError_t launch_decode_cascade(const AttnArgs &a, const CascadeItem *items, const CascadeMember *members,
                                 int n_cascade, int n_decode, int rows, int bs, hipStream_t s) {
  if (n_cascade + n_decode <= 0) return hipSuccess;
  if (rows <= 0 || rows > kCascadeRows || (bs != 16 && bs != 64)) return hipErrorInvalidValue;
  const dim3 grid(n_cascade + n_decode);
#define PA_CASCADE(B, R) \
  hipLaunchKernelGGL((decode_cascade_kernel<B, R>), grid, dim3(64 * cascade_waves(R)), 0, s, a, items, members, n_cascade)
  if (bs == 16) {
    if (rows <= 16) PA_CASCADE(16, 1);
    else if (rows <= 32) PA_CASCADE(16, 2);
    else PA_CASCADE(16, 4);
  } else {
    if (rows <= 16) PA_CASCADE(64, 1);
    else if (rows <= 32) PA_CASCADE(64, 2);
    else PA_CASCADE(64, 4);
  }
#undef PA_CASCADE
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, int n_few, int n_many, int many_rows, hipStream_t s) {
  if (n_few > 0) hipLaunchKernelGGL(merge_kernel, dim3(n_few, kPrefillRowsMax / kMergeRows), dim3(256), 0, s, a);
  if (n_many > 0) hipLaunchKernelGGL(merge_many_kernel, dim3(n_many, many_rows), dim3(256), 0, s, a, n_few);
  return hipGetLastError();
}

}  // namespace pa
