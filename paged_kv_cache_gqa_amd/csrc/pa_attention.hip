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
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// XOR swizzle of 16-byte chunks within an LDS row (D/8 chunks per row).
// Rows r..r+7 map one logical chunk to eight different chunks, and four
// consecutive rows map a 32-byte column slice to four disjoint bank groups,
// so neither the 16-byte A-operand reads nor the transpose reads conflict.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int MASK = D / 16 - 1;
  return chunk ^ ((row & MASK) << 1);
}

// =============================================================================
// Prefill: one work-group (4 waves) per item; 128 query rows (tokens x heads),
// each wave owns 32 rows; 64-key tiles double-buffered through LDS.
template <int D, int BS, bool FP8>
__global__ __launch_bounds__(256, 2) void prefill_kernel(AttnArgs a) {
  constexpr int CPR = D / 8;             // 16-byte bf16 chunks per LDS row
  constexpr int ROWB = D * 2;            // LDS row bytes
  constexpr int TILEB = kKeyTile * ROWB; // one K or V tile in LDS
  constexpr int NCH = kKeyTile * CPR / 256;
  constexpr int NC = D / 16;             // k-steps of the score product
  constexpr int ND = D / 32;             // 32-wide d blocks of the output
  constexpr int EB = FP8 ? 1 : 2;        // cache element bytes
  constexpr int NSC = FP8 ? (BS == 16 ? 4 : 1) : 1;  // scales per tile

  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[4 * TILEB];
  lds_u8 *smem = (lds_u8 *)smem_raw;

  const Item it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // Staging registers for the next tile's K and V chunks.
  typedef typename std::conditional<FP8, uint2, uint4>::type chunk_t;
  chunk_t kr[NCH], vr[NCH];
  float ksc_n[NSC], vsc_n[NSC], ksc[NSC], vsc[NSC];

  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int ci = tid + 256 * i;
      const int r = ci / CPR, ch = ci % CPR;
      const int p = t * kKeyTile + r;
      if (p < it.kv_hi) {
        const int64_t blk = bt[p / BS];
        const int64_t e = ((blk * hkv + it.kvh) * BS + (p % BS)) * D + ch * 8;
        if constexpr (FP8) {
          kr[i] = gload8(kc + e);
          vr[i] = gload8(vc + e);
        } else {
          kr[i] = gload16(kc + e * 2);
          vr[i] = gload16(vc + e * 2);
        }
      } else {
        kr[i] = chunk_t{};
        vr[i] = chunk_t{};
      }
    }
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < NSC; j++) {
        const int p = t * kKeyTile + j * BS;
        if (p < it.kv_hi) {
          const int64_t blk = bt[p / BS];
          ksc_n[j] = a.c.ks[blk * hkv + it.kvh];
          vsc_n[j] = a.c.vs[blk * hkv + it.kvh];
        } else {
          ksc_n[j] = 0.f;
          vsc_n[j] = 0.f;
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
    lds_u8 *kb = smem + buf * 2 * TILEB;
    lds_u8 *vb = kb + TILEB;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int ci = tid + 256 * i;
      const int r = ci / CPR, ch = ci % CPR;
      const int off = r * ROWB + swz<D>(r, ch) * 16;
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

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; t++) {
    const int buf = (t - t_begin) & 1;
    const lds_u8 *Kb = smem + buf * 2 * TILEB;
    const lds_u8 *Vb = Kb + TILEB;
    if (t + 1 < t_end) load_tile(t + 1);

    // ---- S^T = K * Q^T : two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      s[kb] = f32x16{};
      const int krow = kb * 32 + col;
#pragma unroll
      for (int c = 0; c < NC; c++) {
        bf16x8 af = as_bf16x8(lds_load16(Kb + krow * ROWB + swz<D>(krow, 2 * c + hh) * 16));
        s[kb] = mfma32x32x16(af, qf[c], s[kb]);
      }
    }

    // ---- scale, mask, online softmax (this lane: one query row, 32 keys)
    const int kbase = t * kKeyTile;
    const bool need_mask = (kbase + kKeyTile - 1 > it.pos0) || (kbase + kKeyTile > it.kv_hi);
    float x[2][16];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int i = e >> 2, r = e & 3;
        float sl = a.scale_log2;
        if constexpr (FP8) sl *= ksc[(NSC == 1) ? 0 : (kb * 2 + (i >> 1))];
        float v = s[kb][e] * sl;
        if (need_mask) {
          const int key = kbase + kb * 32 + 8 * i + 4 * hh + r;
          if (!(key <= pos && key < it.kv_hi)) v = -INFINITY;
        }
        x[kb][e] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const float p = fast_exp2(x[kb][e] - m_new);
        x[kb][e] = p;
        psum += p;
      }
    l = l * alpha + psum;
#pragma unroll
    for (int db = 0; db < ND; db++) o[db] *= alpha;

    // ---- O^T += V^T * P^T : four 16-key steps
    const int g16 = lane >> 4, j = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int kb = ks >> 1, i0 = (ks & 1) * 2;
      bf16x8 pb;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        float p0 = x[kb][4 * i0 + r], p1 = x[kb][4 * (i0 + 1) + r];
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
        const int d0 = db * 32 + (g16 & 1) * 16 + 4 * (j & 3);
        bf16x4 h0, h1;
        {
          const int vrow = ks * 16 + 4 * hh + (j >> 2);
          h0 = lds_read_tr(Vb + vrow * ROWB + swz<D>(vrow, d0 >> 3) * 16 + (d0 & 7) * 2);
        }
        {
          const int vrow = ks * 16 + 8 + 4 * hh + (j >> 2);
          h1 = lds_read_tr(Vb + vrow * ROWB + swz<D>(vrow, d0 >> 3) * 16 + (d0 & 7) * 2);
        }
        bf16x8 af = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma32x32x16(af, pb, o[db]);
      }
    }

    if (t + 1 < t_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: combine the two key halves' sums, normalise, store
  const float lt = l + __shfl_xor(l, 32);
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
    float *prow = a.part_o + ((int64_t)it.part * kPrefillRows + row) * D;
#pragma unroll
    for (int db = 0; db < ND; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; r++) v[r] = o[db][4 * i + r] * inv;
        *(f32x4 *)(prow + db * 32 + 8 * i + 4 * hh) = v;
      }
    if (hh == 0) a.part_lse[(int64_t)it.part * kPrefillRows + row] = lse2;
  }
}

// =============================================================================
// Decode (and short increments, tokens x G <= 16): one work-group per item;
// its four waves stream disjoint 64-key tiles of the item's range, each with
// its own softmax state, and are combined through LDS at the end.  K goes
// straight from HBM into MFMA A-operand registers; V passes through a
// per-wave LDS tile for the transposed read.  The next tile's K and V are in
// flight while the current one is computed.
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
  constexpr int DQ = D / 4;     // d elements per lane group
  constexpr int ND = D / 16;    // 16-wide d blocks of the output
  constexpr int ROWB = D * 2;
  constexpr int WAVEB = kKeyTile * ROWB;
  constexpr int EB = FP8 ? 1 : 2;
  typedef DecodeRegs<D, FP8> Regs;

  __shared__ __attribute__((aligned(16))) unsigned char smem_raw[4 * WAVEB];
  lds_u8 *smem = (lds_u8 *)smem_raw;

  const Item it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, q4 = lane >> 4;
  const int tok = n >> a.lg, g = n & (a.group - 1);
  const bool active = tok < it.nq;
  const int pos = it.pos0 + tok;
  const int qh = it.kvh * a.group + g;
  const int hkv = a.c.hkv;
  lds_u8 *Vw = smem + wave * WAVEB;

  // Q as the B operand of K * Q^T (16x16x32): lane holds q[n][q4*DQ + 8c .. +7].
  bf16x8 qf[NCK];
  {
    const unsigned char *qrow =
        (const unsigned char *)a.q + (((int64_t)(it.row0 + tok) * a.hq + qh) * D) * 2;
#pragma unroll
    for (int c = 0; c < NCK; c++) {
      uint4 v = active ? gload16(qrow + (q4 * DQ + 8 * c) * 2) : make_uint4(0, 0, 0, 0);
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

  // Issue the loads of tile t (this lane: key row kb*16 + n, d slice q4).
  auto load = [&](Regs &R, int t) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int p = t * kKeyTile + kb * 16 + n;
      const int pc = p < it.kv_hi ? p : it.kv_hi - 1;  // clamp: tail rows masked/zeroed later
      const int64_t blk = bt[pc / BS];
      const int64_t e = ((blk * hkv + it.kvh) * BS + (pc % BS)) * D + q4 * DQ;
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        if constexpr (FP8) {
          R.k[kb][c] = gload8_nt(kc + e + 8 * c);
          R.v[kb][c] = gload8_nt(vc + e + 8 * c);
        } else {
          R.k[kb][c] = gload16_nt(kc + (e + 8 * c) * 2);
          R.v[kb][c] = gload16_nt(vc + (e + 8 * c) * 2);
        }
      }
      if constexpr (FP8) {
        R.ksc[kb] = a.c.ks[blk * hkv + it.kvh];
        R.vsc[kb] = a.c.vs[blk * hkv + it.kvh];
      }
    }
  };

  auto compute = [&](Regs &R, int t) {
    const int kbase = t * kKeyTile;
    // V tile -> this wave's LDS (rows beyond the range zeroed)
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int r = kb * 16 + n;
      const bool ok = kbase + r < it.kv_hi;
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        uint4 v;
        if constexpr (FP8)
          v = e4m3x8_to_bf16x8(R.v[kb][c]);
        else
          v = R.v[kb][c];
        if (!ok) v = make_uint4(0, 0, 0, 0);
        lds_store16(Vw + r * ROWB + swz<D>(r, (q4 * DQ) / 8 + c) * 16, v);
      }
    }
    // S^T = K * Q^T per 16-key block
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      s[kb] = f32x4{};
#pragma unroll
      for (int c = 0; c < NCK; c++) {
        bf16x8 kf;
        if constexpr (FP8)
          kf = as_bf16x8(e4m3x8_to_bf16x8(R.k[kb][c]));
        else
          kf = as_bf16x8(R.k[kb][c]);
        s[kb] = mfma16x16x32(kf, qf[c], s[kb]);
      }
    }
    const bool need_mask = (kbase + kKeyTile - 1 > it.pos0) || (kbase + kKeyTile > it.kv_hi);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        float sl = a.scale_log2;
        if constexpr (FP8) sl *= R.ksc[kb];
        float v = s[kb][r] * sl;
        if (need_mask) {
          const int key = kbase + kb * 16 + 4 * q4 + r;
          if (!(key <= pos && key < it.kv_hi)) v = -INFINITY;
        }
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    m = m_new;
    float psum = 0.f;
    bf16x4 pb[4];
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float p = fast_exp2(s[kb][r] - m_new);
        psum += p;
        float pv = p;
        if constexpr (FP8) pv *= R.vsc[kb];
        pb[kb][r] = (__bf16)pv;
      }
    l = l * alpha + psum;
#pragma unroll
    for (int db = 0; db < ND; db++) o[db] *= alpha;

    // the wave's own LDS writes above must land before its transpose reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int j = lane & 15;
#pragma unroll
    for (int kb = 0; kb < 4; kb++) {
      const int vrow = kb * 16 + 4 * q4 + (j >> 2);
#pragma unroll
      for (int db = 0; db < ND; db++) {
        const int d0 = db * 16 + 4 * (j & 3);
        bf16x4 af = lds_read_tr(Vw + vrow * ROWB + swz<D>(vrow, d0 >> 3) * 16 + (d0 & 7) * 2);
        o[db] = mfma16x16x16(af, pb[kb], o[db]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  Regs A, B;
  int tw = wave;
  if (tw < ntiles) load(A, t_first + tw);
  while (tw < ntiles) {
    if (tw + 4 < ntiles) load(B, t_first + tw + 4);
    compute(A, t_first + tw);
    tw += 4;
    if (tw >= ntiles) break;
    if (tw + 4 < ntiles) load(A, t_first + tw + 4);
    compute(B, t_first + tw);
    tw += 4;
  }

  // ---- combine the four waves' states through LDS
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  __syncthreads();
  float *red_o = (float *)smem_raw;                  // [4][16][D]
  float *red_m = red_o + 4 * 16 * D;                 // [4][16]
  float *red_l = red_m + 4 * 16;                     // [4][16]
#pragma unroll
  for (int db = 0; db < ND; db++)
    *(f32x4 *)(red_o + (wave * 16 + n) * D + db * 16 + 4 * q4) = o[db];
  if (q4 == 0) {
    red_m[wave * 16 + n] = m;
    red_l[wave * 16 + n] = l;
  }
  __syncthreads();
  const int rows = it.nq << a.lg;
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int cn = idx / D, e = idx % D;
    if (cn >= rows) continue;
    float M = red_m[cn];
#pragma unroll
    for (int w = 1; w < 4; w++) M = fmaxf(M, red_m[w * 16 + cn]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
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
// LSE merge of split items ([Agentic] §4.3.3): for each row,
// out = sum_i 2^(lse_i - M) o_i / sum_i 2^(lse_i - M), lse = M + log2(sum),
// M = max_i lse_i, parts without keys (lse = -inf) contribute nothing.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const Merge mt = a.merges[blockIdx.x];
  const float *po = mt.is_decode ? a.part_o_decode : a.part_o_prefill;
  const float *pl = mt.is_decode ? a.part_lse_decode : a.part_lse_prefill;
  const int rows = mt.nq << a.lg;
  const int rpp = mt.rows_per_part;
  __shared__ float sm_max[kPrefillRows], sm_inv[kPrefillRows];
  for (int r = threadIdx.x; r < rows; r += blockDim.x) {
    float M = -INFINITY;
    for (int i = 0; i < mt.nparts; i++) M = fmaxf(M, pl[(int64_t)(mt.part0 + i) * rpp + r]);
    float S = 0.f;
    if (M > -INFINITY)
      for (int i = 0; i < mt.nparts; i++) S += fast_exp2(pl[(int64_t)(mt.part0 + i) * rpp + r] - M);
    sm_max[r] = M;
    sm_inv[r] = S > 0.f ? 1.f / S : 0.f;
    if (a.lse_out) {
      const int64_t orow = (int64_t)(mt.row0 + (r >> a.lg)) * a.hq + mt.kvh * a.group + (r & (a.group - 1));
      a.lse_out[orow] = S > 0.f ? (M + __log2f(S)) * kLn2 : -INFINITY;
    }
  }
  __syncthreads();
  const int d = a.d;
  for (int idx = threadIdx.x; idx < rows * d; idx += blockDim.x) {
    const int r = idx / d, e = idx % d;
    const float M = sm_max[r];
    float O = 0.f;
    if (M > -INFINITY)
      for (int i = 0; i < mt.nparts; i++) {
        const int64_t slot = (int64_t)(mt.part0 + i) * rpp + r;
        const float li = pl[slot];
        if (li > -INFINITY) O += fast_exp2(li - M) * po[slot * d + e];
      }
    const int64_t orow = (int64_t)(mt.row0 + (r >> a.lg)) * a.hq + mt.kvh * a.group + (r & (a.group - 1));
    ((__bf16 *)a.out)[orow * d + e] = (__bf16)(O * sm_inv[r]);
  }
}

// =============================================================================
template <int D, int BS, bool FP8>
static hipError_t launch_prefill_t(const AttnArgs &a, int n, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, BS, FP8>), dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int D, int BS, bool FP8>
static hipError_t launch_decode_t(const AttnArgs &a, int n, hipStream_t s) {
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

hipError_t launch_prefill(const AttnArgs &a, int n, int d, int bs, bool fp8, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  PA_DISPATCH(launch_prefill_t, a, n, s);
}
hipError_t launch_decode(const AttnArgs &a, int n, int d, int bs, bool fp8, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  PA_DISPATCH(launch_decode_t, a, n, s);
}
hipError_t launch_merge(const MergeArgs &a, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(n), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
