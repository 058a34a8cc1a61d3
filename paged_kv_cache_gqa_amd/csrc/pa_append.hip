// pa_append.hip -- kv_append scatter and the block-table gather test hook.
//
// Pages cited (title, then section):
//   [Agentic] "vLLM Agentic 推理｜面向 Agent 负载的推理优化"
//   [AMPD]    "ICML'26 | AMPD：PD 分离遇上多轮推理，incremental prefill 到底该在哪跑"
//   [V1Sched] "vLLM/V1 推理调度器"
//
// kv_append writes the step's new K/V rows into the slots the scheduler
// assigned ([Agentic] §5.2: the KV write precedes the attention that reads
// it; [AMPD] §7: the increment is concatenated onto the cached history).  One
// thread moves one 16-byte chunk (8 elements) of one (token, KV head) row of
// K and of V; a token with a negative slot is skipped.  8-bit caches store
// E4M3(x / scale) with the correctly rounded fp32 quotient, nearest-even
// rounding and saturation to +-448.
#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  // 32-bit index arithmetic within a launch (the host keeps each launch
  // below 2^31 chunks) and shifts for the power-of-two sizes: the 64-bit
  // divisions this replaces cost more instructions than the copy itself
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  if (gid >= a.nchunks) return;
  const uint32_t ch = gid & ((1u << a.lcpr) - 1);
  const uint32_t row = gid >> a.lcpr;  // (token, KV head) row of this launch
  const uint32_t tl = row / (uint32_t)a.hkv;
  const int h = (int)(row - tl * (uint32_t)a.hkv);
  const int64_t t = a.tok0 + tl;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot >> a.lbs, off = slot & (a.bs - 1);
  const int64_t src = (t * a.hkv + h) * a.d + ch * 8;                   // element offset
  const int64_t dst = ((blk * a.hkv + h) * a.bs + off) * a.d + ch * 8;  // element offset
  const uint4 kv = gload16_nt((const unsigned char *)a.k_new + src * 2);
  const uint4 vv = gload16_nt((const unsigned char *)a.v_new + src * 2);
  if constexpr (!FP8) {
    *(uint4 *)((unsigned char *)a.k_cache + dst * 2) = kv;
    *(uint4 *)((unsigned char *)a.v_cache + dst * 2) = vv;
  } else {
    const float ks = a.ks[blk * a.hkv + h];
    const float vs = a.vs[blk * a.hkv + h];
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
    uint32_t ko[2] = {0, 0}, vo[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t kb16 = (kw[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const uint32_t vb16 = (vw[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu;
      const uint32_t kc = float_to_e4m3(bf16_bits_to_float(kb16) / ks);
      const uint32_t vc = float_to_e4m3(bf16_bits_to_float(vb16) / vs);
      ko[i >> 2] |= kc << ((i & 3) * 8);
      vo[i >> 2] |= vc << ((i & 3) * 8);
    }
    *(uint2 *)((unsigned char *)a.k_cache + dst) = make_uint2(ko[0], ko[1]);
    *(uint2 *)((unsigned char *)a.v_cache + dst) = make_uint2(vo[0], vo[1]);
  }
}

// bf16 copy of E4M3 context for the prefill kernels: value = bf16(code *
// scale), the product rounded in fp32, then to bf16, both nearest-even (every
// code is exact in fp32).  A work-group converts blocks j0 .. j1-1 of one
// sequence for all KV heads, 16 codes per thread and step, and writes the
// compact block table entries of those blocks.
__global__ __launch_bounds__(256) void dequant_kernel(DequantArgs a) {
  const DqItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int32_t *btr = a.bt + (int64_t)it.seq * a.max_blocks;
  for (int j = it.j0 + tid; j < it.j1; j += 256) a.bt_out[(int64_t)it.seq * a.mb_out + j] = it.base + j;
  const int cpb = a.bs * a.d / 16;  // 16-byte chunks of codes per (block, head)
  const int64_t total = (int64_t)(it.j1 - it.j0) * a.hkv * cpb;
  constexpr int U = 4;  // chunks per thread whose loads are in flight together
  for (int64_t c0 = tid; c0 < total; c0 += U * 256) {
    uint4 w[U][2];
    int64_t src[U], dst[U];
    float sc[U][2];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int64_t c = min(c0 + u * 256, total - 1);  // a repeat of the last chunk is harmless
      const int ch = (int)(c % cpb);
      const int64_t jh = c / cpb;
      const int h = (int)(jh % a.hkv);
      const int j = it.j0 + (int)(jh / a.hkv);
      const int64_t blk = btr[j];
      src[u] = (blk * a.hkv + h) * a.bs * a.d + ch * 16;
      dst[u] = ((int64_t)(it.base + j) * a.hkv + h) * a.bs * a.d + ch * 16;
      sc[u][0] = a.ks[blk * a.hkv + h];
      sc[u][1] = a.vs[blk * a.hkv + h];
      w[u][0] = gload16_nt((const unsigned char *)a.k + src[u]);
      w[u][1] = gload16_nt((const unsigned char *)a.v + src[u]);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
#pragma unroll
      for (int kv = 0; kv < 2; kv++) {
        const uint32_t wd[4] = {w[u][kv].x, w[u][kv].y, w[u][kv].z, w[u][kv].w};
        const float scale = sc[u][kv];
        uint32_t o[8];
        auto pack = [&](float x, float y) {
          const __bf16 lo = (__bf16)(x * scale), hi = (__bf16)(y * scale);
          return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        };
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const auto f_lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], false);  // codes 4i, 4i+1
          const auto f_hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[i], true);   // codes 4i+2, 4i+3
          o[2 * i] = pack(f_lo[0], f_lo[1]);
          o[2 * i + 1] = pack(f_hi[0], f_hi[1]);
        }
        unsigned char *dp = (unsigned char *)(kv ? a.v_out : a.k_out) + dst[u] * 2;
        *(uint4 *)dp = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4 *)(dp + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

// Work-list copy from a pinned host buffer into the workspace (bytes is a
// multiple of 16, both addresses 16-byte aligned).
__global__ __launch_bounds__(256) void stage_kernel(const uint4 *src, uint4 *dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

hipError_t launch_stage(const void *src_host, void *dst, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 16 != 0 || (uintptr_t)src_host % 16 != 0 || (uintptr_t)dst % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(stage_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, (const uint4 *)src_host,
                     (uint4 *)dst, n16);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs &a, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3(n_items), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Raw gather of one sequence through its block-table row ([V1Sched]
// "Scheduler.schedule — 记账与状态": a request's KV lives in the blocks its
// id list names, in order).  One thread per 16-byte chunk of a row.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.total_chunks) return;
  const int cpr = a.row_bytes / 16;
  const int ch = (int)(gid % cpr);
  const int64_t th = gid / cpr;
  const int h = (int)(th % a.hkv);
  const int64_t p = th / a.hkv;
  const int64_t blk = a.bt_row[p / a.bs];
  const int64_t src = ((blk * a.hkv + h) * a.bs + p % a.bs) * a.row_bytes + ch * 16;
  const int64_t dst = th * a.row_bytes + ch * 16;
  *(uint4 *)((unsigned char *)a.k_out + dst) = *(const uint4 *)((const unsigned char *)a.k + src);
  *(uint4 *)((unsigned char *)a.v_out + dst) = *(const uint4 *)((const unsigned char *)a.v + src);
}

hipError_t launch_append(const AppendArgs &a, bool fp8, int64_t num_tokens, hipStream_t s) {
  // token pieces of at most 2^30 chunks each
  const int64_t row_chunks = (int64_t)a.hkv << a.lcpr;
  const int64_t piece = std::max<int64_t>(1, ((int64_t)1 << 30) / row_chunks);
  for (int64_t t0 = 0; t0 < num_tokens; t0 += piece) {
    AppendArgs b = a;
    b.tok0 = t0;
    b.nchunks = (uint32_t)(std::min(piece, num_tokens - t0) * row_chunks);
    const unsigned blocks = (b.nchunks + 255) / 256;
    if (fp8)
      hipLaunchKernelGGL(append_kernel<true>, dim3(blocks), dim3(256), 0, s, b);
    else
      hipLaunchKernelGGL(append_kernel<false>, dim3(blocks), dim3(256), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  if (a.total_chunks <= 0) return hipSuccess;
  const int64_t blocks = (a.total_chunks + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
