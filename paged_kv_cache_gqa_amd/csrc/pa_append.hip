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
// rounding and saturation to +-448.  4-bit caches ([V41] kernels section: an
// FP4 KV cache) are OCP MXFP4: the four threads of a 32-element group find
// its largest magnitude, whose exponent less 2 (the largest E2M1 exponent),
// clamped at 2^-127, is the group's E8M0 scale; each element divided by it
// (exact: a power of two) rounds to E2M1, nearest-even, saturating at 6.  A
// group holding a NaN or an infinity gets the NaN scale and zero codes.
#include <algorithm>

#include "pa_append.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <int FMT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  if (gid >= a.nchunks) return;
  append_chunk<FMT, true>(a, gid);
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

hipError_t launch_append(const AppendArgs &a, int fmt, int64_t num_tokens, hipStream_t s) {
  // token pieces of at most 2^30 chunks each
  const int64_t row_chunks = (int64_t)a.hkv << a.lcpr;
  const int64_t piece = std::max<int64_t>(1, ((int64_t)1 << 30) / row_chunks);
  for (int64_t t0 = 0; t0 < num_tokens; t0 += piece) {
    AppendArgs b = a;
    b.tok0 = t0;
    b.nchunks = (uint32_t)(std::min(piece, num_tokens - t0) * row_chunks);
    const unsigned blocks = (b.nchunks + 255) / 256;
    if (fmt == kKvE4m3)
      hipLaunchKernelGGL(append_kernel<kKvE4m3>, dim3(blocks), dim3(256), 0, s, b);
    else if (fmt == kKvMxfp4)
      hipLaunchKernelGGL(append_kernel<kKvMxfp4>, dim3(blocks), dim3(256), 0, s, b);
    else
      hipLaunchKernelGGL(append_kernel<kKvBf16>, dim3(blocks), dim3(256), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// MXFP4: the values, widened as the attention kernels widen them (bf16
// [ctx][hkv][d]); one thread per 8 elements: a dword of codes and its
// group's scale byte.
__global__ __launch_bounds__(256) void gather_fp4_kernel(GatherArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.total_chunks) return;
  const int d = a.row_bytes * 2;
  const int cpr = d / 8;
  const int ch = (int)(gid % cpr);
  const int64_t th = gid / cpr;
  const int h = (int)(th % a.hkv);
  const int64_t p = th / a.hkv;
  const int64_t blk = a.bt_row[p / a.bs];
  const int64_t row = (blk * a.hkv + h) * a.bs + p % a.bs;
  const int64_t sc = ((blk * a.hkv + h) * (d / 32) + ch / 4) * a.bs + p % a.bs;
  const int64_t dst = (th * d + ch * 8) * 2;
  const uint32_t kw = *(const uint32_t *)((const unsigned char *)a.k + row * a.row_bytes + ch * 4);
  const uint32_t vw = *(const uint32_t *)((const unsigned char *)a.v + row * a.row_bytes + ch * 4);
  const float ks = e8m0_operand(((const unsigned char *)a.ks)[sc]);
  const float vs = e8m0_operand(((const unsigned char *)a.vs)[sc]);
  *(bf16x8 *)((unsigned char *)a.k_out + dst) = fp4x8_to_bf16x8(kw, ks);
  *(bf16x8 *)((unsigned char *)a.v_out + dst) = fp4x8_to_bf16x8(vw, vs);
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  if (a.total_chunks <= 0) return hipSuccess;
  const int64_t blocks = (a.total_chunks + 255) / 256;
  if (a.fmt == kKvMxfp4)
    hipLaunchKernelGGL(gather_fp4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
