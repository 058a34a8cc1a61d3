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
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

template <bool FP8>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.total_chunks) return;
  const int cpr = a.d / 8;
  const int ch = (int)(gid % cpr);
  const int64_t th = gid / cpr;
  const int h = (int)(th % a.hkv);
  const int64_t t = th / a.hkv;
  const int64_t slot = a.slots[t];
  if (slot < 0) return;
  const int64_t blk = slot / a.bs, off = slot % a.bs;
  const int64_t src = th * a.d + ch * 8;                                // element offset
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

hipError_t launch_append(const AppendArgs &a, bool fp8, hipStream_t s) {
  if (a.total_chunks <= 0) return hipSuccess;
  const int64_t blocks = (a.total_chunks + 255) / 256;
  if (fp8)
    hipLaunchKernelGGL(append_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  if (a.total_chunks <= 0) return hipSuccess;
  const int64_t blocks = (a.total_chunks + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
