// pa_peak.hip -- measurement hooks: the practical ceilings of the two
// resources the attention kernels are bound by, measured with the
// instructions those kernels use, so a kernel's throughput can be read
// against what the chip delivers as well as against its published peaks.
//
//   peak_mfma_kernel  back-to-back v_mfma_f32_16x16x32_bf16 on register
//                     operands, one work-group of 8 waves per CU (the prefill
//                     kernel's shape), eight independent accumulators per wave
//                     so no MFMA waits on the one before it;
//   peak_read_kernel  a streaming read of a device buffer through LDS with
//                     the non-temporal LDS-filling loads of the decode kernels.
#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kPeakMfmaAcc = 8;

__global__ __launch_bounds__(512, 1) void peak_mfma_kernel(float *out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    a[e] = (__bf16)(float)((lane + e) & 7);
    b[e] = (__bf16)(0.125f * (float)e);
  }
  f32x4 acc[kPeakMfmaAcc];
#pragma unroll
  for (int j = 0; j < kPeakMfmaAcc; j++) acc[j] = f32x4{};
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int j = 0; j < kPeakMfmaAcc; j++) acc[j] = mfma16x16x32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakMfmaAcc; j++) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[blockIdx.x * 512 + threadIdx.x] = s;
}

// One work-group of four waves per compute unit (more resident waves measured
// slower: 6.3 TB/s with eight work-groups per CU against 7.2 with one).  Each
// wave streams contiguous 4 KB segments (segments dealt round-robin over the
// waves) into its own 4-stage LDS ring with the decode kernels'
// non-temporal LDS-filling loads (four 1 KB requests per segment), waits for
// a segment with vmcnt, reads it back (a checksum) and requests the segment
// four ahead into its stage.  Requests past the wave's last segment have an
// empty buffer range: they move nothing but keep the vmcnt accounting.
constexpr int kPeakStages = 4;
constexpr int kPeakSeg = 4096;

__global__ __launch_bounds__(256) void peak_read_kernel(const unsigned char *buf, int64_t nseg, uint32_t *out) {
  __shared__ __attribute__((aligned(16))) unsigned char ring_raw[4 * kPeakStages * kPeakSeg];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t nk = gw < nseg ? (nseg - gw + nwaves - 1) / nwaves : 0;  // this wave's segments
  lds_u8 *ring = (lds_u8 *)ring_raw + wave * kPeakStages * kPeakSeg;
  const uint32_t ring_addr = (uint32_t)(uintptr_t)ring;
  auto issue = [&](int64_t k) __attribute__((always_inline)) {
    const int64_t seg = gw + min(k, max(nk - 1, (int64_t)0)) * nwaves;  // this request's segment
    const uint64_t base = (uint64_t)(buf + seg * kPeakSeg);
    const int nrec = __builtin_amdgcn_readfirstlane(k < nk ? kPeakSeg : 0);
    const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                       __builtin_amdgcn_readfirstlane((int)((base >> 32) & 0xFFFF)), nrec, kRsrcFlags};
    const uint32_t st = ring_addr + (uint32_t)(k % kPeakStages) * kPeakSeg;
#pragma unroll
    for (int j = 0; j < 4; j++) dma_load16_nt(r, lane * 16 + j * 1024, st + j * 1024);
  };
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kPeakStages; k++) issue(k);
  for (int64_t k = 0; k < nk; k++) {
    PA_WAIT_VMCNT(4 * (kPeakStages - 1));  // segment k has landed
    const lds_u8 *st = ring + (k % kPeakStages) * kPeakSeg;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const uint4 v = lds_load16(st + j * 1024 + lane * 16);
      x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage is read before it is refilled
    issue(k + kPeakStages);
  }
  PA_WAIT_VMCNT(0);
  out[blockIdx.x * 256 + threadIdx.x] = x;
}

hipError_t launch_peak_mfma(float *out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(kPeakMfmaGroups), dim3(512), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_read(const void *buf, int64_t bytes, uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(peak_read_kernel, dim3(kPeakReadGroups), dim3(256), 0, s,
                     (const unsigned char *)buf, bytes / kPeakSeg, out);
  return hipGetLastError();
}

// Which XCD runs each work-group: work-group w writes the XCC id its waves
// read from the hardware register (one 64-thread work-group per id).
__global__ __launch_bounds__(64) void xcc_ids_kernel(int32_t *out, int n) {
  int xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  if (threadIdx.x == 0 && (int)blockIdx.x < n) out[blockIdx.x] = xcc & 0xF;
}

hipError_t launch_xcc_ids(int32_t *out, int n, hipStream_t s) {
  hipLaunchKernelGGL(xcc_ids_kernel, dim3(n), dim3(64), 0, s, out, n);
  return hipGetLastError();
}

}  // namespace pa
