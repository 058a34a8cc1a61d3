// pa_append.h -- the kv_append chunk routine, shared by the kv_append kernel
// and the one-launch step kernel.
#pragma once
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One thread's 16-byte chunk (8 elements) of one (token, KV head) row: chunk
// gid of the launch's tokens from a.tok0 on.  32-bit index arithmetic within
// a launch (the host keeps each launch below 2^31 chunks) and shifts for the
// power-of-two sizes: the 64-bit divisions this replaces cost more
// instructions than the copy itself.  The four threads of a 32-element group
// are adjacent lanes (MXFP4 reduces its largest magnitude across them).
// NT: bf16 rows are stored non-temporally (the kv_append kernel: the rows
// are read back by a later kernel, if at all; 1.7% faster at 1M tokens than
// ordinary stores); the one-launch step kernel, whose attention reads them
// back within the launch, stores them ordinarily.
template <int FMT, bool NT = false>
__device__ __forceinline__ void append_chunk(const AppendArgs &a, uint32_t gid) {
  const uint32_t ch = gid & ((1u << a.lcpr) - 1);
  const uint32_t row = gid >> a.lcpr;  // (token, KV head) row of this launch
  const uint32_t tl = row / (uint32_t)a.hkv;
  const int h = (int)(row - tl * (uint32_t)a.hkv);
  const int64_t t = a.tok0 + tl;
  const int64_t slot = a.slots[t];
  // (the threads of a row share its slot: a 32-element group, four adjacent
  // lanes of one row, is skipped or kept as a whole)
  if (slot < 0) return;
  const int64_t blk = slot >> a.lbs, off = slot & (a.bs - 1);
  const int64_t src = (t * a.hkv + h) * a.d + ch * 8;                   // element offset
  const int64_t dst = ((blk * a.hkv + h) * a.bs + off) * a.d + ch * 8;  // element offset
  const uint4 kv = gload16_nt((const unsigned char *)a.k_new + src * 2);
  const uint4 vv = gload16_nt((const unsigned char *)a.v_new + src * 2);
  if constexpr (FMT == kKvBf16) {
    if constexpr (NT) {
      __builtin_nontemporal_store(u32x4{kv.x, kv.y, kv.z, kv.w}, (u32x4 *)((unsigned char *)a.k_cache + dst * 2));
      __builtin_nontemporal_store(u32x4{vv.x, vv.y, vv.z, vv.w}, (u32x4 *)((unsigned char *)a.v_cache + dst * 2));
    } else {
      *(uint4 *)((unsigned char *)a.k_cache + dst * 2) = kv;
      *(uint4 *)((unsigned char *)a.v_cache + dst * 2) = vv;
    }
  } else if constexpr (FMT == kKvMxfp4) {
    const int64_t sdst = ((blk * a.hkv + h) * (a.d >> 5) + (ch >> 2)) * a.bs + off;  // scale byte
    auto encode = [&](const uint4 x, unsigned char *codes, unsigned char *scales) {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      float f[8];
      float amax = 0.f;
      bool finite = true;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        f[i] = bf16_bits_to_float((w[i >> 1] >> ((i & 1) * 16)) & 0xFFFFu);
        const float m = __builtin_fabsf(f[i]);
        finite = finite && m <= 3.4028235e38f;  // false for infinities and NaN
        amax = fmaxf(amax, m);
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      int fin = finite ? 1 : 0;
      fin &= __shfl_xor(fin, 1);
      fin &= __shfl_xor(fin, 2);
      // the shared exponent: amax's exponent field less 2, at least 0 (a
      // subnormal or zero amax has field 0)
      const int ef = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFFu);
      const uint32_t e = fin ? (uint32_t)max(ef - 2, 0) : 0xFFu;
      const float inv = __builtin_bit_cast(float, (254u - min(e, 253u)) << 23);  // 2^(127 - e), e <= 252
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 8; i++) packed |= (fin ? e2m1_code(f[i] * inv) : 0u) << (4 * i);
      *(uint32_t *)(codes + dst / 2) = packed;
      if ((ch & 3) == 0) scales[sdst] = (unsigned char)e;
    };
    encode(kv, (unsigned char *)a.k_cache, (unsigned char *)a.ks);
    encode(vv, (unsigned char *)a.v_cache, (unsigned char *)a.vs);
  } else {
    const float ks = ((const float *)a.ks)[blk * a.hkv + h];
    const float vs = ((const float *)a.vs)[blk * a.hkv + h];
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

}  // namespace pa
