// pa_device.h -- gfx950 device helpers: vector types, MFMA wrappers,
// LDS transpose reads, OCP E4M3 <-> float conversions written from the
// format's definition.  Library-internal.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// D = A * B + C on the matrix cores.  Lane layouts (verified on gfx950):
//  32x32x16: A lane l holds row l%32, k = 8*(l/32) .. +7; B lane l holds column
//            l%32, same k; C/D element 4*i+r of lane l is row 8*i + 4*(l/32) + r,
//            column l%32.
//  16x16x32: A row l%16, k = 8*(l/16) .. +7; B column l%16; D element r is row
//            4*(l/16) + r, column l%16.
//  16x16x16: as 16x16x32 with k = 4*(l/16) .. +3.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit elements (row j/4, columns 4*(j%4)..+3 of a
// 4 x 16 tile); lane i receives column i of that tile (rows 0..3).
__device__ __forceinline__ bf16x4 lds_read_tr(const lds_u8 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
}

// Cross-lane reductions between lane l and lane l ^ 32 (or l ^ 16) without
// an LDS round trip.  v_permlane32_swap exchanges lanes 32-63 of its first
// operand with lanes 0-31 of its second; fed the same value twice, the two
// results hold {v[l], v[l ^ 32]} in some order, so any symmetric operation
// of the pair is the same on every lane.  v_permlane16_swap does the same
// between odd and even 16-lane rows (lane l and lane l ^ 16).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ uint4 lds_load16(const lds_u8 *p) {
  u32x4 v = *(const lds_u32x4 *)p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ uint2 lds_load8(const lds_u8 *p) {
  u32x2 v = *(const lds_u32x2 *)p;
  return make_uint2(v[0], v[1]);
}
// Transposing 8-byte read of 8-bit elements: within each 16-lane group,
// lanes 2k and 2k+1 address the two 8-byte halves of "row" k (k = 0..7),
// and lane j of the group receives byte j of each of the 8 rows, row k in
// byte k of the result.
typedef int i32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 lds_read_tr8(const lds_u8 *p) {
  const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t *)p);
  return make_uint2((uint32_t)v[0], (uint32_t)v[1]);
}
__device__ __forceinline__ void lds_store16(lds_u8 *p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  *(lds_u32x4 *)p = w;
}

// Global loads: cached (tiles re-read by other work-groups) and streaming
// (bytes read exactly once, kept out of the caches' way).
__device__ __forceinline__ uint4 gload16(const void *p) { return *(const uint4 *)p; }
__device__ __forceinline__ uint2 gload8(const void *p) { return *(const uint2 *)p; }
__device__ __forceinline__ uint4 gload16_nt(const void *p) {
  u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 gload8_nt(const void *p) {
  u32x2 v = __builtin_nontemporal_load((const u32x2 *)p);
  return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// OCP E4M3 ("e4m3fn"): sign, 4-bit exponent (bias 7), 3-bit mantissa; exponent
// field 0 holds subnormals m * 2^-9; S.1111.111 is NaN; no infinities.

// Exact widening of one code to float (every E4M3 value is a float).
__device__ __forceinline__ float e4m3_to_float(uint32_t c) {
  uint32_t em = c & 0x7Fu;
  float v;
  if (em >= 8u)
    v = __builtin_bit_cast(float, (em << 20) + (120u << 23));  // rebias 7 -> 127
  else
    v = (float)em * 0x1p-9f;
  if (em == 0x7Fu) v = __builtin_nanf("");
  return (c & 0x80u) ? -v : v;
}

// Eight codes (little-endian in two words) -> eight bf16 (exact).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 w) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t word = i < 2 ? w.x : w.y;
    uint32_t sh = (i & 1) * 16;
    float lo = e4m3_to_float((word >> sh) & 0xFFu);
    float hi = e4m3_to_float((word >> (sh + 8)) & 0xFFu);
    // a float holding an E4M3 value has at most 4 significant bits: the
    // upper half is the exact bf16 pattern.
    out[i] = (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// The same widening with gfx950's conversion instruction (OCP E4M3 -> bf16,
// two codes per instruction; a scale of 1.0 leaves the values exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8_hw(uint2 w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true);
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// OCP MXFP4 -> bf16 with gfx950's conversion instruction: byte SEL of w
// holds two E2M1 codes (the lower-indexed element in the low 4 bits); the
// scale operand is the float whose bit pattern is e << 23, which the
// instruction applies as the E8M0 scale 2^(e - 127) (e = 0 and the NaN scale
// e = 255 included -- checked against the format's definition over every
// (byte, e) pair).  A code times a power of two is exact in bf16.
__device__ __forceinline__ float e8m0_operand(uint32_t e) { return __builtin_bit_cast(float, e << 23); }
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w, float sc) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, SEL));
}
// eight codes (one dword, elements in order) sharing one scale
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float sc) {
  return as_bf16x8(make_uint4(fp4x2_to_bf16x2<0>(w, sc), fp4x2_to_bf16x2<1>(w, sc), fp4x2_to_bf16x2<2>(w, sc),
                              fp4x2_to_bf16x2<3>(w, sc)));
}

// E2M1 code of a value already divided by its group's scale: nearest of 0,
// 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even mantissa (rint in the
// binade's step: 0.5 below 2, 1 below 4, 2 above), magnitudes >= 6 saturate;
// the sign bit is v's.  The code is the step count plus the binade's offset.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const uint32_t sign = (__builtin_bit_cast(uint32_t, v) >> 28) & 8u;
  const float a = __builtin_fabsf(v);
  uint32_t c;
  if (a < 2.f)
    c = (uint32_t)__builtin_rintf(a * 2.f);
  else if (a < 4.f)
    c = (uint32_t)__builtin_rintf(a) + 2u;
  else if (a < 6.f)
    c = (uint32_t)__builtin_rintf(a * 0.5f) + 4u;
  else
    c = 7u;
  return sign | c;
}

// Round a float to E4M3, nearest-even, saturating finite and infinite
// magnitudes above 448 to 448; NaN -> 0x7F with the input's sign.
__device__ __forceinline__ uint32_t float_to_e4m3(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448 (and +-inf)
  if (a < 0x3C800000u) {                      // below 2^-6: grid m * 2^-9
    float q = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
    return sign | (uint32_t)q;
  }
  // keep 3 mantissa bits with round-to-nearest-even on the 20 dropped bits;
  // a carry moves into the exponent field by itself
  uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  uint32_t code = r - (120u << 3);  // exponent bias 127 -> 7
  if (code > 0x7Eu) code = 0x7Eu;
  return sign | code;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __builtin_bit_cast(float, b16 << 16);
}

// LDS-filling buffer loads: buffer_load_dwordx4 ... lds writes the 64 lanes'
// 16-byte results to LDS at M0 + 16 * lane.  The resource descriptor is
// {base lo, base hi & 0xFFFF, bytes in range, kRsrcFlags}; lanes whose
// offset lies past the range read zeros.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format

// The compiler does not see inside the asm, so it cannot pad the hazards of
// its operands: the resource words come from v_readfirstlane (a VALU write
// of an SGPR needs 5 wait states before a vector-memory instruction reads
// it) and M0 was just written by a scalar move (1 wait state before a load
// that writes LDS).  The leading s_nop 4 provides both.
__device__ __forceinline__ void dma_load16(i32x4_t rsrc, int voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}
// the same with the non-temporal hint, for data read once
__device__ __forceinline__ void dma_load16_nt(i32x4_t rsrc, int voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}
// one dword per lane (buffer_load_dword ... lds writes lane l's 4 bytes to
// M0 + 4 * lane): with the same offset in every lane, 64 copies of one value
__device__ __forceinline__ void dma_load4(i32x4_t rsrc, int voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}
// s_waitcnt vmcnt(n), expcnt and lgkmcnt unconstrained (n < 64: the count's
// low four bits sit in bits 3:0 of the immediate, its high two in bits 15:14)
#define PA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | (7 << 4) | (15 << 8))

}  // namespace pa
