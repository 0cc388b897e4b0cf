// Device helpers shared by the kernels: vector types, bf16/fp16 conversions and
// the MFMA wrappers.  gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace svdq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// bf16 bits <-> fp32
__device__ __forceinline__ float bf_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// Two fp32 -> packed bf16 pair, round to nearest even, with the gfx950 convert
// (one instruction; a in the low half).
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) { return cvt_bf2(a, b); }

// a / b correctly rounded, given r = 1/b correctly rounded: the estimate a r is
// refined twice with fused multiply-adds (q <- q + (a - q b) r); the first step
// makes the estimate faithful, the second gives the nearest-even quotient.  This
// was checked against IEEE division for every bf16 dividend over 3000 divisors
// and for 8e8 fp32 dividends over fp16-valued divisors, in the range
// |a| >= 2^-80, 2^-100 <= |a / b| < 2^100 (it is Markstein's refinement
// theorem: a faithful quotient refined once with the correctly rounded
// reciprocal is the correctly rounded quotient, while nothing underflows).
// Outside that range (zeros, tiny values whose remainder would underflow, huge
// quotients) the caller uses the IEEE division.
__device__ __forceinline__ float div_refined(float a, float b, float r) {
  float q = a * r;
  q = fmaf(fmaf(-q, b, a), r, q);
  q = fmaf(fmaf(-q, b, a), r, q);
  return q;
}

// The E8M0 exponent byte of a group maximum: e = floor(log2 amax) - 2 clamped to
// [-127, 127], stored as e + 127.  For a normal amax with biased exponent be this is
// be - 2 (at least 0); zero and subnormal maxima give byte 0 (e = -127).
__device__ __forceinline__ uint32_t e8m0_of_amax(float amax) {
  const int be = int((__float_as_uint(amax) >> 23) & 0xFFu);
  return uint32_t(be > 2 ? be - 2 : 0);
}

// The scale byte b as the gfx950 convert's scale operand: the convert divides by
// 2^(E - 127), E the operand's fp32 exponent field, before rounding, so the byte
// goes into that field (b = 0 gives +0.0, i.e. 2^-127).  The division by a power
// of two is exact, so cvt_fp4x2_div(.., x, y, scale_operand(b)) encodes exactly
// x * 2^(127 - b), with no multiply (and no underflow of that product) in fp32.
__device__ __forceinline__ float scale_operand(uint32_t b) { return __uint_as_float(b << 23); }

// Two fp32 -> packed E2M1 pair in byte `sel` of `old` (nearest, ties to even,
// saturating at 6, sign copied): the gfx950 convert with unit scale.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}
// The same of a / 2^(E - 127) and b / 2^(E - 127), E the exponent field of s.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_div(uint32_t old, float a, float b, float s) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, SEL);
}

template <int SEL>
__device__ __forceinline__ v4f mfma_fp4_sel(const uint4& a, const uint4& b, v4f c, uint32_t sa, uint32_t sb) {
  v8i av = {int(a.x), int(a.y), int(a.z), int(a.w), 0, 0, 0, 0};
  v8i bv = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, SEL, int(sa), SEL, int(sb));
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_f16(const uint4& a, const uint4& b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_bf16(const uint4& a, const uint4& b, v4f c) {
  v8s as = {short(a.x), short(a.x >> 16), short(a.y), short(a.y >> 16),
            short(a.z), short(a.z >> 16), short(a.w), short(a.w >> 16)};
  v8s bs = {short(b.x), short(b.x >> 16), short(b.y), short(b.y >> 16),
            short(b.z), short(b.z >> 16), short(b.w), short(b.w >> 16)};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, as), __builtin_bit_cast(v8bf, bs), c, 0, 0, 0);
}

__device__ __forceinline__ v4i mfma_i8(const v4i& a, const v4i& b) {
  v4i z = {0, 0, 0, 0};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, z, 0, 0, 0);
}

// 8 packed two's complement nibbles -> 8 signed bytes, each 16 times its code,
// in two dwords (the low nibbles of the 4 bytes in the first, the high nibbles
// in the second; in the INT4 code order these are codes 0-3 and 4-7).  A
// nibble moved to the top of its byte is its code times 16 as a signed byte, so
// this is one mask per dword and a shift: an int8 product of two such operands
// is 256 times the codes' product, exactly.
__device__ __forceinline__ void unpack_i4x8_x16(uint32_t d, int& first, int& second) {
  first = int((d << 4) & 0xF0F0F0F0u);
  second = int(d & 0xF0F0F0F0u);
}

// 8 packed bf16 -> fp32, element order kept
__device__ __forceinline__ void unpack_bf8(const uint4& r, float (&a)[8]) {
  a[0] = bf_lo(r.x); a[1] = bf_hi(r.x); a[2] = bf_lo(r.y); a[3] = bf_hi(r.y);
  a[4] = bf_lo(r.z); a[5] = bf_hi(r.z); a[6] = bf_lo(r.w); a[7] = bf_hi(r.w);
}

// max over the lanes l and l ^ 16 (the 2 lanes that hold a 16-element half of a row's 32-block)
__device__ __forceinline__ float rowpair_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
}

// Nearest E4M3 byte of a non-negative u (ties to even), saturating at 448 (also
// for +inf).  Below 2^-6 the format's step is 2^-9, so the byte is rint(u 2^9)
// (8 is the smallest normal, whose byte is 8); above, the fp32 mantissa is
// rounded to 3 bits and a carry runs into the exponent field.
__device__ __forceinline__ uint32_t e4m3_rne(float u) {
  if (!(u < 448.0f)) return 0x7Eu;
  const uint32_t b = __float_as_uint(u);
  const int E = int(b >> 23) - 127;
  if (E < -6) return uint32_t(__builtin_rintf(u * 512.0f));
  const uint32_t m = b & 0x7FFFFFu;
  const uint32_t keep = m >> 20, rem = m & 0xFFFFFu;
  const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
  return (uint32_t(E + 7) << 3) + keep + up;
}

// fp32 value of a non-negative E4M3 byte (sign bit clear, not the NaN code):
// (mn + 8) 2^(ex - 10) for ex >= 1, mn 2^-9 for ex = 0.  The gfx950 fp8
// convert decodes the OCP E4M3 format exactly (a device check compared it with
// that formula for every byte 0..126), in one instruction.
__device__ __forceinline__ float e4m3_value(uint32_t s) { return __builtin_amdgcn_cvt_f32_fp8(int(s), 0); }

// max over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the 4 lanes that hold one row's group)
__device__ __forceinline__ float rowgroup_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float a = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const uint32_t ua = __float_as_uint(a);
  const auto p32 = __builtin_amdgcn_permlane32_swap(ua, ua, false, false);
  return fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// sum over the lanes l, l ^ 16, l ^ 32, l ^ 48: rows 0+1 and 2+3, then the two
// pair sums (every lane ends with the same value, in a fixed order)
__device__ __forceinline__ float rowgroup_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto p16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float a = __uint_as_float(p16[0]) + __uint_as_float(p16[1]);
  const uint32_t ua = __float_as_uint(a);
  const auto p32 = __builtin_amdgcn_permlane32_swap(ua, ua, false, false);
  return __uint_as_float(p32[0]) + __uint_as_float(p32[1]);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// True when some of the 16 bf16 values is outside the fast divisions' range:
// a biased exponent outside [87, 187), i.e. |x| < 2^-40 or |x| >= 2^60
// (subnormals and -0 included), except +0, which every path (two-operation,
// refined, IEEE) divides to +0 by a positive divisor.  Per 16-bit half:
// ((bits & 0x7F80) - 0x2B80) mod 2^16 > 0x3180, masked to 0 when bits == 0.
__device__ __forceinline__ bool exp_out_of_range(const uint4& a, const uint4& b) {
  const u16x2 lo = {0x2B80, 0x2B80}, one = {1, 1};
  auto f = [&](uint32_t v) {
    const u16x2 nz = __builtin_elementwise_min(__builtin_bit_cast(u16x2, v), one);
    return (__builtin_bit_cast(u16x2, v & 0x7F807F80u) - lo) * nz;
  };
  const u16x2 m = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_elementwise_max(f(a.x), f(a.y)), __builtin_elementwise_max(f(a.z), f(a.w))),
      __builtin_elementwise_max(__builtin_elementwise_max(f(b.x), f(b.y)), __builtin_elementwise_max(f(b.z), f(b.w))));
  return (m.x > m.y ? m.x : m.y) > 0x3180;
}

// GELU in the erf form, y * Phi(y) = (y + |y| erf(|y| / sqrt 2)) / 2, with erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.28:
//   erf(z) = 1 - 1 / (1 + a1 z + a2 z^2 + ... + a6 z^6)^16,  z >= 0, absolute error <= 3e-7.
// Six FMAs, four squarings and one reciprocal (no exponential); in fp32 the GELU is
// within 1e-6 of the exact one for every y.  A large |y| makes the power overflow to
// +inf, whose reciprocal is 0, so GELU(y) = max(y, 0) there.
__device__ __forceinline__ float gelu_erf(float y) {
  const float z = fabsf(y) * 0.70710678118654752f;
  float p = fmaf(0.0000430638f, z, 0.0002765672f);
  p = fmaf(p, z, 0.0001520143f);
  p = fmaf(p, z, 0.0092705272f);
  p = fmaf(p, z, 0.0422820123f);
  p = fmaf(p, z, 0.0705230784f);
  p = fmaf(p, z, 1.0f);
  p *= p;
  p *= p;
  p *= p;
  p *= p;
  const float erf_z = 1.0f - __builtin_amdgcn_rcpf(p);
  const float hy = 0.5f * y;                        // halved first: no overflow near the fp32 maximum
  return fmaf(fabsf(hy), erf_z, hy);
}

// Hardware round-robins workgroups over the 8 XCDs (workgroup i runs on XCD i % 8).
// Map the dispatch index to a logical tile index so that each XCD works on a
// contiguous range of tiles (and so shares operands in its own L2).
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

// Buffer resource over [base, base + bytes): loads beyond the end return zero
// and stores beyond it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int nx = 8;
  const int xcd = bid % nx, slot = bid / nx;
  const int per = nblocks / nx, rem = nblocks % nx;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

}  // namespace svdq
