// Device-side helpers shared by the gfx950 kernels of libtq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;
constexpr float SQRT_D = 11.313708498984761f;      // sqrt(128)
constexpr float INV_SQRT_D = 0.08838834764831845f;  // 1/sqrt(128)

// 16x16x32 MFMA, fp32 accumulation.  Output lane l holds rows 4*(l/16)+i, column l%16.
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 bf16 values from 16 bytes (16-byte aligned).
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Splits 8 fp32 values in f16's range into two f16 terms hi + lo: hi truncated (round toward
// zero), so that v - hi is exact in fp32, and lo that remainder rounded to nearest.  For v in
// f16's normal range |v - hi - lo| <= 2^-21 |v|; below it the error is at most 2^-25.
__device__ __forceinline__ void split2_f16(const float* v, f16x8& hi, f16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const auto hp = __builtin_amdgcn_cvt_pkrtz(v[2 * p], v[2 * p + 1]);
    const _Float16 l0 = static_cast<_Float16>(v[2 * p] - static_cast<float>(hp[0]));
    const _Float16 l1 = static_cast<_Float16>(v[2 * p + 1] - static_cast<float>(hp[1]));
    h[p] = __builtin_bit_cast(uint32_t, hp);
    l[p] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
  }
  hi = __builtin_bit_cast(f16x8, h);
  lo = __builtin_bit_cast(f16x8, l);
}

// Exact split of 8 fp32 values into three bf16 terms: x = hi + mid + lo.  hi is x truncated
// to its top 16 bits (a bf16 value); the remainder x - hi is exact in fp32 and has at most
// 16 significant bits; mid is that remainder truncated the same way, and the last remainder
// has at most 8 significant bits, so it is a bf16 value too.  Each pair of terms is packed
// from the high halves of two fp32 words with one byte permute.
__device__ __forceinline__ void split3_bf16(const float* v, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  u32x4 h, m, l;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t x0 = __float_as_uint(v[2 * p]), x1 = __float_as_uint(v[2 * p + 1]);
    const float r0 = v[2 * p] - __uint_as_float(x0 & 0xFFFF0000u);
    const float r1 = v[2 * p + 1] - __uint_as_float(x1 & 0xFFFF0000u);
    const uint32_t y0 = __float_as_uint(r0), y1 = __float_as_uint(r1);
    const float s0 = r0 - __uint_as_float(y0 & 0xFFFF0000u);
    const float s1 = r1 - __uint_as_float(y1 & 0xFFFF0000u);
    // bytes 2, 3 of the second operand, then bytes 2, 3 of the first: {a.hi16, b.hi16}
    h[p] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
    m[p] = __builtin_amdgcn_perm(y1, y0, 0x07060302u);
    l[p] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  mid = __builtin_bit_cast(bf16x8, m);
  lo = __builtin_bit_cast(bf16x8, l);
}

}  // namespace tq
