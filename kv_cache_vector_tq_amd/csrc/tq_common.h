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

// fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Exact split of 8 fp32 values into three bf16 terms: x = hi + mid + lo.  Each stage
// rounds to 8 significant bits and its remainder is exact in fp32 (Sterbenz), so the
// last remainder has at most 8 significant bits and fits bf16 exactly.
__device__ __forceinline__ void split3_bf16(const float* v, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  u16x8 h, m, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = v[e];
    const uint16_t bh = f2bf(x);
    const float r1 = x - bf2f(bh);
    const uint16_t bm = f2bf(r1);
    const float r2 = r1 - bf2f(bm);
    h[e] = bh;
    m[e] = bm;
    l[e] = f2bf(r2);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  mid = __builtin_bit_cast(bf16x8, m);
  lo = __builtin_bit_cast(bf16x8, l);
}

}  // namespace tq
