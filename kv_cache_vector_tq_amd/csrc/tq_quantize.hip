// Quantize-on-write kernel for gfx950 and its C-ABI entry point tq_quantize_kv.
//
// What is computed (pages: "Когда в марте 2026 года Google опубликовала статью..." - random
// orthogonal rotation, per-coordinate Lloyd-Max code, QJL correction of the residual;
// "Google TurboQuant простыми словами", step 2 - the residual's Johnson-Lindenstrauss
// sign sketch; section "Бенчмарки TurboQuant" - one 4-byte side value per 128 values):
//   n = ||x||, y = R_eff x / n, z = sqrt(d) y, code_j = #{l : z_j >= t_l};
//   keys with the sketch: r = y - c[code]/sqrt(d) (r = y without codes), rnorm = ||r||,
//   sign_j = [(S_b r)_j >= 0].
//
// One workgroup (4 waves) owns one 64-token block of one (batch row, kv-head), so it is
// the only writer of that block.  Wave w computes output coordinates 32w..32w+31 of all
// 64 tokens with 16x16x32 bf16 MFMAs:
//   * rotation: bf16 inputs are exact, R_eff = R_hi + R_lo takes two passes (fp32 inputs
//     are split into three exact bf16 terms first), all products exact, fp32 accumulation;
//   * sketch: r (fp32) is split into three exact bf16 terms, S_b is bf16, so u = S_b r is
//     the fp32-accumulated product of the fp32 residual.
// The k dimension of every MFMA maps lane group g, element e of k-block kb to coordinate
// 32 g + 8 kb + e on both operands, so the sum runs over all 128 coordinates.
#include <hip/hip_runtime.h>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int XS_BF16 = 136;  // LDS row stride (bf16 elements) of the input tile
constexpr int XS_F32 = 132;   // LDS row stride (floats) of the fp32 input / residual tile
constexpr int IDX_STRIDE = 144;  // LDS row stride (bytes) of the code / sign tiles

struct QuantArgs {
  const void* x;
  int64_t sb, sh, st;
  const int32_t* start_pos;
  int n_new, Hkv, T_cap;
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* s_b;
  uint8_t* codes;  // key codes or value codes of the cache
  uint8_t* signs;
  float* norm;
  float* rnorm;
  float centroids[16];
  float thresholds[16];
};

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p));
}

// Packs 32 codes of BITS bits (code j at bit BITS*j) into BITS dwords.
template <int BITS>
__device__ __forceinline__ void pack32(const uint8_t* c, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t v = c[j];
    const int bit = BITS * j;
    const int word = bit >> 5, off = bit & 31;
    w[word] |= v << off;
    if (off + BITS > 32) w[word + 1] |= v >> (32 - off);
  }
}

// KEY: key layout (and sketch when QJL); otherwise value layout.  BITS = 0 only for keys
// that keep only the sketch.  F32: input elements are fp32 (else bf16).
template <bool KEY, int BITS, bool QJL, bool F32>
__global__ void __launch_bounds__(256) quantize_kernel(QuantArgs a) {
  constexpr int L = 1 << (BITS > 0 ? BITS : 1);
  __shared__ __attribute__((aligned(16))) float s_tile[64 * XS_F32];  // input tile, later residuals
  __shared__ __attribute__((aligned(16))) uint8_t s_idx[64 * IDX_STRIDE];
  __shared__ __attribute__((aligned(16))) uint8_t s_sgn[64 * IDX_STRIDE];
  __shared__ float s_norm[64];
  __shared__ float s_rnorm[64];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int start = a.start_pos[b];
  if (start < 0) return;
  const int end = min(start + a.n_new, a.T_cap);  // one past the last slot written
  const int blk = start / 64 + blockIdx.x;
  const int p0 = blk * 64;
  if (p0 >= end) return;  // uniform over the workgroup
  const int lo_slot = max(start, p0), hi_slot = min(end, p0 + 64);

  // ---- load the tile, row norms ----------------------------------------------------------
  // The norm is taken after an exact power-of-two rescaling by the row's largest magnitude,
  // so that squares neither overflow nor underflow fp32 over the whole bf16 / fp32 range.
  {
    const int row = tid >> 2, q = tid & 3;
    const int slot = p0 + row;
    const bool valid = slot >= lo_slot && slot < hi_slot;
    float v[32];
    if constexpr (F32) {
      const float* src = reinterpret_cast<const float*>(a.x) + (int64_t)b * a.sb + (int64_t)h * a.sh +
                         (int64_t)(slot - start) * a.st + 32 * q;
      float* dst = s_tile + row * XS_F32 + 32 * q;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (valid) x = *reinterpret_cast<const f32x4*>(src + 4 * i);
        *reinterpret_cast<f32x4*>(dst + 4 * i) = x;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = x[e];
      }
    } else {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(a.x) + (int64_t)b * a.sb + (int64_t)h * a.sh +
                            (int64_t)(slot - start) * a.st + 32 * q;
      uint16_t* dst = reinterpret_cast<uint16_t*>(s_tile) + row * XS_BF16 + 32 * q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u16x8 x = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (valid) x = *reinterpret_cast<const u16x8*>(src + 8 * i);
        *reinterpret_cast<u16x8*>(dst + 8 * i) = x;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * i + e] = bf2f(x[e]);
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(v[e]));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    int ex = 0;
    if (mx > 0.f) frexpf(mx, &ex);
    // mx * 2^-ex lies in [0.5, 1); the scale is applied in two exact halves so that neither
    // factor leaves the fp32 range for any finite input
    const float sc1 = ldexpf(1.0f, -ex / 2), sc2 = ldexpf(1.0f, -ex - (-ex / 2));
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float t = (v[e] * sc1) * sc2;
      ss = fmaf(t, t, ss);
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (q == 0) s_norm[row] = mx > 0.f ? ldexpf(sqrtf(ss), ex) : 0.f;
  }
  __syncthreads();

  // ---- rotation: acc[mt][nt] = X[16 mt.., :] R_eff[32 wave + 16 nt.., :]^T ---------------
  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    bf16x8 rh[2][4], rl[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int o = 32 * wave + 16 * nt + col;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        rh[nt][kb] = load_bf16x8(a.r_hi + o * D + 32 * grp + 8 * kb);
        rl[nt][kb] = load_bf16x8(a.r_lo + o * D + 32 * grp + 8 * kb);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int row = 16 * mt + col;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (F32) {
          const float* src = s_tile + row * XS_F32 + 32 * grp + 8 * kb;
          float v[8];
          *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(src);
          *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(src + 4);
          bf16x8 xh, xm, xl;
          split3_bf16(v, xh, xm, xl);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            acc[mt][nt] = mfma_bf16(xh, rh[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xh, rl[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xm, rh[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xm, rl[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xl, rh[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xl, rl[nt][kb], acc[mt][nt]);
          }
        } else {
          const bf16x8 xv =
              load_bf16x8(reinterpret_cast<const uint16_t*>(s_tile) + row * XS_BF16 + 32 * grp + 8 * kb);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            acc[mt][nt] = mfma_bf16(xv, rh[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xv, rl[nt][kb], acc[mt][nt]);
          }
        }
      }
    }
  }
  __syncthreads();  // the input tile is dead from here on; its space holds residuals

  // ---- scale, scalar code, residual -------------------------------------------------------
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * grp + i;
      const float n = s_norm[row];
      const float inv = n > 0.f ? 1.0f / n : 0.f;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int o = 32 * wave + 16 * nt + col;
        const float y = acc[mt][nt][i] * inv;
        const float z = y * SQRT_D;
        float c = 0.f;
        if constexpr (BITS > 0) {
          int idx = 0;
          c = a.centroids[0];
#pragma unroll
          for (int l = 1; l < L; ++l) {
            const bool ge = z >= a.thresholds[l - 1];
            idx = ge ? l : idx;
            c = ge ? a.centroids[l] : c;
          }
          s_idx[row * IDX_STRIDE + o] = static_cast<uint8_t>(idx);
        }
        if constexpr (KEY && QJL) {
          float r = (BITS > 0) ? (y - c * INV_SQRT_D) : y;
          if (!(n > 0.f)) r = 0.f;
          s_tile[row * XS_F32 + o] = r;
        }
      }
    }
  }
  __syncthreads();

  if constexpr (KEY && QJL) {
    // ---- residual norms ---------------------------------------------------------------------
    if constexpr (BITS > 0) {
      const int row = tid >> 2, q = tid & 3;
      const float* src = s_tile + row * XS_F32 + 32 * q;
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) ss += src[j] * src[j];
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if (q == 0) s_rnorm[row] = s_norm[row] > 0.f ? sqrtf(ss) : 0.f;
    }
    // ---- sketch: u = S_b r, signs -----------------------------------------------------------
    bf16x8 sb[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int o = 32 * wave + 16 * nt + col;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sb[nt][kb] = load_bf16x8(a.s_b + o * D + 32 * grp + 8 * kb);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 u[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const int row = 16 * mt + col;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float* src = s_tile + row * XS_F32 + 32 * grp + 8 * kb;
        float v[8];
        *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(src);
        *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(src + 4);
        bf16x8 rh, rm, rl;
        split3_bf16(v, rh, rm, rl);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          u[nt] = mfma_bf16(rh, sb[nt][kb], u[nt]);
          u[nt] = mfma_bf16(rm, sb[nt][kb], u[nt]);
          u[nt] = mfma_bf16(rl, sb[nt][kb], u[nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int orow = 16 * mt + 4 * grp + i;
          s_sgn[orow * IDX_STRIDE + 32 * wave + 16 * nt + col] = u[nt][i] >= 0.f ? 1 : 0;
        }
    }
    __syncthreads();
  }

  // ---- pack and store ------------------------------------------------------------------------
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const int nblk = a.T_cap / 64;
  {
    const int Lc = tid >> 2, part = tid & 3;
    const int c = Lc & 15, g = Lc >> 4;
    if constexpr (KEY) {
      const int row = 16 * part + c;  // part is the tile t of the chunk
      const int slot = p0 + row;
      if (slot >= lo_slot && slot < hi_slot) {
        if constexpr (BITS > 0) {
          uint8_t cv[32];
          *reinterpret_cast<u32x4*>(cv) = *reinterpret_cast<const u32x4*>(s_idx + row * IDX_STRIDE + 32 * g);
          *reinterpret_cast<u32x4*>(cv + 16) =
              *reinterpret_cast<const u32x4*>(s_idx + row * IDX_STRIDE + 32 * g + 16);
          uint32_t w[BITS];
          pack32<BITS>(cv, w);
          uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) + Lc * 16 * BITS +
                                                      part * 4 * BITS);
#pragma unroll
          for (int i = 0; i < BITS; ++i) dst[i] = w[i];
        }
        if constexpr (QJL) {
          uint8_t sv[32];
          *reinterpret_cast<u32x4*>(sv) = *reinterpret_cast<const u32x4*>(s_sgn + row * IDX_STRIDE + 32 * g);
          *reinterpret_cast<u32x4*>(sv + 16) =
              *reinterpret_cast<const u32x4*>(s_sgn + row * IDX_STRIDE + 32 * g + 16);
          uint32_t w[1];
          pack32<1>(sv, w);
          *reinterpret_cast<uint32_t*>(a.signs + (bh * nblk + blk) * 1024 + Lc * 16 + part * 4) = w[0];
        }
      }
    } else {
      // value chunk Lc, fields 8 part .. 8 part + 7; field f = 4 mt + t holds tokens
      // 16 t + 4 g + r (r = 0..3) of coordinate 16 mt + c.
      uint32_t w[BITS], m[BITS];
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = m[i] = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int f = 8 * part + k;
        const int mt = f >> 2, t = f & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + 4 * g + r;
          const int slot = p0 + row;
          const uint32_t v = s_idx[row * IDX_STRIDE + 16 * mt + c];
          const uint32_t mk = (slot >= lo_slot && slot < hi_slot) ? ((1u << BITS) - 1u) : 0u;
          const int bit = 4 * BITS * k + BITS * r;
          const int word = bit >> 5, off = bit & 31;
          w[word] |= (v & mk) << off;
          m[word] |= mk << off;
          if (off + BITS > 32) {
            w[word + 1] |= (v & mk) >> (32 - off);
            m[word + 1] |= mk >> (32 - off);
          }
        }
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) + Lc * 16 * BITS +
                                                  part * 4 * BITS);
#pragma unroll
      for (int i = 0; i < BITS; ++i) {
        if (m[i] == 0xFFFFFFFFu) {
          dst[i] = w[i];
        } else if (m[i] != 0u) {
          dst[i] = (dst[i] & ~m[i]) | w[i];
        }
      }
    }
  }
  if (tid < 64) {
    const int slot = p0 + tid;
    if (slot >= lo_slot && slot < hi_slot) {
      a.norm[bh * a.T_cap + slot] = s_norm[tid];
      if constexpr (KEY && QJL && BITS > 0) a.rnorm[bh * a.T_cap + slot] = s_rnorm[tid];
    }
  }
}

template <bool KEY, int BITS, bool QJL>
hipError_t launch_quantize(const QuantArgs& a, bool f32, int B, hipStream_t s) {
  const dim3 grid((a.n_new + 63) / 64 + 1, a.Hkv, B);
  if (f32)
    hipLaunchKernelGGL((quantize_kernel<KEY, BITS, QJL, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<KEY, BITS, QJL, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t dispatch_keys(const QuantArgs& a, int bits, bool qjl, bool f32, int B, hipStream_t s) {
  if (qjl) {
    switch (bits) {
      case 0: return launch_quantize<true, 0, true>(a, f32, B, s);
      case 1: return launch_quantize<true, 1, true>(a, f32, B, s);
      case 2: return launch_quantize<true, 2, true>(a, f32, B, s);
      case 3: return launch_quantize<true, 3, true>(a, f32, B, s);
      case 4: return launch_quantize<true, 4, true>(a, f32, B, s);
    }
  } else {
    switch (bits) {
      case 1: return launch_quantize<true, 1, false>(a, f32, B, s);
      case 2: return launch_quantize<true, 2, false>(a, f32, B, s);
      case 3: return launch_quantize<true, 3, false>(a, f32, B, s);
      case 4: return launch_quantize<true, 4, false>(a, f32, B, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch_values(const QuantArgs& a, int bits, bool f32, int B, hipStream_t s) {
  switch (bits) {
    case 1: return launch_quantize<false, 1, false>(a, f32, B, s);
    case 2: return launch_quantize<false, 2, false>(a, f32, B, s);
    case 3: return launch_quantize<false, 3, false>(a, f32, B, s);
    case 4: return launch_quantize<false, 4, false>(a, f32, B, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tq

extern "C" int tq_quantize_kv(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v,
                              tq_dtype in_dtype, int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, const int32_t* start_pos, const tq_kv_cache* cache,
                              void* hip_stream) {
  using namespace tq;
  clear_error();
  if (cb == nullptr || p == nullptr || cache == nullptr || start_pos == nullptr)
    return fail(TQ_ERR_INVALID, "cb, p, cache and start_pos must not be NULL");
  int rc = check_config(cb->cfg);
  if (rc != TQ_OK) return rc;
  rc = check_cache(cb->cfg, *cache);
  if (rc != TQ_OK) return rc;
  if (k == nullptr && v == nullptr) return fail(TQ_ERR_INVALID, "k and v are both NULL");
  if (B != cache->B || Hkv != cache->Hkv) return fail(TQ_ERR_INVALID, "B/Hkv do not match the cache");
  if (n_new < 1) return fail(TQ_ERR_INVALID, "n_new must be >= 1");
  if (in_dtype != TQ_DTYPE_BF16 && in_dtype != TQ_DTYPE_F32) return fail(TQ_ERR_UNSUPPORTED, "input dtype");
  const int esz = in_dtype == TQ_DTYPE_F32 ? 4 : 2;
  if (stride_b < 0 || stride_h < 0 || stride_t < 0 || (stride_t < D && n_new > 1))
    return fail(TQ_ERR_INVALID, "strides must be >= 0 and rows of 128 elements must not overlap");
  if (((stride_b * esz) % 16) || ((stride_h * esz) % 16) || ((stride_t * esz) % 16))
    return fail(TQ_ERR_INVALID, "strides must be multiples of 16 bytes");
  if ((k && !aligned(k, 16)) || (v && !aligned(v, 16))) return fail(TQ_ERR_INVALID, "inputs must be 16-byte aligned");
  if (p->r_hi == nullptr || p->r_lo == nullptr || !aligned(p->r_hi, 16) || !aligned(p->r_lo, 16))
    return fail(TQ_ERR_INVALID, "rotation matrices missing or not 16-byte aligned");
  if (cb->cfg.k_qjl && k && (p->s_qjl == nullptr || !aligned(p->s_qjl, 16)))
    return fail(TQ_ERR_INVALID, "sketch matrix missing or not 16-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool f32 = in_dtype == TQ_DTYPE_F32;
  QuantArgs a{};
  a.sb = stride_b;
  a.sh = stride_h;
  a.st = stride_t;
  a.start_pos = start_pos;
  a.n_new = n_new;
  a.Hkv = Hkv;
  a.T_cap = cache->T_cap;
  a.r_hi = p->r_hi;
  a.r_lo = p->r_lo;
  const ProfileEvents& pe = profile_events();
  const bool prof = pe.quant_start && pe.quant_stop;
  if (prof) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(pe.quant_start), s);
  if (k) {
    QuantArgs ak = a;
    ak.x = k;
    ak.s_b = p->s_qjl;
    ak.codes = cache->k_codes;
    ak.signs = cache->k_signs;
    ak.norm = cache->k_norm;
    ak.rnorm = cache->k_rnorm;
    for (int l = 0; l < 16; ++l) {
      ak.centroids[l] = cb->k_centroids[l];
      ak.thresholds[l] = cb->k_thresholds[l];
    }
    hipError_t e = dispatch_keys(ak, cb->cfg.k_bits, cb->cfg.k_qjl != 0, f32, B, s);
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("key quantize launch: ") + hipGetErrorString(e));
  }
  if (v) {
    QuantArgs av = a;
    av.x = v;
    av.codes = cache->v_codes;
    av.norm = cache->v_norm;
    for (int l = 0; l < 16; ++l) {
      av.centroids[l] = cb->v_centroids[l];
      av.thresholds[l] = cb->v_thresholds[l];
    }
    hipError_t e = dispatch_values(av, cb->cfg.v_bits, f32, B, s);
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("value quantize launch: ") + hipGetErrorString(e));
  }
  if (prof) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(pe.quant_stop), s);
  return TQ_OK;
}
