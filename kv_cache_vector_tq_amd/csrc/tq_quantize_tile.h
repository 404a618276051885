// Quantize-on-write of one tile (the part of a 64-token block that a call writes) for gfx950:
// device code shared by the quantize launches and the decode-attention launch that appends
// the step's new token (tq_decode_step).  What is computed is described in tq_quantize.hip.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_common.h"

namespace tq {

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

namespace {


constexpr int XS_BF16 = 136;  // LDS row stride (bf16 elements) of the input tile
constexpr int XS_F32 = 132;   // LDS row stride (floats) of the fp32 input / residual tile
constexpr int IDX_STRIDE = 144;  // LDS row stride (bytes) of the code / sign tiles


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

struct Smem {
  float tile[64 * XS_F32];  // input tile, later residuals
  uint8_t idx[64 * IDX_STRIDE];
  uint8_t sgn[64 * IDX_STRIDE];
  float norm[64];
  float rnorm[64];
  float zs[64];  // sqrt(d) / norm (0 for a zero row)
};

// Rotation (hi, lo) and sketch operands of one wave: lane (col, grp) holds row
// 32 wave + 16 nt + col, columns 32 grp + 8 kb .. + 7.
struct Operands {
  bf16x8 rh[2][4], rl[2][4], sb[2][4];
};

// Quantizes the tokens of block blk of (b, h) that fall in [lo_slot, hi_slot).
// KEY: key layout (and sketch when QJL); otherwise value layout.  BITS = 0 only for keys
// that keep only the sketch.  F32: input elements are fp32 (else bf16).
template <bool KEY, int BITS, bool QJL, bool F32>
__device__ __forceinline__ void quantize_tile(const QuantArgs& a, Smem& sm, const Operands& op, int b, int h,
                                              int start, int blk, int lo_slot, int hi_slot, int tid) {
  constexpr int L = 1 << (BITS > 0 ? BITS : 1);
  float* s_tile = sm.tile;
  uint8_t* s_idx = sm.idx;
  uint8_t* s_sgn = sm.sgn;
  float* s_norm = sm.norm;
  float* s_rnorm = sm.rnorm;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int p0 = blk * 64;
  // 16-token sub-tiles holding at least one token of the call
  const int r0 = lo_slot - p0, r1 = hi_slot - p0;
  bool mt_on[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) mt_on[mt] = (16 * mt < r1) && (16 * mt + 16 > r0);
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const int nblk = a.T_cap / 64;
  // Value words hold codes of 4 tokens: a tile that does not cover the whole block reads the
  // words it will modify now, so the read-modify-write at the end costs no extra round trip.
  const bool partial = lo_slot > p0 || hi_slot < p0 + 64;  // uniform over the workgroup
  uint32_t prev[KEY ? 1 : (BITS > 0 ? BITS : 1)];
  if constexpr (!KEY) {
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) +
                                                           (tid >> 2) * 16 * BITS + (tid & 3) * 4 * BITS);
#pragma unroll
    for (int i = 0; i < BITS; ++i) prev[i] = partial ? pw[i] : 0u;
  }

  // ---- load the tile, row norms ----------------------------------------------------------
  // The norm is taken after an exact power-of-two rescaling by the row's largest magnitude,
  // so that squares neither overflow nor underflow fp32 over the whole bf16 / fp32 range.
  {
    const int row = tid >> 2, q = tid & 3;
    const int slot = p0 + row;
    const bool valid = slot >= lo_slot && slot < hi_slot;
    // all loads first, from a clamped (always written) row, so that they are in flight together;
    // rows outside [lo_slot, hi_slot) are masked afterwards
    constexpr int NW = F32 ? 8 : 4;  // 16-byte words of this thread's 32 elements
    u32x4 w[NW];
    {
      const int srow = min(max(slot, lo_slot), hi_slot - 1);
      const uint8_t* src = reinterpret_cast<const uint8_t*>(a.x) +
                           ((int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)(srow - start) * a.st + 32 * q) *
                               (F32 ? 4 : 2);
#pragma unroll
      for (int i = 0; i < NW; ++i) w[i] = *reinterpret_cast<const u32x4*>(src + 16 * i);
#pragma unroll
      for (int i = 0; i < NW; ++i)
        if (!valid) w[i] = u32x4{0u, 0u, 0u, 0u};
    }
    float v[32];
    if constexpr (F32) {
      float* dst = s_tile + row * XS_F32 + 32 * q;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        *reinterpret_cast<u32x4*>(dst + 4 * i) = w[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = __uint_as_float(w[i][e]);
      }
    } else {
      uint16_t* dst = reinterpret_cast<uint16_t*>(s_tile) + row * XS_BF16 + 32 * q;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<u32x4*>(dst + 8 * i) = w[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * i + 2 * e] = __uint_as_float(w[i][e] << 16);
          v[8 * i + 2 * e + 1] = __uint_as_float(w[i][e] & 0xFFFF0000u);
        }
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
    if (q == 0) {
      const float n = mx > 0.f ? ldexpf(sqrtf(ss), ex) : 0.f;
      s_norm[row] = n;
      sm.zs[row] = n > 0.f ? SQRT_D / n : 0.f;
    }
  }
  __syncthreads();

  // ---- rotation: acc[mt][nt] = X[16 mt.., :] R_eff[32 wave + 16 nt.., :]^T ---------------
  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const auto& rh = op.rh;
    const auto& rl = op.rl;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (!mt_on[mt]) continue;
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

  // ---- scale, scalar code, residual (sub-tiles without a token of the call are skipped; the
  // pack below masks their rows) -----------------------------------------------------------
  // The codebook as wave-uniform register values (readfirstlane), so that the compare chain
  // selects values rather than addresses of the argument block.
  float cent[L], thr[L];
#pragma unroll
  for (int l = 0; l < L; ++l) {
    cent[l] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.centroids[l])));
    thr[l] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.thresholds[l])));
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (!mt_on[mt]) continue;
    // z = sqrt(d) y = acc sqrt(d) / n for the lane's rows 16 mt + 4 grp + i
    const f32x4 zsv = *reinterpret_cast<const f32x4*>(sm.zs + 16 * mt + 4 * grp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * mt + 4 * grp + i;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int o = 32 * wave + 16 * nt + col;
        const float z = acc[mt][nt][i] * zsv[i];
        float c = 0.f;
        if constexpr (BITS > 0) {
          int idx = 0;
          c = cent[0];
#pragma unroll
          for (int l = 1; l < L; ++l) {
            const bool ge = z >= thr[l - 1];
            idx = ge ? l : idx;
            c = ge ? cent[l] : c;
          }
          s_idx[row * IDX_STRIDE + o] = static_cast<uint8_t>(idx);
        }
        if constexpr (KEY && QJL) {
          // r = y - c / sqrt(d) = (z - c) / sqrt(d)
          float r = ((BITS > 0) ? (z - c) : z) * INV_SQRT_D;
          if (!(zsv[i] > 0.f)) r = 0.f;
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
      for (int j = 0; j < 32; j += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + j);
        ss = fmaf(v[0], v[0], fmaf(v[1], v[1], fmaf(v[2], v[2], fmaf(v[3], v[3], ss))));
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
      if (q == 0) s_rnorm[row] = s_norm[row] > 0.f ? sqrtf(ss) : 0.f;
    }
    // ---- sketch: u = S_b r, signs -----------------------------------------------------------
    const auto& sb = op.sb;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (!mt_on[mt]) continue;
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
          dst[i] = (prev[i] & ~m[i]) | w[i];
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

// Rotation (and, with sketch, sketch) operands of thread tid (0..255) of a quantizing group.
template <bool QJL>
__device__ __forceinline__ void load_operands(Operands& op, const QuantArgs& k, bool sketch, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int o = 32 * wave + 16 * nt + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      op.rh[nt][kb] = load_bf16x8(k.r_hi + o * D + 32 * grp + 8 * kb);
      op.rl[nt][kb] = load_bf16x8(k.r_lo + o * D + 32 * grp + 8 * kb);
      if constexpr (QJL) op.sb[nt][kb] = sketch ? load_bf16x8(k.s_b + o * D + 32 * grp + 8 * kb) : bf16x8{};
    }
  }
}


}  // namespace
}  // namespace tq
