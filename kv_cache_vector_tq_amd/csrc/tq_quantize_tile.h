// Quantize-on-write of one tile (the part of a 64-token block that a call writes) for gfx950:
// device code shared by the quantize launches and the decode-attention launch that appends
// the step's new token (tq_decode_step).  What is computed is described in tq_quantize.hip.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

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
  // rotation: one_pass = 0: R_eff = r_hi + r_lo (two bf16 passes), z = sqrt(d) R_eff x / n;
  // one_pass = 1 (Hadamard): r_hi = H diag(s) (+-1), R_eff = r_hi / sqrt(d), so z = r_hi x / n
  // (one pass).  zscale = sqrt(d) or 1: z = zscale * acc / n.
  int one_pass;
  float zscale;
};

// One quantize launch: keys and values of the same call.
struct QuantLaunch {
  QuantArgs k, v;
  int has_k, has_v;
  int Hkv, nblk_max, n_tiles;
};

// A tile the call writes: tokens [lo_slot, hi_slot) of block blk of (b, h), tensor 0 = keys.
struct TileRef {
  int tensor, b, h, start, blk, lo_slot, hi_slot;
};

// A tile's input rows, loaded one tile ahead: each thread's 32 input elements of row
// tid / 4, as 16-byte words.
template <bool F32>
struct TileIn {
  static constexpr int NW = F32 ? 8 : 4;
  u32x4 w[NW];
};

// Whether value tile r leaves other tokens of its block to other calls.
__device__ __forceinline__ bool partial_tile(const TileRef& r) {
  return r.lo_slot > r.blk * 64 || r.hi_slot < r.blk * 64 + 64;
}

namespace {


constexpr int XS_BF16 = 136;  // LDS row stride (bf16 elements) of the input tile
constexpr int XS_F32 = 132;   // LDS row stride (floats) of the fp32 input / residual tile
constexpr int IDX_STRIDE = 144;  // LDS row stride (bytes) of the code / sign tiles
constexpr int PLANE = 64 * XS_BF16;  // bf16 elements of one residual plane (hi, mid or lo)


// Workgroup barrier ordering LDS accesses only: global loads and stores in flight (the next
// tile's inputs, the last tile's outputs) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

struct Smem {
  // input tile; later the fp32 residuals (times 2^10), then their two f16 terms as planes
  float tile[3 * PLANE / 2];
  uint8_t idx[64 * IDX_STRIDE];
  uint8_t sgn[64 * IDX_STRIDE];
  float norm[64];
  float rnorm[64];
  float zs[64];  // zscale / norm (0 for a zero row)
};

// Rotation (hi, lo) and sketch operands of one wave: lane (col, grp) holds row
// 32 wave + 16 nt + col, columns 32 grp + 8 kb .. + 7.  The sketch rows are held as f16 values of
// 2^4 S_b (exact: S_b is bf16, and the factor lifts its small entries into f16's normal range).
struct Operands {
  bf16x8 rh[2][4], rl[2][4];
  f16x8 sb[2][4];
};

// Residual scale: the sketch takes 2^10 r, whose entries lie in f16's normal range down to
// |r| = 2^-24 (the signs of the sketch are those of S_b r).
constexpr float RSCALE = 1024.0f;

// Issues the loads of tile r's input rows.  Rows outside [lo_slot, hi_slot) read a clamped
// (written) row and are masked by the consumer.
template <bool F32>
__device__ __forceinline__ void load_rows(const QuantLaunch& q, const TileRef& r, int tid, TileIn<F32>& in) {
  const int row = tid >> 2, qq = tid & 3;
  const int srow = min(max(r.blk * 64 + row, r.lo_slot), r.hi_slot - 1);
  const void* x = r.tensor == 0 ? q.k.x : q.v.x;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(x) +
                       ((int64_t)r.b * q.k.sb + (int64_t)r.h * q.k.sh + (int64_t)(srow - r.start) * q.k.st + 32 * qq) *
                           (F32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < TileIn<F32>::NW; ++i) in.w[i] = *reinterpret_cast<const u32x4*>(src + 16 * i);
}

// The VB value-code words of a block that thread tid packs and stores: lanemap = 0 (one-token
// calls, packed from LDS): words VB (tid & 3) .. of chunk tid >> 2; lanemap = 1 (packed in the
// rotation's register layout): words VB wave .. of chunk lane, wave = tid >> 6, lane = tid & 63.
template <int VB>
__device__ __forceinline__ int value_word_offset(int tid, bool lanemap) {
  return lanemap ? (tid & 63) * 16 * VB + (tid >> 6) * 4 * VB : (tid >> 2) * 16 * VB + (tid & 3) * 4 * VB;
}

// For a value tile that does not cover its whole block: the value-code words it rewrites
// (4 tokens share a field, 8 fields a thread's words); zero otherwise.  VB: value code bits of
// the launch.
template <int VB>
__device__ __forceinline__ void load_prev(const QuantLaunch& q, const TileRef& r, int tid, bool lanemap,
                                          uint32_t* prev) {
#pragma unroll
  for (int i = 0; i < 4; ++i) prev[i] = 0u;
  if (r.tensor == 1 && partial_tile(r)) {  // uniform
    const int64_t bh = (int64_t)r.b * q.Hkv + r.h;
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(q.v.codes + (bh * (q.v.T_cap / 64) + r.blk) * (1024 * VB) +
                                                           value_word_offset<VB>(tid, lanemap));
#pragma unroll
    for (int i = 0; i < VB; ++i) prev[i] = pw[i];
  }
}

// First step of every tile, keys and values alike: the tile's input rows (from `in`) go to
// LDS, and each row's norm n and sqrt(d) / n are computed.  Rows outside [lo_slot, hi_slot)
// are zero.
template <bool F32>
__device__ __forceinline__ void load_rows_norms(Smem& sm, const TileRef& tr, const TileIn<F32>& in, int tid,
                                                float zscale) {
  const int p0 = tr.blk * 64, lo_slot = tr.lo_slot, hi_slot = tr.hi_slot;
  float* s_tile = sm.tile;
  float* s_norm = sm.norm;
  // The sum of squares is taken directly in fp32 and kept when it lies in [2^-60, 2^120] for
  // every row of the wave: then no square overflowed, the squares lost below fp32's range sum to
  // less than 2^-61 of it, and the rounding is that of the exactly rescaled sum.  Otherwise (a
  // zero row, extreme magnitudes) the norm is taken after an exact power-of-two rescaling by
  // the row's largest magnitude, so that squares neither overflow nor underflow fp32 over the
  // whole bf16 / fp32 range.
  {
    const int row = tid >> 2, q = tid & 3;
    const int slot = p0 + row;
    const bool valid = slot >= lo_slot && slot < hi_slot;
    constexpr int NW = TileIn<F32>::NW;  // 16-byte words of this thread's 32 elements
    u32x4 w[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = valid ? in.w[i] : u32x4{0u, 0u, 0u, 0u};

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
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) ss = fmaf(v[e], v[e], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    const bool exact = !__all(!valid || (ss >= 0x1p-60f && ss <= 0x1p120f));  // uniform
    float mx = 0.f;
    int ex = 0;
    if (exact) {
#pragma unroll
      for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(v[e]));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      if (mx > 0.f) frexpf(mx, &ex);
      // mx * 2^-ex lies in [0.5, 1); ldexp scales exactly over the whole fp32 range
      ss = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const float t = ldexpf(v[e], -ex);
        ss = fmaf(t, t, ss);
      }
      ss += __shfl_xor(ss, 1);
      ss += __shfl_xor(ss, 2);
    }
    if (q == 0) {
      const float n = !exact ? sqrtf(ss) : (mx > 0.f ? ldexpf(sqrtf(ss), ex) : 0.f);
      s_norm[row] = n;
      sm.zs[row] = n > 0.f ? zscale / n : 0.f;
    }
  }
}

// Quantizes the tokens of block blk of (b, h) that fall in [lo_slot, hi_slot).
// KEY: key layout (and sketch when QJL); otherwise value layout.  BITS = 0 only for keys
// that keep only the sketch.  F32: input elements are fp32 (else bf16).
// The input rows and norms are in LDS already (load_rows_norms); prev holds the value words
// a partial value tile rewrites (load_prev).  one: the tile's single token was loaded and is
// computed as row 0 (a one-token call); only the stores use its slot.
// wtab (5..8-bit keys only): the key table in LDS, 2^BITS levels then the thresholds.
// FULL: the call writes the whole block (lo_slot = 64 blk, hi_slot = lo_slot + 64, not a
// one-token call), so every sub-tile is active and no slot is masked: the bulk fill's tiles take
// this instance, whose sub-tile loops have no branches for the compiler to schedule around.
template <bool KEY, int BITS, bool QJL, bool F32, bool FULL = false>
__device__ __forceinline__ void quantize_tile(const QuantArgs& a, Smem& sm, const Operands& op, const TileRef& tr,
                                              const uint32_t* prev, int tid, bool one_call, const float* wtab) {
  const int b = tr.b, h = tr.h, blk = tr.blk;
  const int lo_slot = FULL ? 64 * blk : tr.lo_slot, hi_slot = FULL ? 64 * blk + 64 : tr.hi_slot;
  const bool one = !FULL && one_call;
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
  const int r0 = one ? 0 : lo_slot - p0, r1 = one ? 1 : hi_slot - p0;
  bool mt_on[4];
  int n_on = 0;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    mt_on[mt] = (16 * mt < r1) && (16 * mt + 16 > r0);
    n_on += mt_on[mt] ? 1 : 0;
  }
  const int64_t bh = (int64_t)b * a.Hkv + h;
  const int nblk = a.T_cap / 64;
  const bool partial = !FULL && partial_tile(tr);  // uniform over the workgroup


  // ---- rotation: acc[mt][nt] = X[16 mt.., :] R[32 wave + 16 nt.., :]^T, R = r_hi + r_lo, or
  // r_hi alone in one-pass mode -----------------------------------------------------------------
  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto rotate = [&](auto one_) {
    constexpr bool ONE = decltype(one_)::value;
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
            if constexpr (!ONE) acc[mt][nt] = mfma_bf16(xh, rl[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xm, rh[nt][kb], acc[mt][nt]);
            if constexpr (!ONE) acc[mt][nt] = mfma_bf16(xm, rl[nt][kb], acc[mt][nt]);
            acc[mt][nt] = mfma_bf16(xl, rh[nt][kb], acc[mt][nt]);
            if constexpr (!ONE) acc[mt][nt] = mfma_bf16(xl, rl[nt][kb], acc[mt][nt]);
          }
        } else {
          const bf16x8 xv =
              load_bf16x8(reinterpret_cast<const uint16_t*>(s_tile) + row * XS_BF16 + 32 * grp + 8 * kb);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            acc[mt][nt] = mfma_bf16(xv, rh[nt][kb], acc[mt][nt]);
            if constexpr (!ONE) acc[mt][nt] = mfma_bf16(xv, rl[nt][kb], acc[mt][nt]);
          }
        }
      }
    }
  };
  // The MFMA phases (rotation, sketch) run at raised issue priority: with two waves per SIMD the
  // matrix core is fed while the other wave's code search fills the gaps.
  __builtin_amdgcn_s_setprio(1);
  if (a.one_pass)  // uniform
    rotate(std::true_type{});
  else
    rotate(std::false_type{});
  __builtin_amdgcn_s_setprio(0);
  lds_barrier();  // the input tile is dead from here on; its space holds residuals

  // ---- scale, scalar code, residual (sub-tiles without a token of the call are skipped; the
  // pack below masks their rows) -----------------------------------------------------------
  // The codebook as wave-uniform register values (readfirstlane), so that the compare chain
  // selects values rather than addresses of the argument block.
  constexpr int LR = BITS <= 4 ? L : 1;  // wide tables stay in LDS
  // Keys with the sketch and codes of 1..4 bits select 2^10 c / sqrt(d) instead of c: the scaled
  // residual is then one fma.  (Wide codes keep z - c, exact where z is near c: their residuals
  // are short enough that rounding c / sqrt(d) first would show in the residual norm.)
  constexpr float CSCALE = (KEY && QJL && BITS <= 4) ? RSCALE * INV_SQRT_D : 1.0f;
  float cent[LR], thr[LR];
#pragma unroll
  for (int l = 0; l < LR; ++l) {
    cent[l] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.centroids[l]))) * CSCALE;
    thr[l] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(a.thresholds[l])));
  }
  // Values of a multi-token call: lane (col, grp) of wave w holds rows 16 mt + 4 grp + i of output
  // coordinate 32 w + 16 nt + col, which are exactly the 4 codes of value field 4 (2 w + nt) + mt
  // of chunk col + 16 grp.  Its 8 fields (nt, mt) are that chunk's words VB w .. VB w + VB - 1,
  // so the codes are packed in registers: field (nt, mt) at bit 4 VB (4 nt + mt), code i at
  // + VB i.  (4-bit values keep the LDS path below: packing them in registers beside the 15-step
  // code search spilled registers and made the c5 turbo4 bulk quantize 1.6x slower.  The words
  // a partial tile rewrites are loaded with the matching ownership: load_prev's lanemap.)
  constexpr bool VPACK = !KEY && BITS > 0 && BITS <= 3;
  const bool lanepack = VPACK && !one;  // uniform
  uint32_t vw[VPACK ? BITS : 1];
#pragma unroll
  for (int k = 0; k < (VPACK ? BITS : 1); ++k) vw[k] = 0u;
  auto put_code = [&](int row, int o, int idx, int mt, int nt, int i) {
    if constexpr (VPACK) {
      if (lanepack) {
        const int bit = 4 * BITS * (4 * nt + mt) + BITS * i;  // compile-time after unrolling
        const int word = bit >> 5, off = bit & 31;
        vw[word] |= static_cast<uint32_t>(idx) << off;
        if (off + BITS > 32) vw[word + 1] |= static_cast<uint32_t>(idx) >> (32 - off);
        return;
      }
    }
    s_idx[row * IDX_STRIDE + o] = static_cast<uint8_t>(idx);
  };
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
        if constexpr (BITS == 3 && !(KEY && QJL)) {
          // only the code is needed: binary search over the sorted thresholds (the count of
          // thresholds <= z, as the linear scan below), one compare per code bit.  (For 4-bit
          // codes the select tree of the last step measured slower than the scan.)
          const bool b0 = z >= thr[3];
          const bool b1 = z >= (b0 ? thr[5] : thr[1]);
          const float t2 = b0 ? (b1 ? thr[6] : thr[4]) : (b1 ? thr[2] : thr[0]);
          const int idx = (b0 ? 4 : 0) | (b1 ? 2 : 0) | (z >= t2 ? 1 : 0);
          put_code(row, o, idx, mt, nt, i);
        } else if constexpr (BITS > 4) {
          // binary search over the 2^BITS - 1 sorted thresholds in LDS: after the step of
          // width w, the thresholds below idx are exactly those <= z among the ones seen
          const float* wthr = wtab + L;
          int idx = 0;
#pragma unroll
          for (int w = L / 2; w >= 1; w >>= 1) idx += z >= wthr[idx + w - 1] ? w : 0;
          if constexpr (KEY && QJL) c = wtab[idx];
          s_idx[row * IDX_STRIDE + o] = static_cast<uint8_t>(idx);
        } else if constexpr (BITS > 0) {
          int idx = 0;
          c = cent[0];
#pragma unroll
          for (int l = 1; l < L; ++l) {
            const bool ge = z >= thr[l - 1];
            idx = ge ? l : idx;
            c = ge ? cent[l] : c;
          }
          put_code(row, o, idx, mt, nt, i);
        }
        if constexpr (KEY && QJL) {
          // 2^10 r with r = y - c / sqrt(d) = z / sqrt(d) - c / sqrt(d) (c holding 2^10 c / sqrt(d)
          // for 1..4-bit codes), or (z - c) / sqrt(d) for wide codes.  A zero row keeps this
          // (nonzero) residual: its residual norm and sign word are set to 0 and all ones at the end.
          constexpr float RS = RSCALE * INV_SQRT_D;
          const float r = BITS == 0 ? z * RS : (BITS <= 4 ? fmaf(z, RS, -c) : (z - c) * RS);
          s_tile[row * XS_F32 + o] = r;
        }
      }
    }
  }
  lds_barrier();

  uint32_t sword = 0u;  // keys with the sketch: this lane's sign word (see the sketch below)
  if constexpr (KEY && QJL) {
    // ---- residual norms; with more than one active sub-tile, 2^10 r is split once into its two
    // f16 terms (planes), else each wave splits the sub-tile's rows itself -----------------------
    const bool planes = n_on > 1;  // uniform
    {
      const int row = tid >> 2, q = tid & 3;
      const float* src = s_tile + row * XS_F32 + 32 * q;
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; j += 4) *reinterpret_cast<f32x4*>(v + j) = *reinterpret_cast<const f32x4*>(src + j);
      if constexpr (BITS > 0) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < 32; j += 4) ss = fmaf(v[j], v[j], fmaf(v[j + 1], v[j + 1], fmaf(v[j + 2], v[j + 2], fmaf(v[j + 3], v[j + 3], ss))));
        ss += __shfl_xor(ss, 1);
        ss += __shfl_xor(ss, 2);
        if (q == 0) s_rnorm[row] = s_norm[row] > 0.f ? sqrtf(ss) * (1.0f / RSCALE) : 0.f;
      }
      if (planes) {
        f16x8 ph[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) split2_f16(v + 8 * i, ph[i], pl[i]);
        lds_barrier();  // every residual is read before the planes overwrite the tile
        f16x8* dst = reinterpret_cast<f16x8*>(reinterpret_cast<uint16_t*>(s_tile) + row * XS_BF16 + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[i] = ph[i];
          dst[i + PLANE / 8] = pl[i];
        }
        lds_barrier();
      }
    }
    // ---- sketch: u = (2^4 S_b)(2^10 r), signs ------------------------------------------------
    // Each product takes the two f16 terms of 2^10 r against the exact f16 2^4 S_b (fp32 sums).
    // The terms hold 2^10 r to 2^-21 relative per entry, so u differs from 2^14 S_b r by at most
    // 2^-21 ||S_b row|| ||2^10 r|| (about 7e-6 of 2^14 ||r|| for a row of 128 Gaussian entries):
    // less than the 1e-5 ||r|| from 0 within which a sign is left undecided.
    // Lane (col, grp) of wave w holds u of sketch rows 32 w + 16 nt + col for the rows (tokens)
    // 16 mt + 4 grp + i, so two wave ballots of u >= 0 per (mt, i), one per nt, hold the 32-bit
    // sign words (chunk rows 32 w .. 32 w + 31) of the four tokens 16 mt + 4 grp + i, grp = 0..3,
    // in their 16-bit slices.  Lane (col, grp) keeps the word of token 16 (col / 4) + 4 grp +
    // col % 4 and stores it below.
    const auto& sb = op.sb;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (!mt_on[mt]) continue;
      f32x4 u[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const int row = 16 * mt + col;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        f16x8 rh, rl;
        if (planes) {
          const uint16_t* src = reinterpret_cast<const uint16_t*>(s_tile) + row * XS_BF16 + 32 * grp + 8 * kb;
          rh = *reinterpret_cast<const f16x8*>(src);
          rl = *reinterpret_cast<const f16x8*>(src + PLANE);
        } else {
          const float* src = s_tile + row * XS_F32 + 32 * grp + 8 * kb;
          float v[8];
          *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(src);
          *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(src + 4);
          split2_f16(v, rh, rl);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          u[nt] = mfma_f16(rh, sb[nt][kb], u[nt]);
          u[nt] = mfma_f16(rl, sb[nt][kb], u[nt]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint64_t b0 = __ballot(u[0][i] >= 0.f), b1 = __ballot(u[1][i] >= 0.f);
        const uint32_t w = (static_cast<uint32_t>(b0 >> (16 * grp)) & 0xFFFFu) |
                           (static_cast<uint32_t>(b1 >> (16 * grp)) << 16);
        sword = col == 4 * mt + i ? w : sword;
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- pack and store ------------------------------------------------------------------------
  {
    const int Lc = tid >> 2, part = tid & 3;
    const int c = Lc & 15, g = Lc >> 4;
    if constexpr (KEY) {
      const int row = 16 * part + c;  // part is the tile t of the chunk
      const int slot = p0 + row;
      if (slot >= lo_slot && slot < hi_slot) {
        const int sr = one ? 0 : row;  // LDS row that holds the token
        if constexpr (BITS > 0) {
          uint8_t cv[32];
          *reinterpret_cast<u32x4*>(cv) = *reinterpret_cast<const u32x4*>(s_idx + sr * IDX_STRIDE + 32 * g);
          *reinterpret_cast<u32x4*>(cv + 16) =
              *reinterpret_cast<const u32x4*>(s_idx + sr * IDX_STRIDE + 32 * g + 16);
          uint32_t w[BITS];
          pack32<BITS>(cv, w);
          uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) + Lc * 16 * BITS +
                                                      part * 4 * BITS);
#pragma unroll
          for (int i = 0; i < BITS; ++i) dst[i] = w[i];
        }
      }
      if constexpr (QJL) {
        // the sign word built from the ballots: token row 16 (col / 4) + 4 grp + col % 4 of this
        // wave's chunk rows (a one-token call: lane 0 holds the word of row 0, the token)
        const int rowk = one ? lo_slot - p0 : 16 * (col >> 2) + 4 * grp + (col & 3);
        const int slot_k = p0 + rowk;
        // a zero row's signs are all ones (its residual was not zeroed)
        const uint32_t sw = s_norm[one ? 0 : rowk] > 0.f ? sword : 0xFFFFFFFFu;
        if ((!one || lane == 0) && slot_k >= lo_slot && slot_k < hi_slot)
          *reinterpret_cast<uint32_t*>(a.signs + (bh * nblk + blk) * 1024 + ((rowk & 15) + 16 * wave) * 16 +
                                       (rowk >> 4) * 4) = sw;
      }
    } else if (lanepack) {
      // the words packed in registers during the code search
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) +
                                                  value_word_offset<BITS>(tid, true));
      if (!partial) {
#pragma unroll
        for (int i = 0; i < (VPACK ? BITS : 1); ++i) dst[i] = vw[i];
      } else {
        // a tile that leaves other tokens of its block to other calls: the codes of rows outside
        // [lo_slot, hi_slot) keep the words' previous bits (rows 16 mt + 4 grp + i)
        uint32_t vm[VPACK ? BITS : 1];
#pragma unroll
        for (int k = 0; k < (VPACK ? BITS : 1); ++k) vm[k] = 0u;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int slot = p0 + 16 * mt + 4 * grp + i;
              const uint32_t mk = (slot >= lo_slot && slot < hi_slot) ? ((1u << BITS) - 1u) : 0u;
              const int bit = 4 * BITS * (4 * nt + mt) + BITS * i;
              const int word = bit >> 5, off = bit & 31;
              vm[word] |= mk << off;
              if (off + BITS > 32) vm[word + 1] |= mk >> (32 - off);
            }
#pragma unroll
        for (int i = 0; i < (VPACK ? BITS : 1); ++i) {
          if (vm[i] == 0xFFFFFFFFu) {
            dst[i] = vw[i];
          } else if (vm[i] != 0u) {
            dst[i] = (prev[i] & ~vm[i]) | (vw[i] & vm[i]);
          }
        }
      }
    } else {
      // value chunk Lc, fields 8 part .. 8 part + 7; field f = 4 mt + t holds tokens
      // 16 t + 4 g + r (r = 0..3) of coordinate 16 mt + c.
      uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + (bh * nblk + blk) * (1024 * BITS) + Lc * 16 * BITS +
                                                  part * 4 * BITS);
      if (!partial) {
        // a whole block (every tile of a bulk fill): no slot masks, and every word is written,
        // so the old words are not needed (nor waited for)
        uint32_t w[BITS];
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[i] = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int f = 8 * part + k;
          const int mt = f >> 2, t = f & 3;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t v = s_idx[(16 * t + 4 * g + r) * IDX_STRIDE + 16 * mt + c];
            const int bit = 4 * BITS * k + BITS * r;
            const int word = bit >> 5, off = bit & 31;
            w[word] |= v << off;
            if (off + BITS > 32) w[word + 1] |= v >> (32 - off);
          }
        }
#pragma unroll
        for (int i = 0; i < BITS; ++i) dst[i] = w[i];
      } else {
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
            const uint32_t v = s_idx[(one ? 0 : row) * IDX_STRIDE + 16 * mt + c];
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
  }
  if (tid < 64) {
    const int slot = p0 + tid;
    if (slot >= lo_slot && slot < hi_slot) {
      a.norm[bh * a.T_cap + slot] = s_norm[one ? 0 : tid];
      if constexpr (KEY && QJL && BITS > 0) a.rnorm[bh * a.T_cap + slot] = s_rnorm[one ? 0 : tid];
    }
  }
}

// Rotation (and, with sketch, sketch) operands of thread tid (0..255) of a quantizing group.
template <bool QJL>
__device__ __forceinline__ void load_operands(Operands& op, const QuantArgs& k, bool sketch, int tid) {
  const int wave = tid >> 6, lane = tid & 63;
  // without the sketch the sketch registers read the rotation rows instead (unused): the loads
  // stay unconditional, so the compiler issues them all before the first wait
  const uint16_t* sb = sketch ? k.s_b : k.r_hi;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int o = 32 * wave + 16 * nt + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      op.rh[nt][kb] = load_bf16x8(k.r_hi + o * D + 32 * grp + 8 * kb);
      op.rl[nt][kb] = load_bf16x8(k.r_lo + o * D + 32 * grp + 8 * kb);
      if constexpr (QJL) {
        const u16x8 w = *reinterpret_cast<const u16x8*>(sb + o * D + 32 * grp + 8 * kb);
        f16x8 h;
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(__uint_as_float(static_cast<uint32_t>(w[e]) << 16) * 16.0f);
        op.sb[nt][kb] = h;
      }
    }
  }
}


}  // namespace
}  // namespace tq
