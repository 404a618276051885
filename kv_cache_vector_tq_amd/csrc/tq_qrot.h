// Query rotation of decode attention for gfx950 (device code shared by the attention
// prologue launch and the fused append + rotation launch of a decode step).
//
// Page "Google TurboQuant простыми словами", section "Как работает TurboQuant", step 2 (the
// sign sketch): the score needs q1 = R_eff q and q2 = S_b q1 of every q-head.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_common.h"

namespace tq {
namespace {

// For the G (<= 16) q-heads of a kv-head, q1 = R_eff q and q2 = S_b q1 = M q (M = S_b R_eff,
// given as the bf16 pair m_hi + m_lo) are 16x16x32 bf16 MFMA products: the q-heads are the M
// rows, a wave's 32 output coordinates the N columns.  A bf16 query is exact in one bf16 term
// and an fp32 query is split into three, so the products are exact and the sums fp32.

// Operands of one lane: rows o = 32 wave + 16 nt + col of R_hi, R_lo, M_hi, M_lo (k-slots
// 32 g + 8 kb + e) and the raw words of the query of head col at the same coordinates
// (8 x 16 bytes for fp32, the first 4 x 16 bytes for bf16).  Everything is loaded in one
// batch; the query is converted only when first used.
template <bool QJL>
struct QOperands {
  bf16x8 rh[2][4], rl[2][4], mh[QJL ? 2 : 1][4], ml[QJL ? 2 : 1][4];
  u32x4 raw[8];
  bool valid;  // the lane's column holds a query
};

// qrow: row (in units of 128 elements) of q that holds the lane's query; valid: whether the
// lane's column holds a query at all (the operand is zero otherwise).
template <bool QJL>
__device__ __forceinline__ void load_query_operands(QOperands<QJL>& o, const void* q, bool q_f32, int64_t qrow,
                                                    bool valid, const uint16_t* r_hi, const uint16_t* r_lo,
                                                    const uint16_t* m_hi, const uint16_t* m_lo, int wave, int col,
                                                    int g) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = 32 * wave + 16 * nt + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      o.rh[nt][kb] = load_bf16x8(r_hi + row * D + 32 * g + 8 * kb);
      o.rl[nt][kb] = load_bf16x8(r_lo + row * D + 32 * g + 8 * kb);
      if constexpr (QJL) {
        o.mh[nt][kb] = load_bf16x8(m_hi + row * D + 32 * g + 8 * kb);
        o.ml[nt][kb] = load_bf16x8(m_lo + row * D + 32 * g + 8 * kb);
      }
    }
  }
  // unconditional loads from clamped, in-bounds addresses (no branch that would force an
  // early wait); lanes of rows >= G and the unused chunks of a bf16 query are masked on use
  const int esz = q_f32 ? 4 : 2;
  o.valid = valid;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(q) + (qrow * D + 32 * g) * esz;
  const int last = q_f32 ? 7 : 3;  // last 16-byte chunk of this lane's 32 coordinates
#pragma unroll
  for (int i = 0; i < 8; ++i) o.raw[i] = *reinterpret_cast<const u32x4*>(base + 16 * min(i, last));
}

// Accumulates the products of one k-block for both output tiles: q1 += a (r_hi + r_lo), or
// a r_hi alone in one-pass mode (Hadamard: r_lo = 0); q2 += a (m_hi + m_lo).
template <bool QJL, bool ONE>
__device__ __forceinline__ void rotate_step(const QOperands<QJL>& o, int kb, bf16x8 a, f32x4* d1, f32x4* d2) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    d1[nt] = mfma_bf16(a, o.rh[nt][kb], d1[nt]);
    if constexpr (!ONE) d1[nt] = mfma_bf16(a, o.rl[nt][kb], d1[nt]);
    if constexpr (QJL) {
      d2[nt] = mfma_bf16(a, o.mh[nt][kb], d2[nt]);
      d2[nt] = mfma_bf16(a, o.ml[nt][kb], d2[nt]);
    }
  }
}

// d1 += q (R_hi + R_lo) (q R_hi in one-pass mode), d2 += q (M_hi + M_lo) for the lane's output
// tiles (all k-blocks).
template <bool QJL, bool ONE>
__device__ __forceinline__ void rotate_products(const QOperands<QJL>& o, bool q_f32, f32x4* d1, f32x4* d2) {
  const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  if (q_f32) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float x[8];
      const u32x4 lo = o.raw[2 * kb], hi = o.raw[2 * kb + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = o.valid ? __uint_as_float(lo[e]) : 0.f;
        x[4 + e] = o.valid ? __uint_as_float(hi[e]) : 0.f;
      }
      bf16x8 ph, pm, pl;
      split3_bf16(x, ph, pm, pl);
      rotate_step<QJL, ONE>(o, kb, ph, d1, d2);
      rotate_step<QJL, ONE>(o, kb, pm, d1, d2);
      rotate_step<QJL, ONE>(o, kb, pl, d1, d2);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      rotate_step<QJL, ONE>(o, kb, o.valid ? __builtin_bit_cast(bf16x8, o.raw[kb]) : zero, d1, d2);
  }
}

// Query records: for every q-head, q1[128] then q2[128] (fp32).  One wave computes output
// coordinates 32 tile .. 32 tile + 31 of the G q-heads of one (batch row, kv-head) unit.
constexpr int QREC = 2 * D;  // floats per record

struct PrologueArgs {
  const void* q;  // [B*Hq][128] bf16 or fp32 (q_f32)
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* m_hi;  // NULL without a sketch
  const uint16_t* m_lo;
  float* qrec;  // [B*Hq][QREC]
  int G, q_f32;
  // arrival counters of the attention kernel that follows: cnt_per_unit per (batch row,
  // kv-head) unit, set to zero here (wave 0 of each unit's rotation) before every attention
  // launch, so a workspace needs no initial contents
  unsigned* cnt;
  int cnt_per_unit;
  int one_pass;  // Hadamard mode: q1 = q r_hi (one pass; the record holds sqrt(d) R q)
};

// Output coordinates 32 tile .. 32 tile + 31 of the records of up to 16 queries (one per lane
// column: row qrow of q, `valid` as in load_query_operands); record h (q1[128] then q2[128]) at
// recs + h QREC, for h < nrec.  recs may be global or LDS memory.
template <bool QJL>
__device__ __forceinline__ void rotate_queries(const void* q, bool q_f32, int64_t qrow, bool valid, int one_pass,
                                               const uint16_t* r_hi, const uint16_t* r_lo, const uint16_t* m_hi,
                                               const uint16_t* m_lo, float* recs, int nrec, int tile, int lane) {
  const int col = lane & 15, g = lane >> 4;
  QOperands<QJL> qo;
  load_query_operands<QJL>(qo, q, q_f32, qrow, valid, r_hi, r_lo, m_hi, m_lo, tile, col, g);
  f32x4 d1[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  f32x4 d2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  if (one_pass)
    rotate_products<QJL, true>(qo, q_f32, d1, d2);
  else
    rotate_products<QJL, false>(qo, q_f32, d1, d2);
  // D layout: lane (col, g) holds query 4 g + i, output coordinate 32 tile + 16 nt + col
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    if (h >= nrec) continue;
    float* rec = recs + h * QREC;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      rec[32 * tile + 16 * nt + col] = d1[nt][i];
      rec[D + 32 * tile + 16 * nt + col] = QJL ? d2[nt][i] : 0.f;
    }
  }
}

template <bool QJL>
__device__ __forceinline__ void rotate_query_tile(const PrologueArgs& a, int unit, int tile, int lane) {
  const int col = lane & 15;
  const int G = a.G;
  const int64_t head0 = static_cast<int64_t>(unit) * G;
  if (tile == 0 && lane < a.cnt_per_unit) a.cnt[static_cast<int64_t>(unit) * a.cnt_per_unit + lane] = 0u;
  rotate_queries<QJL>(a.q, a.q_f32 != 0, head0 + (col < G ? col : 0), col < G, a.one_pass, a.r_hi, a.r_lo, a.m_hi,
                      a.m_lo, a.qrec + head0 * QREC, G, tile, lane);
}

}  // namespace
}  // namespace tq
