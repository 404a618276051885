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
// Work is split in tiles: one tile is the part of one 64-token block of one (batch row,
// kv-head, tensor) that the call writes, so each block has a single writer.  Keys and
// values go through one launch; persistent workgroups (4 waves) keep the rotation and
// sketch operands in registers and walk the tiles.  Wave w computes output coordinates
// 32w..32w+31 of the tile's tokens with 16x16x32 MFMAs (16-token sub-tiles that hold no token
// of the call are skipped):
//   * rotation: bf16 inputs are exact, R_eff = R_hi + R_lo takes two passes (fp32 inputs
//     are split into three exact bf16 terms first), all products exact, fp32 accumulation;
//   * sketch: 2^10 r (fp32) is split into two f16 terms (2^-21 relative per entry) against
//     2^4 S_b in f16 (exact), fp32 accumulation; the result differs from 2^14 S_b r by at most
//     2^-21 ||S_b row|| ||2^10 r||, below the band within which the sign of u is left open;
//   * codes: up to 4 bits from the thresholds held in registers (a compare chain, or a
//     binary search at 3 bits); 5..8-bit key codes by a binary search over the thresholds
//     staged in LDS, one compare per code bit.
// Each key code width is instantiated in a translation unit of its own (tq_quantize_k*.hip).
// The k dimension of every MFMA maps lane group g, element e of k-block kb to coordinate
// 32 g + 8 kb + e on both operands, so the sum runs over all 128 coordinates.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_quantize_kernels.h"

namespace tq {
namespace {

hipError_t dispatch(const QuantLaunch& q, const tq_codebook& cb, bool f32, const QuantGrid& g, hipStream_t s,
                    hipEvent_t e0, hipEvent_t e1) {
  switch (cb.cfg.k_bits) {
    case 0: return qk::dispatch_q0(q, cb, f32, g, s, e0, e1);
    case 1: return qk::dispatch_q1(q, cb, f32, g, s, e0, e1);
    case 2: return qk::dispatch_q2(q, cb, f32, g, s, e0, e1);
    case 3: return qk::dispatch_q3(q, cb, f32, g, s, e0, e1);
    case 4: return qk::dispatch_q4(q, cb, f32, g, s, e0, e1);
    case 5: return qk::dispatch_q5(q, cb, f32, g, s, e0, e1);
    case 6: return qk::dispatch_q6(q, cb, f32, g, s, e0, e1);
    case 7: return qk::dispatch_q7(q, cb, f32, g, s, e0, e1);
    case 8: return qk::dispatch_q8(q, cb, f32, g, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tq

namespace tq {

int quantize_args(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v, tq_dtype in_dtype,
                  int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                  const int32_t* start_pos, const tq_kv_cache* cache, QuantArgs* ka, QuantArgs* va) {
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
  a.one_pass = cb->cfg.rotation == TQ_ROTATION_HADAMARD ? 1 : 0;
  a.zscale = a.one_pass ? 1.0f : SQRT_D;
  *ka = a;
  ka->x = k;
  ka->s_b = p->s_qjl;
  ka->codes = cache->k_codes;
  ka->signs = cache->k_signs;
  ka->norm = cache->k_norm;
  ka->rnorm = cache->k_rnorm;
  *va = a;
  va->x = v;
  va->codes = cache->v_codes;
  va->norm = cache->v_norm;
  for (int l = 0; l < 16; ++l) {
    ka->centroids[l] = cb->k_centroids[l];
    ka->thresholds[l] = cb->k_thresholds[l];
    va->centroids[l] = cb->v_centroids[l];
    va->thresholds[l] = cb->v_thresholds[l];
  }
  return TQ_OK;
}

int quantize_launch(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v, tq_dtype in_dtype,
                    int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    const int32_t* start_pos, const tq_kv_cache* cache, void* hip_stream,
                    const QueryRotationArgs* rot) {
  QuantLaunch q{};
  const int rc = quantize_args(cb, p, k, v, in_dtype, B, Hkv, n_new, stride_b, stride_h, stride_t, start_pos,
                               cache, &q.k, &q.v);
  if (rc != TQ_OK) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool f32 = in_dtype == TQ_DTYPE_F32;
  q.has_k = k != nullptr;
  q.has_v = v != nullptr;
  q.Hkv = Hkv;
  q.nblk_max = (n_new + 126) / 64;  // blocks a run of n_new slots can touch
  const int64_t tiles = 2ll * B * Hkv * q.nblk_max;
  if (tiles > (1ll << 30)) return fail(TQ_ERR_INVALID, "too many tokens in one call");
  q.n_tiles = static_cast<int>(tiles);
  // two workgroups per CU are resident (register budget); a larger persistent grid only adds a
  // late-starting tail
  int grid = static_cast<int>(std::min<int64_t>(tiles, 2ll * device_cu_count()));
  // an odd stride lets every workgroup alternate key and value tiles (tiles alternate K, V),
  // so no workgroup is left with only the costlier key tiles
  if (grid < tiles && grid % 2 == 0) --grid;
  const ProfileEvents& pe = profile_events();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (pe.quant_start && pe.quant_stop) {
    e0 = reinterpret_cast<hipEvent_t>(pe.quant_start);
    e1 = reinterpret_cast<hipEvent_t>(pe.quant_stop);
  }
  PrologueArgs pa{};
  QuantGrid qg{grid, nullptr, 0};
  if (rot != nullptr) {
    pa = PrologueArgs{rot->q,    rot->r_hi, rot->r_lo, rot->m_hi,         rot->m_lo, rot->qrec,
                      rot->G,    rot->q_f32, rot->cnt,  rot->cnt_per_unit, q.k.one_pass};
    qg.pa = &pa;
    qg.rot_wgs = rot->units;
  }
  hipError_t e = dispatch(q, *cb, f32, qg, s, e0, e1);
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("quantize launch: ") + hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace tq

extern "C" int tq_quantize_kv(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v,
                              tq_dtype in_dtype, int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h,
                              int64_t stride_t, const int32_t* start_pos, const tq_kv_cache* cache,
                              void* hip_stream) {
  tq::clear_error();
  return tq::quantize_launch(cb, p, k, v, in_dtype, B, Hkv, n_new, stride_b, stride_h, stride_t, start_pos, cache,
                             hip_stream, nullptr);
}
