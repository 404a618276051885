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
// 32w..32w+31 of the tile's tokens with 16x16x32 bf16 MFMAs (16-token sub-tiles that hold
// no token of the call are skipped):
//   * rotation: bf16 inputs are exact, R_eff = R_hi + R_lo takes two passes (fp32 inputs
//     are split into three exact bf16 terms first), all products exact, fp32 accumulation;
//   * sketch: r (fp32) is split into three exact bf16 terms, S_b is bf16, so u = S_b r is
//     the fp32-accumulated product of the fp32 residual.
// The k dimension of every MFMA maps lane group g, element e of k-block kb to coordinate
// 32 g + 8 kb + e on both operands, so the sum runs over all 128 coordinates.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_qrot.h"
#include "tq_quantize_tile.h"

namespace tq {
namespace {

// From tile t on (stride nwg), finds the next tile the call writes (index tf); false when
// there is none.  All values are uniform over the workgroup.
__device__ __forceinline__ bool find_tile(const QuantLaunch& q, int t, int nwg, int& tf, TileRef& r) {
  for (; t < q.n_tiles; t += nwg) {
    const int tensor = t & 1;
    const int rest = t >> 1;
    const int i = rest % q.nblk_max;
    const int bh = rest / q.nblk_max;
    if (tensor == 0 ? !q.has_k : !q.has_v) continue;
    // a scalar load (constant address space: start_pos does not change during the kernel), so
    // waiting for it does not wait for the vector loads in flight
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const int start = ((const_i32_ptr)(uintptr_t)q.k.start_pos)[bh / q.Hkv];
    if (start < 0) continue;
    const int end = min(start + q.k.n_new, q.k.T_cap);  // one past the last slot written
    const int blk = start / 64 + i;
    const int p0 = blk * 64;
    if (p0 >= end) continue;
    r = TileRef{tensor, bh / q.Hkv, bh % q.Hkv, start, blk, max(start, p0), min(end, p0 + 64)};
    tf = t;
    return true;
  }
  return false;
}

// Persistent workgroups walk tiles t = ((b * Hkv + h) * nblk_max + i) * 2 + tensor.  This is
// workgroup blockIdx.x of gridDim.x, or of the first nwg_fused workgroups of a fused launch.
// Each tile's inputs are loaded while the previous tile computes.
template <int KB, bool QJL, int VB, bool F32, bool FUSED>
__device__ __forceinline__ void quantize_workgroup(const QuantLaunch& q, Smem& sm, int nwg_fused) {
  const int wg = static_cast<int>(blockIdx.x);
  const int nwg = FUSED ? nwg_fused : static_cast<int>(gridDim.x);
  const int tid = threadIdx.x;
  Operands op;
  // a workgroup that only sees value tiles (tiles alternate K, V; with one tile per workgroup
  // the odd ones) does not need the sketch matrix.  The operands are requested first: they
  // are the largest loads, and their latency overlaps the search for the first tile.
  const bool sketch = QJL && q.has_k && (nwg < q.n_tiles || (wg & 1) == 0);
  load_operands<QJL>(op, q.k, sketch, tid);
  TileIn<F32> in;
  // A one-token call with a workgroup per tile (a decode step): every step up to the packing
  // works on the token as row 0 of the tile; its slot (start_pos) is needed only by the
  // stores, so its load overlaps the input loads.  start_pos is read with a vector load (the
  // index is offset by a lane count that is always 0): waiting for it then never waits for
  // LDS traffic, as waiting for a scalar load would.
  if (q.k.n_new == 1 && nwg >= q.n_tiles) {  // uniform
    if (wg >= q.n_tiles) return;
    const int tensor = wg & 1, bh = wg >> 1, b = bh / q.Hkv, h = bh % q.Hkv;  // one block per row
    if (tensor == 0 ? !q.has_k : !q.has_v) return;
    const int start_lane = q.k.start_pos[b + static_cast<int>(__builtin_amdgcn_mbcnt_lo(0u, 0u))];
    const TileRef row0{tensor, b, h, 0, 0, 0, 1};
    load_rows<F32>(q, row0, tid, in);
    load_rows_norms<F32>(sm, row0, in, tid, q.k.zscale);
    const int start = __builtin_amdgcn_readfirstlane(start_lane);
    if (start < 0 || start >= q.k.T_cap) return;  // uniform: the row is not written
    const TileRef cur{tensor, b, h, start, start / 64, start, start + 1};
    uint32_t prev[4];
    load_prev<VB>(q, cur, tid, prev);
    lds_barrier();
    if (tensor == 0)
      quantize_tile<true, KB, QJL, F32>(q.k, sm, op, cur, prev, tid, true);
    else
      quantize_tile<false, VB, false, F32>(q.v, sm, op, cur, prev, tid, true);
    return;
  }
  int t;
  TileRef cur;
  if (!find_tile(q, wg, nwg, t, cur)) return;  // uniform
  // issued after the operands, so that waiting for the first tile's rows implies them
  load_rows<F32>(q, cur, tid, in);
  for (;;) {
    int tn = 0;
    TileRef nxt;
    const bool more = find_tile(q, t + nwg, nwg, tn, nxt);
    lds_barrier();  // the previous tile is done with LDS
    load_rows_norms<F32>(sm, cur, in, tid, q.k.zscale);
    uint32_t prev[4];
    load_prev<VB>(q, cur, tid, prev);  // used at the end of the tile
    // the next tile's rows are in flight while this tile computes
    if (more) load_rows<F32>(q, nxt, tid, in);  // uniform
    lds_barrier();
    if (cur.tensor == 0)
      quantize_tile<true, KB, QJL, F32>(q.k, sm, op, cur, prev, tid, false);
    else
      quantize_tile<false, VB, false, F32>(q.v, sm, op, cur, prev, tid, false);
    if (!more) break;
    cur = nxt;
    t = tn;
  }
}

template <int KB, bool QJL, int VB, bool F32>
__global__ void __launch_bounds__(256, 2) quantize_kernel(QuantLaunch q) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  quantize_workgroup<KB, QJL, VB, F32, false>(q, sm, 0);
}

// Decode step: the first n_qwg workgroups quantize the new tokens, each further workgroup
// rotates the queries of one (batch row, kv-head) unit (wave w: output coordinates
// 32 w .. 32 w + 31), all in one launch; the two parts share no data.
template <int KB, bool QJL, int VB, bool F32>
__global__ void __launch_bounds__(256, 2) append_rotate_kernel(QuantLaunch q, PrologueArgs pa, int n_qwg) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  if (static_cast<int>(blockIdx.x) < n_qwg)
    quantize_workgroup<KB, QJL, VB, F32, true>(q, sm, n_qwg);
  else
    rotate_query_tile<QJL>(pa, static_cast<int>(blockIdx.x) - n_qwg, threadIdx.x >> 6, threadIdx.x & 63);
}

// Launch shape: grid workgroups of quantize, plus rot_wgs rotation workgroups when pa is set.
struct QuantGrid {
  int grid;
  const PrologueArgs* pa;
  int rot_wgs;
};

template <int KB, bool QJL, int VB>
hipError_t launch_quantize(const QuantLaunch& q, bool f32, const QuantGrid& g, hipStream_t s, hipEvent_t e0,
                           hipEvent_t e1) {
  const bool ext = e0 != nullptr || e1 != nullptr;
  if (g.pa != nullptr) {
    auto kern = f32 ? append_rotate_kernel<KB, QJL, VB, true> : append_rotate_kernel<KB, QJL, VB, false>;
    const dim3 grid(g.grid + g.rot_wgs);
    if (ext)
      hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, s, e0, e1, 0, q, *g.pa, g.grid);
    else
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, q, *g.pa, g.grid);
  } else {
    auto kern = f32 ? quantize_kernel<KB, QJL, VB, true> : quantize_kernel<KB, QJL, VB, false>;
    if (ext)
      hipExtLaunchKernelGGL(kern, dim3(g.grid), dim3(256), 0, s, e0, e1, 0, q);
    else
      hipLaunchKernelGGL(kern, dim3(g.grid), dim3(256), 0, s, q);
  }
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t dispatch_v(const QuantLaunch& q, int vb, bool f32, const QuantGrid& g, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
  switch (vb) {
    case 1: return launch_quantize<KB, QJL, 1>(q, f32, g, s, e0, e1);
    case 2: return launch_quantize<KB, QJL, 2>(q, f32, g, s, e0, e1);
    case 3: return launch_quantize<KB, QJL, 3>(q, f32, g, s, e0, e1);
    case 4: return launch_quantize<KB, QJL, 4>(q, f32, g, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(const QuantLaunch& q, const tq_config& c, bool f32, const QuantGrid& g, hipStream_t s,
                    hipEvent_t e0, hipEvent_t e1) {
  if (c.k_qjl) {
    switch (c.k_bits) {
      case 0: return dispatch_v<0, true>(q, c.v_bits, f32, g, s, e0, e1);
      case 1: return dispatch_v<1, true>(q, c.v_bits, f32, g, s, e0, e1);
      case 2: return dispatch_v<2, true>(q, c.v_bits, f32, g, s, e0, e1);
      case 3: return dispatch_v<3, true>(q, c.v_bits, f32, g, s, e0, e1);
      case 4: return dispatch_v<4, true>(q, c.v_bits, f32, g, s, e0, e1);
    }
  } else {
    switch (c.k_bits) {
      case 1: return dispatch_v<1, false>(q, c.v_bits, f32, g, s, e0, e1);
      case 2: return dispatch_v<2, false>(q, c.v_bits, f32, g, s, e0, e1);
      case 3: return dispatch_v<3, false>(q, c.v_bits, f32, g, s, e0, e1);
      case 4: return dispatch_v<4, false>(q, c.v_bits, f32, g, s, e0, e1);
    }
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
  hipError_t e = dispatch(q, cb->cfg, f32, qg, s, e0, e1);
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
