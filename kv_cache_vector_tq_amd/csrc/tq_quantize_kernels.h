// Quantize-on-write kernels for gfx950, shared by the translation units that instantiate them
// (one per key code width, compiled in parallel) and by the entry point tq_quantize_kv.  What
// the kernels compute, and how, is described in tq_quantize.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_internal.h"
#include "tq_qrot.h"
#include "tq_quantize_tile.h"

namespace tq {
namespace qk {

// Launch shape: grid workgroups of quantize, plus rot_wgs rotation workgroups when pa is set.
struct QuantGrid {
  int grid;
  const PrologueArgs* pa;
  int rot_wgs;
};

// Key tables of 5..8-bit codes (2^KB levels and 2^KB - 1 thresholds, one unused slot): too wide
// for QuantArgs, they travel as a kernel argument of their own (2 KB at 8 bits) and are
// copied to LDS at kernel start.  Narrower widths carry a one-entry placeholder.
template <int KB>
struct KeyTable {
  static constexpr int N = KB > 4 ? (1 << KB) : 1;
  float cent[N];
  float thr[N];
};

// Launches the quantize kernel (or the fused append + query rotation kernel) for key code width
// KB (k_qjl selects the sign sketch), value width vb; defined in tq_quantize_k<KB>.hip.
#define TQ_QUANT_DISPATCH(KB)                                                                   \
  hipError_t dispatch_q##KB(const QuantLaunch& q, const tq_codebook& cb, bool f32, const QuantGrid& g, \
                            hipStream_t s, hipEvent_t e0, hipEvent_t e1)
TQ_QUANT_DISPATCH(0);
TQ_QUANT_DISPATCH(1);
TQ_QUANT_DISPATCH(2);
TQ_QUANT_DISPATCH(3);
TQ_QUANT_DISPATCH(4);
TQ_QUANT_DISPATCH(5);
TQ_QUANT_DISPATCH(6);
TQ_QUANT_DISPATCH(7);
TQ_QUANT_DISPATCH(8);

}  // namespace qk

namespace {
using qk::KeyTable;
using qk::QuantGrid;

// Copies the wide key table from the kernel argument to LDS (wtab: levels, then thresholds);
// ordered before its first use by the barriers that precede every tile.
template <int KB>
__device__ __forceinline__ void stage_key_table(const KeyTable<KB>& kt, float* wtab, int tid) {
  if constexpr (KB > 4) {
    constexpr int L = 1 << KB;
    for (int i = tid; i < L; i += 256) {
      wtab[i] = kt.cent[i];
      wtab[L + i] = kt.thr[i];
    }
  }
}

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
__device__ __forceinline__ void quantize_workgroup(const QuantLaunch& q, Smem& sm, int nwg_fused,
                                                   const KeyTable<KB>& kt, float* wtab) {
  const int wg = static_cast<int>(blockIdx.x);
  const int nwg = FUSED ? nwg_fused : static_cast<int>(gridDim.x);
  const int tid = threadIdx.x;
  stage_key_table<KB>(kt, wtab, tid);
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
    load_prev<VB>(q, cur, tid, false, prev);
    lds_barrier();
    if (tensor == 0)
      quantize_tile<true, KB, QJL, F32>(q.k, sm, op, cur, prev, tid, true, wtab);
    else
      quantize_tile<false, VB, false, F32>(q.v, sm, op, cur, prev, tid, true, nullptr);
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
    // used at the end of the tile; values of up to 3 bits are packed in registers (lane-owned
    // words), 4-bit values through LDS (thread-owned words)
    load_prev<VB>(q, cur, tid, VB <= 3, prev);
    // the next tile's rows are in flight while this tile computes
    if (more) load_rows<F32>(q, nxt, tid, in);  // uniform
    lds_barrier();
    // whole blocks (every tile of a bulk fill but the first and last of a row) take the
    // instance without slot masks and sub-tile branches
    const bool full = !partial_tile(cur);  // uniform
    if (cur.tensor == 0) {
      if (full)
        quantize_tile<true, KB, QJL, F32, true>(q.k, sm, op, cur, prev, tid, false, wtab);
      else
        quantize_tile<true, KB, QJL, F32>(q.k, sm, op, cur, prev, tid, false, wtab);
    } else {
      if (full)
        quantize_tile<false, VB, false, F32, true>(q.v, sm, op, cur, prev, tid, false, nullptr);
      else
        quantize_tile<false, VB, false, F32>(q.v, sm, op, cur, prev, tid, false, nullptr);
    }
    if (!more) break;
    cur = nxt;
    t = tn;
  }
}

template <int KB, bool QJL, int VB, bool F32>
__global__ void __launch_bounds__(256, 2) quantize_kernel(QuantLaunch q, KeyTable<KB> kt) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  __shared__ float wtab[KB > 4 ? 2 << KB : 1];
  quantize_workgroup<KB, QJL, VB, F32, false>(q, sm, 0, kt, wtab);
}

// Decode step: the first n_qwg workgroups quantize the new tokens, each further workgroup
// rotates the queries of one (batch row, kv-head) unit (wave w: output coordinates
// 32 w .. 32 w + 31), all in one launch; the two parts share no data.
template <int KB, bool QJL, int VB, bool F32>
__global__ void __launch_bounds__(256, 2) append_rotate_kernel(QuantLaunch q, PrologueArgs pa, int n_qwg,
                                                               KeyTable<KB> kt) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  __shared__ float wtab[KB > 4 ? 2 << KB : 1];
  if (static_cast<int>(blockIdx.x) < n_qwg)
    quantize_workgroup<KB, QJL, VB, F32, true>(q, sm, n_qwg, kt, wtab);
  else
    rotate_query_tile<QJL>(pa, static_cast<int>(blockIdx.x) - n_qwg, threadIdx.x >> 6, threadIdx.x & 63);
}

template <int KB, bool QJL, int VB>
hipError_t launch_quantize(const QuantLaunch& q, const KeyTable<KB>& kt, bool f32, const QuantGrid& g, hipStream_t s,
                           hipEvent_t e0, hipEvent_t e1) {
  const bool ext = e0 != nullptr || e1 != nullptr;
  if (g.pa != nullptr) {
    auto kern = f32 ? append_rotate_kernel<KB, QJL, VB, true> : append_rotate_kernel<KB, QJL, VB, false>;
    const dim3 grid(g.grid + g.rot_wgs);
    if (ext)
      hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, s, e0, e1, 0, q, *g.pa, g.grid, kt);
    else
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, q, *g.pa, g.grid, kt);
  } else {
    auto kern = f32 ? quantize_kernel<KB, QJL, VB, true> : quantize_kernel<KB, QJL, VB, false>;
    if (ext)
      hipExtLaunchKernelGGL(kern, dim3(g.grid), dim3(256), 0, s, e0, e1, 0, q, kt);
    else
      hipLaunchKernelGGL(kern, dim3(g.grid), dim3(256), 0, s, q, kt);
  }
  return hipGetLastError();
}

template <int KB, bool QJL>
hipError_t dispatch_v(const QuantLaunch& q, const KeyTable<KB>& kt, int vb, bool f32, const QuantGrid& g,
                      hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (vb) {
    case 1: return launch_quantize<KB, QJL, 1>(q, kt, f32, g, s, e0, e1);
    case 2: return launch_quantize<KB, QJL, 2>(q, kt, f32, g, s, e0, e1);
    case 3: return launch_quantize<KB, QJL, 3>(q, kt, f32, g, s, e0, e1);
    case 4: return launch_quantize<KB, QJL, 4>(q, kt, f32, g, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

// Body of dispatch_q<KB>: the key table of the width, then the (sketch, value width) instance.
template <int KB>
hipError_t dispatch_width(const QuantLaunch& q, const tq_codebook& cb, bool f32, const QuantGrid& g, hipStream_t s,
                          hipEvent_t e0, hipEvent_t e1) {
  KeyTable<KB> kt{};
  if constexpr (KB > 4) {
    for (int l = 0; l < (1 << KB); ++l) kt.cent[l] = cb.k_centroids[l];
    for (int l = 0; l + 1 < (1 << KB); ++l) kt.thr[l] = cb.k_thresholds[l];
  }
  if (cb.cfg.k_qjl) return dispatch_v<KB, true>(q, kt, cb.cfg.v_bits, f32, g, s, e0, e1);
  if constexpr (KB == 0) return hipErrorInvalidValue;  // keys need codes or the sketch
  else return dispatch_v<KB, false>(q, kt, cb.cfg.v_bits, f32, g, s, e0, e1);
}

}  // namespace
}  // namespace tq
