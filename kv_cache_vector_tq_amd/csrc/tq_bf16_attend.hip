// Uncompressed bf16 decode attention for gfx950: the same-box baseline the compressed path is
// compared against (tq_bf16_attend_decode).  Plain softmax attention, fp32 accumulation:
//   p = softmax(scale * K q), out = sum_i p_i V_i, for every (batch row, q-head).
//
// Layout: K bf16 [B][Hkv][T_cap][128] row-major; V bf16 transposed per 32-key chunk,
// [B][Hkv][T_cap/32][128][32], slot s = 8 g + e of a coordinate row holding key
// 16 (e / 4) + 4 g + e % 4 of the chunk (the order in which the score accumulators hold the
// softmax weights, so they feed the value MFMA straight from registers).
//
// Two launches: each wave streams a run of 32-key chunks (16x16x32 bf16 MFMAs, keys on M for
// the scores, coordinates on M for the values, q-heads on N) and writes one partial record
// (sums, max, sum of weights) per q-head; a second launch merges the records (log-sum-exp).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr float BLOG2E = 1.4426950408889634f;
constexpr float BNEG = -1.0e30f;
constexpr int BREC = 132;  // floats per partial record: sums[128], m, l

__device__ __forceinline__ float bcol_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float bcol_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Bf16Args {
  const uint16_t* k;
  const uint16_t* vt;
  const uint16_t* q;
  const int32_t* seq_len;
  float* rec;  // [B*Hq][n_waves][BREC]
  int Hkv, T_cap, max_seq_len, chunks_per_wave, n_waves;
  float scale_log2;
};

// Lane (col, g): q-head col % G (columns >= G repeat heads and are not written).
template <int G>
__global__ void __launch_bounds__(256, 2) bf16_attend_kernel(Bf16Args a) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int Hq = a.Hkv * G;
  const int64_t bh = (int64_t)b * a.Hkv + kvh;
  int seq = a.seq_len[b];
  seq = seq < 1 ? 1 : (seq > a.max_seq_len ? a.max_seq_len : seq);
  const int nch = (seq + 31) / 32;
  const int w = blockIdx.x * 4 + wave;
  const int c_begin = w * a.chunks_per_wave, c_end = min(c_begin + a.chunks_per_wave, nch);
  const int head = col % G;

  bf16x8 bq[4];
  const uint16_t* qh = a.q + ((int64_t)b * Hq + kvh * G + head) * D;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) bq[kb] = load_bf16x8(qh + 32 * g + 8 * kb);

  float m_run = BNEG, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* kbase = a.k + bh * a.T_cap * D;
  const uint16_t* vbase = a.vt + bh * a.T_cap * D;
  for (int c = c_begin; c < c_end; ++c) {
    bf16x8 ka[2][4], va[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) ka[t][kb] = load_bf16x8(kbase + (int64_t)(32 * c + 16 * t + col) * D + 32 * g + 8 * kb);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) va[mt] = load_bf16x8(vbase + (int64_t)c * 4096 + (16 * mt + col) * 32 + 8 * g);
    // scores: tile t holds keys 32 c + 16 t + 4 g + i in row i of this lane
    float lg[2][4];
    float mb = BNEG;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s = mfma_bf16(ka[t][kb], bq[kb], s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * c + 16 * t + 4 * g + i;
        lg[t][i] = key < seq ? s[i] * a.scale_log2 : -INFINITY;
        mb = fmaxf(mb, lg[t][i]);
      }
    }
    mb = bcol_max(mb);
    const float m_new = fmaxf(m_run, mb);
    const float alpha = exp2f(m_run - m_new);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] *= alpha;
    l_run *= alpha;
    m_run = m_new;
    // weights in the value B-operand order: element e = key 16 (e / 4) + 4 g + e % 4
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = exp2f(lg[e / 4][e % 4] - m_new);
      l_run += p;
      pb[e] = static_cast<__bf16>(p);
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) acc[mt] = mfma_bf16(va[mt], pb, acc[mt]);
  }
  const float l_tot = bcol_sum(l_run);
  if (col < G) {
    float* r = a.rec + (((int64_t)b * Hq + kvh * G + col) * a.n_waves + w) * BREC;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) r[16 * mt + 4 * g + i] = acc[mt][i];
    if (g == 0) {
      r[128] = m_run;
      r[129] = l_tot;
    }
  }
}

// One 4-wave workgroup per (batch row, q-head).  Pass 1: the largest running max of the
// head's records.  Pass 2: wave w folds records w, w + 4, ... (lane: coordinates 2 lane and
// 2 lane + 1), rescaled to that max; the four partial sums meet in LDS.
__global__ void __launch_bounds__(256) bf16_merge_kernel(const float* rec, int n_waves, float* out) {
  __shared__ float part[4][130];
  __shared__ float wmax[4];
  const float* r = rec + (int64_t)blockIdx.x * n_waves * BREC;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float M = BNEG;
  for (int i = tid; i < n_waves; i += 256) M = fmaxf(M, r[i * BREC + 128]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) wmax[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float a0 = 0.f, a1 = 0.f, L = 0.f;
#pragma unroll 8
  for (int i = wave; i < n_waves; i += 4) {
    const float* ri = r + i * BREC;
    const float2 x = reinterpret_cast<const float2*>(ri)[lane];
    const float e = exp2f(ri[128] - M);
    a0 = fmaf(e, x.x, a0);
    a1 = fmaf(e, x.y, a1);
    L = fmaf(e, ri[129], L);
  }
  part[wave][2 * lane] = a0;
  part[wave][2 * lane + 1] = a1;
  if (lane == 0) part[wave][128] = L;
  __syncthreads();
  if (tid < D) {
    const float A = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    const float Ls = part[0][128] + part[1][128] + part[2][128] + part[3][128];
    out[(int64_t)blockIdx.x * D + tid] = Ls > 0.f ? A / Ls : 0.f;
  }
}

size_t align256b(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace
}  // namespace tq

extern "C" int tq_bf16_attend_decode(const void* k, const void* vt, int B, int Hkv, int T_cap, const void* q, int Hq,
                                     const int32_t* seq_len, int max_seq_len, float scale, float* out,
                                     void* workspace, size_t* workspace_bytes, void* hip_stream) {
  using namespace tq;
  clear_error();
  if (k == nullptr || vt == nullptr || q == nullptr || seq_len == nullptr || out == nullptr ||
      workspace_bytes == nullptr)
    return fail(TQ_ERR_INVALID, "k, vt, q, seq_len, out and workspace_bytes must not be NULL");
  if (B < 1 || Hkv < 1 || T_cap < 32 || T_cap % 32 != 0)
    return fail(TQ_ERR_INVALID, "need B >= 1, Hkv >= 1 and T_cap a positive multiple of 32");
  if (Hq < 1 || Hq % Hkv != 0) return fail(TQ_ERR_INVALID, "Hq must be a positive multiple of Hkv");
  const int G = Hq / Hkv;
  if (G != 4 && G != 8 && G != 16) return fail(TQ_ERR_UNSUPPORTED, "Hq/Hkv must be 4, 8 or 16");
  if (max_seq_len < 1 || max_seq_len > T_cap) return fail(TQ_ERR_INVALID, "max_seq_len must be in 1..T_cap");
  if (!aligned(k, 16) || !aligned(vt, 16) || !aligned(q, 16) || !aligned(out, 4))
    return fail(TQ_ERR_INVALID, "k, vt, q must be 16-byte aligned and out 4-byte aligned");
  const int units = B * Hkv;
  const int nch = (max_seq_len + 31) / 32;
  // about one workgroup per CU, at least 8 chunks per wave (fewer records to merge)
  const int cus = device_cu_count();
  int n_wg = std::max(1, (cus + units - 1) / units);
  n_wg = std::min(n_wg, std::max(1, (nch + 31) / 32));
  const int cpw = (nch + 4 * n_wg - 1) / (4 * n_wg);
  n_wg = (nch + 4 * cpw - 1) / (4 * cpw);
  const int n_waves = 4 * n_wg;
  const size_t need = align256b(static_cast<size_t>(B) * Hq * n_waves * BREC * sizeof(float));
  if (workspace == nullptr) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return fail(TQ_ERR_WORKSPACE, "workspace too small");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  Bf16Args a{};
  a.k = static_cast<const uint16_t*>(k);
  a.vt = static_cast<const uint16_t*>(vt);
  a.q = static_cast<const uint16_t*>(q);
  a.seq_len = seq_len;
  a.rec = static_cast<float*>(workspace);
  a.Hkv = Hkv;
  a.T_cap = T_cap;
  a.max_seq_len = max_seq_len;
  a.chunks_per_wave = cpw;
  a.n_waves = n_waves;
  a.scale_log2 = (scale == 0.f ? INV_SQRT_D : scale) * BLOG2E;
  const dim3 grid(n_wg, Hkv, B);
  switch (G) {
    case 4: hipLaunchKernelGGL(bf16_attend_kernel<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(bf16_attend_kernel<8>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(bf16_attend_kernel<16>, grid, dim3(256), 0, s, a); break;
  }
  hipLaunchKernelGGL(bf16_merge_kernel, dim3(B * Hq), dim3(256), 0, s, a.rec, n_waves, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("bf16 attention launch: ") + hipGetErrorString(e));
  return TQ_OK;
}
