// Decode attention straight from the packed cache, for gfx950, and its C-ABI entry point
// tq_attend_decode.
//
// What is computed (pages: "Когда в марте 2026 года Google опубликовала статью..." - the
// speed-up is in attention, and the 1-bit correction passes through the softmax;
// "Google TurboQuant простыми словами", step 2 - the sign sketch keeps scores unbiased;
// "KV cache benchmark Qwen 3.6-35B-A3B", section "Неочевидный совет" - decode is bound by
// memory bandwidth):
//   q1 = R_eff q, q2 = S_b q1;
//   score_i = n_i (sum_j q1_j c[code_ij]/sqrt(d) + rnorm_i sqrt(pi/2)/m sum_j q2_j (2 sign_ij - 1));
//   p = softmax(scale * score);  out = R_eff^T sum_i p_i nv_i cv[codev_i] / sqrt(d).
//
// Two launches on the caller's stream:
//  1. query prologue, one single-wave workgroup per (batch row, kv-head, 32 output
//     coordinates): q1, q2 of the G q-heads (MFMA), stored as fp32 records;
//  2. main: one workgroup of 8 waves (one workgroup per CU, two waves per SIMD) per (batch
//     row, kv-head, context slice); each wave streams the 64-key blocks of its sub-slice.
//     Codes are turned into f16 MFMA operands by table lookups in LDS (2 to 8 codes per
//     lookup; one per lookup for 5..8-bit keys); keys sit on the M side of the score MFMAs (one key read serves all G q-heads
//     of the group), the softmax weights of a score tile feed the value MFMA directly from
//     the accumulator layout, and the value sum stays in the rotated domain.  The 8 waves
//     merge their online-softmax states in LDS and write one partial per (q-head, slice).
//     Arrival counters then elect, per
//     (batch row, kv-head), the last workgroup of each group of slices to merge that
//     group (log-sum-exp) and apply R_eff^T to it (exact bf16-split MFMA, fp32 sums), and
//     the last of those to merge the unrotated group results - no separate merge launch.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "tq_attend_kernels.h"

namespace tq {
namespace {

bool supported(const tq_config& c, int G) {
  // every configuration tq_build_codebook accepts: keys of 0..8 bits (0 only with the sketch),
  // values of 1..4 bits
  const bool keys = c.k_bits >= 0 && c.k_bits <= 8 && (c.k_qjl == 1 || c.k_bits > 0);
  return keys && c.v_bits >= 1 && c.v_bits <= 4 && (G == 4 || G == 8 || G == 16);
}

// kcw: the scaled key centroids (all 2^k_bits of them; read for k_bits > 4).
hipError_t dispatch_main(const MainArgs& a, const float* kcw, const tq_config& c, int G, int n_slices, int B, bool pre,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  const bool qjl = c.k_qjl != 0;
  switch (c.k_bits) {
    case 0: return attn::dispatch_k0(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 1: return attn::dispatch_k1(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 2: return attn::dispatch_k2(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 3: return attn::dispatch_k3(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 4: return attn::dispatch_k4(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 5: return attn::dispatch_k5(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 6: return attn::dispatch_k6(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 7: return attn::dispatch_k7(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
    case 8: return attn::dispatch_k8(a, kcw, qjl, c.v_bits, G, n_slices, B, pre, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Integer tuning knob from the environment, clamped to [lo, hi]; dflt when unset.
int env_int(const char* name, int dflt, int lo, int hi) {
  const char* v = getenv(name);
  if (v == nullptr || *v == 0) return dflt;
  const long x = strtol(v, nullptr, 10);
  return static_cast<int>(x < lo ? lo : (x > hi ? hi : x));
}

}  // namespace

int device_cu_count() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(cache.size())) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace tq

namespace tq {
namespace {

// New tokens of a decode step, quantized by the launch that also rotates the queries.
struct StepAppend {
  const void* k;
  const void* v;
  tq_dtype dtype;
  int64_t stride_b, stride_h;
  const int32_t* start_pos;
};

// Relative error of rounding x (> 0, within the f16 normal range) to f16's 11 significant bits,
// ties to even as the device conversion.
double f16_rel_error(float x) {
  int e = 0;
  const double f = std::frexp(static_cast<double>(x), &e);  // x = f 2^e, f in [0.5, 1)
  const double r = std::nearbyint(f * 2048.0) / 2048.0;
  return std::fabs(r - f) / f;
}

// A centroid table holds f16(s c_l) (5..8-bit key tables: the exact f16 pair of s c_l).  A
// common factor s (undone in fp32: with the logit scale
// for keys, with the output normalisation for values) is chosen so that the few distinct
// centroid magnitudes all sit nearly on the f16 grid: s = m / (smallest magnitude) with m an
// 11-bit integer, the m with the smallest largest rounding error.  For 2-bit codes that error
// falls from 2e-4 to 4e-7, for 3-bit codes to 4e-5.  Equal codebooks get equal factors, so a
// table shared by keys and values (equal bit widths) serves both.  Cached per codebook.
float table_scale(const float* cent, int bits) {
  if (bits == 0) return 1.0f;
  if (bits > 4) {
    // wide key tables hold each level as an exact f16 pair (hi, lo): the factor is the power of
    // two that puts the largest level in [2^14, 2^15), so that the lo terms of even the
    // smallest levels stay normal f16 numbers
    float mx = 0.f;
    for (int l = 0; l < (1 << bits); ++l) mx = std::max(mx, std::fabs(cent[l]));
    if (mx == 0.f) return 1.0f;
    int e = 0;
    std::frexp(mx, &e);  // mx in [2^(e-1), 2^e)
    return std::ldexp(1.0f, 15 - e);
  }
  static std::mutex mu;
  static std::vector<std::pair<std::vector<float>, float>> cache;
  std::vector<float> key(cent, cent + (1 << bits));
  std::lock_guard<std::mutex> lock(mu);
  for (const auto& e : cache)
    if (e.first == key) return e.second;
  std::vector<double> mags;
  for (float c : key) {
    const double m = std::fabs(static_cast<double>(c));
    bool seen = false;
    for (double x : mags) seen = seen || x == m;
    if (!seen && m > 0) mags.push_back(m);
  }
  if (mags.empty()) return 1.0f;  // an all-zero table is exact at any scale
  double lo = mags[0], hi = mags[0];
  for (double x : mags) {
    lo = std::min(lo, x);
    hi = std::max(hi, x);
  }
  float best = 1.0f;
  double best_err = 0;
  for (double x : mags) best_err = std::max(best_err, f16_rel_error(static_cast<float>(x)));
  for (int m = 1024; m < 2048; ++m) {
    const float sc = static_cast<float>(m / lo);
    if (static_cast<double>(sc) * hi > 60000.0) break;  // stay inside the f16 range
    double err = 0;
    for (double x : mags) err = std::max(err, f16_rel_error(static_cast<float>(x * sc)));
    if (err < best_err) {
      best_err = err;
      best = sc;
    }
  }
  cache.emplace_back(key, best);
  return best;
}

// Kernel arguments shared by decode and prefill attention: cache arrays, decode tables (centroids
// times their f16 grid factors), logit scale and rotation mode.  scale 0 selects 1/sqrt(d).
// kcw receives all 2^k_bits scaled key centroids (MainArgs holds the first 16).
MainArgs main_args(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache, int max_seq_len,
                   float scale, float* kcw) {
  MainArgs ma{};
  if (scale == 0.f) scale = INV_SQRT_D;
  const int one_pass = cb->cfg.rotation == TQ_ROTATION_HADAMARD ? 1 : 0;
  ma.k_codes = cache->k_codes;
  ma.k_signs = cache->k_signs;
  ma.k_norm = cache->k_norm;
  ma.k_rnorm = cache->k_rnorm;
  ma.v_codes = cache->v_codes;
  ma.v_norm = cache->v_norm;
  ma.rt_hi = p->rt_hi;
  ma.rt_lo = p->rt_lo;
  ma.Hkv = cache->Hkv;
  ma.T_cap = cache->T_cap;
  ma.max_seq_len = max_seq_len;
  ma.scale = scale;
  ma.scale_log2 = scale * LOG2E;
  ma.one_pass = one_pass;
  ma.rot_scale = one_pass ? INV_SQRT_D : 1.0f;
  const float ks = table_scale(cb->k_centroids, cb->cfg.k_bits);
  // equal widths share the key table (built from the key centroids), so they share its factor
  const float vs = cb->cfg.k_bits == cb->cfg.v_bits ? ks : table_scale(cb->v_centroids, cb->cfg.v_bits);
  for (int l = 0; l < 16; ++l) {
    ma.k_cent[l] = static_cast<float>(static_cast<double>(cb->k_centroids[l]) * ks);
    ma.v_cent[l] = static_cast<float>(static_cast<double>(cb->v_centroids[l]) * vs);
  }
  for (int l = 0; l < (cb->cfg.k_bits > 0 ? 1 << cb->cfg.k_bits : 0); ++l)
    kcw[l] = static_cast<float>(static_cast<double>(cb->k_centroids[l]) * ks);
  ma.k_unscale = static_cast<float>(1.0 / static_cast<double>(ks));
  ma.v_unscale = static_cast<float>(1.0 / static_cast<double>(vs));
  return ma;
}

// tq_attend_decode; with step != NULL the query rotation runs inside the quantize launch of
// the step's new tokens instead of a launch of its own.
int attend(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache, const void* q, tq_dtype q_dtype,
           int Hq, const int32_t* seq_len, int max_seq_len, float scale, float* out, float* scores_out,
           void* workspace, size_t* workspace_bytes, void* hip_stream, const StepAppend* step) {
  if (cb == nullptr || p == nullptr || cache == nullptr || q == nullptr || seq_len == nullptr || out == nullptr ||
      workspace_bytes == nullptr)
    return fail(TQ_ERR_INVALID, "cb, p, cache, q, seq_len, out and workspace_bytes must not be NULL");
  int rc = check_config(cb->cfg);
  if (rc != TQ_OK) return rc;
  rc = check_cache(cb->cfg, *cache);
  if (rc != TQ_OK) return rc;
  if (Hq < 1 || Hq % cache->Hkv != 0) return fail(TQ_ERR_INVALID, "Hq must be a positive multiple of Hkv");
  const int G = Hq / cache->Hkv;
  if (!supported(cb->cfg, G))
    return fail(TQ_ERR_UNSUPPORTED, "attention supports Hq/Hkv in {4, 8, 16}");
  if (max_seq_len < 1 || max_seq_len > cache->T_cap) return fail(TQ_ERR_INVALID, "max_seq_len must be in 1..T_cap");
  if (q_dtype != TQ_DTYPE_BF16 && q_dtype != TQ_DTYPE_F32) return fail(TQ_ERR_UNSUPPORTED, "query dtype");
  if (p->r_hi == nullptr || p->r_lo == nullptr || p->rt_hi == nullptr || p->rt_lo == nullptr ||
      (cb->cfg.k_qjl && (p->m_hi == nullptr || p->m_lo == nullptr)))
    return fail(TQ_ERR_INVALID, "device parameter matrices missing");
  if (!aligned(out, 4) || (scores_out && !aligned(scores_out, 4)) || !aligned(q, q_dtype == TQ_DTYPE_F32 ? 4 : 2))
    return fail(TQ_ERR_INVALID, "misaligned q / out / scores_out");

  const int B = cache->B;
  const int nblk_max = (max_seq_len + 63) / 64;
  const int units = B * cache->Hkv;
  // One workgroup of NW waves per CU (two waves per SIMD); each wave streams a run of
  // consecutive blocks of at least MIN_BLOCKS_PER_WAVE.
  static const int MIN_BLOCKS_PER_WAVE = env_int("TQ_ATTN_MIN_BLOCKS", 2, 1, 1 << 20);
  const int cus = device_cu_count();
  int n_slices = (cus + units - 1) / units;
  const int max_slices = std::max(1, (nblk_max + NW * MIN_BLOCKS_PER_WAVE - 1) / (NW * MIN_BLOCKS_PER_WAVE));
  n_slices = std::max(1, std::min({n_slices, max_slices, MAX_SLICES}));
  const int bpw = (nblk_max + NW * n_slices - 1) / (NW * n_slices);
  n_slices = (nblk_max + NW * bpw - 1) / (NW * bpw);

  // groups of 16 slices by default (TQ_ATTN_MGROUP, up to MGROUP: one load batch per merger);
  // a single group needs no second level, and at most MAX_GROUPS groups are formed.  On the
  // Llama-3.1-8B decode step (32 slices per unit) two groups of 16 took the 32-layer step from
  // 0.90 to 0.85 ms against one group of 32.
  static const int MGROUP_ASKED = env_int("TQ_ATTN_MGROUP", 16, 1, MGROUP);
  const int mgroup = std::max(MGROUP_ASKED, (n_slices + MAX_GROUPS - 1) / MAX_GROUPS);
  const int n_mgroups = (n_slices + mgroup - 1) / mgroup;
  const size_t cnt_bytes = align256(static_cast<size_t>(B) * cache->Hkv * CNT_PER_UNIT * sizeof(unsigned));
  const size_t part_bytes = align256(static_cast<size_t>(B) * Hq * n_slices * PREC * sizeof(float));
  const size_t gpart_bytes =
      n_mgroups > 1 ? align256(static_cast<size_t>(B) * Hq * n_mgroups * PREC * sizeof(float)) : 0;
  const size_t qrec_bytes = align256(static_cast<size_t>(B) * Hq * QREC * sizeof(float));
  const size_t need = qrec_bytes + cnt_bytes + part_bytes + gpart_bytes;
  if (workspace == nullptr) {
    *workspace_bytes = need;
    return TQ_OK;
  }
  if (*workspace_bytes < need) {
    *workspace_bytes = need;
    return fail(TQ_ERR_WORKSPACE, "workspace too small");
  }
  if (!aligned(workspace, 256)) return fail(TQ_ERR_INVALID, "workspace must be 256-byte aligned");

  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace) + qrec_bytes;  // after the query records
  float* qrec = reinterpret_cast<float*>(workspace);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws);  // CNT_PER_UNIT per unit, zeroed by the rotation launch
  float* part = reinterpret_cast<float*>(ws + cnt_bytes);
  float* gpart = n_mgroups > 1 ? reinterpret_cast<float*>(ws + cnt_bytes + part_bytes)
                               : nullptr;
  if (scale == 0.f) scale = INV_SQRT_D;

  // Hadamard mode: r_hi = H diag(s) = sqrt(d) R, one product pass; 1/sqrt(d) joins the scales
  const int one_pass = cb->cfg.rotation == TQ_ROTATION_HADAMARD ? 1 : 0;
  const uint16_t* m_hi = cb->cfg.k_qjl ? p->m_hi : nullptr;
  const uint16_t* m_lo = cb->cfg.k_qjl ? p->m_lo : nullptr;
  if (step != nullptr) {
    // the step's new tokens and the query rotation in one launch (it validates the append on
    // the host and launches nothing when that fails)
    const QueryRotationArgs rot{q,    q_dtype == TQ_DTYPE_F32 ? 1 : 0, G, units, qrec, p->r_hi, p->r_lo, m_hi, m_lo,
                                cnt, CNT_PER_UNIT};
    rc = quantize_launch(cb, p, step->k, step->v, step->dtype, B, cache->Hkv, 1, step->stride_b, step->stride_h, D,
                         step->start_pos, cache, hip_stream, &rot);
    if (rc != TQ_OK) return rc;
  } else {
    PrologueArgs pa{q,   p->r_hi,      p->r_lo, m_hi, m_lo, qrec, G, q_dtype == TQ_DTYPE_F32 ? 1 : 0,
                    cnt, CNT_PER_UNIT, one_pass};
    if (cb->cfg.k_qjl)
      hipLaunchKernelGGL(prologue_kernel<true>, dim3(units, 4), dim3(64), 0, s, pa);
    else
      hipLaunchKernelGGL(prologue_kernel<false>, dim3(units, 4), dim3(64), 0, s, pa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("query prologue launch: ") + hipGetErrorString(e));
  }

  float kcw[TQ_MAX_K_LEVELS];
  MainArgs ma = main_args(cb, p, cache, max_seq_len, scale, kcw);
  ma.seq_len = seq_len;
  ma.qrec = qrec;
  ma.part = part;
  ma.gpart = gpart;
  ma.cnt = cnt;
  ma.out = out;
  ma.scores_out = scores_out;
  ma.blocks_per_wave = bpw;
  ma.n_slices = n_slices;
  // decode tables replicated per lane slot when each wave streams REPL_MIN_BLOCKS blocks or
  // more (building them costs more than they save on short streams); TQ_ATTN_REPL = 0 or 1
  // forces them off or on (read at every call; the result is the same either way)
  const char* repl_env = getenv("TQ_ATTN_REPL");
  ma.repl = repl_env != nullptr && repl_env[0] == '0' ? 0
            : repl_env != nullptr && repl_env[0] == '1' ? 1
                                                        : (bpw >= REPL_MIN_BLOCKS ? 1 : 0);
  ma.mgroup = mgroup;
  const ProfileEvents& pe = profile_events();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (pe.attend_start && pe.attend_stop) {
    e0 = reinterpret_cast<hipEvent_t>(pe.attend_start);
    e1 = reinterpret_cast<hipEvent_t>(pe.attend_stop);
  }
  const hipError_t e = dispatch_main(ma, kcw, cb->cfg, G, n_slices, B, false, s, e0, e1);
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("attention launch: ") + hipGetErrorString(e));
  return TQ_OK;
}

}  // namespace
}  // namespace tq

extern "C" int tq_attend_decode(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                                const void* q, tq_dtype q_dtype, int Hq, const int32_t* seq_len, int max_seq_len,
                                float scale, float* out, float* scores_out, void* workspace,
                                size_t* workspace_bytes, void* hip_stream) {
  tq::clear_error();
  return tq::attend(cb, p, cache, q, q_dtype, Hq, seq_len, max_seq_len, scale, out, scores_out, workspace,
                    workspace_bytes, hip_stream, nullptr);
}

extern "C" int tq_decode_step(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                              const void* k, const void* v, tq_dtype kv_dtype, int64_t kv_stride_b,
                              int64_t kv_stride_h, const int32_t* start_pos, const void* q, tq_dtype q_dtype,
                              int Hq, const int32_t* seq_len, int max_seq_len, float scale, float* out,
                              float* scores_out, void* workspace, size_t* workspace_bytes, void* hip_stream) {
  tq::clear_error();
  const tq::StepAppend step{k, v, kv_dtype, kv_stride_b, kv_stride_h, start_pos};
  return tq::attend(cb, p, cache, q, q_dtype, Hq, seq_len, max_seq_len, scale, out, scores_out, workspace,
                    workspace_bytes, hip_stream, &step);
}

// ---- attention for callers that cannot allocate -----------------------------------------------
// The workspace of tq_attend_decode_noalloc is a fixed array in device memory, one per GPU the
// library runs on, held until the process ends.  Host code never uses the array's name as an
// address (on the host it names a stand-in, not device memory): each device's address is looked
// up once, with that device current, and kept.
namespace tq {
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(TQ_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device (looked up on the first call per device);
// NULL with the error set when the lookup fails.
void* scratch_address() {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(TQ_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= static_cast<int>(addr.size())) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(TQ_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = ptr;
  }
  return addr[dev];
}

}  // namespace
}  // namespace tq

extern "C" int tq_attend_decode_noalloc(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                                        const void* q, tq_dtype q_dtype, int Hq, const int32_t* seq_len,
                                        int max_seq_len, float scale, float* out, float* scores_out,
                                        void* hip_stream) {
  tq::clear_error();
  size_t need = 0;
  // the size query validates every argument on the host and launches nothing
  int rc = tq::attend(cb, p, cache, q, q_dtype, Hq, seq_len, max_seq_len, scale, out, scores_out, nullptr, &need,
                      hip_stream, nullptr);
  if (rc != TQ_OK) return rc;
  if (need > tq::NOALLOC_SCRATCH_BYTES)
    return tq::fail(TQ_ERR_WORKSPACE, "the call needs " + std::to_string(need) +
                                          " bytes of workspace, more than the fixed scratch of " +
                                          std::to_string(tq::NOALLOC_SCRATCH_BYTES) + " bytes");
  void* ws = tq::scratch_address();
  if (ws == nullptr) return TQ_ERR_DEVICE;
  size_t have = tq::NOALLOC_SCRATCH_BYTES;
  return tq::attend(cb, p, cache, q, q_dtype, Hq, seq_len, max_seq_len, scale, out, scores_out, ws, &have,
                    hip_stream, nullptr);
}

// ---- prefill attention ------------------------------------------------------------------------
extern "C" int tq_attend_prefill(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                                 const void* q, tq_dtype q_dtype, int Hq, int T_q, const int32_t* q_start,
                                 int max_seq_len, float scale, float* out, void* hip_stream) {
  using namespace tq;
  clear_error();
  if (cb == nullptr || p == nullptr || cache == nullptr || q == nullptr || q_start == nullptr || out == nullptr)
    return fail(TQ_ERR_INVALID, "cb, p, cache, q, q_start and out must not be NULL");
  int rc = check_config(cb->cfg);
  if (rc != TQ_OK) return rc;
  rc = check_cache(cb->cfg, *cache);
  if (rc != TQ_OK) return rc;
  if (Hq < 1 || Hq % cache->Hkv != 0) return fail(TQ_ERR_INVALID, "Hq must be a positive multiple of Hkv");
  const int G = Hq / cache->Hkv;
  if (!supported(cb->cfg, G)) return fail(TQ_ERR_UNSUPPORTED, "attention supports Hq/Hkv in {4, 8, 16}");
  if (T_q < 1) return fail(TQ_ERR_INVALID, "T_q must be >= 1");
  if (max_seq_len < 1 || max_seq_len > cache->T_cap) return fail(TQ_ERR_INVALID, "max_seq_len must be in 1..T_cap");
  if (q_dtype != TQ_DTYPE_BF16 && q_dtype != TQ_DTYPE_F32) return fail(TQ_ERR_UNSUPPORTED, "query dtype");
  if (p->r_hi == nullptr || p->r_lo == nullptr || p->rt_hi == nullptr || p->rt_lo == nullptr ||
      (cb->cfg.k_qjl && (p->m_hi == nullptr || p->m_lo == nullptr)))
    return fail(TQ_ERR_INVALID, "device parameter matrices missing");
  if (!aligned(q, 16) || !aligned(out, 4)) return fail(TQ_ERR_INVALID, "q must be 16-byte and out 4-byte aligned");
  const int qpg = (G > 8 ? G : 8) / G;  // query positions per unit (max(8, G) columns of (position, q-head))
  const int64_t NG = (static_cast<int64_t>(T_q) + qpg - 1) / qpg;
  if (NG * cache->Hkv > (1ll << 30)) return fail(TQ_ERR_INVALID, "too many queries in one call");
  float kcw[TQ_MAX_K_LEVELS];
  MainArgs ma = main_args(cb, p, cache, max_seq_len, scale, kcw);
  ma.out = out;
  ma.q_start = q_start;
  ma.q = q;
  ma.q_f32 = q_dtype == TQ_DTYPE_F32 ? 1 : 0;
  ma.r_hi = p->r_hi;
  ma.r_lo = p->r_lo;
  ma.m_hi = cb->cfg.k_qjl ? p->m_hi : nullptr;
  ma.m_lo = cb->cfg.k_qjl ? p->m_lo : nullptr;
  ma.T_q = T_q;
  ma.NG = static_cast<int>(NG);
  ma.n_slices = 1;
  ma.mgroup = 1;
  ma.repl = 1;
  const ProfileEvents& pe = profile_events();
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (pe.attend_start && pe.attend_stop) {
    e0 = reinterpret_cast<hipEvent_t>(pe.attend_start);
    e1 = reinterpret_cast<hipEvent_t>(pe.attend_stop);
  }
  const hipError_t e =
      dispatch_main(ma, kcw, cb->cfg, G, 1, cache->B, true, reinterpret_cast<hipStream_t>(hip_stream), e0, e1);
  if (e != hipSuccess) return fail(TQ_ERR_DEVICE, std::string("prefill attention launch: ") + hipGetErrorString(e));
  return TQ_OK;
}
