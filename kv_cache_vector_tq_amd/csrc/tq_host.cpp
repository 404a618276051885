// Host side of libtq: parameter build (codebooks, rotation, sketch), cache sizing,
// argument checks and error reporting.  Pure C++; no device code.
//
// Parameter build follows the pages' description of the method (page "Когда в марте 2026
// года Google опубликовала статью...", ai-news.ru: random orthogonal rotation, Lloyd-Max
// codebook computed once for the near-normal coordinates; page "Google TurboQuant простыми
// словами", step 2: Gaussian Johnson-Lindenstrauss sketch for the 1-bit correction).  The
// generator, QR convention and bf16 split are this library's fixed reading of "random".
#include <cmath>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "tq_internal.h"

namespace tq {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

ProfileEvents& profile_events() {
  static thread_local ProfileEvents ev;
  return ev;
}

int check_config(const tq_config& cfg) {
  if (cfg.d != TQ_HEAD_DIM) return fail(TQ_ERR_UNSUPPORTED, "only d = 128 is supported");
  if (cfg.k_bits < 0 || cfg.k_bits > 8) return fail(TQ_ERR_UNSUPPORTED, "k_bits must be in 0..8");
  if (cfg.v_bits < 1 || cfg.v_bits > 4) return fail(TQ_ERR_UNSUPPORTED, "v_bits must be in 1..4");
  if (cfg.k_qjl != 0 && cfg.k_qjl != 1) return fail(TQ_ERR_UNSUPPORTED, "k_qjl must be 0 or 1");
  if (cfg.k_bits == 0 && cfg.k_qjl == 0)
    return fail(TQ_ERR_UNSUPPORTED, "keys need a scalar code (k_bits > 0) or the sign sketch");
  if (cfg.rotation != TQ_ROTATION_HAAR && cfg.rotation != TQ_ROTATION_HADAMARD)
    return fail(TQ_ERR_UNSUPPORTED, "rotation must be TQ_ROTATION_HAAR or TQ_ROTATION_HADAMARD");
  return TQ_OK;
}

int check_cache(const tq_config& cfg, const tq_kv_cache& c) {
  if (c.B < 1 || c.Hkv < 1 || c.T_cap < TQ_BLOCK_TOKENS || c.T_cap % TQ_BLOCK_TOKENS != 0)
    return fail(TQ_ERR_INVALID, "cache needs B >= 1, Hkv >= 1 and T_cap a positive multiple of 64");
  struct P {
    const void* p;
    bool needed;
    const char* name;
  } ps[] = {
      {c.k_codes, cfg.k_bits > 0, "k_codes"}, {c.k_signs, cfg.k_qjl != 0, "k_signs"},
      {c.k_norm, true, "k_norm"},           {c.k_rnorm, cfg.k_qjl != 0 && cfg.k_bits > 0, "k_rnorm"},
      {c.v_codes, true, "v_codes"},         {c.v_norm, true, "v_norm"},
  };
  for (const P& e : ps) {
    if (!e.needed) continue;
    if (e.p == nullptr) return fail(TQ_ERR_INVALID, std::string("cache.") + e.name + " is NULL");
    if (!aligned(e.p, 16)) return fail(TQ_ERR_INVALID, std::string("cache.") + e.name + " is not 16-byte aligned");
  }
  return TQ_OK;
}

}  // namespace tq

namespace {

// ---- Lloyd-Max fixed point for N(0,1) -------------------------------------------------
// Levels start evenly spaced on [-3, 3]; thresholds are midpoints; each level becomes
// the conditional mean of its cell, (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Cell masses
// use erfc on the side away from the mean so that tail cells keep their digits.
// The iteration slows down as the level count grows (at 64 levels and more it is far from
// converged after 10^5 steps), so after LLOYD_STEPS steps without convergence the same
// equations c = F(c) are solved by Newton's method.  F_l depends on c_{l-1}, c_l, c_{l+1}
// through its cell edges a = (c_{l-1} + c_l)/2 and b = (c_l + c_{l+1})/2, with
// dF_l/da = phi(a) (F_l - a) / P_l and dF_l/db = phi(b) (b - F_l) / P_l, so the Jacobian is
// tridiagonal and each step is one forward / backward elimination.
double normal_pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return std::exp(-0.5 * x * x) / std::sqrt(2.0 * M_PI);
}

double normal_mass(double a, double b) {
  const double s = std::sqrt(2.0);
  if (a >= 0.0) return 0.5 * (std::erfc(a / s) - std::erfc(b / s));
  if (b <= 0.0) return 0.5 * (std::erfc(-b / s) - std::erfc(-a / s));
  return 1.0 - 0.5 * std::erfc(b / s) - 0.5 * std::erfc(-a / s);
}

constexpr int LLOYD_STEPS = 1000;
constexpr int NEWTON_STEPS = 50;
constexpr double LLOYD_TOL = 1e-15;
constexpr double NEWTON_TOL = 1e-11;  // fp64 evaluation noise of F is near 1e-13

// Cell edges of levels lv (edges[0] = -inf, edges[L] = +inf, midpoints between).
void cell_edges(const std::vector<double>& lv, std::vector<double>& edges) {
  const int L = static_cast<int>(lv.size());
  const double inf = std::numeric_limits<double>::infinity();
  edges[0] = -inf;
  edges[L] = inf;
  for (int l = 1; l < L; ++l) edges[l] = 0.5 * (lv[l - 1] + lv[l]);
}

void lloyd_max(int bits, double* c, double* t, double* mse) {
  const int L = 1 << bits;
  std::vector<double> lv(L), nv(L), edges(L + 1);
  for (int l = 0; l < L; ++l) lv[l] = -3.0 + 6.0 * (l + 0.5) / L;
  bool converged = false;
  for (int it = 0; it < LLOYD_STEPS && !converged; ++it) {
    cell_edges(lv, edges);
    double delta = 0.0;
    for (int l = 0; l < L; ++l) {
      nv[l] = (normal_pdf(edges[l]) - normal_pdf(edges[l + 1])) / normal_mass(edges[l], edges[l + 1]);
      delta = std::fmax(delta, std::fabs(nv[l] - lv[l]));
    }
    lv.swap(nv);
    converged = delta < LLOYD_TOL;
  }
  if (!converged) {
    std::vector<double> lo(L), hi(L), w(L), x(L);
    for (int it = 0; it < NEWTON_STEPS; ++it) {
      cell_edges(lv, edges);
      for (int l = 0; l < L; ++l) {
        const double a = edges[l], b = edges[l + 1], m = normal_mass(a, b);
        const double f = (normal_pdf(a) - normal_pdf(b)) / m;
        lo[l] = std::isinf(a) ? 0.0 : normal_pdf(a) * (f - a) / m;  // dF_l/da
        hi[l] = std::isinf(b) ? 0.0 : normal_pdf(b) * (b - f) / m;  // dF_l/db
        nv[l] = f;
      }
      // (J - I) x = c - F(c): row l has 0.5 lo[l] at l - 1, 0.5 (lo[l] + hi[l]) - 1 at l and
      // 0.5 hi[l] at l + 1.  Forward elimination keeps the reduced upper entry in w, the
      // reduced right side in x.
      double piv = 0.5 * (lo[0] + hi[0]) - 1.0;
      w[0] = L > 1 ? 0.5 * hi[0] / piv : 0.0;
      x[0] = (lv[0] - nv[0]) / piv;
      for (int l = 1; l < L; ++l) {
        const double sub = 0.5 * lo[l];
        piv = 0.5 * (lo[l] + hi[l]) - 1.0 - sub * w[l - 1];
        w[l] = l + 1 < L ? 0.5 * hi[l] / piv : 0.0;
        x[l] = (lv[l] - nv[l] - sub * x[l - 1]) / piv;
      }
      for (int l = L - 2; l >= 0; --l) x[l] -= w[l] * x[l + 1];
      double step = 0.0;
      for (int l = 0; l < L; ++l) {
        lv[l] += x[l];
        step = std::fmax(step, std::fabs(x[l]));
      }
      if (step < NEWTON_TOL) break;
    }
    // the law is symmetric and so is its quantizer: mirror pairs are averaged, which removes
    // the solve's fp64 noise from the middle threshold (exactly 0, as for narrow tables)
    for (int l = 0; l < L / 2; ++l) {
      const double v = 0.5 * (lv[L - 1 - l] - lv[l]);
      lv[l] = -v;
      lv[L - 1 - l] = v;
    }
  }
  cell_edges(lv, edges);
  double s = 0.0;
  for (int l = 0; l < L; ++l) {
    const double dphi = normal_pdf(edges[l]) - normal_pdf(edges[l + 1]);
    s += dphi * dphi / normal_mass(edges[l], edges[l + 1]);
  }
  for (int l = 0; l < L; ++l) c[l] = lv[l];
  for (int l = 1; l < L; ++l) t[l - 1] = edges[l];
  *mse = 1.0 - s;
}

// ---- SplitMix64 and Box-Muller ---------------------------------------------------------
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    s += 0x9E3779B97F4A7C15ull;
    uint64_t z = s;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return static_cast<double>(next() >> 11) * 0x1.0p-53; }
};

void gaussian_fill(uint64_t state, double* out, int n) {
  SplitMix64 g{state};
  int i = 0;
  while (i < n) {
    const double u1 = 1.0 - g.uniform();
    const double u2 = g.uniform();
    const double r = std::sqrt(-2.0 * std::log(u1));
    out[i++] = r * std::cos(2.0 * M_PI * u2);
    if (i < n) out[i++] = r * std::sin(2.0 * M_PI * u2);
  }
}

// ---- randomized Walsh-Hadamard rotation: R = H diag(s) / sqrt(d) ------------------------
// H_ij = (-1)^popcount(i & j) (Sylvester); s_j = -1 when the top bit of the j-th output of
// the stream is set.  R x flips the signs of x, then applies the Walsh-Hadamard transform.
void hadamard_rotation(uint64_t state, double* R, int d) {
  SplitMix64 g{state};
  std::vector<double> s(d);
  for (int j = 0; j < d; ++j) s[j] = (g.next() >> 63) ? -1.0 : 1.0;
  const double inv = 1.0 / std::sqrt(static_cast<double>(d));
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j)
      R[i * d + j] = ((__builtin_popcount(static_cast<unsigned>(i & j)) & 1) ? -inv : inv) * s[j];
}

// ---- Householder QR: G = Q U; returns Q diag(sign U_kk) --------------------------------
void haar_rotation(const double* G, double* R, int d) {
  std::vector<double> A(G, G + d * d);  // row-major, overwritten by U
  std::vector<double> V(static_cast<size_t>(d) * d, 0.0);  // reflector k in column k
  std::vector<double> diag(d);
  for (int k = 0; k < d; ++k) {
    double norm2 = 0.0;
    for (int i = k; i < d; ++i) norm2 += A[i * d + k] * A[i * d + k];
    const double norm = std::sqrt(norm2);
    const double x0 = A[k * d + k];
    const double alpha = (x0 >= 0.0) ? -norm : norm;  // reflect away from x0 for stability
    // v = x - alpha e1, normalized
    double vnorm2 = 0.0;
    for (int i = k; i < d; ++i) {
      const double vi = A[i * d + k] - (i == k ? alpha : 0.0);
      V[i * d + k] = vi;
      vnorm2 += vi * vi;
    }
    const double vn = std::sqrt(vnorm2);
    if (vn > 0.0)
      for (int i = k; i < d; ++i) V[i * d + k] /= vn;
    // apply H = I - 2 v v^T to columns k..d-1 of A
    for (int j = k; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[i * d + k] * A[i * d + j];
      for (int i = k; i < d; ++i) A[i * d + j] -= 2.0 * V[i * d + k] * dot;
    }
    diag[k] = A[k * d + k];
  }
  // Q = H_0 H_1 ... H_{d-1}: apply reflectors to the identity from the last one back.
  std::vector<double> Q(static_cast<size_t>(d) * d, 0.0);
  for (int i = 0; i < d; ++i) Q[i * d + i] = 1.0;
  for (int k = d - 1; k >= 0; --k) {
    for (int j = 0; j < d; ++j) {
      double dot = 0.0;
      for (int i = k; i < d; ++i) dot += V[i * d + k] * Q[i * d + j];
      for (int i = k; i < d; ++i) Q[i * d + j] -= 2.0 * V[i * d + k] * dot;
    }
  }
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) R[i * d + j] = Q[i * d + j] * (diag[j] < 0.0 ? -1.0 : 1.0);
}

// bf16 bit pattern: round to fp32 (ties to even, the C conversion), then to bf16 (ties to even).
uint16_t to_bf16(double v) {
  const float f = static_cast<float>(v);
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  const uint32_t lsb = (u >> 16) & 1u;
  return static_cast<uint16_t>((u + 0x7FFFu + lsb) >> 16);
}

double from_bf16(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

}  // namespace

extern "C" {

int tq_abi_version(void) { return TQ_ABI_VERSION; }

int tq_profile_events(void* attend_start, void* attend_stop, void* quant_start, void* quant_stop) {
  tq::ProfileEvents& ev = tq::profile_events();
  ev.attend_start = attend_start;
  ev.attend_stop = attend_stop;
  ev.quant_start = quant_start;
  ev.quant_stop = quant_stop;
  return TQ_OK;
}

const char* tq_last_error(void) { return tq::g_last_error.c_str(); }

int tq_build_codebook(const tq_config* cfg, tq_codebook* cb, tq_host_params* out) {
  tq::clear_error();
  if (cfg == nullptr || cb == nullptr) return tq::fail(TQ_ERR_INVALID, "cfg and cb must not be NULL");
  int rc = tq::check_config(*cfg);
  if (rc != TQ_OK) return rc;
  std::memset(cb, 0, sizeof(*cb));
  cb->cfg = *cfg;
  double c[TQ_MAX_K_LEVELS], t[TQ_MAX_K_LEVELS], mse = 0.0;
  if (cfg->k_bits > 0) {
    lloyd_max(cfg->k_bits, c, t, &mse);
    for (int l = 0; l < (1 << cfg->k_bits); ++l) cb->k_centroids[l] = static_cast<float>(c[l]);
    for (int l = 0; l + 1 < (1 << cfg->k_bits); ++l) cb->k_thresholds[l] = static_cast<float>(t[l]);
    cb->k_mse = mse;
  }
  lloyd_max(cfg->v_bits, c, t, &mse);
  for (int l = 0; l < (1 << cfg->v_bits); ++l) cb->v_centroids[l] = static_cast<float>(c[l]);
  for (int l = 0; l + 1 < (1 << cfg->v_bits); ++l) cb->v_thresholds[l] = static_cast<float>(t[l]);
  cb->v_mse = mse;

  if (out == nullptr) return TQ_OK;
  const int d = cfg->d;
  const size_t n = static_cast<size_t>(d) * d;
  std::vector<double> G(n), R(n), Reff(n), S(n), Sb(n);
  if (cfg->rotation == TQ_ROTATION_HADAMARD) {
    hadamard_rotation(2ull * cfg->seed, R.data(), d);
  } else {
    gaussian_fill(2ull * cfg->seed, G.data(), d * d);
    haar_rotation(G.data(), R.data(), d);
  }
  // Haar: R_eff = R_hi + R_lo, the bf16 split of R.  Hadamard: R = H diag(s) / sqrt(d) with
  // H diag(s) = +-1 exact in bf16, so R_hi = H diag(s), R_lo = 0 and R_eff = R exactly (the
  // kernels apply 1/sqrt(d) as a scale).
  const bool hadamard = cfg->rotation == TQ_ROTATION_HADAMARD;
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) {
      const double r = R[static_cast<size_t>(i) * d + j];
      const uint16_t hi = hadamard ? to_bf16(r < 0.0 ? -1.0 : 1.0) : to_bf16(r);
      const uint16_t lo = hadamard ? uint16_t(0) : to_bf16(r - from_bf16(hi));
      Reff[static_cast<size_t>(i) * d + j] = hadamard ? r : from_bf16(hi) + from_bf16(lo);
      if (out->r_hi) out->r_hi[i * d + j] = hi;
      if (out->r_lo) out->r_lo[i * d + j] = lo;
      if (out->rt_hi) out->rt_hi[j * d + i] = hi;
      if (out->rt_lo) out->rt_lo[j * d + i] = lo;
    }
  gaussian_fill(2ull * cfg->seed + 1ull, S.data(), d * d);
  for (size_t i = 0; i < n; ++i) {
    const uint16_t b = to_bf16(S[i]);
    Sb[i] = from_bf16(b);
    if (out->s_qjl) out->s_qjl[i] = b;
  }
  if (out->m_hi || out->m_lo) {
    for (int i = 0; i < d; ++i)
      for (int j = 0; j < d; ++j) {
        double m = 0.0;  // M = S_b R_eff (Haar: every product exact in fp64, 8 x 16 significant bits)
        for (int k = 0; k < d; ++k) m += Sb[static_cast<size_t>(i) * d + k] * Reff[static_cast<size_t>(k) * d + j];
        const uint16_t hi = to_bf16(m);
        if (out->m_hi) out->m_hi[i * d + j] = hi;
        if (out->m_lo) out->m_lo[i * d + j] = to_bf16(m - from_bf16(hi));
      }
  }
  return TQ_OK;
}

int tq_cache_layout(const tq_config* cfg, int B, int Hkv, int T_cap, tq_cache_sizes* out) {
  tq::clear_error();
  if (cfg == nullptr || out == nullptr) return tq::fail(TQ_ERR_INVALID, "cfg and out must not be NULL");
  int rc = tq::check_config(*cfg);
  if (rc != TQ_OK) return rc;
  if (B < 1 || Hkv < 1 || T_cap < TQ_BLOCK_TOKENS || T_cap % TQ_BLOCK_TOKENS != 0)
    return tq::fail(TQ_ERR_INVALID, "need B >= 1, Hkv >= 1, T_cap a positive multiple of 64");
  const size_t slots = static_cast<size_t>(B) * Hkv * T_cap;
  const size_t blocks = slots / TQ_BLOCK_TOKENS;
  out->k_codes = blocks * 1024u * cfg->k_bits;
  out->k_signs = cfg->k_qjl ? blocks * 1024u : 0;
  out->k_norm = slots * 4;
  out->k_rnorm = (cfg->k_qjl && cfg->k_bits > 0) ? slots * 4 : 0;
  out->v_codes = blocks * 1024u * cfg->v_bits;
  out->v_norm = slots * 4;
  out->bytes_per_token = 16u * cfg->k_bits + (cfg->k_qjl ? 16u : 0u) + 4u +
                         ((cfg->k_qjl && cfg->k_bits > 0) ? 4u : 0u) + 16u * cfg->v_bits + 4u;
  return TQ_OK;
}

}  // extern "C"
