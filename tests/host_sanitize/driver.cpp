// Host-only driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the library's
// host code (tq_host.cpp: parameter build, cache sizing, configuration and cache checks, error
// reporting).  Built with g++ by tests/test_host_sanitized.py; exits non-zero on the first
// wrong result, and the sanitizers abort on the first memory or undefined-behaviour error.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../kv_cache_vector_tq_amd/csrc/tq_internal.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, tq_last_error());
    ++failures;
  }
}

tq_config config(int kb, int kq, int vb, int rot, uint64_t seed) {
  tq_config c;
  std::memset(&c, 0, sizeof(c));
  c.d = TQ_HEAD_DIM;
  c.k_bits = kb;
  c.k_qjl = kq;
  c.v_bits = vb;
  c.rotation = rot;
  c.seed = seed;
  return c;
}

}  // namespace

int main() {
  expect(tq_abi_version() == TQ_ABI_VERSION, "abi version");
  // every accepted configuration, with exactly sized host buffers (one 128x128 matrix each)
  const size_t n = static_cast<size_t>(TQ_HEAD_DIM) * TQ_HEAD_DIM;
  for (int rot = 0; rot < 2; ++rot)
    for (int kb = 0; kb <= 8; ++kb)
      for (int kq = 0; kq <= 1; ++kq) {
        if (kb == 0 && kq == 0) continue;
        const int vb = 1 + (kb + kq + rot) % 4;
        std::vector<std::vector<uint16_t>> m(7, std::vector<uint16_t>(n));
        tq_host_params hp{m[0].data(), m[1].data(), m[2].data(), m[3].data(), m[4].data(), m[5].data(), m[6].data()};
        tq_codebook cb;
        tq_config c = config(kb, kq, vb, rot, 17 + kb);
        expect(tq_build_codebook(&c, &cb, (kb % 3 == 0) ? nullptr : &hp) == TQ_OK, "build");
        const int L = kb > 0 ? 1 << kb : 0;
        for (int l = 1; l < L; ++l) expect(cb.k_centroids[l - 1] < cb.k_centroids[l], "ascending key levels");
        for (int l = L; l < TQ_MAX_K_LEVELS; ++l) expect(cb.k_centroids[l] == 0.f, "unused key levels are zero");
        if (L > 1) expect(cb.k_thresholds[L / 2 - 1] == 0.f, "middle threshold");
        tq_cache_sizes cs;
        expect(tq_cache_layout(&c, 3, 5, 640, &cs) == TQ_OK, "layout");
        expect(cs.k_codes == static_cast<size_t>(3) * 5 * 10 * 1024 * kb, "key code bytes");
        expect(cs.bytes_per_token == 16u * kb + (kq ? 16u : 0u) + 4u + ((kq && kb) ? 4u : 0u) + 16u * vb + 4u,
               "bytes per token");
      }
  // rejected configurations leave a message
  const int bad[][4] = {{9, 0, 4, 0}, {-1, 1, 3, 0}, {0, 0, 3, 0}, {2, 2, 3, 0}, {2, 1, 0, 0}, {2, 1, 5, 0}, {2, 1, 3, 7}};
  for (const auto& b : bad) {
    tq_codebook cb;
    tq_config c = config(b[0], b[1], b[2], b[3], 1);
    expect(tq_build_codebook(&c, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "bad config rejected");
    expect(std::strlen(tq_last_error()) > 0, "error text");
  }
  tq_config c = config(2, 1, 3, 0, 0);
  c.d = 64;
  tq_codebook cb;
  expect(tq_build_codebook(&c, &cb, nullptr) == TQ_ERR_UNSUPPORTED, "d != 128 rejected");
  expect(tq_build_codebook(nullptr, &cb, nullptr) == TQ_ERR_INVALID, "NULL cfg");
  c = config(2, 1, 3, 0, 0);
  expect(tq_build_codebook(&c, nullptr, nullptr) == TQ_ERR_INVALID, "NULL codebook");
  tq_cache_sizes cs;
  expect(tq_cache_layout(&c, 0, 1, 64, &cs) == TQ_ERR_INVALID, "B = 0");
  expect(tq_cache_layout(&c, 1, 1, 100, &cs) == TQ_ERR_INVALID, "T_cap not a multiple of 64");
  expect(tq_cache_layout(&c, 1, 1, 64, nullptr) == TQ_ERR_INVALID, "NULL sizes");
  // large shapes: sizes are computed in size_t without overflow
  c = config(8, 1, 4, 0, 0);
  expect(tq_cache_layout(&c, 1024, 64, 1 << 20, &cs) == TQ_OK, "large layout");
  expect(cs.k_codes == static_cast<size_t>(1024) * 64 * (1 << 20) / 64 * 1024 * 8, "large key code bytes");
  // cache descriptor checks
  alignas(16) static uint8_t buf[256];
  tq_kv_cache kv;
  std::memset(&kv, 0, sizeof(kv));
  kv.B = 1;
  kv.Hkv = 1;
  kv.T_cap = 64;
  c = config(2, 1, 3, 0, 0);
  expect(tq::check_cache(c, kv) == TQ_ERR_INVALID, "NULL arrays rejected");
  kv.k_codes = buf;
  kv.k_signs = buf + 16;
  kv.k_norm = reinterpret_cast<float*>(buf + 32);
  kv.k_rnorm = reinterpret_cast<float*>(buf + 48);
  kv.v_codes = buf + 64;
  kv.v_norm = reinterpret_cast<float*>(buf + 80);
  expect(tq::check_cache(c, kv) == TQ_OK, "valid cache");
  kv.v_codes = buf + 65;
  expect(tq::check_cache(c, kv) == TQ_ERR_INVALID, "misaligned array rejected");
  kv.v_codes = buf + 64;
  kv.T_cap = 96;
  expect(tq::check_cache(c, kv) == TQ_ERR_INVALID, "T_cap not a multiple of 64");
  // the timing hook only stores pointers
  expect(tq_profile_events(nullptr, nullptr, nullptr, nullptr) == TQ_OK, "profile events");
  if (failures == 0) std::printf("host checks passed\n");
  return failures == 0 ? 0 : 1;
}
