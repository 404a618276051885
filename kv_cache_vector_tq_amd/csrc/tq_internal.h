// Internal declarations shared by the host and device translation units of libtq.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/tq.h"

namespace tq {

// Sets the thread-local error text and returns code.
int fail(int code, const std::string& msg);
void clear_error();

// Checks a configuration (d, bit widths, sketch flag); returns TQ_OK or an error code.
int check_config(const tq_config& cfg);

// Checks that a cache descriptor matches cfg (pointers present, 16-byte aligned, sizes > 0).
int check_cache(const tq_config& cfg, const tq_kv_cache& cache);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Number of compute units of the current device (cached per device id).
int device_cu_count();

// Query rotation run by the quantize launch of a decode step (tq_decode_step): q1, q2 records
// of every q-head (see the query prologue of tq_attend_decode), one 4-wave workgroup per
// (batch row, kv-head) unit next to the quantize workgroups.
struct QueryRotationArgs {
  const void* q;  // [units * G][128] bf16 or fp32
  int q_f32, G, units;
  float* qrec;  // [units * G][256]
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* m_hi;  // NULL without the sketch
  const uint16_t* m_lo;
  unsigned* cnt;  // arrival counters to zero, cnt_per_unit per unit
  int cnt_per_unit;
};

// tq_quantize_kv with the query rotation of a decode step in the same launch (rot may be
// NULL: plain quantize).  Validates its arguments on the host before launching.
int quantize_launch(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v, tq_dtype in_dtype,
                    int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                    const int32_t* start_pos, const tq_kv_cache* cache, void* hip_stream,
                    const QueryRotationArgs* rot);

// Validates the arguments of a quantize call (those of tq_quantize_kv) and fills the kernel
// arguments of its keys and values (tq_quantize_tile.h).
struct QuantArgs;
int quantize_args(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v, tq_dtype in_dtype,
                  int B, int Hkv, int n_new, int64_t stride_b, int64_t stride_h, int64_t stride_t,
                  const int32_t* start_pos, const tq_kv_cache* cache, QuantArgs* ka, QuantArgs* va);

// Events of the timing hook (tq_profile_events), per thread; NULL when disabled.
struct ProfileEvents {
  void* attend_start = nullptr;
  void* attend_stop = nullptr;
  void* quant_start = nullptr;
  void* quant_stop = nullptr;
};
ProfileEvents& profile_events();

}  // namespace tq
