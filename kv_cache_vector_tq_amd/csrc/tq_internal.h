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

// Events of the timing hook (tq_profile_events), per thread; NULL when disabled.
struct ProfileEvents {
  void* attend_start = nullptr;
  void* attend_stop = nullptr;
  void* quant_start = nullptr;
  void* quant_stop = nullptr;
};
ProfileEvents& profile_events();

}  // namespace tq
