// Read-bandwidth probe for gfx950: the rate at which a plain streaming kernel reads HBM with
// 16-byte loads, the practical ceiling that the attention kernel's rate is compared with.
// Not part of the compressed path; exported for benchmarks (tq_read_probe in tq.h).
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <string>

#include "tq_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int PROBE_THREADS = 256;
constexpr int PROBE_UNROLL = 8;  // 16-byte loads in flight per lane

// Each lane reads PROBE_UNROLL 16-byte words per round, spaced a grid apart, so that every
// wave's loads are contiguous 1 KB runs; the words are folded with xor.  The fold reaches
// memory only if it equals a value that the caller's data never produce (key), which keeps
// every load alive without writing anything.
__global__ void __launch_bounds__(PROBE_THREADS) read_probe_kernel(const u32x4* src, int64_t n16, uint32_t key,
                                                                    uint32_t* sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * PROBE_THREADS;
  int64_t i = static_cast<int64_t>(blockIdx.x) * PROBE_THREADS + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (PROBE_UNROLL - 1) * stride < n16; i += PROBE_UNROLL * stride) {
    u32x4 w[PROBE_UNROLL];
#pragma unroll
    for (int k = 0; k < PROBE_UNROLL; ++k) w[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < PROBE_UNROLL; ++k) acc ^= w[k];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == key) sink[0] = x;
}

}  // namespace
}  // namespace tq

extern "C" int tq_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, void* hip_stream) {
  tq::clear_error();
  if (src == nullptr || sink == nullptr) return tq::fail(TQ_ERR_INVALID, "src and sink must not be NULL");
  if (!tq::aligned(src, 16) || bytes % 16 != 0 || bytes == 0)
    return tq::fail(TQ_ERR_INVALID, "src must be 16-byte aligned and bytes a positive multiple of 16");
  if (grid < 1 || grid > (1 << 20)) return tq::fail(TQ_ERR_INVALID, "grid must be in 1..2^20");
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  hipLaunchKernelGGL(tq::read_probe_kernel, dim3(grid), dim3(tq::PROBE_THREADS), 0, s,
                     reinterpret_cast<const tq::u32x4*>(src), static_cast<int64_t>(bytes / 16), 0xA5A5A5A5u, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return tq::fail(TQ_ERR_DEVICE, std::string("read probe launch: ") + hipGetErrorString(e));
  return TQ_OK;
}
