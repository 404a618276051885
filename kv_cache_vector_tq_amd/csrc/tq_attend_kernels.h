// Decode-attention kernels for gfx950, shared by the translation units that instantiate them
// (one per key code width, compiled in parallel) and by the host entry point tq_attend_decode.
// What the kernels compute, and how, is described in tq_attend.hip.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <type_traits>
#include <vector>

#include "tq_common.h"
#include "tq_qrot.h"
#include "tq_internal.h"

namespace tq {
namespace attn {

struct MainArgs {
  const uint8_t* k_codes;
  const uint8_t* k_signs;
  const float* k_norm;
  const float* k_rnorm;
  const uint8_t* v_codes;
  const float* v_norm;
  const int32_t* seq_len;
  const float* qrec;      // [B*Hq][QREC] query records of the prologue
  const uint16_t* rt_hi;  // R_hi^T, R_lo^T
  const uint16_t* rt_lo;
  float* part;        // [B*Hq][n_slices][PREC]: rotated sums, m, l of each slice
  float* gpart;       // [B*Hq][n_groups][PREC]: the same per group of mgroup slices
  unsigned* cnt;      // [B*Hkv][MAX_GROUPS + 1] arrival counters: one per merge group, then the
                      // top-level one; zeroed by the query rotation launched before this kernel
  float* out;         // [B*Hq][128]
  float* scores_out;  // NULL or [B*Hq][T_cap]
  int Hkv, T_cap, max_seq_len, blocks_per_wave, n_slices, mgroup;
  int repl;           // decode: replicated decode tables (the kernel instance; prefill always)
  float scale_log2;   // scale * log2(e)
  float scale;
  float k_cent[16];   // key centroids times a factor k_scale (table_scale in tq_attend.hip)
  float k_unscale;     // 1 / k_scale
  float v_cent[16];   // value centroids times v_scale
  float v_unscale;     // 1 / v_scale
  // rotation: one_pass = 0: R_eff = rt_hi^T + rt_lo^T; one_pass = 1 (Hadamard): R_eff =
  // rt_hi^T / sqrt(d) (rt_lo = 0), the query records hold sqrt(d) R_eff q, and rot_scale =
  // 1/sqrt(d) scales the key-code term of the scores and the unrotated outputs
  int one_pass;
  float rot_scale;
  // prefill (causal attention of a prompt's queries): query t of row b sits at position
  // q_start[b] + t and attends keys 0 .. q_start[b] + t; units of 16 / G consecutive queries
  // times the G q-heads of a kv-head, NG units per (row, kv-head); the kernel rotates its
  // queries itself (q [B][Hq][T_q][128], q_f32) and writes out [B][Hq][T_q][128]
  const int32_t* q_start;
  const void* q;
  const uint16_t* r_hi;  // R_hi, R_lo, M_hi, M_lo (query rotation)
  const uint16_t* r_lo;
  const uint16_t* m_hi;
  const uint16_t* m_lo;
  int q_f32, T_q, NG;
};

// Launches the attention kernel for key code width KB (k_qjl selects the sign sketch), value
// width vb and group size G; defined in tq_attend_k<KB>.hip.
// kcw: host array of the 2^KB scaled key centroids when KB > 4 (unused otherwise).
#define TQ_ATTN_DISPATCH(KB)                                                                       \
  hipError_t dispatch_k##KB(const MainArgs& a, const float* kcw, bool qjl, int vb, int G, int n_slices, int B, \
                            bool pre, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
TQ_ATTN_DISPATCH(0);
TQ_ATTN_DISPATCH(1);
TQ_ATTN_DISPATCH(2);
TQ_ATTN_DISPATCH(3);
TQ_ATTN_DISPATCH(4);
TQ_ATTN_DISPATCH(5);
TQ_ATTN_DISPATCH(6);
TQ_ATTN_DISPATCH(7);
TQ_ATTN_DISPATCH(8);

// Key centroids of 5..8-bit codes (times the table factor): too many for MainArgs, they are a
// kernel argument of their own (1 KB at 8 bits); narrower widths carry a one-entry placeholder.
template <int KB>
struct KeyCent {
  float c[KB > 4 ? (1 << KB) : 1];
};

}  // namespace attn

namespace {
using attn::MainArgs;


constexpr float LOG2E = 1.4426950408889634f;
constexpr float KAPPA = 0.009791666936874390f;  // sqrt(pi/2)/128
constexpr float NEG_BIG = -1.0e30f;
constexpr int PREC = 132;   // floats per partial record: sums[128], m, l, scale, pad
constexpr int NW = 8;                            // waves per attention workgroup (one per CU)
constexpr int NT = 64 * NW;                      // threads per attention workgroup
constexpr int MGROUP = 32;                       // slices per first-level merge group
constexpr int MAX_GROUPS = 32;                   // merge groups per (batch row, kv-head)
constexpr int MAX_SLICES = MGROUP * MAX_GROUPS;  // context slices per (batch row, kv-head)
constexpr int CNT_PER_UNIT = MAX_GROUPS + 1;     // arrival counters per (batch row, kv-head)
constexpr int REPL_MIN_BLOCKS = 8;               // decode waves streaming this many blocks replicate tables

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ---- code decoding ------------------------------------------------------------------------
// Codes become f16 MFMA operands through lookup tables in LDS built at kernel start.  A table
// Tab<B, K> maps a K-bit key (CPL = K / B consecutive B-bit codes, or K sign bits) to the CPL
// f16 values, EBYTES = 2 CPL bytes per entry, one entry after the other:
//   B = 1 and sign bits: an 8-bit key -> 8 values (16-byte entries, 256 entries);
//   B = 2: an 8-bit key -> 4 codes (8-byte entries, 256 entries);
//   B = 3: a 12-bit key -> 4 codes (8-byte entries, 4096 entries);
//   B = 4: an 8-bit key -> 2 codes (4-byte entries, 256 entries);
//   B = 5..8: one code -> its value as an exact pair of f16 terms hi + lo (4-byte entries,
//     2^B entries); the score takes a product with each term.  (One f16 term alone leaves the
//     many distinct levels of a wide table a relative error up to 2^-12 each, which no common
//     factor can remove and which reaches the logits; the pair holds each level to ~2^-24.)
// Keys and values of the same width share one table.  Long streams replicate the tables of
// 8-bit keys per lane slot (REP below), which frees a wave's random lookups of LDS bank
// conflicts.
template <int B>
struct Tab {
  static constexpr int K = B > 4 ? B : ((B == 3) ? 12 : 8);  // key bits
  static constexpr int CPL = K / B;                           // codes per lookup
  static constexpr int EBYTES = B > 4 ? 4 : 2 * CPL;          // bytes per entry
  static constexpr int SHIFT = EBYTES == 16 ? 4 : (EBYTES == 8 ? 3 : (EBYTES == 4 ? 2 : 1));
  static constexpr int BYTES = (1 << K) * EBYTES;
};

// Geometry of Tab<B> as constexpr functions of a runtime-free B (0: no table).
constexpr int tab_k(int B) { return B > 4 ? B : (B == 3 ? 12 : 8); }
constexpr int tab_ebytes(int B) { return B > 4 ? 4 : 2 * (tab_k(B) / B); }
constexpr int tab_bytes(int B) { return B == 0 ? 0 : (1 << tab_k(B)) * tab_ebytes(B); }

// How a lookup finds its entry in LDS.  PTR: the table sits below 64 KB and the entry's byte
// offset is added to the table's address (the constant part travels in the instruction's offset
// field).  ORB: a 12-bit-key table at a 32 KB-aligned base anywhere in LDS; mask and base come
// from registers (lo = base, mk = mask), so one AND-OR replaces the mask alone.  REP: a
// replicated 8-bit-key table (below).
enum { PTR = 0, ORB = 1, REP = 2 };

// A replicated table (8-bit keys, B = 1, 2 or 4): entry e fills the 256 bytes at base + 256 e
// with 256 / EBYTES copies of itself, and lane slot c = lane mod (256 / EBYTES) reads copy c.
// The lanes of a wave then read disjoint banks whatever their keys (random keys into one copy
// collide in the banks: measured at several percent of the batch-16 128K-context decode), and
// the address base + 256 e + EBYTES c is one byte permute of the code word and a per-lane
// constant lo = EBYTES c + base (base a multiple of 64 KB, in byte 2).
constexpr int REP_BYTES = 256 * 256;

__device__ __forceinline__ uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Fills table Tab<B> at tab: entry e holds the f16 values of its CPL codes (code i = bits
// B i .. B i + B - 1 of e), or for SIGN the values -1 / +1 of its 8 bits.  All NT threads of
// the workgroup write 16-byte chunks.
template <int B, bool SIGN>
__device__ void build_table(uint8_t* tab, const float* cent, int tid) {
  using T = Tab<B>;
  constexpr int L = 1 << B;
  if constexpr (T::CPL == 1) {  // one code per entry: entry e is (hi, lo) with hi + lo = cent[e]
    static_assert(!SIGN && T::EBYTES == 4 && T::BYTES % 16 == 0, "wide key tables");
    for (int c = tid; c < T::BYTES / 16; c += NT) {
      u32x4 w;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float x = cent[4 * c + h];
        const _Float16 hi = static_cast<_Float16>(x);
        // x - hi is exact in fp32 (hi is x rounded to 11 significant bits)
        w[h] = pack_f16x2(hi, static_cast<_Float16>(x - static_cast<float>(hi)));
      }
      *reinterpret_cast<u32x4*>(tab + 16 * c) = w;
    }
    return;
  }
  _Float16 c16[L];
#pragma unroll
  for (int l = 0; l < L; ++l) c16[l] = SIGN ? static_cast<_Float16>(l ? 1.0f : -1.0f) : static_cast<_Float16>(cent[l]);
  for (int c = tid; c < T::BYTES / 16; c += NT) {
    uint16_t v[8];  // the 8 halves of chunk c
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int e = (8 * c + h) / T::CPL;  // entry
      const int i = (8 * c + h) % T::CPL;  // code within the entry
      const int code = (e >> (B * i)) & (L - 1);
      _Float16 x = c16[0];
#pragma unroll
      for (int l = 1; l < L; ++l) x = code == l ? c16[l] : x;  // no dynamic register indexing
      v[h] = __builtin_bit_cast(uint16_t, x);
    }
    u32x4 w;
#pragma unroll
    for (int h = 0; h < 4; ++h) w[h] = static_cast<uint32_t>(v[2 * h]) | (static_cast<uint32_t>(v[2 * h + 1]) << 16);
    *reinterpret_cast<u32x4*>(tab + 16 * c) = w;
  }
}

// Fills the replicated table of B-bit codes (B = 1, 2, 4; SIGN: the -1 / +1 values of sign
// bits) at tab: two threads per entry, each writing half of its 256-byte row.
template <int B, bool SIGN>
__device__ void build_table_rep(uint8_t* tab, const float* cent, int tid) {
  static_assert(tab_k(B) == 8 && NT == 512, "replicated tables: 8-bit keys, two threads per entry");
  constexpr int L = 1 << B, CPL = 8 / B;
  _Float16 c16[L];
#pragma unroll
  for (int l = 0; l < L; ++l) c16[l] = SIGN ? static_cast<_Float16>(l ? 1.0f : -1.0f) : static_cast<_Float16>(cent[l]);
  const int e = tid >> 1, half = tid & 1;
  uint16_t v[8];  // the entry's CPL values, repeated to 16 bytes
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    const int code = (e >> (B * (h % CPL))) & (L - 1);
    _Float16 x = c16[0];
#pragma unroll
    for (int l = 1; l < L; ++l) x = code == l ? c16[l] : x;  // no dynamic register indexing
    v[h] = __builtin_bit_cast(uint16_t, x);
  }
  u32x4 w;
#pragma unroll
  for (int h = 0; h < 4; ++h) w[h] = static_cast<uint32_t>(v[2 * h]) | (static_cast<uint32_t>(v[2 * h + 1]) << 16);
  // the 8 chunks of the half row in an order rotated by the entry: the 64 lanes of a store then
  // spread over all banks (in order, every lane's chunk would sit in the same two bank groups)
  u32x4* dst = reinterpret_cast<u32x4*>(tab + 256 * e + 128 * half);
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[(j + e) & 7] = w;
}

// Bits P .. P+N-1 of the little-endian dword array dw, shifted left by S.
template <int P, int N, int S>
__device__ __forceinline__ uint32_t field(const uint32_t* dw) {
  constexpr int w = P >> 5, o = P & 31;
  constexpr uint32_t mask = ((1u << N) - 1u) << S;
  if constexpr (o + N <= 32) {
    if constexpr (o >= S)
      return (dw[w] >> (o - S)) & mask;
    else
      return (dw[w] << (S - o)) & mask;
  } else {
    return __builtin_amdgcn_alignbit(dw[w + 1], dw[w], o - S) & mask;
  }
}

// Byte address (relative to tab) of the entry of the key at bit P of dw in a table of mode MODE
// at LDS offset OFF (see PTR, ORB, REP).
template <int B, int P, int MODE, int OFF>
__device__ __forceinline__ uint32_t entry(const uint32_t* dw, uint32_t lo, uint32_t mk) {
  using T = Tab<B>;
  if constexpr (MODE == REP) {
    static_assert(T::K == 8 && P % 8 == 0, "replicated tables take byte-aligned 8-bit keys");
    // bytes: lo.0 (lane slot), the key byte, lo.2 (base / 64 KB), 0
    constexpr uint32_t sel = 0x0C020000u | ((4u + (P / 8) % 4) << 8);
    return __builtin_amdgcn_perm(dw[P / 32], lo, sel);
  } else if constexpr (MODE == ORB) {
    static_assert(T::K == 12 && OFF % 32768 == 0, "OR-ed bases: 12-bit keys, 32 KB-aligned tables");
    // the field of field<P, 12, SHIFT> before its mask, then (x & mk) | lo with mk = the mask
    constexpr int w = P >> 5, o = P & 31, S = T::SHIFT;
    uint32_t x;
    if constexpr (o + T::K > 32)
      x = __builtin_amdgcn_alignbit(dw[w + 1], dw[w], o - S);
    else if constexpr (o >= S)
      x = dw[w] >> (o - S);
    else
      x = dw[w] << (S - o);
    return (x & mk) | lo;
  } else {
    return field<P, T::K, T::SHIFT>(dw);
  }
}

// The 8 codes (B bits each, or sign bits for B = 1 in the sign table) starting at bit P of dw ->
// f16x8, through table Tab<B>: at tab (MODE PTR) or at the workgroup's LDS base tab (ORB, REP).
template <int B, int P, int MODE = PTR, int OFF = 0>
__device__ __forceinline__ f16x8 decode8(const uint32_t* dw, const uint8_t* tab, uint32_t lo = 0, uint32_t mk = 0) {
  using T = Tab<B>;
  constexpr int K = T::K;
  if constexpr (T::EBYTES == 16) {
    return *reinterpret_cast<const f16x8*>(tab + entry<B, P, MODE, OFF>(dw, lo, mk));
  } else if constexpr (T::EBYTES == 8) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(tab + entry<B, P, MODE, OFF>(dw, lo, mk));
    const u32x2 y = *reinterpret_cast<const u32x2*>(tab + entry<B, P + K, MODE, OFF>(dw, lo, mk));
    return __builtin_bit_cast(f16x8, u32x4{x[0], x[1], y[0], y[1]});
  } else {
    return __builtin_bit_cast(f16x8, u32x4{*reinterpret_cast<const uint32_t*>(tab + entry<B, P, MODE, OFF>(dw, lo, mk)),
                                           *reinterpret_cast<const uint32_t*>(tab + entry<B, P + K, MODE, OFF>(dw, lo, mk)),
                                           *reinterpret_cast<const uint32_t*>(tab + entry<B, P + 2 * K, MODE, OFF>(dw, lo, mk)),
                                           *reinterpret_cast<const uint32_t*>(tab + entry<B, P + 3 * K, MODE, OFF>(dw, lo, mk))});
  }
}

// Wide codes (B = 5..8): the 8 codes starting at bit P of dw -> the hi and lo f16 terms of their
// values, one 4-byte lookup per code; hi takes the low halves of the entries, lo the high ones.
template <int B, int P>
__device__ __forceinline__ void decode8_pair(const uint32_t* dw, const uint8_t* tab, f16x8& hi, f16x8& lo) {
  using T = Tab<B>;
  static_assert(T::CPL == 1 && T::EBYTES == 4, "wide key tables");
  constexpr int K = T::K, S = T::SHIFT;
  u32x4 h, l;
  static_for<0, 4>([&](auto I_) {
    constexpr int i = decltype(I_)::value;
    const uint32_t e0 = *reinterpret_cast<const uint32_t*>(tab + field<P + 2 * i * K, K, S>(dw));
    const uint32_t e1 = *reinterpret_cast<const uint32_t*>(tab + field<P + (2 * i + 1) * K, K, S>(dw));
    h[i] = __builtin_amdgcn_perm(e1, e0, 0x05040100u);  // e0 bytes 0-1, e1 bytes 0-1
    l[i] = __builtin_amdgcn_perm(e1, e0, 0x07060302u);  // e0 bytes 2-3, e1 bytes 2-3
  });
  hi = __builtin_bit_cast(f16x8, h);
  lo = __builtin_bit_cast(f16x8, l);
}

// Reductions over the 4 lanes of a column (lanes l, l^16, l^32, l^48) with the gfx950
// row-swap instructions (VALU, no LDS round trip): each swap returns this lane's value and
// its partner's, in some order, so max / sum of the pair is the pairwise reduction.
__device__ __forceinline__ float col_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The value of the lane N columns before this one, cyclically within its row of 16 lanes (row
// rotation right), an operand modifier of the add that consumes it.  Every lane has a source,
// so the destination's previous value is never kept: it is left undefined (no zeroing move).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  static_assert(N > 0 && N < 16, "rotation within a row");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xF, 0xF, true));
}

template <int N>
__device__ __forceinline__ void load_dwords(uint32_t* dst, const uint8_t* src) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i)
    *reinterpret_cast<u32x4*>(dst + 4 * i) = *reinterpret_cast<const u32x4*>(src + 16 * i);
}

// ---- query prologue --------------------------------------------------------------------------
// One single-wave workgroup per (batch row, kv-head, 32 output coordinates) writes q1 and q2
// (fp32) of the G q-heads into a record per q-head (rotate_query_tile).
constexpr int QS = 132;  // LDS row stride (floats) of the merged sums in the epilogue

template <bool QJL>
__global__ void __launch_bounds__(64) prologue_kernel(PrologueArgs a) {
  rotate_query_tile<QJL>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// ---- main kernel ----------------------------------------------------------------------------

// Partial results crossing workgroups are written and read with device-scope (coherent)
// atomic accesses, which bypass the non-coherent per-XCD caching of ordinary accesses.  A
// writer drains its stores (s_waitcnt) before the workgroup barrier that precedes its
// arrival increment; a reader issues its loads only after its own increment has returned
// with the final count.  No cache-wide writeback or invalidate is needed.
__device__ __forceinline__ void st_dev2(float* p, float x, float y) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(x)) | (static_cast<uint64_t>(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
__device__ __forceinline__ void drain_stores() { __builtin_amdgcn_s_waitcnt(0); }

// LDS of the epilogue (aliases the decode tables)
struct Epi {
  float rec[64][PREC];  // per wave 0..3 and lane column: rotated sums, m, l, value scale
  float w64[64];        // weight of each record in its q-head's merge
  float amat[16][QS];   // merged rotated sums of the q-heads (rows >= G unused)
  float st[16][2];      // merged max and sum of each q-head
  int stage;
};

struct Merged {
  float A0, A1;  // weighted sums of coordinates 2 lane, 2 lane + 1
  float M, L;
};

// Log-sum-exp merge of `count` partial records (sums[128], m, l at stride PREC from hs) by one
// wave: lane l takes sums 2 l and 2 l + 1 of every record, so one 8-byte load per lane covers
// a whole record, and lane k of a batch loads (m, l) of its record k, which the merge reads
// back as wave-uniform values.  Records are loaded NB at a time from clamped (always valid)
// indices, all loads of a batch in flight together, and merged online; the surplus of a
// partial batch is masked after its loads.
template <int NB>
__device__ Merged merge_batches(const float* hs, int count, int lane) {
  static_assert(NB <= 64, "one (m, l) pair per lane");
  float M = NEG_BIG, L = 0.f, A0 = 0.f, A1 = 0.f;
  for (int r0 = 0; r0 < count; r0 += NB) {
    float2 v[NB];
    const float2 mine = ld_dev2(hs + static_cast<int64_t>(min(r0 + lane % NB, count - 1)) * PREC + 128);
#pragma unroll
    for (int k = 0; k < NB; ++k) v[k] = ld_dev2(hs + static_cast<int64_t>(min(r0 + k, count - 1)) * PREC + 2 * lane);
    float mk[NB], lk[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      mk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mine.x), k));
      lk[k] = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(mine.y), k));
      if (r0 + k >= count) {
        mk[k] = NEG_BIG;
        lk[k] = 0.f;
      }
    }
    float Mb = M;
#pragma unroll
    for (int k = 0; k < NB; ++k) Mb = fmaxf(Mb, mk[k]);
    const float sc = exp2f(M - Mb);
    A0 *= sc;
    A1 *= sc;
    L *= sc;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      // 0 for masked and empty records, unless every record so far is empty (then v = l = 0)
      const float e = r0 + k < count ? exp2f(mk[k] - Mb) : 0.f;
      A0 = fmaf(e, v[k].x, A0);
      A1 = fmaf(e, v[k].y, A1);
      L = fmaf(e, lk[k], L);
    }
    M = Mb;
  }
  return Merged{A0, A1, M, L};
}
// batch size by count: one round of loads for up to 32 records
__device__ __forceinline__ Merged merge_records(const float* hs, int count, int lane) {
  if (count <= 4) return merge_batches<4>(hs, count, lane);
  if (count <= 16) return merge_batches<16>(hs, count, lane);
  return merge_batches<32>(hs, count, lane);
}


template <int KB, bool QJL, int VB, int G, bool REPL>
struct MainCfg {
  static constexpr int TPD = 16 / G;       // score tiles packed into one accumulator set
  static constexpr int NSETS = 4 / TPD;    // accumulator sets per 64-key block
  // Score terms: the key-code part (C) and the sign part (S), each as the product with an f16
  // hi and lo term of the (scaled) query coordinates: kinds 0 = C hi, 1 = C lo, 2 = S hi,
  // 3 = S lo.  The 16 columns of a score MFMA hold NP = 16 / G parts of G q-heads each; the
  // NT terms fill the parts of NA accumulators, term (a NP + k) % NT in part k of accumulator a
  // (with fewer terms than parts they repeat), except that one accumulator with all four terms
  // orders its parts C hi, S hi, C lo, S lo (see the score assembly).
  static constexpr int NT = (KB > 0 ? 2 : 0) + (QJL ? 2 : 0);
  static constexpr int NP = 16 / G;
  static constexpr int NA = NT > NP ? NT / NP : 1;
  static constexpr bool MIXED = NA == 1 && NT == 4;  // C and S terms share the accumulator
  static constexpr int kind(int a, int k) {
    if (MIXED) return k == 0 ? 0 : (k == 1 ? 2 : (k == 2 ? 1 : 3));
    const int i = (a * NP + k) % NT;
    return KB > 0 ? i : i + 2;
  }
  static constexpr bool has_c(int a) {
    bool r = false;
    for (int k = 0; k < NP; ++k) r = r || kind(a, k) < 2;
    return r;
  }
  static constexpr bool has_s(int a) {
    bool r = false;
    for (int k = 0; k < NP; ++k) r = r || kind(a, k) >= 2;
    return r;
  }
  static constexpr bool SHARED = (KB == VB);  // one table serves keys and values
  // ---- LDS layout of the decode tables.  Roles 0 = key codes, 1 = signs, 2 = value codes (none
  // when SHARED), each a Tab<B> (B = 0: no table).  With REPL, 8-bit-key tables are replicated
  // (REP, 64 KB each) as far as they fit in the 160 KB of LDS: signs first, then key codes, then
  // value codes.  Tables that are not replicated sit below 64 KB (PTR) unless their keys are
  // 12-bit (ORB: anywhere, 32 KB-aligned).  The G query records are staged behind the tables
  // when they fit there, else over the start of the table space before the tables are built
  // (QALIAS).  The epilogue reuses the whole space after the block loop.  Replication pays on
  // long streams; its 64 KB stores per table and the serialized build of QALIAS cost more than
  // they save on launches of a few blocks per wave, which keep REPL off.
  static constexpr int LDS_MAX = 160 * 1024;
  static constexpr int RB0 = KB, RB1 = QJL ? 1 : 0, RB2 = SHARED ? 0 : VB;
  static constexpr int rb(int r) { return r == 0 ? RB0 : (r == 1 ? RB1 : RB2); }
  static constexpr bool repable(int r) { return rb(r) == 1 || rb(r) == 2 || rb(r) == 4; }
  static constexpr int QSTAGE = G * QREC * 4;
  static constexpr int MERGE = static_cast<int>(sizeof(Epi));
  struct Plan {
    int mode[3], off[3], tables, lds;
    bool qalias, fits;
  };
  static constexpr Plan plan(int mask) {  // mask: roles asked to be replicated
    Plan pl{{PTR, PTR, PTR}, {0, 0, 0}, 0, 0, false, true};
    int low = 0;
    bool any_rep = false;
    for (int r = 0; r < 3; ++r) any_rep = any_rep || (rb(r) != 0 && ((mask >> r) & 1) && repable(r));
    for (int r = 0; r < 3; ++r) {
      const bool rep = ((mask >> r) & 1) && repable(r);
      if (rb(r) == 0) continue;
      if (rep) {
        pl.mode[r] = REP;
      } else if (rb(r) == 3 && any_rep) {  // without replication every table stays below 64 KB
        pl.mode[r] = ORB;
      } else {
        pl.mode[r] = PTR;
        pl.off[r] = low;
        low += tab_bytes(rb(r));
      }
    }
    if (low > 65536) pl.fits = false;
    int pos = low;
    if (any_rep) {
      pos = low == 0 ? 0 : 65536;
      for (int r = 0; r < 3; ++r)
        if (rb(r) != 0 && pl.mode[r] == REP) {
          pl.off[r] = pos;
          pos += REP_BYTES;
        }
    }
    for (int r = 0; r < 3; ++r)
      if (rb(r) != 0 && pl.mode[r] == ORB) {
        pos = (pos + 32767) / 32768 * 32768;
        pl.off[r] = pos;
        pos += tab_bytes(rb(r));
      }
    pl.tables = pos;
    pl.qalias = pos + QSTAGE > LDS_MAX;
    const int used = pl.qalias ? pos : pos + QSTAGE;
    pl.lds = used > MERGE ? used : MERGE;
    if (pl.lds > LDS_MAX || pos > LDS_MAX || (pl.qalias && QSTAGE > pos)) pl.fits = false;
    return pl;
  }
  static constexpr Plan choose() {
    // replication sets by preference: all, {S, K}, {S, V}, {K, V}, {S}, {K}, {V}, none
    constexpr int order[8] = {7, 3, 6, 5, 2, 1, 4, 0};
    for (int i = 0; i < 8; ++i) {
      const Plan pl = plan(order[i]);
      if (pl.fits) return pl;
    }
    return plan(0);
  }
  static constexpr Plan PL = REPL ? choose() : plan(0);
  static constexpr int KMODE = PL.mode[0], SMODE = PL.mode[1], VMODE = SHARED ? PL.mode[0] : PL.mode[2];
  static constexpr int KOFF = PL.off[0], SOFF = PL.off[1], VOFF = SHARED ? PL.off[0] : PL.off[2];
  static constexpr int TABLES = PL.tables;
  static constexpr bool QALIAS = PL.qalias;
  static constexpr int QOFF = QALIAS ? 0 : TABLES;
  static constexpr int LDS = PL.lds;
  static constexpr bool FITS = PL.fits;
};

// Streams the 64-key blocks of one slice.  SCORES: also write the logits (parity runs).
// PRE: prefill - every lane column class is its own query (GC = max(8, G) columns: GC / G
// consecutive positions times the G q-heads), each with its causal limit; one workgroup per
// unit, whose 8 waves split the unit's blocks; queries are rotated in the kernel; outputs are
// written directly.  (Eight columns rather than sixteen keep the hi and lo query terms in the
// columns of one accumulator, which halves the query operands held in registers.)
template <int KB, bool QJL, int VB, int G, bool SCORES, bool PRE, bool REPL>
__global__ void __launch_bounds__(NT, 1) attend_kernel(MainArgs a, attn::KeyCent<KB> kcent) {
  constexpr int GC = PRE ? (G > 8 ? G : 8) : G;  // query columns per unit
  constexpr int QPG = GC / G;                     // prefill: query positions per unit
  using C = MainCfg<KB, QJL, VB, GC, REPL>;
  constexpr int TPD = C::TPD, NSETS = C::NSETS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  constexpr int KBT = KB > 0 ? KB : 1;  // key code width of the (unused when KB = 0) key table

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int tcls = col / GC;   // which tile of a set this lane's column belongs to
  const int hh = col % GC;     // query column within the unit
  const int Hq = a.Hkv * G;
  const int b = blockIdx.z;
  // decode: unit (b, kv-head blockIdx.y), slice blockIdx.x; prefill: unit blockIdx.x = kv-head
  // NG + (NG - 1 - query group) (the longest causal ranges start first)
  const int kvh = PRE ? static_cast<int>(blockIdx.x) / a.NG : static_cast<int>(blockIdx.y);
  const int qgrp = PRE ? a.NG - 1 - static_cast<int>(blockIdx.x) % a.NG : 0;
  const int64_t cu = (int64_t)b * a.Hkv + kvh;           // (row, kv-head) of the cache
  const int64_t bh = PRE ? cu * a.NG + qgrp : cu;         // unit of the partial records
  const int nblk_cap = a.T_cap / 64;

  int seq, lim = 0;
  if constexpr (PRE) {
    const int qs = max(a.q_start[b], 0);
    const int t_col = qgrp * QPG + hh / G;  // the lane column's query position in the unit
    const int t_last = min(a.T_q, qgrp * QPG + QPG) - 1;
    seq = min(qs + t_last + 1, a.max_seq_len);
    lim = t_col < a.T_q ? min(qs + t_col + 1, a.max_seq_len) : 0;  // keys 0 .. lim - 1 visible
  } else {
    seq = a.seq_len[b];
    seq = seq < 1 ? 1 : (seq > a.max_seq_len ? a.max_seq_len : seq);
  }
  const int nblk = (seq + 63) / 64;
  const int bpw = PRE ? (nblk + NW - 1) / NW : a.blocks_per_wave;
  const int slice = PRE ? wave : static_cast<int>(blockIdx.x) * NW + wave;
  const int blk_begin = slice * bpw;
  const int blk_end = min(blk_begin + bpw, nblk);

  // online softmax per lane column: m_run (log2 domain), l_run = sum 2^(lg - m_run);
  // acc = sum P' V with P' = 2^(lg - m_run) nv / s_run and s_run >= 2^-12 times every such
  // product (inv_run = 1 / s_run)
  float m_run = NEG_BIG, l_run = 0.f, s_run = 0.f, inv_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block data of one lane.  Codes of the next block are loaded while the current one is
  // processed; so are its norms, up to 8 q-heads per kv-head (see the block loop below).
  struct Blk {
    uint32_t kd[KB > 0 ? 4 * KB : 1];
    uint32_t sd[4];
    uint32_t vd[4 * VB];
  };
  auto load_block = [&](int blk, Blk& d) {
    if constexpr (KB > 0)
      load_dwords<4 * KB>(d.kd, a.k_codes + (cu * nblk_cap + blk) * (1024 * KB) + lane * 16 * KB);
    if constexpr (QJL) load_dwords<4>(d.sd, a.k_signs + (cu * nblk_cap + blk) * 1024 + lane * 16);
    load_dwords<4 * VB>(d.vd, a.v_codes + (cu * nblk_cap + blk) * (1024 * VB) + lane * 16 * VB);
  };
  // Norms of the lane's kept keys (set s: tile s TPD + tcls, rows 4 g .. 4 g + 3).
  struct Norms {
    f32x4 kn[NSETS], kr[NSETS], vn[NSETS];
  };
  auto load_norms = [&](int blk, Norms& d) {
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const int64_t tok = cu * a.T_cap + blk * 64 + 16 * (s * TPD + tcls) + 4 * g;
      d.kn[s] = *reinterpret_cast<const f32x4*>(a.k_norm + tok);
      if constexpr (QJL && KB > 0) d.kr[s] = *reinterpret_cast<const f32x4*>(a.k_rnorm + tok);
      d.vn[s] = *reinterpret_cast<const f32x4*>(a.v_norm + tok);
    }
  };
  constexpr int QWORDS = GC * QREC / 4;
  constexpr int QPT = PRE ? 1 : (QWORDS + NT - 1) / NT;
  float* const qst = reinterpret_cast<float*>(smem + C::QOFF);
  f32x4 qw[QPT];
  if constexpr (!PRE) {
    const float* qsrc = a.qrec + ((int64_t)b * Hq + kvh * G) * QREC;
#pragma unroll
    for (int k = 0; k < QPT; ++k) qw[k] = *reinterpret_cast<const f32x4*>(qsrc + 4 * min(tid + k * NT, QWORDS - 1));
  }
  // The G query records of this kv-head (contiguous) go through LDS: one 16-byte load per
  // thread (two for G = 16), issued before the block loads, so that no wave's query waits
  // behind other waves' block loads.  (Each lane loading its own 256 bytes of records instead
  // measured 10 % slower on the 32K-context Llama-3.1-8B layer.)
  // Block loads are unconditional, from clamped (always in-bounds) block indices: a load under
  // a branch would make the compiler wait for every load in flight where the branches join,
  // which would serialize the prefetch with the current block's compute.
  Blk cur, nxt;
  load_block(min(blk_begin, nblk_cap - 1), cur);  // in flight while the tables are built

  auto build_tables = [&]() {
    if constexpr (KB > 4)
      build_table<KBT, false>(smem + C::KOFF, kcent.c, tid);
    else if constexpr (KB > 0 && C::KMODE == REP)
      build_table_rep<KBT, false>(smem + C::KOFF, a.k_cent, tid);
    else if constexpr (KB > 0)
      build_table<KBT, false>(smem + C::KOFF, a.k_cent, tid);
    if constexpr (QJL && C::SMODE == REP)
      build_table_rep<1, true>(smem + C::SOFF, nullptr, tid);
    else if constexpr (QJL)
      build_table<1, true>(smem + C::SOFF, nullptr, tid);
    if constexpr (!C::SHARED && C::VMODE == REP)
      build_table_rep<VB, false>(smem + C::VOFF, a.v_cent, tid);
    else if constexpr (!C::SHARED)
      build_table<VB, false>(smem + C::VOFF, a.v_cent, tid);
  };
  // with the query records staged over the table space, the tables follow the operands below
  if constexpr (!C::QALIAS) build_tables();
  if constexpr (PRE) {
    // waves 0..3 rotate the unit's 16 queries, 32 output coordinates each, into the records
    if (wave < 4) {
      const int cq = col % GC;  // lanes of columns >= GC rotate a copy (not stored)
      const int t = qgrp * QPG + cq / G;
      const int64_t qrow = ((int64_t)b * Hq + kvh * G + cq % G) * a.T_q + min(t, a.T_q - 1);
      rotate_queries<QJL>(a.q, a.q_f32 != 0, qrow, t < a.T_q, a.one_pass, a.r_hi, a.r_lo, a.m_hi, a.m_lo, qst,
                          GC, wave, lane);
    }
  } else {
#pragma unroll
    for (int k = 0; k < QPT; ++k)
      if (tid + k * NT < QWORDS) *reinterpret_cast<f32x4*>(qst + 4 * (tid + k * NT)) = qw[k];
  }
  __syncthreads();  // query records (and tables unless they follow below) ready
  // Score operands.  For q-head hh = col % G: x1 = q1 c1 and x2 = q2 c2 with the constant factors
  // of the score folded in (c1 = log2(e) scale / sqrt(d) / k_scale (/ sqrt(d) in one-pass
  // rotation mode): the key term is q1 . c / sqrt(d); c2 = log2(e) scale sqrt(pi/2) / m: the sign
  // term), each scaled by a power of two 2^-e that brings its largest magnitude into [0.5, 1) (the
  // 4 lanes of a column hold the 128 coordinates), then split into two f16 terms (hi + lo, the
  // fp32 value to about 22 bits: one f16 term alone leaves a relative error of 2^-12 per
  // coordinate, which large logits carry into the softmax weights).  Lane (col, g) holds, for
  // k-block kb, coordinates 32 g + 8 kb + e of the term of its part k = col / G in each
  // accumulator (zero in the code operand for sign terms and the other way round); u1 and u2
  // undo the two scalings.
  const int part = col / GC;
  f16x8 bc[C::NA][4], bsg[C::NA][4];
  float u1, u2;
  {
    const float lscale = a.scale * LOG2E;
    const float c1 = INV_SQRT_D * lscale * a.k_unscale * a.rot_scale, c2 = KAPPA * lscale;
    f32x4 qv1[8], qv2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qv1[i] = KB > 0 ? *reinterpret_cast<const f32x4*>(qst + hh * QREC + 32 * g + 4 * i) * c1
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      qv2[i] = QJL ? *reinterpret_cast<const f32x4*>(qst + hh * QREC + D + 32 * g + 4 * i) * c2
                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m1 = 0.f, m2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        m1 = fmaxf(m1, fabsf(qv1[i][e]));
        m2 = fmaxf(m2, fabsf(qv2[i][e]));
      }
    m1 = col_max(m1);
    m2 = col_max(m2);
    int e1 = 0, e2 = 0;
    if (m1 > 0.f) frexpf(m1, &e1);
    if (m2 > 0.f) frexpf(m2, &e2);
    const float s1 = ldexpf(1.0f, -e1), s2 = ldexpf(1.0f, -e2);  // exact powers of two
    u1 = ldexpf(1.0f, e1);
    u2 = ldexpf(1.0f, e2);
    // this lane's term in each accumulator (part = col / G), as bit masks that pick the hi or
    // lo f16 term of a code or sign coordinate pair, or neither (branch-free selects: written as
    // conditional assignments, the per-element choice compiled to divergent branches)
    uint32_t mch[C::NA], mcl[C::NA], msh[C::NA], msl[C::NA];
    static_for<0, C::NA>([&](auto A_) {
      constexpr int ac = decltype(A_)::value;
      int kd = C::kind(ac, 0);
      static_for<1, C::NP>([&](auto K_) { kd = part == decltype(K_)::value ? C::kind(ac, decltype(K_)::value) : kd; });
      mch[ac] = kd == 0 ? ~0u : 0u;
      mcl[ac] = kd == 1 ? ~0u : 0u;
      msh[ac] = kd == 2 ? ~0u : 0u;
      msl[ac] = kd == 3 ? ~0u : 0u;
    });
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4 wc[C::NA], ws[C::NA];
#pragma unroll
      for (int jp = 0; jp < 4; ++jp) {  // coordinate pairs 2 jp, 2 jp + 1 of the k-block
        uint32_t hp1, lp1, hp2, lp2;
        {
          const float x1a = qv1[2 * kb + jp / 2][2 * (jp % 2)] * s1, x1b = qv1[2 * kb + jp / 2][2 * (jp % 2) + 1] * s1;
          const float x2a = qv2[2 * kb + jp / 2][2 * (jp % 2)] * s2, x2b = qv2[2 * kb + jp / 2][2 * (jp % 2) + 1] * s2;
          const _Float16 h1a = static_cast<_Float16>(x1a), h1b = static_cast<_Float16>(x1b);
          const _Float16 h2a = static_cast<_Float16>(x2a), h2b = static_cast<_Float16>(x2b);
          hp1 = pack_f16x2(h1a, h1b);
          lp1 = pack_f16x2(static_cast<_Float16>(x1a - static_cast<float>(h1a)),
                           static_cast<_Float16>(x1b - static_cast<float>(h1b)));
          hp2 = pack_f16x2(h2a, h2b);
          lp2 = pack_f16x2(static_cast<_Float16>(x2a - static_cast<float>(h2a)),
                           static_cast<_Float16>(x2b - static_cast<float>(h2b)));
        }
        static_for<0, C::NA>([&](auto A_) {
          constexpr int ac = decltype(A_)::value;
          // operands only for the accumulators that take that kind of term
          if constexpr (C::has_c(ac)) wc[ac][jp] = (hp1 & mch[ac]) | (lp1 & mcl[ac]);
          if constexpr (C::has_s(ac)) ws[ac][jp] = (hp2 & msh[ac]) | (lp2 & msl[ac]);
        });
      }
      static_for<0, C::NA>([&](auto A_) {
        constexpr int ac = decltype(A_)::value;
        if constexpr (C::has_c(ac)) bc[ac][kb] = __builtin_bit_cast(f16x8, wc[ac]);
        if constexpr (C::has_s(ac)) bsg[ac][kb] = __builtin_bit_cast(f16x8, ws[ac]);
      });
    }
  }

  if constexpr (C::QALIAS) {
    __syncthreads();  // every wave has read the query records
    build_tables();
    __syncthreads();  // tables ready
  }
  // Per-lane constants of the replicated tables: the lane slot's byte offset in an entry's row,
  // and the table's base / 64 KB in byte 2.
  auto rep_lo = [&](int B, int off) -> uint32_t {
    const int eb = tab_ebytes(B);
    return static_cast<uint32_t>((lane & (256 / eb - 1)) * eb) | (static_cast<uint32_t>(off >> 16) << 16);
  };
  // ORB tables: base and mask as register values (an instruction takes one constant operand)
  uint32_t orb_mask = (0xFFFu << 3);
  if constexpr (C::KMODE == ORB || C::VMODE == ORB) asm volatile("" : "+v"(orb_mask));
  auto lo_of = [&](int mode, int B, int off) -> uint32_t {
    if (mode == REP) return rep_lo(B, off);
    return mode == ORB ? static_cast<uint32_t>(off) : 0u;
  };
  uint32_t lo_k = lo_of(C::KMODE, KBT, C::KOFF), lo_s = lo_of(C::SMODE, 1, C::SOFF), lo_v = lo_of(C::VMODE, VB, C::VOFF);
  if constexpr (C::KMODE == ORB) asm volatile("" : "+v"(lo_k));
  if constexpr (C::VMODE == ORB) asm volatile("" : "+v"(lo_v));
  uint8_t* const ktab = C::KMODE == PTR ? smem + C::KOFF : smem;
  uint8_t* const stab = C::SMODE == PTR ? smem + C::SOFF : smem;
  uint8_t* const vtab = C::VMODE == PTR ? smem + C::VOFF : smem;

  // One block: scores, online softmax, value sums.  `d` holds the block's codes, `nrm` its norms.
  auto process = [&](const Blk& cur, const Norms& nrm, int blk) {
    // Issue priority by phase: the score MFMAs (and the table reads feeding them) highest, the
    // value MFMAs next, the softmax lowest, so that with two waves per SIMD the matrix core is
    // fed while the other wave's softmax chain fills the gaps.
    __builtin_amdgcn_s_setprio(2);

    // ---- scores: tile t = keys 16 t .. 16 t + 15 of the block.  Per accumulator, the code and
    // sign MFMAs (operands zero outside their own terms' columns) sum into one register set.
    // The hi and lo parts are then summed across lanes (row rotations by G columns) and, for
    // the shared accumulator of G = 4, the sign sum brought next to the code sum (parts C hi,
    // S hi, C lo, S lo: rotating by 2 G gives C or S in every lane, rotating that by G the
    // other one).  Each lane keeps the pair (p, q) of the tile of its column class in every set
    // (tile s TPD + tcls of set s) ------------------------------------------------------------
    f32x4 cp[NSETS], cq[NSETS];
    [[maybe_unused]] f32x4 pm[4];  // shared accumulator: each tile's column sums (C or S by part)
    static_for<0, 4>([&](auto T_) {
      constexpr int t = decltype(T_)::value;
      f32x4 v[C::NA];
      static_for<0, C::NA>([&](auto A_) {
        constexpr int ac = decltype(A_)::value;
        f32x4 d = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (KB > 0 && C::has_c(ac)) {
          static_for<0, 4>([&](auto KB_) {
            constexpr int kb = decltype(KB_)::value;
            constexpr int P = 32 * KB * t + 8 * KB * kb;
            if constexpr (KB > 4) {  // the two terms of every level against the same operand
              f16x8 kh, kl;
              decode8_pair<KBT, P>(cur.kd, smem + C::KOFF, kh, kl);
              d = mfma_f16(kh, bc[ac][kb], d);
              d = mfma_f16(kl, bc[ac][kb], d);
            } else {
              d = mfma_f16(decode8<KBT, P, C::KMODE, C::KOFF>(cur.kd, ktab, lo_k, orb_mask), bc[ac][kb], d);
            }
          });
        }
        if constexpr (QJL && C::has_s(ac)) {
          static_for<0, 4>([&](auto KB_) {
            constexpr int kb = decltype(KB_)::value;
            d = mfma_f16(decode8<1, 32 * t + 8 * kb, C::SMODE, C::SOFF>(cur.sd, stab, lo_s), bsg[ac][kb], d);
          });
        }
        v[ac] = d;
      });
      f32x4 p, q = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (C::MIXED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pm[t][i] = v[0][i] + row_ror<2 * GC>(v[0][i]);
        return;  // tiles are selected below, once all four are summed
      } else if constexpr (C::NP >= 2) {  // NA = 1 (one kind of term) or 2 (C, S): hi, lo parts
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = v[0][i] + row_ror<GC>(v[0][i]);
          if constexpr (C::NA == 2) q[i] = v[1][i] + row_ror<GC>(v[1][i]);
        }
      } else {  // G = 16: one term per accumulator, in lane order C hi, C lo, S hi, S lo
        p = v[0] + v[1];
        if constexpr (C::NA == 4) q = v[2] + v[3];
      }
      constexpr int st_ = t / TPD, ct = t % TPD;
      if constexpr (ct == 0) {
        cp[st_] = p;
        cq[st_] = q;
      } else {
        if (tcls == ct) {
          cp[st_] = p;
          cq[st_] = q;
        }
      }
    });
    if constexpr (C::MIXED) {
      // The lane of part k (= its tile class) keeps tile k's sum and takes tile k's other sum
      // from the lane of part k - 1 (the rotation's source), which offers its tile k (one row
      // rotation by G columns instead of one per tile).
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float own = pm[0][i], offer = pm[1][i];
        own = part == 1 ? pm[1][i] : own;
        own = part == 2 ? pm[2][i] : own;
        own = part == 3 ? pm[3][i] : own;
        offer = part == 1 ? pm[2][i] : offer;
        offer = part == 2 ? pm[3][i] : offer;
        offer = part == 3 ? pm[0][i] : offer;
        cp[0][i] = own;
        cq[0][i] = row_ror<GC>(offer);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // logit * log2(e) = n (u1 C + u2 rnorm S): C, S are p, q (or q, p in the odd parts of a
    // shared accumulator); with one kind of term, p alone
    const bool odd = C::MIXED && (part & 1);
    const float a1 = odd ? 0.f : u1, a2 = odd ? u1 : 0.f;  // weights of p and q for C
    const float b1 = odd ? u2 : 0.f, b2 = odd ? 0.f : u2;  // weights of p and q for S

    // ---- logits of this lane's keys: set s, row i -> key 16 (s TPD + tcls) + 4 g + i --------
    // lg = logit * log2(e); lgb = lg + an upper bound of log2(nv) (from the float exponent),
    // so that 2^(lg - m) nv <= 2^(lgb - m).  One column reduction of (max lg, max lgb).
    float lg[NSETS][4];
    float mb = NEG_BIG, mvb = NEG_BIG;
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = blk * 64 + 16 * (s * TPD + tcls) + 4 * g + i;
        float sc;
        if constexpr (C::NT == 4) {
          const float r = nrm.kr[s][i];
          sc = fmaf(cp[s][i], fmaf(r, b1, a1), cq[s][i] * fmaf(r, b2, a2));
        } else {
          sc = cp[s][i] * (KB > 0 ? u1 : u2);
        }
        const float l2 = nrm.kn[s][i] * sc;
        const bool valid = key < (PRE ? lim : seq);
        if constexpr (SCORES) {
          if (valid) a.scores_out[((int64_t)b * Hq + kvh * G + hh) * a.T_cap + key] = l2 * (1.0f / LOG2E);
        }
        lg[s][i] = valid ? l2 : -INFINITY;
        const float ebound = static_cast<float>(static_cast<int>(__float_as_uint(nrm.vn[s][i]) >> 23) - 126);
        mb = fmaxf(mb, lg[s][i]);
        mvb = fmaxf(mvb, lg[s][i] + ebound);
      }
    }
    mb = col_max(mb);
    mvb = col_max(mvb);
    // Lazy rescaling: a column keeps its (m_run, s_run) while the block's weights P' under them
    // stay at most 2^12 (f16 holds such weights as exactly as weights below 1) and its logits
    // within 2^32 of m_run; otherwise both move to the block's bounds, with weights at most 1.
    // The accumulator is rescaled only when some column moved.  (Detecting an unchanged scale
    // from f = s rcp(s) instead fails most of the time: that product is not exactly 1 in fp32.)
    const bool keep = mb <= m_run + 32.f && __builtin_amdgcn_exp2f(mvb - m_run) <= s_run * 4096.f;
    const float m_new = keep ? m_run : fmaxf(m_run, mb);
    const float alpha = keep ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float s_scaled = s_run * alpha;
    const float s_new = keep ? s_run : fmaxf(s_scaled, __builtin_amdgcn_exp2f(mvb - m_new));
    const float inv = keep ? inv_run : (s_new > 0.f ? __builtin_amdgcn_rcpf(s_new) : 0.f);
    const float f = (keep || !(s_new > 0.f)) ? 1.0f : s_scaled * inv;
    if (__any(f != 1.0f)) {  // rescale only when some column's scale moved
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[mt] *= f;
    }
    float lsum = 0.f;
    uint32_t pw[NSETS][2];
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = __builtin_amdgcn_exp2f(lg[s][i] - m_new);  // 0 for keys past the sequence
        lsum += pr;
        x[i] = pr > 0.f ? fminf(pr * nrm.vn[s][i] * inv, 4096.f) : 0.f;
      }
      pw[s][0] = pack_f16x2(static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]));
      pw[s][1] = pack_f16x2(static_cast<_Float16>(x[2]), static_cast<_Float16>(x[3]));
    }
    m_run = m_new;
    s_run = s_new;
    inv_run = inv;
    l_run = fmaf(l_run, alpha, lsum);

    __builtin_amdgcn_s_setprio(1);
    // ---- value MFMAs: k-block kb2 holds tiles 2 kb2 (elements 0..3) and 2 kb2 + 1 (4..7) ---
    static_for<0, 2>([&](auto KB2) {
      constexpr int kb2 = decltype(KB2)::value;
      u32x4 bpw;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int te = 2 * kb2 + hf;
        const bool mine = (te % TPD) == tcls;
        bpw[2 * hf] = mine ? pw[te / TPD][0] : 0u;
        bpw[2 * hf + 1] = mine ? pw[te / TPD][1] : 0u;
      }
      const f16x8 bp = __builtin_bit_cast(f16x8, bpw);
      static_for<0, 8>([&](auto MT) {
        constexpr int mt = decltype(MT)::value;
        const f16x8 av = decode8<VB, 8 * VB * (2 * mt + kb2), C::VMODE, C::VOFF>(cur.vd, vtab, lo_v, orb_mask);
        acc[mt] = mfma_f16(av, bp, acc[mt]);
      });
    });
    __builtin_amdgcn_s_setprio(0);
  };
  // Two blocks per iteration with the buffers swapping roles, so that the prefetched block never
  // has to be copied into the current one.  Up to 8 q-heads per kv-head, the next block's norms
  // are loaded one block ahead as well (norms loaded at the block's own start are waited for
  // after its score MFMAs); with 16 q-heads the extra registers would spill, and the norms are
  // loaded at the block's start.
  if constexpr (G <= 8) {
    Norms ncur, nnxt;
    load_norms(min(blk_begin, nblk_cap - 1), ncur);
    for (int blk = blk_begin; blk < blk_end; blk += 2) {
      load_block(min(blk + 1, blk_end - 1), nxt);
      load_norms(min(blk + 1, blk_end - 1), nnxt);
      process(cur, ncur, blk);
      if (blk + 1 >= blk_end) break;  // uniform
      load_block(min(blk + 2, blk_end - 1), cur);
      load_norms(min(blk + 2, blk_end - 1), ncur);
      process(nxt, nnxt, blk + 1);
    }
  } else {
    for (int blk = blk_begin; blk < blk_end; blk += 2) {
      {
        Norms nrm;
        load_norms(blk, nrm);
        load_block(min(blk + 1, blk_end - 1), nxt);
        process(cur, nrm, blk);
      }
      if (blk + 1 >= blk_end) break;  // uniform
      Norms nrm;
      load_norms(blk + 1, nrm);
      load_block(min(blk + 2, blk_end - 1), cur);
      process(nxt, nrm, blk + 1);
    }
  }

  // Operands of R_eff^T for the unrotation, in case this workgroup becomes a merger: rows
  // k = 16 wave + col.  Loaded now, so that their latency overlaps the epilogue below instead
  // of following the arrival count.
  bf16x8 th[4], tl[4];
  {
    const int k = 16 * wave + col;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      th[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(a.rt_hi + k * D + 32 * g + 8 * kb));
      tl[kb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(a.rt_lo + k * D + 32 * g + 8 * kb));
    }
  }

  // ---- merge the waves and the TPD column classes of each q-head in LDS ------------------------
  // Waves 4..7 hand their state to wave w - 4 (same lane columns, hence the same q-heads), which
  // folds it into its own: sums weighted by s 2^(m - M), so the folded record has scale 1.
  float l_tot = col_sum(l_run);
  __syncthreads();  // every wave is done with the tables
  Epi* ep = reinterpret_cast<Epi*>(smem);
  auto put_record = [&](int r) {
    float* rec = ep->rec[r];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[16 * mt + 4 * g + i] = acc[mt][i];
    if (g == 0) {
      rec[128] = m_run;
      rec[129] = l_tot;
      rec[130] = s_run;
    }
  };
  if (wave >= 4) put_record((wave - 4) * 16 + col);
  __syncthreads();
  if (wave < 4) {
    const float* pr = ep->rec[wave * 16 + col];
    const float m2 = pr[128], l2 = pr[129], s2 = pr[130];
    const float M = fmaxf(m_run, m2);
    const float e1 = exp2f(m_run - M), e2 = exp2f(m2 - M);
    const float w1 = s_run * e1, w2 = s2 * e2;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][i] = fmaf(acc[mt][i], w1, pr[16 * mt + 4 * g + i] * w2);
    m_run = M;
    l_tot = fmaf(l_tot, e1, l2 * e2);
    s_run = 1.0f;
  }
  __syncthreads();  // the handed-over records are consumed
  if (wave < 4) put_record(wave * 16 + col);
  __syncthreads();
  // record r = 16 w + c GC + h belongs to query column h; wave 0 finds each column's maximum and
  // the record weights over the lanes with the same h (xor offsets that keep r mod GC)
  if (tid < 64) {
    const float* rec = ep->rec[tid];
    const float m = rec[128];
    float M = m;
#pragma unroll
    for (int o = GC; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float e = exp2f(m - M);
    ep->w64[tid] = rec[130] * e;
    float l = rec[129] * e;
#pragma unroll
    for (int o = GC; o < 64; o <<= 1) l += __shfl_xor(l, o);
    if (tid < GC) {
      if constexpr (PRE) {
        ep->st[tid][0] = M;
        ep->st[tid][1] = l;
      } else {
        st_dev2(a.part + ((bh * GC + tid) * a.n_slices + blockIdx.x) * PREC + 128, M, l);
      }
    }
  }
  __syncthreads();
  // prefill: the weighted sums of the workgroup are the unit's result (amat aliases no record)
  for (int idx = tid; idx < GC * D / 2; idx += NT) {
    const int h = idx / (D / 2), j = 2 * (idx % (D / 2));
    float A0 = 0.f, A1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int c = 0; c < TPD; ++c) {
        const int r = 16 * w + c * GC + h;
        A0 = fmaf(ep->rec[r][j], ep->w64[r], A0);
        A1 = fmaf(ep->rec[r][j + 1], ep->w64[r], A1);
      }
    if constexpr (PRE) {
      ep->amat[h][j] = A0;
      ep->amat[h][j + 1] = A1;
    } else {
      st_dev2(a.part + ((bh * GC + h) * a.n_slices + blockIdx.x) * PREC + j, A0, A1);
    }
  }

  // ---- merge over the slices: the last workgroup of each group of MGROUP slices merges the
  // group and applies R_eff^T, the last group merger merges the groups ---------------------
  const int ns = PRE ? 1 : a.n_slices;
  const int mgroup = a.mgroup;
  const int ngrp = PRE ? 1 : (ns + mgroup - 1) / mgroup;
  const int grp = PRE ? 0 : static_cast<int>(blockIdx.x) / mgroup;
  drain_stores();
  __syncthreads();
  unsigned* const cnt_top = PRE ? nullptr : a.cnt + bh * CNT_PER_UNIT + MAX_GROUPS;
  if constexpr (PRE) {
    // the workgroup holds the whole unit: unrotate and write its outputs below
  } else if (tid == 0) {
    // counters start at zero (the query rotation launch zeroes them before every call)
    int stage = 0;
    unsigned* cnt = ngrp == 1 ? cnt_top : a.cnt + bh * CNT_PER_UNIT + grp;
    const unsigned last = ngrp == 1 ? ns - 1 : min(mgroup, ns - mgroup * grp) - 1;
    if (atomicAdd(cnt, 1u) == last) stage = ngrp == 1 ? 2 : 1;
    ep->stage = stage;
  }
  __syncthreads();
  if (!PRE && ep->stage == 0) return;
  // This workgroup merges: it applies R_eff^T to what it merged (the unrotation is linear, so
  // merging unrotated group results is the same as unrotating the merge).  Merge the slices of
  // this group (or all slices with a single group) into ep->amat, ep->st; wave w takes q-heads
  // w, w + 4, ...
  if constexpr (!PRE) {
    const int first = ngrp == 1 ? 0 : mgroup * grp;
    const int count = ngrp == 1 ? ns : min(mgroup, ns - mgroup * grp);
    for (int h = wave; h < G; h += NW) {
      const Merged r = merge_records(a.part + ((bh * G + h) * ns + first) * PREC, count, lane);
      *reinterpret_cast<float2*>(&ep->amat[h][2 * lane]) = make_float2(r.A0, r.A1);
      if (lane == 0) {
        ep->st[h][0] = r.M;
        ep->st[h][1] = r.L;
      }
    }
    __syncthreads();
  }
  // U[h][k] = sum_j A[h][j] R_eff[j][k]: rows = q-heads (rows >= G are not used), columns
  // k = 16 wave + col.  Each product of a split term of A with R_hi or R_lo accumulates in its
  // own registers (six independent MFMA chains).
  f32x4 uh[3][2];
#pragma unroll
  for (int t = 0; t < 3; ++t) uh[t][0] = uh[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto unrotate = [&](auto one_) {
    constexpr bool ONE = decltype(one_)::value;  // R_lo^T = 0: one pass
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float v[8];
      const float* src = &ep->amat[col][32 * g + 8 * kb];
      *reinterpret_cast<f32x4*>(v) = *reinterpret_cast<const f32x4*>(src);
      *reinterpret_cast<f32x4*>(v + 4) = *reinterpret_cast<const f32x4*>(src + 4);
      bf16x8 p[3];
      split3_bf16(v, p[0], p[1], p[2]);
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        uh[t][0] = mfma_bf16(p[t], th[kb], uh[t][0]);
        if constexpr (!ONE) uh[t][1] = mfma_bf16(p[t], tl[kb], uh[t][1]);
      }
    }
  };
  if (a.one_pass)  // uniform
    unrotate(std::true_type{});
  else
    unrotate(std::false_type{});
  const f32x4 u = (uh[0][0] + uh[0][1]) + ((uh[1][0] + uh[1][1]) + (uh[2][0] + uh[2][1]));
  if (ngrp == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      if (h >= GC) continue;
      const float L = ep->st[h][1];
      // value centroids enter as c v_scale / sqrt(d)
      const float f = L > 0.f ? INV_SQRT_D * a.v_unscale * a.rot_scale / L : 0.f;
      float* dst;
      if constexpr (PRE) {  // column h: query qgrp QPG + h / G of q-head kvh G + h % G
        const int t = qgrp * QPG + h / G;
        if (t >= a.T_q) continue;
        dst = a.out + (((int64_t)b * Hq + kvh * G + h % G) * a.T_q + t) * D;
      } else {
        dst = a.out + (bh * G + h) * D;
      }
      dst[16 * wave + col] = u[i] * f;
    }
    return;
  }
  // publish the group's unrotated record, then the last group merges the groups
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    if (h >= G) continue;
    float* dst = a.gpart + ((bh * G + h) * ngrp + grp) * PREC;
    __hip_atomic_store(dst + 16 * wave + col, u[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < G) st_dev2(a.gpart + ((bh * G + tid) * ngrp + grp) * PREC + 128, ep->st[tid][0], ep->st[tid][1]);
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    ep->stage = 0;
    if (atomicAdd(cnt_top, 1u) == static_cast<unsigned>(ngrp - 1)) ep->stage = 2;
  }
  __syncthreads();
  if (ep->stage != 2) return;
  for (int h = wave; h < G; h += NW) {
    const Merged r = merge_records(a.gpart + (bh * G + h) * ngrp * PREC, ngrp, lane);
    // value centroids enter as c v_scale / sqrt(d)
    const float f = r.L > 0.f ? INV_SQRT_D * a.v_unscale * a.rot_scale / r.L : 0.f;
    float* o = a.out + (bh * G + h) * D + 2 * lane;  // out is only 4-byte aligned
    o[0] = r.A0 * f;
    o[1] = r.A1 * f;
  }
}

template <int KB, bool QJL, int VB, int G>
hipError_t launch_main(const MainArgs& a, const attn::KeyCent<KB>& kc, int n_slices, int B, bool pre, hipStream_t s,
                       hipEvent_t e0, hipEvent_t e1) {
  static_assert(MainCfg<KB, QJL, VB, G, false>::FITS && MainCfg<KB, QJL, VB, G, true>::FITS, "attention LDS budget");
  static_assert(MainCfg<KB, QJL, VB, (G > 8 ? G : 8), true>::FITS, "prefill LDS budget");
  const bool repl = a.repl != 0;
  auto kern = pre ? attend_kernel<KB, QJL, VB, G, false, true, true>
                  : (a.scores_out != nullptr
                         ? (repl ? attend_kernel<KB, QJL, VB, G, true, false, true>
                                 : attend_kernel<KB, QJL, VB, G, true, false, false>)
                         : (repl ? attend_kernel<KB, QJL, VB, G, false, false, true>
                                 : attend_kernel<KB, QJL, VB, G, false, false, false>));
  // decode: (slices, kv-heads, rows); prefill: (kv-heads x query groups, 1, rows)
  const dim3 grid = pre ? dim3(a.Hkv * a.NG, 1, B) : dim3(n_slices, a.Hkv, B);
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL(kern, grid, dim3(NT), 0, s, e0, e1, 0, a, kc);
  else
    hipLaunchKernelGGL(kern, grid, dim3(NT), 0, s, a, kc);
  return hipGetLastError();
}

template <int KB, bool QJL, int VB>
hipError_t dispatch_g(const MainArgs& a, const attn::KeyCent<KB>& kc, int G, int n_slices, int B, bool pre,
                      hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (G) {
    case 4: return launch_main<KB, QJL, VB, 4>(a, kc, n_slices, B, pre, s, e0, e1);
    case 8: return launch_main<KB, QJL, VB, 8>(a, kc, n_slices, B, pre, s, e0, e1);
    case 16: return launch_main<KB, QJL, VB, 16>(a, kc, n_slices, B, pre, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int KB, bool QJL>
hipError_t dispatch_v(const MainArgs& a, const attn::KeyCent<KB>& kc, int VB, int G, int n_slices, int B, bool pre,
                      hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (VB) {
    case 1: return dispatch_g<KB, QJL, 1>(a, kc, G, n_slices, B, pre, s, e0, e1);
    case 2: return dispatch_g<KB, QJL, 2>(a, kc, G, n_slices, B, pre, s, e0, e1);
    case 3: return dispatch_g<KB, QJL, 3>(a, kc, G, n_slices, B, pre, s, e0, e1);
    case 4: return dispatch_g<KB, QJL, 4>(a, kc, G, n_slices, B, pre, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

// Body of dispatch_k<KB>: the wide key centroids (KB > 4), then the (sketch, value width, group
// size) instance.  Keys without codes need the sketch.
template <int KB>
hipError_t dispatch_width(const MainArgs& a, const float* kcw, bool qjl, int vb, int G, int n_slices, int B, bool pre,
                          hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  attn::KeyCent<KB> kc{};
  if constexpr (KB > 4)
    for (int l = 0; l < (1 << KB); ++l) kc.c[l] = kcw[l];
  if (qjl) return dispatch_v<KB, true>(a, kc, vb, G, n_slices, B, pre, s, e0, e1);
  if constexpr (KB == 0) return hipErrorInvalidValue;
  else return dispatch_v<KB, false>(a, kc, vb, G, n_slices, B, pre, s, e0, e1);
}

}  // namespace
}  // namespace tq
