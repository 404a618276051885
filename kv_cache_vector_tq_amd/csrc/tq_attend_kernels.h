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
  unsigned* cnt_grp;  // [B*Hkv][MAX_GROUPS] arrival counters (zero between calls)
  unsigned* cnt_top;  // [B*Hkv]
  float* out;         // [B*Hq][128]
  float* scores_out;  // NULL or [B*Hq][T_cap]
  int Hkv, T_cap, max_seq_len, blocks_per_wave, n_slices, mgroup;
  float scale_log2;   // scale * log2(e)
  float scale;
  float k_cent[16];   // key centroids times a factor k_scale (table_scale in tq_attend.hip)
  float k_unscale;     // 1 / k_scale
  float v_cent[16];   // value centroids times v_scale
  float v_unscale;     // 1 / v_scale
};

// Launches the attention kernel for key code width KB (k_qjl selects the sign sketch), value
// width vb and group size G; defined in tq_attend_k<KB>.hip.
#define TQ_ATTN_DISPATCH(KB)                                                                       \
  hipError_t dispatch_k##KB(const MainArgs& a, bool qjl, int vb, int G, int n_slices, int B, hipStream_t s, \
                            hipEvent_t e0, hipEvent_t e1)
TQ_ATTN_DISPATCH(0);
TQ_ATTN_DISPATCH(1);
TQ_ATTN_DISPATCH(2);
TQ_ATTN_DISPATCH(3);
TQ_ATTN_DISPATCH(4);

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

// ---- code decoding ------------------------------------------------------------------------
// An 8-code window of a lane's chunk becomes one f16x8 MFMA operand (element e = code at bits
// B*e of the window) through wide LDS lookups (few LDS instructions per code):
//   B = 1 and sign bits: an 8-bit key -> 8 values (16-byte entries, 256 entries);
//   B = 2: an 8-bit key -> 4 codes (8-byte entries, 256 entries);
//   B = 3: a 12-bit key -> 4 codes (8-byte entries, 4096 entries);
//   B = 4: an 8-bit key -> 2 codes (4-byte entries, 256 entries).
// Tables depend only on the bit width (codebooks do), so keys and values of the same width
// share one table.
template <int B>
struct Dec {
  static constexpr int KEYBITS = (B == 3) ? 12 : 8;
  static constexpr int CPL = (B == 1) ? 8 : (B == 4) ? 2 : 4;  // codes per lookup
  static constexpr int EBYTES = 2 * CPL;
  static constexpr int LDS_BYTES = (1 << KEYBITS) * EBYTES;
};
constexpr int SIGN_TABLE_BYTES = 256 * 16;

__device__ __forceinline__ uint32_t pack_f16x2(_Float16 a, _Float16 b) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <int B>
__device__ void build_code_table(uint8_t* tab, const float* cent, int tid) {
  using T = Dec<B>;
  typedef _Float16 entry_t __attribute__((ext_vector_type(T::CPL)));
  _Float16 c16[1 << B];
#pragma unroll
  for (int l = 0; l < (1 << B); ++l) c16[l] = static_cast<_Float16>(cent[l]);
  if constexpr (B == 3) {
    // entry e = tid + 256 k (k < 16) holds codes e & 7, (e >> 3) & 7, (e >> 6) & 7, e >> 9:
    // the first two depend only on the lane (e & 63 = tid & 63), the third is
    // c[w + 4 (k & 1)] for the wave w = tid >> 6, the fourth c[k >> 1]
    const int lane = tid & 63, w = tid >> 6;
    const uint32_t lo = pack_f16x2(c16[lane & 7], c16[(lane >> 3) & 7]);
    const _Float16 x0 = c16[w], x1 = c16[w + 4];
#pragma unroll
    for (int k = 0; k < 16; ++k)
      *reinterpret_cast<u32x2*>(tab + (tid + 256 * k) * 8) = u32x2{lo, pack_f16x2((k & 1) ? x1 : x0, c16[k >> 1])};
    return;
  }
  for (int e = tid; e < (1 << T::KEYBITS); e += 256) {
    entry_t v;
#pragma unroll
    for (int i = 0; i < T::CPL; ++i) v[i] = c16[(e >> (B * i)) & ((1 << B) - 1)];
    *reinterpret_cast<entry_t*>(tab + e * T::EBYTES) = v;
  }
}

__device__ void build_sign_table(uint8_t* tab, int tid) {
  f16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = ((tid >> i) & 1) ? static_cast<_Float16>(1.0f) : static_cast<_Float16>(-1.0f);
  *reinterpret_cast<f16x8*>(tab + tid * 16) = v;
}

// Bits P .. P+N-1 of the little-endian dword array dw, shifted left by S (a byte offset).
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

// The 8 B-bit codes starting at bit P of dw -> f16x8, via the LDS table tab.
template <int B, int P>
__device__ __forceinline__ f16x8 decode8(const uint32_t* dw, const uint8_t* tab) {
  if constexpr (B == 1) {
    return *reinterpret_cast<const f16x8*>(tab + field<P, 8, 4>(dw));
  } else if constexpr (B == 2 || B == 3) {
    constexpr int K = Dec<B>::KEYBITS;
    const u32x2 a = *reinterpret_cast<const u32x2*>(tab + field<P, K, 3>(dw));
    const u32x2 b = *reinterpret_cast<const u32x2*>(tab + field<P + K, K, 3>(dw));
    return __builtin_bit_cast(f16x8, u32x4{a[0], a[1], b[0], b[1]});
  } else {
    return __builtin_bit_cast(f16x8, u32x4{*reinterpret_cast<const uint32_t*>(tab + field<P, 8, 2>(dw)),
                                           *reinterpret_cast<const uint32_t*>(tab + field<P + 8, 8, 2>(dw)),
                                           *reinterpret_cast<const uint32_t*>(tab + field<P + 16, 8, 2>(dw)),
                                           *reinterpret_cast<const uint32_t*>(tab + field<P + 24, 8, 2>(dw))});
  }
}

// 8 sign bits starting at bit P of dw -> f16x8 of +1 / -1.
template <int P>
__device__ __forceinline__ f16x8 decode_signs(const uint32_t* dw, const uint8_t* tab) {
  return *reinterpret_cast<const f16x8*>(tab + field<P, 8, 4>(dw));
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

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
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


template <int KB, bool QJL, int VB, int G>
struct MainCfg {
  static constexpr int TPD = 16 / G;       // score tiles packed into one accumulator set
  static constexpr int NSETS = 4 / TPD;    // accumulator sets per 64-key block
  static constexpr bool SHARED = (KB == VB);  // one table serves keys and values
  static constexpr int KTAB = KB > 0 ? Dec<(KB > 0 ? KB : 1)>::LDS_BYTES : 0;
  static constexpr int STAB = QJL ? SIGN_TABLE_BYTES : 0;
  static constexpr int VTAB = SHARED ? 0 : Dec<VB>::LDS_BYTES;
  static constexpr int TABLES = KTAB + STAB + VTAB;
  // the epilogue reuses the table space once every wave has left the block loop
  static constexpr int MERGE = static_cast<int>(sizeof(Epi));
  // the G query records are staged behind the tables before the block loop (the epilogue,
  // which aliases both, comes after it)
  static constexpr int QSTAGE = G * QREC * 4;
  static constexpr int LDS = TABLES + QSTAGE > MERGE ? TABLES + QSTAGE : MERGE;
};

// Streams the 64-key blocks of one slice.  SCORES: also write the logits (parity runs).
template <int KB, bool QJL, int VB, int G, bool SCORES>
__global__ void __launch_bounds__(NT, 1) attend_kernel(MainArgs a) {
  using C = MainCfg<KB, QJL, VB, G>;
  constexpr int TPD = C::TPD, NSETS = C::NSETS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  uint8_t* ktab = smem;
  uint8_t* stab = smem + C::KTAB;
  uint8_t* vtab = C::SHARED ? smem : smem + C::KTAB + C::STAB;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int tcls = col / G;   // which tile of a set this lane's column belongs to
  const int hh = col % G;     // q-head within the group
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int Hq = a.Hkv * G;
  const int64_t bh = (int64_t)b * a.Hkv + kvh;
  const int nblk_cap = a.T_cap / 64;

  int seq = a.seq_len[b];
  seq = seq < 1 ? 1 : (seq > a.max_seq_len ? a.max_seq_len : seq);
  const int nblk = (seq + 63) / 64;
  const int slice = blockIdx.x * NW + wave;
  const int blk_begin = slice * a.blocks_per_wave;
  const int blk_end = min(blk_begin + a.blocks_per_wave, nblk);

  // online softmax per lane column: m_run (log2 domain), l_run = sum 2^(lg - m_run);
  // acc = sum P' V with P' = 2^(lg - m_run) nv / s_run and s_run >= every such product
  float m_run = NEG_BIG, l_run = 0.f, s_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Block data of one lane.  Codes of the next block are loaded while the current one is
  // processed; the norms of the current block are loaded at its start (they are first needed
  // after the score MFMAs).
  struct Blk {
    uint32_t kd[KB > 0 ? 4 * KB : 1];
    uint32_t sd[4];
    uint32_t vd[4 * VB];
  };
  auto load_block = [&](int blk, Blk& d) {
    if constexpr (KB > 0)
      load_dwords<4 * KB>(d.kd, a.k_codes + (bh * nblk_cap + blk) * (1024 * KB) + lane * 16 * KB);
    if constexpr (QJL) load_dwords<4>(d.sd, a.k_signs + (bh * nblk_cap + blk) * 1024 + lane * 16);
    load_dwords<4 * VB>(d.vd, a.v_codes + (bh * nblk_cap + blk) * (1024 * VB) + lane * 16 * VB);
  };
  struct Norms {
    f32x4 kn[NSETS], kr[NSETS], vn[NSETS];
  };
  auto load_norms = [&](int blk, Norms& d) {
#pragma unroll
    for (int s = 0; s < NSETS; ++s) {
      const int64_t tok = bh * a.T_cap + blk * 64 + 16 * (s * TPD + tcls) + 4 * g;
      d.kn[s] = *reinterpret_cast<const f32x4*>(a.k_norm + tok);
      if constexpr (QJL && KB > 0) d.kr[s] = *reinterpret_cast<const f32x4*>(a.k_rnorm + tok);
      d.vn[s] = *reinterpret_cast<const f32x4*>(a.v_norm + tok);
    }
  };
  // score operands from the prologue's record of head hh: lane (col, g) holds
  // q[hh][32 g + 8 kb + e] of every k-block kb as two f16 terms (hi + lo, the fp32 value to
  // about 22 bits), scaled by 2^-e with e the exponent of the vector's largest magnitude (the
  // 4 lanes of a column hold the 128 coordinates).  One f16 term alone leaves a relative
  // error of 2^-12 per coordinate, which large logits carry into the softmax weights.
  // logit * log2(e) = n (code_acc * c1 + rnorm * sign_acc * c2): the table holds centroids c,
  // the key term is q1 . c / sqrt(d), the sign term carries sqrt(pi/2)/m.
  // The G query records of this kv-head (contiguous) go through LDS: one 16-byte load per
  // thread (two for G = 16), issued before the block loads, so that no wave's query waits
  // behind other waves' block loads.
  constexpr int QWORDS = G * QREC / 4;
  constexpr int QPT = (QWORDS + NT - 1) / NT;
  float* const qst = reinterpret_cast<float*>(smem + C::TABLES);
  f32x4 qw[QPT];
  {
    const float* qsrc = a.qrec + ((int64_t)b * Hq + kvh * G) * QREC;
#pragma unroll
    for (int k = 0; k < QPT; ++k) qw[k] = *reinterpret_cast<const f32x4*>(qsrc + 4 * min(tid + k * NT, QWORDS - 1));
  }
  // Block loads are unconditional, from clamped (always in-bounds) block indices: a load under
  // a branch would make the compiler wait for every load in flight where the branches join,
  // which would serialize the prefetch with the current block's compute.
  Blk cur, nxt;
  load_block(min(blk_begin, nblk_cap - 1), cur);  // in flight while the tables are built

  if (wave < 4) {  // the table builders take 256 threads
    if constexpr (KB > 0) build_code_table<(KB > 0 ? KB : 1)>(ktab, a.k_cent, tid);
    if constexpr (QJL) build_sign_table(stab, tid);
    if constexpr (!C::SHARED) build_code_table<VB>(vtab, a.v_cent, tid);
  }
#pragma unroll
  for (int k = 0; k < QPT; ++k)
    if (tid + k * NT < QWORDS) *reinterpret_cast<f32x4*>(qst + 4 * (tid + k * NT)) = qw[k];
  __syncthreads();  // tables and query records ready
  f16x8 bq[4], bs[4], bql[4], bsl[4];
  float c1, c2;
  {
    f32x4 qv1[8], qv2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qv1[i] = *reinterpret_cast<const f32x4*>(qst + hh * QREC + 32 * g + 4 * i);
      qv2[i] = QJL ? *reinterpret_cast<const f32x4*>(qst + hh * QREC + D + 32 * g + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
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
    auto lo16 = [](float x, _Float16 hi) { return static_cast<_Float16>(x - static_cast<float>(hi)); };
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x1 = qv1[2 * kb + j / 4][j % 4] * s1, x2 = qv2[2 * kb + j / 4][j % 4] * s2;
        const _Float16 h1 = static_cast<_Float16>(x1), h2 = static_cast<_Float16>(x2);
        bq[kb][j] = h1;
        bql[kb][j] = lo16(x1, h1);
        bs[kb][j] = h2;
        bsl[kb][j] = lo16(x2, h2);
      }
    const float lscale = a.scale * LOG2E;
    c1 = ldexpf(1.0f, e1) * INV_SQRT_D * lscale * a.k_unscale;
    c2 = ldexpf(1.0f, e2) * KAPPA * lscale;
  }

  for (int blk = blk_begin; blk < blk_end; ++blk) {
    Norms nrm;
    load_norms(blk, nrm);
    load_block(min(blk + 1, blk_end - 1), nxt);

    // ---- score MFMAs: tile t = keys 16 t .. 16 t + 15 of the block; each lane keeps the
    // tile of its column class in every set (tile s TPD + tcls of set s) ----------------------
    f32x4 cs[NSETS], ss[NSETS];
    static_for<0, 4>([&](auto T_) {
      constexpr int t = decltype(T_)::value;
      f32x4 dc = f32x4{0.f, 0.f, 0.f, 0.f}, ds = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 dcl = f32x4{0.f, 0.f, 0.f, 0.f}, dsl = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KB > 0) {
        static_for<0, 4>([&](auto KB_) {
          constexpr int kb = decltype(KB_)::value;
          const f16x8 ak = decode8<KB, 32 * KB * t + 8 * KB * kb>(cur.kd, ktab);
          dc = mfma_f16(ak, bq[kb], dc);
          dcl = mfma_f16(ak, bql[kb], dcl);
        });
      }
      if constexpr (QJL) {
        static_for<0, 4>([&](auto KB_) {
          constexpr int kb = decltype(KB_)::value;
          const f16x8 as = decode_signs<32 * t + 8 * kb>(cur.sd, stab);
          ds = mfma_f16(as, bs[kb], ds);
          dsl = mfma_f16(as, bsl[kb], dsl);
        });
      }
      dc += dcl;
      ds += dsl;
      constexpr int st_ = t / TPD, ct = t % TPD;
      if constexpr (ct == 0) {
        cs[st_] = dc;
        ss[st_] = ds;
      } else {
        if (tcls == ct) {
          cs[st_] = dc;
          ss[st_] = ds;
        }
      }
    });

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
        float est = 0.f;
        if constexpr (KB > 0) est = cs[s][i] * c1;
        if constexpr (QJL) est = fmaf((KB > 0 ? nrm.kr[s][i] : 1.0f) * ss[s][i], c2, est);
        const float l2 = nrm.kn[s][i] * est;
        const bool valid = key < seq;
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
    const float m_new = fmaxf(m_run, mb);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float s_scaled = s_run * alpha;
    const float s_new = fmaxf(s_scaled, __builtin_amdgcn_exp2f(mvb - m_new));
    const float inv = s_new > 0.f ? __builtin_amdgcn_rcpf(s_new) : 0.f;
    const float f = s_new > 0.f ? s_scaled * inv : 1.0f;
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
        x[i] = pr > 0.f ? fminf(pr * nrm.vn[s][i] * inv, 1.0f) : 0.f;
      }
      pw[s][0] = pack_f16x2(static_cast<_Float16>(x[0]), static_cast<_Float16>(x[1]));
      pw[s][1] = pack_f16x2(static_cast<_Float16>(x[2]), static_cast<_Float16>(x[3]));
    }
    m_run = m_new;
    s_run = s_new;
    l_run = fmaf(l_run, alpha, lsum);

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
        const f16x8 av = decode8<VB, 8 * VB * (2 * mt + kb2)>(cur.vd, vtab);
        acc[mt] = mfma_f16(av, bp, acc[mt]);
      });
    });
    cur = nxt;
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
  // record r = 16 w + c G + h belongs to q-head h; wave 0 finds each head's maximum and the
  // record weights over the lanes with the same h (xor offsets that keep r mod G)
  if (tid < 64) {
    const float* rec = ep->rec[tid];
    const float m = rec[128];
    float M = m;
#pragma unroll
    for (int o = G; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float e = exp2f(m - M);
    ep->w64[tid] = rec[130] * e;
    float l = rec[129] * e;
#pragma unroll
    for (int o = G; o < 64; o <<= 1) l += __shfl_xor(l, o);
    if (tid < G) st_dev2(a.part + ((bh * G + tid) * a.n_slices + blockIdx.x) * PREC + 128, M, l);
  }
  __syncthreads();
  for (int idx = tid; idx < G * D / 2; idx += NT) {
    const int h = idx / (D / 2), j = 2 * (idx % (D / 2));
    float A0 = 0.f, A1 = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int c = 0; c < TPD; ++c) {
        const int r = 16 * w + c * G + h;
        A0 = fmaf(ep->rec[r][j], ep->w64[r], A0);
        A1 = fmaf(ep->rec[r][j + 1], ep->w64[r], A1);
      }
    st_dev2(a.part + ((bh * G + h) * a.n_slices + blockIdx.x) * PREC + j, A0, A1);
  }

  // ---- merge over the slices: the last workgroup of each group of MGROUP slices merges the
  // group and applies R_eff^T, the last group merger merges the groups ---------------------
  const int ns = a.n_slices;
  const int mgroup = a.mgroup;
  const int ngrp = (ns + mgroup - 1) / mgroup;
  const int grp = blockIdx.x / mgroup;
  drain_stores();
  __syncthreads();
  if (tid == 0) {
    // the last arrival resets its counter, so counters are zero again after every call
    int stage = 0;
    unsigned* cnt = ngrp == 1 ? a.cnt_top + bh : a.cnt_grp + bh * MAX_GROUPS + grp;
    const unsigned last = ngrp == 1 ? ns - 1 : min(mgroup, ns - mgroup * grp) - 1;
    if (atomicAdd(cnt, 1u) == last) {
      __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      stage = ngrp == 1 ? 2 : 1;
    }
    ep->stage = stage;
  }
  __syncthreads();
  if (ep->stage == 0) return;
  // This workgroup merges: it applies R_eff^T to what it merged (the unrotation is linear, so
  // merging unrotated group results is the same as unrotating the merge).  Merge the slices of
  // this group (or all slices with a single group) into ep->amat, ep->st; wave w takes q-heads
  // w, w + 4, ...
  {
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
      uh[t][1] = mfma_bf16(p[t], tl[kb], uh[t][1]);
    }
  }
  const f32x4 u = (uh[0][0] + uh[0][1]) + ((uh[1][0] + uh[1][1]) + (uh[2][0] + uh[2][1]));
  if (ngrp == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      if (h >= G) continue;
      const float L = ep->st[h][1];
      // value centroids enter as c v_scale / sqrt(d)
      const float f = L > 0.f ? INV_SQRT_D * a.v_unscale / L : 0.f;
      a.out[(bh * G + h) * D + 16 * wave + col] = u[i] * f;
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
    if (atomicAdd(a.cnt_top + bh, 1u) == static_cast<unsigned>(ngrp - 1)) {
      __hip_atomic_store(a.cnt_top + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ep->stage = 2;
    }
  }
  __syncthreads();
  if (ep->stage != 2) return;
  for (int h = wave; h < G; h += NW) {
    const Merged r = merge_records(a.gpart + (bh * G + h) * ngrp * PREC, ngrp, lane);
    // value centroids enter as c v_scale / sqrt(d)
    const float f = r.L > 0.f ? INV_SQRT_D * a.v_unscale / r.L : 0.f;
    float* o = a.out + (bh * G + h) * D + 2 * lane;  // out is only 4-byte aligned
    o[0] = r.A0 * f;
    o[1] = r.A1 * f;
  }
}

template <int KB, bool QJL, int VB, int G>
hipError_t launch_main(const MainArgs& a, int n_slices, int B, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  using C = MainCfg<KB, QJL, VB, G>;
  static_assert(C::LDS <= 65536, "attention LDS budget");
  auto kern = a.scores_out != nullptr ? attend_kernel<KB, QJL, VB, G, true> : attend_kernel<KB, QJL, VB, G, false>;
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL(kern, dim3(n_slices, a.Hkv, B), dim3(NT), 0, s, e0, e1, 0, a);
  else
    hipLaunchKernelGGL(kern, dim3(n_slices, a.Hkv, B), dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int KB, bool QJL, int VB>
hipError_t dispatch_g(const MainArgs& a, int G, int n_slices, int B, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  switch (G) {
    case 4: return launch_main<KB, QJL, VB, 4>(a, n_slices, B, s, e0, e1);
    case 8: return launch_main<KB, QJL, VB, 8>(a, n_slices, B, s, e0, e1);
    case 16: return launch_main<KB, QJL, VB, 16>(a, n_slices, B, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int KB, bool QJL>
hipError_t dispatch_v(const MainArgs& a, int VB, int G, int n_slices, int B, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1) {
  switch (VB) {
    case 1: return dispatch_g<KB, QJL, 1>(a, G, n_slices, B, s, e0, e1);
    case 2: return dispatch_g<KB, QJL, 2>(a, G, n_slices, B, s, e0, e1);
    case 3: return dispatch_g<KB, QJL, 3>(a, G, n_slices, B, s, e0, e1);
    case 4: return dispatch_g<KB, QJL, 4>(a, G, n_slices, B, s, e0, e1);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tq
