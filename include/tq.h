/*
 * tq.h - C ABI of the TurboQuant compressed KV-cache hot path for MI355X (gfx950).
 *
 * What the calls compute (sources are web pages on TurboQuant; cited by title and section):
 *  - "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru overview): each
 *    key/value vector is multiplied by a random orthogonal matrix, each rotated coordinate
 *    is quantized with a Lloyd-Max codebook computed once for the (near-normal) post-rotation
 *    law, with no per-group scales and no calibration data, and the residual gets a 1-bit
 *    QJL correction.
 *  - "Google TurboQuant простыми словами" (tproger.ru), section "Как работает TurboQuant",
 *    step 2: QJL is a Johnson-Lindenstrauss projection of the residual that keeps one sign
 *    bit per projected coordinate and removes the bias of the inner-product estimate.
 *    Section "Бенчмарки TurboQuant", list "Из независимых реализаций": 52 bytes per 128
 *    values at 3 bits (48 bytes of codes plus a 4-byte side value).
 *  - "KV cache benchmark Qwen 3.6-35B-A3B" (ai-manual.ru), section "Неочевидный совет":
 *    decode over a long context is bound by memory bandwidth, so attention reads the
 *    compressed cache directly.
 *
 * Conventions for every call:
 *  - d (head dimension) is 128; the sketch has m = d rows.
 *  - Device pointers are plain HIP device addresses; host pointers are ordinary memory.
 *  - The library never allocates or frees device memory and never synchronizes: kernels
 *    are enqueued on the caller's stream (hip_stream, a hipStream_t; NULL = default
 *    stream) and results are valid once that stream has been synchronized.
 *  - Return value 0 (TQ_OK) or a negative TQ_ERR_* code.  Every argument check runs on the
 *    host before any launch; tq_last_error() then describes the failure (thread-local).
 *  - Non-finite inputs give unspecified codes; they are not checked.
 *
 * State the library keeps between calls (everything else lives in caller-owned memory):
 *  - per thread: the last error text (tq_last_error) and the timing-hook events
 *    (tq_profile_events);
 *  - per process, read-only after first use and guarded by a mutex: the compute-unit count of
 *    each device, the f16 table factor of each codebook (a pure function of its levels), and
 *    the environment knobs TQ_ATTN_MIN_BLOCKS / TQ_ATTN_MGROUP (read once; they change only the
 *    context split of tq_attend_decode); TQ_ATTN_REPL is read at every tq_attend_decode call;
 *  - per device: the fixed scratch array of tq_attend_decode_noalloc.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 4
#define TQ_MAX_K_LEVELS 256 /* key codes of up to 8 bits */
#define TQ_HEAD_DIM 128
#define TQ_BLOCK_TOKENS 64

enum {
  TQ_OK = 0,
  TQ_ERR_INVALID = -1,     /* NULL / misaligned pointer, bad shape, bad size */
  TQ_ERR_UNSUPPORTED = -2, /* d != 128, bit width or group size not supported */
  TQ_ERR_WORKSPACE = -3,   /* workspace too small; required size written back */
  TQ_ERR_DEVICE = -4       /* HIP runtime error at launch */
};

typedef enum { TQ_DTYPE_BF16 = 0, TQ_DTYPE_F32 = 1 } tq_dtype;

/* Rotation modes (tq_config.rotation). */
#define TQ_ROTATION_HAAR 0     /* seeded Haar-random orthogonal matrix */
#define TQ_ROTATION_HADAMARD 1 /* randomized Walsh-Hadamard: H diag(s) / sqrt(d) */

/* Cache configuration.  k_bits: scalar code bits per key coordinate (0..8; 0 = keys keep
 * only the sign sketch); k_qjl: 1 = keys carry the 1-bit sign sketch of their residual;
 * v_bits: value code bits (1..4); rotation: TQ_ROTATION_*; seed: fixes the rotation and the
 * sketch.  Presets: turbo2 = (1, 1, 2), turbo3 = (2, 1, 3), turbo4 = (3, 1, 4), sign-only
 * keys = (0, 1, 3); keys wider than values, e.g. K8V4 = (8, 0, 4) (overview page, paragraph on
 * K/V asymmetry: keys need more bits than values). */
typedef struct tq_config {
  int32_t d;
  int32_t k_bits;
  int32_t k_qjl;
  int32_t v_bits;
  int32_t rotation;
  uint64_t seed;
} tq_config;

/* Static Lloyd-Max tables for N(0,1), stored as fp32 copies of fp64 values: 2^bits levels
 * (ascending) and 2^bits - 1 decision thresholds (midpoints); entries past those are 0.  A
 * coordinate z of the rotated, sqrt(d)-scaled unit vector gets code #{l : z >= threshold[l]}.
 * *_mse is the fp64 Gaussian distortion of the table.  The tables are the fixed point of
 * Lloyd's conditions (levels = conditional means of their cells, thresholds = midpoints),
 * found by Lloyd's iteration and, for codes of 5 bits and more, finished by Newton's method
 * on the same equations. */
typedef struct tq_codebook {
  tq_config cfg;
  float k_centroids[TQ_MAX_K_LEVELS];
  float k_thresholds[TQ_MAX_K_LEVELS];
  float v_centroids[16];
  float v_thresholds[16];
  double k_mse;
  double v_mse;
} tq_codebook;

/* Parameter matrices, row-major d x d, bf16 bit patterns, all derived from cfg->seed:
 *   r_hi, r_lo    the rotation: R_eff = r_hi + r_lo (Haar mode) or r_hi / sqrt(128) with
 *                 r_lo = 0 (Hadamard mode); y = R_eff x;
 *   s_qjl         the sketch S_b (u = S_b r);
 *   rt_hi, rt_lo  r_hi and r_lo transposed (the unrotation R_eff^T of attention outputs);
 *   m_hi, m_lo    M = S_b R_eff (exact product, then m_hi = bf16(M), m_lo = bf16(M - m_hi)):
 *                 a query's sketch coordinates S_b (R_eff q) in one product.
 * tq_host_params: caller-allocated host buffers of 16384 uint16 each (any may be NULL to
 * skip it).  tq_dev_params: device copies (16-byte aligned).  s_qjl, m_hi and m_lo may be NULL
 * when keys carry no sketch; rt_hi, rt_lo, m_hi and m_lo are read only by tq_attend_decode. */
typedef struct tq_host_params {
  uint16_t* r_hi;
  uint16_t* r_lo;
  uint16_t* s_qjl;
  uint16_t* rt_hi;
  uint16_t* rt_lo;
  uint16_t* m_hi;
  uint16_t* m_lo;
} tq_host_params;

typedef struct tq_dev_params {
  const uint16_t* r_hi;
  const uint16_t* r_lo;
  const uint16_t* s_qjl;
  const uint16_t* rt_hi;
  const uint16_t* rt_lo;
  const uint16_t* m_hi;
  const uint16_t* m_lo;
} tq_dev_params;

/* Packed cache of B batch rows x Hkv kv-heads x T_cap token slots (T_cap a multiple of 64).
 * All arrays are device memory owned by the caller, contiguous, 16-byte aligned:
 *   k_codes [B][Hkv][T_cap/64][1024*k_bits] bytes   (NULL when k_bits == 0)
 *   k_signs [B][Hkv][T_cap/64][1024] bytes           (NULL when k_qjl == 0)
 *   k_norm  [B][Hkv][T_cap] fp32  key norms ||x||
 *   k_rnorm [B][Hkv][T_cap] fp32  residual norms    (NULL unless k_qjl && k_bits > 0)
 *   v_codes [B][Hkv][T_cap/64][1024*v_bits] bytes
 *   v_norm  [B][Hkv][T_cap] fp32  value norms
 * Inside a 64-token block the bits follow this fixed arrangement (64 chunks; chunk L has
 * c = L % 16, g = L / 16; bit k is bit k % 8 of byte k / 8):
 *   key codes (b bits, 1..8): chunk L = 16 b bytes holds tokens 16 t + c (t = 0..3) and
 *     coordinates 32 g + j (j = 0..31); code (t, j) starts at bit 32 b t + b j.
 *   sign bits: chunk L = 16 bytes; bit 32 t + j is the sign of sketch row 32 g + j of
 *     token 16 t + c.
 *   value codes (b bits): chunk L = 16 b bytes holds coordinates 16 mt + c (mt = 0..7) of
 *     tokens 16 t + 4 g + r (t, r = 0..3); code (mt, t, r) starts at bit 4 b (4 mt + t) + b r.
 * Slots never written hold whatever the memory held; attention reads only slots below
 * seq_len. */
typedef struct tq_kv_cache {
  uint8_t* k_codes;
  uint8_t* k_signs;
  float* k_norm;
  float* k_rnorm;
  uint8_t* v_codes;
  float* v_norm;
  int32_t B;
  int32_t Hkv;
  int32_t T_cap;
} tq_kv_cache;

/* Byte sizes of the arrays of tq_kv_cache for a configuration (0 for arrays not used). */
typedef struct tq_cache_sizes {
  size_t k_codes;
  size_t k_signs;
  size_t k_norm;
  size_t k_rnorm;
  size_t v_codes;
  size_t v_norm;
  size_t bytes_per_token; /* stored bytes per token and kv-head, all arrays */
} tq_cache_sizes;

/* One-time parameter build, host only, deterministic in cfg->seed ("Когда в марте 2026 года
 * Google опубликовала статью...": a random orthogonal rotation, and a Lloyd-Max codebook computed
 * once for the near-normal rotated coordinates; "Google TurboQuant простыми словами", section "Как
 * работает TurboQuant", step 2: a Gaussian Johnson-Lindenstrauss projection for the sign bits).
 * Fills *cb with the key and value codebooks (Lloyd-Max fixed point for N(0,1)) and, when
 * out is not NULL, the parameter matrices of tq_host_params:
 *   Haar mode: G = 128x128 N(0,1) from SplitMix64 started at state 2*seed (Box-Muller,
 *     row-major); R = Q diag(sign U_ii) from the Householder QR G = Q U;
 *   Hadamard mode (the Hadamard-transform speed-up named in "Google TurboQuant простыми
 *     словами", section on TurboQuant in llama.cpp): R = H diag(s) / sqrt(128) with
 *     H_ij = (-1)^popcount(i & j) and s_j = -1 when the top bit of the j-th output of the
 *     stream started at 2*seed is set, else +1;
 *   Haar mode: R_hi = bf16(R), R_lo = bf16(R - R_hi), bf16() = round to fp32 then to bf16, ties
 *     to even, and the applied rotation is R_eff = R_hi + R_lo;
 *   Hadamard mode: R_hi = H diag(s) (entries +-1, exact in bf16), R_lo = 0, and the applied
 *     rotation is R_eff = R = R_hi / sqrt(128) exactly: the kernels apply one bf16 product pass
 *     instead of two and fold 1/sqrt(128) into their fp32 scales;
 *   S_b = bf16(S), S = 128x128 N(0,1) from the stream started at 2*seed + 1.
 * Errors: TQ_ERR_INVALID (NULL cfg/cb), TQ_ERR_UNSUPPORTED (d != 128, k_bits outside 0..8,
 * v_bits outside 1..4, k_qjl not 0/1, k_bits == 0 with k_qjl == 0, or an unknown rotation). */
int tq_build_codebook(const tq_config* cfg, tq_codebook* cb, tq_host_params* out);

/* Sizes of the cache arrays for B x Hkv x T_cap slots (T_cap a positive multiple of 64).
 * Errors: TQ_ERR_INVALID (bad sizes / NULL), TQ_ERR_UNSUPPORTED (bad config). */
int tq_cache_layout(const tq_config* cfg, int B, int Hkv, int T_cap, tq_cache_sizes* out);

/* Quantize-on-write of n_new tokens per (batch row, kv-head) into the packed cache
 * ("Когда в марте 2026 года Google опубликовала статью...": rotate, quantize every coordinate
 * with the stored codebook, correct the residual with one QJL bit; "Google TurboQuant простыми
 * словами", step 2: one sign bit per projected residual coordinate; section "Бенчмарки
 * TurboQuant", list "Из независимых реализаций": one 4-byte side value per 128 values).
 * k, v: device inputs, element (b, h, t, j) at offset b*stride_b + h*stride_h + t*stride_t + j
 *   (strides in elements; the 128 coordinates of a vector are contiguous); dtype in_dtype.
 *   Either may be NULL to write only keys or only values.
 * start_pos: device int32 [B]; token t of row b goes to slot start_pos[b] + t.  Slots at or
 *   beyond T_cap are skipped, and a negative start_pos[b] skips row b (the positions live in
 *   device memory, so they are not checked on the host).  n_new = 1 is the per-step append, n_new = T the bulk (prefill) fill.
 * Per vector x: n = ||x||, y = R_eff x / n, z = sqrt(d) y, code = #{l : z >= threshold[l]};
 *   keys with the sketch: r = y - c[code]/sqrt(d) (r = y when k_bits == 0), stored residual
 *   norm ||r||, sign bits [S_b r >= 0].  A zero vector gets code 2^(b-1), residual norm 0,
 *   all sign bits 1.
 * Errors: TQ_ERR_INVALID (NULL cb/p/cache/start_pos, both k and v NULL, B/Hkv mismatch with
 *   the cache, n_new < 1, misaligned input, bad strides), TQ_ERR_UNSUPPORTED (config),
 *   TQ_ERR_DEVICE (launch failure). */
int tq_quantize_kv(const tq_codebook* cb, const tq_dev_params* p, const void* k, const void* v,
                   tq_dtype in_dtype, int B, int Hkv, int n_new, int64_t stride_b,
                   int64_t stride_h, int64_t stride_t, const int32_t* start_pos,
                   const tq_kv_cache* cache, void* hip_stream);

/* One decode step of attention for all (batch row, q-head) straight from the packed cache
 * ("Когда в марте 2026 года Google опубликовала статью...": attention is computed from the
 * compressed keys, with the 1-bit correction carried into the scores; "Google TurboQuant
 * простыми словами", step 2: the sign term makes the inner-product estimate unbiased; "KV cache
 * benchmark Qwen 3.6-35B-A3B", section "Неочевидный совет": decode is bound by memory bandwidth,
 * so the codes are read once, directly).
 * q: device [B][Hq][128] in q_dtype.  q-head h reads kv-head h / (Hq / Hkv); Hq / Hkv must
 *   be 4, 8 or 16.  Every configuration tq_build_codebook accepts is supported (keys of 0..8
 *   code bits with or without the sign sketch, values of 1..4 bits).
 * seq_len: device int32 [B], keys 0 .. seq_len[b]-1 are attended (1 <= seq_len[b] <= max_seq_len;
 *   values outside that range are clamped into it on the device).
 * max_seq_len: host bound on seq_len (<= T_cap); sizes the split of the context.
 * scale: logit scale; 0 selects 1/sqrt(128).
 * For q-head h: q1 = R_eff q, q2 = S_b q1; for key i
 *   score_i = n_i (sum_j q1_j c[code_ij]/sqrt(d) + rnorm_i sqrt(pi/2)/m sum_j q2_j (2 sign_ij - 1))
 *   (rnorm = 1 when k_bits == 0); p = softmax(scale * score);
 *   out = R_eff^T sum_i p_i nv_i cv[codev_i]/sqrt(d)   (fp32 [B][Hq][128]).
 * scores_out: NULL or device fp32 [B][Hq][T_cap]; receives scale * score_i for i < seq_len[b].
 * workspace: device scratch of *workspace_bytes bytes (256-byte aligned), owned by the caller.
 *   Call with workspace == NULL to get the required size in *workspace_bytes (returns TQ_OK).
 *   It needs no initial contents: every call first sets the arrival counters it keeps there
 *   to zero (in its query-rotation launch), so a workspace can be reused across calls of any
 *   shape, also after an earlier call that did not finish.  Calls that share a workspace must
 *   not run concurrently (same stream, or otherwise ordered).
 * Environment (read once per process; both change the split, and so the workspace size and
 *   the fp32 summation order, not the result's bound): TQ_ATTN_MIN_BLOCKS (default 2) is the
 *   smallest number of 64-key blocks a wave streams when the context is split over
 *   workgroups; TQ_ATTN_MGROUP (default 16, at most 32) is the number of context slices a
 *   first-level merge combines.  TQ_ATTN_REPL (read at every call) selects the kernel instance
 *   that keeps one copy of each 8-bit-key decode table per lane slot in LDS: 1 always, 0
 *   never, unset when each wave streams at least 8 blocks.  The outputs are bit-identical
 *   either way.
 * Errors: TQ_ERR_INVALID (NULL arguments, Hq not a multiple of Hkv, max_seq_len outside
 *   1..T_cap), TQ_ERR_UNSUPPORTED (group size or config), TQ_ERR_WORKSPACE (too small;
 *   required size written to *workspace_bytes), TQ_ERR_DEVICE (launch failure). */
int tq_attend_decode(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                     const void* q, tq_dtype q_dtype, int Hq, const int32_t* seq_len,
                     int max_seq_len, float scale, float* out, float* scores_out,
                     void* workspace, size_t* workspace_bytes, void* hip_stream);

/* One decode step of a layer in two launches (the calls above, per generated token):
 * quantize-on-write of one new token per
 * (batch row, kv-head) exactly as tq_quantize_kv with n_new = 1 (k, v, kv_dtype, strides and
 * start_pos as there; the token is at offset b*kv_stride_b + h*kv_stride_h), then attention
 * exactly as tq_attend_decode.  The query rotation that tq_attend_decode launches on its own
 * runs here inside the quantize launch (the two share no data), so a step costs one launch
 * less.  seq_len must count the new token.  Workspace, outputs and errors as tq_attend_decode
 * (a workspace query, workspace == NULL, launches nothing); the append's argument errors are
 * those of tq_quantize_kv, also detected before any launch. */
int tq_decode_step(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                   const void* k, const void* v, tq_dtype kv_dtype, int64_t kv_stride_b,
                   int64_t kv_stride_h, const int32_t* start_pos, const void* q, tq_dtype q_dtype,
                   int Hq, const int32_t* seq_len, int max_seq_len, float scale, float* out,
                   float* scores_out, void* workspace, size_t* workspace_bytes, void* hip_stream);

/* Prefill attention: causal attention of a prompt's queries straight from the packed cache
 * (pages: "Когда в марте 2026 года Google опубликовала статью...", paragraph "Теперь про цифры",
 * quantization overhead at prefill; "Google TurboQuant простыми словами", section "Как
 * попробовать TurboQuant прямо сейчас", prefill throughput with the compressed cache).  The
 * prompt's keys and values are first written with tq_quantize_kv; then query t of row b, at
 * position q_start[b] + t, attends keys 0 .. q_start[b] + t with the score, softmax and value sum
 * of tq_attend_decode (keys at positions >= max_seq_len are never read: limits are clamped to it).
 * q: device [B][Hq][T_q][128] in q_dtype, contiguous, 16-byte aligned; q-head h reads kv-head
 *   h / (Hq / Hkv), Hq / Hkv in {4, 8, 16}.
 * q_start: device int32 [B] (negative values count as 0).
 * max_seq_len: host bound (1 .. T_cap) on q_start[b] + T_q.
 * scale: logit scale; 0 selects 1/sqrt(128).
 * out: device fp32 [B][Hq][T_q][128] (4-byte aligned).
 * One launch; no workspace: each workgroup takes max(8, G) / G consecutive queries of all G q-heads
 * of a kv-head, rotates them itself and writes their outputs.
 * Errors: TQ_ERR_INVALID (NULL or misaligned arguments, bad shapes), TQ_ERR_UNSUPPORTED (group size,
 *   config or dtype), TQ_ERR_DEVICE (launch failure). */
int tq_attend_prefill(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache, const void* q,
                      tq_dtype q_dtype, int Hq, int T_q, const int32_t* q_start, int max_seq_len, float scale,
                      float* out, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): tq_attend_decode with its workspace taken from a
 * fixed array of TQ_NOALLOC_SCRATCH_BYTES bytes of device memory that the library holds, one per
 * GPU it runs on, until the process ends.  Arguments, outputs and errors as tq_attend_decode
 * without workspace / workspace_bytes; it calls no allocating routine.  A call whose workspace
 * would exceed TQ_NOALLOC_SCRATCH_BYTES fails with TQ_ERR_WORKSPACE before any launch (the
 * workspace grows with B * Hq and with the context split; B * Hq up to about 8192 fits).  Every
 * call on one GPU shares that GPU's array and leaves its contents there; each call first sets
 * what must start at zero (the arrival counters).  Calls that overlap on one GPU (different
 * streams, or threads without ordering) race on the array and give undefined results. */
#define TQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int tq_attend_decode_noalloc(const tq_codebook* cb, const tq_dev_params* p, const tq_kv_cache* cache,
                             const void* q, tq_dtype q_dtype, int Hq, const int32_t* seq_len, int max_seq_len,
                             float scale, float* out, float* scores_out, void* hip_stream);

/* Baseline for comparison: uncompressed bf16 decode attention at the same shapes (not part of
 * the compressed path).  p = softmax(scale * K q) (scale 0 selects 1/sqrt(128)),
 * out = sum_i p_i V_i, fp32 accumulation, for all (batch row, q-head); q-head h reads kv-head
 * h / (Hq / Hkv), Hq / Hkv in {4, 8, 16}; keys 0 .. seq_len[b]-1 (clamped into 1..max_seq_len).
 * k: device bf16 [B][Hkv][T_cap][128]; vt: device bf16 [B][Hkv][T_cap/32][128][32], V
 * transposed per 32-key chunk, slot 8 g + e of a coordinate row holding key
 * 16 (e / 4) + 4 g + e % 4 of the chunk; q: device bf16 [B][Hq][128]; out: fp32 [B][Hq][128].
 * T_cap a positive multiple of 32; k, vt, q 16-byte aligned.  workspace: device scratch of
 * *workspace_bytes bytes (query with workspace == NULL); no initial contents needed.
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED (group size), TQ_ERR_WORKSPACE, TQ_ERR_DEVICE. */
int tq_bf16_attend_decode(const void* k, const void* vt, int B, int Hkv, int T_cap, const void* q, int Hq,
                          const int32_t* seq_len, int max_seq_len, float scale, float* out, void* workspace,
                          size_t* workspace_bytes, void* hip_stream);

/* Diagnostic timing hook (for benchmarks): events (hipEvent_t, created by the caller) that
 * later calls on this thread record on their stream, attend_* immediately before and after
 * the main attention kernel of tq_attend_decode (scores, softmax, value sums, merge over
 * context slices and unrotation; not its query prologue) and
 * quant_* before the first and after the last kernel of tq_quantize_kv.  NULL disables a
 * pair.  The events are only recorded; the caller reads them after synchronizing.  Returns
 * TQ_OK. */
int tq_profile_events(void* attend_start, void* attend_stop, void* quant_start, void* quant_stop);

/* Read-bandwidth probe (for benchmarks; not part of the compressed path): one launch of a
 * streaming kernel that reads the `bytes` bytes at device address src with 16-byte loads
 * (grid workgroups of 256 lanes, 8 loads in flight per lane, each wave reading contiguous
 * 1 KB runs) and folds them with xor.  sink: device uint32, written only if the fold equals
 * 0xA5A5A5A5 (it keeps the loads alive; a zero-filled source never writes it).  src 16-byte
 * aligned, bytes a positive multiple of 16, grid in 1..2^20.  Asynchronous on hip_stream.
 * Errors: TQ_ERR_INVALID, TQ_ERR_DEVICE. */
int tq_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, void* hip_stream);

/* Description of the last error on this thread ("" when none). */
const char* tq_last_error(void);

/* TQ_ABI_VERSION of the built library. */
int tq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
