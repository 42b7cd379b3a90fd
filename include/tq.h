/*
 * tq.h -- C ABI of the MI355X (gfx950) TurboQuant-style KV-cache library.
 *
 * The operations follow three summary pages, cited by tag:
 *   [P1] "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
 *        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
 *   [P2] "Resumo Técnico: Ablação, Inferência Estatística e Validação para
 *        Compressão de KV-Cache"
 *   [P3] "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
 *        Espaço de Pontuação para Quantização de KV-Cache"
 *
 * Conventions for every entry point
 *   - Pointers documented as "device" are HIP device memory owned by the
 *     caller; "host" pointers are ordinary CPU memory.  The library owns only
 *     its cached per-(device, seed, d) constants (freed by
 *     tq_release_cache) and the static workspace of
 *     tq_decode_attention_static.  A tq_quantize of a HEADQ tensor also
 *     takes a buffer for the rotated basis (4 H d rank bytes) from the
 *     stream's memory pool and returns it before the call's work completes
 *     on that stream.
 *   - Every call returns tq_status.  All argument and descriptor checks run
 *     on the host before any HIP call, so a rejected call touches no GPU
 *     state.  tq_last_error() returns a thread-local message for the last
 *     failure on the calling thread.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     tq_quantize and tq_decode_attention are stream-ordered and return
 *     before the GPU work finishes; tq_metrics synchronises the stream.
 *   - Head dimension d must be a power of two in [32, 1024].  Non-finite
 *     inputs give unspecified (but memory-safe) output.
 *
 * Packed cache (one tq_packed per tensor, K or V)
 *   Vector index v = (b*H + h)*T_cap + t.  Structure-of-arrays planes:
 *     codes      uint8 [v][d*w/8]      LSB-first bitstream of d fields of w bits,
 *                                      field i in bits [w*i, w*i+w):
 *                                        PLAIN, MSE, HEADQ: w = bits, the
 *                                          Lloyd-Max index of coordinate i;
 *                                        PROD: w = bits+1, that index | s_i << bits
 *                                          with s_i = [(S r)_i >= 0], the QJL
 *                                          sign of sketch row i (m = d)
 *     norms      fp32  [v]             ||x||
 *     gamma      fp32  [v]             PROD: ||r||
 *     side       uint8 [v][rank*side_bits/8]  HEADQ side code, LSB-first
 *     side_scale fp32  [v]             HEADQ: s_z
 *   Every plane base must be 16-byte aligned.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_ABI_VERSION 7

typedef enum tq_status {
  TQ_OK = 0,
  TQ_EINVAL = 1,       /* bad argument, NULL or misaligned pointer, bad size  */
  TQ_EUNSUPPORTED = 2, /* valid but not supported (e.g. d = 2048)             */
  TQ_EMISMATCH = 3,    /* descriptors disagree (K vs V, q vs cache, workspace)*/
  TQ_ENOMEM = 4,       /* workspace too small or device allocation failed     */
  TQ_EDEVICE = 5       /* a HIP call failed                                    */
} tq_status;

typedef enum tq_dtype { TQ_F32 = 0, TQ_F16 = 1 } tq_dtype;
typedef enum tq_tensor { TQ_KEYS = 0, TQ_VALUES = 1 } tq_tensor;

/* Per-tensor quantiser modes.
 *   PLAIN: [P1] "Esquemas de Cuantización" 1 and [P2] "Contribuições
 *          Principais" 1 (Plain-KV): norm split + scalar Lloyd-Max on the
 *          unrotated unit vector.
 *   MSE:   [P2] "Contribuições Principais" 1 (TQ-KV): norm split, seeded
 *          sign flip + normalised Walsh-Hadamard rotation, Beta Lloyd-Max.
 *   PROD:  [P1] "Esquemas de Cuantización" 2-3: MSE at n-1 bits plus a 1-bit
 *          QJL sketch sign(S r) and ||r|| of the rotated residual.
 *   HEADQ: [P3] section 3 "Metodologia: HeadQ": MSE base at 2 bits plus a
 *          rank-r side code of the residual in a query-PCA basis (keys only).
 *   SPECTRAL: [P2] "Configuração Experimental" (SpectralQuant) with the
 *          uniform allocation of "Recomendações Práticas" 2-3 (SQU-KV): the
 *          norm split about a calibrated mean mu, x - mu = nu u; the direction
 *          in a calibrated per-head eigenbasis V, z = V^T u; every coordinate
 *          coded at the same width against the Lloyd-Max codebook of N(0, 1)
 *          after scaling by its calibrated spread s_i: idx_i = #{k : z_i >=
 *          s_i t_k}; x_hat = mu + nu V (s * c[idx]).  No sketch.  The decision
 *          is taken in double precision (the small spreads of a low-rank head
 *          would turn float rounding into code changes).  d <= 128. */
typedef enum tq_mode {
  TQ_MODE_PLAIN = 0, TQ_MODE_MSE = 1, TQ_MODE_PROD = 2, TQ_MODE_HEADQ = 3, TQ_MODE_SPECTRAL = 4
} tq_mode;

/* Scheme presets at a budget of n bits per coordinate ([P1] "Esquemas de
 * Cuantización", [P2] "Contribuições Principais" 1, [P3] section 3):
 *   KV     K PLAIN(n)  V PLAIN(n)      TQ_KV  K MSE(n)   V MSE(n)
 *   KQV    K MSE(n)    V PROD(n)       QKQV   K PROD(n)  V PROD(n)
 *   TQ_QKV K PROD(n)   V MSE(n)        HEADQ  K HEADQ(2) V MSE(n)
 *   SQU_KV K SPECTRAL(n) V SPECTRAL(n)  ([P2] "Recomendações Práticas" 2)   */
typedef enum tq_scheme {
  TQ_SCHEME_KV = 0, TQ_SCHEME_TQ_KV = 1, TQ_SCHEME_KQV = 2,
  TQ_SCHEME_QKQV = 3, TQ_SCHEME_TQ_QKV = 4, TQ_SCHEME_HEADQ = 5, TQ_SCHEME_SQU_KV = 6
} tq_scheme;

/* Per-tensor choice of quantiser mode and index width, overriding the
 * scheme preset ([P1] "Esquemas de Cuantización" and [P2] "Contribuições
 * Principais" 1 compare per-tensor choices of rotation, scalar code and QJL
 * sketch; the presets above are the combinations the pages name).
 *   mode:  tq_mode.  HEADQ only for keys (and with a tq_headq).
 *   bits:  width of the Lloyd-Max index, in [1, 4] (PLAIN, MSE, SPECTRAL), [1, 3]
 *          (PROD: each field is bits + 1 wide, the QJL sign beside the
 *          index), 2 (HEADQ base).  A PROD tensor at bits = b spends b + 1
 *          bits per coordinate, the budget of a preset at n = b + 1. */
typedef struct tq_mode_override {
  int32_t mode;
  int32_t bits;
} tq_mode_override;

/* Dense device tensor [B][H][T][d]; the last dimension is contiguous and the
 * other strides are in elements.  Queries use T = 1 and H = number of query
 * heads. */
typedef struct tq_tensor_desc {
  const void* data;
  int32_t dtype; /* tq_dtype */
  int32_t B, H, T, d;
  int64_t stride_b, stride_h, stride_t;
} tq_tensor_desc;

/* Bytes per vector of each plane. */
typedef struct tq_layout {
  int32_t code_bytes;
  int32_t qjl_bytes;   /* 0: PROD keeps its sign bits in the code fields */
  int32_t side_bytes;  /* 0 unless HEADQ */
  int32_t has_gamma;
  int32_t has_side_scale;
} tq_layout;

/* HeadQ side-code parameters ([P3] section 3).  basis: device fp32
 * [H][d][rank], column j of head h is U_h[:, j]; caller-owned and read by
 * both tq_quantize and the decode/metrics calls. */
typedef struct tq_headq {
  const float* basis;
  int32_t rank;      /* r in {8, 16, 24, 32}, with d * r <= 16384 */
  int32_t side_bits; /* q_s in [2, 8]                              */
} tq_headq;

/* One packed tensor.  The caller sets T_cap and the plane pointers (and,
 * for SPECTRAL, basis, mean and scale); the other header fields are written
 * by tq_quantize. */
typedef struct tq_packed {
  int32_t B, H, T, T_cap, d;
  int32_t mode;      /* tq_mode                                           */
  int32_t bits;      /* width of the Lloyd-Max index (PROD: n-1, HEADQ: 2) */
  int32_t side_rank, side_bits;
  uint64_t seed;
  uint8_t* codes;
  float* norms;
  uint8_t* qjl;       /* unused (the sign bits live in the code fields) */
  float* gamma;
  uint8_t* side;
  float* side_scale;
  const float* basis; /* HEADQ: U, device [H][d][side_rank];
                         SPECTRAL: V, device [H][d][d], V[h][k][i] = entry k of
                         eigenvector i, 16-byte aligned (caller-owned, set
                         before tq_quantize) */
  const float* mean;  /* SPECTRAL: mu, device [H][d], 4-byte aligned       */
  const float* scale; /* SPECTRAL: s, device [H][d] (s_i >= 0), 4-byte aligned */
} tq_packed;

/* Quality measures ([P1] "Métricas de Evaluación" and "Significado y
 * Afirmaciones" 1; [P2] "Configuração Experimental").  KL is
 * KL(p_ref || p_quant) in nats over each query's softmax, with its mean and
 * worst case over queries; top-5 recall is |top5(s) ∩ top5(s_hat)| / 5 (ties
 * to the lower index) averaged over queries; relMSE is pooled,
 * sum ||x - x_hat||^2 / sum ||x||^2; dir_err is the mean of 1 - cos(x, x_hat)
 * over vectors with non-zero norm on both sides.  Fields whose inputs were
 * not given are NaN. */
typedef struct tq_metrics_out {
  double kl_mean, kl_max, top5_recall;
  double relmse_k, relmse_v, dir_err_k, dir_err_v;
  int64_t n_queries;
  /* Score space ([P3] section 2.1, Eq. 6: KL is locally a Fisher-weighted
   * variance of the score errors): per query 1/2 Var_p(s_hat - s), p the
   * reference softmax, s in natural units (q^T k / sqrt(d)); mean and max
   * over queries.  Needs q. */
  double fisher_mean, fisher_max;
  /* Spearman rank correlation (ties at their average rank) across the
   * queries of this call between KL and the Fisher score error, and between
   * KL and the raw key MSE of the query's KV head (mean ||k_hat - k||^2 over
   * its tokens) ([P3] section 4: score-space error predicts KL better than
   * raw key MSE).  Need q; NaN when a sample is constant. */
  double spearman_fisher_kl, spearman_keymse_kl;
  /* 6D error framework ([P1] "Métricas de Evaluación"): scale and direction
   * at the key cache, the value cache and the attention output.  SNR in dB,
   * pooled: 10 log10(sum ||x||^2 / sum ||x - x_hat||^2); phi: mean angle in
   * radians between x and x_hat over vectors with non-zero norms.  Output
   * site: the exact attention over the raw K, V against tq_decode_attention
   * over the packed cache; needs q, k_ref, v_ref and v. */
  double snr_k_db, snr_v_db, snr_out_db;
  double phi_k, phi_v, phi_out;
  /* A^2-weighted value distortion ([P3] section 2.2): per query
   * sum_j p_j^2 ||v_hat_j - v_j||^2, mean over queries; needs q, k_ref, v_ref
   * and v. */
  double a2_value_mean;
} tq_metrics_out;

int32_t tq_abi_version(void);
const char* tq_status_str(tq_status s);
const char* tq_last_error(void);

/* Beta((d-1)/2,(d-1)/2) Lloyd-Max codebook for one coordinate of a unit
 * vector in R^d ([P1] "Marco Teórico"; [P2] "Configuração Experimental").
 * Host only.  centroids: host double[2^bits] ascending; boundaries: host
 * double[2^bits - 1] (midpoints).  bits in [1, 8]; d power of two in
 * [32, 1024]. */
tq_status tq_codebook_build(int32_t d, int32_t bits, double* centroids, double* boundaries);

/* Scheme preset -> (mode, index bits) of one tensor.  Host only. */
tq_status tq_scheme_modes(int32_t scheme, int32_t n_bits, int32_t which, int32_t* mode, int32_t* bits);

/* Bytes per vector of each plane for (d, mode, index bits, side code). */
tq_status tq_packed_layout(int32_t d, int32_t mode, int32_t bits, int32_t side_rank,
                           int32_t side_bits, tq_layout* out);

/* The seeded random state of the rotation and the sketch ([P2]
 * "Configuração Experimental": random Walsh-Hadamard transform and QJL
 * sketch).  Host only.  signs: host float[d] (+1/-1); S: host float[d*d]
 * row-major (m = d rows), either may be NULL.  Both come from SplitMix64
 * streams started at seed ^ 0x243F6A8885A308D3 (signs: D_i = -1 iff bit 63 of
 * output i is set) and seed ^ 0x13198A2E03707344 (S: Box-Muller pairs in
 * double, u1 = ((o1 >> 11) + 1) 2^-53, u2 = (o2 >> 11) 2^-53, each value
 * rounded to the nearest fp16). */
tq_status tq_rotation_state(uint64_t seed, int32_t d, float* signs, float* S);

/* Write side: quantise x [B][H][T][d] (fp16 or fp32, device) into `out`.
 * Mode and bits come from (scheme, n_bits, which), or from `ovr` when it is
 * non-NULL (scheme and n_bits are then ignored; `which` still decides
 * whether HEADQ is allowed).  n_bits in [1, 4] (PROD needs n_bits >= 2).
 * hq must be non-NULL exactly when the mode is HEADQ; for SPECTRAL the caller
 * sets out->basis, out->mean and out->scale (d <= 128).  out->T_cap >= x->T
 * (0 means x->T); the planes the mode needs must be set, 16-byte aligned and
 * sized per tq_packed_layout.  Writes tokens [0, x->T) and sets out->T =
 * x->T.  Stream-ordered. */
tq_status tq_quantize(const tq_tensor_desc* x, int32_t which, int32_t scheme, int32_t n_bits,
                      uint64_t seed, const tq_mode_override* ovr, const tq_headq* hq, tq_packed* out,
                      void* stream);

/* Append to a packed cache (the generation loop around the read side:
 * [P2] "Resumo" and "Contribuições Principais" place the cost in long-context
 * generation, where the cache grows by one token per step).  Quantises
 * x [B][H][Tn][d] exactly as tq_quantize does and writes token t of
 * sequence b to slot pos[b] + t of `cache`.  pos: device int32 [B], read by
 * the kernels (no host synchronisation); a token whose slot falls outside
 * [0, cache->T_cap) is not written.  `cache` must carry a header written by
 * tq_quantize with the same mode, bits and seed as (scheme, n_bits, which,
 * seed) or `ovr`, the same B, H and d as x, and for HEADQ the same basis, rank and
 * side bits as hq; otherwise TQ_EMISMATCH.  cache->T is not changed: the
 * caller tracks lengths (tq_decode_attention_lens).  Stream-ordered. */
tq_status tq_quantize_append(const tq_tensor_desc* x, int32_t which, int32_t scheme, int32_t n_bits,
                             uint64_t seed, const tq_mode_override* ovr, const tq_headq* hq,
                             const int32_t* pos, tq_packed* cache, void* stream);

/* Workspace bytes tq_decode_attention needs for Hq query heads. */
tq_status tq_decode_workspace_size(const tq_packed* k, const tq_packed* v, int32_t Hq, size_t* bytes);

/* Read side ([P3] sections 2.1, 2.2 and 3; [P1] "Esquemas de Cuantización"):
 * for every query q [B][Hq][1][d] (device, fp16/fp32) attend over the packed
 * cache: s_j = (q^T k_hat_j + HeadQ correction q^T U z_hat_j) / sqrt(d),
 * p = softmax(s), out = sum_j p_j v_hat_j.  Query head g reads KV head
 * g / (Hq / H); k and v must agree on B, H, T, T_cap and d (else
 * TQ_EMISMATCH).  out: device fp32 [B][Hq][d]; lse: device fp32 [B][Hq]
 * (log-sum-exp of s, may be NULL).  ws: device workspace of at least
 * tq_decode_workspace_size bytes, 256-byte aligned.  Stream-ordered. */
tq_status tq_decode_attention(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                              float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* tq_decode_attention over per-sequence lengths: the queries of sequence b
 * attend over tokens [0, len[b]) of the cache, len[b] clamped to
 * [0, k->T] (so k->T should be the longest length; the splits are planned
 * on it).  lens: device int32 [B], 4-byte aligned, read by the kernels.  A
 * sequence of length 0 gets out = 0 and lse = -inf.  Same workspace as
 * tq_decode_attention.  Stream-ordered. */
tq_status tq_decode_attention_lens(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                                   const int32_t* lens, float* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream);

/* tq_decode_attention (lens == NULL) or tq_decode_attention_lens (lens:
 * device int32 [B], 4-byte aligned) without a caller workspace and without
 * allocating: for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops, harnesses that forbid allocation).  The
 * workspace is a static 64 MiB device array of the library, one per device,
 * held until the process ends; its address is taken once per device, on the
 * first call there.  A decode whose workspace (tq_decode_workspace_size)
 * exceeds 64 MiB is refused with TQ_ENOMEM.  A cache with a QJL sketch needs
 * that sketch (seed, d) already resident on the device -- any earlier
 * tq_quantize or tq_decode_attention with it puts it there -- else
 * TQ_EINVAL.  Every call on a device shares that device's array: calls that
 * overlap in time on one device (other streams, other threads) race and
 * must be ordered by the caller.  No part of the array needs clearing
 * between calls.  Stream-ordered. */
tq_status tq_decode_attention_static(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                                     const int32_t* lens, float* out, float* lse, void* stream);

/* Workspace bytes tq_metrics needs. */
tq_status tq_metrics_workspace_size(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                                    size_t* bytes);

/* Quality measures of the packed cache against the raw tensors.  q may be
 * NULL (no KL / top-5); k_ref or v_ref may be NULL (no relMSE/dir_err for
 * that tensor; k_ref is required when q is given).  Synchronises `stream`
 * and writes *out (host). */
tq_status tq_metrics(const tq_tensor_desc* q, const tq_tensor_desc* k_ref, const tq_tensor_desc* v_ref,
                     const tq_packed* k, const tq_packed* v, tq_metrics_out* out, void* ws,
                     size_t ws_bytes, void* stream);

/* SpectralQuant calibration ([P2] "Configuração Experimental": a per-head
 * eigenvector basis from representative tokens; K and V calibrated on
 * separate sets): from calib [N][d] (host fp32, one head's vectors), the
 * mean (host fp32 [d]), the eigenvectors of the centred covariance as the
 * columns of basis (host fp32 [d][d], descending eigenvalues, each column's
 * largest-magnitude entry positive) and the spreads scale_i =
 * sqrt(lambda_i / sum lambda) (host fp32 [d]).  Host only, synchronous. */
tq_status tq_spectral_fit(const float* calib, int32_t N, int32_t d, float* basis, float* mean, float* scale);

/* HeadQ calibration ([P3] section 3, "Calibração"): rank-r PCA of the
 * centred calibration queries calib [N][d] (host fp32).  U: host fp32
 * [d][rank], columns = eigenvectors of the largest eigenvalues, each with
 * its largest-magnitude entry positive.  Host only, synchronous. */
tq_status tq_headq_fit(const float* calib, int32_t N, int32_t d, int32_t rank, float* U);

/* ---- A^2-weighted value policy ([P3] section 2.2: values are read by
 * o = sum_j p_j v_j, and sum_j p_j^2 ||dv_j||^2 is the value error that
 * matters; section 5: HeadQ keys with a value policy weighted by it at 2
 * bits).  The policy splits each (batch, head)'s tokens into a high and a
 * low value tier at a fixed mean number of index bits; attention does not
 * depend on the order of the (key, value) pairs, so each tier is an
 * ordinary packed cache over a permutation of the tokens, and the two
 * tiers' attention outputs combine with tq_attention_merge. */

/* Workspace bytes of tq_a2_weights. */
tq_status tq_a2_workspace_size(const tq_tensor_desc* q_probe, const tq_tensor_desc* k_ref, size_t* bytes);

/* A_j = mean over the probe queries of KV head h of p_j(q)^2, p(q) the
 * softmax of q^T k_j / sqrt(d) over the T raw keys of the sequence.
 * q_probe: device [B][Hq][Np][d] (Np probes per query head, the tensor's T
 * dimension), Hq a multiple of k_ref->H; the probes of KV head h are those of
 * its Hq / H query heads, at most 16384 / d of them.  k_ref: device
 * [B][H][T][d].  weights: device fp32 [B][H][T].  ws: 256-byte aligned,
 * tq_a2_workspace_size bytes.  Stream-ordered. */
tq_status tq_a2_weights(const tq_tensor_desc* q_probe, const tq_tensor_desc* k_ref, float* weights, void* ws,
                        size_t ws_bytes, void* stream);

/* Candidates and choice of tq_value_policy. */
typedef struct tq_value_plan {
  int32_t b_lo, b_hi;      /* index bits of the low and high value tiers (equal: uniform) */
  int32_t n_high;          /* tokens per (batch, head) in the high tier                   */
  int32_t n_candidates;
  int32_t cand_lo[3], cand_hi[3], cand_high[3];
  double surrogate[3];     /* sum_j A_j ||v_j||^2 D_{b_j} of each candidate                */
} tq_value_plan;

/* Workspace bytes of tq_value_policy. */
tq_status tq_value_policy_workspace_size(const tq_tensor_desc* v_ref, size_t* bytes);

/* The two-tier value plan at a mean of budget_bits index bits per value
 * coordinate (budget_bits in [1, 4]).  Candidates, in this order: uniform
 * budget_bits; (budget_bits - 1, budget_bits + 1) with floor(T/2) tokens high;
 * (budget_bits - 1, budget_bits + 2) with floor(T/3) high (widths in [1, 4]).
 * In each, the high tokens of a (batch, head) are those with the largest
 * w_j = A_j ||v_j||^2 (ties to the lower index).  The candidate with the
 * smallest surrogate sum_j w_j D_{b_j} over the whole tensor is chosen (ties
 * to the earlier one), D_b = the relative MSE of the b-bit TQ-MSE code.
 * weights: device fp32 [B][H][T] (tq_a2_weights); v_ref: device [B][H][T][d]
 * raw values.  perm: device int32 [B][H][T], the chosen high tier first,
 * each tier in increasing token order.  *plan (host) receives the choice
 * and the candidates.  Synchronises `stream`. */
tq_status tq_value_policy(const float* weights, const tq_tensor_desc* v_ref, int32_t budget_bits, int32_t* perm,
                          tq_value_plan* plan, void* ws, size_t ws_bytes, void* stream);

/* out[b][h][t] = x[b][h][perm[b][h][t0 + t]] for t in [0, out->T): the
 * tokens of one tier, in order.  x: device [B][H][T][d]; perm: device
 * int32 [B][H][x->T] (a permutation of [0, x->T) per (b, h)); out: device,
 * same B, H, d and dtype, out->T <= x->T - t0.  Stream-ordered. */
tq_status tq_gather_tokens(const tq_tensor_desc* x, const int32_t* perm, int32_t t0, const tq_tensor_desc* out,
                           void* stream);

/* Attention over the union of two disjoint token sets from the outputs and
 * log-sum-exps of each (device fp32 out_* [n][d], lse_* [n]): out =
 * sum_s exp(lse_s - lse) out_s, lse = log(exp(lse_a) + exp(lse_b)); a side
 * with lse = -inf contributes nothing.  lse may be NULL.  Stream-ordered. */
tq_status tq_attention_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b,
                             int32_t n, int32_t d, float* out, float* lse, void* stream);

/* Diagnostic: reads `bytes` (a positive multiple of 16) of device memory at
 * `src` (16-byte aligned) with the non-temporal 128-bit loads the decode
 * kernels stream the packed cache with, and writes one XOR checksum per block
 * to `sink` (device, at least 2048 * 4 bytes).  Measures the achievable
 * streaming-read bandwidth and serves as the known-size reference for the
 * HBM byte counters.  Stream-ordered. */
tq_status tq_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Diagnostic: the memory traffic of the write side with no arithmetic.  For
 * each of `rows` rows, reads `in_row_bytes` at src + row * in_row_bytes and
 * writes `out_row_bytes` (their XOR fold) at dst + row * out_row_bytes, plus
 * one float per row to each of `nplanes` planes (planes + p * rows + row), in
 * the access pattern of the d = 128 quantiser (16 rows per wave, 16-byte
 * non-temporal loads and stores).  in_row_bytes and out_row_bytes are
 * multiples of 64 in [64, 4096]; nplanes in [0, 4] (planes may be NULL when
 * 0); src and dst 16-byte aligned, planes 4-byte aligned; rows in
 * [1, 2^35].  Its time is the floor for a quantise that moves the same
 * bytes (input rows, packed codes, per-token norms).  Stream-ordered. */
tq_status tq_stream_rw(const void* src, int64_t rows, int32_t in_row_bytes, void* dst, int32_t out_row_bytes,
                       float* planes, int32_t nplanes, void* stream);

/* Frees the cached device constants of every device. */
tq_status tq_release_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
