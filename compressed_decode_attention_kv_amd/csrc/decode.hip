// Read side of libtq: decode attention straight from the packed cache, in
// the rotated domain, plus the score/metric kernels of tq_metrics.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P3] = "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
//        Espaço de Pontuação para Quantização de KV-Cache"
//
// Algebra (Pi orthogonal): with k_hat = nu Pi^T (c[idx] + a gamma S^T sigma),
// a = sqrt(pi/2)/m,
//   q^T k_hat = nu (<Pi q, c[idx]> + a gamma <S Pi q, sigma>)
// and the value read sum_j p_j v_hat_j equals
//   Pi^T (sum_j p_j nu_j c[idx_j] + a S^T sum_j p_j nu_j gamma_j sigma_j),
// so S^T and Pi^T are applied once per query (in the combine kernel), never
// per token.  HeadQ adds q^T U z_hat / sqrt(d) = <U^T q, z_hat> / sqrt(d)
// ([P3] section 3).
#include <cfloat>
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;  // log2 units: rescale only when the max grows by > 2^8

__device__ __forceinline__ float safe_exp2_diff(float a, float m) {
  return (a == -INFINITY) ? 0.f : exp2f(a - m);
}

// Block-wide max / sum of one value per thread (kThreads threads; `red`
// holds kThreads / 64 floats and is free on entry).
__device__ __forceinline__ float block_max(float v, float* red) {
  for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r += red[w];
  return r;
}

// From this head dimension on, S q of sketched keys and S^T acc_sk of
// sketched values run as one tiled product over all queries (sproj_kernel)
// instead of once per query block: S is d^2 floats (4 MB at d = 1024).
constexpr int kBigD = 512;

// ---- query preparation -------------------------------------------------------
// q_rot = Pi q (rotated keys) or q; q_sk = S q_rot (QJL keys); q_w = U_h^T q
// (HeadQ keys).  One block per query.
__global__ __launch_bounds__(kThreads) void qprep_kernel(QPrepParams p) {
  __shared__ float s_q[kMaxD], s_r[kMaxD];
  const int qi = blockIdx.x, b = qi / p.Hq, g = qi % p.Hq;
  const int d = p.d;
  const int kvh = g / (p.Hq / p.Hkv);
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float v;
    if (p.dtype == TQ_F16)
      v = (float)reinterpret_cast<const _Float16*>(p.q)[(int64_t)b * p.sb + (int64_t)g * p.sh + i];
    else
      v = reinterpret_cast<const float*>(p.q)[(int64_t)b * p.sb + (int64_t)g * p.sh + i];
    s_q[i] = v;
    s_r[i] = (p.rotate && ((p.signbits[i >> 5] >> (i & 31)) & 1u)) ? -v : v;
  }
  __syncthreads();
  if (p.rotate && d == 128) {
    // The same butterflies in the registers of one wave: lane l holds
    // elements 2l and 2l + 1; the stage of span h > 1 pairs lane l with lane
    // l ^ (h / 2), whose value comes first in the sum or the difference
    // when this lane is the pair's upper half (same operations, same result).
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      const float a = s_r[2 * l], c = s_r[2 * l + 1];
      float x0 = a + c, x1 = a - c;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const float y0 = __shfl_xor(x0, m, 64), y1 = __shfl_xor(x1, m, 64);
        const bool upper = (l & m) != 0;
        x0 = upper ? y0 - x0 : x0 + y0;
        x1 = upper ? y1 - x1 : x1 + y1;
      }
      s_r[2 * l] = x0 * p.inv_sqrt_d;
      s_r[2 * l + 1] = x1 * p.inv_sqrt_d;
    }
    __syncthreads();
  } else if (p.rotate) {
    for (int h = 1; h < d; h <<= 1) {
      for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
        const int lo = (i / h) * 2 * h + (i % h), hi = lo + h;
        float a = s_r[lo], c = s_r[hi];
        s_r[lo] = a + c;
        s_r[hi] = a - c;
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < d; i += blockDim.x) s_r[i] *= p.inv_sqrt_d;
    __syncthreads();
  }
  if (p.kspectral) {
    // q . k_hat = q . mu + nu sum_i (s_i (V^T q)_i) c[idx_i]: the score runs
    // on s * V^T q like a rotated query; the mean adds q . mu / sqrt(d) to
    // every score of the query (softmax-invariant; only the LSE moves).
    // The head's basis is staged in (dynamic) LDS with 16-byte loads, all
    // in flight at once: read straight from L2, the d-long dependent loop
    // waited one load latency per term.
    __shared__ float s_red[kThreads / 64];
    extern __shared__ float4 s_dyn[];
    float* sV = reinterpret_cast<float*>(s_dyn);
    const float4* V4 = reinterpret_cast<const float4*>(p.sbasis + (size_t)kvh * d * d);
    const float* sc = p.sscale + (size_t)kvh * d;
    const float* mu = p.smean + (size_t)kvh * d;
    for (int e = threadIdx.x; e < d * d / 4; e += blockDim.x) s_dyn[e] = V4[e];
    __syncthreads();
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(sV[k * d + i], s_q[k], acc);
      s_r[i] = sc[i] * acc;
    }
    float part = 0.f;
    for (int k = threadIdx.x; k < d; k += blockDim.x) part = fmaf(s_q[k], mu[k], part);
    for (int m = 32; m > 0; m >>= 1) part += __shfl_xor(part, m, 64);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int w = 0; w < (int)blockDim.x / 64; ++w) t += s_red[w];
      p.qoff[qi] = t * p.inv_sqrt_d;
    }
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x) p.qrot[(size_t)qi * d + i] = s_r[i];
  if (p.qraw)
    for (int i = threadIdx.x; i < d; i += blockDim.x) p.qraw[(size_t)qi * d + i] = s_q[i];
  if (p.kqjl && d < kBigD) {
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      const float* srow = p.S + (size_t)i * d;
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(srow[k], s_r[k], acc);
      p.qsk[(size_t)qi * d + i] = acc;
    }
  }
  if (p.kside) {
    const float* U = p.basis + (size_t)kvh * d * p.rank;
    for (int r = threadIdx.x; r < p.rank; r += blockDim.x) {
      float acc = 0.f;
      for (int k = 0; k < d; ++k) acc = fmaf(U[(size_t)k * p.rank + r], s_q[k], acc);
      p.qw[(size_t)qi * p.rank + r] = acc;
    }
  }
}

// Map a linear work-unit id to (query-in-group g, rest) so that the G
// queries sharing one KV chunk run on the same XCD (ids congruent mod 8 go
// to the same XCD) and close in time, so the chunk is read from HBM once.
__device__ __forceinline__ bool unit_map(int id, int G, int R, int* g, int* r) {
  const int x = id & 7, k = id >> 3;
  *g = k % G;
  *r = (k / G) * 8 + x;
  return *r < R;
}

// Score contribution of one lane (its 32 coordinates) for one token.
template <int KB, bool KQ, bool KS>
struct KScorer {
  float qf[32];
  float uf[KQ ? 32 : 1];
  float wf[KS ? 32 : 1];  // HeadQ: this lane's share of U^T q (codes j, j+L, ...)
  int nside;

  __device__ void init(const DecodeParams& p, int qi, int j, int L) {
#pragma unroll
    for (int e = 0; e < 32; ++e) qf[e] = p.qrot[(size_t)qi * p.d + 32 * j + e];
    if (KQ) {
#pragma unroll
      for (int e = 0; e < 32; ++e) uf[e] = p.qsk[(size_t)qi * p.d + 32 * j + e];
    }
    if (KS) {
      nside = 0;
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const int r = j + s * L;
        wf[s] = (r < p.rank) ? p.qw[(size_t)qi * p.rank + r] : 0.f;
      }
    }
  }

  // Returns this lane's share of s_j * sqrt(d) (natural units before scaling).
  __device__ float score(const DecodeParams& p, const float* kc, int64_t vec, int j, int L) const {
    const int d = p.d;
    // PROD keys: (KB+1)-bit fields, code | sign << KB.
    constexpr int KF = Field<KB, KQ>::kBits;
    uint32_t w[KF];
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(p.k.codes + vec * (d * KF / 8)) + j * KF;
#pragma unroll
    for (int k = 0; k < KF; ++k) w[k] = ld_nt(cw + k);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc = fmaf(qf[e], kc[code_at<KF>(w, e) & Field<KB, false>::kCodeMask], acc);
    const float nu = ld_nt(p.k.norms + vec);
    float part = nu * acc;
    if (KQ) {
      const uint32_t sw = sign_word<KB>(w);
      float pq = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) pq += ((sw >> e) & 1u) ? uf[e] : -uf[e];
      part = fmaf(nu * p.k_qjl * ld_nt(p.k.gamma + vec), pq, part);
    }
    if (KS) {
      const int sb = p.side_bits, lev = (1 << (sb - 1)) - 1, nbytes = p.rank * sb / 8;
      const uint8_t* sc = p.k.side + vec * nbytes;
      const float sz = ld_nt(p.k.side_scale + vec);
      float cs = 0.f;
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const int r = j + s * L;
        if (r < p.rank) {
          const int bit = sb * r, by = bit >> 3;
          uint32_t raw = sc[by];
          if (by + 1 < nbytes) raw |= (uint32_t)sc[by + 1] << 8;
          const int code = (int)((raw >> (bit & 7)) & ((1u << sb) - 1u));
          cs = fmaf(wf[s], (float)(code - lev), cs);
        }
      }
      part = fmaf(sz, cs, part);
    }
    return part;
  }
};

// ---- split decode --------------------------------------------------------------
// One block = 4 waves = one (query, context chunk).  Within a wave, L = d/32
// lanes own one token (32 coordinates each) and 64/L tokens are in flight;
// every token slot keeps its own online-softmax state, merged at the end.
template <int KB, bool KQ, bool KS, int VB, bool VQ>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeParams p) {
  __shared__ float s_kc[16], s_vc[16];
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][2 * kMaxD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = p.L, j = lane & (L - 1), slot = lane / L, vpw = 64 / L;
  const int d = p.d;
  if (threadIdx.x < 16) { s_kc[threadIdx.x] = p.kc[threadIdx.x]; s_vc[threadIdx.x] = p.vc[threadIdx.x]; }
  __syncthreads();

  int g, r;
  if (!unit_map(blockIdx.x, p.G, p.B * p.Hkv * p.nsplit, &g, &r)) return;
  const int split = r % p.nsplit, bkv = r / p.nsplit;
  const int b = bkv / p.Hkv, kvh = bkv % p.Hkv;
  const int qi = b * p.Hq + kvh * p.G + g;
  // Per-sequence length (clamped to [0, T]); a split past it has no tokens.
  const int Tb = p.lens ? min(max(p.lens[b], 0), p.T) : p.T;
  const int t0 = split * p.chunk, t1 = min(Tb, t0 + p.chunk);
  const int64_t vbase = (int64_t)bkv * p.T_cap;

  KScorer<KB, KQ, KS> ks;
  ks.init(p, qi, j, L);
  float acc[32], ask[VQ ? 32 : 1];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.f;
  if (VQ) {
#pragma unroll
    for (int e = 0; e < 32; ++e) ask[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int base = t0 + wave * vpw; base < t1; base += 4 * vpw) {
    const int t = base + slot;
    const bool valid = t < t1;
    const int64_t vec = vbase + (valid ? t : t1 - 1);
    float s = group_sum(ks.score(p, s_kc, vec, j, L), L) * p.scale_log2;
    if (!valid) s = -INFINITY;
    if (s > m + kRescaleSlack) {
      const float alpha = safe_exp2_diff(m, s);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] *= alpha;
      if (VQ) {
#pragma unroll
        for (int e = 0; e < 32; ++e) ask[e] *= alpha;
      }
      m = s;
    }
    const float pt = valid ? exp2f(s - m) : 0.f;
    l += pt;
    const float wv = pt * ld_nt(p.v.norms + vec);
    // PROD values: (VB+1)-bit fields, code | sign << VB.
    constexpr int VF = Field<VB, VQ>::kBits;
    uint32_t w[VF];
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(p.v.codes + vec * (d * VF / 8)) + j * VF;
#pragma unroll
    for (int k = 0; k < VF; ++k) w[k] = ld_nt(cw + k);
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = fmaf(wv, s_vc[code_at<VF>(w, e) & Field<VB, false>::kCodeMask], acc[e]);
    if (VQ) {
      const float wq = wv * ld_nt(p.v.gamma + vec);
      const uint32_t sw = sign_word<VB>(w);
#pragma unroll
      for (int e = 0; e < 32; ++e) ask[e] += ((sw >> e) & 1u) ? wq : -wq;
    }
  }

  // Merge the token slots of the wave (lanes with equal j).
  for (int off = L; off < 64; off <<= 1) {
    const float mo = shfl_xor_f(m, off), lo = shfl_xor_f(l, off);
    const float M = fmaxf(m, mo);
    const float a = safe_exp2_diff(m, M), c = safe_exp2_diff(mo, M);
    l = l * a + lo * c;
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = acc[e] * a + shfl_xor_f(acc[e], off) * c;
    if (VQ) {
#pragma unroll
      for (int e = 0; e < 32; ++e) ask[e] = ask[e] * a + shfl_xor_f(ask[e], off) * c;
    }
    m = M;
  }
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < 32; ++e) s_acc[wave][32 * j + e] = acc[e];
    if (VQ) {
#pragma unroll
      for (int e = 0; e < 32; ++e) s_acc[wave][d + 32 * j + e] = ask[e];
    }
    if (j == 0) { s_m[wave] = m; s_l[wave] = l; }
  }
  __syncthreads();
  // Merge the 4 waves and write this split's partial: [m, l, acc[d], ask[d]].
  float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float sc[4], lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) { sc[w] = safe_exp2_diff(s_m[w], M); lt += s_l[w] * sc[w]; }
  float* out = p.part + ((size_t)qi * p.nsplit + split) * p.part_stride;
  const int nvals = VQ ? 2 * d : d;
  for (int i = threadIdx.x; i < nvals; i += blockDim.x) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) v += s_acc[w][i] * sc[w];
    out[2 + i] = v;
  }
  if (threadIdx.x == 0) { out[0] = M; out[1] = lt; }
}

// ---- S x and S^T x for many queries (d >= kBigD) ---------------------------------
// Y[q][i] = sum_k M(i, k) X[q][k], M = S (trans = 0) or S^T (trans = 1), k
// ascending: the fma sequence of the per-query loops, so the result is the
// same bit for bit.  Block: 16 queries x 64 outputs, thread (query tq, outputs
// 4 ti .. 4 ti + 3); K in steps of 128 through LDS, the next step's tiles
// loaded into registers while the current ones are used (a step's work
// covers the L2 latency of the next one's loads).
constexpr int kSpK = 128;
__global__ __launch_bounds__(kThreads) void sproj_kernel(SProjParams p) {
  __shared__ float Xs[16][kSpK + 4];
  __shared__ __attribute__((aligned(16))) float Ms[kSpK][68];
  const int d = p.d, q0 = blockIdx.x * 16, i0 = blockIdx.y * 64;
  const int tq = threadIdx.x >> 4, ti = threadIdx.x & 15;
  constexpr int NX = 16 * kSpK / kThreads, NM = 64 * kSpK / kThreads;
  float xr[NX], mr[NM];
  auto load = [&](int k0) {
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int e = threadIdx.x + kThreads * n, q = e / kSpK, k = e % kSpK;
      xr[n] = q0 + q < p.nq ? p.X[(size_t)(q0 + q) * d + k0 + k] : 0.f;
    }
#pragma unroll
    for (int n = 0; n < NM; ++n) {
      const int e = threadIdx.x + kThreads * n;
      mr[n] = p.trans ? p.S[(size_t)(k0 + (e >> 6)) * d + i0 + (e & 63)]
                      : p.S[(size_t)(i0 + e / kSpK) * d + k0 + e % kSpK];
    }
  };
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int k0 = 0; k0 < d; k0 += kSpK) {
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NX; ++n) {
      const int e = threadIdx.x + kThreads * n;
      Xs[e / kSpK][e % kSpK] = xr[n];
    }
#pragma unroll
    for (int n = 0; n < NM; ++n) {
      const int e = threadIdx.x + kThreads * n;
      if (p.trans) Ms[e >> 6][e & 63] = mr[n];
      else Ms[e % kSpK][e / kSpK] = mr[n];
    }
    __syncthreads();
    if (k0 + kSpK < d) load(k0 + kSpK);
#pragma unroll 8
    for (int k = 0; k < kSpK; ++k) {
      const float x = Xs[tq][k];
      const float4 m = *reinterpret_cast<const float4*>(&Ms[k][4 * ti]);
      acc[0] = fmaf(m.x, x, acc[0]);
      acc[1] = fmaf(m.y, x, acc[1]);
      acc[2] = fmaf(m.z, x, acc[2]);
      acc[3] = fmaf(m.w, x, acc[3]);
    }
  }
  if (q0 + tq < p.nq)
    *reinterpret_cast<float4*>(p.Y + (size_t)(q0 + tq) * d + i0 + 4 * ti) = float4{acc[0], acc[1], acc[2], acc[3]};
}

// ---- combine + finalize --------------------------------------------------------
// LSE-merge of the splits, then out = Pi^T (acc/l + a S^T ask / l) (rotated V),
// mu + V (s * acc / l) (SPECTRAL V) or acc / l (plain V).  One block per query;
// the split weights are reduced block-wide (thread s takes split s).
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineParams p) {
  __shared__ float s_o[kMaxD], s_k[kMaxD];
  __shared__ float s_w[256];
  __shared__ float s_M, s_L;
  __shared__ float s_red[kThreads / 64];
  const int qi = blockIdx.x, d = p.d;
  const float* part = p.part + (size_t)qi * p.nsplit * p.part_stride;
  // Stage 2 of a split combine: o + a S^T k from the workspace, then Pi^T.
  if (p.stage == 2) {
    for (int i = threadIdx.x; i < d; i += blockDim.x)
      s_o[i] = fmaf(p.v_qjl, p.add[(size_t)qi * d + i], p.ow[(size_t)qi * d + i]);
    __syncthreads();
  } else {
  {
    const int sp = threadIdx.x;  // nsplit <= 256 = kThreads
    const float ms = sp < p.nsplit ? part[(size_t)sp * p.part_stride] : -INFINITY;
    const float M = block_max(ms, s_red);
    const float w = sp < p.nsplit ? safe_exp2_diff(ms, M) : 0.f;
    if (sp < p.nsplit) s_w[sp] = w;
    const float L = block_sum(sp < p.nsplit ? part[(size_t)sp * p.part_stride + 1] * w : 0.f, s_red);
    if (threadIdx.x == 0) { s_M = M; s_L = L; }
  }
  __syncthreads();
  // A sequence with no tokens (length 0) has l = 0: its output is 0 and its
  // log-sum-exp -inf.
  const float invl = s_L > 0.f ? 1.0f / s_L : 0.f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    float a = 0.f, k = 0.f;
    for (int sp = 0; sp < p.nsplit; ++sp) {
      a = fmaf(part[(size_t)sp * p.part_stride + 2 + i], s_w[sp], a);
      if (p.vqjl) k = fmaf(part[(size_t)sp * p.part_stride + 2 + d + i], s_w[sp], k);
    }
    s_o[i] = a * invl;
    s_k[i] = k * invl;
  }
  __syncthreads();
  if (p.stage == 1) {
    // Stage 1 of a split combine: o = acc / l and k = acc_sk / l to the
    // workspace (S^T k follows for all queries at once), and the LSE.
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      p.ow[(size_t)qi * d + i] = s_o[i];
      p.kw[(size_t)qi * d + i] = s_k[i];
    }
    if (threadIdx.x == 0 && p.lse)
      p.lse[qi] = s_L > 0.f ? (s_M + log2f(s_L)) * 0.69314718055994530942f + (p.qoff ? p.qoff[qi] : 0.f) : -INFINITY;
    return;
  }
  if (p.vqjl && d < (int)blockDim.x) {
    // S^T acc_sk with blockDim / d threads per column, each over its own
    // slice of rows with all of the slice's loads in flight (one L2 round
    // trip instead of one per 16 rows), the slices summed in LDS.
    const int nsl = (int)blockDim.x / d, rows = d / nsl;
    const int kk = threadIdx.x % d, sl = threadIdx.x / d;
    float acc = 0.f;
    if (sl < nsl) {
      const float* Sc = p.S + (size_t)sl * rows * d + kk;
      const float* kc = s_k + sl * rows;
#pragma unroll 64
      for (int i = 0; i < rows; ++i) acc = fmaf(Sc[(size_t)i * d], kc[i], acc);
    }
    s_w[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x < d) {
      float t = 0.f;
      for (int u = 0; u < nsl; ++u) t += s_w[u * d + threadIdx.x];
      s_o[threadIdx.x] = fmaf(p.v_qjl, t, s_o[threadIdx.x]);
    }
    __syncthreads();
  } else if (p.vqjl) {
    float add[kMaxD / kThreads];
    for (int c = 0; c < d / (int)blockDim.x + 1; ++c) {
      const int kk = threadIdx.x + c * blockDim.x;
      if (kk < d && c < kMaxD / kThreads) {
        // S^T acc_sk: coalesced across kk; unrolled so that several L2
        // loads are in flight per thread.
        float acc = 0.f;
#pragma unroll 16
        for (int i = 0; i < d; ++i) acc = fmaf(p.S[(size_t)i * d + kk], s_k[i], acc);
        add[c] = acc;
      }
    }
    __syncthreads();
    for (int c = 0; c < d / (int)blockDim.x + 1; ++c) {
      const int kk = threadIdx.x + c * blockDim.x;
      if (kk < d && c < kMaxD / kThreads) s_o[kk] = fmaf(p.v_qjl, add[c], s_o[kk]);
    }
    __syncthreads();
  }
  if (p.vspectral) {
    // out = mu + V (s * acc / l), V row-major [k][i], d <= 128.  The basis is
    // staged in (dynamic) LDS as for the query prep; thread k then forms row
    // k (reads spread over the banks by the per-row offset k).
    const int kvh = (qi % p.Hq) / p.G;
    extern __shared__ float4 s_dyn[];
    float* sV = reinterpret_cast<float*>(s_dyn);
    const float4* V4 = reinterpret_cast<const float4*>(p.vbasis + (size_t)kvh * d * d);
    const float* sc = p.vscale + (size_t)kvh * d;
    const float* mu = p.vmean + (size_t)kvh * d;
    for (int e = threadIdx.x; e < d * d / 4; e += blockDim.x) s_dyn[e] = V4[e];
    for (int i = threadIdx.x; i < d; i += blockDim.x) s_k[i] = sc[i] * s_o[i];
    __syncthreads();
    for (int k = threadIdx.x; k < d; k += blockDim.x) {
      float acc = 0.f;
      for (int u = 0; u < d; ++u) {
        const int i = (u + k) & (d - 1);
        acc = fmaf(sV[k * d + i], s_k[i], acc);
      }
      s_w[k] = mu[k] + acc;
    }
    __syncthreads();
    // A sequence with no tokens keeps its zero output.
    for (int i = threadIdx.x; i < d; i += blockDim.x) s_o[i] = s_L > 0.f ? s_w[i] : 0.f;
    __syncthreads();
  }
  }  // stage 0 / 1
  if (p.vrotate) {
    for (int h = 1; h < d; h <<= 1) {
      for (int i = threadIdx.x; i < d / 2; i += blockDim.x) {
        const int lo = (i / h) * 2 * h + (i % h), hi = lo + h;
        float a = s_o[lo], c = s_o[hi];
        s_o[lo] = a + c;
        s_o[hi] = a - c;
      }
      __syncthreads();
    }
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
      const float sg = ((p.signbits[i >> 5] >> (i & 31)) & 1u) ? -1.f : 1.f;
      s_o[i] *= sg * p.inv_sqrt_d;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < d; i += blockDim.x) p.out[(size_t)qi * d + i] = s_o[i];
  if (p.stage == 0 && threadIdx.x == 0 && p.lse)
    p.lse[qi] = s_L > 0.f ? (s_M + log2f(s_L)) * 0.69314718055994530942f + (p.qoff ? p.qoff[qi] : 0.f) : -INFINITY;
}

// ---- metric scores ---------------------------------------------------------------
// Reference scores from the raw keys and quantised scores from the packed
// cache, for every (query, token).  Same lane layout as the split decode.
template <int KB, bool KQ, bool KS, typename TIN>
__global__ __launch_bounds__(kThreads) void metric_scores_kernel(MetricScoreParams mp) {
  __shared__ float s_kc[16];
  const DecodeParams& p = mp.dp;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = p.L, j = lane & (L - 1), slot = lane / L, vpw = 64 / L;
  if (threadIdx.x < 16) s_kc[threadIdx.x] = p.kc[threadIdx.x];
  __syncthreads();
  int g, r;
  if (!unit_map(blockIdx.x, p.G, p.B * p.Hkv * p.nsplit, &g, &r)) return;
  const int split = r % p.nsplit, bkv = r / p.nsplit;
  const int b = bkv / p.Hkv, kvh = bkv % p.Hkv;
  const int qi = b * p.Hq + kvh * p.G + g;
  const int t0 = split * p.chunk, t1 = min(p.T, t0 + p.chunk);
  const int64_t vbase = (int64_t)bkv * p.T_cap;
  KScorer<KB, KQ, KS> ks;
  ks.init(p, qi, j, L);
  float qraw[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) qraw[e] = mp.qraw[(size_t)qi * p.d + 32 * j + e];
  const TIN* kbase = reinterpret_cast<const TIN*>(mp.kref) + (int64_t)b * mp.ksb + (int64_t)kvh * mp.ksh;
  const float inv_sqrt_d = p.scale_log2 / 1.4426950408889634f;
  for (int base = t0 + wave * vpw; base < t1; base += 4 * vpw) {
    const int t = base + slot;
    const bool valid = t < t1;
    const int tc = valid ? t : t1 - 1;
    const int64_t vec = vbase + tc;
    const float sh = group_sum(ks.score(p, s_kc, vec, j, L), L) * inv_sqrt_d + (p.qoff ? p.qoff[qi] : 0.f);
    float kv[32];
    load32<TIN>(kbase + (int64_t)tc * mp.kst + 32 * j, kv);
    float sr = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) sr = fmaf(qraw[e], kv[e], sr);
    sr = group_sum(sr, L) * inv_sqrt_d;
    if (valid && j == 0) {
      mp.s_ref[(size_t)qi * p.T + t] = sr;
      mp.s_hat[(size_t)qi * p.T + t] = sh;
    }
  }
}

// ---- metric reduce -----------------------------------------------------------------
// Per query: KL(p_ref || p_hat) from the logits and top-5 recall (ties to the
// lower index) ([P1] "Métricas de Evaluación").
struct Top5 {
  float v[5];
  int i[5];
  __device__ void init() {
    for (int k = 0; k < 5; ++k) { v[k] = -INFINITY; i[k] = 0x7fffffff; }
  }
  __device__ static bool better(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }
  __device__ void push(float x, int ix) {
    if (!better(x, ix, v[4], i[4])) return;
    int k = 4;
    while (k > 0 && better(x, ix, v[k - 1], i[k - 1])) { v[k] = v[k - 1]; i[k] = i[k - 1]; --k; }
    v[k] = x; i[k] = ix;
  }
};

__global__ __launch_bounds__(kThreads) void metric_reduce_kernel(MetricReduceParams p) {
  __shared__ double s_red[kThreads];
  __shared__ float s_tv[kThreads * 5];
  __shared__ int s_ti[kThreads * 5];
  __shared__ int s_top_ref[5];
  const int qi = blockIdx.x, T = p.T, tid = threadIdx.x;
  const float* sr = p.s_ref + (size_t)qi * T;
  const float* sh = p.s_hat + (size_t)qi * T;
  auto block_reduce = [&](double v, bool is_max) -> double {
    s_red[tid] = v;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) s_red[tid] = is_max ? fmax(s_red[tid], s_red[tid + w]) : s_red[tid] + s_red[tid + w];
      __syncthreads();
    }
    double r = s_red[0];
    __syncthreads();
    return r;
  };
  double mr = -INFINITY, mh = -INFINITY;
  for (int t = tid; t < T; t += kThreads) { mr = fmax(mr, (double)sr[t]); mh = fmax(mh, (double)sh[t]); }
  mr = block_reduce(mr, true);
  mh = block_reduce(mh, true);
  double zr = 0.0, zh = 0.0, cross = 0.0;
  for (int t = tid; t < T; t += kThreads) {
    const double er = exp((double)sr[t] - mr);
    zr += er;
    zh += exp((double)sh[t] - mh);
    cross += er * ((double)sr[t] - (double)sh[t]);
  }
  zr = block_reduce(zr, false);
  zh = block_reduce(zh, false);
  cross = block_reduce(cross, false);
  const double kl = cross / zr - (mr + log(zr)) + (mh + log(zh));
  // Fisher score error 1/2 Var_p(s_hat - s_ref), two passes (mean, then
  // spread), and the A^2 value distortion sum_j p_j^2 ||v_hat_j - v_j||^2.
  const int b = qi / p.Hq, kvh = (qi % p.Hq) / p.G;
  const float* verr = p.verr ? p.verr + ((size_t)b * p.Hkv + kvh) * p.T_cap : nullptr;
  double m1 = 0.0, a2 = 0.0;
  for (int t = tid; t < T; t += kThreads) {
    const double pt = exp((double)sr[t] - mr) / zr;
    m1 += pt * ((double)sh[t] - (double)sr[t]);
    if (verr) a2 += pt * pt * (double)verr[t];
  }
  m1 = block_reduce(m1, false);
  a2 = block_reduce(a2, false);
  double var = 0.0;
  for (int t = tid; t < T; t += kThreads) {
    const double pt = exp((double)sr[t] - mr) / zr;
    const double dv = (double)sh[t] - (double)sr[t] - m1;
    var += pt * dv * dv;
  }
  var = block_reduce(var, false);
  // top-5 of each score row
  int hits = 0;
  for (int pass = 0; pass < 2; ++pass) {
    const float* s = pass == 0 ? sr : sh;
    Top5 t5;
    t5.init();
    for (int t = tid; t < T; t += kThreads) t5.push(s[t], t);
    for (int k = 0; k < 5; ++k) { s_tv[tid * 5 + k] = t5.v[k]; s_ti[tid * 5 + k] = t5.i[k]; }
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
      if (tid < w) {
        Top5 a;
        for (int k = 0; k < 5; ++k) { a.v[k] = s_tv[tid * 5 + k]; a.i[k] = s_ti[tid * 5 + k]; }
        for (int k = 0; k < 5; ++k) a.push(s_tv[(tid + w) * 5 + k], s_ti[(tid + w) * 5 + k]);
        for (int k = 0; k < 5; ++k) { s_tv[tid * 5 + k] = a.v[k]; s_ti[tid * 5 + k] = a.i[k]; }
      }
      __syncthreads();
    }
    if (tid == 0) {
      if (pass == 0) {
        for (int k = 0; k < 5; ++k) s_top_ref[k] = s_ti[k];
      } else {
        for (int k = 0; k < 5; ++k)
          for (int k2 = 0; k2 < 5; ++k2) hits += (s_ti[k] == s_top_ref[k2] && s_ti[k] < T) ? 1 : 0;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    double* o = p.per_query + (size_t)qi * kPerQuery;
    o[0] = kl;
    o[1] = (double)hits / 5.0;
    o[2] = 0.5 * var;
    o[3] = verr ? a2 : NAN;
    o[4] = mr + log(zr);
  }
}

// o_ref = sum_t p_t v_t over the raw values, p_t = exp(s_ref_t - lse_ref):
// one block per query, wave w takes tokens t = w mod 4, lane i coordinates
// i, i + 64, ...; the four waves' sums meet in LDS.
template <typename TIN>
__global__ __launch_bounds__(kThreads) void attn_ref_kernel(AttnRefParams p) {
  __shared__ float s_acc[kThreads / 64][kMaxD];
  const int qi = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b = qi / p.Hq, kvh = (qi % p.Hq) / p.G, d = p.d;
  const float* sr = p.s_ref + (size_t)qi * p.T;
  const double lse = p.per_query[(size_t)qi * kPerQuery + 4];
  const TIN* v = reinterpret_cast<const TIN*>(p.v) + (int64_t)b * p.vsb + (int64_t)kvh * p.vsh;
  float acc[kMaxD / 64];
#pragma unroll
  for (int c = 0; c < kMaxD / 64; ++c) acc[c] = 0.f;
  for (int t = wave; t < p.T; t += kThreads / 64) {
    const float pt = (float)exp((double)sr[t] - lse);
    const TIN* row = v + (int64_t)t * p.vst;
#pragma unroll
    for (int c = 0; c < kMaxD / 64; ++c)
      if (64 * c + lane < d) acc[c] = fmaf(pt, (float)row[64 * c + lane], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < kMaxD / 64; ++c)
    if (64 * c + lane < d) s_acc[wave][64 * c + lane] = acc[c];
  __syncthreads();
  for (int i = threadIdx.x; i < d; i += kThreads) {
    float o = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) o += s_acc[w][i];
    p.o_ref[(size_t)qi * d + i] = o;
  }
}

template <int KB, bool KQ, bool KS, int VB, bool VQ>
hipError_t launch_split(const DecodeParams& p, hipStream_t s) {
  hipLaunchKernelGGL((decode_split_kernel<KB, KQ, KS, VB, VQ>), dim3(p.units), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int KB, bool KQ, bool KS>
hipError_t launch_ms(const MetricScoreParams& p, hipStream_t s) {
  if (p.kdtype == TQ_F16)
    hipLaunchKernelGGL((metric_scores_kernel<KB, KQ, KS, _Float16>), dim3(p.dp.units), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((metric_scores_kernel<KB, KQ, KS, float>), dim3(p.dp.units), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sproj(const SProjParams& p, hipStream_t s) {
  hipLaunchKernelGGL(sproj_kernel, dim3((p.nq + 15) / 16, p.d / 64), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_qprep(const QPrepParams& p, hipStream_t s) {
  const size_t dyn = p.kspectral ? (size_t)p.d * p.d * sizeof(float) : 0;  // the SPECTRAL basis (d <= 128)
  hipLaunchKernelGGL(qprep_kernel, dim3(p.B * p.Hq), dim3(kThreads), dyn, s, p);
  if (p.kqjl && p.d >= kBigD) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_sproj(SProjParams{p.S, p.qrot, p.qsk, p.B * p.Hq, p.d, 0}, s);
  }
  return hipGetLastError();
}

bool combine_splits(int d, bool vqjl, bool vspectral) { return vqjl && !vspectral && d >= kBigD; }

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const size_t dyn = p.vspectral ? (size_t)p.d * p.d * sizeof(float) : 0;  // the SPECTRAL basis (d <= 128)
  if (combine_splits(p.d, p.vqjl, p.vspectral) && p.ow && p.kw && p.add) {
    CombineParams c = p;
    c.stage = 1;
    hipLaunchKernelGGL(combine_kernel, dim3(p.nq), dim3(kThreads), 0, s, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_sproj(SProjParams{p.S, p.kw, p.add, p.nq, p.d, 1}, s);
    if (e != hipSuccess) return e;
    c.stage = 2;
    hipLaunchKernelGGL(combine_kernel, dim3(p.nq), dim3(kThreads), 0, s, c);
    return hipGetLastError();
  }
  CombineParams c = p;
  c.stage = 0;
  hipLaunchKernelGGL(combine_kernel, dim3(p.nq), dim3(kThreads), dyn, s, c);
  return hipGetLastError();
}

hipError_t launch_metric_reduce(const MetricReduceParams& p, hipStream_t s) {
  hipLaunchKernelGGL(metric_reduce_kernel, dim3(p.nq), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_attn_ref(const AttnRefParams& p, hipStream_t s) {
  if (p.vdtype == TQ_F16)
    hipLaunchKernelGGL(attn_ref_kernel<_Float16>, dim3(p.nq), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(attn_ref_kernel<float>, dim3(p.nq), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// Key variants: (index bits, QJL, side) -> 0..7 ; value variants (bits, QJL).
#define TQ_V_CASES(KB, KQ, KS)                                              \
  switch (vbits * 2 + vqjl) {                                               \
    case 2: return launch_split<KB, KQ, KS, 1, false>(p, s);                \
    case 4: return launch_split<KB, KQ, KS, 2, false>(p, s);                \
    case 6: return launch_split<KB, KQ, KS, 3, false>(p, s);                \
    case 8: return launch_split<KB, KQ, KS, 4, false>(p, s);                \
    case 3: return launch_split<KB, KQ, KS, 1, true>(p, s);                 \
    case 5: return launch_split<KB, KQ, KS, 2, true>(p, s);                 \
    case 7: return launch_split<KB, KQ, KS, 3, true>(p, s);                 \
  }

hipError_t launch_decode_split(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl,
                               hipStream_t s, bool* supported) {
  *supported = true;
  if (kside) {
    if (kbits == 2) { TQ_V_CASES(2, false, true) }
  } else if (kqjl) {
    switch (kbits) {
      case 1: { TQ_V_CASES(1, true, false) } break;
      case 2: { TQ_V_CASES(2, true, false) } break;
      case 3: { TQ_V_CASES(3, true, false) } break;
    }
  } else {
    switch (kbits) {
      case 1: { TQ_V_CASES(1, false, false) } break;
      case 2: { TQ_V_CASES(2, false, false) } break;
      case 3: { TQ_V_CASES(3, false, false) } break;
      case 4: { TQ_V_CASES(4, false, false) } break;
    }
  }
  *supported = false;
  return hipSuccess;
}

hipError_t launch_metric_scores(const MetricScoreParams& p, int kbits, int kqjl, int kside, hipStream_t s,
                                bool* supported) {
  *supported = true;
  if (kside && kbits == 2) return launch_ms<2, false, true>(p, s);
  if (kqjl) {
    switch (kbits) { case 1: return launch_ms<1, true, false>(p, s); case 2: return launch_ms<2, true, false>(p, s);
                     case 3: return launch_ms<3, true, false>(p, s); }
  } else if (!kside) {
    switch (kbits) { case 1: return launch_ms<1, false, false>(p, s); case 2: return launch_ms<2, false, false>(p, s);
                     case 3: return launch_ms<3, false, false>(p, s); case 4: return launch_ms<4, false, false>(p, s); }
  }
  *supported = false;
  return hipSuccess;
}

}  // namespace tq
