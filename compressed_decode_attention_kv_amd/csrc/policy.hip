// A^2-weighted value policy: the per-token weights, the selection of the
// high-precision value tier, the token permutation, the gather of a tier's
// tokens and the log-sum-exp merge of two tiers' attention.
//
// [P3] = "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
//        Espaço de Pontuação para Quantização de KV-Cache"
//
// [P3] section 2.2 takes sum_j p_j^2 ||dv_j||^2 as the value read error;
// section 5 pairs HeadQ keys with a value policy weighted by it.  Here:
//   weights    A_j = mean over the probe queries of a KV head of p_j(q)^2,
//              p(q) the softmax of q^T k_j / sqrt(d) over the raw keys;
//   gains      w_j = A_j ||v_j||^2;
//   selection  the R largest w_j of each (batch, head), ties to the lower
//              index, by a 4-pass radix select on the float bits (w >= 0,
//              so the bit patterns order like the values);
//   layout     the high tier first, each tier in increasing token order;
//              attention is order-invariant, so each tier is an ordinary
//              packed cache and the two attentions merge by log-sum-exp.
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kPThreads = 256;
constexpr int kSelThreads = 1024;

// ---- A^2 weights ----------------------------------------------------------------
// Scores of all P probes of one KV head against a chunk of its raw keys:
// L = d/32 lanes per token, the probes in LDS, each key read once.
template <typename TIN>
__global__ __launch_bounds__(kPThreads) void a2_scores_kernel(A2Params p) {
  extern __shared__ float s_probe[];    // [P][d]
  const int bkv = blockIdx.y, b = bkv / p.Hkv, kvh = bkv % p.Hkv;
  const int d = p.d, L = d / 32, vpw = 64 / L, P = p.P;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (L - 1), slot = lane / L;
  // Probe rows of this KV head: query heads kvh*G .. kvh*G + G - 1, each with Np probes.
  const int row0 = (b * p.Hq + kvh * p.G) * p.Np;
  for (int i = threadIdx.x; i < P * d; i += kPThreads) {
    const int r = i / d, c = i - r * d;
    const int hq = kvh * p.G + r / p.Np, n = r % p.Np;
    const int64_t off = (int64_t)b * p.qsb + (int64_t)hq * p.qsh + (int64_t)n * p.qst + c;
    s_probe[i] = p.qdtype == TQ_F16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off]
                                    : reinterpret_cast<const float*>(p.q)[off];
  }
  __syncthreads();
  const TIN* kb = reinterpret_cast<const TIN*>(p.k) + (int64_t)b * p.ksb + (int64_t)kvh * p.ksh;
  const int t0 = blockIdx.x * p.chunk, t1 = min(p.T, t0 + p.chunk);
  for (int base = t0 + wave * vpw; base < t1; base += 4 * vpw) {
    const int t = base + slot;
    const bool valid = t < t1;
    float kv[32];
    load32<TIN>(kb + (int64_t)(valid ? t : t1 - 1) * p.kst + 32 * j, kv);
    for (int r = 0; r < P; ++r) {
      const float* qr = s_probe + r * d + 32 * j;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc = fmaf(qr[e], kv[e], acc);
      acc = group_sum(acc, L) * p.inv_sqrt_d;
      if (valid && j == 0) p.scores[(size_t)(row0 + r) * p.T + t] = acc;
    }
  }
}

// Log-sum-exp of one probe row (one block per row), in double.
__global__ __launch_bounds__(kPThreads) void a2_lse_kernel(A2Params p) {
  __shared__ double s_red[kPThreads / 64];
  const int row = blockIdx.x;
  const float* s = p.scores + (size_t)row * p.T;
  auto block_reduce = [&](double v, bool is_max) {
    for (int m = 32; m > 0; m >>= 1) {
      const double o = __shfl_xor(v, m, 64);
      v = is_max ? fmax(v, o) : v + o;
    }
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = s_red[0];
    for (int w = 1; w < kPThreads / 64; ++w) r = is_max ? fmax(r, s_red[w]) : r + s_red[w];
    __syncthreads();
    return r;
  };
  double m = -INFINITY;
  for (int t = threadIdx.x; t < p.T; t += kPThreads) m = fmax(m, (double)s[t]);
  m = block_reduce(m, true);
  double z = 0.0;
  for (int t = threadIdx.x; t < p.T; t += kPThreads) z += exp((double)s[t] - m);
  z = block_reduce(z, false);
  if (threadIdx.x == 0) p.lse[row] = m + log(z);
}

// A[bkv][t] = (1/P) sum over the head's probes of exp(2 (s - lse)).
__global__ __launch_bounds__(kPThreads) void a2_weight_kernel(A2Params p) {
  const int bkv = blockIdx.y, b = bkv / p.Hkv, kvh = bkv % p.Hkv;
  const int t = blockIdx.x * kPThreads + threadIdx.x;
  if (t >= p.T) return;
  const int row0 = (b * p.Hq + kvh * p.G) * p.Np;
  double acc = 0.0;
  for (int r = 0; r < p.P; ++r) {
    const double e = (double)p.scores[(size_t)(row0 + r) * p.T + t] - p.lse[row0 + r];
    acc += exp(2.0 * e);
  }
  p.weights[(size_t)bkv * p.T + t] = (float)(acc / p.P);
}

// ---- gains --------------------------------------------------------------------
template <typename TIN>
__global__ __launch_bounds__(kPThreads) void gain_kernel(PolicyParams p) {
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int L = p.d / 32, vpw = 64 / L;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (L - 1), slot = lane / L;
  const TIN* vb = reinterpret_cast<const TIN*>(p.v) + (int64_t)b * p.vsb + (int64_t)h * p.vsh;
  const int t = (blockIdx.x * 4 + wave) * vpw + slot;
  const bool valid = t < p.T;
  float x[32];
  load32<TIN>(vb + (int64_t)(valid ? t : p.T - 1) * p.vst + 32 * j, x);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) ss = fmaf(x[e], x[e], ss);
  ss = group_sum(ss, L);
  if (valid && j == 0) p.gain[(size_t)bh * p.T + t] = p.weights[(size_t)bh * p.T + t] * ss;
}

// ---- selection ------------------------------------------------------------------
// Block-wide inclusive prefix sum of one int per thread (1024 threads).
__device__ int block_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      const int c = s_wave[w];
      s_wave[w] = acc;
      acc += c;
    }
    s_wave[kSelThreads / 64] = acc;
  }
  __syncthreads();
  const int r = x + s_wave[wave];
  *total = s_wave[kSelThreads / 64];
  __syncthreads();
  return r;
}

// For each candidate count R_c of one (batch, head): the bit pattern of the
// R_c-th largest gain, how many of its equals are taken, and the sum of the
// R_c largest gains; also the sum of all gains.
__global__ __launch_bounds__(kSelThreads) void select_kernel(PolicyParams p) {
  __shared__ int s_hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  __shared__ double s_red[kSelThreads / 64];
  const int bh = blockIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(p.gain + (size_t)bh * p.T);
  auto block_sum = [&](double v) {
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
    for (int w = 0; w < kSelThreads / 64; ++w) r += s_red[w];
    __syncthreads();
    return r;
  };
  double all = 0.0;
  for (int t = threadIdx.x; t < p.T; t += kSelThreads) all += (double)__uint_as_float(key[t]);
  all = block_sum(all);
  if (threadIdx.x == 0) p.total[bh] = all;
  for (int c = 0; c < p.ncand; ++c) {
    const int R = p.cand_R[c];
    PolicySel out{0u, 0, 0.0};
    if (R > 0) {
      uint32_t prefix = 0, mask = 0;
      if (threadIdx.x == 0) s_remaining = R;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < 256; i += kSelThreads) s_hist[i] = 0;
        __syncthreads();
        for (int t = threadIdx.x; t < p.T; t += kSelThreads) {
          const uint32_t k = key[t];
          if ((k & mask) == prefix) atomicAdd(&s_hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
          int rem = s_remaining, dg = 255;
          for (; dg > 0; --dg) {
            if (s_hist[dg] >= rem) break;
            rem -= s_hist[dg];
          }
          s_remaining = rem;
          s_prefix = prefix | ((uint32_t)dg << shift);
        }
        __syncthreads();
        prefix = s_prefix;
        mask |= 255u << shift;
      }
      // prefix is the R-th largest pattern; s_remaining of its equals are taken.
      const int need_eq = s_remaining;
      double above = 0.0;
      for (int t = threadIdx.x; t < p.T; t += kSelThreads)
        if (key[t] > prefix) above += (double)__uint_as_float(key[t]);
      above = block_sum(above);
      out.thr = prefix;
      out.need_eq = need_eq;
      out.top = above + need_eq * (double)__uint_as_float(prefix);
    }
    if (threadIdx.x == 0) p.sel[(size_t)bh * p.ncand + c] = out;
    __syncthreads();
  }
}

// Permutation of one (batch, head) for the chosen candidate: selected tokens
// (gain above the threshold, or equal to it among the first need_eq equals)
// at [0, R) in token order, the rest at [R, T) in token order.
__global__ __launch_bounds__(kSelThreads) void permute_kernel(PolicyParams p) {
  __shared__ int s_wave[kSelThreads / 64 + 1];
  const int bh = blockIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(p.gain + (size_t)bh * p.T);
  const PolicySel sel = p.sel[(size_t)bh * p.ncand + p.chosen];
  const int R = p.cand_R[p.chosen];
  int32_t* perm = p.perm + (size_t)bh * p.T;
  int eq_before = 0, sel_before = 0;
  for (int base = 0; base < p.T; base += kSelThreads) {
    const int t = base + threadIdx.x;
    const uint32_t k = t < p.T ? key[t] : 0u;
    const bool in = t < p.T && R > 0;
    const int eq = (in && k == sel.thr) ? 1 : 0;
    int eq_total;
    const int eq_incl = block_scan(eq, s_wave, &eq_total);
    const int eq_rank = eq_before + eq_incl - eq;
    const int s = (in && (k > sel.thr || (eq && eq_rank < sel.need_eq))) ? 1 : 0;
    int s_total;
    const int s_incl = block_scan(s, s_wave, &s_total);
    const int s_excl = sel_before + s_incl - s;
    if (t < p.T) perm[s ? s_excl : R + (t - s_excl)] = t;
    eq_before += eq_total;
    sel_before += s_total;
  }
}

// ---- gather and merge -------------------------------------------------------------
// out[b][h][t] = x[b][h][perm[b][h][t0 + t]] for t < tn; 16-byte chunks.
__global__ __launch_bounds__(kPThreads) void gather_kernel(GatherParams p) {
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int chunks = p.row_bytes / 16;
  const int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
  if (i >= (int64_t)p.tn * chunks) return;
  const int t = (int)(i / chunks), c = (int)(i - (int64_t)t * chunks);
  const int src = p.perm[(size_t)bh * p.T + p.t0 + t];
  const char* sx = reinterpret_cast<const char*>(p.x) + ((int64_t)b * p.xsb + (int64_t)h * p.xsh + (int64_t)src * p.xst) * p.es;
  char* so = reinterpret_cast<char*>(p.out) + ((int64_t)b * p.osb + (int64_t)h * p.osh + (int64_t)t * p.ost) * p.es;
  *reinterpret_cast<uint4*>(so + 16 * c) = *reinterpret_cast<const uint4*>(sx + 16 * c);
}

__global__ __launch_bounds__(kPThreads) void merge_kernel(MergeParams p) {
  const int64_t i = (int64_t)blockIdx.x * kPThreads + threadIdx.x;
  if (i >= (int64_t)p.n * p.d) return;
  const int q = (int)(i / p.d);
  const float la = p.lse_a[q], lb = p.lse_b[q];
  const float m = fmaxf(la, lb);
  float wa = 0.f, wb = 0.f, l = -INFINITY;
  if (m != -INFINITY) {
    const float ea = expf(la - m), eb = expf(lb - m);
    wa = ea / (ea + eb);
    wb = eb / (ea + eb);
    l = m + logf(ea + eb);
  }
  p.out[i] = wa * p.out_a[i] + wb * p.out_b[i];
  if (p.lse && i % p.d == 0) p.lse[q] = l;
}

}  // namespace

// The same scores on the matrix cores: per wave 16 tokens x 16 probes per
// v_mfma_f32_16x16x32_f16 product, the contraction over d in steps of 32.
// Keys enter exact (fp16) or as fp16 hi + lo (fp32); the probes as fp16 hi +
// lo parts (about 22 bits), held in LDS in operand order: (probe block pb,
// step ks, lane (h, n)) holds coordinates 32 ks + 8 h .. + 7 of probe
// 16 pb + n (zero past the last probe).  Lane (h, t) takes token t's
// coordinates 32 ks + 8 h .. + 7; the result hands lane (h, n) tokens
// 4 h .. 4 h + 3 of probe 16 pb + n.
typedef _Float16 a2_half8 __attribute__((ext_vector_type(8)));
typedef float a2_float4 __attribute__((ext_vector_type(4)));

template <typename TIN, int NPB>
__global__ __launch_bounds__(kPThreads) void a2_scores_mfma_kernel(A2Params p) {
  extern __shared__ __attribute__((aligned(16))) char s_raw[];
  const int d = p.d, KS = d / 32, P = p.P;
  a2_half8* s_qh = reinterpret_cast<a2_half8*>(s_raw);
  a2_half8* s_ql = s_qh + NPB * KS * 64;
  const int bkv = blockIdx.y, b = bkv / p.Hkv, kvh = bkv % p.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hq = lane >> 4, mm = lane & 15;
  const int row0 = (b * p.Hq + kvh * p.G) * p.Np;
  for (int i = threadIdx.x; i < NPB * KS * 64; i += kPThreads) {
    const int l = i & 63, pk = i >> 6, ks = pk % KS, pb = pk / KS;
    const int r = 16 * pb + (l & 15), c = 32 * ks + 8 * (l >> 4);
    a2_half8 h, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = 0.f;
      if (r < P) {
        const int hq2 = kvh * p.G + r / p.Np, n = r % p.Np;
        const int64_t off = (int64_t)b * p.qsb + (int64_t)hq2 * p.qsh + (int64_t)n * p.qst + c + e;
        v = p.qdtype == TQ_F16 ? (float)reinterpret_cast<const _Float16*>(p.q)[off]
                               : reinterpret_cast<const float*>(p.q)[off];
      }
      h[e] = (_Float16)v;
      lo[e] = (_Float16)(v - (float)h[e]);
    }
    s_qh[i] = h;
    s_ql[i] = lo;
  }
  __syncthreads();
  const TIN* kb = reinterpret_cast<const TIN*>(p.k) + (int64_t)b * p.ksb + (int64_t)kvh * p.ksh;
  const int t0 = blockIdx.x * p.chunk, t1 = min(p.T, t0 + p.chunk);
  for (int base = t0 + 16 * wave; base < t1; base += 16 * (kPThreads / 64)) {
    const TIN* krow = kb + (int64_t)min(base + mm, t1 - 1) * p.kst + 8 * hq;
    a2_float4 S[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) S[pb] = a2_float4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      a2_half8 kh, kl;
      if constexpr (sizeof(TIN) == 2) {
        kh = *reinterpret_cast<const a2_half8*>(krow + 32 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = krow[32 * ks + e];
          kh[e] = (_Float16)v;
          kl[e] = (_Float16)(v - (float)kh[e]);
        }
      }
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const a2_half8 qh = s_qh[(pb * KS + ks) * 64 + lane], ql = s_ql[(pb * KS + ks) * 64 + lane];
        S[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qh, S[pb], 0, 0, 0);
        S[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, ql, S[pb], 0, 0, 0);
        if constexpr (sizeof(TIN) == 4) S[pb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qh, S[pb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      const int r = 16 * pb + mm;
      if (r >= P) continue;
      float* dst = p.scores + (size_t)(row0 + r) * p.T;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = base + 4 * hq + i;
        if (t < t1) dst[t] = S[pb][i] * p.inv_sqrt_d;
      }
    }
  }
}

size_t a2_workspace_bytes(int rows, int T) {
  return ((size_t)rows * T * 4 + 255) / 256 * 256 + (size_t)rows * 8;
}

hipError_t launch_a2_weights(const A2Params& p, hipStream_t s) {
  const int L = p.d / 32;
  const dim3 g1((p.T + p.chunk - 1) / p.chunk, p.B * p.Hkv);
  const size_t dyn = (size_t)p.P * p.d * sizeof(float);
  (void)L;
  // Up to 64 probes per KV head on the matrix cores (chunks of whole 64-token
  // block steps); more on the vector units.
  const int npb = (p.P + 15) / 16;
  if (npb <= 4 && p.d % 32 == 0 && p.chunk % 64 == 0) {
    const int nb = npb <= 1 ? 1 : (npb <= 2 ? 2 : 4);
    const size_t dq = (size_t)2 * nb * 16 * p.d * sizeof(_Float16);
    const bool f16 = p.kdtype == TQ_F16;
#define TQ_A2M(NB)                                                                                   \
    if (nb == NB) {                                                                                  \
      if (f16) hipLaunchKernelGGL((a2_scores_mfma_kernel<_Float16, NB>), g1, dim3(kPThreads), dq, s, p); \
      else hipLaunchKernelGGL((a2_scores_mfma_kernel<float, NB>), g1, dim3(kPThreads), dq, s, p);       \
    }
    TQ_A2M(1) TQ_A2M(2) TQ_A2M(4)
#undef TQ_A2M
  } else if (p.kdtype == TQ_F16) {
    hipLaunchKernelGGL(a2_scores_kernel<_Float16>, g1, dim3(kPThreads), dyn, s, p);
  } else {
    hipLaunchKernelGGL(a2_scores_kernel<float>, g1, dim3(kPThreads), dyn, s, p);
  }
  hipLaunchKernelGGL(a2_lse_kernel, dim3(p.B * p.Hq * p.Np), dim3(kPThreads), 0, s, p);
  hipLaunchKernelGGL(a2_weight_kernel, dim3((p.T + kPThreads - 1) / kPThreads, p.B * p.Hkv), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_policy_select(const PolicyParams& p, hipStream_t s) {
  const int vpw = 64 / (p.d / 32);
  const dim3 g((p.T + 4 * vpw - 1) / (4 * vpw), p.B * p.H);
  if (p.vdtype == TQ_F16)
    hipLaunchKernelGGL(gain_kernel<_Float16>, g, dim3(kPThreads), 0, s, p);
  else
    hipLaunchKernelGGL(gain_kernel<float>, g, dim3(kPThreads), 0, s, p);
  hipLaunchKernelGGL(select_kernel, dim3(p.B * p.H), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_policy_permute(const PolicyParams& p, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(p.B * p.H), dim3(kSelThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.tn * (p.row_bytes / 16);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((n + kPThreads - 1) / kPThreads), p.B * p.H), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.n * p.d;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + kPThreads - 1) / kPThreads)), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tq
