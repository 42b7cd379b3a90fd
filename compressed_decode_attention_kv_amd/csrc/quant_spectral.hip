// Write side of SpectralQuant with uniform allocation (SQU-KV) and its
// reconstruction error for tq_metrics.
//
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
//
// [P2] "Configuração Experimental" (SpectralQuant: a calibrated per-head
// eigenbasis) with the uniform allocation of "Recomendações Práticas" 2-3:
// x - mu = nu u (nu = ||x - mu||), z = V^T u, idx_i = #{k : z_i >= s_i t_k}
// against the Lloyd-Max codebook of N(0, 1), every coordinate at the same
// width; x_hat = mu + nu V (s * c[idx]).
//
// The decision is taken in double precision.  A low-rank head has spreads
// s_i of ~1e-3 on its noise coordinates, so its decision boundaries s_i t_k
// sit ~1e-3 apart in the unit-vector domain: float rounding of the
// projection (~1e-7) would move a code at a rate of ~1e-4 per decision.  In
// double the projection z' = V^T (x - mu) is compared with nu s_i t_k
// (no division), all in double, with x and mu converted exactly.
//
// Layout: one block (4 waves) per tile of 8192 / d tokens of one head; the
// head's basis in LDS as float [k][i] (64 KB at d = 128).
//   1. centre: L = d/32 lanes per token (lane j holds coordinates 32 j ..
//      32 j + 31), x - mu into LDS in double, nu (a double sum of squares);
//   2. project: thread (i, g) holds column i of V in registers and forms
//      z'_i of 32 tokens against the broadcast tile rows; index into LDS;
//   3. pack: the token's lanes gather their 32 indices, pack b-bit fields
//      (LSB first) and store them (non-temporal).
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kSqThreads = 256;
constexpr int kSqMaxD = 128;

template <int D>
struct SqGeom {
  static constexpr int L = D / 32;                  // lanes per token
  static constexpr int VPW = 64 / L;                // tokens per wave
  static constexpr int TT = 4 * VPW;                // tokens per tile (8192 / D)
  static constexpr int GROUPS = kSqThreads / D;     // threads per basis column
  static constexpr int TPG = TT / GROUPS;           // tokens per thread in the projection
  static_assert(TPG * GROUPS == TT, "projection split");
};

template <int D, int BITS, typename TIN>
__global__ __launch_bounds__(kSqThreads) void quant_spectral_kernel(QuantParams p) {
  using G = SqGeom<D>;
  constexpr int NB = (1 << BITS) - 1;
  __shared__ float s_basis[D * D];              // V[k][i]
  __shared__ double s_x[G::TT * D];             // x - mu, row per token
  __shared__ double s_nu[G::TT];
  __shared__ uint8_t s_idx[G::TT * D];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (G::L - 1), slot = lane / G::L;
  const int tph = (p.T + G::TT - 1) / G::TT;
  const int bh = blockIdx.x / tph;
  const int t0 = (blockIdx.x - bh * tph) * G::TT;
  const int b = bh / p.H, h = bh - b * p.H;
  const float* basis = p.basis + (size_t)h * D * D;
  const float* mean = p.smean + (size_t)h * D;
  const float* scale = p.sscale + (size_t)h * D;
  for (int i = threadIdx.x; i < D * D; i += kSqThreads) s_basis[i] = basis[i];

  // ---- 1. centre the tile's tokens, norms ------------------------------------------
  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t slot0 = p.pos ? p.pos[b] : 0;
  const size_t vbase = (size_t)bh * p.T_cap;
  {
    const int m = wave * G::VPW + slot;
    const int t = t0 + m;
    const bool valid = t < p.T;
    float v[32];
    load32<TIN>(xbase + (int64_t)min(t, p.T - 1) * p.st + 32 * j, v);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const double xc = valid ? (double)v[e] - (double)mean[32 * j + e] : 0.0;
      s_x[m * D + 32 * j + e] = xc;
      ss = fma(xc, xc, ss);
    }
    for (int off = 1; off < G::L; off <<= 1) ss += __shfl_xor(ss, off, 64);
    const double nu = sqrt(ss);
    if (j == 0) s_nu[m] = nu;
    const int64_t tw = slot0 + t;
    if (valid && j == 0 && tw >= 0 && tw < p.T_cap) __builtin_nontemporal_store((float)nu, p.norms + vbase + tw);
  }
  __syncthreads();

  // ---- 2. z'_i = sum_k V[k][i] (x_k - mu_k) and the index, in double ---------------
  {
    const int i = threadIdx.x % D, g = threadIdx.x / D;
    float col[D];
#pragma unroll
    for (int k = 0; k < D; ++k) col[k] = s_basis[k * D + i];
    const double si = (double)scale[i];
    double thr[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) thr[k] = si * p.gbounds[k];
    for (int u = 0; u < G::TPG; ++u) {
      const int m = g * G::TPG + u;
      const double* xr = s_x + m * D;
      double acc0 = 0.0, acc1 = 0.0, acc2 = 0.0, acc3 = 0.0;
#pragma unroll
      for (int k = 0; k < D; k += 4) {
        acc0 = fma((double)col[k], xr[k], acc0);
        acc1 = fma((double)col[k + 1], xr[k + 1], acc1);
        acc2 = fma((double)col[k + 2], xr[k + 2], acc2);
        acc3 = fma((double)col[k + 3], xr[k + 3], acc3);
      }
      const double z = (acc0 + acc1) + (acc2 + acc3);
      const double nu = s_nu[m];
      uint32_t c = 0;
#pragma unroll
      for (int k = 0; k < NB; ++k) c += (z >= nu * thr[k]) ? 1u : 0u;
      s_idx[m * D + i] = (uint8_t)(nu > 0.0 ? c : 0u);
    }
  }
  __syncthreads();

  // ---- 3. pack and store ------------------------------------------------------------
  {
    const int m = wave * G::VPW + slot;
    const int t = t0 + m;
    const int64_t tw = slot0 + t;
    if (t < p.T && tw >= 0 && tw < p.T_cap) {
      uint32_t w[BITS];
#pragma unroll
      for (int k = 0; k < BITS; ++k) w[k] = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t c = s_idx[m * D + 32 * j + e];
        const int bit = BITS * e, wi = bit >> 5, sh = bit & 31;
        w[wi] |= c << sh;
        if (sh + BITS > 32) w[wi + 1] |= c >> (32 - sh);
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + (vbase + tw) * (size_t)(D * BITS / 8)) + j * BITS;
#pragma unroll
      for (int k = 0; k < BITS; ++k) __builtin_nontemporal_store(w[k], dst + k);
    }
  }
}

// Reconstruction error of a SPECTRAL tensor against its raw input, with the
// block layout of relerr_kernel (4 waves, 4 steps of 64/L tokens per wave):
// x_hat = mu + nu V (s * c[idx]) densely in the original domain, lane j its
// 32 coordinates.
constexpr int kRelSteps = 4;

template <int D, int BITS, typename TIN>
__global__ __launch_bounds__(kSqThreads) void relerr_spectral_kernel(RelErrParams p) {
  constexpr int L = D / 32, VPW = 64 / L;
  __shared__ float s_basis[D * D];
  __shared__ float s_y[4 * VPW * D];            // per wave: its tokens' s * c[idx]
  __shared__ float s_cent[16];
  __shared__ double s_red[kSqThreads / 64][5];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & (L - 1), slot = lane / L;
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const float* basis = p.basis + (size_t)h * D * D;
  const float* mean = p.smean + (size_t)h * D;
  const float* scale = p.sscale + (size_t)h * D;
  for (int i = threadIdx.x; i < D * D; i += kSqThreads) s_basis[i] = basis[i];
  if (threadIdx.x < 16) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  __syncthreads();
  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t vbase = (int64_t)bh * p.T_cap;
  double e2 = 0.0, r2 = 0.0, dsum = 0.0, cnt = 0.0, asum = 0.0;
  float* yrow = s_y + (wave * VPW + slot) * D;
  for (int step = 0; step < kRelSteps; ++step) {
    const int t = blockIdx.x * (4 * VPW * kRelSteps) + (step * 4 + wave) * VPW + slot;
    const bool valid = t < p.T;
    const int tc = valid ? t : p.T - 1;
    const int64_t vec = vbase + tc;
    float a[32];
    load32<TIN>(xbase + (int64_t)tc * p.st + 32 * j, a);
    uint32_t w[BITS];
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(p.planes.codes + vec * (D * BITS / 8)) + j * BITS;
#pragma unroll
    for (int k = 0; k < BITS; ++k) w[k] = cw[k];
    const float nu = p.planes.norms[vec];
#pragma unroll
    for (int e = 0; e < 32; ++e) yrow[32 * j + e] = scale[32 * j + e] * s_cent[code_at<BITS>(w, e)];
    __syncthreads();
    float ah[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) ah[e] = 0.f;
    const float* vr = s_basis + (32 * j) * D;
#pragma unroll 2
    for (int i = 0; i < D; ++i) {
      const float yi = yrow[i];
#pragma unroll
      for (int e = 0; e < 32; ++e) ah[e] = fmaf(vr[e * D + i], yi, ah[e]);
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) ah[e] = mean[32 * j + e] + nu * ah[e];
    __syncthreads();
    float le2 = 0.f, lr2 = 0.f, ldot = 0.f, lh2 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float df = a[e] - ah[e];
      le2 = fmaf(df, df, le2);
      lr2 = fmaf(a[e], a[e], lr2);
      ldot = fmaf(a[e], ah[e], ldot);
      lh2 = fmaf(ah[e], ah[e], lh2);
    }
    le2 = group_sum(le2, L); lr2 = group_sum(lr2, L);
    ldot = group_sum(ldot, L); lh2 = group_sum(lh2, L);
    if (valid && j == 0) {
      e2 += le2; r2 += lr2;
      if (lr2 > 0.f && lh2 > 0.f) {
        const double c = (double)ldot / sqrt((double)lr2 * (double)lh2);
        dsum += 1.0 - c;
        asum += acos(fmin(1.0, fmax(-1.0, c)));
        cnt += 1.0;
      }
      if (p.per_vec) p.per_vec[vec] = le2;
    }
  }
  for (int m = 1; m < 64; m <<= 1) {
    e2 += __shfl_xor(e2, m, 64); r2 += __shfl_xor(r2, m, 64);
    dsum += __shfl_xor(dsum, m, 64); cnt += __shfl_xor(cnt, m, 64);
    asum += __shfl_xor(asum, m, 64);
  }
  if (lane == 0) {
    s_red[wave][0] = e2; s_red[wave][1] = r2; s_red[wave][2] = dsum; s_red[wave][3] = cnt; s_red[wave][4] = asum;
  }
  __syncthreads();
  if (threadIdx.x < 5) {
    double s = 0.0;
    for (int wv = 0; wv < kSqThreads / 64; ++wv) s += s_red[wv][threadIdx.x];
    p.block_sums[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 5 + threadIdx.x] = s;
  }
}

template <int D, int BITS>
hipError_t launch_sq(const QuantParams& p, hipStream_t s) {
  const long tiles = (long)p.B * p.H * ((p.T + SqGeom<D>::TT - 1) / SqGeom<D>::TT);
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((quant_spectral_kernel<D, BITS, _Float16>), dim3((unsigned)tiles), dim3(kSqThreads), 0, s, p);
  else
    hipLaunchKernelGGL((quant_spectral_kernel<D, BITS, float>), dim3((unsigned)tiles), dim3(kSqThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sq_d(const QuantParams& p, hipStream_t s) {
  switch (p.bits) {
    case 1: return launch_sq<D, 1>(p, s);
    case 2: return launch_sq<D, 2>(p, s);
    case 3: return launch_sq<D, 3>(p, s);
    case 4: return launch_sq<D, 4>(p, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int BITS>
hipError_t launch_rsq(const RelErrParams& p, hipStream_t s) {
  constexpr int VPW = 64 / (D / 32);
  dim3 grid((p.T + 4 * VPW * kRelSteps - 1) / (4 * VPW * kRelSteps), p.B * p.H);
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((relerr_spectral_kernel<D, BITS, _Float16>), grid, dim3(kSqThreads), 0, s, p);
  else
    hipLaunchKernelGGL((relerr_spectral_kernel<D, BITS, float>), grid, dim3(kSqThreads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_rsq_d(const RelErrParams& p, hipStream_t s) {
  switch (p.bits) {
    case 1: return launch_rsq<D, 1>(p, s);
    case 2: return launch_rsq<D, 2>(p, s);
    case 3: return launch_rsq<D, 3>(p, s);
    case 4: return launch_rsq<D, 4>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int spectral_max_d() { return kSqMaxD; }

hipError_t launch_quantize_spectral(const QuantParams& p, hipStream_t s) {
  switch (p.d) {
    case 32: return launch_sq_d<32>(p, s);
    case 64: return launch_sq_d<64>(p, s);
    case 128: return launch_sq_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_relerr_spectral(const RelErrParams& p, hipStream_t s) {
  switch (p.d) {
    case 32: return launch_rsq_d<32>(p, s);
    case 64: return launch_rsq_d<64>(p, s);
    case 128: return launch_rsq_d<128>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
