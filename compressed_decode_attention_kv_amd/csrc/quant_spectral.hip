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

// ---- d = 128 on the matrix cores, decisions certified --------------------------------
// The projection z' = V^T (x - mu) of a tile of 64 tokens is a [64 x 128] x
// [128 x 128] product: v_mfma_f32_32x32x16_f16 on fp16 hi + lo splits of the
// centred inputs (scaled by sigma = 2^(13 - e), nu in [2^(e-1), 2^e), so
// sigma nu in [2^12, 2^13)) and of V (scaled by 2^12), the hi x hi products
// in four accumulators of 32 terms each and the hi x lo + lo x hi terms in a
// fifth.  In the unit domain (z = z' / nu) the computed value is within
// kSmEps of the exact one: 2 * 2^-24 per addition over 32 terms against
// sum |terms| <= 1 (Cauchy-Schwarz, the columns of V are unit vectors), plus
// the dropped lo x lo term (2^-22), the split and centring roundings and
// fp16 denormals (each < 4e-7).  A decision is certified when no boundary
// s_i t_k lies within kSmEps of z; the others (a few per thousand) are
// queued and recomputed exactly in double, as the fp64 kernel above does
// for every decision.
constexpr int kSmThreads = 256;
constexpr int kSmD = 128;
constexpr int kSmTT = 64;                 // tokens per tile
constexpr int kSmRow = kSmD + 8;          // fp16 per A row: rows 4 banks apart
constexpr int kSmIRow = kSmD + 16;        // bytes per index row: rows 4 banks apart
constexpr int kSmQueue = 4096;
constexpr int kSmLutMax = 256;
constexpr int kSmTilesPerBlock = 16;
constexpr float kSmEps = 8e-6f;
constexpr float kSmVScale = 4096.0f;      // V x 2^12 before the split

typedef _Float16 sm_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 sm_half2 __attribute__((ext_vector_type(2)));
typedef float sm_float16 __attribute__((ext_vector_type(16)));
typedef float sm_float4 __attribute__((ext_vector_type(4)));

struct SmLut {
  float t;
  uint32_t base;
};

// The exact recomputations read V and the raw inputs from global memory (L2):
// they are rare, and without copies of them here a block fits twice per CU.
struct SmShared {
  _Float16 ah[kSmTT * kSmRow];      // sigma (x - mu), fp16 hi
  _Float16 al[kSmTT * kSmRow];      // and lo
  uint8_t idx[kSmTT * kSmIRow];
  uint16_t queue[kSmQueue];         // (token << 7) | coordinate of uncertain decisions
  float mean[kSmD], scale[kSmD];
  double nu[kSmTT];
  float zinv[kSmTT];                // 1 / (sigma 2^12 nu), 0 for a zero (or padding) token
  SmLut lut[kSmLutMax];
  int qcount;
};

template <int BITS, typename TIN>
__global__ __launch_bounds__(kSmThreads) void quant_spectral_mfma_kernel(QuantParams p, QuantGrid grid) {
  constexpr int NB = (1 << BITS) - 1;
  __shared__ __attribute__((aligned(16))) SmShared sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 3, slot = lane >> 2;        // phase 1: 4 lanes per token, 32 coordinates each
  const int hh = lane >> 5, mm = lane & 31;        // phases 2-3: operand / result lane
  const int tph = (p.T + kSmTT - 1) / kSmTT;        // tiles per head
  const int cph = (tph + kSmTilesPerBlock - 1) / kSmTilesPerBlock;
  const int bh = blockIdx.x / cph;
  const int tile0 = (blockIdx.x - bh * cph) * kSmTilesPerBlock;
  const int tile1 = min(tph, tile0 + kSmTilesPerBlock);
  const int b = bh / p.H, h = bh - b * p.H;

  // ---- per head: mean, spreads, the grid table; B operands in registers ------------
  const float* V = p.basis + (size_t)h * kSmD * kSmD;
  {
    if (threadIdx.x < kSmD) {
      sh.mean[threadIdx.x] = p.smean[(size_t)h * kSmD + threadIdx.x];
      sh.scale[threadIdx.x] = p.sscale[(size_t)h * kSmD + threadIdx.x];
    }
    for (int n = threadIdx.x; n < grid.cells; n += kSmThreads) {
      const float lo = ((float)(n - 1) - 0.5f - (float)grid.center) / grid.scale;
      const float hi = ((float)(n + 1) + 0.5f - (float)grid.center) / grid.scale;
      uint32_t base = 0;
      float t = INFINITY;
      for (int k = 0; k < NB; ++k) {
        const float bk = p.bounds[k];
        if (bk < lo) base++;
        else if (bk < hi && t == INFINITY) t = bk;
      }
      sh.lut[n].t = t;
      sh.lut[n].base = base;
    }
  }
  __syncthreads();
  // Wave w owns eigen-coordinates 32 w .. 32 w + 31; lane (hh, mm) holds V[k][32 w + mm]
  // for k = 16 ks + 8 hh + e, e < 8, as fp16 hi + lo of V x 2^12.
  const int col = 32 * wave + mm;
  sm_half8 Bh[8], Bl[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const float* src = V + (size_t)(16 * ks + 8 * hh) * kSmD + col;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = src[(size_t)e * kSmD] * kSmVScale;
      const _Float16 hi = (_Float16)v;
      Bh[ks][e] = hi;
      Bl[ks][e] = (_Float16)(v - (float)hi);
    }
  }
  const float s_col = sh.scale[col];
  const float inv_s = s_col > 0.f ? 1.0f / s_col : 0.f;
  float tmax = 0.f;
  for (int k = 0; k < NB; ++k) tmax = fmaxf(tmax, fabsf(p.bounds[k]));
  const float umax = tmax + 2.0f / grid.scale;
  const bool lut_ok = s_col * grid.scale > 2.0f * kSmEps;  // margin within one grid cell in u
  const float gbias = 12582912.0f + (float)grid.center;

  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t slot0 = p.pos ? p.pos[b] : 0;
  const size_t vbase = (size_t)bh * p.T_cap;
  const int m1 = wave * 16 + slot;                  // phase-1 token of this lane
  float xin[32];
  auto load_tile = [&](int tile) {
    const int t = tile * kSmTT + m1;
    load32<TIN>(xbase + (int64_t)min(t, p.T - 1) * p.st + 32 * j, xin);
    if (t >= p.T) {
#pragma unroll
      for (int e = 0; e < 32; ++e) xin[e] = 0.f;
    }
  };
  if (tile0 < tile1) load_tile(tile0);

  for (int tile = tile0; tile < tile1; ++tile) {
    const int tt0 = tile * kSmTT;
    // ---- 1. centre, norm (double), scale, split into the A tile -----------------------
    {
      float mu[32];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const sm_float4 v4 = *reinterpret_cast<const sm_float4*>(sh.mean + 32 * j + 4 * q);
        mu[4 * q] = v4.x; mu[4 * q + 1] = v4.y; mu[4 * q + 2] = v4.z; mu[4 * q + 3] = v4.w;
      }
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const double xc = (double)xin[e] - (double)mu[e];
        ss = fma(xc, xc, ss);
      }
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      const double nu = sqrt(ss);
      int ex = 0;
      (void)frexp(nu, &ex);
      // x - mu in fp32 (one rounding, within the margin), times a power of two.
      const float sigma = nu > 0.0 ? ldexpf(1.0f, 13 - ex) : 0.f;
      _Float16* dh = sh.ah + m1 * kSmRow + 32 * j;
      _Float16* dl = sh.al + m1 * kSmRow + 32 * j;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sm_half8 h8, l8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = (xin[8 * q + e] - mu[8 * q + e]) * sigma;
          const _Float16 hi = (_Float16)v;
          h8[e] = hi;
          l8[e] = (_Float16)(v - (float)hi);
        }
        *reinterpret_cast<sm_half8*>(dh + 8 * q) = h8;
        *reinterpret_cast<sm_half8*>(dl + 8 * q) = l8;
      }
      if (j == 0) {
        sh.nu[m1] = nu;
        sh.zinv[m1] = nu > 0.0 ? (float)(1.0 / ((double)sigma * (double)kSmVScale * nu)) : 0.f;
        const int t = tt0 + m1;
        const int64_t tw = slot0 + t;
        if (t < p.T && tw >= 0 && tw < p.T_cap) __builtin_nontemporal_store((float)nu, p.norms + vbase + tw);
      }
      if (threadIdx.x == 0) sh.qcount = 0;
    }
    __syncthreads();
    if (tile + 1 < tile1) load_tile(tile + 1);     // in flight during phases 2-5

    // ---- 2./3. projection on the matrix cores, certified decisions ---------------------
#pragma unroll 1
    for (int tb = 0; tb < 2; ++tb) {
      sm_float16 acc[4], accc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0][i] = 0.f; acc[1][i] = 0.f; acc[2][i] = 0.f; acc[3][i] = 0.f; accc[i] = 0.f;
      }
      const _Float16* arow_h = sh.ah + (tb * 32 + mm) * kSmRow + 8 * hh;
      const _Float16* arow_l = sh.al + (tb * 32 + mm) * kSmRow + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const sm_half8 xh = *reinterpret_cast<const sm_half8*>(arow_h + 16 * ks);
        const sm_half8 xl = *reinterpret_cast<const sm_half8*>(arow_l + 16 * ks);
        acc[ks >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, Bh[ks], acc[ks >> 1], 0, 0, 0);
        accc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, Bl[ks], accc, 0, 0, 0);
        accc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, Bh[ks], accc, 0, 0, 0);
      }
      // Register i: token tb*32 + 8 (i/4) + 4 hh + i % 4, coordinate col.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = tb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const float zs = ((acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i])) + accc[i];
        const float zi = sh.zinv[m];
        const float z = zs * zi;                    // unit domain
        // Grid lookup of u = z / s_i (clamped: no boundary lies beyond umax).
        const float u = fminf(fmaxf(z * inv_s, -umax), umax);
        const float f = fmaf(u, grid.scale, gbias);
        const SmLut ent = sh.lut[__float_as_uint(f) - 0x4B400000u];
        uint32_t c = ent.base + (u >= ent.t ? 1u : 0u);
        bool sure = !(fabsf(z - s_col * ent.t) <= kSmEps);    // t = inf: sure
        // Spreads too small for the grid: sure only beyond every boundary.
        const bool far = fabsf(z) > s_col * tmax + kSmEps;
        c = lut_ok ? c : (z > 0.f ? (uint32_t)NB : 0u);
        sure = lut_ok ? sure : far;
        // Zero (or padding) token: every field 0.
        c = zi == 0.f ? 0u : c;
        sure = sure || zi == 0.f;
        sh.idx[m * kSmIRow + col] = (uint8_t)c;
        if (!sure) {
          const int q = atomicAdd(&sh.qcount, 1);
          if (q < kSmQueue) sh.queue[q] = (uint16_t)((m << 7) | col);
        }
      }
    }
    __syncthreads();

    // ---- 4. exact decisions for the queue: 16 lanes per decision, in double ------------
    {
      const int qn = sh.qcount;
      const bool all = qn > kSmQueue;              // overflow: recompute every decision
      const int n_items = all ? kSmTT * kSmD : qn;
      const int grp = threadIdx.x >> 4, gl = threadIdx.x & 15;
      for (int it = grp; it < n_items; it += kSmThreads / 16) {
        const uint32_t item = all ? (uint32_t)it : sh.queue[it];
        const int m = (int)(item >> 7), i = (int)(item & 127);
        // Token tt0 + m's raw input (a padding token past T reads the last
        // token; its nu is 0, so its fields are 0 whatever the sum) and
        // column i of V, coordinates 8 gl .. 8 gl + 7.
        const TIN* xr = xbase + (int64_t)min(tt0 + m, p.T - 1) * p.st + 8 * gl;
        const float* vr = V + (size_t)(8 * gl) * kSmD + i;
        const float* mu = sh.mean + 8 * gl;
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fma((double)(float)xr[e] - (double)mu[e], (double)vr[(size_t)e * kSmD], a);
        a += __shfl_xor(a, 1, 64);
        a += __shfl_xor(a, 2, 64);
        a += __shfl_xor(a, 4, 64);
        a += __shfl_xor(a, 8, 64);
        if (gl == 0) {
          const double nu = sh.nu[m];
          const double si = (double)sh.scale[i];
          uint32_t c = 0;
          for (int k = 0; k < NB; ++k) c += (a >= nu * (si * p.gbounds[k])) ? 1u : 0u;
          sh.idx[m * kSmIRow + i] = (uint8_t)(nu > 0.0 ? c : 0u);
        }
      }
    }
    __syncthreads();

    // ---- 5. pack and store ------------------------------------------------------------
    {
      const int t = tt0 + m1;
      const int64_t tw = slot0 + t;
      if (t < p.T && tw >= 0 && tw < p.T_cap) {
        uint32_t w[BITS];
#pragma unroll
        for (int k = 0; k < BITS; ++k) w[k] = 0;
        uint32_t cb[8];
        {
          const uint4 a = *reinterpret_cast<const uint4*>(sh.idx + m1 * kSmIRow + 32 * j);
          const uint4 b2 = *reinterpret_cast<const uint4*>(sh.idx + m1 * kSmIRow + 32 * j + 16);
          cb[0] = a.x; cb[1] = a.y; cb[2] = a.z; cb[3] = a.w; cb[4] = b2.x; cb[5] = b2.y; cb[6] = b2.z; cb[7] = b2.w;
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const uint32_t c = (cb[e >> 2] >> (8 * (e & 3))) & 0xFFu;
          const int bit = BITS * e, wi = bit >> 5, shf = bit & 31;
          w[wi] |= c << shf;
          if (shf + BITS > 32) w[wi + 1] |= c >> (32 - shf);
        }
        uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + (vbase + tw) * (size_t)(kSmD * BITS / 8)) + j * BITS;
#pragma unroll
        for (int k = 0; k < BITS; ++k) __builtin_nontemporal_store(w[k], dst + k);
      }
    }
    __syncthreads();
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

template <int BITS>
hipError_t launch_sm(const QuantParams& p, const QuantGrid& grid, hipStream_t s) {
  const long tph = (p.T + kSmTT - 1) / kSmTT;
  const long blocks = (long)p.B * p.H * ((tph + kSmTilesPerBlock - 1) / kSmTilesPerBlock);
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((quant_spectral_mfma_kernel<BITS, _Float16>), dim3((unsigned)blocks), dim3(kSmThreads), 0, s, p, grid);
  else
    hipLaunchKernelGGL((quant_spectral_mfma_kernel<BITS, float>), dim3((unsigned)blocks), dim3(kSmThreads), 0, s, p, grid);
  return hipGetLastError();
}

}  // namespace

int spectral_max_d() { return kSqMaxD; }

bool spectral_mfma_supported(const QuantParams& p, const QuantGrid& grid) {
  return p.d == kSmD && p.bits >= 1 && p.bits <= 4 && grid.cells >= 1 && grid.cells <= kSmLutMax;
}

hipError_t launch_quantize_spectral(const QuantParams& p, const QuantGrid* grid, hipStream_t s) {
  if (grid && spectral_mfma_supported(p, *grid)) {
    switch (p.bits) {
      case 1: return launch_sm<1>(p, *grid, s);
      case 2: return launch_sm<2>(p, *grid, s);
      case 3: return launch_sm<3>(p, *grid, s);
      case 4: return launch_sm<4>(p, *grid, s);
    }
    return hipErrorInvalidValue;
  }
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
