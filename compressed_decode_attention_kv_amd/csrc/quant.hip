// Write side of libtq: norm split, seeded sign flip + normalised
// Walsh-Hadamard rotation, Beta Lloyd-Max index, bit packing, optional QJL
// sketch or HeadQ side code.  Also the per-vector reconstruction error used
// by tq_metrics (relMSE and direction error).
//
// Packed planes are written with non-temporal stores: a decode that streams
// the cache soon after a quantize otherwise meets its lines still dirty in
// the caches and runs ~20% slower.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
// [P3] = "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
//        Espaço de Pontuação para Quantização de KV-Cache"
#include "device_common.h"

namespace tq {
namespace {

constexpr int kThreads = 256;
constexpr int kSteps = 4;            // wave steps per block
constexpr int kMaxSideLds = 16384;   // floats of the rotated HeadQ basis in LDS

// U'_h = Pi U_h = H D U_h / sqrt(d), column by column, into LDS as [d][rank].
// The side code of [P3] section 3 projects the residual k - k_base on U_h;
// with the residual held rotated, U'^T (Pi e) = U^T e gives the same value.
__device__ void rotated_basis(const float* U, int d, int rank, const uint32_t* signbits,
                              float inv_sqrt_d, float* lds) {
  const int n = d * rank;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int k = i / rank;
    const float s = ((signbits[k >> 5] >> (k & 31)) & 1u) ? -1.f : 1.f;
    lds[i] = U[i] * s;
  }
  __syncthreads();
  for (int h = 1; h < d; h <<= 1) {
    for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
      const int col = i % rank, pr = i / rank;           // pair index over k
      const int lo = (pr / h) * 2 * h + (pr % h), hi = lo + h;
      float a = lds[lo * rank + col], c = lds[hi * rank + col];
      lds[lo * rank + col] = a + c;
      lds[hi * rank + col] = a - c;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < n; i += blockDim.x) lds[i] *= inv_sqrt_d;
  __syncthreads();
}

// HeadQ side code of one vector ([P3] section 3): e' = nu (y - c[idx]) =
// Pi (k - k_base) held rotated, z = U'^T e' with U'^T = (Pi U)^T in LDS as
// [rank][d] (each z_r a dot product over the lane's 32 contiguous entries),
// s_z = max |z| / lev, code = clamp(rne(z / s_z), -lev, lev) + lev.
__device__ __forceinline__ void headq_side(const QuantParams& p, const float* v, const uint32_t* idx, float nu,
                                           const float* s_cent, const float* s_side, int j, int L, bool valid,
                                           int64_t vec) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const int rank = p.rank;
  float ep[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) ep[e] = nu > 0.f ? nu * (v[e] - s_cent[idx[e]]) : 0.f;
  float z[32];
  float zmax = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    z[r] = 0.f;
    if (r < rank) {  // uniform
      const f4* ur = reinterpret_cast<const f4*>(s_side + r * p.d + 32 * j);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const f4 u = ur[i];
        a0 = fmaf(u.x, ep[4 * i], a0);
        a1 = fmaf(u.y, ep[4 * i + 1], a1);
        a0 = fmaf(u.z, ep[4 * i + 2], a0);
        a1 = fmaf(u.w, ep[4 * i + 3], a1);
      }
      z[r] = group_sum(a0 + a1, L);
      zmax = fmaxf(zmax, fabsf(z[r]));
    }
  }
  const int lev = (1 << (p.side_bits - 1)) - 1;
  const float sz = zmax / (float)lev;
  if (valid && j == 0) {
    uint32_t sw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) sw[k] = 0;
    const int sb = p.side_bits;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      if (r < rank) {
        int c = lev;
        if (sz > 0.f) {
          float q = rintf(z[r] / sz);
          q = fminf(fmaxf(q, (float)-lev), (float)lev);
          c = (int)q + lev;
        }
        const int bit = sb * r, wi = bit >> 5, sh = bit & 31;
        sw[wi] |= (uint32_t)c << sh;
        if (sh + sb > 32) sw[wi + 1] |= (uint32_t)c >> (32 - sh);
      }
    }
    const int nbytes = rank * sb / 8;
    uint8_t* dst = p.side + vec * nbytes;
    if ((nbytes & 3) == 0) {
      for (int k = 0; k < nbytes / 4; ++k) __builtin_nontemporal_store(sw[k], reinterpret_cast<uint32_t*>(dst) + k);
    } else {
      for (int k = 0; k < nbytes; ++k) __builtin_nontemporal_store((uint8_t)(sw[k >> 2] >> (8 * (k & 3))), dst + k);
    }
    __builtin_nontemporal_store(sz, p.side_scale + vec);
  }
}

// Grid lookup of the Lloyd-Max index (as in the matrix-core quantisers):
// cell n = round(y * scale) + center holds the boundary inside the cell's
// window (+inf if none) and the number of boundaries below it, so the index
// is base + [y >= t], the same count as comparing y with every boundary.
struct QLut {
  float t;
  uint32_t base;
};
constexpr int kQLutMax = 1024;

template <int BITS, int MODE, typename TIN>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantParams p, QuantGrid grid) {
  __shared__ float s_cent[16], s_bnd[16];
  __shared__ __attribute__((aligned(8))) QLut s_lut[kQLutMax];
  // Dynamic LDS (sized at launch).  HEADQ: (Pi U_h)^T, d * rank floats.
  // PROD: each wave's token residuals, 64 / L tokens x d floats per wave.
  extern __shared__ float s_side[];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = p.L, j = lane & (L - 1), slot = lane / L, vpw = 64 / L;
  const int bh = p.bh0 + blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int d = p.d;
  const int tend = min(p.T, p.t0 + p.tn);

  if (threadIdx.x < 16) {
    s_cent[threadIdx.x] = p.centroids[threadIdx.x];
    s_bnd[threadIdx.x] = p.bounds[threadIdx.x];
  }
  constexpr int NB = (1 << BITS) - 1;
  // grid.cells == 0: no table (every boundary compared instead).
  for (int n = threadIdx.x; n < grid.cells; n += blockDim.x) {
    const float lo = ((float)n - (0.5f + kGridMargin) - (float)grid.center) / grid.scale;
    const float hi = ((float)n + (0.5f + kGridMargin) - (float)grid.center) / grid.scale;
    uint32_t base = 0;
    float t = INFINITY;
    for (int k = 0; k < NB; ++k) {
      const float bk = p.bounds[k];
      if (bk < lo) base++;
      else if (bk < hi && t == INFINITY) t = bk;
    }
    s_lut[n].t = t;
    s_lut[n].base = base;
  }
  // 1.5 * 2^23 + center: fma(y, scale, bias) holds round(y * scale) + center
  // in its low mantissa bits.
  const float gbias = 12582912.0f + (float)grid.center;
  if (MODE == TQ_MODE_HEADQ) {
    // (Pi U_h)^T, [rank][d], computed once per head by rotate_basis_kernel.
    const float* src = p.rbasis + (size_t)h * d * p.rank;
    for (int i = threadIdx.x; i < d * p.rank; i += blockDim.x) s_side[i] = src[i];
  }
  __syncthreads();

  const uint32_t myword = p.signbits[j];
  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t vbase = (int64_t)bh * p.T_cap;
  const int tok_per_block = 4 * vpw * kSteps;
  const int64_t slot0 = p.pos ? p.pos[b] : 0;  // destination slot of token 0

  for (int step = 0; step < kSteps; ++step) {
    const int t = p.t0 + blockIdx.x * tok_per_block + (step * 4 + wave) * vpw + slot;
    const bool valid = t < tend;
    const int tc = valid ? t : tend - 1;
    float v[32];
    load32<TIN>(xbase + (int64_t)tc * p.st + 32 * j, v);

    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) ss = fmaf(v[e], v[e], ss);
    ss = group_sum(ss, L);
    const float nu = sqrtf(ss);
    float inv;
    if (MODE == TQ_MODE_PLAIN) {
      inv = nu > 0.f ? 1.0f / nu : 0.f;
    } else {
      apply_signs(v, myword);
      wht_group(v, j, L);
      inv = nu > 0.f ? p.inv_sqrt_d / nu : 0.f;
    }
    uint32_t idx[32];
    if (grid.cells > 0) {
      // All table reads of the lane issued before any is used.
      QLut ent[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        v[e] *= inv;  // y: the rotated unit vector
        ent[e] = s_lut[__float_as_uint(fmaf(v[e], grid.scale, gbias)) - 0x4B400000u];
      }
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t c = ent[e].base + (v[e] >= ent[e].t ? 1u : 0u);
        idx[e] = nu > 0.f ? c : 0u;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        v[e] *= inv;
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < NB; ++k) c += (v[e] >= s_bnd[k]) ? 1u : 0u;
        idx[e] = nu > 0.f ? c : 0u;
      }
    }
    // PROD: (BITS+1)-bit fields; the sketch signs are added below.
    constexpr int FB = Field<BITS, MODE == TQ_MODE_PROD>::kBits;
    uint32_t w[FB];
#pragma unroll
    for (int k = 0; k < FB; ++k) w[k] = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int bit = FB * e, wi = bit >> 5, sh = bit & 31;
      w[wi] |= idx[e] << sh;
      if (sh + FB > 32) w[wi + 1] |= idx[e] >> (32 - sh);
    }
    // Destination slot: t, or pos[b] + t when appending; never outside [0, T_cap).
    const int64_t tw = slot0 + t;
    const bool wr = valid && tw >= 0 && tw < p.T_cap;
    const int64_t vec = vbase + tw;

    if (MODE == TQ_MODE_PROD) {
      // Residual of the rotated unit vector and its 1-bit Gaussian sketch
      // ([P1] "Esquemas de Cuantización" 2-3, "Contribuciones Clave" 1).
      // This kernel takes PROD only at d <= 128 (and as a fallback for
      // launches the matrix-core sketch kernel cannot index): the token's
      // residual goes through LDS and lane j forms sketch rows 32 j .. 32 j
      // + 31 as fp32 dot products against S (exact in fp32).
      float g2 = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        v[e] = nu > 0.f ? v[e] - s_cent[idx[e]] : 0.f;
        g2 = fmaf(v[e], v[e], g2);
      }
      g2 = group_sum(g2, L);
      float* rs = s_side + (wave * vpw + slot) * d;
      __syncthreads();  // the previous step's readers are done with rs
#pragma unroll
      for (int e = 0; e < 32; ++e) rs[32 * j + e] = v[e];
      __syncthreads();
      typedef float f4 __attribute__((ext_vector_type(4)));
      uint32_t sw = 0;
      for (int i = 0; i < 32; ++i) {
        const f4* srow = reinterpret_cast<const f4*>(p.S + (size_t)(32 * j + i) * d);
        const f4* rr = reinterpret_cast<const f4*>(rs);
        float a0 = 0.f, a1 = 0.f;
        for (int k = 0; k < d / 4; ++k) {
          const f4 sv = srow[k], rv = rr[k];
          a0 = fmaf(sv.x, rv.x, a0);
          a1 = fmaf(sv.y, rv.y, a1);
          a0 = fmaf(sv.z, rv.z, a0);
          a1 = fmaf(sv.w, rv.w, a1);
        }
        sw |= (a0 + a1 >= 0.f ? 1u : 0u) << i;
      }
      if (!(nu > 0.f)) sw = 0;  // a zero vector keeps all-zero fields
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int bit = FB * e + BITS;
        w[bit >> 5] |= ((sw >> e) & 1u) << (bit & 31);
      }
      if (j == 0 && wr) __builtin_nontemporal_store(nu > 0.f ? sqrtf(g2) : 0.f, p.gamma + vec);
    }
    if (wr) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + vec * (d * FB / 8)) + j * FB;
#pragma unroll
      for (int k = 0; k < FB; ++k) __builtin_nontemporal_store(w[k], dst + k);
      if (j == 0) __builtin_nontemporal_store(nu, p.norms + vec);
    }

    if (MODE == TQ_MODE_HEADQ) {
      headq_side(p, v, idx, nu, s_cent, s_side, j, L, wr, vec);
    }
  }
}

// Per-vector reconstruction error in the rotated domain, where
// ||x - x_hat|| = ||Pi x - Pi x_hat|| and <x, x_hat> = <Pi x, Pi x_hat>
// ([P2] "Configuração Experimental": relMSE and cosine direction error).
template <int BITS, int MODE, typename TIN>
__global__ __launch_bounds__(kThreads) void relerr_kernel(RelErrParams p) {
  __shared__ float s_cent[16];
  __shared__ float s_side[MODE == TQ_MODE_HEADQ ? kMaxSideLds : 1];
  __shared__ double s_red[kThreads / 64][5];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int L = p.L, j = lane & (L - 1), slot = lane / L, vpw = 64 / L;
  const int bh = blockIdx.y, b = bh / p.H, h = bh % p.H;
  const int d = p.d;
  if (threadIdx.x < 16) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  if (MODE == TQ_MODE_HEADQ)
    rotated_basis(p.basis + (size_t)h * d * p.rank, d, p.rank, p.signbits, p.inv_sqrt_d, s_side);
  __syncthreads();

  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t vbase = (int64_t)bh * p.T_cap;
  const int tok_per_block = 4 * vpw * kSteps;
  double e2 = 0.0, r2 = 0.0, dsum = 0.0, cnt = 0.0, asum = 0.0;
  for (int step = 0; step < kSteps; ++step) {
    const int t = blockIdx.x * tok_per_block + (step * 4 + wave) * vpw + slot;
    const bool valid = t < p.T;
    const int tc = valid ? t : p.T - 1;
    const int64_t vec = vbase + tc;
    float a[32];
    load32<TIN>(xbase + (int64_t)tc * p.st + 32 * j, a);
    if (p.rotate) {
      apply_signs(a, p.signbits[j]);
      wht_group(a, j, L);
#pragma unroll
      for (int e = 0; e < 32; ++e) a[e] *= p.inv_sqrt_d;
    }
    constexpr int FB = Field<BITS, MODE == TQ_MODE_PROD>::kBits;
    uint32_t w[FB];
    const uint32_t* cw = reinterpret_cast<const uint32_t*>(p.planes.codes + vec * (d * FB / 8)) + j * FB;
#pragma unroll
    for (int k = 0; k < FB; ++k) w[k] = cw[k];
    const float nu = p.planes.norms[vec];
    float ah[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) ah[e] = s_cent[code_at<FB>(w, e) & Field<BITS, false>::kCodeMask];
    if (MODE == TQ_MODE_PROD) {
      // y_hat += sqrt(pi/2)/m gamma S^T sigma, sigma from every group's fields
      const float g = p.planes.gamma[vec] * p.qjl_c;
      const uint32_t* vf = reinterpret_cast<const uint32_t*>(p.planes.codes + vec * (d * FB / 8));
      for (int iw = 0; iw < d / 32; ++iw) {
        uint32_t gw[FB];
#pragma unroll
        for (int k = 0; k < FB; ++k) gw[k] = vf[iw * FB + k];
        const uint32_t bits = sign_word<BITS>(gw);
        for (int ib = 0; ib < 32; ++ib) {
          const float sg = ((bits >> ib) & 1u) ? g : -g;
          const float* srow = p.S + (size_t)(32 * iw + ib) * d + 32 * j;
#pragma unroll
          for (int e = 0; e < 32; ++e) ah[e] = fmaf(sg, srow[e], ah[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) ah[e] *= nu;
    if (MODE == TQ_MODE_HEADQ) {
      const int rank = p.rank, sbits = p.side_bits, lev = (1 << (sbits - 1)) - 1;
      const float sz = p.planes.side_scale[vec];
      const uint8_t* sc = p.planes.side + vec * (rank * sbits / 8);
      for (int r = 0; r < rank; ++r) {
        const int bit = sbits * r;
        uint32_t raw = (uint32_t)sc[bit >> 3] | ((uint32_t)sc[(bit >> 3) + 1 < rank * sbits / 8 ? (bit >> 3) + 1 : (bit >> 3)] << 8);
        const int code = (int)((raw >> (bit & 7)) & ((1u << sbits) - 1u));
        const float zh = sz * (float)(code - lev);
#pragma unroll
        for (int e = 0; e < 32; ++e) ah[e] = fmaf(s_side[(32 * j + e) * rank + r], zh, ah[e]);
      }
    }
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
    for (int w = 0; w < kThreads / 64; ++w) s += s_red[w][threadIdx.x];
    const size_t blk = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    p.block_sums[blk * 5 + threadIdx.x] = s;
  }
}

// (Pi U_h)^T for every head h (one block per head) into out [H][rank][d];
// with out16, also 2^10 times it as fp16 hi (out16) and lo (out16 + H rank d),
// the matrix-core quantiser's operands.
__global__ __launch_bounds__(kThreads) void rotate_basis_kernel(QuantParams p, float* out, _Float16* out16) {
  __shared__ float s_side[kMaxSideLds];
  const int h = blockIdx.x, n = p.d * p.rank;
  rotated_basis(p.basis + (size_t)h * n, p.d, p.rank, p.signbits, p.inv_sqrt_d, s_side);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int r = i / p.d, k = i % p.d;
    const float u = s_side[k * p.rank + r];
    out[(size_t)h * n + i] = u;
    if (out16) {
      float uv = u * 1024.0f;
      asm volatile("" : "+v"(uv));
      const _Float16 hi = (_Float16)uv;
      out16[(size_t)h * n + i] = hi;
      out16[(size_t)(p.H + h) * n + i] = (_Float16)(uv - (float)hi);
    }
  }
}

template <int BITS, int MODE>
hipError_t launch_q(const QuantParams& p, const QuantGrid& g, hipStream_t s) {
  const int vpw = 64 / p.L;
  dim3 grid((p.tn + 4 * vpw * kSteps - 1) / (4 * vpw * kSteps), p.nbh);
  const size_t dyn = MODE == TQ_MODE_HEADQ ? (size_t)p.d * p.rank * sizeof(float)
                    : MODE == TQ_MODE_PROD ? (size_t)(kThreads / 64) * vpw * p.d * sizeof(float) : 0;
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((quant_kernel<BITS, MODE, _Float16>), grid, dim3(kThreads), dyn, s, p, g);
  else
    hipLaunchKernelGGL((quant_kernel<BITS, MODE, float>), grid, dim3(kThreads), dyn, s, p, g);
  return hipGetLastError();
}

template <int BITS, int MODE>
hipError_t launch_r(const RelErrParams& p, hipStream_t s) {
  const int vpw = 64 / p.L;
  dim3 grid((p.T + 4 * vpw * kSteps - 1) / (4 * vpw * kSteps), p.B * p.H);
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((relerr_kernel<BITS, MODE, _Float16>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((relerr_kernel<BITS, MODE, float>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int relerr_blocks(int T, int L, int BH) {
  const int vpw = 64 / L;
  return ((T + 4 * vpw * kSteps - 1) / (4 * vpw * kSteps)) * BH;
}

hipError_t launch_quantize(const QuantParams& p, const QuantGrid* grid, hipStream_t s) {
  QuantGrid g{0.f, 0, 0};
  if (grid && grid->cells <= kQLutMax) g = *grid;
  switch (p.mode) {
    case TQ_MODE_PLAIN:
      switch (p.bits) { case 1: return launch_q<1, TQ_MODE_PLAIN>(p, g, s); case 2: return launch_q<2, TQ_MODE_PLAIN>(p, g, s);
                        case 3: return launch_q<3, TQ_MODE_PLAIN>(p, g, s); case 4: return launch_q<4, TQ_MODE_PLAIN>(p, g, s); }
      break;
    case TQ_MODE_MSE:
      switch (p.bits) { case 1: return launch_q<1, TQ_MODE_MSE>(p, g, s); case 2: return launch_q<2, TQ_MODE_MSE>(p, g, s);
                        case 3: return launch_q<3, TQ_MODE_MSE>(p, g, s); case 4: return launch_q<4, TQ_MODE_MSE>(p, g, s); }
      break;
    case TQ_MODE_PROD:
      switch (p.bits) { case 1: return launch_q<1, TQ_MODE_PROD>(p, g, s); case 2: return launch_q<2, TQ_MODE_PROD>(p, g, s);
                        case 3: return launch_q<3, TQ_MODE_PROD>(p, g, s); }
      break;
    case TQ_MODE_HEADQ:
      if (p.bits == 2) return launch_q<2, TQ_MODE_HEADQ>(p, g, s);
      break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rotate_basis(const QuantParams& p, float* out, _Float16* out16, hipStream_t s) {
  hipLaunchKernelGGL(rotate_basis_kernel, dim3(p.H), dim3(kThreads), 0, s, p, out, out16);
  return hipGetLastError();
}

hipError_t launch_relerr(const RelErrParams& p, int, hipStream_t s) {
  switch (p.mode) {
    case TQ_MODE_PLAIN:
    case TQ_MODE_MSE:
      switch (p.bits) { case 1: return launch_r<1, TQ_MODE_MSE>(p, s); case 2: return launch_r<2, TQ_MODE_MSE>(p, s);
                        case 3: return launch_r<3, TQ_MODE_MSE>(p, s); case 4: return launch_r<4, TQ_MODE_MSE>(p, s); }
      break;
    case TQ_MODE_PROD:
      switch (p.bits) { case 1: return launch_r<1, TQ_MODE_PROD>(p, s); case 2: return launch_r<2, TQ_MODE_PROD>(p, s);
                        case 3: return launch_r<3, TQ_MODE_PROD>(p, s); }
      break;
    case TQ_MODE_HEADQ:
      if (p.bits == 2) return launch_r<2, TQ_MODE_HEADQ>(p, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
