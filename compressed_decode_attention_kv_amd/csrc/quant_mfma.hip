// Write side for fp16 inputs at d = 128 on the matrix cores.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
//
// Same result as quant_kernel (norm split, seeded sign flip + normalised
// Walsh-Hadamard rotation, Beta Lloyd-Max index, LSB-first packing, QJL
// sketch of the rotated residual), organised as:
//   * rotation: H_128 = H_8 (x) H_16.  The 16-point blocks run on
//     v_mfma_f32_16x16x32_f16 with the constant operand H_16 diag(D_block)
//     (fp16 inputs times +-1 are exact, accumulation fp32); the 8-point
//     stage across blocks is three in-register butterfly stages.  A wave
//     handles 16 tokens; afterwards lane (g, tau) holds coordinates
//     16c + 4g + i (c < 8, i < 4) of token tau.
//   * index: one fma with a 1.5*2^23 bias yields the grid cell of y and,
//     shifted, the LDS address of that cell's entry (boundary inside the
//     cell and its two neighbours, count of boundaries below); one compare
//     finishes the Lloyd-Max index.
//   * packing: 4-index chunks are merged across the four lanes of a token
//     in two exchange rounds, after which lane g holds the `bits` whole
//     dwords [bits*g, bits*g + bits) of the token's code block.
//   * QJL ([P1] "Contribuciones Clave" 1): S r on the matrix cores.  S is
//     exact in fp16; the residual, scaled by 2^12, is split exactly enough
//     into fp16 hi + lo parts (two MFMAs per tile, fp32 accumulation).
//     The 16x16 output tiles have the same lane layout as the codes, so the
//     sign bits are packed by the same exchange.
#include <cfloat>
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kThreadsM = 256;
constexpr int kWavesM = kThreadsM / 64;
constexpr int kLutMax = 1024;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct LutEntry {
  float t;        // the boundary inside cells n-1..n+1 (+inf if none)
  uint32_t base;  // number of boundaries below cell n-1
};

__device__ __forceinline__ int parity(uint32_t x) { return __builtin_popcount(x) & 1; }

// Merge 4-index chunks (each 4*B bits, chunk c covers coordinates
// 16c + 4g .. 16c + 4g + 3 of the lane group's token) across the four lanes
// g = 0..3 of the token (lanes tau + 16 g).  Returns, in out[], the B dwords
// of bits [32 B g, 32 B g + 32 B) of the token's bitstream.
template <int B>
__device__ __forceinline__ void merge_chunks(const uint32_t* chunk, int g, uint32_t* out) {
  const int s = g & 1, t = g >> 1;
  uint32_t kept[4], half[4];
  uint32_t o01, o23;
  {
    uint32_t out4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lo_c = (q & 1) | ((q >> 1) << 2), hi_c = lo_c | 2;
      kept[q] = s ? chunk[hi_c] : chunk[lo_c];
      out4[q] = s ? chunk[lo_c] : chunk[hi_c];
    }
    o01 = out4[0] | (out4[1] << 16);
    o23 = out4[2] | (out4[3] << 16);
  }
  const uint32_t i01 = shfl_xor_u(o01, 16), i23 = shfl_xor_u(o23, 16);
  const uint32_t in4[4] = {i01 & 0xFFFFu, i01 >> 16, i23 & 0xFFFFu, i23 >> 16};
#pragma unroll
  for (int q = 0; q < 4; ++q)
    half[q] = s ? (in4[q] | (kept[q] << (4 * B))) : (kept[q] | (in4[q] << (4 * B)));
  // Round 2: keep blocks 2g, 2g+1.
  uint32_t keep2[2], send2[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    keep2[r] = t ? half[2 + r] : half[r];
    send2[r] = t ? half[r] : half[2 + r];
  }
  uint64_t blk[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint64_t in = shfl_xor_u(send2[r], 32);
    blk[r] = t ? (in | ((uint64_t)keep2[r] << (8 * B))) : ((uint64_t)keep2[r] | (in << (8 * B)));
  }
  // Concatenate the two 16B-bit blocks: 32B bits = B dwords.
  if (B == 1) {
    out[0] = (uint32_t)(blk[0] | (blk[1] << 16));
  } else if (B == 2) {
    out[0] = (uint32_t)blk[0];
    out[1] = (uint32_t)blk[1];
  } else if (B == 3) {
    out[0] = (uint32_t)blk[0];
    out[1] = (uint32_t)(blk[0] >> 32) | (uint32_t)(blk[1] << 16);
    out[2] = (uint32_t)(blk[1] >> 16);
  } else {
    out[0] = (uint32_t)blk[0];
    out[1] = (uint32_t)(blk[0] >> 32);
    out[2] = (uint32_t)blk[1];
    out[3] = (uint32_t)(blk[1] >> 32);
  }
}

template <int BITS, int MODE>
__global__ __launch_bounds__(kThreadsM) void quant_mfma_kernel(QuantParams p, QuantGrid grid) {
  constexpr bool kProd = MODE == TQ_MODE_PROD;
  __shared__ __attribute__((aligned(16))) LutEntry s_lut[kLutMax];
  __shared__ float s_cent[16];
  __shared__ __attribute__((aligned(16))) half8 s_S[kProd ? 8 * 4 * 64 : 1];
  __shared__ __attribute__((aligned(16))) half8 s_A[8 * 64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tau = lane & 15, g = lane >> 4;
  constexpr int NB = (1 << BITS) - 1;

  // ---- per-block tables -------------------------------------------------------------
  for (int n = threadIdx.x; n < grid.cells; n += kThreadsM) {
    const float lo = ((float)(n - 1) - 0.5f - (float)grid.center) / grid.scale;
    const float hi = ((float)(n + 1) + 0.5f - (float)grid.center) / grid.scale;
    uint32_t base = 0;
    float t = INFINITY;
    for (int k = 0; k < NB; ++k) {
      const float b = p.bounds[k];
      if (b < lo) base++;
      else if (b < hi && t == INFINITY) t = b;
    }
    s_lut[n].t = t;
    s_lut[n].base = base;
  }
  if (threadIdx.x < 16) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  if constexpr (kProd) {
    // S_perm[mb][pp][l] = S[16 mb + (l % 16)][16 (2 pp + j / 4) + 4 (l / 16) + j % 4], j < 8.
    for (int i = threadIdx.x; i < 8 * 4 * 64; i += kThreadsM) {
      const int l = i & 63, pp = (i >> 6) & 3, mb = i >> 8;
      const int row = 16 * mb + (l & 15), gg = l >> 4;
      half8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (_Float16)p.S[row * 128 + 16 * (2 * pp + j / 4) + 4 * gg + (j & 3)];
      s_S[i] = v;
    }
  }
  __syncthreads();

  // ---- constant operands of the 16-point blocks: A_a[e][k] = H16[e][k'] D[coord] ----
  // Kept in LDS (entry a * 64 + lane holds lane's 8 values of operand a) so
  // that they do not occupy 32 registers for the whole kernel.
  for (int i = threadIdx.x; i < 8 * 64; i += kThreadsM) {
    const int a = i >> 6, ln = i & 63, ltau = ln & 15, lg = ln >> 4;
    const int pp = a >> 1, odd = a & 1;
    half8 op;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kappa = 8 * lg + j;
      float v = 0.f;
      if ((kappa >> 4) == odd) {
        const int bcol = kappa & 15, coord = 32 * pp + kappa;
        if (MODE == TQ_MODE_PLAIN) {
          v = (bcol == ltau) ? 1.f : 0.f;
        } else {
          const float h = parity((uint32_t)(ltau & bcol)) ? -1.f : 1.f;
          const float dsg = ((p.signbits[coord >> 5] >> (coord & 31)) & 1u) ? -1.f : 1.f;
          v = h * dsg;
        }
      }
      op[j] = (_Float16)v;
    }
    s_A[i] = op;
  }
  __syncthreads();

  const int64_t N = (int64_t)p.B * p.H * p.T;
  const int64_t ntiles = (N + 15) >> 4;
  const float magic = 12582912.0f;  // 1.5 * 2^23: fma(y, s, magic) rounds y*s to an integer in the low bits
  const float inv_sqrt_d = p.inv_sqrt_d;

  for (int64_t tile = (int64_t)blockIdx.x * kWavesM + wave; tile < ntiles; tile += (int64_t)gridDim.x * kWavesM) {
    const int64_t v = tile * 16 + tau;
    const bool valid = v < N;
    const int64_t vc = valid ? v : N - 1;
    const int bh = (int)(vc / p.T), t = (int)(vc % p.T);
    const int b = bh / p.H, h = bh % p.H;
    const _Float16* xrow = reinterpret_cast<const _Float16*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh +
                           (int64_t)t * p.st;
    half8 xin[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) xin[pp] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(xrow + 32 * pp + 8 * g));

    // ||x||^2: fp16 products are exact in fp32.
    float ss = 0.f;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        half2v a2;
        a2.x = xin[pp][j];
        a2.y = xin[pp][j + 1];
        ss = __builtin_amdgcn_fdot2(a2, a2, ss, false);
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float nu = sqrtf(ss);

    // ---- rotation -------------------------------------------------------------------
    float4v Z[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      float4v z = {0.f, 0.f, 0.f, 0.f};
      Z[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(s_A[a * 64 + lane], xin[a >> 1], z, 0, 0, 0);
    }
    float y[8][4];  // y[c][i] <-> coordinate 16c + 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float w8[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) w8[a] = Z[a][i];
      if (MODE != TQ_MODE_PLAIN) {
#pragma unroll
        for (int hs = 1; hs < 8; hs <<= 1) {
#pragma unroll
          for (int a = 0; a < 8; ++a) {
            if (!(a & hs)) {
              const float x0 = w8[a], x1 = w8[a | hs];
              w8[a] = x0 + x1;
              w8[a | hs] = x0 - x1;
            }
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c][i] = w8[c];
    }
    const float inv = nu > 0.f ? (MODE == TQ_MODE_PLAIN ? 1.0f / nu : inv_sqrt_d / nu) : 0.f;

    // ---- index ------------------------------------------------------------------------
    uint32_t chunk[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t ch = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float yy = y[c][i] * inv;
        y[c][i] = yy;
        const float f = fmaf(yy, grid.scale, magic);
        const LutEntry e = s_lut[(int)(__float_as_uint(f) - 0x4B400000u) + grid.center];
        const uint32_t idx = e.base + (yy >= e.t ? 1u : 0u);
        ch |= idx << (BITS * i);
        if (kProd) y[c][i] = yy - s_cent[idx];   // residual
      }
      chunk[c] = ch;
    }
    uint32_t words[BITS];
    merge_chunks<BITS>(chunk, g, words);
    const int64_t vec = (int64_t)bh * p.T_cap + t;
    if (valid) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + vec * (16 * BITS)) + BITS * g;
      if (!(nu > 0.f)) {
#pragma unroll
        for (int k = 0; k < BITS; ++k) words[k] = 0;
      }
      if (BITS == 4) {
        u32x4 w4 = {words[0], words[1], words[2], words[3]};
        *reinterpret_cast<u32x4*>(dst) = w4;
      } else if (BITS == 3) {
        u32x3 w3 = {words[0], words[1], words[2]};
        *reinterpret_cast<u32x3*>(dst) = w3;
      } else if (BITS == 2) {
        u32x2 w2 = {words[0], words[1]};
        *reinterpret_cast<u32x2*>(dst) = w2;
      } else {
        dst[0] = words[0];
      }
      if (g == 0) p.norms[vec] = nu;
    }

    if (kProd) {
      // ---- QJL sketch of the residual ----------------------------------------------
      const float rs = nu > 0.f ? 4096.0f : 0.f;
      float g2 = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) g2 = fmaf(y[c][i], y[c][i], g2);
      g2 += __shfl_xor(g2, 16, 64);
      g2 += __shfl_xor(g2, 32, 64);
      // Exact-enough fp16 split of the scaled residual: hi rounds toward
      // zero, so r - hi is exact in fp32 and lo keeps its leading 11 bits.
      half8 Bhi[4], Blo[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float r0 = y[2 * pp + j / 4][j & 3] * rs, r1 = y[2 * pp + (j + 1) / 4][(j + 1) & 3] * rs;
          const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0, r1));
          const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0 - (float)hi.x, r1 - (float)hi.y));
          Bhi[pp][j] = hi.x; Bhi[pp][j + 1] = hi.y;
          Blo[pp][j] = lo.x; Blo[pp][j + 1] = lo.y;
        }
      }
      // Two 16-row blocks of S in flight at a time keeps the S operands
      // (LDS reads) from all being hoisted into registers.
      uint32_t sbits = 0;  // 4 sign bits per row block mb
#pragma unroll 2
      for (int mb = 0; mb < 8; ++mb) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const half8 A = s_S[(mb * 4 + pp) * 64 + lane];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bhi[pp], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Blo[pp], acc, 0, 0, 0);
        }
        uint32_t sc = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) sc |= (acc[i] >= 0.f ? 1u : 0u) << i;
        sbits |= sc << (4 * mb);
      }
      uint32_t schunk[8];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) schunk[mb] = (sbits >> (4 * mb)) & 15u;
      uint32_t sw[1];
      merge_chunks<1>(schunk, g, sw);
      if (valid) {
        reinterpret_cast<uint32_t*>(p.qjl + vec * 16)[g] = nu > 0.f ? sw[0] : 0u;
        if (g == 0) p.gamma[vec] = nu > 0.f ? sqrtf(g2) : 0.f;
      }
    }
  }
}

template <int BITS, int MODE>
hipError_t launch_m(const QuantParams& p, const QuantGrid& grid, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((quant_mfma_kernel<BITS, MODE>), dim3(nblocks), dim3(kThreadsM), 0, s, p, grid);
  return hipGetLastError();
}

}  // namespace

bool quant_mfma_supported(const QuantParams& p) {
  return p.d == 128 && p.dtype == TQ_F16 && p.mode != TQ_MODE_HEADQ && p.bits >= 1 && p.bits <= 4;
}

int quant_mfma_lut_max() { return kLutMax; }

hipError_t launch_quantize_mfma(const QuantParams& p, const QuantGrid& grid, int nblocks, hipStream_t s) {
  switch (p.mode * 8 + p.bits) {
    case TQ_MODE_PLAIN * 8 + 1: return launch_m<1, TQ_MODE_PLAIN>(p, grid, nblocks, s);
    case TQ_MODE_PLAIN * 8 + 2: return launch_m<2, TQ_MODE_PLAIN>(p, grid, nblocks, s);
    case TQ_MODE_PLAIN * 8 + 3: return launch_m<3, TQ_MODE_PLAIN>(p, grid, nblocks, s);
    case TQ_MODE_PLAIN * 8 + 4: return launch_m<4, TQ_MODE_PLAIN>(p, grid, nblocks, s);
    case TQ_MODE_MSE * 8 + 1: return launch_m<1, TQ_MODE_MSE>(p, grid, nblocks, s);
    case TQ_MODE_MSE * 8 + 2: return launch_m<2, TQ_MODE_MSE>(p, grid, nblocks, s);
    case TQ_MODE_MSE * 8 + 3: return launch_m<3, TQ_MODE_MSE>(p, grid, nblocks, s);
    case TQ_MODE_MSE * 8 + 4: return launch_m<4, TQ_MODE_MSE>(p, grid, nblocks, s);
    case TQ_MODE_PROD * 8 + 1: return launch_m<1, TQ_MODE_PROD>(p, grid, nblocks, s);
    case TQ_MODE_PROD * 8 + 2: return launch_m<2, TQ_MODE_PROD>(p, grid, nblocks, s);
    case TQ_MODE_PROD * 8 + 3: return launch_m<3, TQ_MODE_PROD>(p, grid, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
