// Write side for fp16 and fp32 inputs at d = 128 on the matrix cores.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
//
// Same result as quant_kernel (norm split, seeded sign flip + normalised
// Walsh-Hadamard rotation, Beta Lloyd-Max index, LSB-first packing, QJL
// sketch of the rotated residual), organised so that every lane ends up
// owning 32 consecutive coordinates of one token and writes its own code
// and sign words without any exchange:
//   * rotation: a Sylvester Hadamard entry is a product over index bits, so
//     H_128 = H_64 (x) H_2 with the 64-point factor acting on bits 1..6 and
//     the 2-point factor on bit 0.  The 64-point part runs on
//     v_mfma_f32_16x16x32_f16 (4 row blocks x 2 K blocks per value a of the
//     low input bit) with the constant operand H_64; D is applied to the fp16
//     input by flipping sign bits (exact), and products of fp16 inputs with
//     +-1 are exact in the fp32 accumulation; the 2-point part is one
//     in-register butterfly stage.  A wave handles 16 tokens; the rows of the products
//     are ordered so that lane (g, tau) holds coordinates 32 g + 8 rb + 2 i +
//     b (rb, i < 4, b < 2) of token tau.
//   * index: one fma with a biased 1.5*2^23 constant yields the grid cell of
//     y and, shifted, the LDS address of that cell's entry (boundary inside
//     the cell and its two neighbours, count of boundaries below); one
//     compare finishes the Lloyd-Max index, which goes straight into the
//     lane's `bits` code dwords.
//   * QJL ([P1] "Contribuciones Clave" 1): S r on the matrix cores.  S is
//     exact in fp16; the residual, scaled by 2^12, is split into fp16 hi
//     (rounded toward zero) + lo parts, so r - hi is exact and two products
//     per tile with fp32 accumulation keep about 22 bits.  The rows of S are
//     ordered so that lane (g, tau) receives sketch rows 32 g .. 32 g + 31:
//     its 32 sign bits are word g of the token's sign block, shifted in one
//     per row with a funnel shift of the product's sign bit.
//   * sketched and HeadQ modes run the index search on y 2^12 (boundaries,
//     centroids and grid scale scaled to match, all by a power of two, so
//     every decision and the residual are those of y itself, scaled), which
//     leaves the residual already at the scale its fp16 split needs.
//   * stores: non-temporal, so that a decode streaming the cache soon after
//     does not meet its lines still dirty in the caches (~20% slower).
#include <cfloat>
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kThreadsM = 256;
constexpr int kWavesM = kThreadsM / 64;
constexpr int kLutMax = 1024;
constexpr float kSplitScale = 16384.0f;  // fp32 input: 2^14 / ||x|| before the fp16 hi/lo split

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct LutEntry {
  float t;        // the boundary inside cell n's window (+inf if none)
  uint32_t base;  // number of boundaries below the window
};

__device__ __forceinline__ int parity(uint32_t x) { return __builtin_popcount(x) & 1; }

// Put the BITS-bit index of coordinate O (of the lane's 32) into its place
// in the lane's LSB-first bitstream words.  The fields are disjoint, so an
// add is the same as an or and becomes one shift-and-add.
template <int BITS, int O>
__device__ __forceinline__ void put_index(uint32_t* words, uint32_t idx) {
  constexpr int bit = BITS * O, w = bit >> 5, sh = bit & 31;
  words[w] += idx << sh;
  if constexpr (sh + BITS > 32) words[w + 1] += idx >> (32 - sh);
}

// One tile's input for this lane: x[32 pp + 8 g + j] of token tau.  fp16:
// four half8; fp32: eight float4 (c = 2 pp + k holds j = 4 k .. 4 k + 3).
template <typename TIN> struct RawTile;
template <> struct RawTile<_Float16> { half8 x[4]; };
template <> struct RawTile<float> { float4v x[8]; };

template <int BITS, int MODE, typename TIN>
__global__ __launch_bounds__(kThreadsM) void quant_mfma_kernel(QuantParams p, QuantGrid grid) {
  constexpr bool kProd = MODE == TQ_MODE_PROD;
  constexpr bool kHeadq = MODE == TQ_MODE_HEADQ;  // 2-bit base + rank-16 4-bit side code
  constexpr bool kF32 = sizeof(TIN) == 4;
  // Index search on y * kRes: the residual comes out at the 2^12 scale of its fp16 split.
  constexpr float kRes = (kProd || kHeadq) ? 4096.0f : 1.0f;
  __shared__ __attribute__((aligned(16))) LutEntry s_lut[kLutMax];
  __shared__ float s_cent[16];
  __shared__ __attribute__((aligned(16))) half8 s_S[kProd ? 8 * 4 * 64 : 1];
  __shared__ __attribute__((aligned(16))) half8 s_A[8 * 64];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tau = lane & 15, g = lane >> 4;
  constexpr int NB = (1 << BITS) - 1;

  // ---- per-block tables -------------------------------------------------------------
  for (int n = threadIdx.x; n < grid.cells; n += kThreadsM) {
    const float lo = ((float)n - (0.5f + kGridMargin) - (float)grid.center) / grid.scale;
    const float hi = ((float)n + (0.5f + kGridMargin) - (float)grid.center) / grid.scale;
    uint32_t base = 0;
    float t = INFINITY;
    for (int k = 0; k < NB; ++k) {
      const float b = p.bounds[k];
      if (b < lo) base++;
      else if (b < hi && t == INFINITY) t = b;
    }
    s_lut[n].t = t * kRes;
    s_lut[n].base = base;
  }
  if (threadIdx.x < 16) s_cent[threadIdx.x] = p.centroids[threadIdx.x] * kRes;
  if constexpr (kProd) {
    // Operand (mb, pp), lane (gk, e): S[row][col + j], j < 8, with
    // row = 32 (e / 4) + 4 mb + e % 4 and col = 32 gk + 8 pp.
    for (int i = threadIdx.x; i < 8 * 4 * 64; i += kThreadsM) {
      const int l = i & 63, pp = (i >> 6) & 3, mb = i >> 8;
      const int e = l & 15, gk = l >> 4;
      const int row = 32 * (e >> 2) + 4 * mb + (e & 3), col = 32 * gk + 8 * pp;
      half8 v;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (_Float16)p.S[row * 128 + col + j];
      s_S[i] = v;
    }
  }
  // Rotation operand (rb, kb) at s_A[(rb * 2 + kb) * 64 + lane]: lane (gA, e),
  // slot jj holds H64[r][jh] (identity for PLAIN) with the output row
  // r = 16 (e / 4) + 4 rb + e % 4 and the input index
  // jh = 16 (2 kb + jj / 4) + 4 gA + jj % 4 (what lane gA's B slots carry).
  for (int i = threadIdx.x; i < 8 * 64; i += kThreadsM) {
    const int op = i >> 6, ln = i & 63, e = ln & 15, gA = ln >> 4;
    const int rb = op >> 1, kb = op & 1;
    const int r = 16 * (e >> 2) + 4 * rb + (e & 3);
    half8 v8;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int jh = 16 * (2 * kb + (jj >> 2)) + 4 * gA + (jj & 3);
      float v;
      if (MODE == TQ_MODE_PLAIN) v = (r == jh) ? 1.f : 0.f;
      else v = parity((uint32_t)(r & jh)) ? -1.f : 1.f;
      v8[jj] = (_Float16)v;
    }
    s_A[i] = v8;
  }
  // Sign flips D as XOR masks on the lane's fp16 input dwords: dword w of
  // xin[pp] holds coordinates 32 pp + 8 g + 2 w and + 1.
  uint32_t dmask[4][4];
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c0 = 32 * pp + 8 * g + 2 * w;
      const uint32_t b0 = (p.signbits[c0 >> 5] >> (c0 & 31)) & 1u, b1 = (p.signbits[c0 >> 5] >> ((c0 + 1) & 31)) & 1u;
      dmask[pp][w] = MODE == TQ_MODE_PLAIN ? 0u : (b0 << 15) | (b1 << 31);
    }
  }
  __syncthreads();

  // Tiles are 16 consecutive tokens of one (b, h); the host guarantees that
  // the tile count and every per-head byte offset fit 31 / 32 bits.
  const int tph = (p.T + 15) >> 4;
  const int ntiles = p.B * p.H * tph;
  // 1.5 * 2^23 + center: fma(y, scale, bias) leaves round(y * scale) + center
  // in the low mantissa bits, so (bits << 3) + const is the entry's LDS offset.
  const float bias = 12582912.0f + (float)grid.center;
  const float gscale = grid.scale / kRes;
  const char* lut_bytes = reinterpret_cast<const char*>(s_lut);
  const float inv_sqrt_d = p.inv_sqrt_d;

  // The lane's input of token tau of a tile (clamped to the head's last
  // token past its end).
  auto load_tile = [&](int tl, RawTile<TIN>& raw) {
    const int bh = tl / tph;
    const int t = min((tl - bh * tph) * 16 + tau, p.T - 1);
    const int b = bh / p.H, h = bh - b * p.H;
    const TIN* xrow = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh + (int64_t)t * p.st;
    if constexpr (kF32) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        raw.x[c] = __builtin_nontemporal_load(reinterpret_cast<const float4v*>(xrow + 32 * (c >> 1) + 8 * g + 4 * (c & 1)));
    } else {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) raw.x[pp] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(xrow + 32 * pp + 8 * g));
    }
  };
  const int tstride = gridDim.x * kWavesM;
  int tile = blockIdx.x * kWavesM + wave;
  // The next tile's input is loaded while this one is processed (always
  // issued, clamped to the last tile, so the wait before use is static).
  // PROD's occupancy is set by its 48 KB of LDS (3 blocks per CU), so the
  // second buffer's registers cost it no waves.
  RawTile<TIN> xnext;
  load_tile(min(tile, ntiles - 1), xnext);
  for (; tile < ntiles; tile += tstride) {
    const RawTile<TIN> raw = xnext;
    load_tile(min(tile + tstride, ntiles - 1), xnext);
    const int bh = tile / tph;
    const int t = (tile - bh * tph) * 16 + tau;
    const bool valid = t < p.T;
    // Destination slot: t, or pos[b] + t when appending; never outside [0, T_cap).
    const int64_t tw64 = (int64_t)t + (p.pos ? p.pos[bh / p.H] : 0);
    const bool wr = valid && tw64 >= 0 && tw64 < p.T_cap;
    const uint32_t tw = (uint32_t)tw64;

    // ||x||^2: fp16 products are exact in fp32.  fp32 input: the vector is
    // scaled by 2^14 / nu (entries at most 2^14, inside fp16's range; typical
    // entries large enough that the lo part stays a normal fp16) and split
    // into fp16 hi + lo parts, about 22 significant bits together; both parts
    // go through the same exact +-1 products into one fp32 accumulator.
    half8 xin[kF32 ? 2 : 1][4];
    float ss = 0.f;
    if constexpr (kF32) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) ss = fmaf(raw.x[c][i], raw.x[c][i], ss);
    } else {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        xin[0][pp] = raw.x[pp];
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          half2v a2;
          a2.x = xin[0][pp][j];
          a2.y = xin[0][pp][j + 1];
          ss = __builtin_amdgcn_fdot2(a2, a2, ss, false);
        }
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    // fp16 input: the hardware square root and reciprocal square root (about
    // 1 ulp each; the norm is compared at 1e-6 and a decision moves only
    // next to a boundary).  fp32 input: correctly rounded, its 2^14 / nu
    // feeds the hi + lo split.
    const float nu = kF32 ? sqrtf(ss) : __builtin_amdgcn_sqrtf(ss);
    if constexpr (kF32) {
      const float rn = nu > 0.f ? kSplitScale / nu : 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // v is kept as the rounded fp32 product: left to itself the compiler
          // rounds the exact product straight to fp16 for hi but subtracts a
          // hi re-derived from the fp32 value for lo, which disagree next to
          // an fp16 rounding tie (lo then lands on the wrong side).
          float v = raw.x[c][i] * rn;
          asm volatile("" : "+v"(v));
          const _Float16 hi = (_Float16)v;
          xin[0][c >> 1][4 * (c & 1) + i] = hi;
          xin[1][c >> 1][4 * (c & 1) + i] = (_Float16)(v - (float)hi);
        }
    }

    // ---- rotation -------------------------------------------------------------------
    // Z[a][rb][i]: the 64-point product for input bit 0 = a at output index
    // 16 g + 4 rb + i.  B slot jj of K block kb = x[2 jh + a], jh as above:
    // halves a of dwords 2 m, 2 m + 1 of xin[2 kb + n / 2], m = n % 2.
    float4v Z[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) Z[a][rb] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int part = 0; part < (kF32 ? 2 : 1); ++part) {
      u32x4 xw[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        xw[pp] = __builtin_bit_cast(u32x4, xin[part][pp]);
        if (MODE != TQ_MODE_PLAIN) {
#pragma unroll
          for (int w = 0; w < 4; ++w) xw[pp][w] ^= dmask[pp][w];
        }
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const uint32_t sel = a ? 0x07060302u : 0x05040100u;
        u32x4 bw[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int pp = 2 * kb + (n >> 1), m = 2 * (n & 1);
            bw[kb][n] = __builtin_amdgcn_perm(xw[pp][m + 1], xw[pp][m], sel);
          }
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
          const float4v acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(s_A[(rb * 2 + 0) * 64 + lane],
                                                                    __builtin_bit_cast(half8, bw[0]), Z[a][rb], 0, 0, 0);
          Z[a][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(s_A[(rb * 2 + 1) * 64 + lane],
                                                             __builtin_bit_cast(half8, bw[1]), acc, 0, 0, 0);
        }
      }
    }
    // The scale to the unit vector (times kRes): fp32 input was already
    // scaled by 2^14 / nu; fp16 input takes 1 / nu as rsq(||x||^2).
    const float inv = nu > 0.f ? (kF32 ? (MODE == TQ_MODE_PLAIN ? 1.0f / kSplitScale : inv_sqrt_d * (kRes / kSplitScale))
                                       : (MODE == TQ_MODE_PLAIN ? 1.0f : inv_sqrt_d * kRes) * __builtin_amdgcn_rsqf(ss))
                               : 0.f;
    // y[rb][2 i + b] <-> coordinate 32 g + 8 rb + 2 i + b, scaled: the
    // 2-point stage (z0 +- z1) inv as z0 inv +- z1 inv, one product and two fmas.
    float y[4][8];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float z0 = Z[0][rb][i], z1 = Z[1][rb][i];
        if (MODE == TQ_MODE_PLAIN) {
          y[rb][2 * i] = z0 * inv;
          y[rb][2 * i + 1] = z1 * inv;
        } else {
          const float t1 = z1 * inv;
          y[rb][2 * i] = fmaf(z0, inv, t1);
          y[rb][2 * i + 1] = fmaf(z0, inv, -t1);
        }
      }
    }

    // ---- index and packing ----------------------------------------------------------
    // PROD: (BITS+1)-bit fields, the sign bits filled in after the sketch.
    constexpr int FB = kProd ? BITS + 1 : BITS;
    uint32_t words[FB];
#pragma unroll
    for (int k = 0; k < FB; ++k) words[k] = 0;
#define TQ_QIDX(I, A)                                                                          \
    {                                                                                          \
      const float yy = y[I][A];                                                                \
      const float f = fmaf(yy, gscale, bias);                                                  \
      const LutEntry e = *reinterpret_cast<const LutEntry*>(                                   \
          lut_bytes + ((__float_as_uint(f) << 3) - (0x4B400000u << 3)));                       \
      const uint32_t idx = e.base + (yy >= e.t ? 1u : 0u);                                     \
      put_index<FB, 8 * (I) + (A)>(words, idx);                                                \
      y[I][A] = (kProd || kHeadq) ? yy - s_cent[idx] : yy;                                     \
    }
#define TQ_QROW(I) TQ_QIDX(I, 0) TQ_QIDX(I, 1) TQ_QIDX(I, 2) TQ_QIDX(I, 3) \
                   TQ_QIDX(I, 4) TQ_QIDX(I, 5) TQ_QIDX(I, 6) TQ_QIDX(I, 7)
    TQ_QROW(0) TQ_QROW(1) TQ_QROW(2) TQ_QROW(3)
#undef TQ_QROW
#undef TQ_QIDX

    // Per-head planes: scalar base + 32-bit lane offset.
    const size_t vbase = (size_t)bh * p.T_cap;
    auto store_codes = [&]() {
      if (!wr) return;
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + vbase * (16 * FB) + (uint32_t)(tw * (16 * FB) + g * (4 * FB)));
      if (!(nu > 0.f)) {
#pragma unroll
        for (int k = 0; k < FB; ++k) words[k] = 0;
      }
      if constexpr (FB == 4) {
        u32x4 w4 = {words[0], words[1], words[2], words[3]};
        __builtin_nontemporal_store(w4, reinterpret_cast<u32x4*>(dst));
      } else if constexpr (FB == 3) {
        u32x3 w3 = {words[0], words[1], words[2]};
        __builtin_nontemporal_store(w3, reinterpret_cast<u32x3*>(dst));
      } else if constexpr (FB == 2) {
        u32x2 w2 = {words[0], words[1]};
        __builtin_nontemporal_store(w2, reinterpret_cast<u32x2*>(dst));
      } else {
        __builtin_nontemporal_store(words[0], dst);
      }
      if (g == 0) __builtin_nontemporal_store(nu, p.norms + vbase + tw);
    };
    if constexpr (!kProd) store_codes();

    if constexpr (kHeadq) {
      // ---- HeadQ side code ([P3] section 3) ----------------------------------------
      // z = U'^T e' with e' = nu (y - c[idx]) (the residual k - k_base, rotated)
      // and U' = Pi U_h: a [16 ranks x 128] x [128 x 16 tokens] product on the
      // matrix cores.  K block kb takes row 8 g + j from lane (g, tau)'s own
      // coordinate 32 g + 8 kb + j (its y[kb][j]), so the A operand holds
      // U'[32 g + 8 kb + j][tau] at lane (g, tau) and the result gives lane
      // (g, tau) ranks 4 g .. 4 g + 3 of token tau.  Both factors are split
      // into fp16 hi + lo (residual x 2^12, basis x 2^10; each value pinned as
      // its rounded fp32 before the split) and hi hi + hi lo + lo hi summed;
      // the basis parts come split already (rotate_basis_kernel).
      // y holds the residual times 2^12 already; for nu = 0 the scale zs below is 0.
      const size_t uo = (size_t)(bh % p.H) * (16 * 128) + tau * 128 + 32 * g;
      const _Float16* ubh = p.rbasis16 + uo;
      const _Float16* ubl = p.rbasis16 + (size_t)p.H * (16 * 128) + uo;
      float4v zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        half8 eh, el;
        const half8 uh = *reinterpret_cast<const half8*>(ubh + 8 * kb);
        const half8 ul = *reinterpret_cast<const half8*>(ubl + 8 * kb);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float ev = y[kb][j];
          asm volatile("" : "+v"(ev));
          const _Float16 ehj = (_Float16)ev;
          eh[j] = ehj;
          el[j] = (_Float16)(ev - (float)ehj);
        }
        zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(uh, eh, zacc, 0, 0, 0);
        zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(uh, el, zacc, 0, 0, 0);
        zacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ul, eh, zacc, 0, 0, 0);
      }
      // z_r = nu * zacc / 2^22; s_z = max_r |z_r| / 7; code = clamp(rne(z / s_z), -7, 7) + 7.
      const float zs = nu * (1.0f / 4194304.0f);
      float z[4], zmax = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = zacc[i] * zs;
        zmax = fmaxf(zmax, fabsf(z[i]));
      }
      zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
      zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
      const float sz = zmax / 7.0f;
      uint32_t half = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int c = 7;
        if (sz > 0.f) {
          float qz = rintf(z[i] / sz);
          qz = fminf(fmaxf(qz, -7.0f), 7.0f);
          c = (int)qz + 7;
        }
        half |= (uint32_t)c << (4 * i);
      }
      if (wr) {
        // Ranks 4 g .. 4 g + 3 are bits 16 g .. 16 g + 15 of the token's 8-byte code.
        __builtin_nontemporal_store((uint16_t)half,
                                    reinterpret_cast<uint16_t*>(p.side + vbase * 8 + (uint32_t)(tw * 8 + 2 * g)));
        if (g == 0) __builtin_nontemporal_store(sz, p.side_scale + vbase + tw);
      }
    }

    if constexpr (kProd) {
      // ---- QJL sketch of the residual ----------------------------------------------
      // y holds r 2^12: g2 = 2^24 ||r||^2 exactly, and sqrt of it 2^12 ||r||.
      float g2 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int a = 0; a < 8; ++a) g2 = fmaf(y[i][a], y[i][a], g2);
      g2 += __shfl_xor(g2, 16, 64);
      g2 += __shfl_xor(g2, 32, 64);
      // Operand pp, slot j = coordinate 32 g + 8 pp + j = y[pp][j].
      // r - hi (exact) as one mixed-precision fma per element, hi * m1 + r: m1
      // is -1 kept opaque so that it is not folded into a subtraction, which
      // would first convert hi to fp32.
      float m1 = -1.0f;
      asm volatile("" : "+s"(m1));
      half8 Bhi[4], Blo[4];
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const float r0 = y[pp][j], r1 = y[pp][j + 1];
          const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0, r1));
          const half2v lo = __builtin_bit_cast(
              half2v, __builtin_amdgcn_cvt_pkrtz(fmaf((float)hi.x, m1, r0), fmaf((float)hi.y, m1, r1)));
          Bhi[pp][j] = hi.x; Bhi[pp][j + 1] = hi.y;
          Blo[pp][j] = lo.x; Blo[pp][j + 1] = lo.y;
        }
      }
      // Row block mb gives lane (g, tau) sketch rows 32 g + 4 mb + i, i < 4,
      // whose sign bit is bit [p >= 0], the complement of the product's sign
      // bit (they differ only at p = -0, where p is exactly zero).  Two
      // blocks in flight at a time keep the S operands (LDS reads) from all
      // being hoisted into registers.  Rows are visited from 31 down.
      //   4-bit fields: each row's sign bit is funnel-shifted in 4 bits at a
      //   time (with 3 bits of exponent below it, masked off), so that rows
      //   8 w .. 8 w + 7 end in nibbles 0 .. 7 of cur; the four dwords roll
      //   through sx0..sx3.  Other widths: one bit per row, spread after.
      uint32_t sx0 = 0, sx1 = 0, sx2 = 0, sx3 = 0, sneg = 0;
#pragma unroll 1
      for (int t = 3; t >= 0; --t) {
        uint32_t cur = 0;
#pragma unroll
        for (int h = 1; h >= 0; --h) {
          const int mb = 2 * t + h;
          float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const half8 A = s_S[(mb * 4 + pp) * 64 + lane];
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bhi[pp], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Blo[pp], acc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 3; i >= 0; --i) {
            if constexpr (FB == 4) cur = __builtin_amdgcn_alignbit(cur, __float_as_uint(acc[i]), 28);
            else sneg = __builtin_amdgcn_alignbit(sneg, __float_as_uint(acc[i]), 31);
          }
        }
        sx3 = sx2; sx2 = sx1; sx1 = sx0; sx0 = cur;
      }
      if constexpr (FB == 4) {
        words[0] |= ~sx0 & 0x88888888u;
        words[1] |= ~sx1 & 0x88888888u;
        words[2] |= ~sx2 & 0x88888888u;
        words[3] |= ~sx3 & 0x88888888u;
      } else {
        const uint32_t sbits = ~sneg;
#pragma unroll
        for (int o = 0; o < 32; ++o) {
          const int bit = FB * o + BITS;
          words[bit >> 5] |= ((sbits >> o) & 1u) << (bit & 31);
        }
      }
      store_codes();
      if (wr && g == 0) __builtin_nontemporal_store(nu > 0.f ? sqrtf(g2) * (1.0f / 4096.0f) : 0.f, p.gamma + vbase + tw);
    }
  }
}

template <int BITS, int MODE>
hipError_t launch_m(const QuantParams& p, const QuantGrid& grid, int nblocks, hipStream_t s) {
  if (p.dtype == TQ_F32)
    hipLaunchKernelGGL((quant_mfma_kernel<BITS, MODE, float>), dim3(nblocks), dim3(kThreadsM), 0, s, p, grid);
  else
    hipLaunchKernelGGL((quant_mfma_kernel<BITS, MODE, _Float16>), dim3(nblocks), dim3(kThreadsM), 0, s, p, grid);
  return hipGetLastError();
}

}  // namespace

bool quant_mfma_supported(const QuantParams& p) {
  // 32-bit tile indices and per-head byte offsets (at most 64 bytes per token).
  const long tiles = (long)p.B * p.H * ((p.T + 15) / 16);
  // HeadQ: the 2-bit base with a rank-16, 4-bit side code, once the rotated
  // basis (Pi U_h)^T [H][16][128] is in p.rbasis and its fp16 split in p.rbasis16.
  const bool headq_ok = p.mode == TQ_MODE_HEADQ && p.bits == 2 && p.rank == 16 && p.side_bits == 4 && p.rbasis16;
  return p.d == 128 && (p.dtype == TQ_F16 || p.dtype == TQ_F32) && (p.mode != TQ_MODE_HEADQ || headq_ok) &&
         p.bits >= 1 && p.bits <= 4 &&
         tiles < (1L << 31) && p.T_cap <= (1 << 24);
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
    case TQ_MODE_HEADQ * 8 + 2: return launch_m<2, TQ_MODE_HEADQ>(p, grid, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
