// Write side of QJL-sketched (PROD) tensors at d = 256, 512 and 1024, with
// the sketch projection S r on the matrix cores.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
//
// Same result as the other quantisers (norm split, seeded sign flip +
// normalised Walsh-Hadamard rotation, Beta Lloyd-Max index, LSB-first
// (b+1)-bit fields index | sign << b, [P1] "Esquemas de Cuantización" 2-3),
// with the sketch signs sign(S r) of the rotated residual r = y - c[idx]
// ([P1] "Contribuciones Clave" 1).  At these head dims S r is a real matrix
// product over the token batch: [tokens x d] x [d x d] per tile.  One block
// (8 waves) owns a tile of MT = 32768 / d tokens of one head:
//   1. quantise: L = d/32 lanes per token (lane j holds coordinates
//      32 j .. 32 j + 31); norm, sign flip, butterfly rotation, index search,
//      code fields, gamma = ||r||; the residual, scaled by 2^12, goes to LDS
//      as fp16 hi (rounded toward zero) and lo parts, so r - hi is exact and
//      the two products keep about 22 bits;
//   2. project: P = R S^T with v_mfma_f32_32x32x16_f16, S exact in fp16 and
//      streamed from L2 (the whole of S is read once per tile); each wave
//      owns 32 tokens x 128 sketch rows (four 32 x 32 output blocks) and runs
//      the d-long contraction in steps of 64, loading the next step's S
//      fragments while the current ones feed the matrix cores.  S is stored
//      in the order the operand registers take it (sketch_fragment_index
//      below), so each fragment load is one contiguous 1 KB run per wave
//      instead of a gather over 32 rows;
//   3. signs: one ballot per output register turns 32 lanes' [P >= 0] into
//      the sign word of 32 sketch rows of one token; the lanes of phase 1
//      merge their token's word into their code fields and store them.
// Every token's projection is the same sequence of operations whatever its
// slot in the tile, so appends reproduce a whole-sequence quantise bit for
// bit.  Stores are non-temporal (the decode streams the cache next).
#include "device_common.h"

namespace tq {
namespace {

constexpr int kSkThreads = 1024;
constexpr int kSkWaves = kSkThreads / 64;
constexpr int kRowPad = 8;  // fp16 per LDS residual row beyond d: rows 4 banks apart

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct SkGeom {
  static constexpr int L = D / 32;                         // lanes per token
  static constexpr int VPW = 64 / L;                       // tokens per wave step
  static constexpr int MT = 32 * 1024 / D;                 // tokens per tile
  static constexpr int STEPS = MT / (kSkWaves * VPW);      // token steps of phase 1
  static constexpr int ROW = D + kRowPad;                  // fp16 per residual row
  static constexpr int TB = MT / 32;                       // 32-token blocks of the product
  static constexpr int WPT = kSkWaves / TB;                // waves per token block
  static constexpr int RBW = (D / 32) / WPT;               // 32-row blocks per wave
  static constexpr int KSTEPS = D / 64;                    // contraction steps of 64
  // Residual rows (hi, lo), sign words, and the code words of phase 1 (at
  // most 4 bits per coordinate), which wait there for their sign bits
  // instead of in registers across the product.
  static constexpr size_t kLds = 2 * (size_t)MT * ROW * 2 + (size_t)MT * (D / 32) * 4 + (size_t)MT * D / 2;
  static_assert(STEPS * kSkWaves * VPW == MT, "tile split");
  static_assert(RBW == 2 && KSTEPS % 2 == 0, "product split");
};

}  // namespace

// Position in the fragment-ordered copy of S of element S[row][col]: the
// operand of sketch-row block rb = row / 32, contraction step c = col / 64,
// sub-step u = (col % 32) / 8, lane (hh, mm) = ((col % 64) / 32, row % 32),
// slot e = col % 8, as [rb][c][u][lane][e].
size_t sketch_fragment_index(int d, int row, int col) {
  const int rb = row >> 5, mm = row & 31, c = col >> 6, hh = (col >> 5) & 1, u = (col >> 3) & 3, e = col & 7;
  return ((((size_t)rb * (d / 64) + c) * 4 + u) * 64 + (hh * 32 + mm)) * 8 + e;
}

namespace {

// Grid lookup of the Lloyd-Max index: cell n = round(y * scale) + center
// holds the boundary inside the cell's window (+inf if none) and the number of
// boundaries below it, so the index is base + [y >= t].
struct SkLut {
  float t;
  uint32_t base;
};
constexpr int kSkLutMax = 512;  // cells of a 3-bit grid at d = 1024: 165

template <int D, int BITS, typename TIN>
__global__ __launch_bounds__(kSkThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void quant_sketch_kernel(QuantParams p, QuantGrid grid) {
  using G = SkGeom<D>;
  constexpr int FB = BITS + 1;           // field width: index | sign << BITS
  constexpr int NB = (1 << BITS) - 1;    // boundaries
  constexpr int NW = D / 32;             // sign words per token
  __shared__ __attribute__((aligned(16))) char smem[G::kLds];
  __shared__ float s_cent[16];
  __shared__ __attribute__((aligned(8))) SkLut s_lut[kSkLutMax];
  static_assert(G::kLds + sizeof(float) * 16 + sizeof(SkLut) * kSkLutMax <= 163840, "LDS budget");
  _Float16* a_hi = reinterpret_cast<_Float16*>(smem);
  _Float16* a_lo = a_hi + G::MT * G::ROW;
  uint32_t* sgn = reinterpret_cast<uint32_t*>(a_lo + G::MT * G::ROW);
  uint32_t* cwords = sgn + G::MT * NW;  // [token m][lane j][FB]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & (G::L - 1), slot = lane / G::L;
  if (threadIdx.x < 16) s_cent[threadIdx.x] = p.centroids[threadIdx.x];
  for (int n = threadIdx.x; n < grid.cells; n += kSkThreads) {
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
  __syncthreads();

  const int tph = (p.T + G::MT - 1) / G::MT;
  const int bh = blockIdx.x / tph;
  const int t0 = (blockIdx.x - bh * tph) * G::MT;
  const int b = bh / p.H, h = bh - b * p.H;
  const TIN* xbase = reinterpret_cast<const TIN*>(p.x) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int64_t slot0 = p.pos ? p.pos[b] : 0;  // destination slot of token 0 (append)
  const size_t vbase = (size_t)bh * p.T_cap;
  const uint32_t dword = p.signbits[j];

  // ---- 1. quantise the tile's tokens ------------------------------------------------
  uint32_t words[G::STEPS][FB];
  bool nonzero[G::STEPS];
  static_assert(FB <= 4, "code words per lane");
#pragma unroll
  for (int s = 0; s < G::STEPS; ++s) {
    const int m = s * (kSkWaves * G::VPW) + wave * G::VPW + slot;  // token within the tile
    const int t = t0 + m;
    const bool valid = t < p.T;
    float v[32];
    load32<TIN>(xbase + (int64_t)min(t, p.T - 1) * p.st + 32 * j, v);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) ss = fmaf(v[e], v[e], ss);
    ss = group_sum(ss, G::L);
    const float nu = sqrtf(ss);
    const bool nz = valid && nu > 0.f;
    nonzero[s] = nz;
    apply_signs(v, dword);
    wht_group(v, j, G::L);
    const float inv = nz ? p.inv_sqrt_d / nu : 0.f;
#pragma unroll
    for (int k = 0; k < FB; ++k) words[s][k] = 0;
    float g2 = 0.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float y = v[e] * inv;  // the rotated unit vector (0 for a zero or padding token)
      const float f = fmaf(y, grid.scale, gbias);
      const SkLut ent = s_lut[__float_as_uint(f) - 0x4B400000u];
      uint32_t c = ent.base + (y >= ent.t ? 1u : 0u);
      c = nz ? c : 0u;
      const float r = nz ? y - s_cent[c] : 0.f;
      g2 = fmaf(r, r, g2);
      v[e] = r * 4096.0f;
      const int bit = FB * e, wi = bit >> 5, sh = bit & 31;
      words[s][wi] |= c << sh;
      if (sh + FB > 32) words[s][wi + 1] |= c >> (32 - sh);
    }
    g2 = group_sum(g2, G::L);
    const int64_t tw = slot0 + t;
    if (valid && j == 0 && tw >= 0 && tw < p.T_cap) {
      __builtin_nontemporal_store(nu, p.norms + vbase + tw);
      __builtin_nontemporal_store(nz ? sqrtf(g2) : 0.f, p.gamma + vbase + tw);
    }
    {
      uint32_t* cw = cwords + ((size_t)m * G::L + j) * FB;
#pragma unroll
      for (int k = 0; k < FB; ++k) cw[k] = words[s][k];
    }
    // Residual x 2^12 as fp16 hi (toward zero) + lo into row m of the tile.
    _Float16* dh = a_hi + m * G::ROW + 32 * j;
    _Float16* dl = a_lo + m * G::ROW + 32 * j;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half8 hi8, lo8;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float r0 = v[8 * q + e], r1 = v[8 * q + e + 1];
        const half2v hi = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0, r1));
        const half2v lo = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(r0 - (float)hi.x, r1 - (float)hi.y));
        hi8[e] = hi.x; hi8[e + 1] = hi.y;
        lo8[e] = lo.x; lo8[e + 1] = lo.y;
      }
      *reinterpret_cast<half8*>(dh + 8 * q) = hi8;
      *reinterpret_cast<half8*>(dl + 8 * q) = lo8;
    }
  }
  __syncthreads();

  // ---- 2. P = R S^T on the matrix cores -----------------------------------------------
  // Wave: token block tb (32 tokens), sketch-row blocks rb0 .. rb0 + 3.  Lane
  // (hh, mm) = (lane / 32, lane % 32).  Contraction step c covers
  // coordinates 64 c .. 64 c + 63; its sub-step u gives half hh the eight
  // coordinates 64 c + 32 hh + 8 u .. + 7, the same slots in the A operand
  // (token tb*32 + mm) and the B operand (sketch row 32 rb + mm).
  {
    const int tb = wave / G::WPT, rb0 = (wave % G::WPT) * G::RBW;
    const int hh = lane >> 5, mm = lane & 31;
    const _Float16* ah = a_hi + (tb * 32 + mm) * G::ROW + 32 * hh;
    const _Float16* al = a_lo + (tb * 32 + mm) * G::ROW + 32 * hh;
    // Fragment-ordered S: block (rb, c, u) is 64 lanes x 8 fp16, contiguous.
    const _Float16* sb = p.S16 + (size_t)rb0 * (G::KSTEPS * 4 * 512) + lane * 8;
    float16v acc[G::RBW];
#pragma unroll
    for (int r = 0; r < G::RBW; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][i] = 0.f;
    half8 B0[G::RBW][4], B1[G::RBW][4];
    auto load_b = [&](half8 (&Bx)[G::RBW][4], int c) {
#pragma unroll
      for (int r = 0; r < G::RBW; ++r)
#pragma unroll
        for (int u = 0; u < 4; ++u) Bx[r][u] = *reinterpret_cast<const half8*>(sb + ((size_t)(r * G::KSTEPS + c) * 4 + u) * 512);
    };
    auto product = [&](const half8 (&Bx)[G::RBW][4], int c) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const half8 xh = *reinterpret_cast<const half8*>(ah + 64 * c + 8 * u);
        const half8 xl = *reinterpret_cast<const half8*>(al + 64 * c + 8 * u);
#pragma unroll
        for (int r = 0; r < G::RBW; ++r) {
          acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xh, Bx[r][u], acc[r], 0, 0, 0);
          acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xl, Bx[r][u], acc[r], 0, 0, 0);
        }
      }
    };
    // The scheduling barriers keep each step's S loads where they are
    // issued, a whole step ahead of their use: left free, the scheduler sank
    // them to the end of the previous step's products and the L2 latency
    // showed.
    load_b(B0, 0);
#pragma unroll 1
    for (int c = 0; c < G::KSTEPS; c += 2) {
      load_b(B1, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      product(B0, c);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 2 < G::KSTEPS) load_b(B0, c + 2);
      __builtin_amdgcn_sched_barrier(0);
      product(B1, c + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- 3a. sign words: register i of block r holds P[token][row] for
    // token 8 (i / 4) + 4 hh + i % 4 of the block and row 32 (rb0 + r) + mm.
#pragma unroll
    for (int r = 0; r < G::RBW; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint64_t bal = __ballot(acc[r][i] >= 0.f);
        const int tok = tb * 32 + 8 * (i >> 2) + (i & 3);
        if (lane == 0) sgn[tok * NW + rb0 + r] = (uint32_t)bal;
        if (lane == 32) sgn[(tok + 4) * NW + rb0 + r] = (uint32_t)(bal >> 32);
      }
    }
  }
  __syncthreads();

  // ---- 3b. sign bits into the code fields, codes out -----------------------------------
#pragma unroll
  for (int s = 0; s < G::STEPS; ++s) {
    const int m = s * (kSkWaves * G::VPW) + wave * G::VPW + slot;
    const int t = t0 + m;
    const int64_t tw = slot0 + t;
    if (!(t < p.T && tw >= 0 && tw < p.T_cap)) continue;
    const uint32_t sw = nonzero[s] ? sgn[m * NW + j] : 0u;  // a zero vector keeps all-zero fields
    {
      const uint32_t* cw = cwords + ((size_t)m * G::L + j) * FB;
#pragma unroll
      for (int k = 0; k < FB; ++k) words[s][k] = cw[k];
    }
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int bit = FB * e + BITS;
      words[s][bit >> 5] |= ((sw >> e) & 1u) << (bit & 31);
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(p.codes + (vbase + tw) * (size_t)(D * FB / 8)) + j * FB;
    if constexpr (FB == 4) {
      __builtin_nontemporal_store(u32x4{words[s][0], words[s][1], words[s][2], words[s][3]}, reinterpret_cast<u32x4*>(dst));
    } else if constexpr (FB == 3) {
      __builtin_nontemporal_store(u32x3{words[s][0], words[s][1], words[s][2]}, reinterpret_cast<u32x3*>(dst));
    } else {
      __builtin_nontemporal_store(u32x2{words[s][0], words[s][1]}, reinterpret_cast<u32x2*>(dst));
    }
  }
}

template <int D, int BITS>
hipError_t launch_sk(const QuantParams& p, const QuantGrid& grid, hipStream_t s) {
  const long tiles = (long)p.B * p.H * ((p.T + SkGeom<D>::MT - 1) / SkGeom<D>::MT);
  if (p.dtype == TQ_F16)
    hipLaunchKernelGGL((quant_sketch_kernel<D, BITS, _Float16>), dim3((unsigned)tiles), dim3(kSkThreads), 0, s, p, grid);
  else
    hipLaunchKernelGGL((quant_sketch_kernel<D, BITS, float>), dim3((unsigned)tiles), dim3(kSkThreads), 0, s, p, grid);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sk_d(const QuantParams& p, const QuantGrid& grid, hipStream_t s) {
  switch (p.bits) {
    case 1: return launch_sk<D, 1>(p, grid, s);
    case 2: return launch_sk<D, 2>(p, grid, s);
    case 3: return launch_sk<D, 3>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool quant_sketch_supported(const QuantParams& p, const QuantGrid& grid) {
  const long tiles = (long)p.B * p.H * ((p.T + 31) / 32);
  return p.mode == TQ_MODE_PROD && (p.d == 256 || p.d == 512 || p.d == 1024) && p.bits >= 1 && p.bits <= 3 &&
         tiles < (1L << 31) && grid.cells <= kSkLutMax;
}

hipError_t launch_quantize_sketch(const QuantParams& p, const QuantGrid& grid, hipStream_t s) {
  switch (p.d) {
    case 256: return launch_sk_d<256>(p, grid, s);
    case 512: return launch_sk_d<512>(p, grid, s);
    case 1024: return launch_sk_d<1024>(p, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
