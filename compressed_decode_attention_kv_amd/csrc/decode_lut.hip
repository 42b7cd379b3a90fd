// Table-driven split decode for 2- to 4-bit keys and 1- to 4-bit values at
// d = 128..1024, the read side of [P1] "Esquemas de Cuantización" (KV, KQV,
// QKQV at n = 4) and [P2] "Contribuições Principais" 1 (TQ-KV, TQ-QKV at
// n = 2..4), plus HeadQ keys (2-bit base with a rank-16 4-bit side code, [P3]
// section 3 "Metodologia: HeadQ") over 1- to 4-bit values.
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
//
// Same arithmetic as decode_split_kernel (scores and value sums in the
// rotated domain), organised so that each byte of packed cache costs about
// one VALU instruction:
//   * a packed byte (two 4-bit codes, two (3-bit code, sign) fields of a
//     sketched tensor, or four 2-bit codes) is turned into an LDS address by
//     one v_perm, a 6-bit field (two 3-bit codes) by a shift and one
//     v_and_or_b32, and one LDS read returns the centroids (and the signs);
//   * the LDS tables are replicated across lanes so that every read of a
//     wave hits distinct banks (see the map below);
//   * key centroids stay fp32 (scores are exact in fp32); value centroids and
//     the +-1 sign patterns are fp16 and enter v_fma_mix_f32 with fp32
//     weights and fp32 accumulators; the key sketch term <S q, sigma> runs
//     on v_dot2_f32_f16 with S q in fp16 pairs (scaled by a power of two, its
//     largest entry in [1/2, 1)) against the exact +-1 pairs where registers
//     allow (d = 128, or both sides sketched), else in fp32 fma;
//   * with sketched values a lane adds two tokens' values at once:
//     their 4-bit fields merged nibble by nibble index the same table, and
//     v_dot2_f32_f16 takes both tokens' fp16 weights (kept in (0, 2^8] by a
//     running exponent frame of their own);
//   * d/32 lanes per token, lane j owns coordinates [32j, 32j+32); the
//     per-token scalars (norms, residual norms) are loaded by lanes 0..3 of
//     the token's group and broadcast (DPP within a quad at d = 128);
//   * all packed data is streamed with non-temporal loads, one token step
//     ahead of the arithmetic, addressed as a per-head base (scalar) plus a
//     32-bit per-lane offset;
//   * one persistent block per CU loops over (query, context chunk) units.
#include <cfloat>
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

// Block size and token loop, per variant (chosen by measurement):
//   * sketched values: 8 waves (2 per SIMD, up to 256 VGPRs) and two tokens
//     per lane step (below); every other variant 12 waves (3 per SIMD, 168
//     VGPRs) and one token per lane step;
//   * one token step is prefetched.  Two register buffers used in turn save
//     the copies of a prefetch-then-copy loop, and win at d <= 256; with a
//     sketch on one side only at d >= 512 they spill and serialise the table
//     reads, and the copy loop is kept there.  Deeper prefetch (three or four
//     buffers) measured no faster.
constexpr int lut_threads(bool sketched_values) { return sketched_values ? 512 : 768; }
constexpr bool lut_two_buffers(int d, bool kq, bool vq) { return kq == vq || d <= 256; }
// A value table indexed by a byte of two 4-bit fields (3-bit code | sketch
// sign) also serves a lane's two tokens at once: a byte made of field i of
// each token returns both tokens' centroids and signs, and one v_dot2_f32_f16
// with the two tokens' fp16 weights adds both.  Taken wherever the values
// carry a sketch, at 8 waves (registers to spare; at 12 waves the loop it
// needs measured no faster than the single-token one).
constexpr bool lut_pair_values(int vb, bool vq) {
  return vq && vb == 3;
}
constexpr int kMaxLutWaves = 12;
// LDS map.  A table indexed by a whole packed byte needs a 64 KB window
// (entry e at window + e*256, the byte lands in address bits 8..15 straight
// from v_perm); at most two such tables are live (one per tensor).  Tables
// indexed by a 6-bit field (3-bit codes without a sketch) hold 64 entries
// (16 KB) and sit above, followed by the wave-merge buffer.
// Replication per table (chosen by measurement of read throughput):
//   value pairs        fp16x2            b32   one copy per lane      (lane * 4)
//   sketched values    fp16x2 + 2 signs  b64   a copy per lane % 32   ((lane & 31) * 8)
//   key pairs          fp32x2            b64   a copy per lane % 32   ((lane & 31) * 8)
//   sketched keys      fp32x2 + 2 signs  b128  a copy per lane % 16   ((lane & 15) * 16)
//   key quads          fp32x4            b128  a copy per lane % 16   ((lane & 15) * 16), 2-bit keys
//   value quads        fp16x4            b64   a copy per lane % 32   ((lane & 31) * 8), 2-bit values
//   value octets       fp16x8            b128  a copy per lane % 16   ((lane & 15) * 16), 1-bit values
// A sketched tensor stores per coordinate a 4-bit field, 3-bit code | sign << 3
// (the sign of the same-index sketch row), so a byte holds two of them.
// KB == 2 is a 2-bit key code: the HeadQ base when the kernel's KS is set
// (with its side code), plain TQ-MSE otherwise.
template <int D, int KB, bool KQ, int VB, bool VQ>
struct LutMap {
  static constexpr bool kKeyByte = KB == 4 || KB == 2 || KQ;
  static constexpr bool kValByte = VB == 4 || VB <= 2 || VQ;
  static constexpr bool kKeySix = KB == 3 && !KQ, kValSix = VB == 3 && !VQ;
  static constexpr uint32_t nbyte_tables = kKeyByte + kValByte;
  static constexpr uint32_t six_base = 0x10000u * nbyte_tables;
  static constexpr uint32_t k_base = kKeyByte ? 0u : six_base;
  static constexpr uint32_t v_base = kValByte ? (kKeyByte ? 0x10000u : 0u) : six_base + (kKeySix ? 0x4000u : 0u);
  static constexpr uint32_t merge = six_base + 0x4000u * (kKeySix + kValSix);
  // The wave-merge buffer exists at d = 128 only; wider heads write one
  // partial per wave and leave the merge to the combine step.
  static constexpr uint32_t bytes = merge + (D == 128 ? kMaxLutWaves * (2 + 2 * 128) * 4 + 256 : 0);
  static_assert(nbyte_tables <= 2, "at most two byte-indexed tables");
  static_assert(bytes <= 163840, "LDS budget");
};
constexpr float kSlack = 8.0f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// LDS address of byte K of w: [lanereg.b0, w.bK, lanereg.b2, 0].
template <int K>
__device__ __forceinline__ uint32_t byte_addr(uint32_t w, uint32_t lanereg) {
  return __builtin_amdgcn_perm(w, lanereg, 0x0C020000u | ((4u + K) << 8));
}

// (x & m) | (y & ~m): one v_bfi_b32.
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t x, uint32_t y) { return (x & m) | (y & ~m); }

// LDS address of the 6-bit field at bit offset O of a 3-dword run:
// (field << 8) | lanereg, as one shift (or funnel shift) that puts the field
// at bits 8..13 and one v_and_or_b32.  The and-or is written out because the
// compiler otherwise splits it into an and plus an add.
template <int O>
__device__ __forceinline__ uint32_t field6_addr(const uint32_t* w, uint32_t lanereg) {
  constexpr int wi = O >> 5, sh = O & 31;
  uint32_t x;
  if constexpr (sh + 6 <= 32) {
    if constexpr (sh >= 8) x = w[wi] >> (sh - 8);
    else x = w[wi] << (8 - sh);
  } else {
    x = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh - 8);  // sh >= 27 here
  }
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(0x3f00u), "v"(lanereg));
  return r;
}

__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  return v;
}

template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), J * 0x55, 0xF, 0xF, true));
}

// Value of lane J of this lane's token group (L lanes per token).
template <int L, int J>
__device__ __forceinline__ float tok_bcast(float v, int lane) {
  if constexpr (L == 4) return quad_bcast<J>(v);
  else return __shfl(v, (lane & ~(L - 1)) | J, 64);
}

// Maximum over the L lanes of this lane's token group.
template <int L>
__device__ __forceinline__ float tok_max(float v) {
#pragma unroll
  for (int off = 1; off < L; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Sum over the L lanes of this lane's token group.
template <int L>
__device__ __forceinline__ float tok_sum(float v) {
  v = quad_sum(v);
#pragma unroll
  for (int off = 4; off < L; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Dwords per lane per token: b-bit codes, or 4-bit (code, sign) fields.
template <int B, bool Q>
constexpr int lane_dwords() { return Q ? B + 1 : B; }

template <int KB, bool KQ, int VB, bool VQ>
struct TokenData {
  uint32_t k[lane_dwords<KB, KQ>()];
  uint32_t ks;   // the HeadQ side-code dword (KS)
  uint32_t v[lane_dwords<VB, VQ>()];
  float sc;      // this lane's per-token scalar (lane j: nu_k, gamma_k, nu_v, gamma_v)
};

// Planes of one (batch, kv head): scalar base pointers.
struct HeadPlanes {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint8_t* ks;  // the HeadQ side codes (KS)
};

// A 32-bit lane offset the compiler keeps as is, so that loads take the
// scalar-base + vector-offset form instead of 64-bit address arithmetic.
__device__ __forceinline__ uint32_t lane_off(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <uint32_t BYTES>
__device__ __forceinline__ uint32_t token_bytes(uint32_t tr) {
  if constexpr ((BYTES & (BYTES - 1)) == 0) return tr * BYTES;
  else return __umul24(tr, BYTES);
}

// Token tr (index within the head) for lane j.  The host sends only
// T_cap <= 2^24 with T_cap * d / 2 < 2^32 here, so tr fits a 24-bit multiply
// (full rate, unlike a 32-bit one) and every byte offset fits 32 bits.
// Key words, side codes and the per-token scalar:
template <int D, bool KS, int KB, bool KQ, int VB, bool VQ>
__device__ __forceinline__ void load_keys(const HeadPlanes& h, uint32_t tr, int j, const float* sc_head,
                                          TokenData<KB, KQ, VB, VQ>& t) {
  constexpr int KW = lane_dwords<KB, KQ>();
  const uint32_t* kc = reinterpret_cast<const uint32_t*>(h.kc + lane_off(token_bytes<(uint32_t)D * KW / 8>(tr) + (uint32_t)j * (4u * KW)));
  if constexpr (KW == 4) {
    u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kc));
    t.k[0] = x.x; t.k[1] = x.y; t.k[2] = x.z; t.k[3] = x.w;
  } else if constexpr (KB == 2) {
    u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kc));
    t.k[0] = x.x; t.k[1] = x.y;
    // Side codes: 16 x 4 bits = 8 bytes per token; lane j uses codes 4j..4j+3.
    if constexpr (KS)
      t.ks = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(h.ks + lane_off(tr * 8u + (uint32_t)(j >> 1) * 4u)));
  } else {
#pragma unroll
    for (int i = 0; i < KW; ++i) t.k[i] = __builtin_nontemporal_load(kc + i);
  }
  t.sc = __builtin_nontemporal_load(sc_head + tr);
}

// Value words:
template <int D, int KB, bool KQ, int VB, bool VQ>
__device__ __forceinline__ void load_values(const HeadPlanes& h, uint32_t tr, int j, TokenData<KB, KQ, VB, VQ>& t) {
  constexpr int VW = lane_dwords<VB, VQ>();
  const uint32_t* vc = reinterpret_cast<const uint32_t*>(h.vc + lane_off(token_bytes<(uint32_t)D * VW / 8>(tr) + (uint32_t)j * (4u * VW)));
  if constexpr (VW == 4) {
    u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vc));
    t.v[0] = x.x; t.v[1] = x.y; t.v[2] = x.z; t.v[3] = x.w;
  } else if constexpr (VW == 2) {
    u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vc));
    t.v[0] = x.x; t.v[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < VW; ++i) t.v[i] = __builtin_nontemporal_load(vc + i);
  }
}

template <int D, bool KS, int KB, bool KQ, int VB, bool VQ>
__device__ __forceinline__ void load_token(const HeadPlanes& h, uint32_t tr, int j, const float* sc_head,
                                           TokenData<KB, KQ, VB, VQ>& t) {
  load_keys<D, KS>(h, tr, j, sc_head, t);
  load_values<D>(h, tr, j, t);
}

template <int D, int KB, bool KQ, bool KS, int VB, bool VQ>
__global__ __launch_bounds__(lut_threads(VQ))
__attribute__((amdgpu_waves_per_eu(lut_threads(VQ) / 256, lut_threads(VQ) / 256)))
void decode_lut_kernel(DecodeParams p) {
  constexpr int kLutThreads = lut_threads(VQ);
  constexpr int kLutWaves = kLutThreads / 64;
  using Map = LutMap<D, KB, KQ, VB, VQ>;
  __shared__ __attribute__((aligned(16))) char smem[LutMap<D, KB, KQ, VB, VQ>::bytes];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int d = D, L = D / 32, vpw = 64 / L;  // L lanes per token, 64/L tokens per wave step
  const int j = lane & (L - 1), slot = lane / L;

  // ---- tables -------------------------------------------------------------------
  {
    if constexpr (VQ) {
      // Byte e = (code0 | s0 << 3) | (code1 | s1 << 3) << 4: both centroids and both signs.
      for (int i = threadIdx.x; i < 256 * 32; i += kLutThreads) {
        const int e = i >> 5, l = i & 31;
        half4_t h;
        h.x = (_Float16)p.vc[e & 7];
        h.y = (_Float16)p.vc[(e >> 4) & 7];
        h.z = (e & 8) ? (_Float16)1.0f : (_Float16)-1.0f;
        h.w = (e & 128) ? (_Float16)1.0f : (_Float16)-1.0f;
        *reinterpret_cast<half4_t*>(smem + Map::v_base + e * 256 + l * 8) = h;
      }
    }
    if constexpr (VB == 2 && !VQ) {
      // Byte e: four 2-bit codes, coordinate i of the byte in bits 2i..2i+1.
      for (int i = threadIdx.x; i < 256 * 32; i += kLutThreads) {
        const int e = i >> 5, l = i & 31;
        half4_t h;
        h.x = (_Float16)p.vc[e & 3];
        h.y = (_Float16)p.vc[(e >> 2) & 3];
        h.z = (_Float16)p.vc[(e >> 4) & 3];
        h.w = (_Float16)p.vc[e >> 6];
        *reinterpret_cast<half4_t*>(smem + Map::v_base + e * 256 + l * 8) = h;
      }
    }
    if constexpr (VB == 1 && !VQ) {
      // Byte e: eight 1-bit codes, coordinate i of the byte in bit i.
      for (int i = threadIdx.x; i < 256 * 16; i += kLutThreads) {
        const int e = i >> 4, l = i & 15;
        half8_t h;
#pragma unroll
        for (int b = 0; b < 8; ++b) h[b] = (_Float16)p.vc[(e >> b) & 1];
        *reinterpret_cast<half8_t*>(smem + Map::v_base + e * 256 + l * 16) = h;
      }
    }
    constexpr int NV = (VQ || VB <= 2) ? 0 : (VB == 4 ? 256 : 64);
    for (int i = threadIdx.x; i < NV * 64; i += kLutThreads) {
      const int e = i >> 6, l = i & 63;
      const int lo = VB == 4 ? (e & 15) : (e & 7), hi = VB == 4 ? (e >> 4) : (e >> 3);
      half2_t h;
      h.x = (_Float16)p.vc[lo];
      h.y = (_Float16)p.vc[hi];
      *reinterpret_cast<half2_t*>(smem + Map::v_base + e * 256 + l * 4) = h;
    }
    if constexpr (KB == 2) {
      for (int i = threadIdx.x; i < 256 * 16; i += kLutThreads) {
        const int e = i >> 4, l = i & 15;
        float4_t c;
        c.x = p.kc[e & 3];
        c.y = p.kc[(e >> 2) & 3];
        c.z = p.kc[(e >> 4) & 3];
        c.w = p.kc[e >> 6];
        *reinterpret_cast<float4_t*>(smem + Map::k_base + e * 256 + l * 16) = c;
      }
    }
    if constexpr (KQ) {
      // Byte e as for sketched values: fp32 centroids, fp16 signs in z.
      for (int i = threadIdx.x; i < 256 * 16; i += kLutThreads) {
        const int e = i >> 4, l = i & 15;
        half2_t sg;
        sg.x = (e & 8) ? (_Float16)1.0f : (_Float16)-1.0f;
        sg.y = (e & 128) ? (_Float16)1.0f : (_Float16)-1.0f;
        float4_t c;
        c.x = p.kc[e & 7];
        c.y = p.kc[(e >> 4) & 7];
        c.z = __builtin_bit_cast(float, sg);
        c.w = 0.f;
        *reinterpret_cast<float4_t*>(smem + Map::k_base + e * 256 + l * 16) = c;
      }
    }
    constexpr int NK = KB == 4 ? 256 : (Map::kKeySix ? 64 : 0);
    for (int i = threadIdx.x; i < NK * 32; i += kLutThreads) {
      const int e = i >> 5, l = i & 31;
      const int lo = KB == 4 ? (e & 15) : (e & 7), hi = KB == 4 ? (e >> 4) : (e >> 3);
      float2_t c;
      c.x = p.kc[lo];
      c.y = p.kc[hi];
      *reinterpret_cast<float2_t*>(smem + Map::k_base + e * 256 + l * 8) = c;
    }
  }
  __syncthreads();

  const uint32_t lr_v = (VQ || VB == 2) ? (Map::v_base | ((uint32_t)(lane & 31) << 3))
                       : (VB == 1 ? (Map::v_base | ((uint32_t)(lane & 15) << 4)) : (Map::v_base | ((uint32_t)lane * 4u)));
  const uint32_t lr_k = (KB == 2 || KQ) ? (Map::k_base | ((uint32_t)(lane & 15) << 4)) : (Map::k_base | ((uint32_t)(lane & 31) << 3));
  // Lane j of a quad streams one per-token scalar: 0 nu_k, 1 gamma_k (or the
  // HeadQ side scale), 2 nu_v, 3 gamma_v.
  // (Lanes j >= 4 of wider groups load a norm they do not use.)
  const float* sc_src = j == 0 ? p.k.norms : (j == 1 ? (KQ ? p.k.gamma : (KS ? p.k.side_scale : p.k.norms))
                                          : (j == 2 ? p.v.norms : (j == 3 ? (VQ ? p.v.gamma : p.v.norms) : p.k.norms)));
  float* merge = reinterpret_cast<float*>(smem + Map::merge);
  const int R = p.B * p.Hkv * p.nsplit;

  for (int unit = blockIdx.x; unit < p.units; unit += gridDim.x) {
    const int x = unit & 7, kk = unit >> 3;
    const int g = kk % p.G, r = (kk / p.G) * 8 + x;
    if (r >= R) continue;  // uniform per block
    const int split = r % p.nsplit, bkv = r / p.nsplit;
    const int b = bkv / p.Hkv, kvh = bkv % p.Hkv;
    const int qi = b * p.Hq + kvh * p.G + g;
    // Per-sequence length (clamped to [0, T]); a split past it has no tokens.
    const int Tb = p.lens ? min(max(p.lens[b], 0), p.T) : p.T;
    const int t0 = split * p.chunk, t1 = min(Tb, t0 + p.chunk);
    const size_t vbase = (size_t)bkv * p.T_cap;
    HeadPlanes hp;
    hp.kc = p.k.codes + vbase * (D * lane_dwords<KB, KQ>() / 8);
    hp.vc = p.v.codes + vbase * (D * lane_dwords<VB, VQ>() / 8);
    hp.ks = KS ? p.k.side + vbase * 8 : nullptr;
    const float* sc_head = sc_src + vbase;

    constexpr bool kUDot = KQ && (VQ || D == 128);
    float q[32], u[KQ && !kUDot ? 32 : 1];
#pragma unroll
    for (int e = 0; e < 32; ++e) q[e] = p.qrot[(size_t)qi * d + 32 * j + e];
    if constexpr (KQ && !kUDot) {
#pragma unroll
      for (int e = 0; e < 32; ++e) u[e] = p.qsk[(size_t)qi * d + 32 * j + e];
    }
    // kUDot: S q as fp16 pairs times 2^-e (largest |entry| of the whole
    // vector in [1/2, 1): an exact scaling, taken back in uscale).
    half2_t uh[kUDot ? 16 : 1];
    float uscale = p.k_qjl;
    if constexpr (kUDot) {
      float uf[32], mx = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        uf[e] = p.qsk[(size_t)qi * d + 32 * j + e];
        mx = fmaxf(mx, fabsf(uf[e]));
      }
      mx = tok_max<L>(mx);
      int ex = 0;
      (void)frexpf(mx, &ex);
      const float down = ldexpf(1.0f, -ex);
      uscale = ldexpf(p.k_qjl, ex);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uh[i].x = (_Float16)(uf[2 * i] * down);
        uh[i].y = (_Float16)(uf[2 * i + 1] * down);
      }
    }
    // HeadQ: this lane's 4 entries of w = U^T q (side codes 4j..4j+3) and the
    // offset lev * sum(w) that turns a 4-bit code into code - lev.
    float sw4[KS ? 4 : 1], swoff = 0.f;
    if constexpr (KS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sw4[i] = p.qw[(size_t)qi * 16 + 4 * j + i];
        swoff += sw4[i];
      }
      swoff *= 7.0f;
    }
    float acc[32], ask[VQ ? 32 : 1];
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    if (VQ) {
#pragma unroll
      for (int e = 0; e < 32; ++e) ask[e] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    // Paired values: acc and ask hold sums in units of 2^M, M a running
    // maximum of s + log2(nu_v) (a finite sentinel until the first non-zero
    // value vector), so that every fp16 weight 2^(s + log2 nu_v - M) lies in
    // (0, 2^8] whatever the norms; the sums move to the 2^m frame of l at the end.
    constexpr float kNoFrame = -1e30f;
    float M = kNoFrame;

    const int stride = kLutWaves * vpw;
    int base = t0 + wave * vpw;
    // Score of this lane's token (log2 units, -inf past the end).
    auto score = [&](const TokenData<KB, KQ, VB, VQ>& cur, bool valid) -> float {
      // ---- key score: this lane's 32 coordinates ---------------------------------
      float sa = 0.f, sb = 0.f, pa = 0.f, pb = 0.f;
      if constexpr (KQ) {
        // Byte BB of dword w: coordinates (and sketch rows) 8 w + 2 BB, + 1.
        // The entry is read as float4 and the sign pair taken out of it through
        // an opaque copy: with bit casts of the elements of a 128-bit integer
        // read (or of the sign element of a float4 read), this compiler
        // (AMD clang 22, ROCm 7.2) fed element 0 to the later uses.
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#define TQ_KQBYTE(BB)                                                                          \
          {                                                                                    \
            const float4_t c = *reinterpret_cast<const float4_t*>(smem + byte_addr<BB>(cur.k[w], lr_k)); \
            sa = fmaf(q[8 * w + 2 * BB], c.x, sa);                                             \
            sb = fmaf(q[8 * w + 2 * BB + 1], c.y, sb);                                         \
            uint32_t sgw = __float_as_uint(c.z);                                               \
            asm("" : "+v"(sgw));                                                                \
            const half2_t sg = __builtin_bit_cast(half2_t, sgw);                               \
            if constexpr (kUDot) {                                                             \
              if ((BB) & 1) pb = __builtin_amdgcn_fdot2(uh[4 * w + BB], sg, pb, false);        \
              else pa = __builtin_amdgcn_fdot2(uh[4 * w + BB], sg, pa, false);                 \
            } else {                                                                           \
              pa = fmaf(u[8 * w + 2 * BB], (float)sg.x, pa);                                   \
              pb = fmaf(u[8 * w + 2 * BB + 1], (float)sg.y, pb);                               \
            }                                                                                  \
          }
          TQ_KQBYTE(0) TQ_KQBYTE(1) TQ_KQBYTE(2) TQ_KQBYTE(3)
#undef TQ_KQBYTE
        }
      } else if constexpr (KB == 2) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
#define TQ_K2BYTE(BB)                                                                          \
          {                                                                                    \
            const float4_t c = *reinterpret_cast<const float4_t*>(smem + byte_addr<BB>(cur.k[w], lr_k)); \
            sa = fmaf(q[16 * w + 4 * BB], c.x, sa);                                            \
            sb = fmaf(q[16 * w + 4 * BB + 1], c.y, sb);                                        \
            sa = fmaf(q[16 * w + 4 * BB + 2], c.z, sa);                                        \
            sb = fmaf(q[16 * w + 4 * BB + 3], c.w, sb);                                        \
          }
          TQ_K2BYTE(0) TQ_K2BYTE(1) TQ_K2BYTE(2) TQ_K2BYTE(3)
#undef TQ_K2BYTE
        }
      } else if (KB == 4) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#define TQ_KBYTE(BB)                                                                          \
          {                                                                                   \
            const float2_t c = *reinterpret_cast<const float2_t*>(smem + byte_addr<BB>(cur.k[w], lr_k)); \
            sa = fmaf(q[8 * w + 2 * BB], c.x, sa);                                            \
            sb = fmaf(q[8 * w + 2 * BB + 1], c.y, sb);                                        \
          }
          TQ_KBYTE(0) TQ_KBYTE(1) TQ_KBYTE(2) TQ_KBYTE(3)
#undef TQ_KBYTE
        }
      } else {
#define TQ_KPAIR(M)                                                                            \
        {                                                                                      \
          const uint32_t a = field6_addr<6 * (M)>(cur.k, lr_k);                                \
          const float2_t c = *reinterpret_cast<const float2_t*>(smem + a);                     \
          sa = fmaf(q[2 * (M)], c.x, sa);                                                      \
          sb = fmaf(q[2 * (M) + 1], c.y, sb);                                                  \
        }
        TQ_KPAIR(0) TQ_KPAIR(1) TQ_KPAIR(2) TQ_KPAIR(3) TQ_KPAIR(4) TQ_KPAIR(5) TQ_KPAIR(6) TQ_KPAIR(7)
        TQ_KPAIR(8) TQ_KPAIR(9) TQ_KPAIR(10) TQ_KPAIR(11) TQ_KPAIR(12) TQ_KPAIR(13) TQ_KPAIR(14) TQ_KPAIR(15)
#undef TQ_KPAIR
      }
      const float nu_k = tok_bcast<L, 0>(cur.sc, lane);
      float part = nu_k * (sa + sb);
      if constexpr (KS) {
        // Side-code correction s_z (w . (code - lev)) of this lane's 4 codes.
        const uint32_t sd = cur.ks >> (16 * (j & 1));
        float cs = -swoff;
#pragma unroll
        for (int i = 0; i < 4; ++i) cs = fmaf(sw4[i], (float)((sd >> (4 * i)) & 15u), cs);
        part = fmaf(tok_bcast<L, 1>(cur.sc, lane), cs, part);
      }
      if (KQ) {
        const float g_k = tok_bcast<L, 1>(cur.sc, lane);
        part = fmaf(nu_k * uscale * g_k, pa + pb, part);
      }
      const float s = tok_sum<L>(part) * p.scale_log2;
      return valid ? s : -INFINITY;
    };

    // One token step of this lane (slot, j): score, online softmax, value sums.
    auto step = [&](const TokenData<KB, KQ, VB, VQ>& cur, int sbase) {
      const bool valid = sbase + slot < t1;
      const float s = score(cur, valid);

      // ---- online softmax (per token slot) ----------------------------------------
      if (s > m + kSlack) {
        // s - m > 8 here and m is finite or -inf: the raw exp2 is exact enough
        // and gives 0 for m = -inf.
        const float alpha = __builtin_amdgcn_exp2f(m - s);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < 32; ++e) acc[e] *= alpha;
        if (VQ) {
#pragma unroll
          for (int e = 0; e < 32; ++e) ask[e] *= alpha;
        }
        m = s;
      }
      const float pt = valid ? __builtin_amdgcn_exp2f(s - m) : 0.f;  // s - m <= 8
      l += pt;
      const float wv = pt * tok_bcast<L, 2>(cur.sc, lane);

      // ---- value accumulation -----------------------------------------------------
      if constexpr (VQ) {
        // Byte BB of dword w: coordinates (and sketch rows) 8 w + 2 BB, + 1.
        const float wq = wv * tok_bcast<L, 3>(cur.sc, lane);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#define TQ_VQBYTE(BB)                                                                          \
          {                                                                                    \
            const half4_t h = *reinterpret_cast<const half4_t*>(smem + byte_addr<BB>(cur.v[w], lr_v)); \
            acc[8 * w + 2 * BB] = fmaf(wv, (float)h.x, acc[8 * w + 2 * BB]);                   \
            acc[8 * w + 2 * BB + 1] = fmaf(wv, (float)h.y, acc[8 * w + 2 * BB + 1]);           \
            ask[8 * w + 2 * BB] = fmaf(wq, (float)h.z, ask[8 * w + 2 * BB]);                   \
            ask[8 * w + 2 * BB + 1] = fmaf(wq, (float)h.w, ask[8 * w + 2 * BB + 1]);           \
          }
          TQ_VQBYTE(0) TQ_VQBYTE(1) TQ_VQBYTE(2) TQ_VQBYTE(3)
#undef TQ_VQBYTE
        }
      } else if constexpr (VB == 2) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
#define TQ_V2BYTE(BB)                                                                          \
          {                                                                                    \
            const half4_t h = *reinterpret_cast<const half4_t*>(smem + byte_addr<BB>(cur.v[w], lr_v)); \
            acc[16 * w + 4 * BB] = fmaf(wv, (float)h.x, acc[16 * w + 4 * BB]);                 \
            acc[16 * w + 4 * BB + 1] = fmaf(wv, (float)h.y, acc[16 * w + 4 * BB + 1]);         \
            acc[16 * w + 4 * BB + 2] = fmaf(wv, (float)h.z, acc[16 * w + 4 * BB + 2]);         \
            acc[16 * w + 4 * BB + 3] = fmaf(wv, (float)h.w, acc[16 * w + 4 * BB + 3]);         \
          }
          TQ_V2BYTE(0) TQ_V2BYTE(1) TQ_V2BYTE(2) TQ_V2BYTE(3)
#undef TQ_V2BYTE
        }
      } else if constexpr (VB == 1) {
#define TQ_V1BYTE(BB)                                                                          \
        {                                                                                      \
          const half8_t h = *reinterpret_cast<const half8_t*>(smem + byte_addr<BB>(cur.v[0], lr_v)); \
          _Pragma("unroll") for (int i = 0; i < 8; ++i) acc[8 * BB + i] = fmaf(wv, (float)h[i], acc[8 * BB + i]); \
        }
        TQ_V1BYTE(0) TQ_V1BYTE(1) TQ_V1BYTE(2) TQ_V1BYTE(3)
#undef TQ_V1BYTE
      } else if (VB == 4) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#define TQ_VBYTE(BB)                                                                           \
          {                                                                                    \
            const half2_t h = *reinterpret_cast<const half2_t*>(smem + byte_addr<BB>(cur.v[w], lr_v)); \
            acc[8 * w + 2 * BB] = fmaf(wv, (float)h.x, acc[8 * w + 2 * BB]);                   \
            acc[8 * w + 2 * BB + 1] = fmaf(wv, (float)h.y, acc[8 * w + 2 * BB + 1]);           \
          }
          TQ_VBYTE(0) TQ_VBYTE(1) TQ_VBYTE(2) TQ_VBYTE(3)
#undef TQ_VBYTE
        }
      } else {
#define TQ_VPAIR(M)                                                                            \
        {                                                                                      \
          const uint32_t a = field6_addr<6 * (M)>(cur.v, lr_v);                                \
          const half2_t h = *reinterpret_cast<const half2_t*>(smem + a);                       \
          acc[2 * (M)] = fmaf(wv, (float)h.x, acc[2 * (M)]);                                   \
          acc[2 * (M) + 1] = fmaf(wv, (float)h.y, acc[2 * (M) + 1]);                           \
        }
        TQ_VPAIR(0) TQ_VPAIR(1) TQ_VPAIR(2) TQ_VPAIR(3) TQ_VPAIR(4) TQ_VPAIR(5) TQ_VPAIR(6) TQ_VPAIR(7)
        TQ_VPAIR(8) TQ_VPAIR(9) TQ_VPAIR(10) TQ_VPAIR(11) TQ_VPAIR(12) TQ_VPAIR(13) TQ_VPAIR(14) TQ_VPAIR(15)
#undef TQ_VPAIR
      }
    };

    if constexpr (lut_pair_values(VB, VQ)) {
      // Tokens t and t + stride of this slot per step, two pairs of buffers
      // used in turn: the next pair's value words are loaded as a step
      // begins, its key words once this step's scores are in.  Past the end
      // the token index is clamped (re-reads).
      TokenData<KB, KQ, VB, VQ> xa, xb, ya, yb;
      const int s2 = 2 * stride;
      auto pair_step = [&](TokenData<KB, KQ, VB, VQ>& ta, TokenData<KB, KQ, VB, VQ>& tb,
                           TokenData<KB, KQ, VB, VQ>& na, TokenData<KB, KQ, VB, VQ>& nb, int pb) {
        load_values<D>(hp, (uint32_t)min(pb + s2 + slot, t1 - 1), j, na);
        load_values<D>(hp, (uint32_t)min(pb + s2 + stride + slot, t1 - 1), j, nb);
        const bool va = pb + slot < t1, vb = pb + stride + slot < t1;
        // Scheduling fences (measured): with sketched keys the scheduler
        // otherwise interleaves the two key phases and the value dwords and
        // runs out of registers (QKQV 0.50 -> 0.74 ms without them); with
        // plain keys it is better left free (KQV 0.44 -> 0.41 ms).
        const float sA = score(ta, va);
        if constexpr (KQ) __builtin_amdgcn_sched_barrier(0);
        const float sB = score(tb, vb);
        if constexpr (KQ) __builtin_amdgcn_sched_barrier(0);
        const float nuA = tok_bcast<L, 2>(ta.sc, lane), nuB = tok_bcast<L, 2>(tb.sc, lane);
        float gA = 0.f, gB = 0.f;
        if constexpr (VQ) {
          gA = tok_bcast<L, 3>(ta.sc, lane);
          gB = tok_bcast<L, 3>(tb.sc, lane);
        }
        load_keys<D, KS>(hp, (uint32_t)min(pb + s2 + slot, t1 - 1), j, sc_head, na);
        load_keys<D, KS>(hp, (uint32_t)min(pb + s2 + stride + slot, t1 - 1), j, sc_head, nb);
        // ---- online softmax (per token slot): l in the 2^m frame -----------------------
        const float smax = fmaxf(sA, sB);
        if (smax > m + kSlack) {
          l *= __builtin_amdgcn_exp2f(m - smax);  // 0 while m = -inf
          m = smax;
        }
        l += (va ? __builtin_amdgcn_exp2f(sA - m) : 0.f) + (vb ? __builtin_amdgcn_exp2f(sB - m) : 0.f);
        // Value weights in the 2^M frame (nu_v = 0 or past the end: weight 0).
        const float lamA = sA + __builtin_amdgcn_logf(nuA), lamB = sB + __builtin_amdgcn_logf(nuB);
        const float lmax = fmaxf(lamA, lamB);
        if (lmax > M + kSlack) {
          const float f = __builtin_amdgcn_exp2f(M - lmax);
#pragma unroll
          for (int e = 0; e < 32; ++e) acc[e] *= f;
          if (VQ) {
#pragma unroll
            for (int e = 0; e < 32; ++e) ask[e] *= f;
          }
          M = lmax;
        }
        const float wA = __builtin_amdgcn_exp2f(lamA - M), wB = __builtin_amdgcn_exp2f(lamB - M);
        half2_t wv2, wq2;
        wv2.x = (_Float16)wA;
        wv2.y = (_Float16)wB;
        if constexpr (VQ) {
          wq2.x = (_Float16)(wA * gA);
          wq2.y = (_Float16)(wB * gB);
        }

        // ---- value sums of the pair ----------------------------------------------------
        // Byte BB of lo (hi) is field 2 BB (2 BB + 1) of dword w of each token:
        // coordinate 8 w + 2 BB (+ 1), token A in the low nibble.
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (KQ) __builtin_amdgcn_sched_barrier(0);
          const uint32_t lo = bitsel(0x0F0F0F0Fu, ta.v[w], tb.v[w] << 4);
          const uint32_t hi = bitsel(0x0F0F0F0Fu, ta.v[w] >> 4, tb.v[w]);
#define TQ_VQPAIR(WORD, BB, E)                                                                 \
          {                                                                                  \
            const half4_t h = *reinterpret_cast<const half4_t*>(smem + byte_addr<BB>(WORD, lr_v)); \
            acc[E] = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 0, 1), wv2, acc[E], false); \
            ask[E] = __builtin_amdgcn_fdot2(__builtin_shufflevector(h, h, 2, 3), wq2, ask[E], false); \
          }
          TQ_VQPAIR(lo, 0, 8 * w) TQ_VQPAIR(hi, 0, 8 * w + 1) TQ_VQPAIR(lo, 1, 8 * w + 2) TQ_VQPAIR(hi, 1, 8 * w + 3)
          TQ_VQPAIR(lo, 2, 8 * w + 4) TQ_VQPAIR(hi, 2, 8 * w + 5) TQ_VQPAIR(lo, 3, 8 * w + 6) TQ_VQPAIR(hi, 3, 8 * w + 7)
#undef TQ_VQPAIR
        }
      };
      if (base < t1) {
        load_keys<D, KS>(hp, (uint32_t)min(base + slot, t1 - 1), j, sc_head, xa);
        load_keys<D, KS>(hp, (uint32_t)min(base + stride + slot, t1 - 1), j, sc_head, xb);
        load_values<D>(hp, (uint32_t)min(base + slot, t1 - 1), j, xa);
        load_values<D>(hp, (uint32_t)min(base + stride + slot, t1 - 1), j, xb);
      }
      while (base < t1) {
        pair_step(xa, xb, ya, yb, base);
        base += s2;
        if (base >= t1) break;
        pair_step(ya, yb, xa, xb, base);
        base += s2;
      }
      // Sums from the 2^M frame to the 2^m frame (no valid token: all zero).
      const float f = m == -INFINITY ? 0.f : exp2f(M - m);
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] *= f;
      if (VQ) {
#pragma unroll
        for (int e = 0; e < 32; ++e) ask[e] *= f;
      }
    } else if constexpr (lut_two_buffers(D, KQ, VQ)) {
      // Two buffers used in turn, so that the next step's loads never
      // overwrite registers that the current step still reads (no copies).
      // The next step is loaded unconditionally (the token index is clamped,
      // so past the end it re-reads token t1 - 1): with a fixed number of
      // loads in flight the wait before each step leaves the other buffer's
      // loads outstanding.
      TokenData<KB, KQ, VB, VQ> ta, tb;
      if (base < t1) load_token<D, KS>(hp, (uint32_t)min(base + slot, t1 - 1), j, sc_head, ta);
      while (base < t1) {
        load_token<D, KS>(hp, (uint32_t)min(base + stride + slot, t1 - 1), j, sc_head, tb);
        step(ta, base);
        base += stride;
        if (base >= t1) break;
        load_token<D, KS>(hp, (uint32_t)min(base + stride + slot, t1 - 1), j, sc_head, ta);
        step(tb, base);
        base += stride;
      }
    } else {
      TokenData<KB, KQ, VB, VQ> nxt;
      if (base < t1) load_token<D, KS>(hp, (uint32_t)min(base + slot, t1 - 1), j, sc_head, nxt);
      for (; base < t1; base += stride) {
        const TokenData<KB, KQ, VB, VQ> cur = nxt;
        if (base + stride < t1) load_token<D, KS>(hp, (uint32_t)min(base + stride + slot, t1 - 1), j, sc_head, nxt);
        step(cur, base);
      }
    }

    // ---- merge the token slots of the wave (lanes with equal j) -----------------------
    for (int off = L; off < 64; off <<= 1) {
      const float mo = __shfl_xor(m, off, 64), lo = __shfl_xor(l, off, 64);
      const float M = fmaxf(m, mo);
      const float a = (m == -INFINITY) ? 0.f : exp2f(m - M);
      const float c = (mo == -INFINITY) ? 0.f : exp2f(mo - M);
      l = l * a + lo * c;
#pragma unroll
      for (int e = 0; e < 32; ++e) acc[e] = acc[e] * a + __shfl_xor(acc[e], off, 64) * c;
      if (VQ) {
#pragma unroll
        for (int e = 0; e < 32; ++e) ask[e] = ask[e] * a + __shfl_xor(ask[e], off, 64) * c;
      }
      m = M;
    }
    if constexpr (D > 128) {
      // One partial per wave, [m, l, acc[d], ask[d]], merged by the combine
      // step with the other waves and splits of this query.
      if (slot == 0) {
        float* out = p.part + (((size_t)qi * p.nsplit + split) * kLutWaves + wave) * p.part_stride;
#pragma unroll
        for (int e = 0; e < 32; ++e) out[2 + 32 * j + e] = acc[e];
        if (VQ) {
#pragma unroll
          for (int e = 0; e < 32; ++e) out[2 + d + 32 * j + e] = ask[e];
        }
        if (j == 0) { out[0] = m; out[1] = l; }
      }
      continue;
    }
    const int rec = 2 + 2 * d;
    if (slot == 0) {
      float* wm = merge + wave * rec;
#pragma unroll
      for (int e = 0; e < 32; ++e) wm[2 + 32 * j + e] = acc[e];
      if (VQ) {
#pragma unroll
        for (int e = 0; e < 32; ++e) wm[2 + d + 32 * j + e] = ask[e];
      }
      if (j == 0) { wm[0] = m; wm[1] = l; }
    }
    __syncthreads();
    {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kLutWaves; ++w) M = fmaxf(M, merge[w * rec]);
      float sc[kLutWaves], lt = 0.f;
#pragma unroll
      for (int w = 0; w < kLutWaves; ++w) {
        const float mw = merge[w * rec];
        sc[w] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        lt += merge[w * rec + 1] * sc[w];
      }
      float* out = p.part + ((size_t)qi * p.nsplit + split) * p.part_stride;
      const int nvals = VQ ? 2 * d : d;
      for (int i = threadIdx.x; i < nvals; i += kLutThreads) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kLutWaves; ++w) v += merge[w * rec + 2 + i] * sc[w];
        out[2 + i] = v;
      }
      if (threadIdx.x == 0) { out[0] = M; out[1] = lt; }
    }
    __syncthreads();
  }
}

template <int D, int KB, bool KQ, bool KS, int VB, bool VQ>
hipError_t launch_lut_d(const DecodeParams& p, int nblocks, hipStream_t s) {
  hipLaunchKernelGGL((decode_lut_kernel<D, KB, KQ, KS, VB, VQ>), dim3(nblocks), dim3(lut_threads(VQ)), 0, s, p);
  return hipGetLastError();
}

template <int KB, bool KQ, int VB, bool VQ>
hipError_t launch_lut(const DecodeParams& p, int nblocks, hipStream_t s) {
  switch (p.d) {
    case 128: return launch_lut_d<128, KB, KQ, false, VB, VQ>(p, nblocks, s);
    case 256: return launch_lut_d<256, KB, KQ, false, VB, VQ>(p, nblocks, s);
    case 512: return launch_lut_d<512, KB, KQ, false, VB, VQ>(p, nblocks, s);
    case 1024: return launch_lut_d<1024, KB, KQ, false, VB, VQ>(p, nblocks, s);
  }
  return hipErrorInvalidValue;
}

// Value widths for one key variant: 4, 3 (with or without a sketch), 2, 1.
template <int KB, bool KQ>
hipError_t launch_lut_v(const DecodeParams& p, int vbits, int vqjl, int nblocks, hipStream_t s) {
  if (vqjl) return launch_lut<KB, KQ, 3, true>(p, nblocks, s);
  switch (vbits) {
    case 4: return launch_lut<KB, KQ, 4, false>(p, nblocks, s);
    case 3: return launch_lut<KB, KQ, 3, false>(p, nblocks, s);
    case 2: return launch_lut<KB, KQ, 2, false>(p, nblocks, s);
    case 1: return launch_lut<KB, KQ, 1, false>(p, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int lut_waves(int vqjl) { return lut_threads(vqjl) / 64; }

bool lut_supported(int d, int kbits, int kqjl, int kside, int side_rank, int side_bits, int vbits, int vqjl) {
  if (d != 128 && d != 256 && d != 512 && d != 1024) return false;
  const bool vok = vbits >= 1 && vbits <= 4 && (!vqjl || vbits == 3);
  if (kside) return d == 128 && kbits == 2 && side_rank == 16 && side_bits == 4 && vok && !vqjl;
  return kbits >= 2 && kbits <= 4 && (!kqjl || kbits == 3) && vok;
}


hipError_t launch_decode_lut(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl,
                             int nblocks, hipStream_t s) {
  if (kside) {  // HeadQ keys (2-bit base + side code) at d = 128, 1- to 4-bit values
    switch (vbits) {
      case 4: return launch_lut_d<128, 2, false, true, 4, false>(p, nblocks, s);
      case 3: return launch_lut_d<128, 2, false, true, 3, false>(p, nblocks, s);
      case 2: return launch_lut_d<128, 2, false, true, 2, false>(p, nblocks, s);
      case 1: return launch_lut_d<128, 2, false, true, 1, false>(p, nblocks, s);
    }
    return hipErrorInvalidValue;
  }
  if (kqjl) return launch_lut_v<3, true>(p, vbits, vqjl, nblocks, s);
  switch (kbits) {
    case 4: return launch_lut_v<4, false>(p, vbits, vqjl, nblocks, s);
    case 3: return launch_lut_v<3, false>(p, vbits, vqjl, nblocks, s);
    case 2: return launch_lut_v<2, false>(p, vbits, vqjl, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
