// Grouped-query decode on the matrix cores at d = 128..1024: the G >= 2 query heads
// of a KV head read each packed token once, as one block of up to 16
// queries ([P3] section 3 attends with several query heads per KV head;
// [P1] "Esquemas de Cuantización" and [P2] "Contribuições Principais" 1
// define the scores and value sums computed here, in the rotated domain).
//
// [P1] = "Resumen Técnico: Inferencia Estadística y Medidas de Calidad de
//        Cuantizaciones de Cache KV Inspiradas en TurboQuant"
// [P2] = "Resumo Técnico: Ablação, Inferência Estatística e Validação para
//        Compressão de KV-Cache"
// [P3] = "Resumo Técnico: HeadQ: Distorção Visível ao Modelo e Correção no
//        Espaço de Pontuação para Quantização de KV-Cache"
//
// A unit is (KV head, block of 16 query heads, context chunk), walked in steps
// of 16 tokens; at d = 128 one wave is one unit's worker, above d / 128 waves
// share a unit, each on 128 coordinates, and add their partial scores
// through LDS (one barrier per step):
//   * scores S[token][query] = sum_i c[idx_i] q_rot,i on
//     v_mfma_f32_16x16x32_f16 (A: the token's centroids, decoded from its
//     code bytes through LDS tables, lane (h, t) holding coordinates
//     32 h + 8 ks .. + 7 of token t; B: the queries, same slots; three
//     products per 32 coordinates, see below), times nu_k; HeadQ adds
//     s_z sum_r w_r (code_r - 7) on v_mfma_f32_16x16x16_f16 over the 16 ranks;
//     sketched keys add gamma_k sqrt(pi/2)/d sum_i (S q)_i sign_i with the
//     signs as exact fp16 +-1 against S q in hi + lo;
//   * online softmax per query in log2 units (the result layout gives lane
//     (h, g) tokens 4 h .. 4 h + 3 of query g, exactly the slots of the value
//     product's second operand), value weights 2^(s + log2 nu_v - M) in fp16
//     against a running frame M of their own (lazy rescale, weights in
//     (0, 2^8]) so no norm can overflow them;
//   * values: eight v_mfma_f32_16x16x16_f16 against the weights, product j
//     taking coordinate 8 m + j of the wave's 128 in row m: lane (h, m) reads
//     the fields of coordinates 8 m .. 8 m + 7 of tokens 4 h .. 4 h + 3 (one
//     load per token) and looks their centroids up by pairs (or quads) of
//     tokens, so the operand arrives already in the token-major slots the
//     product needs; sketched values also look up their signs, against the
//     weights times gamma_v (the sums the combine step turns into S^T acc_sk).
// Each lookup is one LDS read per table part at entry * stride + copy offset;
// the step's planes are read through buffer descriptors that end at the
// chunk's last token, so the tail of a chunk needs no clamps (reads past it
// return 0: finite centroids, zero norms, zero weights).
// Key centroids, queries and the HeadQ side weights enter the scores as fp16
// hi + lo pairs (hi x hi + hi x lo + lo x hi, about 22 bits: in fp16 alone
// the score error reached ~7e-4 at unit-variance keys); value centroids and
// weights are fp16 as in the table-driven decode; accumulation is fp32.  The partial
// record per (query, chunk) is the table-driven kernel's, merged by the
// combine step.
#pragma once
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

// Units (waves) per block at d = 128: one block per CU shares one set of
// tables, whose copies then fill most of the LDS; 12 waves (3 per SIMD, the
// register budget of 168), or 8 with a sketch (whose registers exceed it).
constexpr int mq_upb(int D, bool KQ, bool VQ) { return D == 128 ? (KQ || VQ ? 8 : 12) : 1; }
constexpr float kMqSlack = 8.0f;          // log2 units
constexpr int kMqRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw 32-bit data
constexpr int kMqNT = 2;                  // buffer load cache policy: non-temporal

// Waves per block: at d = 128 four independent workers; above, one unit's
// d / 128 waves, each on 128 coordinates.
constexpr int mq_threads(int D, bool KQ, bool VQ) { return 64 * (D == 128 ? mq_upb(D, KQ, VQ) : D / 128); }

// LDS budgets of the key and value tables: at d = 128 most of the LDS (one
// block per CU); at d = 256 and 512 small enough for several blocks per CU; at
// d = 1024 (one block of 8 waves per CU, by registers) 64 KB each beside the
// partial scores' 16 KB (at most 144 KB in all): two-part tables (keys' hi
// and lo; sketched values' centroids and signs) at 32 copies.
constexpr int mq_kbudget(int D, bool) { return D == 128 ? 65536 : D == 256 ? 16384 : D == 512 ? 32768 : 65536; }
constexpr int mq_vbudget(int D, bool) { return D == 128 ? 65536 : D == 256 ? 8192 : D == 512 ? 16384 : 65536; }

typedef _Float16 mq_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 mq_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 mq_half2 __attribute__((ext_vector_type(2)));
typedef float mq_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t mq_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mq_u32x2 __attribute__((ext_vector_type(2)));

// Table of one tensor's centroids indexed by a unit of W-bit fields, the first
// field in the lowest bits and the first slot: two 4-bit fields (half2; with a
// sketch a field is 3-bit code | sign << 3 and the code is taken), two 3-bit
// fields (a 6-bit index, half2), four 2-bit fields (half4) or four 1-bit
// fields (a 4-bit index, half4).  Each entry sits
// in C copies, copy = lane % C, against bank conflicts.  Two parts
// share one indexing: keys hold the fp16 hi parts of the centroids and the lo
// parts (c - hi) (a sketched key's signs are formed from its code words);
// values the centroids and, with a sketch, the signs (bit 3 of each field) as
// fp16 +-1 (+1 for a set bit).
template <int W, int PARTS, int C>
struct MqTab {
  static constexpr int entries = W == 3 ? 64 : W == 1 ? 16 : 256;
  static constexpr int bytes_per = W <= 2 ? 8 : 4;        // one copy of one part of an entry
  static constexpr int stride = C * bytes_per;            // bytes between entries
  // Parts lie 16 B further apart than their size: no multiple of 256 B and
  // more than 2 KB, so reads of two parts at one index never merge into one
  // wider LDS read (whose halves would then be moved apart into two operands).
  static constexpr int part = entries * stride + 16;
  static constexpr int bytes = PARTS * part;
};

// Copies of a table, copy = lane % copies: the most (a power of two, at most
// 64) within budget bytes.  At 64 copies every lane of a wave reads its
// own bank; at 32 two lanes share a bank (a conflict when their entries differ
// but fall into the same bank), at 8, eight.
constexpr int mq_copies(int W, int PARTS, int budget) {
  int c = 64;
  while (c > 1 && PARTS * (W == 3 ? 64 : W == 1 ? 16 : 256) * (W <= 2 ? 8 : 4) * c > budget) c /= 2;
  return c;
}

template <int W, int PARTS, int C, bool LO, bool SIGNS, bool MASK>
__device__ __forceinline__ void build_tab(char* tab, const float* c, int tid, int nthreads) {
  using Tab = MqTab<W, PARTS, C>;
  constexpr int N = W <= 2 ? 4 : 2;               // fields per entry
  for (int i = tid; i < Tab::entries * C; i += nthreads) {
    const int e = i / C;
    _Float16* d0 = reinterpret_cast<_Float16*>(tab + i * Tab::bytes_per);
#pragma unroll
    for (int q = 0; q < N; ++q) {
      const int f = (e >> (W * q)) & ((1 << W) - 1);
      const float v = c[MASK ? (f & 7) : f];
      const _Float16 h = (_Float16)v;
      d0[q] = h;
      if constexpr (LO) d0[Tab::part / 2 + q] = (_Float16)(v - (float)h);
      if constexpr (SIGNS) d0[(LO ? 2 : 1) * Tab::part / 2 + q] = ((f >> 3) & 1) ? (_Float16)1.0f : (_Float16)-1.0f;
    }
  }
}

__device__ __forceinline__ uint32_t mq_bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// Part P of the entry at byte offset a (entry * stride + the lane's copy offset).
template <int W, int PARTS, int C, int P>
__device__ __forceinline__ auto mq_ent(const char* tab, uint32_t a) {
  if constexpr (W <= 2) return *reinterpret_cast<const mq_half4*>(tab + P * MqTab<W, PARTS, C>::part + a);
  else return *reinterpret_cast<const mq_half2*>(tab + P * MqTab<W, PARTS, C>::part + a);
}

// Key operands of coordinates 8 ks .. 8 ks + 7 of the lane's 32 (its words w,
// LSB-first W-bit fields): hi parts, lo parts and, with a sketch, the signs.
template <int W, int PARTS, int C, bool SIGNS>
__device__ __forceinline__ void key8(const char* tab, const uint32_t* w, int ks, uint32_t cofs, mq_half8& ah,
                                     mq_half8& al, mq_half8& as) {
  constexpr uint32_t S = MqTab<W, PARTS, C>::stride;
  if constexpr (W == 2) {
    const uint32_t x = w[ks >> 1] >> (16 * (ks & 1));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t a = ((x >> (8 * q)) & 255u) * S + cofs;
      const mq_half4 h = mq_ent<W, PARTS, C, 0>(tab, a), l = mq_ent<W, PARTS, C, 1>(tab, a);
#pragma unroll
      for (int e = 0; e < 4; ++e) { ah[4 * q + e] = h[e]; al[4 * q + e] = l[e]; }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t f;
      if constexpr (W == 4) {
        f = (w[ks] >> (8 * q)) & 255u;
      } else {
        const int bit = 24 * ks + 6 * q, wi = bit >> 5, sh = bit & 31;
        f = w[wi] >> sh;
        if (sh > 26) f |= w[wi + 1] << (32 - sh);
        f &= 63u;
      }
      const uint32_t a = f * S + cofs;
      const mq_half2 h = mq_ent<W, PARTS, C, 0>(tab, a), l = mq_ent<W, PARTS, C, 1>(tab, a);
      ah[2 * q] = h.x; ah[2 * q + 1] = h.y;
      al[2 * q] = l.x; al[2 * q + 1] = l.y;
      if constexpr (SIGNS) {
        // The sign bit (bit 3) of fields 2q and 2q + 1 as fp16 +1 / -1
        // (0x3C00 / 0xBC00) straight from the word: each byte of lsg / hsg is
        // 0xBC with bit 7 flipped by the sign of the byte's low / high field,
        // and byte q of each goes to the high byte of its half.
        const uint32_t x = w[ks];
        const uint32_t lsg = ((x & 0x08080808u) << 4) ^ 0xBCBCBCBCu, hsg = (x & 0x80808080u) ^ 0xBCBCBCBCu;
        const uint32_t sel = 0x000C000Cu | ((uint32_t)q << 8) | ((uint32_t)(4 + q) << 24);
        const mq_half2 s = __builtin_bit_cast(mq_half2, __builtin_amdgcn_perm(hsg, lsg, sel));
        as[2 * q] = s.x; as[2 * q + 1] = s.y;
      }
    }
  }
}

// Value fields: vr holds, for each token 4 hq + e of the step, the fields of
// coordinates 8 mm .. 8 mm + 7 of the wave's 128 (W = 4: a word; W = 2: 16
// bits; W = 1: a byte; W = 3: the two words that hold its 24 bits, vsh bits
// into the first).
// value_index turns them once per step into the table indices of the value
// products: the pair (tokens 0, 1 | 2, 3) or quad entries of each coordinate.
template <int W>
__device__ __forceinline__ void value_index(const uint32_t* vr, uint32_t vsh, uint32_t* ix) {
  if constexpr (W == 4) {
    // byte k: field 2 k (ix[0], ix[2]) or 2 k + 1 (ix[1], ix[3]) of the two tokens
    ix[0] = mq_bfi(0x0F0F0F0Fu, vr[0], vr[1] << 4);
    ix[1] = mq_bfi(0x0F0F0F0Fu, vr[0] >> 4, vr[1]);
    ix[2] = mq_bfi(0x0F0F0F0Fu, vr[2], vr[3] << 4);
    ix[3] = mq_bfi(0x0F0F0F0Fu, vr[2] >> 4, vr[3]);
  } else if constexpr (W == 3) {
#pragma unroll
    for (int e = 0; e < 4; ++e) ix[e] = __builtin_amdgcn_alignbit(vr[2 * e + 1], vr[2 * e], vsh);
  } else if constexpr (W == 1) {
    // The 4 x 8 bit matrix (byte e = token e, bit j = coordinate j) transposed
    // by two delta swaps: byte k then holds coordinate k's four bits in its
    // low nibble and coordinate k + 4's in its high nibble (token e at bit e).
    uint32_t x = vr[0] | (vr[1] << 8) | (vr[2] << 16) | (vr[3] << 24);
    uint32_t t = (x ^ (x >> 7)) & 0x00AA00AAu;
    x ^= t ^ (t << 7);
    t = (x ^ (x >> 14)) & 0x0000CCCCu;
    x ^= t ^ (t << 14);
    ix[0] = x;
  } else {
    // Nibbles of R: fields 2 i of tokens 0 | 1 (low half) and 2 | 3 (high
    // half); of S: fields 2 i + 1.  Bytes 0 and 1 of ix[] then pair them up:
    // ix[0]: fields 0, 4; ix[1]: 2, 6; ix[2]: 1, 5; ix[3]: 3, 7.
    const uint32_t P = vr[0] | (vr[2] << 16), Q = vr[1] | (vr[3] << 16);
    const uint32_t R = mq_bfi(0x33333333u, P, Q << 2), S = mq_bfi(0x33333333u, P >> 2, Q);
    ix[0] = mq_bfi(0x0F0Fu, R, R >> 12);
    ix[1] = mq_bfi(0x0F0Fu, R >> 4, R >> 16);
    ix[2] = mq_bfi(0x0F0Fu, S, S >> 12);
    ix[3] = mq_bfi(0x0F0Fu, S >> 4, S >> 16);
  }
}

// First operand of value product j: coordinate 8 mm + j of tokens 4 hq .. 4 hq
// + 3 (and, with a sketch, their signs).
template <int W, int PARTS, int C, bool SIGNS>
__device__ __forceinline__ void value_ops(const char* tab, const uint32_t* ix, int j, uint32_t cofs, mq_half4& A,
                                          mq_half4& As) {
  constexpr uint32_t S = MqTab<W, PARTS, C>::stride;
  // With 256-byte entries an index byte k of a word becomes the offset
  // byte k * 256 + copy offset in one byte permute (result bytes: the copy
  // offset, byte k, zero, zero).
  constexpr bool PERM = S == 256 && (W == 4 || W == 2);
  auto at = [&](uint32_t word, int k) -> uint32_t {
    if constexpr (PERM) return __builtin_amdgcn_perm(word, cofs, 0x0C0C0000u | ((4u + k) << 8));
    else return ((word >> (8 * k)) & 255u) * S + cofs;
  };
  if constexpr (W == 2) {
    A = mq_ent<W, PARTS, C, 0>(tab, at(ix[(j & 1) * 2 + ((j >> 1) & 1)], j >> 2));
  } else if constexpr (W == 1) {
    const uint32_t f = (ix[0] >> (8 * (j & 3) + 4 * (j >> 2))) & 15u;
    A = mq_ent<W, PARTS, C, 0>(tab, f * S + cofs);
  } else {
    uint32_t a01, a23;
    if constexpr (W == 4) {
      a01 = at(ix[j & 1], j >> 1);
      a23 = at(ix[2 + (j & 1)], j >> 1);
    } else {
      const uint32_t f01 = ((ix[0] >> (3 * j)) & 7u) | (((ix[1] >> (3 * j)) & 7u) << 3);
      const uint32_t f23 = ((ix[2] >> (3 * j)) & 7u) | (((ix[3] >> (3 * j)) & 7u) << 3);
      a01 = f01 * S + cofs;
      a23 = f23 * S + cofs;
    }
    const mq_half2 h01 = mq_ent<W, PARTS, C, 0>(tab, a01), h23 = mq_ent<W, PARTS, C, 0>(tab, a23);
    A = mq_half4{h01.x, h01.y, h23.x, h23.y};
    if constexpr (SIGNS) {
      const mq_half2 s01 = mq_ent<W, PARTS, C, 1>(tab, a01), s23 = mq_ent<W, PARTS, C, 1>(tab, a23);
      As = mq_half4{s01.x, s01.y, s23.x, s23.y};
    }
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mq_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kMqRsrcWord3);
}

__device__ __forceinline__ mq_float4 mq_ldf4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(mq_float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// KB, VB: index bits; KQ, VQ: sketched (4-bit fields, KB = VB = 3); KS: HeadQ
// side code (d = 128).
template <int D, int KB, bool KQ, bool KS, int VB, bool VQ>
__global__ __launch_bounds__(mq_threads(D, KQ, VQ)) void decode_mq_kernel(DecodeParams p) {
  constexpr int NT = mq_threads(D, KQ, VQ);
  constexpr int NW = NT / 64;                      // waves per block
  constexpr int NWU = D / 128;                     // waves per unit
  constexpr int UPB = NW / NWU;                    // units per block (mq_upb at d = 128, else 1)
  constexpr int KW = KQ ? 4 : KB, VW = VQ ? 4 : VB;  // field widths
  constexpr int KPARTS = 2, VPARTS = VQ ? 2 : 1;  // key signs come from the code words
  constexpr int CK = mq_copies(KW, KPARTS, mq_kbudget(D, KQ)), CV = mq_copies(VW, VPARTS, mq_vbudget(D, KQ));
  constexpr uint32_t RBK = D * KW / 8, RBV = D * VW / 8;  // code bytes per token
  // One LDS block: the value table first (at address 0, so that its lookup
  // offsets need no base), the key table, and for d > 128 the partial scores
  // of the unit's waves, double-buffered by step parity.
  constexpr int VBYTES = (MqTab<VW, VPARTS, CV>::bytes + 15) / 16 * 16;
  constexpr int KBYTES = (MqTab<KW, KPARTS, CK>::bytes + 15) / 16 * 16;
  constexpr int RED = NWU > 1 ? 2 * NWU * 64 : 0;   // float4 entries
  __shared__ __attribute__((aligned(16))) char s_lds[VBYTES + KBYTES + 16 * RED + 16];
  char* const s_vtab = s_lds;
  char* const s_ktab = s_lds + VBYTES;
  typedef mq_float4 RedRow[NWU > 1 ? NWU : 1][NWU > 1 ? 64 : 1];
  RedRow* const s_red = reinterpret_cast<RedRow*>(s_lds + VBYTES + KBYTES);
  build_tab<KW, KPARTS, CK, true, false, KQ>(s_ktab, p.kc, threadIdx.x, NT);
  build_tab<VW, VPARTS, CV, false, VQ, VQ>(s_vtab, p.vc, threadIdx.x, NT);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wu = NWU > 1 ? wave : 0;               // wave within the unit: coordinates 128 wu ..
  const int hq = lane >> 4, mm = lane & 15;        // operand / result lane (h, m)
  // Key lookups: the key table's base rides in the lane's copy offset (kept
  // opaque, so it is not split off into an LDS offset field too narrow for it).
  uint32_t kcofs = VBYTES + (lane & (CK - 1)) * MqTab<KW, KPARTS, CK>::bytes_per;
  asm volatile("" : "+v"(kcofs));
  const uint32_t vcofs = (lane & (CV - 1)) * MqTab<VW, VPARTS, CV>::bytes_per;
  // Lane offsets within a step: key words of token mm, slice 4 wu + hq (32
  // coordinates); value fields of coordinates 8 mm .. of the wave's 128, token
  // 4 hq (+ e rows); per-token scalars of tokens 4 hq .. 4 hq + 3.
  const uint32_t vk = mm * RBK + 4 * KW * (4 * wu + hq);
  const uint32_t vj0 = VW == 3 ? (3 * mm) >> 2 : 0;
  const uint32_t vv = 4 * hq * RBV + 16 * VW * wu + (VW == 4 ? 4 * mm : VW == 2 ? 2 * mm : VW == 1 ? mm : 4 * vj0);
  const uint32_t vv2 = vv + (VW == 3 && vj0 < 11 ? 4 : 0);
  const uint32_t vsh = VW == 3 ? 8 * ((3 * mm) & 3) : 0;
  const uint32_t vn = 16 * hq, vsd = 8 * mm + 2 * hq;
  const int nqb = (p.G + 15) >> 4;
  const int R = p.B * p.Hkv * nqb * p.nsplit;
  const int u0 = NWU > 1 ? blockIdx.x : blockIdx.x * UPB + wave;
  const int ustride = NWU > 1 ? gridDim.x : gridDim.x * UPB;

  for (int unit = u0; unit < R; unit += ustride) {
    const int split = unit % p.nsplit;
    const int rest = unit / p.nsplit;
    const int qb = rest % nqb, bkv = rest / nqb;
    const int b = bkv / p.Hkv, kvh = bkv % p.Hkv;
    const int g = qb * 16 + mm;                     // this lane's query (result and weight slots)
    const bool gvalid = g < p.G;
    const int qi = b * p.Hq + kvh * p.G + min(g, p.G - 1);
    const int Tb = p.lens ? min(max(p.lens[b], 0), p.T) : p.T;
    const int t0 = split * p.chunk, t1 = min(Tb, t0 + p.chunk);
    const size_t vbase = (size_t)bkv * p.T_cap;
    // The head's planes up to token t1: reads of tokens t1 and beyond return 0
    // (finite centroids, zero norms; their weights are 0).
    const uint32_t n1 = t1 > 0 ? (uint32_t)t1 : 0u;
    const __amdgpu_buffer_rsrc_t rk = mq_rsrc(p.k.codes + vbase * RBK, n1 * RBK);
    const __amdgpu_buffer_rsrc_t rv = mq_rsrc(p.v.codes + vbase * RBV, n1 * RBV);
    const __amdgpu_buffer_rsrc_t rnk = mq_rsrc(p.k.norms + vbase, 4 * n1);
    const __amdgpu_buffer_rsrc_t rnv = mq_rsrc(p.v.norms + vbase, 4 * n1);
    __amdgpu_buffer_rsrc_t rsd = rnk, rsz = rnk, rgk = rnk, rgv = rnk;
    if constexpr (KS) {
      rsd = mq_rsrc(p.k.side + vbase * 8, 8 * n1);
      rsz = mq_rsrc(p.k.side_scale + vbase, 4 * n1);
    }
    if constexpr (KQ) rgk = mq_rsrc(p.k.gamma + vbase, 4 * n1);
    if constexpr (VQ) rgv = mq_rsrc(p.v.gamma + vbase, 4 * n1);

    // Queries (second operand of the scores): slots 128 wu + 32 h + 8 ks + e of
    // query g, and the same slots of S q for sketched keys.
    mq_half8 Qh[4], Ql[4], Uh[KQ ? 4 : 1], Ul[KQ ? 4 : 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t o = (size_t)qi * D + 128 * wu + 32 * hq + 8 * ks + e;
        const float v = gvalid ? p.qrot[o] : 0.f;
        Qh[ks][e] = (_Float16)v;
        Ql[ks][e] = (_Float16)(v - (float)Qh[ks][e]);
        if constexpr (KQ) {
          const float u = gvalid ? p.qsk[o] : 0.f;
          Uh[ks][e] = (_Float16)u;
          Ul[ks][e] = (_Float16)(u - (float)Uh[ks][e]);
        }
      }
    mq_half4 Wh, Wl;
    if constexpr (KS) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = gvalid ? p.qw[(size_t)qi * 16 + 4 * hq + e] : 0.f;
        Wh[e] = (_Float16)v;
        Wl[e] = (_Float16)(v - (float)Wh[e]);
      }
    }
    // acc[j], ask[j]: rows = coordinate groups m (coordinate 8 m + j), columns = queries.
    mq_float4 acc[8], ask[VQ ? 8 : 1];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mq_float4{0.f, 0.f, 0.f, 0.f};
    if constexpr (VQ) {
#pragma unroll
      for (int j = 0; j < 8; ++j) ask[j] = mq_float4{0.f, 0.f, 0.f, 0.f};
    }
    // Running score maximum m and value frame M start below every score, so
    // that 2^(s - m) of a masked token (s = -inf) is 0; c = 2^(m - M).
    constexpr float kNoFrame = -1e30f;
    float m = kNoFrame, l = 0.f, M = kNoFrame, c = 1.f;

    // One step's loads (buffer offsets: the step's first token in the scalar
    // offset, the lane's part in the vector offset).
    struct Step {
      uint32_t kw[KW], vr[VW == 3 ? 8 : 4], side;
      mq_float4 nuk, nuv, sz, gk, gv;
    };
    auto load_step = [&](int base, Step& st) {
      const uint32_t sk = (uint32_t)base * RBK, sv = (uint32_t)base * RBV, sn = 4u * (uint32_t)base;
      if constexpr (KW == 4) {
        const mq_u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rk, vk, sk, kMqNT);
        st.kw[0] = x.x; st.kw[1] = x.y; st.kw[2] = x.z; st.kw[3] = x.w;
      } else if constexpr (KW == 2) {
        const mq_u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rk, vk, sk, kMqNT);
        st.kw[0] = x.x; st.kw[1] = x.y;
      } else {
#pragma unroll
        for (int i = 0; i < KW; ++i) st.kw[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, vk + 4 * i, sk, kMqNT);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (VW == 4) {
          st.vr[e] = __builtin_amdgcn_raw_buffer_load_b32(rv, vv + e * RBV, sv, kMqNT);
        } else if constexpr (VW == 2) {
          st.vr[e] = __builtin_amdgcn_raw_buffer_load_b16(rv, vv + e * RBV, sv, kMqNT);
        } else if constexpr (VW == 1) {
          st.vr[e] = __builtin_amdgcn_raw_buffer_load_b8(rv, vv + e * RBV, sv, kMqNT);
        } else {
          st.vr[2 * e] = __builtin_amdgcn_raw_buffer_load_b32(rv, vv + e * RBV, sv, kMqNT);
          st.vr[2 * e + 1] = __builtin_amdgcn_raw_buffer_load_b32(rv, vv2 + e * RBV, sv, kMqNT);
        }
      }
      st.side = 0;
      if constexpr (KS) st.side = __builtin_amdgcn_raw_buffer_load_b16(rsd, vsd, 8u * (uint32_t)base, kMqNT);
      // 16-byte loads of four tokens' scalars (the range check is per dword).
      st.nuk = mq_ldf4(rnk, vn, sn);
      st.nuv = mq_ldf4(rnv, vn, sn);
      st.sz = st.gk = st.gv = mq_float4{0.f, 0.f, 0.f, 0.f};
      if constexpr (KS) st.sz = mq_ldf4(rsz, vn, sn);
      if constexpr (KQ) st.gk = mq_ldf4(rgk, vn, sn);
      if constexpr (VQ) st.gv = mq_ldf4(rgv, vn, sn);
    };
    int parity = 0;
    auto step = [&](int base, const Step& cur) __attribute__((always_inline)) {
      const int tr = base + 4 * hq;

      // ---- scores (this wave's 128 coordinates) ------------------------------------------
      mq_float4 S = {0.f, 0.f, 0.f, 0.f}, Sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        mq_half8 Ah, Al, As;
        key8<KW, KPARTS, CK, KQ>(s_lds, cur.kw, ks, kcofs, Ah, Al, As);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Qh[ks], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Ql[ks], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Qh[ks], S, 0, 0, 0);
        if constexpr (KQ) {
          Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(As, Uh[ks], Sk, 0, 0, 0);
          Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(As, Ul[ks], Sk, 0, 0, 0);
        }
      }
      if constexpr (NWU > 1) {
        // Sum the partial scores of the unit's waves, each with its share of
        // the sketch term already added (one exchange instead of two).
        if constexpr (KQ) {
#pragma unroll
          for (int i = 0; i < 4; ++i) S[i] = fmaf(cur.gk[i] * p.k_qjl, Sk[i], S[i]);
        }
        s_red[parity][wu][lane] = S;
        __syncthreads();
        S = s_red[parity][0][lane];
#pragma unroll
        for (int w = 1; w < NWU; ++w) S += s_red[parity][w][lane];
        parity ^= 1;
      }
      mq_float4 Ss = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KS) {
        // code - 7 as fp16: 0x6400 | code is 1024 + code exactly, less 1031 (exact).
        const uint32_t sd = cur.side;
        const uint32_t p01 = (sd & 0xFu) | ((sd & 0xF0u) << 12) | 0x64006400u;
        const uint32_t p23 = ((sd >> 8) & 0xFu) | ((sd & 0xF000u) << 4) | 0x64006400u;
        const mq_half2 lev = {(_Float16)1031.0f, (_Float16)1031.0f};
        const mq_half2 a01 = __builtin_bit_cast(mq_half2, p01) - lev, a23 = __builtin_bit_cast(mq_half2, p23) - lev;
        const mq_half4 A = {a01.x, a01.y, a23.x, a23.y};
        Ss = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wh, Ss, 0, 0, 0);
        Ss = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wl, Ss, 0, 0, 0);
      }
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[i];
        if constexpr (KQ && NWU == 1) v = fmaf(cur.gk[i] * p.k_qjl, Sk[i], v);
        v *= cur.nuk[i];
        if constexpr (KS) v = fmaf(cur.sz[i], Ss[i], v);
        s[i] = v * p.scale_log2;
      }
      if (base + 16 > t1) {
        // The chunk's last step: tokens past its end score -inf.
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = tr + i < t1 ? s[i] : -INFINITY;
      }
      float smax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      smax = fmaxf(smax, __shfl_xor(smax, 16, 64));
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      if (smax > m + kMqSlack) {
        l *= __builtin_amdgcn_exp2f(m - smax);
        m = smax;
        c = __builtin_amdgcn_exp2f(m - M);
      }
      // Value weights 2^(s + log2 nu_v - M) = 2^(s - m) nu_v c, at most 2^8;
      // past the end or at nu_v = 0 they are 0.
      float w[4];
      bool big = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[i] - m);
        l += e;
        w[i] = e * (cur.nuv[i] * c);
        big |= !(w[i] <= 256.f);
      }
      // Rare (the first weights, or a weight beyond 2^8 moves the frame): one
      // wave-uniform branch.
      if (__builtin_amdgcn_ballot_w64(big) != 0) {
        float lam[4], lmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lam[i] = s[i] + __builtin_amdgcn_logf(cur.nuv[i]);
          lmax = fmaxf(lmax, lam[i]);
        }
        lmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
        lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
        const bool up = lmax > M + kMqSlack;
        const float f = up ? __builtin_amdgcn_exp2f(M - lmax) : 1.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= f;
        if constexpr (VQ) {
#pragma unroll
          for (int j = 0; j < 8; ++j) ask[j] *= f;
        }
        M = up ? lmax : M;
        c = __builtin_amdgcn_exp2f(m - M);
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = __builtin_amdgcn_exp2f(lam[i] - M);
      }
      mq_half4 Wv, Wq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Wv[i] = (_Float16)w[i];
        if constexpr (VQ) Wq[i] = (_Float16)(w[i] * cur.gv[i]);
      }

      // ---- values: coordinate 8 mm + j of tokens 4 hq .. 4 hq + 3 per product ----------
      uint32_t ix[4];
      value_index<VW>(cur.vr, vsh, ix);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mq_half4 A, As;
        value_ops<VW, VPARTS, CV, VQ>(s_vtab, ix, j, vcofs, A, As);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wv, acc[j], 0, 0, 0);
        if constexpr (VQ) ask[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(As, Wq, ask[j], 0, 0, 0);
      }
    };
    // The next step's loads are in flight while a step computes (loads two
    // steps ahead, or two buffers in turn instead of the copy, measured slower).
    Step nxt;
    if (t0 < t1) load_step(t0, nxt);
    for (int base = t0; base < t1; base += 16) {
      const Step cur = nxt;
      if (base + 16 < t1) load_step(base + 16, nxt);
      step(base, cur);
    }

    // ---- partial record: [m, l, acc[d] (, ask[d])] in the 2^m frame, query g ----------
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (m == kNoFrame) m = -INFINITY;             // no token scored
    const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - m);
    if (gvalid) {
      float* out = p.part + ((size_t)qi * p.nsplit + split) * p.part_stride;
      // Result rows 4 hq + i of product j: coordinate 8 (4 hq + i) + j.
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = 128 * wu + 32 * hq + 8 * i + j;
          out[2 + c] = acc[j][i] * f;
          if constexpr (VQ) out[2 + D + c] = ask[j][i] * f;
        }
      if (hq == 0 && wu == 0) { out[0] = m; out[1] = l; }
    }
  }
}

template <int D, int KB, bool KQ, bool KS>
hipError_t launch_mq_v(const DecodeParams& p, int vbits, int vqjl, int nblocks, hipStream_t s) {
  if (vqjl) {
    hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 3, true>), dim3(nblocks), dim3(mq_threads(D, KQ, true)), 0, s,
                       p);
    return hipGetLastError();
  }
  constexpr int NT = mq_threads(D, KQ, false);
  switch (vbits) {
    case 4: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 4, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    case 3: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 3, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 2, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    case 1: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 1, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_mq_d(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl, int nblocks,
                       hipStream_t s) {
  if constexpr (D == 128) {
    if (kside) return launch_mq_v<128, 2, false, true>(p, vbits, vqjl, nblocks, s);
  }
  if (kqjl) return launch_mq_v<D, 3, true, false>(p, vbits, vqjl, nblocks, s);
  switch (kbits) {
    case 4: return launch_mq_v<D, 4, false, false>(p, vbits, vqjl, nblocks, s);
    case 3: return launch_mq_v<D, 3, false, false>(p, vbits, vqjl, nblocks, s);
    case 2: return launch_mq_v<D, 2, false, false>(p, vbits, vqjl, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace tq
