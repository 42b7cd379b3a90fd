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
//   * values: the token's centroids go to an LDS tile row by row and come
//     back transposed as the first operand of eight v_mfma_f32_16x16x16_f16
//     (16 coordinates x 16 tokens each) against the weights; sketched values
//     also send their signs through a second tile against the weights times
//     gamma_v (the sums the combine step turns into S^T acc_sk).
// Key centroids, queries and the HeadQ side weights enter the scores as fp16
// hi + lo pairs (hi x hi + hi x lo + lo x hi, about 22 bits: in fp16 alone
// the score error reached ~7e-4 at unit-variance keys); value centroids and
// weights are fp16 as in the table-driven decode; accumulation is fp32.  The partial
// record per (query, chunk) is the table-driven kernel's, merged by the
// combine step.
#include <cmath>

#include "device_common.h"

namespace tq {
namespace {

constexpr int kMqRow = 136;               // fp16 per row of a wave's centroid tile (16 B pad)
constexpr int kMqCopies = 8;              // table copies (lane % 8) against bank conflicts
constexpr float kMqSlack = 8.0f;          // log2 units

// Waves per block: at d = 128 four independent workers; above, one unit's
// d / 128 waves, each on 128 coordinates.
constexpr int mq_threads(int D) { return D == 128 ? 256 : 64 * (D / 128); }

typedef _Float16 mq_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 mq_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 mq_half2 __attribute__((ext_vector_type(2)));
typedef float mq_float4 __attribute__((ext_vector_type(4)));
typedef uint32_t mq_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t mq_u32x2 __attribute__((ext_vector_type(2)));

// Table of one tensor's centroids indexed by a packed unit: a byte of two
// 4-bit fields (half2; with a sketch the fields are 3-bit code | sign << 3
// and the sign bit is masked off), a byte of four 2-bit codes (half4) or a
// 6-bit field of two 3-bit codes (half2).  With SPLIT (keys) each entry holds
// the fp16 hi parts followed by the lo parts (c - hi).
// W is the field width in the packed words (B, or 4 for a sketched 3-bit code).
template <int W, bool SPLIT>
struct MqTab {
  static constexpr int entries = W == 3 ? 64 : 256;
  static constexpr int bytes_per = (W == 2 ? 8 : 4) * (SPLIT ? 2 : 1);
  static constexpr int bytes = entries * kMqCopies * bytes_per;
};

template <int W, bool SPLIT>
__device__ __forceinline__ void build_tab(char* tab, const float* c, int tid, int nthreads) {
  constexpr int N = W == 2 ? 4 : 2;               // centroids per entry
  for (int i = tid; i < MqTab<W, SPLIT>::entries * kMqCopies; i += nthreads) {
    const int e = i / kMqCopies;
    _Float16 h[2 * N];
#pragma unroll
    for (int q = 0; q < N; ++q) {
      // 4-bit fields: the low 3 bits are the code when a sketch sign sits in bit 3
      // (codes of a 4-bit index never exceed 15, so masking with 15 is the identity).
      const int code = W == 2 ? (e >> (2 * q)) & 3 : (W == 4 ? (e >> (4 * q)) & 15 : (e >> (3 * q)) & 7);
      const float v = c[code];
      h[q] = (_Float16)v;
      h[N + q] = (_Float16)(v - (float)h[q]);
    }
    _Float16* dst = reinterpret_cast<_Float16*>(tab + i * MqTab<W, SPLIT>::bytes_per);
#pragma unroll
    for (int q = 0; q < (SPLIT ? 2 * N : N); ++q) dst[q] = h[q];
  }
}

// A sketched tensor's 4-bit fields carry the code in bits 0..2: its table
// entries use c[field & 7].  Built like build_tab<4> over masked codes.
template <bool SPLIT>
__device__ __forceinline__ void build_tab_sketched(char* tab, const float* c, int tid, int nthreads) {
  for (int i = tid; i < 256 * kMqCopies; i += nthreads) {
    const int e = i / kMqCopies;
    const float v0 = c[e & 7], v1 = c[(e >> 4) & 7];
    const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;
    _Float16* dst = reinterpret_cast<_Float16*>(tab + i * MqTab<4, SPLIT>::bytes_per);
    dst[0] = h0;
    dst[1] = h1;
    if constexpr (SPLIT) {
      dst[2] = (_Float16)(v0 - (float)h0);
      dst[3] = (_Float16)(v1 - (float)h1);
    }
  }
}

// Eight consecutive coordinates 8 k .. 8 k + 7 of a lane's 32, decoded from
// its words (LSB-first W-bit fields): hi parts in r, lo parts in rl (SPLIT).
template <int W, bool SPLIT>
__device__ __forceinline__ void decode8(const char* tab, const uint32_t* w, int k, int copy, mq_half8& r,
                                        mq_half8& rl) {
  constexpr int BP = MqTab<W, SPLIT>::bytes_per;
  if constexpr (W == 4 || W == 3) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t f;
      if constexpr (W == 4) {
        f = (w[k] >> (8 * q)) & 255u;
      } else {
        const int bit = 24 * k + 6 * q, wi = bit >> 5, sh = bit & 31;
        f = w[wi] >> sh;
        if (sh > 26) f |= w[wi + 1] << (32 - sh);
        f &= 63u;
      }
      const char* ent = tab + (f * kMqCopies + copy) * BP;
      if constexpr (SPLIT) {
        const mq_half4 h = *reinterpret_cast<const mq_half4*>(ent);
        r[2 * q] = h.x; r[2 * q + 1] = h.y;
        rl[2 * q] = h.z; rl[2 * q + 1] = h.w;
      } else {
        const mq_half2 h = *reinterpret_cast<const mq_half2*>(ent);
        r[2 * q] = h.x; r[2 * q + 1] = h.y;
      }
    }
  } else {
    const uint32_t x = w[k >> 1] >> (16 * (k & 1));
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const char* ent = tab + (((x >> (8 * q)) & 255u) * kMqCopies + copy) * BP;
      if constexpr (SPLIT) {
        const mq_half8 h = *reinterpret_cast<const mq_half8*>(ent);
#pragma unroll
        for (int e = 0; e < 4; ++e) { r[4 * q + e] = h[e]; rl[4 * q + e] = h[4 + e]; }
      } else {
        const mq_half4 h = *reinterpret_cast<const mq_half4*>(ent);
        r[4 * q] = h.x; r[4 * q + 1] = h.y; r[4 * q + 2] = h.z; r[4 * q + 3] = h.w;
      }
    }
  }
}

// The sketch signs (bit 3 of each 4-bit field) of coordinates 8 k .. 8 k + 7
// as fp16 +-1 (+1 for a set bit).
__device__ __forceinline__ mq_half8 signs8(const uint32_t* w, int k) {
  mq_half8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = ((w[k] >> (4 * e + 3)) & 1u) ? (_Float16)1.0f : (_Float16)-1.0f;
  return r;
}

// W dwords of slice s of a vector with (D * W / 8)-byte code rows.
template <int D, int W>
__device__ __forceinline__ void load_words(const uint8_t* plane, size_t vec, int s, uint32_t* w) {
  const uint32_t* src = reinterpret_cast<const uint32_t*>(plane + vec * (size_t)(D * W / 8)) + W * s;
  if constexpr (W == 4) {
    const mq_u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const mq_u32x4*>(src));
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (W == 2) {
    const mq_u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const mq_u32x2*>(src));
    w[0] = x.x; w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; ++i) w[i] = __builtin_nontemporal_load(src + i);
  }
}

// Four per-token scalars of tokens t .. t + 3 of a head (clamped past the
// end).  (A branch that skips the clamps away from the end measured slower.)
__device__ __forceinline__ mq_float4 load_f4(const float* base, int t, int t1) {
  mq_float4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = base[min(t + i, t1 - 1)];
  return r;
}

// KB, VB: index bits; KQ, VQ: sketched (4-bit fields, KB = VB = 3); KS: HeadQ
// side code (d = 128).
template <int D, int KB, bool KQ, bool KS, int VB, bool VQ>
__global__ __launch_bounds__(mq_threads(D)) void decode_mq_kernel(DecodeParams p) {
  constexpr int NT = mq_threads(D);
  constexpr int NW = NT / 64;                      // waves per block
  constexpr int NWU = D / 128;                     // waves per unit
  constexpr int UPB = NW / NWU;                    // units per block (4 at d = 128, else 1)
  constexpr int KW = KQ ? 4 : KB, VW = VQ ? 4 : VB;  // field widths
  __shared__ __attribute__((aligned(16))) char s_ktab[MqTab<KW, true>::bytes];
  __shared__ __attribute__((aligned(16))) char s_vtab[MqTab<VW, false>::bytes];
  __shared__ __attribute__((aligned(16))) _Float16 s_tile[NW][16 * kMqRow];
  __shared__ __attribute__((aligned(16))) _Float16 s_stile[VQ ? NW : 1][VQ ? 16 * kMqRow : 8];
  // Partial scores of the waves of a unit (d > 128), double-buffered by step parity.
  __shared__ __attribute__((aligned(16))) mq_float4 s_red[NWU > 1 ? 2 : 1][NWU > 1 ? NWU : 1][NWU > 1 ? (KQ ? 128 : 64) : 1];
  if constexpr (KQ) build_tab_sketched<true>(s_ktab, p.kc, threadIdx.x, NT);
  else build_tab<KW, true>(s_ktab, p.kc, threadIdx.x, NT);
  if constexpr (VQ) build_tab_sketched<false>(s_vtab, p.vc, threadIdx.x, NT);
  else build_tab<VW, false>(s_vtab, p.vc, threadIdx.x, NT);
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wu = NWU > 1 ? wave : 0;               // wave within the unit: coordinates 128 wu ..
  const int slice = 4 * wu;                         // first 32-coordinate slice of the wave
  const int hq = lane >> 4, mm = lane & 15;        // operand / result lane (h, m)
  const int copy = lane & (kMqCopies - 1);
  _Float16* tile = s_tile[wave];
  _Float16* stile = s_stile[VQ ? wave : 0];
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
    mq_float4 acc[8], ask[VQ ? 8 : 1];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[cb] = mq_float4{0.f, 0.f, 0.f, 0.f};
    if constexpr (VQ) {
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) ask[cb] = mq_float4{0.f, 0.f, 0.f, 0.f};
    }
    float m = -INFINITY, l = 0.f;
    constexpr float kNoFrame = -1e30f;
    float M = kNoFrame;

    // One step's loads: this lane's token base + mm (code words of slice
    // slice + hq, side code) and the per-token scalars of the result rows,
    // tokens base + 4 hq + i; past the end the token index is clamped (re-reads).
    struct Step {
      uint32_t kw[KW], vw[VW], side;
      mq_float4 nuk, nuv, sz, gk, gv;
    };
    auto load_step = [&](int base, Step& st) {
      const int tk = min(base + mm, t1 - 1);
      load_words<D, KW>(p.k.codes, vbase + tk, slice + hq, st.kw);
      load_words<D, VW>(p.v.codes, vbase + tk, slice + hq, st.vw);
      st.side = 0;
      if constexpr (KS)
        st.side = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p.k.side + (vbase + tk) * 8 + 2 * hq));
      const int tr = base + 4 * hq;
      st.nuk = load_f4(p.k.norms + vbase, tr, t1);
      st.nuv = load_f4(p.v.norms + vbase, tr, t1);
      st.sz = mq_float4{0.f, 0.f, 0.f, 0.f};
      st.gk = st.sz;
      st.gv = st.sz;
      if constexpr (KS) st.sz = load_f4(p.k.side_scale + vbase, tr, t1);
      if constexpr (KQ) st.gk = load_f4(p.k.gamma + vbase, tr, t1);
      if constexpr (VQ) st.gv = load_f4(p.v.gamma + vbase, tr, t1);
    };
    Step nxt;
    if (t0 < t1) load_step(t0, nxt);
    int parity = 0;
    for (int base = t0; base < t1; base += 16) {
      // The next step's loads are in flight while this step computes.
      const Step cur = nxt;
      if (base + 16 < t1) load_step(base + 16, nxt);
      const int tr = base + 4 * hq;

      // ---- scores (this wave's 128 coordinates) ------------------------------------------
      mq_float4 S = {0.f, 0.f, 0.f, 0.f}, Sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        mq_half8 Ah, Al;
        decode8<KW, true>(s_ktab, cur.kw, ks, copy, Ah, Al);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Qh[ks], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, Ql[ks], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, Qh[ks], S, 0, 0, 0);
        if constexpr (KQ) {
          const mq_half8 As = signs8(cur.kw, ks);
          Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(As, Uh[ks], Sk, 0, 0, 0);
          Sk = __builtin_amdgcn_mfma_f32_16x16x32_f16(As, Ul[ks], Sk, 0, 0, 0);
        }
      }
      if constexpr (NWU > 1) {
        // Sum the partial scores of the unit's waves.
        s_red[parity][wu][lane] = S;
        if constexpr (KQ) s_red[parity][wu][64 + lane] = Sk;
        __syncthreads();
        S = s_red[parity][0][lane];
        if constexpr (KQ) Sk = s_red[parity][0][64 + lane];
#pragma unroll
        for (int w = 1; w < NWU; ++w) {
          S += s_red[parity][w][lane];
          if constexpr (KQ) Sk += s_red[parity][w][64 + lane];
        }
        parity ^= 1;
      }
      mq_float4 Ss = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KS) {
        mq_half4 A;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] = (_Float16)((float)((cur.side >> (4 * e)) & 15u) - 7.0f);
        Ss = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wh, Ss, 0, 0, 0);
        Ss = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wl, Ss, 0, 0, 0);
      }
      float s[4];
      float smax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = S[i];
        if constexpr (KQ) v = fmaf(cur.gk[i] * p.k_qjl, Sk[i], v);
        v *= cur.nuk[i];
        if constexpr (KS) v = fmaf(cur.sz[i], Ss[i], v);
        v *= p.scale_log2;
        s[i] = (tr + i < t1) ? v : -INFINITY;
        smax = fmaxf(smax, s[i]);
      }
      smax = fmaxf(smax, __shfl_xor(smax, 16, 64));
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      if (smax > m + kMqSlack) {
        l *= __builtin_amdgcn_exp2f(m - smax);      // 0 while m = -inf
        m = smax;
      }
      // Weights in the 2^M frame of the value sums (nu_v = 0 or past the end: 0).
      float lam[4], lmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        l += s[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[i] - m);
        lam[i] = s[i] + __builtin_amdgcn_logf(cur.nuv[i]);
        lmax = fmaxf(lmax, lam[i]);
      }
      lmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
      lmax = fmaxf(lmax, __shfl_xor(lmax, 32, 64));
      // Rare (the frame moves only when a weight would exceed 2^8): one
      // wave-uniform branch.
      if (__builtin_amdgcn_ballot_w64(lmax > M + kMqSlack) != 0) {
        const bool up = lmax > M + kMqSlack;
        const float f = up ? __builtin_amdgcn_exp2f(M - lmax) : 1.0f;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) acc[cb] *= f;
        if constexpr (VQ) {
#pragma unroll
          for (int cb = 0; cb < 8; ++cb) ask[cb] *= f;
        }
        M = up ? lmax : M;
      }
      mq_half4 Wv, Wq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float wgt = __builtin_amdgcn_exp2f(lam[i] - M);
        Wv[i] = (_Float16)wgt;
        if constexpr (VQ) Wq[i] = (_Float16)(wgt * cur.gv[i]);
      }

      // ---- values: centroids (and signs) to the tiles, rows = tokens --------------------
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        mq_half8 vh, unused;
        decode8<VW, false>(s_vtab, cur.vw, k, copy, vh, unused);
        *reinterpret_cast<mq_half8*>(tile + mm * kMqRow + 32 * hq + 8 * k) = vh;
        if constexpr (VQ) *reinterpret_cast<mq_half8*>(stile + mm * kMqRow + 32 * hq + 8 * k) = signs8(cur.vw, k);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        // First operand: coordinate 16 cb + mm of tokens 4 hq .. 4 hq + 3.
        mq_half4 A;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] = tile[(4 * hq + e) * kMqRow + 16 * cb + mm];
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x16f16(A, Wv, acc[cb], 0, 0, 0);
        if constexpr (VQ) {
          mq_half4 As;
#pragma unroll
          for (int e = 0; e < 4; ++e) As[e] = stile[(4 * hq + e) * kMqRow + 16 * cb + mm];
          ask[cb] = __builtin_amdgcn_mfma_f32_16x16x16f16(As, Wq, ask[cb], 0, 0, 0);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- partial record: [m, l, acc[d] (, ask[d])] in the 2^m frame, query g ----------
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float f = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - m);
    if (gvalid) {
      float* out = p.part + ((size_t)qi * p.nsplit + split) * p.part_stride;
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 128 * wu + 16 * cb + 4 * hq + i;
          out[2 + c] = acc[cb][i] * f;
          if constexpr (VQ) out[2 + D + c] = ask[cb][i] * f;
        }
      if (hq == 0 && wu == 0) { out[0] = m; out[1] = l; }
    }
  }
}

template <int D, int KB, bool KQ, bool KS>
hipError_t launch_mq_v(const DecodeParams& p, int vbits, int vqjl, int nblocks, hipStream_t s) {
  constexpr int NT = mq_threads(D);
  if (vqjl) {
    hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 3, true>), dim3(nblocks), dim3(NT), 0, s, p);
    return hipGetLastError();
  }
  switch (vbits) {
    case 4: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 4, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    case 3: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 3, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_mq_kernel<D, KB, KQ, KS, 2, false>), dim3(nblocks), dim3(NT), 0, s, p); break;
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

bool mq_supported(int d, int G, int kbits, int kqjl, int kside, int side_rank, int side_bits, int vbits, int vqjl) {
  if ((d != 128 && d != 256 && d != 512 && d != 1024) || G < 2) return false;
  if (vqjl ? vbits != 3 : (vbits < 2 || vbits > 4)) return false;
  if (kside) return d == 128 && !kqjl && kbits == 2 && side_rank == 16 && side_bits == 4;
  return kqjl ? kbits == 3 : (kbits >= 2 && kbits <= 4);
}

int mq_waves_per_unit(int d) { return d == 128 ? 1 : d / 128; }
int mq_units_per_block(int d) { return d == 128 ? 4 : 1; }

hipError_t launch_decode_mq(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl, int nblocks,
                            hipStream_t s) {
  switch (p.d) {
    case 128: return launch_mq_d<128>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 256: return launch_mq_d<256>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 512: return launch_mq_d<512>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
    case 1024: return launch_mq_d<1024>(p, kbits, kqjl, kside, vbits, vqjl, nblocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
