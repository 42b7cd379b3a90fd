// Device helpers shared by the libtq kernels (gfx950, wave64).
//
// Lane layout used everywhere: a d-dimensional vector is owned by L = d/32
// consecutive lanes; lane j of the group holds coordinates [32 j, 32 j + 32).
// A packed b-bit code block therefore gives lane j exactly b whole dwords
// (bits [32 b j, 32 b (j+1))), and a 1-bit sign block gives it one dword.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "internal.h"

namespace tq {

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m, 64);
}

// Sum over the L lanes of one vector group (L a power of two <= 32).
__device__ __forceinline__ float group_sum(float v, int L) {
  for (int m = 1; m < L; m <<= 1) v += shfl_xor_f(v, m);
  return v;
}
__device__ __forceinline__ float group_max(float v, int L) {
  for (int m = 1; m < L; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

// Streaming (non-temporal) loads of read-once data.
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ld_nt(const float* p) { return __builtin_nontemporal_load(p); }

// Index i (0..31) of a b-bit LSB-first code run held in `w` (b dwords).
template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int i) {
  const int bit = BITS * i, wi = bit >> 5, sh = bit & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// PROD stores index i as one (b+1)-bit field, code | sign << b, where the
// sign is bit i of the QJL sketch; a 32-index group is b+1 dwords.
template <int BITS, bool SKETCH>
struct Field {
  static constexpr int kBits = BITS + (SKETCH ? 1 : 0);   // field width
  static constexpr uint32_t kCodeMask = (1u << BITS) - 1u;
};

// The 32 sign bits of a group of (BITS+1)-bit fields held in `w`.
template <int BITS>
__device__ __forceinline__ uint32_t sign_word(const uint32_t* w) {
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) s |= (code_at<BITS + 1>(w, i) >> BITS) << i;
  return s;
}

// Load 32 consecutive input elements (fp16 or fp32) as float.
template <typename T>
__device__ __forceinline__ void load32(const T* src, float* v);

template <>
__device__ __forceinline__ void load32<float>(const float* src, float* v) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4* p = reinterpret_cast<const f4*>(src);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    f4 t = __builtin_nontemporal_load(p + k);
    v[4 * k] = t.x; v[4 * k + 1] = t.y; v[4 * k + 2] = t.z; v[4 * k + 3] = t.w;
  }
}

template <>
__device__ __forceinline__ void load32<_Float16>(const _Float16* src, float* v) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8* p = reinterpret_cast<const h8*>(src);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h8 t = __builtin_nontemporal_load(p + k);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * k + e] = (float)t[e];
  }
}

// In-place unnormalised Walsh-Hadamard transform (Sylvester order) of a
// vector spread over L lanes, 32 values per lane: five in-lane butterfly
// stages, then one cross-lane stage per lane bit.
__device__ __forceinline__ void wht_group(float* v, int j, int L) {
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if (!(e & s)) {
        float a = v[e], c = v[e | s];
        v[e] = a + c;
        v[e | s] = a - c;
      }
    }
  }
  // Cross-lane stage: the upper lane of a pair keeps o - v, the lower v + o,
  // both as one fma with a +-1 factor (o - v and v + o exactly).
  for (int m = 1; m < L; m <<= 1) {
    const float sg = (j & m) ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float o = shfl_xor_f(v[e], m);
      v[e] = fmaf(v[e], sg, o);
    }
  }
}

// Multiply the lane's 32 coordinates by the sign vector D (bit set = -1).
__device__ __forceinline__ void apply_signs(float* v, uint32_t word) {
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = ((word >> e) & 1u) ? -v[e] : v[e];
}

}  // namespace tq
