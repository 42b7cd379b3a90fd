// C ABI of libtq (declared in include/tq.h): argument validation on the host
// (before any HIP call), the per-device cache of the seeded sketch, and the
// dispatch of the write-side, read-side and metric kernels.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "internal.h"

namespace tq {
int relerr_blocks(int T, int L, int BH);
}

using namespace tq;

namespace {

thread_local std::string g_err;

tq_status fail(tq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

tq_status ok() { return TQ_OK; }

// Modes coded in the seeded rotated domain (the SPECTRAL basis is the
// caller's, and PLAIN is not rotated).
bool rotated(int mode) { return mode == TQ_MODE_MSE || mode == TQ_MODE_PROD || mode == TQ_MODE_HEADQ; }

bool pow2_in(int d, int lo, int hi) { return d >= lo && d <= hi && (d & (d - 1)) == 0; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int elem_size(int dtype) { return dtype == TQ_F16 ? 2 : 4; }

tq_status check_d(int d) {
  if (!pow2_in(d, 32, kMaxD)) return fail(TQ_EUNSUPPORTED, "head dim d=%d must be a power of two in [32, 1024]", d);
  return TQ_OK;
}

tq_status modes_of(int scheme, int n_bits, int which, int* mode, int* bits) {
  if (which != TQ_KEYS && which != TQ_VALUES) return fail(TQ_EINVAL, "which=%d is neither TQ_KEYS nor TQ_VALUES", which);
  if (n_bits < 1 || n_bits > kMaxIndexBits) return fail(TQ_EINVAL, "n_bits=%d outside [1, %d]", n_bits, kMaxIndexBits);
  int km, vm;
  switch (scheme) {
    case TQ_SCHEME_KV: km = TQ_MODE_PLAIN; vm = TQ_MODE_PLAIN; break;
    case TQ_SCHEME_TQ_KV: km = TQ_MODE_MSE; vm = TQ_MODE_MSE; break;
    case TQ_SCHEME_KQV: km = TQ_MODE_MSE; vm = TQ_MODE_PROD; break;
    case TQ_SCHEME_QKQV: km = TQ_MODE_PROD; vm = TQ_MODE_PROD; break;
    case TQ_SCHEME_TQ_QKV: km = TQ_MODE_PROD; vm = TQ_MODE_MSE; break;
    case TQ_SCHEME_HEADQ: km = TQ_MODE_HEADQ; vm = TQ_MODE_MSE; break;
    case TQ_SCHEME_SQU_KV: km = TQ_MODE_SPECTRAL; vm = TQ_MODE_SPECTRAL; break;
    default: return fail(TQ_EINVAL, "unknown scheme %d", scheme);
  }
  const int m = which == TQ_KEYS ? km : vm;
  int b = n_bits;
  if (m == TQ_MODE_PROD) {
    if (n_bits < 2) return fail(TQ_EINVAL, "a QJL tensor needs n_bits >= 2 (n-1 index bits + 1 sketch bit)");
    b = n_bits - 1;
  }
  if (m == TQ_MODE_HEADQ) b = 2;
  *mode = m;
  *bits = b;
  return TQ_OK;
}

// (mode, index bits) of one tensor: the scheme preset, or the caller's
// per-tensor override (then scheme and n_bits are not used).
tq_status resolve_mode(int scheme, int n_bits, int which, const tq_mode_override* ovr, int* mode, int* bits) {
  if (!ovr) return modes_of(scheme, n_bits, which, mode, bits);
  if (which != TQ_KEYS && which != TQ_VALUES) return fail(TQ_EINVAL, "which=%d is neither TQ_KEYS nor TQ_VALUES", which);
  const int m = ovr->mode, b = ovr->bits;
  switch (m) {
    case TQ_MODE_PLAIN:
    case TQ_MODE_MSE:
    case TQ_MODE_SPECTRAL:
      if (b < 1 || b > kMaxIndexBits) return fail(TQ_EINVAL, "override: index bits %d outside [1, %d]", b, kMaxIndexBits);
      break;
    case TQ_MODE_PROD:
      if (b < 1 || b > kMaxIndexBits - 1)
        return fail(TQ_EINVAL, "override: a QJL tensor takes 1..%d index bits (got %d)", kMaxIndexBits - 1, b);
      break;
    case TQ_MODE_HEADQ:
      if (which != TQ_KEYS) return fail(TQ_EINVAL, "override: HeadQ is a key-side mode");
      if (b != 2) return fail(TQ_EUNSUPPORTED, "override: the HeadQ base takes 2 index bits (got %d)", b);
      break;
    default: return fail(TQ_EINVAL, "override: unknown mode %d", m);
  }
  *mode = m;
  *bits = b;
  return TQ_OK;
}

tq_status layout_of(int d, int mode, int bits, int side_rank, int side_bits, tq_layout* out) {
  if (tq_status s = check_d(d)) return s;
  if (mode < TQ_MODE_PLAIN || mode > TQ_MODE_SPECTRAL) return fail(TQ_EINVAL, "unknown mode %d", mode);
  if (bits < 1 || bits > kMaxIndexBits) return fail(TQ_EINVAL, "index bits %d outside [1, %d]", bits, kMaxIndexBits);
  if (mode == TQ_MODE_SPECTRAL && d > spectral_max_d())
    return fail(TQ_EUNSUPPORTED, "SPECTRAL supports d <= %d (got %d): the head's basis is held on chip", spectral_max_d(), d);
  // PROD: one (bits+1)-bit field per coordinate, code | QJL sign << bits.
  out->code_bytes = d * (bits + (mode == TQ_MODE_PROD ? 1 : 0)) / 8;
  out->qjl_bytes = 0;
  out->has_gamma = mode == TQ_MODE_PROD;
  out->side_bytes = 0;
  out->has_side_scale = 0;
  if (mode == TQ_MODE_HEADQ) {
    if (side_rank < 8 || side_rank > 32 || side_rank % 8) return fail(TQ_EUNSUPPORTED, "HeadQ rank %d: must be 8, 16, 24 or 32", side_rank);
    if (side_bits < 2 || side_bits > 8) return fail(TQ_EINVAL, "HeadQ side bits %d outside [2, 8]", side_bits);
    if (d * side_rank > 16384) return fail(TQ_EUNSUPPORTED, "HeadQ d*rank=%d exceeds 16384", d * side_rank);
    out->side_bytes = side_rank * side_bits / 8;
    out->has_side_scale = 1;
  }
  return TQ_OK;
}

tq_status check_tensor(const tq_tensor_desc* x, const char* name) {
  if (!x) return fail(TQ_EINVAL, "%s descriptor is NULL", name);
  if (!x->data) return fail(TQ_EINVAL, "%s data pointer is NULL", name);
  if (x->dtype != TQ_F16 && x->dtype != TQ_F32) return fail(TQ_EINVAL, "%s dtype %d is neither F16 nor F32", name, x->dtype);
  if (x->B < 1 || x->H < 1 || x->T < 1) return fail(TQ_EINVAL, "%s has an empty dimension (B=%d H=%d T=%d)", name, x->B, x->H, x->T);
  if (tq_status s = check_d(x->d)) return s;
  const int es = elem_size(x->dtype);
  if (!aligned(x->data, 16)) return fail(TQ_EINVAL, "%s data is not 16-byte aligned", name);
  if (x->stride_t < x->d && x->T > 1) return fail(TQ_EINVAL, "%s stride_t < d", name);
  if ((x->stride_t * es) % 16 || (x->stride_h * es) % 16 || (x->stride_b * es) % 16)
    return fail(TQ_EINVAL, "%s strides must be multiples of 16 bytes", name);
  return TQ_OK;
}

void fill_signbits(uint64_t seed, int d, uint32_t* words) {
  std::vector<float> s(d);
  sign_vector(seed, d, s.data());
  for (int i = 0; i < kMaxD / 32; ++i) words[i] = 0;
  for (int i = 0; i < d; ++i)
    if (s[i] < 0) words[i >> 5] |= 1u << (i & 31);
}

// ---- per-device cache of the Gaussian sketch S ------------------------------------
std::mutex g_cache_mu;
std::map<std::tuple<int, uint64_t, int>, float*> g_sketch;
// S in fp16 (S is exactly representable in fp16), per (device, seed, d), in
// the fragment order of the matrix-core sketch kernel at d >= 256.
std::map<std::tuple<int, uint64_t, int>, _Float16*> g_sketch16;

// The device copy of S for (current device, seed, d), made on first use.
tq_status sketch_on_device(uint64_t seed, int d, const float** out, bool may_alloc = true) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_EDEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_cache_mu);
  auto key = std::make_tuple(dev, seed, d);
  auto it = g_sketch.find(key);
  if (it != g_sketch.end()) { *out = it->second; return TQ_OK; }
  if (!may_alloc)
    return fail(TQ_EINVAL, "the QJL sketch for seed %llu, d=%d is not resident on device %d: quantize or decode "
                "once with it through an allocating call first", (unsigned long long)seed, d, dev);
  std::vector<float> S((size_t)d * d);
  gaussian_sketch(seed, d, S.data());
  float* p = nullptr;
  if (hipMalloc(&p, S.size() * sizeof(float)) != hipSuccess) return fail(TQ_ENOMEM, "hipMalloc of the sketch failed");
  if (hipMemcpy(p, S.data(), S.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(TQ_EDEVICE, "hipMemcpy of the sketch failed");
  }
  g_sketch[key] = p;
  *out = p;
  return TQ_OK;
}

tq_status sketch16_on_device(uint64_t seed, int d, const _Float16** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TQ_EDEVICE, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_cache_mu);
  auto key = std::make_tuple(dev, seed, d);
  auto it = g_sketch16.find(key);
  if (it != g_sketch16.end()) { *out = it->second; return TQ_OK; }
  std::vector<float> S((size_t)d * d);
  gaussian_sketch(seed, d, S.data());
  std::vector<_Float16> h(S.size());
  for (int row = 0; row < d; ++row)
    for (int col = 0; col < d; ++col)  // exact: S is defined in fp16
      h[sketch_fragment_index(d, row, col)] = (_Float16)S[(size_t)row * d + col];
  _Float16* p = nullptr;
  if (hipMalloc(&p, h.size() * sizeof(_Float16)) != hipSuccess) return fail(TQ_ENOMEM, "hipMalloc of the sketch failed");
  if (hipMemcpy(p, h.data(), h.size() * sizeof(_Float16), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(p);
    return fail(TQ_EDEVICE, "hipMemcpy of the sketch failed");
  }
  g_sketch16[key] = p;
  *out = p;
  return TQ_OK;
}

tq_status hip_status(hipError_t e, const char* what);

// Grid for the index search: a cell width of gap / 1.25 (gap = the smallest
// distance between boundaries) keeps the window of 1 + 2 kGridMargin cells
// around any cell narrower than the gap, so it holds at most one boundary.
// Coarse cells keep the table small: the coordinates of a token fall into a
// few dozen adjacent entries, which spread over distinct LDS banks.
bool quant_grid(int d, int bits, QuantGrid* g) {
  std::vector<double> c, t;
  if (!codebook(d, bits, &c, &t)) return false;
  double gap = 2.0;
  for (size_t k = 1; k < t.size(); ++k) gap = std::min(gap, t[k] - t[k - 1]);
  g->scale = (float)(1.25 / gap);
  g->center = (int)std::ceil(g->scale) + 2;
  g->cells = 2 * g->center + 1;
  return g->cells <= quant_mfma_lut_max();
}

// Compute units of the current device (cached per device).
hipError_t cu_count(int* out) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) { *out = it->second; return hipSuccess; }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cache[dev] = n;
  *out = n;
  return hipSuccess;
}

tq_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TQ_EDEVICE, "%s: %s", what, hipGetErrorString(e));
  return TQ_OK;
}

// The SPECTRAL state: basis 16-byte aligned (read with 16-byte loads),
// mean and spreads 4-byte aligned.
bool spectral_ok(const float* basis, const float* mean, const float* scale) {
  return basis && mean && scale && aligned(basis, 16) && aligned(mean, 4) && aligned(scale, 4);
}

tq_status check_packed(const tq_packed* p, const char* name) {
  if (!p) return fail(TQ_EINVAL, "%s packed descriptor is NULL", name);
  if (p->B < 1 || p->H < 1 || p->T < 1 || p->T_cap < p->T)
    return fail(TQ_EINVAL, "%s header is empty or T > T_cap (B=%d H=%d T=%d T_cap=%d)", name, p->B, p->H, p->T, p->T_cap);
  tq_layout lay;
  if (tq_status s = layout_of(p->d, p->mode, p->bits, p->side_rank, p->side_bits, &lay)) return s;
  if (!p->codes || !p->norms) return fail(TQ_EINVAL, "%s codes/norms plane is NULL", name);
  if (!aligned(p->codes, 16) || !aligned(p->norms, 16)) return fail(TQ_EINVAL, "%s planes must be 16-byte aligned", name);
  if (p->mode == TQ_MODE_PROD && (!p->gamma || !aligned(p->gamma, 16)))
    return fail(TQ_EINVAL, "%s QJL gamma plane missing or misaligned", name);
  if (p->mode == TQ_MODE_HEADQ && (!p->side || !p->side_scale || !p->basis || !aligned(p->side, 16) || !aligned(p->side_scale, 16)))
    return fail(TQ_EINVAL, "%s HeadQ planes or basis missing or misaligned", name);
  if (p->mode == TQ_MODE_SPECTRAL && !spectral_ok(p->basis, p->mean, p->scale))
    return fail(TQ_EINVAL, "%s SPECTRAL basis (16-byte aligned), mean or scale (4-byte aligned) missing or misaligned", name);
  return TQ_OK;
}

// Kernel instantiations that exist (see launch_decode_split).
bool key_supported(int kbits, bool kq, bool ksd) {
  if (ksd) return !kq && kbits == 2;
  if (kq) return kbits >= 1 && kbits <= 3;
  return kbits >= 1 && kbits <= 4;
}
bool decode_supported(int kbits, bool kq, bool ksd, int vbits, bool vq) {
  if (!key_supported(kbits, kq, ksd)) return false;
  return vq ? (vbits >= 1 && vbits <= 3) : (vbits >= 1 && vbits <= 4);
}

struct DecodePlan {
  int nsplit, chunk, part_stride, units, G;
  int nparts;  // partials per query: nsplit, times the waves per block at d > 128 (table-driven)
  bool lut;
  bool mq;     // grouped-query matrix-core decode (units: KV head x block of 16 queries x chunk)
  size_t off_qrot, off_qsk, off_qw, off_part, off_qraw, off_qoff, off_comb, bytes;
  bool comb;   // split combine (large d, sketched values): three [nq][d] float arrays at off_comb
};

tq_status plan_decode(const tq_packed* k, const tq_packed* v, int Hq, bool with_qraw, DecodePlan* pl) {
  if (tq_status s = check_packed(k, "K")) return s;
  if (v) {
    if (tq_status s = check_packed(v, "V")) return s;
    // The kernels address both tensors' planes with one head stride, T_cap.
    if (k->B != v->B || k->H != v->H || k->T != v->T || k->T_cap != v->T_cap || k->d != v->d)
      return fail(TQ_EMISMATCH, "K and V packed headers disagree (B, H, T, T_cap or d)");
    if (v->mode == TQ_MODE_HEADQ) return fail(TQ_EINVAL, "HeadQ is a key-side mode");
  }
  if (Hq < 1 || Hq % k->H) return fail(TQ_EMISMATCH, "Hq=%d is not a multiple of the KV heads H=%d", Hq, k->H);
  const int d = k->d, L = d / 32, vpw = 64 / L;
  const int G = Hq / k->H;
  const int nq = k->B * Hq;
  // The table-driven kernel addresses a head's planes with 24-bit token
  // indices and 32-bit byte offsets (at most d/2 code bytes per token),
  // hence the T_cap bounds.
  // Several query heads per KV head: the grouped-query kernel reads each
  // token once per block of 16 of them, through buffer descriptors of at most
  // 2^32 bytes per head plane (at most d/2 code bytes per token).
  const bool mq = v && (long)k->T_cap * (d / 2) < (1L << 32) &&
                  mq_supported(d, G, k->bits, k->mode == TQ_MODE_PROD, k->mode == TQ_MODE_HEADQ, k->side_rank,
                               k->side_bits, v->bits, v->mode == TQ_MODE_PROD);
  const bool lut = !mq && v && k->T_cap <= (1 << 24) && (long)k->T_cap * (d / 2) < (1L << 32) &&
                   lut_supported(d, k->bits, k->mode == TQ_MODE_PROD, k->mode == TQ_MODE_HEADQ, k->side_rank,
                                 k->side_bits, v->bits, v->mode == TQ_MODE_PROD);
  // The table-driven kernel walks 8-12 waves x (64/L) tokens per block step
  // and runs one persistent block per CU; the generic one 4 waves per block;
  // the grouped-query one steps 16 tokens per wave.
  const int step = mq ? 16 : (lut ? 8 : 4) * vpw;
  const long groups = mq ? (long)k->B * k->H * ((G + 15) / 16) : (long)k->B * k->H * G;
  // Work units (query, context chunk): the generic kernel wants ~2048 blocks
  // in flight; the persistent table-driven kernel wants few, long units
  // (about two per CU) because each unit ends with a merge of its token slots;
  // the grouped-query kernel about as many units as fit on the device at once
  // (d/128 waves each; at d = 128 exactly one round): every unit writes 16
  // partials of 2 + 2d floats, which the combine step reads back.
  // (Without a device, e.g. a size query on a host without one: 256 CUs.)
  int cus = 256;
  if (mq && (cu_count(&cus) != hipSuccess || cus < 1)) cus = 256;
  const long target = mq ? mq_target_units(d, k->mode == TQ_MODE_PROD, v->mode == TQ_MODE_PROD, cus)
                         : (lut ? 512 : 2048);
  int nsplit = (int)std::max<long>(1, (target + groups - 1) / groups);
  int chunk = (k->T + nsplit - 1) / nsplit;
  chunk = std::max(step, (chunk + step - 1) / step * step);
  nsplit = (k->T + chunk - 1) / chunk;
  // The combine step merges at most 256 partials per query; the table-driven
  // kernel at d > 128 writes one per wave.
  const bool vq = v && v->mode == TQ_MODE_PROD;
  const int per_split = (lut && d > 128) ? lut_waves(vq) : 1;
  const int max_split = 256 / per_split;
  if (nsplit > max_split) {
    chunk = (k->T + max_split - 1) / max_split;
    chunk = (chunk + step - 1) / step * step;
    nsplit = (k->T + chunk - 1) / chunk;
  }
  pl->nsplit = nsplit;
  pl->nparts = nsplit * per_split;
  pl->chunk = chunk;
  pl->lut = lut;
  pl->mq = mq;
  pl->G = G;
  pl->part_stride = (int)round_up(2 + d + (vq ? d : 0), 4);
  const long R = (long)k->B * k->H * nsplit;
  pl->units = (int)(round_up(R, 8) * G);
  size_t off = 0;
  pl->off_qrot = off; off = round_up(off + (size_t)nq * d * 4, 256);
  pl->off_qsk = off;  off = round_up(off + (k->mode == TQ_MODE_PROD ? (size_t)nq * d * 4 : 0), 256);
  pl->off_qw = off;   off = round_up(off + (k->mode == TQ_MODE_HEADQ ? (size_t)nq * k->side_rank * 4 : 0), 256);
  pl->off_qraw = off; off = round_up(off + (with_qraw ? (size_t)nq * d * 4 : 0), 256);
  pl->off_qoff = off; off = round_up(off + (k->mode == TQ_MODE_SPECTRAL ? (size_t)nq * 4 : 0), 256);
  pl->off_part = off; off = round_up(off + (v ? (size_t)nq * pl->nparts * pl->part_stride * 4 : 0), 256);
  pl->comb = vq && combine_splits(d, true, v->mode == TQ_MODE_SPECTRAL);
  pl->off_comb = off; off = round_up(off + (pl->comb ? 3 * (size_t)nq * d * 4 : 0), 256);
  pl->bytes = off;
  return TQ_OK;
}

tq_status check_query(const tq_tensor_desc* q, const tq_packed* k) {
  if (tq_status s = check_tensor(q, "q")) return s;
  if (q->T != 1) return fail(TQ_EINVAL, "queries must have T = 1 (got %d)", q->T);
  if (q->B != k->B || q->d != k->d) return fail(TQ_EMISMATCH, "query B/d (%d, %d) differ from the cache (%d, %d)", q->B, q->d, k->B, k->d);
  if (q->H % k->H) return fail(TQ_EMISMATCH, "query heads %d not a multiple of KV heads %d", q->H, k->H);
  return TQ_OK;
}

void fill_qprep(const tq_tensor_desc* q, const tq_packed* k, const float* S, char* ws, const DecodePlan& pl,
                bool qraw, QPrepParams* qp) {
  std::memset(qp, 0, sizeof(*qp));
  qp->q = q->data; qp->dtype = q->dtype; qp->B = q->B; qp->Hq = q->H; qp->d = q->d; qp->Hkv = k->H;
  qp->sb = q->stride_b; qp->sh = q->stride_h;
  qp->rotate = rotated(k->mode);
  qp->kqjl = k->mode == TQ_MODE_PROD;
  qp->kside = k->mode == TQ_MODE_HEADQ;
  qp->rank = k->side_rank;
  if (k->mode == TQ_MODE_SPECTRAL) {
    qp->kspectral = 1;
    qp->sbasis = k->basis; qp->smean = k->mean; qp->sscale = k->scale;
    qp->qoff = reinterpret_cast<float*>(ws + pl.off_qoff);
  }
  fill_signbits(k->seed, k->d, qp->signbits);
  qp->inv_sqrt_d = 1.0f / std::sqrt((float)k->d);
  qp->S = S; qp->basis = k->basis;
  qp->qrot = reinterpret_cast<float*>(ws + pl.off_qrot);
  qp->qsk = reinterpret_cast<float*>(ws + pl.off_qsk);
  qp->qw = reinterpret_cast<float*>(ws + pl.off_qw);
  qp->qraw = qraw ? reinterpret_cast<float*>(ws + pl.off_qraw) : nullptr;
}

// Centroids and boundaries of a tensor's scalar code: the Beta sphere
// marginal of the rotated modes, the standard normal for SPECTRAL.
tq_status fill_codebook(int mode, int d, int bits, float* c16, float* b16) {
  std::vector<double> c, t;
  const bool okc = mode == TQ_MODE_SPECTRAL ? gaussian_codebook(bits, &c, &t) : codebook(d, bits, &c, &t);
  if (!okc) return fail(TQ_EINVAL, "codebook(mode=%d, d=%d, bits=%d) failed", mode, d, bits);
  for (int i = 0; i < 16; ++i) {
    c16[i] = i < (int)c.size() ? (float)c[i] : 0.f;
    b16[i] = i < (int)t.size() ? (float)t[i] : INFINITY;
  }
  return TQ_OK;
}

tq_status quantize_core(const tq_tensor_desc* x, int mode, int bits, uint64_t seed, const tq_headq* hq,
                        const tq_packed* out, int T_cap, const int32_t* pos, void* stream);
tq_status decode_core(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v, const int32_t* lens,
                      float* out, float* lse, void* ws, size_t ws_bytes, void* stream, bool may_alloc = true);

void fill_scoring(const tq_tensor_desc* q, const tq_packed* k, const DecodePlan& pl, char* ws, DecodeParams* dp) {
  std::memset(dp, 0, sizeof(*dp));
  dp->B = k->B; dp->Hkv = k->H; dp->G = pl.G; dp->Hq = q->H; dp->T = k->T; dp->T_cap = k->T_cap;
  dp->d = k->d; dp->L = k->d / 32; dp->nsplit = pl.nsplit; dp->chunk = pl.chunk;
  dp->part_stride = pl.part_stride; dp->units = pl.units;
  dp->k = {k->codes, k->norms, k->qjl, k->gamma, k->side, k->side_scale};
  dp->rank = k->side_rank; dp->side_bits = k->side_bits;
  float bnd[16];
  fill_codebook(k->mode, k->d, k->bits, dp->kc, bnd);
  dp->k_qjl = (float)(std::sqrt(M_PI / 2.0) / k->d);
  dp->scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)k->d));
  dp->qrot = reinterpret_cast<const float*>(ws + pl.off_qrot);
  dp->qsk = reinterpret_cast<const float*>(ws + pl.off_qsk);
  dp->qw = reinterpret_cast<const float*>(ws + pl.off_qw);
  dp->qoff = k->mode == TQ_MODE_SPECTRAL ? reinterpret_cast<const float*>(ws + pl.off_qoff) : nullptr;
  dp->part = reinterpret_cast<float*>(ws + pl.off_part);
}

// Workspace of tq_metrics: the scoring plan (query prep), the score rows,
// the per-query measures; with packed values also the per-vector value
// errors, a decode workspace and the two output sets of the output site; the
// per-block sums of the reconstruction-error pass.
struct MetricsLayout {
  bool site = false;
  DecodePlan pl{}, dpl{};
  size_t nq = 0, off_s = 0, off_perq = 0, off_verr = 0, off_dec = 0, off_o = 0, off_blk = 0, bytes = 0;
};

tq_status metrics_layout(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v, MetricsLayout* m) {
  size_t off = 0;
  if (q) {
    if (!k) return fail(TQ_EINVAL, "KL/top-5 need the packed keys");
    if (tq_status s = plan_decode(k, nullptr, q->H, true, &m->pl)) return s;
    m->nq = (size_t)k->B * q->H;
    off = m->pl.bytes;
    m->off_s = off;    off = round_up(off + 2 * m->nq * k->T * 4, 256);
    m->off_perq = off; off = round_up(off + m->nq * kPerQuery * 8, 256);
    if (v) {
      if (tq_status s = plan_decode(k, v, q->H, false, &m->dpl)) return s;
      m->site = true;
      m->off_verr = off; off = round_up(off + (size_t)v->B * v->H * v->T_cap * 4, 256);
      m->off_dec = off;  off = round_up(off + m->dpl.bytes, 256);
      m->off_o = off;    off = round_up(off + 2 * m->nq * k->d * 4, 256);
    }
  }
  size_t nb = 0;
  for (const tq_packed* p : {k, v}) {
    if (!p) continue;
    if (tq_status s = check_packed(p, "packed")) return s;
    nb = std::max(nb, (size_t)relerr_blocks(p->T, p->d / 32, p->B * p->H));
  }
  m->off_blk = off;
  off = round_up(off + nb * 5 * 8, 256);
  m->bytes = off;
  return TQ_OK;
}

double snr_db(double signal2, double noise2) {
  if (!(signal2 > 0)) return NAN;
  return noise2 > 0 ? 10.0 * std::log10(signal2 / noise2) : INFINITY;
}

// Spearman rank correlation: Pearson correlation of the ranks, ties at the
// mean of their ranks; NaN when a sample is constant.
double spearman(const std::vector<double>& a, const std::vector<double>& b) {
  auto ranks = [](const std::vector<double>& x) {
    const size_t n = x.size();
    std::vector<size_t> order(n);
    for (size_t i = 0; i < n; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t i, size_t j) { return x[i] < x[j]; });
    std::vector<double> r(n);
    for (size_t i = 0; i < n;) {
      size_t j = i;
      while (j + 1 < n && x[order[j + 1]] == x[order[i]]) ++j;
      for (size_t t = i; t <= j; ++t) r[order[t]] = 0.5 * (double)(i + j) + 1.0;
      i = j + 1;
    }
    return r;
  };
  if (a.size() != b.size() || a.size() < 2) return NAN;
  for (double x : a) if (!std::isfinite(x)) return NAN;
  for (double x : b) if (!std::isfinite(x)) return NAN;
  std::vector<double> ra = ranks(a), rb = ranks(b);
  const double n = (double)a.size(), mean = 0.5 * (n + 1.0);
  double sab = 0, saa = 0, sbb = 0;
  for (size_t i = 0; i < a.size(); ++i) {
    const double x = ra[i] - mean, y = rb[i] - mean;
    sab += x * y; saa += x * x; sbb += y * y;
  }
  return (saa > 0 && sbb > 0) ? sab / std::sqrt(saa * sbb) : NAN;
}

// Reconstruction error of a packed tensor against its raw input: pooled
// relMSE, mean 1 - cos, SNR (dB), mean angle, and the squared error summed
// per (b, h); per_vec (optional) receives ||x_hat - x||^2 of every vector.
struct RelErrOut {
  double rel = NAN, dir = NAN, snr = NAN, phi = NAN;
  std::vector<double> head_e2;
};

tq_status relerr(const tq_tensor_desc* x, const tq_packed* pk, double* blk, float* per_vec, hipStream_t st,
                 RelErrOut* o) {
  if (tq_status s = check_tensor(x, "reference")) return s;
  if (x->B != pk->B || x->H != pk->H || x->T != pk->T || x->d != pk->d)
    return fail(TQ_EMISMATCH, "reference tensor shape differs from the packed tensor");
  RelErrParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = x->data; p.dtype = x->dtype; p.B = x->B; p.H = x->H; p.T = x->T; p.T_cap = pk->T_cap; p.d = x->d; p.L = x->d / 32;
  p.sb = x->stride_b; p.sh = x->stride_h; p.st = x->stride_t;
  p.mode = pk->mode; p.bits = pk->bits; p.rotate = rotated(pk->mode);
  p.kqjl = pk->mode == TQ_MODE_PROD; p.kside = pk->mode == TQ_MODE_HEADQ;
  p.rank = pk->side_rank; p.side_bits = pk->side_bits;
  float bnd[16];
  if (tq_status s = fill_codebook(pk->mode, pk->d, pk->bits, p.centroids, bnd)) return s;
  fill_signbits(pk->seed, pk->d, p.signbits);
  p.inv_sqrt_d = 1.0f / std::sqrt((float)pk->d);
  p.qjl_c = (float)(std::sqrt(M_PI / 2.0) / pk->d);
  if (p.kqjl) { if (tq_status s = sketch_on_device(pk->seed, pk->d, &p.S)) return s; }
  p.basis = pk->basis;
  p.planes = {pk->codes, pk->norms, pk->qjl, pk->gamma, pk->side, pk->side_scale};
  p.block_sums = blk;
  p.per_vec = per_vec;
  const int BH = pk->B * pk->H;
  const int nb = relerr_blocks(pk->T, pk->d / 32, BH);
  if (pk->mode == TQ_MODE_SPECTRAL) {
    // Same block count and (b, h)-major block order as relerr_kernel.
    p.smean = pk->mean; p.sscale = pk->scale;
    if (tq_status s = hip_status(launch_relerr_spectral(p, st), "relerr launch")) return s;
  } else {
    if (tq_status s = hip_status(launch_relerr(p, nb, st), "relerr launch")) return s;
  }
  std::vector<double> host((size_t)nb * 5);
  if (tq_status s = hip_status(hipMemcpyAsync(host.data(), blk, host.size() * 8, hipMemcpyDeviceToHost, st), "copy")) return s;
  if (tq_status s = hip_status(hipStreamSynchronize(st), "sync")) return s;
  double e2 = 0, r2 = 0, ds = 0, cnt = 0, as = 0;
  o->head_e2.assign(BH, 0.0);
  const int gx = nb / BH;  // blocks per (b, h): block index = bh * gx + x
  for (int b = 0; b < nb; ++b) {
    e2 += host[b * 5]; r2 += host[b * 5 + 1]; ds += host[b * 5 + 2]; cnt += host[b * 5 + 3]; as += host[b * 5 + 4];
    o->head_e2[b / gx] += host[b * 5];
  }
  o->rel = r2 > 0 ? e2 / r2 : NAN;
  o->dir = cnt > 0 ? ds / cnt : NAN;
  o->phi = cnt > 0 ? as / cnt : NAN;
  o->snr = snr_db(r2, e2);
  return TQ_OK;
}

}  // namespace

extern "C" {

int32_t tq_abi_version(void) { return TQ_ABI_VERSION; }

const char* tq_status_str(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_EINVAL: return "TQ_EINVAL";
    case TQ_EUNSUPPORTED: return "TQ_EUNSUPPORTED";
    case TQ_EMISMATCH: return "TQ_EMISMATCH";
    case TQ_ENOMEM: return "TQ_ENOMEM";
    case TQ_EDEVICE: return "TQ_EDEVICE";
  }
  return "TQ_UNKNOWN";
}

const char* tq_last_error(void) { return g_err.c_str(); }

tq_status tq_codebook_build(int32_t d, int32_t bits, double* centroids, double* boundaries) {
  if (tq_status s = check_d(d)) return s;
  if (bits < 1 || bits > 8) return fail(TQ_EINVAL, "bits=%d outside [1, 8]", bits);
  if (!centroids || !boundaries) return fail(TQ_EINVAL, "output pointer is NULL");
  std::vector<double> c, t;
  if (!codebook(d, bits, &c, &t)) return fail(TQ_EINVAL, "codebook failed");
  std::copy(c.begin(), c.end(), centroids);
  std::copy(t.begin(), t.end(), boundaries);
  return ok();
}

tq_status tq_scheme_modes(int32_t scheme, int32_t n_bits, int32_t which, int32_t* mode, int32_t* bits) {
  if (!mode || !bits) return fail(TQ_EINVAL, "output pointer is NULL");
  int m, b;
  if (tq_status s = modes_of(scheme, n_bits, which, &m, &b)) return s;
  *mode = m;
  *bits = b;
  return ok();
}

tq_status tq_packed_layout(int32_t d, int32_t mode, int32_t bits, int32_t side_rank, int32_t side_bits, tq_layout* out) {
  if (!out) return fail(TQ_EINVAL, "output pointer is NULL");
  return layout_of(d, mode, bits, side_rank, side_bits, out);
}

tq_status tq_rotation_state(uint64_t seed, int32_t d, float* signs, float* S) {
  if (tq_status s = check_d(d)) return s;
  if (signs) sign_vector(seed, d, signs);
  if (S) gaussian_sketch(seed, d, S);
  return ok();
}

tq_status tq_quantize(const tq_tensor_desc* x, int32_t which, int32_t scheme, int32_t n_bits, uint64_t seed,
                      const tq_mode_override* ovr, const tq_headq* hq, tq_packed* out, void* stream) {
  if (tq_status s = check_tensor(x, "x")) return s;
  int mode, bits;
  if (tq_status s = resolve_mode(scheme, n_bits, which, ovr, &mode, &bits)) return s;
  if (!out) return fail(TQ_EINVAL, "output packed descriptor is NULL");
  if ((mode == TQ_MODE_HEADQ) != (hq != nullptr))
    return fail(TQ_EINVAL, mode == TQ_MODE_HEADQ ? "HeadQ keys need a tq_headq" : "tq_headq given for a non-HeadQ tensor");
  if (mode == TQ_MODE_SPECTRAL && !spectral_ok(out->basis, out->mean, out->scale))
    return fail(TQ_EINVAL, "SPECTRAL needs out->basis (16-byte aligned), out->mean and out->scale (4-byte aligned) on the device");
  tq_layout lay;
  if (tq_status s = layout_of(x->d, mode, bits, hq ? hq->rank : 0, hq ? hq->side_bits : 0, &lay)) return s;
  if (hq && (!hq->basis || !aligned(hq->basis, 4))) return fail(TQ_EINVAL, "HeadQ basis is NULL or misaligned");
  const int T_cap = out->T_cap == 0 ? x->T : out->T_cap;
  if (T_cap < x->T) return fail(TQ_EINVAL, "T_cap=%d < T=%d", T_cap, x->T);
  if (!out->codes || !out->norms || !aligned(out->codes, 16) || !aligned(out->norms, 16))
    return fail(TQ_EINVAL, "codes/norms planes missing or not 16-byte aligned");
  if (mode == TQ_MODE_PROD && (!out->gamma || !aligned(out->gamma, 16)))
    return fail(TQ_EINVAL, "QJL gamma plane missing or not 16-byte aligned");
  if (mode == TQ_MODE_HEADQ && (!out->side || !out->side_scale || !aligned(out->side, 16) || !aligned(out->side_scale, 16)))
    return fail(TQ_EINVAL, "HeadQ side planes missing or not 16-byte aligned");
  if ((long)x->B * x->H * (long)T_cap > (1L << 40)) return fail(TQ_EINVAL, "cache too large");
  if (tq_status s = quantize_core(x, mode, bits, seed, hq, out, T_cap, nullptr, stream)) return s;
  out->B = x->B; out->H = x->H; out->T = x->T; out->T_cap = T_cap; out->d = x->d;
  out->mode = mode; out->bits = bits; out->seed = seed;
  out->side_rank = hq ? hq->rank : 0; out->side_bits = hq ? hq->side_bits : 0;
  if (mode != TQ_MODE_SPECTRAL) {
    out->basis = hq ? hq->basis : nullptr;
    out->mean = nullptr;
    out->scale = nullptr;
  }
  return ok();
}

tq_status tq_quantize_append(const tq_tensor_desc* x, int32_t which, int32_t scheme, int32_t n_bits, uint64_t seed,
                             const tq_mode_override* ovr, const tq_headq* hq, const int32_t* pos, tq_packed* cache,
                             void* stream) {
  if (tq_status s = check_tensor(x, "x")) return s;
  int mode, bits;
  if (tq_status s = resolve_mode(scheme, n_bits, which, ovr, &mode, &bits)) return s;
  if (tq_status s = check_packed(cache, "cache")) return s;
  if (!pos || !aligned(pos, 4)) return fail(TQ_EINVAL, "positions NULL or not 4-byte aligned");
  if (cache->B != x->B || cache->H != x->H || cache->d != x->d)
    return fail(TQ_EMISMATCH, "new tokens (B=%d H=%d d=%d) do not match the cache (B=%d H=%d d=%d)", x->B, x->H, x->d,
                cache->B, cache->H, cache->d);
  if (cache->mode != mode || cache->bits != bits || cache->seed != seed)
    return fail(TQ_EMISMATCH, "scheme/override/seed give mode %d with %d bits, seed %llu; the cache holds mode %d, %d bits, seed %llu",
                mode, bits, (unsigned long long)seed, cache->mode, cache->bits, (unsigned long long)cache->seed);
  if ((mode == TQ_MODE_HEADQ) != (hq != nullptr))
    return fail(TQ_EINVAL, mode == TQ_MODE_HEADQ ? "HeadQ keys need a tq_headq" : "tq_headq given for a non-HeadQ tensor");
  if (hq && (hq->basis != cache->basis || hq->rank != cache->side_rank || hq->side_bits != cache->side_bits))
    return fail(TQ_EMISMATCH, "HeadQ basis, rank or side bits differ from the cache's");
  if (x->T > cache->T_cap) return fail(TQ_EINVAL, "%d new tokens exceed T_cap=%d", x->T, cache->T_cap);
  tq_packed planes = *cache;
  return quantize_core(x, mode, bits, seed, hq, &planes, cache->T_cap, pos, stream);
}

}  // extern "C"

namespace {

tq_status quantize_core(const tq_tensor_desc* x, int mode, int bits, uint64_t seed, const tq_headq* hq,
                        const tq_packed* out, int T_cap, const int32_t* pos, void* stream) {
  QuantParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = x->data; p.dtype = x->dtype; p.B = x->B; p.H = x->H; p.T = x->T; p.T_cap = T_cap; p.d = x->d; p.L = x->d / 32;
  p.sb = x->stride_b; p.sh = x->stride_h; p.st = x->stride_t;
  p.mode = mode; p.bits = bits; p.rotate = rotated(mode);
  if (tq_status s = fill_codebook(mode, x->d, bits, p.centroids, p.bounds)) return s;
  fill_signbits(seed, x->d, p.signbits);
  p.inv_sqrt_d = 1.0f / std::sqrt((float)x->d);
  if (mode == TQ_MODE_PROD) {
    if (tq_status s = sketch_on_device(seed, x->d, &p.S)) return s;
  }
  if (hq) { p.basis = hq->basis; p.rank = hq->rank; p.side_bits = hq->side_bits; }
  p.codes = out->codes; p.norms = out->norms; p.qjl = out->qjl; p.gamma = out->gamma;
  p.side = out->side; p.side_scale = out->side_scale;
  p.pos = pos;
  hipStream_t st = (hipStream_t)stream;
  // HeadQ: Pi U_h once per head, [H][rank][d], in stream-ordered scratch,
  // followed by its fp16 hi and lo parts (times 2^10) for the matrix cores.
  void* rb = nullptr;
  if (mode == TQ_MODE_HEADQ) {
    const size_t n = (size_t)x->H * x->d * hq->rank;
    if (hipMallocAsync(&rb, n * (sizeof(float) + 2 * sizeof(_Float16)), st) != hipSuccess)
      return fail(TQ_ENOMEM, "rotated-basis scratch allocation failed");
    _Float16* rb16 = reinterpret_cast<_Float16*>(reinterpret_cast<float*>(rb) + n);
    if (tq_status s = hip_status(launch_rotate_basis(p, reinterpret_cast<float*>(rb), rb16, st),
                                 "basis rotation launch")) {
      (void)hipFreeAsync(rb, st);
      return s;
    }
    p.rbasis = reinterpret_cast<const float*>(rb);
    p.rbasis16 = rb16;
  }
  tq_status status = TQ_OK;
  QuantGrid grid;
  if (mode == TQ_MODE_SPECTRAL) {
    // The caller's per-head basis, mean and spreads; decisions in double
    // against the N(0, 1) boundaries.
    std::vector<double> c, t;
    if (!gaussian_codebook(bits, &c, &t)) return fail(TQ_EINVAL, "Gaussian codebook (%d bits) failed", bits);
    for (int k = 0; k < 16; ++k) p.gbounds[k] = k < (int)t.size() ? t[k] : INFINITY;
    p.basis = out->basis; p.smean = out->mean; p.sscale = out->scale;
    // Lookup grid over u = z / s_i: cells a third of the smallest boundary gap
    // wide, covering the boundaries plus two cells.
    double gap = 2.0, tmax = 0.0;
    for (size_t k = 0; k < t.size(); ++k) {
      tmax = std::max(tmax, std::fabs(t[k]));
      if (k) gap = std::min(gap, t[k] - t[k - 1]);
    }
    QuantGrid g;
    g.scale = (float)(3.2 / gap);
    g.center = (int)std::ceil((tmax + 2.0 / g.scale) * g.scale) + 2;
    g.cells = 2 * g.center + 1;
    status = hip_status(launch_quantize_spectral(p, &g, st), "quantize launch");
  } else if (quant_mfma_supported(p) && quant_grid(x->d, bits, &grid)) {
    int cus = 0;
    status = hip_status(cu_count(&cus), "device query");
    if (status == TQ_OK) {
      const long tiles = (long)x->B * x->H * ((x->T + 15) / 16);  // 16-token tiles within a head
      const int nblocks = (int)std::max<long>(1, std::min<long>((tiles + 3) / 4, (long)cus * 8));
      status = hip_status(launch_quantize_mfma(p, grid, nblocks, st), "quantize launch");
    }
  } else if (mode == TQ_MODE_PROD && quant_grid(x->d, bits, &grid) && quant_sketch_supported(p, grid)) {
    // PROD at d >= 256: the sketch projection is a real GEMM over the token
    // batch, on the matrix cores.
    if (tq_status s = sketch16_on_device(seed, x->d, &p.S16)) status = s;
    else status = hip_status(launch_quantize_sketch(p, grid, st), "quantize launch");
  } else {
    p.bh0 = 0; p.nbh = x->B * x->H; p.t0 = 0; p.tn = x->T;
    const bool have_grid = quant_grid(x->d, bits, &grid);
    status = hip_status(launch_quantize(p, have_grid ? &grid : nullptr, st), "quantize launch");
  }
  if (rb) (void)hipFreeAsync(rb, st);
  if (status != TQ_OK) return status;
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_decode_workspace_size(const tq_packed* k, const tq_packed* v, int32_t Hq, size_t* bytes) {
  if (!bytes) return fail(TQ_EINVAL, "output pointer is NULL");
  if (!v) return fail(TQ_EINVAL, "V packed descriptor is NULL");
  DecodePlan pl;
  if (tq_status s = plan_decode(k, v, Hq, false, &pl)) return s;
  *bytes = pl.bytes;
  return ok();
}

tq_status tq_decode_attention(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v, float* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
  return decode_core(q, k, v, nullptr, out, lse, ws, ws_bytes, stream);
}

tq_status tq_decode_attention_lens(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                                   const int32_t* lens, float* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!lens || !aligned(lens, 4)) return fail(TQ_EINVAL, "lengths NULL or not 4-byte aligned");
  return decode_core(q, k, v, lens, out, lse, ws, ws_bytes, stream);
}

tq_status tq_decode_attention_static(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v,
                                     const int32_t* lens, float* out, float* lse, void* stream) {
  if (lens && !aligned(lens, 4)) return fail(TQ_EINVAL, "lengths not 4-byte aligned");
  if (!k || !v) return fail(TQ_EINVAL, "packed descriptor is NULL");
  if (!q) return fail(TQ_EINVAL, "query descriptor is NULL");
  DecodePlan pl;
  if (tq_status s = plan_decode(k, v, q->H, false, &pl)) return s;
  if (pl.bytes > static_scratch_bytes())
    return fail(TQ_ENOMEM, "this decode needs a %zu-byte workspace; the static one holds %zu bytes "
                "(use tq_decode_attention with a workspace of its own)", pl.bytes, static_scratch_bytes());
  if (tq_status s = check_query(q, k)) return s;
  void* ws = nullptr;
  if (tq_status s = hip_status(static_scratch(&ws), "static workspace address")) return s;
  return decode_core(q, k, v, lens, out, lse, ws, static_scratch_bytes(), stream, false);
}

}  // extern "C"

namespace {

tq_status decode_core(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v, const int32_t* lens,
                      float* out, float* lse, void* ws, size_t ws_bytes, void* stream, bool may_alloc) {
  if (!k || !v) return fail(TQ_EINVAL, "packed descriptor is NULL");
  if (!q) return fail(TQ_EINVAL, "query descriptor is NULL");
  DecodePlan pl;
  if (tq_status s = plan_decode(k, v, q->H, false, &pl)) return s;
  if (tq_status s = check_query(q, k)) return s;
  if (!out || !aligned(out, 4) || (lse && !aligned(lse, 4))) return fail(TQ_EINVAL, "out/lse NULL or misaligned");
  if (!ws || !aligned(ws, 256)) return fail(TQ_EINVAL, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < pl.bytes) return fail(TQ_ENOMEM, "workspace %zu bytes < required %zu", ws_bytes, pl.bytes);
  const bool kq = k->mode == TQ_MODE_PROD, ksd = k->mode == TQ_MODE_HEADQ, vq = v->mode == TQ_MODE_PROD;
  if (!decode_supported(k->bits, kq, ksd, v->bits, vq))
    return fail(TQ_EUNSUPPORTED, "no decode kernel for K (mode %d, %d bits) with V (mode %d, %d bits)", k->mode, k->bits, v->mode, v->bits);
  const float* Sk = nullptr;
  const float* Sv = nullptr;
  if (kq) { if (tq_status s = sketch_on_device(k->seed, k->d, &Sk, may_alloc)) return s; }
  if (vq) { if (tq_status s = sketch_on_device(v->seed, v->d, &Sv, may_alloc)) return s; }
  char* w = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;

  DecodeParams dp;
  fill_scoring(q, k, pl, w, &dp);
  dp.v = {v->codes, v->norms, v->qjl, v->gamma, v->side, v->side_scale};
  dp.lens = lens;
  float vb[16];
  if (tq_status s = fill_codebook(v->mode, v->d, v->bits, dp.vc, vb)) return s;
  dp.v_qjl = (float)(std::sqrt(M_PI / 2.0) / v->d);

  QPrepParams qp;
  fill_qprep(q, k, Sk, w, pl, false, &qp);
  CombineParams cp;
  std::memset(&cp, 0, sizeof(cp));
  cp.nq = q->B * q->H; cp.d = k->d; cp.nsplit = pl.nparts; cp.part_stride = pl.part_stride;
  cp.vqjl = vq; cp.vrotate = rotated(v->mode); cp.v_qjl = dp.v_qjl;
  fill_signbits(v->seed, v->d, cp.signbits);
  cp.inv_sqrt_d = 1.0f / std::sqrt((float)k->d);
  cp.S = Sv; cp.part = dp.part; cp.out = out; cp.lse = lse;
  cp.Hq = q->H; cp.G = pl.G;
  if (v->mode == TQ_MODE_SPECTRAL) {
    cp.vspectral = 1;
    cp.vbasis = v->basis; cp.vmean = v->mean; cp.vscale = v->scale;
  }
  cp.qoff = dp.qoff;
  if (pl.comb) {
    float* cw = reinterpret_cast<float*>(w + pl.off_comb);
    const size_t n = (size_t)cp.nq * k->d;
    cp.ow = cw; cp.kw = cw + n; cp.add = cw + 2 * n;
  }

  bool supported = true;
  if (tq_status s = hip_status(launch_qprep(qp, st), "query prep launch")) return s;
  if (pl.mq) {
    int cus = 0;
    if (tq_status s = hip_status(cu_count(&cus), "device query")) return s;
    const long units = (long)k->B * k->H * ((pl.G + 15) / 16) * pl.nsplit;
    const int upb = mq_units_per_block(k->d, kq, vq);
    const long cap = (long)cus * (8 / mq_waves_per_unit(k->d) > 0 ? 8 / mq_waves_per_unit(k->d) : 1) * (k->d == 128 ? 1 : 2);
    const int nblocks = (int)std::max<long>(1, std::min<long>((units + upb - 1) / upb, cap));
    if (tq_status s = hip_status(launch_decode_mq(dp, k->bits, kq, ksd, v->bits, vq, nblocks, st), "decode launch")) return s;
  } else if (pl.lut) {
    int cus = 0;
    if (tq_status s = hip_status(cu_count(&cus), "device query")) return s;
    const int nblocks = std::min(pl.units, std::max(1, cus));
    if (tq_status s = hip_status(launch_decode_lut(dp, k->bits, kq, ksd, v->bits, vq, nblocks, st), "decode launch")) return s;
  } else {
    if (tq_status s = hip_status(launch_decode_split(dp, k->bits, kq, ksd, v->bits, vq, st, &supported), "decode launch")) return s;
  }
  if (!supported) return fail(TQ_EUNSUPPORTED, "K/V mode combination has no decode kernel");
  if (tq_status s = hip_status(launch_combine(cp, st), "combine launch")) return s;
  return ok();
}

}  // namespace

extern "C" {

tq_status tq_metrics_workspace_size(const tq_tensor_desc* q, const tq_packed* k, const tq_packed* v, size_t* bytes) {
  if (!bytes) return fail(TQ_EINVAL, "output pointer is NULL");
  MetricsLayout m;
  if (tq_status s = metrics_layout(q, k, v, &m)) return s;
  *bytes = m.bytes;
  return ok();
}

tq_status tq_metrics(const tq_tensor_desc* q, const tq_tensor_desc* k_ref, const tq_tensor_desc* v_ref,
                     const tq_packed* k, const tq_packed* v, tq_metrics_out* out, void* ws, size_t ws_bytes,
                     void* stream) {
  if (!out) return fail(TQ_EINVAL, "output pointer is NULL");
  MetricsLayout m;
  if (tq_status s = metrics_layout(q, k, v, &m)) return s;
  if (!ws || !aligned(ws, 256)) return fail(TQ_EINVAL, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < m.bytes) return fail(TQ_ENOMEM, "workspace %zu bytes < required %zu", ws_bytes, m.bytes);
  if (q && !k_ref) return fail(TQ_EINVAL, "KL/top-5 need the raw keys");
  if ((k_ref && !k) || (v_ref && !v)) return fail(TQ_EINVAL, "a reference tensor was given without its packed tensor");
  if (q) {
    if (tq_status s = check_query(q, k)) return s;
    if (tq_status s = check_tensor(k_ref, "k_ref")) return s;
    if (k_ref->B != k->B || k_ref->H != k->H || k_ref->T != k->T || k_ref->d != k->d)
      return fail(TQ_EMISMATCH, "k_ref shape differs from the packed keys");
  }
  if (v_ref) { if (tq_status s = check_tensor(v_ref, "v_ref")) return s; }
  const double nan = NAN;
  out->kl_mean = out->kl_max = out->top5_recall = nan;
  out->relmse_k = out->relmse_v = out->dir_err_k = out->dir_err_v = nan;
  out->fisher_mean = out->fisher_max = out->spearman_fisher_kl = out->spearman_keymse_kl = nan;
  out->snr_k_db = out->snr_v_db = out->snr_out_db = nan;
  out->phi_k = out->phi_v = out->phi_out = nan;
  out->a2_value_mean = nan;
  out->n_queries = 0;
  char* w = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  double* blk = reinterpret_cast<double*>(w + m.off_blk);
  // Output site and A^2 measure: queries, both raw tensors and the packed values.
  const bool site = q && m.site && v_ref;
  float* verr = site ? reinterpret_cast<float*>(w + m.off_verr) : nullptr;

  // 1. Values first: their per-vector errors feed the A^2 measure.
  RelErrOut ev, ek;
  if (v_ref && v) { if (tq_status s = relerr(v_ref, v, blk, verr, st, &ev)) return s; }

  // 2. Score rows and the per-query measures.
  double* perq = nullptr;
  float* o_hat = nullptr;
  float* o_ref = nullptr;
  const size_t nq = m.nq;
  if (q) {
    const DecodePlan& pl = m.pl;
    if (!key_supported(k->bits, k->mode == TQ_MODE_PROD, k->mode == TQ_MODE_HEADQ))
      return fail(TQ_EUNSUPPORTED, "no scoring kernel for key mode %d with %d bits", k->mode, k->bits);
    const float* Sk = nullptr;
    if (k->mode == TQ_MODE_PROD) { if (tq_status s = sketch_on_device(k->seed, k->d, &Sk)) return s; }
    float* s_ref = reinterpret_cast<float*>(w + m.off_s);
    float* s_hat = s_ref + nq * k->T;
    perq = reinterpret_cast<double*>(w + m.off_perq);
    QPrepParams qp;
    fill_qprep(q, k, Sk, w, pl, true, &qp);
    MetricScoreParams mp;
    std::memset(&mp, 0, sizeof(mp));
    fill_scoring(q, k, pl, w, &mp.dp);
    mp.kref = k_ref->data; mp.kdtype = k_ref->dtype;
    mp.ksb = k_ref->stride_b; mp.ksh = k_ref->stride_h; mp.kst = k_ref->stride_t;
    mp.qraw = reinterpret_cast<const float*>(w + pl.off_qraw);
    mp.s_ref = s_ref; mp.s_hat = s_hat;
    MetricReduceParams rp;
    std::memset(&rp, 0, sizeof(rp));
    rp.nq = (int)nq; rp.T = k->T; rp.s_ref = s_ref; rp.s_hat = s_hat; rp.per_query = perq;
    rp.verr = verr; rp.Hq = q->H; rp.G = pl.G; rp.Hkv = k->H; rp.T_cap = v ? v->T_cap : 0;
    bool supported = true;
    if (tq_status s = hip_status(launch_qprep(qp, st), "query prep launch")) return s;
    if (tq_status s = hip_status(launch_metric_scores(mp, k->bits, k->mode == TQ_MODE_PROD, k->mode == TQ_MODE_HEADQ, st, &supported), "score launch")) return s;
    if (!supported) return fail(TQ_EUNSUPPORTED, "key mode has no scoring kernel");
    if (tq_status s = hip_status(launch_metric_reduce(rp, st), "reduce launch")) return s;

    // 3. Output site: exact attention over the raw values against the decode.
    if (site) {
      if (v_ref->B != v->B || v_ref->H != v->H || v_ref->T != v->T || v_ref->d != v->d)
        return fail(TQ_EMISMATCH, "v_ref shape differs from the packed values");
      o_hat = reinterpret_cast<float*>(w + m.off_o);
      o_ref = o_hat + nq * k->d;
      if (tq_status s = decode_core(q, k, v, nullptr, o_hat, nullptr, w + m.off_dec, m.dpl.bytes, stream)) return s;
      AttnRefParams ap;
      std::memset(&ap, 0, sizeof(ap));
      ap.nq = (int)nq; ap.T = k->T; ap.d = k->d; ap.Hq = q->H; ap.G = pl.G; ap.Hkv = k->H;
      ap.s_ref = s_ref; ap.per_query = perq;
      ap.v = v_ref->data; ap.vdtype = v_ref->dtype;
      ap.vsb = v_ref->stride_b; ap.vsh = v_ref->stride_h; ap.vst = v_ref->stride_t;
      ap.o_ref = o_ref;
      if (tq_status s = hip_status(launch_attn_ref(ap, st), "reference attention launch")) return s;
    }
  }

  // 4. Keys.
  if (k_ref && k) { if (tq_status s = relerr(k_ref, k, blk, nullptr, st, &ek)) return s; }

  // 5. Host side: per-query statistics, rank correlations and the output site.
  out->relmse_k = ek.rel; out->dir_err_k = ek.dir; out->snr_k_db = ek.snr; out->phi_k = ek.phi;
  out->relmse_v = ev.rel; out->dir_err_v = ev.dir; out->snr_v_db = ev.snr; out->phi_v = ev.phi;
  if (q) {
    std::vector<double> host(nq * kPerQuery);
    if (tq_status s = hip_status(hipMemcpyAsync(host.data(), perq, host.size() * 8, hipMemcpyDeviceToHost, st), "copy")) return s;
    std::vector<float> oh, orf;
    if (site) {
      oh.resize(nq * k->d);
      orf.resize(nq * k->d);
      if (tq_status s = hip_status(hipMemcpyAsync(oh.data(), o_hat, oh.size() * 4, hipMemcpyDeviceToHost, st), "copy")) return s;
      if (tq_status s = hip_status(hipMemcpyAsync(orf.data(), o_ref, orf.size() * 4, hipMemcpyDeviceToHost, st), "copy")) return s;
    }
    if (tq_status s = hip_status(hipStreamSynchronize(st), "sync")) return s;
    std::vector<double> kl(nq), fisher(nq), kmse(nq);
    double klsum = 0, klmax = -INFINITY, rec = 0, fsum = 0, fmax = -INFINITY, a2sum = 0;
    for (size_t i = 0; i < nq; ++i) {
      const double* r = &host[i * kPerQuery];
      kl[i] = r[0]; fisher[i] = r[2];
      klsum += r[0]; klmax = std::max(klmax, r[0]); rec += r[1];
      fsum += r[2]; fmax = std::max(fmax, r[2]); a2sum += r[3];
      const int b = (int)(i / q->H), kvh = (int)(i % q->H) / m.pl.G;
      kmse[i] = ek.head_e2.empty() ? nan : ek.head_e2[(size_t)b * k->H + kvh] / k->T;
    }
    out->kl_mean = klsum / nq; out->kl_max = klmax; out->top5_recall = rec / nq;
    out->fisher_mean = fsum / nq; out->fisher_max = fmax;
    out->spearman_fisher_kl = spearman(fisher, kl);
    out->spearman_keymse_kl = ek.head_e2.empty() ? nan : spearman(kmse, kl);
    if (site) {
      out->a2_value_mean = a2sum / nq;
      double s2 = 0, e2 = 0, asum = 0, cnt = 0;
      const int d = k->d;
      for (size_t i = 0; i < nq; ++i) {
        double r2 = 0, h2 = 0, dot = 0, de = 0;
        for (int c = 0; c < d; ++c) {
          const double a = orf[i * d + c], h = oh[i * d + c];
          r2 += a * a; h2 += h * h; dot += a * h; de += (a - h) * (a - h);
        }
        s2 += r2; e2 += de;
        if (r2 > 0 && h2 > 0) {
          asum += std::acos(std::min(1.0, std::max(-1.0, dot / std::sqrt(r2 * h2))));
          cnt += 1;
        }
      }
      out->snr_out_db = snr_db(s2, e2);
      out->phi_out = cnt > 0 ? asum / cnt : nan;
    }
    out->n_queries = (int64_t)nq;
  }
  if (tq_status s = hip_status(hipStreamSynchronize(st), "sync")) return s;
  return ok();
}

tq_status tq_spectral_fit(const float* calib, int32_t N, int32_t d, float* basis, float* mean, float* scale) {
  if (!calib || !basis || !mean || !scale) return fail(TQ_EINVAL, "NULL pointer");
  if (tq_status s = check_d(d)) return s;
  if (d > spectral_max_d()) return fail(TQ_EUNSUPPORTED, "SPECTRAL supports d <= %d (got %d)", spectral_max_d(), d);
  if (N < 2) return fail(TQ_EINVAL, "N=%d: at least two calibration vectors", N);
  std::vector<float> lam(d);
  if (!pca_basis(calib, N, d, d, basis, lam.data(), mean)) return fail(TQ_EINVAL, "eigendecomposition failed");
  double total = 0.0;
  for (int i = 0; i < d; ++i) total += lam[i];
  for (int i = 0; i < d; ++i) scale[i] = total > 0 ? (float)std::sqrt((double)lam[i] / total) : 0.f;
  return ok();
}

tq_status tq_headq_fit(const float* calib, int32_t N, int32_t d, int32_t rank, float* U) {
  if (!calib || !U) return fail(TQ_EINVAL, "NULL pointer");
  if (tq_status s = check_d(d)) return s;
  if (N < 2 || rank < 1 || rank > d) return fail(TQ_EINVAL, "N=%d rank=%d invalid", N, rank);
  if (!pca_basis(calib, N, d, rank, U)) return fail(TQ_EINVAL, "PCA failed");
  return ok();
}

// ---- A^2-weighted value policy --------------------------------------------------
namespace {

tq_status check_a2(const tq_tensor_desc* q, const tq_tensor_desc* k, int* P) {
  if (tq_status s = check_tensor(q, "q_probe")) return s;
  if (tq_status s = check_tensor(k, "k_ref")) return s;
  if (q->B != k->B || q->d != k->d) return fail(TQ_EMISMATCH, "probe B/d (%d, %d) differ from the keys (%d, %d)", q->B, q->d, k->B, k->d);
  if (q->H % k->H) return fail(TQ_EMISMATCH, "probe heads %d not a multiple of KV heads %d", q->H, k->H);
  *P = (q->H / k->H) * q->T;
  if ((long)*P * q->d > 16384) return fail(TQ_EUNSUPPORTED, "%d probes per KV head at d=%d exceed 16384 / d", *P, q->d);
  return TQ_OK;
}

size_t a2_bytes(const tq_tensor_desc* q, const tq_tensor_desc* k) {
  return a2_workspace_bytes(q->B * q->H * q->T, k->T);
}

// Workspace of the policy: gains [BH][T], selections [BH][3], totals [BH].
struct PolicyLayout { size_t off_gain, off_sel, off_total, bytes; };
PolicyLayout policy_layout(const tq_tensor_desc* v) {
  PolicyLayout l;
  const size_t BH = (size_t)v->B * v->H;
  size_t off = 0;
  l.off_gain = off;  off = round_up(off + BH * v->T * 4, 256);
  l.off_sel = off;   off = round_up(off + BH * 3 * sizeof(PolicySel), 256);
  l.off_total = off; off = round_up(off + BH * 8, 256);
  l.bytes = off;
  return l;
}

}  // namespace

tq_status tq_a2_workspace_size(const tq_tensor_desc* q_probe, const tq_tensor_desc* k_ref, size_t* bytes) {
  if (!bytes) return fail(TQ_EINVAL, "output pointer is NULL");
  int P;
  if (tq_status s = check_a2(q_probe, k_ref, &P)) return s;
  *bytes = a2_bytes(q_probe, k_ref);
  return ok();
}

tq_status tq_a2_weights(const tq_tensor_desc* q_probe, const tq_tensor_desc* k_ref, float* weights, void* ws,
                        size_t ws_bytes, void* stream) {
  int P;
  if (tq_status s = check_a2(q_probe, k_ref, &P)) return s;
  if (!weights || !aligned(weights, 4)) return fail(TQ_EINVAL, "weights NULL or not 4-byte aligned");
  const size_t need = a2_bytes(q_probe, k_ref);
  if (!ws || !aligned(ws, 256)) return fail(TQ_EINVAL, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < need) return fail(TQ_ENOMEM, "workspace %zu bytes < required %zu", ws_bytes, need);
  A2Params p;
  std::memset(&p, 0, sizeof(p));
  p.q = q_probe->data; p.qdtype = q_probe->dtype;
  p.qsb = q_probe->stride_b; p.qsh = q_probe->stride_h; p.qst = q_probe->stride_t;
  p.k = k_ref->data; p.kdtype = k_ref->dtype;
  p.ksb = k_ref->stride_b; p.ksh = k_ref->stride_h; p.kst = k_ref->stride_t;
  p.B = k_ref->B; p.Hq = q_probe->H; p.Hkv = k_ref->H; p.G = q_probe->H / k_ref->H; p.Np = q_probe->T;
  p.P = P; p.T = k_ref->T; p.d = k_ref->d;
  p.chunk = 8 * 4 * (64 / (k_ref->d / 32));   // 8 steps of the block's 4 waves
  p.inv_sqrt_d = 1.0f / std::sqrt((float)k_ref->d);
  char* w = static_cast<char*>(ws);
  const size_t rows = (size_t)p.B * p.Hq * p.Np;
  p.scores = reinterpret_cast<float*>(w);
  p.lse = reinterpret_cast<double*>(w + round_up(rows * p.T * 4, 256));
  p.weights = weights;
  return hip_status(launch_a2_weights(p, (hipStream_t)stream), "A^2 weight launch");
}

tq_status tq_value_policy_workspace_size(const tq_tensor_desc* v_ref, size_t* bytes) {
  if (!bytes) return fail(TQ_EINVAL, "output pointer is NULL");
  if (tq_status s = check_tensor(v_ref, "v_ref")) return s;
  *bytes = policy_layout(v_ref).bytes;
  return ok();
}

tq_status tq_value_policy(const float* weights, const tq_tensor_desc* v_ref, int32_t budget_bits, int32_t* perm,
                          tq_value_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  if (tq_status s = check_tensor(v_ref, "v_ref")) return s;
  if (!weights || !aligned(weights, 4) || !perm || !aligned(perm, 4) || !plan)
    return fail(TQ_EINVAL, "weights, perm or plan NULL or misaligned");
  if (budget_bits < 1 || budget_bits > kMaxIndexBits) return fail(TQ_EINVAL, "budget_bits=%d outside [1, %d]", budget_bits, kMaxIndexBits);
  const PolicyLayout lay = policy_layout(v_ref);
  if (!ws || !aligned(ws, 256)) return fail(TQ_EINVAL, "workspace NULL or not 256-byte aligned");
  if (ws_bytes < lay.bytes) return fail(TQ_ENOMEM, "workspace %zu bytes < required %zu", ws_bytes, lay.bytes);
  // Candidates: uniform, (b-1, b+1) with half high, (b-1, b+2) with a third high.
  tq_value_plan pl;
  std::memset(&pl, 0, sizeof(pl));
  const int T = v_ref->T;
  auto add = [&](int lo, int hi, int num, int den) {
    if (lo < 1 || hi > kMaxIndexBits) return;
    const int c = pl.n_candidates++;
    pl.cand_lo[c] = lo; pl.cand_hi[c] = hi; pl.cand_high[c] = (int)(((long)T * num) / den);
  };
  add(budget_bits, budget_bits, 0, 1);
  add(budget_bits - 1, budget_bits + 1, 1, 2);
  add(budget_bits - 1, budget_bits + 2, 1, 3);
  char* w = static_cast<char*>(ws);
  hipStream_t st = (hipStream_t)stream;
  PolicyParams p;
  std::memset(&p, 0, sizeof(p));
  p.v = v_ref->data; p.vdtype = v_ref->dtype;
  p.vsb = v_ref->stride_b; p.vsh = v_ref->stride_h; p.vst = v_ref->stride_t;
  p.B = v_ref->B; p.H = v_ref->H; p.T = T; p.d = v_ref->d;
  p.weights = weights;
  p.gain = reinterpret_cast<float*>(w + lay.off_gain);
  p.sel = reinterpret_cast<PolicySel*>(w + lay.off_sel);
  p.total = reinterpret_cast<double*>(w + lay.off_total);
  p.perm = perm;
  p.ncand = pl.n_candidates;
  for (int c = 0; c < pl.n_candidates; ++c) p.cand_R[c] = pl.cand_high[c];
  if (tq_status s = hip_status(launch_policy_select(p, st), "policy selection launch")) return s;
  const size_t BH = (size_t)p.B * p.H;
  std::vector<PolicySel> sel(BH * p.ncand);
  std::vector<double> total(BH);
  if (tq_status s = hip_status(hipMemcpyAsync(sel.data(), p.sel, sel.size() * sizeof(PolicySel), hipMemcpyDeviceToHost, st), "copy")) return s;
  if (tq_status s = hip_status(hipMemcpyAsync(total.data(), p.total, BH * 8, hipMemcpyDeviceToHost, st), "copy")) return s;
  if (tq_status s = hip_status(hipStreamSynchronize(st), "sync")) return s;
  int best = 0;
  for (int c = 0; c < pl.n_candidates; ++c) {
    const double Dl = codebook_distortion(v_ref->d, pl.cand_lo[c]), Dh = codebook_distortion(v_ref->d, pl.cand_hi[c]);
    double sur = 0.0;
    for (size_t bh = 0; bh < BH; ++bh) {
      const double top = sel[bh * p.ncand + c].top;
      sur += Dl * (total[bh] - top) + Dh * top;
    }
    pl.surrogate[c] = sur;
    if (sur < pl.surrogate[best]) best = c;
  }
  pl.b_lo = pl.cand_lo[best]; pl.b_hi = pl.cand_hi[best]; pl.n_high = pl.cand_high[best];
  p.chosen = best;
  if (tq_status s = hip_status(launch_policy_permute(p, st), "permutation launch")) return s;
  if (tq_status s = hip_status(hipStreamSynchronize(st), "sync")) return s;
  *plan = pl;
  return ok();
}

tq_status tq_gather_tokens(const tq_tensor_desc* x, const int32_t* perm, int32_t t0, const tq_tensor_desc* out,
                           void* stream) {
  if (tq_status s = check_tensor(x, "x")) return s;
  if (tq_status s = check_tensor(out, "out")) return s;
  if (!perm || !aligned(perm, 4)) return fail(TQ_EINVAL, "perm NULL or not 4-byte aligned");
  if (x->B != out->B || x->H != out->H || x->d != out->d || x->dtype != out->dtype)
    return fail(TQ_EMISMATCH, "out differs from x in B, H, d or dtype");
  if (t0 < 0 || (long)t0 + out->T > x->T) return fail(TQ_EINVAL, "tokens [%d, %d) outside [0, %d)", t0, t0 + out->T, x->T);
  GatherParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = x->data; p.out = const_cast<void*>(out->data); p.es = elem_size(x->dtype);
  p.xsb = x->stride_b; p.xsh = x->stride_h; p.xst = x->stride_t;
  p.osb = out->stride_b; p.osh = out->stride_h; p.ost = out->stride_t;
  p.B = x->B; p.H = x->H; p.T = x->T; p.t0 = t0; p.tn = out->T; p.row_bytes = x->d * p.es;
  p.perm = perm;
  return hip_status(launch_gather(p, (hipStream_t)stream), "gather launch");
}

tq_status tq_attention_merge(const float* out_a, const float* lse_a, const float* out_b, const float* lse_b,
                             int32_t n, int32_t d, float* out, float* lse, void* stream) {
  if (!out_a || !lse_a || !out_b || !lse_b || !out) return fail(TQ_EINVAL, "NULL pointer");
  if (n < 1 || d < 1) return fail(TQ_EINVAL, "n=%d d=%d", n, d);
  MergeParams p{out_a, lse_a, out_b, lse_b, n, d, out, lse};
  return hip_status(launch_merge(p, (hipStream_t)stream), "merge launch");
}

tq_status tq_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(TQ_EINVAL, "src must be 16-byte aligned, sink 4-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(TQ_EINVAL, "bytes must be a positive multiple of 16");
  return hip_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream), "stream read launch");
}

tq_status tq_stream_rw(const void* src, int64_t rows, int32_t in_row_bytes, void* dst, int32_t out_row_bytes,
                       float* planes, int32_t nplanes, void* stream) {
  if (!src || !dst || (nplanes > 0 && !planes)) return fail(TQ_EINVAL, "NULL pointer");
  if (!aligned(src, 16) || !aligned(dst, 16) || (planes && !aligned(planes, 4)))
    return fail(TQ_EINVAL, "src and dst must be 16-byte aligned, planes 4-byte aligned");
  if (in_row_bytes < 64 || in_row_bytes > 4096 || in_row_bytes % 64 || out_row_bytes < 64 || out_row_bytes > 4096 ||
      out_row_bytes % 64)
    return fail(TQ_EINVAL, "row sizes must be multiples of 64 in [64, 4096]");
  if (nplanes < 0 || nplanes > 4) return fail(TQ_EINVAL, "nplanes must be in [0, 4]");
  if (rows < 1 || rows > (int64_t(1) << 35)) return fail(TQ_EINVAL, "rows must be in [1, 2^35]");
  int cus = 0;
  if (tq_status st = hip_status(cu_count(&cus), "device query")) return st;
  return hip_status(launch_stream_rw(src, (long)rows, in_row_bytes, dst, out_row_bytes, planes, nplanes, cus,
                                     (hipStream_t)stream),
                    "stream read-write launch");
}

tq_status tq_release_cache(void) {
  std::lock_guard<std::mutex> lk(g_cache_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_sketch) {
    (void)hipSetDevice(std::get<0>(kv.first));
    (void)hipFree(kv.second);
  }
  g_sketch.clear();
  for (auto& kv : g_sketch16) {
    (void)hipSetDevice(std::get<0>(kv.first));
    (void)hipFree(kv.second);
  }
  g_sketch16.clear();
  (void)hipSetDevice(cur);
  return ok();
}

}  // extern "C"
