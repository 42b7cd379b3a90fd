// Internal declarations shared by the host dispatch and the HIP kernel
// launchers of libtq.  Not part of the public ABI (include/tq.h is).
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxIndexBits = 4;   // Lloyd-Max index width supported by the kernels
constexpr int kMaxD = 1024;
constexpr int kCoordsPerLane = 32; // every kernel gives a lane 32 consecutive coordinates
constexpr int kMaxSideRank = 64;

// ---- host math (host_math.cpp) -------------------------------------------
// Beta((d-1)/2,(d-1)/2) Lloyd-Max codebook in double, cached per (d, bits).
bool codebook(int d, int bits, std::vector<double>* centroids, std::vector<double>* boundaries);
// SplitMix64 streams for the sign vector and the Gaussian sketch.
void sign_vector(uint64_t seed, int d, float* signs);
void gaussian_sketch(uint64_t seed, int d, float* S);  // m = d rows, row-major
// Rank-r PCA of centred rows, Jacobi eigensolver: the top-r eigenvectors as
// the columns of U [d][rank] (largest-|.| entry positive); optionally their
// eigenvalues [rank] and the mean [d].
bool pca_basis(const float* X, int N, int d, int rank, float* U, float* eigenvalues = nullptr,
               float* mean = nullptr);
// Lloyd-Max codebook of N(0, 1) in double, cached per bits.
bool gaussian_codebook(int bits, std::vector<double>* centroids, std::vector<double>* boundaries);
// Relative MSE of the b-bit Beta Lloyd-Max code (TQ-MSE) at head dim d.
double codebook_distortion(int d, int bits);

// ---- kernel parameter blocks ----------------------------------------------
struct QuantParams {
  const void* x;
  int dtype;            // tq_dtype
  int B, H, T, T_cap, d, L;  // L = d / 32 lanes per vector
  int64_t sb, sh, st;   // input strides (elements)
  int mode, bits;
  int rotate;           // 1 for MSE/PROD/HEADQ
  float centroids[16];
  float bounds[16];     // 2^bits - 1 used
  uint32_t signbits[kMaxD / 32];  // bit i set <=> D_i = -1
  float inv_sqrt_d;
  const float* S;       // PROD: m x d row-major (device)
  const float* basis;   // HEADQ: [H][d][rank] (device)
  int rank, side_bits;
  uint8_t* codes; float* norms; uint8_t* qjl; float* gamma; uint8_t* side; float* side_scale;
  // Window of a generic-kernel launch: heads [bh0, bh0 + nbh), tokens
  // [t0, t0 + tn).
  int bh0, nbh, t0, tn;
  const _Float16* S16;    // PROD at d >= 256: S in fp16 (exact), fragment order (device)
  const float* rbasis;    // HEADQ: (Pi U_h)^T per head, [H][rank][d]
  // HEADQ at d = 128, rank 16: rbasis times 2^10 split into fp16 hi (first
  // [H][rank][d] block) and lo = rest (second block); NULL elsewhere.
  const _Float16* rbasis16;
  // SPECTRAL: basis (V, [H][d][d]) in `basis`, the mean and spreads [H][d],
  // and the N(0, 1) Lloyd-Max boundaries in double.
  const float* smean;
  const float* sscale;
  double gbounds[16];
  // Append: token t of sequence b is written to slot pos[b] + t (device
  // int32 [B]); slots outside [0, T_cap) are skipped.  NULL: slot t.
  const int* pos;
};

// Uniform grid over the unit-sphere coordinate y in [-1, 1] used to find the
// Lloyd-Max index: cell n = round(y * scale) + center, cells = 2 center + 1.
// A coordinate in cell n lies within half a cell of its centre; the window
// of half-width 0.5 + kGridMargin cells around it holds at most one boundary
// (the cell width is below the smallest gap / (1 + 2 kGridMargin)), so a
// cell's entry is that boundary and the count of boundaries below the window.
constexpr float kGridMargin = 0.0625f;
struct QuantGrid {
  float scale;
  int center, cells;
};

struct TensorPlanes {
  const uint8_t* codes; const float* norms; const uint8_t* qjl; const float* gamma;
  const uint8_t* side; const float* side_scale;
};

struct DecodeParams {
  int B, Hkv, G, Hq, T, T_cap, d, L;
  int nsplit, chunk;    // tokens per split (multiple of 64)
  int part_stride;      // floats per partial record
  int units;            // number of (query, split) work units, see the XCD mapping
  TensorPlanes k, v;
  int rank, side_bits;
  float kc[16], vc[16];
  float k_qjl, v_qjl;   // sqrt(pi/2)/m
  float scale_log2;     // log2(e)/sqrt(d)
  const float* qrot; const float* qsk; const float* qw;
  const float* qoff;    // SPECTRAL keys: per-query score offset q . mu / sqrt(d), else NULL
  float* part;
  // Per-sequence lengths (device int32 [B]), each clamped to [0, T); NULL:
  // every sequence has T tokens.
  const int* lens;
};

struct QPrepParams {
  const void* q; int dtype; int B, Hq, d, Hkv;
  int64_t sb, sh;
  int rotate, kqjl, kside, rank;
  // SPECTRAL keys: q_rot = s * (V^T q) with the query's KV head's basis,
  // spreads and mean; qoff = q . mu / sqrt(d) (the score offset the mean adds).
  int kspectral;
  const float* sbasis; const float* smean; const float* sscale;
  float* qoff;
  uint32_t signbits[kMaxD / 32];
  float inv_sqrt_d;
  const float* S; const float* basis;
  float* qrot; float* qsk; float* qw;
  float* qraw;          // optional copy of the raw query (metrics)
};

struct CombineParams {
  int nq, d, nsplit, part_stride, vqjl, vrotate;
  float v_qjl;
  uint32_t signbits[kMaxD / 32];
  float inv_sqrt_d;
  const float* S;
  const float* part;
  float* out; float* lse;
  // SPECTRAL values: out = mu + V (s * acc / l) with the query's KV head's
  // basis, mean and spreads (query qi reads KV head (qi % Hq) / G).
  int vspectral, Hq, G;
  const float* vbasis; const float* vmean; const float* vscale;
  // SPECTRAL keys: the per-query score offset added to the log-sum-exp.
  const float* qoff;
  // Large d with sketched values (combine_splits): workspace for o = acc / l,
  // k = acc_sk / l and S^T k, [nq][d] floats each; the combine then runs as
  // merge (stage 1), one S^T product over all queries, finalize (stage 2).
  // NULL: one pass (stage 0).  `stage` is set by launch_combine.
  float* ow; float* kw; float* add;
  int stage;
};

// Y[q][i] = sum_k M(i, k) X[q][k] for nq queries, M = S (trans = 0) or S^T.
struct SProjParams {
  const float* S; const float* X; float* Y;
  int nq, d, trans;
};

struct MetricScoreParams {
  DecodeParams dp;      // scoring half of the decode parameters (k planes, q prep)
  const void* kref; int kdtype; int64_t ksb, ksh, kst;
  const float* qraw;    // [B*Hq][d] raw queries
  float* s_ref; float* s_hat;  // [B*Hq][T]
};

// Per-query measures from the score rows: KL, top-5 recall, the Fisher
// score error 1/2 Var_p(s_hat - s_ref), the A^2 value distortion
// sum_j p_j^2 verr[j] (when verr, per value vector, is given) and the
// reference log-sum-exp.
constexpr int kPerQuery = 5;
struct MetricReduceParams {
  int nq, T;
  const float* s_ref; const float* s_hat;
  double* per_query;  // [nq][kPerQuery] = kl, recall, fisher, a2, lse_ref
  const float* verr;  // [B*Hkv][T_cap] ||v_hat - v||^2, or NULL
  int Hq, G, Hkv, T_cap;
};

// Exact attention output over the raw values: o_ref = sum_j p_j v_j with p
// from the reference score rows and their log-sum-exp.
struct AttnRefParams {
  int nq, T, d, Hq, G, Hkv;
  const float* s_ref; const double* per_query;
  const void* v; int vdtype; int64_t vsb, vsh, vst;
  float* o_ref;       // [nq][d]
};

struct RelErrParams {
  const void* x; int dtype; int B, H, T, T_cap, d, L;
  int64_t sb, sh, st;
  int mode, bits, rotate, kqjl, kside, rank, side_bits;
  float centroids[16];
  uint32_t signbits[kMaxD / 32];
  float inv_sqrt_d, qjl_c;
  const float* S; const float* basis;
  const float* smean; const float* sscale;  // SPECTRAL: mean and spreads [H][d]
  TensorPlanes planes;
  double* block_sums;  // [gridDim][5] = err2, ref2, (1-cos) sum, count, angle sum
  float* per_vec;      // [B*H][T_cap] ||x_hat - x||^2 per vector, or NULL
};

// ---- launchers (defined in the .hip files) --------------------------------
// grid: the index-search table's grid (NULL or too many cells: every
// boundary is compared instead).
hipError_t launch_quantize(const QuantParams& p, const QuantGrid* grid, hipStream_t s);
// SPECTRAL at d = 32, 64, 128 (quant_spectral.hip) and its reconstruction error.
int spectral_max_d();
// d = 128 takes the matrix-core kernel with certified decisions when `grid`
// (the N(0, 1) boundaries' lookup grid) fits; otherwise the fp64 kernel.
hipError_t launch_quantize_spectral(const QuantParams& p, const QuantGrid* grid, hipStream_t s);
hipError_t launch_relerr_spectral(const RelErrParams& p, hipStream_t s);
// PROD at d = 256..1024 with the sketch projection on the matrix cores (quant_sketch.hip).
bool quant_sketch_supported(const QuantParams& p, const QuantGrid& grid);
// Index of S[row][col] in the fragment-ordered fp16 copy of S that the
// matrix-core sketch kernel reads (QuantParams::S16).
size_t sketch_fragment_index(int d, int row, int col);
hipError_t launch_quantize_sketch(const QuantParams& p, const QuantGrid& grid, hipStream_t s);
// (Pi U_h)^T of every head into out [H][rank][d] (device).
hipError_t launch_rotate_basis(const QuantParams& p, float* out, _Float16* out16, hipStream_t s);
// Matrix-core write side (fp16 input, d = 128, PLAIN/MSE/PROD).
bool quant_mfma_supported(const QuantParams& p);
int quant_mfma_lut_max();
hipError_t launch_quantize_mfma(const QuantParams& p, const QuantGrid& grid, int nblocks, hipStream_t s);
hipError_t launch_qprep(const QPrepParams& p, hipStream_t s);
hipError_t launch_decode_split(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl,
                               hipStream_t s, bool* supported);
hipError_t launch_combine(const CombineParams& p, hipStream_t s);
// Whether the combine of a decode with these values takes the split form
// (its workspace then holds three [nq][d] float arrays).
bool combine_splits(int d, bool vqjl, bool vspectral);
// Table-driven decode (3/4-bit codes at d = 128), persistent blocks.
bool lut_supported(int d, int kbits, int kqjl, int kside, int side_rank, int side_bits, int vbits, int vqjl);
// Waves per block of the table-driven kernel (at d > 128 each wave writes its
// own partial).
int lut_waves(int vqjl);
hipError_t launch_decode_lut(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl, int nblocks,
                             hipStream_t s);
// Grouped-query decode on the matrix cores (decode_mq.hip): d = 128..1024,
// G >= 2 query heads per KV head, 2- to 4-bit keys (3-bit with a sketch) or
// HeadQ at d = 128, 1- to 4-bit values (3-bit with a sketch).  A unit (KV
// head, 16 queries, chunk) takes mq_waves_per_unit(d) waves; a block holds
// mq_units_per_block(d, kqjl, vqjl) units.
bool mq_supported(int d, int G, int kbits, int kqjl, int kside, int side_rank, int side_bits, int vbits, int vqjl);
int mq_waves_per_unit(int d);
int mq_units_per_block(int d, int kqjl, int vqjl);
int mq_target_units(int d, int kqjl, int vqjl, int cus);
hipError_t launch_decode_mq(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl, int nblocks,
                            hipStream_t s);
// The same for d = 256..1024 (decode_mq_wide.hip).
hipError_t launch_decode_mq_wide(const DecodeParams& p, int kbits, int kqjl, int kside, int vbits, int vqjl,
                                 int nblocks, hipStream_t s);
hipError_t launch_metric_scores(const MetricScoreParams& p, int kbits, int kqjl, int kside, hipStream_t s,
                                bool* supported);
hipError_t launch_metric_reduce(const MetricReduceParams& p, hipStream_t s);
hipError_t launch_attn_ref(const AttnRefParams& p, hipStream_t s);
hipError_t launch_relerr(const RelErrParams& p, int nblocks, hipStream_t s);
// The static decode workspace (noalloc.hip): its size, and this device's
// address of it (hipGetSymbolAddress, taken once per device).
// ---- A^2-weighted value policy (policy.hip) -----------------------------------
struct A2Params {
  const void* q; int qdtype; int64_t qsb, qsh, qst;   // probes [B][Hq][Np][d]
  const void* k; int kdtype; int64_t ksb, ksh, kst;   // raw keys [B][Hkv][T][d]
  int B, Hq, Hkv, G, Np, P, T, d, chunk;              // P = G * Np probes per KV head
  float inv_sqrt_d;
  float* scores;        // [B*Hq*Np][T]
  double* lse;          // [B*Hq*Np]
  float* weights;       // [B*Hkv][T]
};
struct PolicySel {
  uint32_t thr;         // bit pattern of the R-th largest gain
  int need_eq;          // how many tokens equal to it are taken (lowest indices)
  double top;           // sum of the R largest gains
};
struct PolicyParams {
  const void* v; int vdtype; int64_t vsb, vsh, vst;   // raw values [B][H][T][d]
  int B, H, T, d;
  const float* weights; float* gain;                  // [B*H][T]
  int ncand, chosen;
  int cand_R[4];
  PolicySel* sel;       // [B*H][ncand]
  double* total;        // [B*H]
  int32_t* perm;        // [B*H][T]
};
struct GatherParams {
  const void* x; void* out; int es;
  int64_t xsb, xsh, xst, osb, osh, ost;
  int B, H, T, t0, tn, row_bytes;
  const int32_t* perm;
};
struct MergeParams {
  const float* out_a; const float* lse_a; const float* out_b; const float* lse_b;
  int n, d;
  float* out; float* lse;
};
size_t a2_workspace_bytes(int rows, int T);
hipError_t launch_a2_weights(const A2Params& p, hipStream_t s);
hipError_t launch_policy_select(const PolicyParams& p, hipStream_t s);
hipError_t launch_policy_permute(const PolicyParams& p, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);

size_t static_scratch_bytes();
hipError_t static_scratch(void** out);
int stream_read_blocks();
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s);
hipError_t launch_stream_rw(const void* src, long rows, int in_row_bytes, void* dst, int out_row_bytes, float* planes,
                            int nplanes, int cus, hipStream_t s);

}  // namespace tq
