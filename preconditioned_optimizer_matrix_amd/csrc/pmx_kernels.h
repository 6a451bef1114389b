// Parameter blocks and launchers of the non-GEMM kernels of libpmx.
#pragma once

#include "pmx_internal.h"

namespace pmx {

// Partial-sum slots reserved per matrix for the elementwise reductions and
// for the residual GEMM (one slot per output tile).
constexpr int kPartialsPerMatrix = 1024;

// Blocks per matrix of a row-looping kernel over a batch: about `total`
// blocks in all, at most `cap` and at most one per row.  Kernels that end in a
// last-block reduction take total = 1024: every block pays a device-wide fence
// before its arrival, so one block per row of a large batch (32768 blocks for
// 64 matrices of order 512) spent over a millisecond in fences.
inline int blocks_per_matrix(int rows, int batch, int total, int cap) {
  int per = (total + batch - 1) / batch;
  if (per > cap) per = cap;
  if (per > rows) per = rows;
  return per < 1 ? 1 : per;
}
// Gram share slots per skinny block (J (J + 1) / 2 <= 45 entries, J <= 9).
constexpr int kGramShare = 48;

// bf16 storage type: raw bits, converted explicitly (round to nearest even).
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float((uint32_t)x.bits << 16);
}
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return bf16_t{(uint16_t)0x7FC0};
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t{(uint16_t)(u >> 16)};
}

struct StageInitParams {
  const float* a;        // stage 0 input A
  int64_t lda, a_stride;
  float* ybuf[2];        // ping-pong Y buffers (n x n, ld n)
  float* r;              // residual buffer
  int64_t buf_stride;    // batch stride of the work buffers
  int n, stage;
  Ctrl* ctrl;
  double* partials;
  int64_t partial_stride;
  IterCfg cfg;
  SketchJob sketch;      // S_0 of this stage
};

struct PolarInitParams {
  const void* g;
  int64_t ldg, g_stride;
  void* x;               // X_0 (rows x cols, ld cols)
  int64_t x_stride;
  int rows, cols, transpose;
  Ctrl* ctrl;
  SketchJob sketch;      // the first sketch, generated on the side
};

struct SkinnyJob {
  const float* mat;
  int64_t mat_ld, mat_stride;
  int in_col, out_col;
  int pow;               // output scaled by ||R||_F^-pow; 0: the complement
                         // in - Mat in, unscaled
};

// Coefficient vectors of r(xi; alpha) = sum_j (a0_j + alpha a1_j + alpha^2 a2_j) xi^j.
struct AlphaCoef {
  double a[3][8];  // coefficients of xi^0 .. xi^{2d+1}, d <= 3
  double taylor_d;
};

// Coefficient vectors a_0..a_p (powers xi^0 .. xi^{p d + 1}, p d + 1 <= 9) of
// the inverse Newton residual map r(xi; alpha) = sum_i alpha^i a_i(xi).
struct AlphaCoefN {
  double a[5][10];
  double taylor_d;
};

struct SkinnyParams {
  SkinnyJob job[2];
  float* kbuf;
  int64_t kld, kstride;
  int n, q;
  int variant;  // 0: In staged through LDS, 1: In read directly
  int mfma;     // set by the launcher: the matrix-core form
  Ctrl* ctrl;
  // last pass only: Gram shares (kGramShare doubles per block) and the alpha
  // solve; a matrix at degree d uses K_1..K_{2d+1} (the pass writes one of
  // them, the others are read back), coef and [cfg.lo, cfg.hi] at the
  // configured degree, coef_up and [lo_up, hi_up] at the raised one
  double* gram_partials;
  int64_t gram_stride;
  IterCfg cfg;
  AlphaCoef coef, coef_up;
  float lo_up, hi_up;
  // inverse Newton (newton_p = p > 0): J = gram_j Krylov blocks and the
  // objective of degree 2p built from coef_n
  int newton_p, gram_j;
  AlphaCoefN coef_n;
};

struct FormGParams {
  const float* r;
  const float* r2;       // R^2 (d >= 2), may alias dst
  const float* r3;       // R^3 (d = 3), may alias dst
  void* dst;             // fp32, or bf16 with dst_bf16
  float* dst2;           // optional second fp32 copy (same layout)
  int64_t stride;        // elements, shared by r, r2 and dst
  int n, degree;
  int dst_bf16;
  int vec;               // set by the launcher
  float c0, c1, c2;      // Taylor coefficients c_0 .. c_{d-1} (c2 for d = 3)
  int adaptive;          // 1: each matrix's degree from its control block
  int first_scale;       // 1: g times the control block's inv_s (polar, estimated scale)
  Ctrl* ctrl;
  SketchJob sketch;      // the next iteration's sketch, generated on the side
};

// 64 x 64 tile transpose to bf16: out_t[j][i] = f(in[i][j]) (cols x rows) and
// optionally out_n[i][j] = f(in[i][j]); f is the identity or, with `poly`, the
// PRISM polynomial c0 [i == j] + c1 R + alpha R2 (d = 2) / c0 [i == j] + alpha R.
struct XposeParams {
  const void* a;
  const float* a2;
  int a_bf16;
  int64_t lda, sa;
  uint16_t* out_t;
  int64_t ldt, st;
  uint16_t* out_n;
  int64_t ldn, sn;
  int rows, cols;
  int poly, degree;
  int scale_inv_c;  // multiply the input by 1 / ctrl.c first (needs ctrl)
  float c0, c1;
  Ctrl* ctrl;  // null: unconditional; else skipped when the matrix is not running
  SketchJob sketch;  // a sketch generated on the side (needs ctrl)
  int vec4;  // set by the launcher: bf16 input, no polynomial; 1: 8-byte accesses, 2: 16-byte
};

struct RootFinishParams {
  float* ybuf[2];
  float* zbuf[2];
  int64_t buf_stride;
  float* x;
  int64_t ldx, x_stride;
  float* aux;
  int64_t ldaux, aux_stride;
  int n;
  double expo_x, expo_aux;  // X = c^expo_x Z, aux = c^expo_aux Y
  Ctrl* ctrl;
};

// U from the final iterate X = xbuf[iter & 1] (rows x cols, ld cols): U = X,
// or U = X^T with `transpose` (ld ldu either way); NaN when the call failed.
struct PolarFinishParams {
  void* xbuf[2];
  int64_t buf_stride;
  void* u;
  int64_t ldu, u_stride;
  int rows, cols, transpose;
  int vec;  // set by the launcher
  Ctrl* ctrl;
};

// Fused small-matrix calls: one workgroup per matrix runs the whole iteration
// with every matrix in LDS (order n <= kSmallMaxN; polar rows, cols <= it).
constexpr int kSmallMaxN = 64;

struct SmallRootParams {
  const float* a;
  int64_t lda, a_stride;
  float* x;
  int64_t ldx, x_stride;
  float* aux;  // may be null
  int64_t ldaux, aux_stride;
  int n, stages;
  double expo_x, expo_aux;  // X = c^expo_x Z, X_aux = c^expo_aux Y
  float c0, c1;             // Taylor coefficients c_0, c_1
  IterCfg cfg;
  AlphaCoef coef;
};

struct SmallPolarParams {
  const float* g;
  int64_t ldg, g_stride;
  float* u;
  int64_t ldu, u_stride;
  int rows, cols, transpose;  // the iterate is rows x cols (G^T when transpose)
  float c0, c1;
  IterCfg cfg;
  AlphaCoef coef;
  // variable shapes: block b is blocks[b] (its own pointers, shape and
  // leading dimensions; g, u, rows, cols and transpose above are unused)
  const pmx_polar_block* blocks;
  int bf16;  // elements of G and U are bf16 (fp32 inside)
};

hipError_t launch_small_root(const SmallRootParams& p, int batch, hipStream_t s);
// Variable-size polar factor, blocks above kSmallMaxN: pack one shape group
// (blocks[idx[0 .. count)], all m x n) into dst (count x m x n fp32, dense),
// and scatter the group's factors and info records back.
hipError_t launch_varbatch_gather(const pmx_polar_block* blocks, const int32_t* idx, bool bf16,
                                  float* dst, int m, int n, int count, hipStream_t s);
hipError_t launch_varbatch_scatter(const pmx_polar_block* blocks, const int32_t* idx, bool bf16,
                                   const float* src, int m, int n, int count,
                                   const pmx_matfn_info* info_src, pmx_matfn_info* info_dst,
                                   hipStream_t s);
hipError_t launch_small_polar(const SmallPolarParams& p, int batch, hipStream_t s);

// fp64 leading updates of an inverse root (square n x n buffers, ld n).
struct Gemm64Operand {
  const double* p;
};

struct Gemm64Problem {
  Gemm64Operand a, b;
  double* c;
  float* c32;  // optional fp32 copy of C (stride32)
};

struct Gemm64Params {
  Gemm64Problem prob[2];
  int nprob, n, batch;
  int sym;     // symmetric product (R^2, I - Z Y): upper-triangle tiles, mirrored
  int tile;    // block tile 64 or 128 (0: by the launch's size)
  int num_cu;
  int64_t stride;    // doubles between the matrices of a batch
  int64_t stride32;  // floats between the fp32 copies
  Ctrl* ctrl;
  int degree;
  double c0, c1;
  double* partials;  // ROLE_RESID: Frobenius partials, one per tile
  int64_t partial_stride;
  int products, count_update;
  IterCfg cfg;
  SketchJob sketch;
};

struct StageInit64Params {
  const float* a;
  int64_t lda, a_stride;
  float* ybuf32[2];  // the previous stage's Y (stage 1)
  int64_t stride32;
  double* y64;
  double* r64;
  float* r32;
  int64_t stride;
  int n, stage;
  Ctrl* ctrl;
  double* partials;
  int64_t partial_stride;
  IterCfg cfg;
  SketchJob sketch;
};

struct FormG64Params {
  const double* r;
  const double* r2;
  double* dst;
  int64_t stride;
  int n, degree;
  double c0, c1;
  Ctrl* ctrl;
};

struct Handover64Params {
  double* y64[2];
  double* z64[2];
  float* y32[2];
  float* z32[2];
  int64_t stride, stride32;
  int n, stage;
  Ctrl* ctrl;
};

hipError_t launch_gemm_f64(const Gemm64Params& p, int role, hipStream_t s);
hipError_t launch_stage_init_f64(const StageInit64Params& p, int batch, hipStream_t s);
hipError_t launch_form_g_f64(const FormG64Params& p, int batch, hipStream_t s);
hipError_t launch_handover_f64(const Handover64Params& p, int batch, hipStream_t s);

// Resets the control blocks and infos of a call and zeroes nzero words at zero.
hipError_t launch_ctrl_reset(Ctrl* ctrl, pmx_matfn_info* info, int batch, int degree,
                             uint32_t* zero, int nzero, hipStream_t s);
hipError_t launch_fro_scale(const void* x, bool bf16, int rows, int cols, int64_t ld,
                            int64_t stride, int batch, Ctrl* ctrl, double* partials,
                            int64_t pstride, pmx_matfn_info* info, hipStream_t s);
hipError_t launch_sqrt_stage_init(const StageInitParams& p, int batch, hipStream_t s);
hipError_t launch_polar_init(const PolarInitParams& p, bool bf16, int batch, hipStream_t s);
hipError_t launch_skinny(const SkinnyParams& p, int njobs, bool gram, int batch, hipStream_t s);
int skinny_blocks(int n, int q);
// The power estimate of the input scale (inverse roots, scale_mode 1):
// launch_sketch writes the start block V_0 (the sketch of `sj`, columns
// [0, p) of the Krylov buffer) of every running matrix; after the skinny
// passes K_t = (A / c) K_{t-1}, launch_power_scale sets
// c <- c min(1, factor max_j ||K_t[:, j]|| / ||K_{t-1}[:, j]||) from the
// column blocks at col_last (K_t) and col_prev (K_{t-1}).
constexpr int kPowerStage = 2;   // sketch stream of V_0 (stages 0, 1 are the iteration's)
// t = 8: an isolated top eigenvalue over a bulk below lambda_max / 2 gains
// 2^16 over the bulk in the squared column norms, more than the 1 / n weight
// it starts with for every order up to 32768, so mu >= lambda_max / 2 and c
// stays above the spectrum
constexpr int kPowerPasses = 8;
constexpr double kPowerFactor = 2.0;
hipError_t launch_sketch(const SketchJob& sj, const Ctrl* ctrl, int batch, hipStream_t s);
// pmx_sketch_gaussian: the sketch of (matrix b, stage, iteration k) into S
// (n x p, row stride lds) and optionally its raw Philox words (n x p, dense).
hipError_t launch_sketch_export(uint64_t seed, int b, int stage, int k, int n, int p, float* S,
                                int64_t lds, uint32_t* words, hipStream_t s);
// polar = 0: c <- c min(1, factor mu); polar = 1 (mu estimates the top
// eigenvalue of X_0^T X_0): s = sqrt(min(1, factor mu)), inv_s = 1 / s and
// c <- c s.
hipError_t launch_power_scale(Ctrl* ctrl, const float* kbuf, int64_t kld, int64_t kstride,
                              int n, int p, int col_prev, int col_last, double factor,
                              int polar, pmx_matfn_info* info, int batch, hipStream_t s);
// Polar factor with the estimated scale: R_0 <- I - (I - R_0) inv_s^2 (fp32
// R and, when rh is set, its bf16 copy) for the matrices with inv_s > 1, and
// the decision on r_0 again from the new ||R_0||_F (same stage, k = 0).
hipError_t launch_polar_rescale(Ctrl* ctrl, float* r, uint16_t* rh, int64_t stride, int n,
                                double* partials, int64_t pstride, IterCfg cfg, int batch,
                                hipStream_t s);

// dst (pinned host memory, device-mapped) = 1 if any of ctrl[0 .. batch) is
// still PMX_RUNNING, else 0; one block, a system-scope store.
hipError_t launch_publish_running(const Ctrl* ctrl, int batch, int32_t* dst, hipStream_t s);

hipError_t launch_form_g(const FormGParams& p, int batch, hipStream_t s);
// Statistics operands: G^T (cols x rows fp32, dense) and, when gn is set, G
// widened to fp32 (rows x cols, dense), per batch matrix; zeroes zero[0, nzero).
hipError_t launch_stats_operands(const void* g, bool bf16, int64_t ld, int64_t sg, int rows,
                                 int cols, int batch, float* gt, float* gn, uint32_t* zero,
                                 int nzero, hipStream_t s);
// Elementwise copy between fp32 and bf16 matrices (rows x cols, strided batch);
// bf16 -> fp32 is exact, fp32 -> bf16 rounds to nearest even.
hipError_t launch_convert(const void* src, bool src_bf16, int64_t lds, int64_t ss, void* dst,
                          bool dst_bf16, int64_t ldd, int64_t sd, int rows, int cols, int batch,
                          hipStream_t s);
hipError_t launch_gemm_bf16(const GemmParams& p, int role, hipStream_t s);
hipError_t launch_xpose(const XposeParams& p, int batch, hipStream_t s);
hipError_t launch_root_finish(const RootFinishParams& p, int batch, hipStream_t s);
hipError_t launch_polar_finish(const PolarFinishParams& p, bool bf16, int batch, hipStream_t s);


}  // namespace pmx
