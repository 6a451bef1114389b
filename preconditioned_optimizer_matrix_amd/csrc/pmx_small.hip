// Fused PRISM iteration for small matrices on gfx950: one workgroup runs a
// whole inverse root (n <= 64) or fp32 polar factor (rows, cols <= 64) with
// every matrix in LDS, so a call is one launch instead of about eight per
// iteration.  The steps, their order, the sketch generator, the Krylov
// scaling, the alpha fit and the stopping rule are those of the multi-kernel
// path (the same device functions where they are shared); only the order of
// floating-point summation differs.
//
//  * Matrices are stored 64 x 64 (row stride 68 floats) with zeros outside
//    the n x n block, so every product may run over the padded order: the
//    identity terms are restricted to i < n and the padding stays zero.
//  * Dense products on fp32 MFMA, one 32 x 32 quarter per wave.  The
//    contraction always runs over the padded 64 (the padding and the rows of
//    the Krylov buffer beyond n are zero), so every loop unrolls.
//  * The Krylov blocks (64 x p) are 16 x 16 MFMA tiles spread over the four
//    waves; their Gram is summed in fp64 by 16 threads per entry.
//  * The control block lives in LDS; thread 0 applies decide() and the
//    alpha fit, a barrier publishes the outcome.  While thread 0 solves for
//    alpha, the other three waves draw the next iteration's sketch.
#include "pmx_alpha.h"
#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr int SN = 64;    // padded order
constexpr int SLD = 68;   // LDS row stride (floats)
constexpr int SMAT = SN * SLD;
constexpr int SNT = 256;
// Krylov buffer row stride: (2d + 2) p <= 96 columns, odd so that the four
// 16-lane groups of an MFMA operand read (rows 16 apart) fall in distinct banks
constexpr int SKLD = 6 * 16 + 1;

struct SmallShared {
  float m[6][SMAT];
  float kb[SN * SKLD];
  double red[SNT / 64][16];
  double gsum[16];
  Ctrl c;
};

__device__ __forceinline__ double block_total(double v, SmallShared& sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sh.red[w][0] = v;
  __syncthreads();
  return ((sh.red[0][0] + sh.red[1][0]) + sh.red[2][0]) + sh.red[3][0];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C = op(A) B over the padded order (every operand is zero outside its
// block, so the contraction always runs over 64), op(A) = A (A[i][k]) or,
// with TA, A^T (A stored k-major: A[k][i]).  Wave w computes the 32 x 32
// quarter (32 (w / 2), 32 (w % 2)) with 32 v_mfma_f32_32x32x2_f32: step m
// takes k = m from lanes 0-31 and k = m + 32 from lanes 32-63, so a lane's
// A values of one row are contiguous (16-byte reads when A is not
// transposed).  RESID: C = I_n - acc and the fp64 sum of squares is returned
// (block total); otherwise 0.
// The update polynomial g = c0 I_n + c1 R + alpha R2 (d = 2) or c0 I_n +
// alpha R (d = 1), formed element by element where a product reads it.
struct SmallPoly {
  const float* r;
  const float* r2;
  float c0, c1, alpha;
  int d, n;
  __device__ __forceinline__ float at(float rv, float r2v, bool diag) const {
    float v = (d == 2) ? c1 * rv + alpha * r2v : alpha * rv;
    if (diag) v += c0;
    return v;
  }
};

template <bool TA, bool RESID, int POLY = 0>
__device__ double small_gemm(float* C, const float* A, const float* B, int n_id,
                             SmallShared& sh, const SmallPoly* pg = nullptr) {
  // POLY = 2: B is g, formed from pg while loading
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
  const int li = lane & 31, kh = (lane >> 5) * 32;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const float* bcol = (POLY == 2 ? pg->r : B) + kh * SLD + wn + li;
  const float* bcol2 = POLY == 2 ? pg->r2 + kh * SLD + wn + li : nullptr;
  auto bval = [&](int m) {
    if constexpr (POLY == 2) {
      const int k = kh + m;
      return pg->at(bcol[m * SLD], bcol2[m * SLD], k == wn + li && k < pg->n);
    } else {
      return bcol[m * SLD];
    }
  };
  if (TA) {
    const float* acol = A + kh * SLD + wm + li;
#pragma unroll
    for (int m = 0; m < 32; ++m)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(acol[m * SLD], bval(m), acc, 0, 0, 0);
  } else {
    const float* arow = A + (wm + li) * SLD + kh;
#pragma unroll
    for (int m4 = 0; m4 < 8; ++m4) {
      const float4 a = *reinterpret_cast<const float4*>(arow + 4 * m4);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bval(4 * m4 + 0), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bval(4 * m4 + 1), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bval(4 * m4 + 2), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bval(4 * m4 + 3), acc, 0, 0, 0);
    }
  }
  // lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + (v % 4)
  double fro = 0.0;
  const int col = wn + li;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = wm + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    float x = acc[v];
    if (RESID) {
      x = ((row == col && row < n_id) ? 1.f : 0.f) - x;
      fro += (double)x * (double)x;
    }
    C[row * SLD + col] = x;
  }
  __syncthreads();
  return RESID ? block_total(fro, sh) : 0.0;
}

// S (n x p) of matrix b, stage, iteration k into columns [0, p) of the Krylov
// buffer: the counter layout and transform of the library's sketch generator.
// Threads [t0, SNT) take part (no barrier here).
__device__ void small_sketch(SmallShared& sh, int n, int p, int k, int stage, int b,
                             uint32_t seed_lo, uint32_t seed_hi, int t0 = 0) {
  const int calls = (n * p + 3) / 4;
  if ((int)threadIdx.x < t0) return;
  for (int q = (int)threadIdx.x - t0; q < calls; q += SNT - t0) {
    uint32_t c[4] = {(uint32_t)q, (uint32_t)k, (uint32_t)stage, (uint32_t)b};
    philox4x32_10(c, seed_lo, seed_hi);
    double z[4];
    philox_normals(c, z);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int e = q * 4 + w;
      if (e < n * p) sh.kb[(e / p) * SKLD + (e % p)] = (float)z[w];
    }
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16 x 16 tile of kb cols [oc, oc + q) = scale * mat * kb cols [ic, ic + q)
// (rows 16 rt.., block columns 16 ct..) with 16 v_mfma_f32_16x16x4f32.  The
// contraction runs over the padded 64 (mat and the Krylov rows beyond n are
// zero).  In step m, lane group g = l / 16 carries k = 16 g + m, so a lane's
// 16 values of mat are one contiguous run of its row (four 16-byte reads).
// All 20 operand reads are issued before the first product (the scheduling
// barrier keeps the compiler from interleaving them with the products, which
// would wait on LDS once per pair).  A block column at or beyond q reads
// column q - 1 (in bounds); a product's column j depends on B's column j
// alone, so those columns are only left unstored.
__device__ __forceinline__ f32x4 krylov_tile(float* kb, const float* mat, int ic, int oc, int q,
                                             float scale, int rt, int ct) {
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const int col = 16 * ct + li;
  const bool live = col < q;
  const float* arow = mat + (16 * rt + li) * SLD + 16 * g;
  const float* bcol = kb + (16 * g) * SKLD + ic + (live ? col : q - 1);
  float4 a[4];
  float bv[16];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) a[m4] = *reinterpret_cast<const float4*>(arow + 4 * m4);
#pragma unroll
  for (int m = 0; m < 16; ++m) bv[m] = bcol[m * SKLD];
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m4].x, bv[4 * m4 + 0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m4].y, bv[4 * m4 + 1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m4].z, bv[4 * m4 + 2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m4].w, bv[4 * m4 + 3], acc, 0, 0, 0);
  }
  // lane l holds block column l % 16 of rows 4 (l / 16) + r
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] *= scale;
  if (live) {
#pragma unroll
    for (int r = 0; r < 4; ++r) kb[(16 * rt + 4 * g + r) * SKLD + oc + col] = acc[r];
  }
  return acc;
}

struct KrylovJob {
  const float* mat;
  int ic, oc, q;
  float scale;
};

// Two independent tiles (rows 16 rt of job a and of job b, block columns
// 0..15 of each) with their 40 operand reads issued first and the two chains
// of 16 products interleaved.
__device__ __forceinline__ void krylov_tiles2(float* kb, const KrylovJob& ja,
                                              const KrylovJob& jb, int rt) {
  const int lane = threadIdx.x & 63, li = lane & 15, g = lane >> 4;
  const bool la = li < ja.q, lb = li < jb.q;
  const float* arow_a = ja.mat + (16 * rt + li) * SLD + 16 * g;
  const float* arow_b = jb.mat + (16 * rt + li) * SLD + 16 * g;
  const float* bcol_a = kb + (16 * g) * SKLD + ja.ic + (la ? li : ja.q - 1);
  const float* bcol_b = kb + (16 * g) * SKLD + jb.ic + (lb ? li : jb.q - 1);
  float4 a0[4], a1[4];
  float b0[16], b1[16];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    a0[m4] = *reinterpret_cast<const float4*>(arow_a + 4 * m4);
    a1[m4] = *reinterpret_cast<const float4*>(arow_b + 4 * m4);
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    b0[m] = bcol_a[m * SKLD];
    b1[m] = bcol_b[m * SKLD];
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[m4].x, b0[4 * m4 + 0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[m4].x, b1[4 * m4 + 0], c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[m4].y, b0[4 * m4 + 1], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[m4].y, b1[4 * m4 + 1], c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[m4].z, b0[4 * m4 + 2], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[m4].z, b1[4 * m4 + 2], c1, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[m4].w, b0[4 * m4 + 3], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[m4].w, b1[4 * m4 + 3], c1, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (la) kb[(16 * rt + 4 * g + r) * SKLD + ja.oc + li] = c0[r] * ja.scale;
    if (lb) kb[(16 * rt + 4 * g + r) * SKLD + jb.oc + li] = c1[r] * jb.scale;
  }
}

// One step of the Krylov recursion: the tiles of up to two independent
// products, tile t on wave t % 4, then a barrier.  With q <= 16 (p <= 8, or
// p <= 16 outside the double-width step) every wave owns row band w of each
// job: one tile, or two interleaved.
__device__ void krylov_step(SmallShared& sh, KrylovJob j0, KrylovJob j1, int jobs) {
  const int w = threadIdx.x >> 6;
  if (j0.q <= 16 && (jobs == 1 || j1.q <= 16)) {
    if (jobs == 2) krylov_tiles2(sh.kb, j0, j1, w);
    else krylov_tile(sh.kb, j0.mat, j0.ic, j0.oc, j0.q, j0.scale, w, 0);
  } else {
    int t = 0;
    for (int jb = 0; jb < jobs; ++jb) {
      const KrylovJob& j = jb ? j1 : j0;
      const int cts = (j.q + 15) >> 4;
      for (int ct = 0; ct < cts; ++ct)
        for (int rt = 0; rt < 4; ++rt, ++t)
          if ((t & 3) == w) krylov_tile(sh.kb, j.mat, j.ic, j.oc, j.q, j.scale, rt, ct);
    }
  }
  __syncthreads();
}

// The next iteration's sketch, drawn while thread 0 fits alpha.
struct NextSketch {
  int on, k, stage, b;
};

// The products of one lane's four Krylov rows (rows 16 w + 4 g4 + r,
// column li < p) for the packed upper triangle of the J x J Gram: K_J from
// the lane's registers, K_1 .. K_{J-1} from LDS.
template <int J>
__device__ __forceinline__ void gram_rows(double (&gs)[16], const float* kb, const f32x4& kj,
                                          int w, int g4, int li, int p) {
#pragma unroll
  for (int e = 0; e < 16; ++e) gs[e] = 0.0;
  if (li >= p) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float* row = kb + (16 * w + 4 * g4 + r) * SKLD + li;
    double x[J];
#pragma unroll
    for (int j = 0; j + 1 < J; ++j) x[j] = (double)row[(j + 1) * p];
    x[J - 1] = (double)kj[r];
    int t = 0;
#pragma unroll
    for (int a = 0; a < J; ++a)
#pragma unroll
      for (int b = a; b < J; ++b, ++t) gs[t] += x[a] * x[b];
  }
}

// Krylov blocks of R (and R2), their Gram and alpha (d = 1 or 2), in the
// order and scaling of the multi-kernel path; alpha lands in sh.c.alpha.
__device__ void small_alpha(SmallShared& sh, const float* R, const float* R2, int n,
                            const IterCfg& cfg, const AlphaCoef& coef, NextSketch nx) {
  const int p = cfg.p, d = cfg.degree;
  const double fro = sh.c.fro;
  const float s1 = (float)(1.0 / fro), s2 = (float)(1.0 / (fro * fro));
  const int J = 2 * d + 1, NE = J * (J + 1) / 2;
  // the last Krylov block K_J: wave w's tile (rows 16 w .., q = p <= 16)
  KrylovJob last;
  if (d == 2) {
    // K1 = R S / s and K2 = R^2 S / s^2; [K3 | K4] = R^2 [K1 | K2] / s^2;
    // K5 = R^2 K3 / s^2
    krylov_step(sh, {R, 0, p, p, s1}, {R2, 0, 2 * p, p, s2}, 2);
    krylov_step(sh, {R2, p, 3 * p, 2 * p, s2}, {}, 1);
    last = {R2, 3 * p, 5 * p, p, s2};
  } else {
    for (int j = 1; j <= 2; ++j) krylov_step(sh, {R, (j - 1) * p, j * p, p, s1}, {}, 1);
    last = {R, 2 * p, 3 * p, p, s1};
  }
  // The last block and the Gram in one step (q = p <= PMX_MAX_SKETCH = 16:
  // one tile per wave): each wave adds the products of its own 16 rows (K_J
  // from its registers, the others from LDS) into 16 fp64 sums, halves them
  // over the wave and leaves one row of wave shares; entry e is then the
  // shares of waves 0..3 added in order.
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, li = lane & 15, g4 = lane >> 4;
  const f32x4 kj = krylov_tile(sh.kb, last.mat, last.ic, last.oc, last.q, last.scale, w, 0);
  double gs[16];
  if (J == 5) gram_rows<5>(gs, sh.kb, kj, w, g4, li, p);
  else gram_rows<3>(gs, sh.kb, kj, w, g4, li, p);
  halve_reduce_d<16, 32>(gs, lane);
  if ((lane & 3) == 0) sh.red[w][lane >> 2] = gs[0];
  __syncthreads();
  if (threadIdx.x < NE)
    sh.gsum[threadIdx.x] = ((sh.red[0][threadIdx.x] + sh.red[1][threadIdx.x]) +
                            sh.red[2][threadIdx.x]) + sh.red[3][threadIdx.x];
  __syncthreads();
  if (threadIdx.x == 0) {
    // d <= 2 here: J = 3 or 5 (no code for the degree-3 solve)
    const double alpha = J == 3 ? alpha_from_gram_t<3>(sh.gsum, fro, coef, cfg.lo, cfg.hi, nullptr)
                                : alpha_from_gram_t<5>(sh.gsum, fro, coef, cfg.lo, cfg.hi, nullptr);
    sh.c.alpha = alpha;
    sh.c.sketch_products += J;
    const int k = sh.c.iter;
    if (cfg.info && k < PMX_TRACE_LEN) cfg.info->alpha[sh.c.stage][k] = (float)alpha;
  } else if (nx.on && threadIdx.x >= 64) {
    // S_{k+1} into columns [0, p): the Krylov blocks no longer need S_k
    small_sketch(sh, n, p, nx.k, nx.stage, nx.b, cfg.seed_lo, cfg.seed_hi, 64);
  }
  __syncthreads();
}

// G = c0 I_n + c1 R + alpha R2 (d = 2) or c0 I_n + alpha R (d = 1), in place of R2.
__device__ void small_poly(float* G, const float* R, int n, int d, float c0, float c1,
                           float alpha) {
#pragma unroll
  for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / 4 / SNT; e += SNT, ++r_) {
    const int i = e >> 4, j0 = (e & 15) * 4;
    const float4 r4 = *reinterpret_cast<const float4*>(R + i * SLD + j0);
    const float4 g4 = *reinterpret_cast<const float4*>(G + i * SLD + j0);
    const float rv[4] = {r4.x, r4.y, r4.z, r4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w};
    float o[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      o[v] = (d == 2) ? c1 * rv[v] + alpha * gv[v] : alpha * rv[v];
      if (i == j0 + v && i < n) o[v] += c0;
    }
    *reinterpret_cast<float4*>(G + i * SLD + j0) = make_float4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();
}

__device__ void small_fill(float* M, int n, float diag) {
  #pragma unroll
  for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / SNT; e += SNT, ++r_) {
    const int i = e >> 6, j = e & 63;
    M[i * SLD + j] = (i == j && i < n) ? diag : 0.f;
  }
  __syncthreads();
}

// Control block and info at the start of a call (the reset of the
// multi-kernel path), then c = ||src||_F; status NONFINITE when c is not a
// positive finite number.
__device__ void small_start(SmallShared& sh, pmx_matfn_info* info, double fro2, int degree) {
  if (threadIdx.x == 0) {
    Ctrl c;
    c.c = sqrt(fro2);
    c.r_prev = 0.0;
    c.fro = 0.0;
    c.alpha = 0.0;
    c.inv_s = 0.0;
    c.status = PMX_RUNNING;
    c.status_all = PMX_CONVERGED;
    c.iter = 0;
    c.stage = 0;
    c.gemms = 0;
    c.sketch_products = 0;
    c.counter = 0u;
    c.degree = degree;
    c.degree_next = degree;
    c.pad = 0;
    if (!(c.c > 0.0) || !isfinite(c.c)) {
      c.status = PMX_NONFINITE;
      c.status_all = PMX_NONFINITE;
    }
    sh.c = c;
  }
  if (info) {
    int32_t* w = reinterpret_cast<int32_t*>(info);
    for (int i = threadIdx.x; i < (int)(sizeof(pmx_matfn_info) / 4); i += SNT) w[i] = 0;
  }
  for (int i = threadIdx.x; i < SN * SKLD; i += SNT) sh.kb[i] = 0.f;
  __syncthreads();
  if (threadIdx.x == 0 && info) {
    info->scale = (float)sh.c.c;
    if (sh.c.status == PMX_NONFINITE) info->status = PMX_NONFINITE;
  }
  __syncthreads();
}

__device__ __forceinline__ int32_t small_status(SmallShared& sh) {
  return *(volatile int32_t*)&sh.c.status;
}

__global__ __launch_bounds__(SNT, 1) void small_root_kernel(SmallRootParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SmallShared& sh = *reinterpret_cast<SmallShared*>(smem_raw);
  const int b = blockIdx.x;
  const int n = p.n;
  IterCfg cfg = p.cfg;
  if (cfg.info) cfg.info += b;
  const float* A = p.a + (int64_t)b * p.a_stride;
  float* Y = sh.m[0];
  float* Yn = sh.m[1];
  float* Z = sh.m[2];
  float* Zn = sh.m[3];
  float* R = sh.m[4];
  float* R2 = sh.m[5];
  // A into Y (zero padded) and ||A||_F; a thread's 16 loads are all in
  // flight before the first is used
  double acc = 0.0;
  {
    float v[SN * SN / SNT];
#pragma unroll
    for (int r = 0; r < SN * SN / SNT; ++r) {
      const int e = threadIdx.x + r * SNT, i = e >> 6, j = e & 63;
      v[r] = (i < n && j < n) ? A[(int64_t)i * p.lda + j] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < SN * SN / SNT; ++r) {
      const int e = threadIdx.x + r * SNT, i = e >> 6, j = e & 63;
      Y[i * SLD + j] = v[r];
      acc += (double)v[r] * (double)v[r];
    }
  }
  small_start(sh, cfg.info, block_total(acc, sh), cfg.degree);
  const bool accel = cfg.accelerate != 0;
  const int d = cfg.degree;
  for (int stage = 0; stage < p.stages; ++stage) {
    if (stage == 0) {
      if (small_status(sh) != PMX_RUNNING) break;
      const float fs = (float)(1.0 / sh.c.c);
      #pragma unroll
      for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / SNT; e += SNT, ++r_) {
        const int i = e >> 6, j = e & 63;
        Y[i * SLD + j] *= fs;
      }
    } else {
      const int prev = sh.c.status_all;
      if (prev == PMX_NONFINITE || prev == PMX_DIVERGED) break;
    }
    __syncthreads();
    // R_0 = I - Y_0 (Z_0 = I), the first sketch, the decision on r_0
    double f2 = 0.0;
    #pragma unroll
    for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / SNT; e += SNT, ++r_) {
      const int i = e >> 6, j = e & 63;
      const float rv = ((i == j && i < n) ? 1.f : 0.f) - Y[i * SLD + j];
      R[i * SLD + j] = rv;
      f2 += (double)rv * (double)rv;
    }
    small_fill(Z, n, 1.f);
    if (accel) small_sketch(sh, n, cfg.p, 0, stage, b, cfg.seed_lo, cfg.seed_hi);
    const double tot = block_total(f2, sh);
    if (threadIdx.x == 0) {
      sh.c.stage = stage;
      sh.c.iter = 0;
      sh.c.r_prev = 0.0;
      sh.c.status = PMX_RUNNING;
      decide(sh.c, cfg, cfg.info, tot);
    }
    __syncthreads();
    while (small_status(sh) == PMX_RUNNING) {
      const int k = sh.c.iter;
      if (d == 2) small_gemm<false, false>(R2, R, R, n, sh);
      if (accel) small_alpha(sh, R, R2, n, cfg, p.coef, {k + 1 < cfg.max_iter, k + 1, stage, b});
      // g in place of R2 (forming it while loading the two update products'
      // operands measured slower here: 2.1k cycles of this pass against 3.5k
      // more in the products; the polar kernel, with one product, forms it)
      small_poly(R2, R, n, d, p.c0, p.c1, (float)sh.c.alpha);
      small_gemm<false, false>(Yn, Y, R2, n, sh);  // Y g
      if (k == 0) {
        #pragma unroll
        for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / SNT; e += SNT, ++r_) {
          const int i = e >> 6, j = e & 63;
          Zn[i * SLD + j] = R2[i * SLD + j];  // Z_1 = g
        }
        __syncthreads();
      } else {
        small_gemm<false, false>(Zn, R2, Z, n, sh);  // g Z
      }
      float* t = Y;
      Y = Yn;
      Yn = t;
      t = Z;
      Z = Zn;
      Zn = t;
      const double f = small_gemm<false, true>(R, Z, Y, n, sh);  // I - Z Y
      if (threadIdx.x == 0) {
        sh.c.iter += 1;
        sh.c.gemms += (d - 1) + 1 + (k > 0 ? 1 : 0) + 1;
        decide(sh.c, cfg, cfg.info, f);
      }
      __syncthreads();
    }
  }
  // outputs: X = c^{-1/p} Z, X_aux = c^{1/p} Y; NaN when the call failed
  const int st = sh.c.status_all;
  const bool bad = (st == PMX_NONFINITE || st == PMX_DIVERGED);
  const double c = sh.c.c;
  const float sx = (float)pow(c, p.expo_x), sa = (float)pow(c, p.expo_aux);
  float* X = p.x + (int64_t)b * p.x_stride;
  float* XA = p.aux ? p.aux + (int64_t)b * p.aux_stride : nullptr;
  for (int e = threadIdx.x; e < n * n; e += SNT) {
    const int i = e / n, j = e - (e / n) * n;
    X[(int64_t)i * p.ldx + j] = bad ? NAN : Z[i * SLD + j] * sx;
    if (XA) XA[(int64_t)i * p.ldaux + j] = bad ? NAN : Y[i * SLD + j] * sa;
  }
}

__global__ __launch_bounds__(SNT, 1) void small_polar_kernel(SmallPolarParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SmallShared& sh = *reinterpret_cast<SmallShared*>(smem_raw);
  const int b = blockIdx.x;
  // the iterate X is rows x cols, rows >= cols (G^T when transpose)
  int rows = p.rows, cols = p.cols, transpose = p.transpose;
  const void* G = p.g + (int64_t)b * p.g_stride;
  void* Uo = p.u + (int64_t)b * p.u_stride;
  int64_t ldg = p.ldg, ldu = p.ldu;
  if (p.blocks) {
    const pmx_polar_block blk = p.blocks[b];
    // blocks above the fused order go through the batched path instead
    if (blk.m > SN || blk.n > SN) return;
    transpose = blk.m < blk.n;
    rows = transpose ? blk.n : blk.m;
    cols = transpose ? blk.m : blk.n;
    G = blk.g;
    Uo = blk.u;
    ldg = blk.ldg;
    ldu = blk.ldu;
  }
  auto load = [&](int64_t e) {
    return p.bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(G)[e] << 16)
                  : reinterpret_cast<const float*>(G)[e];
  };
  IterCfg cfg = p.cfg;
  cfg.n = cols;  // r_k = ||R_k||_F / sqrt(cols), per block
  if (cfg.info) cfg.info += b;
  float* X = sh.m[0];
  float* Xn = sh.m[1];
  float* R = sh.m[4];
  float* R2 = sh.m[5];
  double acc = 0.0;
  {
    float v[SN * SN / SNT];
#pragma unroll
    for (int r = 0; r < SN * SN / SNT; ++r) {
      const int e = threadIdx.x + r * SNT, i = e >> 6, j = e & 63;
      v[r] = (i < rows && j < cols)
                 ? (transpose ? load((int64_t)j * ldg + i) : load((int64_t)i * ldg + j))
                 : 0.f;
    }
#pragma unroll
    for (int r = 0; r < SN * SN / SNT; ++r) {
      const int e = threadIdx.x + r * SNT, i = e >> 6, j = e & 63;
      X[i * SLD + j] = v[r];
      acc += (double)v[r] * (double)v[r];
    }
  }
  small_start(sh, cfg.info, block_total(acc, sh), cfg.degree);
  const bool accel = cfg.accelerate != 0;
  const int d = cfg.degree;
  if (small_status(sh) == PMX_RUNNING) {
    const float fs = (float)(1.0 / sh.c.c);
    #pragma unroll
    for (int e = threadIdx.x, r_ = 0; r_ < SN * SN / SNT; e += SNT, ++r_) {
      const int i = e >> 6, j = e & 63;
      X[i * SLD + j] *= fs;
    }
    __syncthreads();
    // R_0 = I - X_0^T X_0 (a product), the first sketch, the decision on r_0
    const double f = small_gemm<true, true>(R, X, X, cols, sh);
    if (accel) small_sketch(sh, cols, cfg.p, 0, 0, b, cfg.seed_lo, cfg.seed_hi);
    if (threadIdx.x == 0) {
      sh.c.gemms += 1;
      decide(sh.c, cfg, cfg.info, f);
    }
    __syncthreads();
    while (small_status(sh) == PMX_RUNNING) {
      const int k = sh.c.iter;
      if (d == 2) small_gemm<false, false>(R2, R, R, cols, sh);
      if (accel) small_alpha(sh, R, R2, cols, cfg, p.coef, {k + 1 < cfg.max_iter, k + 1, 0, b});
      const SmallPoly pg{R, R2, p.c0, p.c1, (float)sh.c.alpha, d, cols};
      small_gemm<false, false, 2>(Xn, X, nullptr, cols, sh, &pg);  // X g, g formed on load
      float* t = X;
      X = Xn;
      Xn = t;
      const double f2 = small_gemm<true, true>(R, X, X, cols, sh);  // I - X^T X
      if (threadIdx.x == 0) {
        sh.c.iter += 1;
        sh.c.gemms += (d - 1) + 1 + 1;
        decide(sh.c, cfg, cfg.info, f2);
      }
      __syncthreads();
    }
  }
  const int st = sh.c.status_all;
  const bool bad = (st == PMX_NONFINITE || st == PMX_DIVERGED);
  for (int e = threadIdx.x; e < rows * cols; e += SNT) {
    const int i = e / cols, j = e - (e / cols) * cols;
    const float v = bad ? NAN : X[i * SLD + j];
    const int64_t o = transpose ? (int64_t)j * ldu + i : (int64_t)i * ldu + j;
    if (p.bf16) {
      reinterpret_cast<uint16_t*>(Uo)[o] = from_f32<bf16_t>(v).bits;  // nearest even
    } else {
      reinterpret_cast<float*>(Uo)[o] = v;
    }
  }
}

}  // namespace

size_t small_lds_bytes() { return sizeof(SmallShared); }

hipError_t launch_small_root(const SmallRootParams& p, int batch, hipStream_t s) {
  const size_t lds = sizeof(SmallShared);
  static_assert(sizeof(SmallShared) <= 160 * 1024, "LDS budget");
  hipError_t e = hipFuncSetAttribute((const void*)small_root_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(small_root_kernel, dim3(batch), dim3(SNT), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_small_polar(const SmallPolarParams& p, int batch, hipStream_t s) {
  const size_t lds = sizeof(SmallShared);
  hipError_t e = hipFuncSetAttribute((const void*)small_polar_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(small_polar_kernel, dim3(batch), dim3(SNT), lds, s, p);
  return hipGetLastError();
}

}  // namespace pmx
