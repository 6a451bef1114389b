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
//  * The control block lives in LDS; thread 0 applies decide() and the
//    alpha fit, a barrier publishes the outcome.
#include "pmx_alpha.h"
#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr int SN = 64;    // padded order
constexpr int SLD = 68;   // LDS row stride (floats)
constexpr int SMAT = SN * SLD;
constexpr int SNT = 256;
constexpr int SKLD = 6 * 16;  // Krylov buffer row stride: (2d + 2) p <= 96

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
template <bool TA, bool RESID>
__device__ double small_gemm(float* C, const float* A, const float* B, int n_id,
                             SmallShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
  const int li = lane & 31, kh = (lane >> 5) * 32;
  f32x16 acc;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = 0.f;
  const float* bcol = B + kh * SLD + wn + li;
  if (TA) {
    const float* acol = A + kh * SLD + wm + li;
#pragma unroll
    for (int m = 0; m < 32; ++m)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(acol[m * SLD], bcol[m * SLD], acc, 0, 0, 0);
  } else {
    const float* arow = A + (wm + li) * SLD + kh;
#pragma unroll
    for (int m4 = 0; m4 < 8; ++m4) {
      const float4 a = *reinterpret_cast<const float4*>(arow + 4 * m4);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bcol[(4 * m4 + 0) * SLD], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, bcol[(4 * m4 + 1) * SLD], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, bcol[(4 * m4 + 2) * SLD], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, bcol[(4 * m4 + 3) * SLD], acc, 0, 0, 0);
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
__device__ void small_sketch(SmallShared& sh, int n, int p, int k, int stage, int b,
                             uint32_t seed_lo, uint32_t seed_hi) {
  const int calls = (n * p + 3) / 4;
  for (int q = threadIdx.x; q < calls; q += SNT) {
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

// out cols [oc, oc + q) = scale * Mat * in cols [ic, ic + q) (n x n Mat; rows
// of the Krylov buffer beyond n are zero, so the sum runs over 64).  Thread t
// owns row t / 4 and columns 4 (t % 4) + 16 h .. + 3.
__device__ void small_skinny(SmallShared& sh, const float* mat, int n, int q, int ic, int oc,
                             float scale) {
  const int i = threadIdx.x >> 2, cg = (threadIdx.x & 3) * 4;
  const bool vec = ((q | ic | oc) & 3) == 0;
  for (int h = 0; h < q; h += 16) {
    const int c = h + cg;
    if (c >= q) break;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
#pragma unroll 16
      for (int j = 0; j < SN; ++j) {
        const float a = mat[i * SLD + j];
        const float4 x = *reinterpret_cast<const float4*>(sh.kb + j * SKLD + ic + c);
        acc[0] += a * x.x;
        acc[1] += a * x.y;
        acc[2] += a * x.z;
        acc[3] += a * x.w;
      }
    } else {
#pragma unroll 8
      for (int j = 0; j < SN; ++j) {
        const float a = mat[i * SLD + j];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (c + v < q) acc[v] += a * sh.kb[j * SKLD + ic + c + v];
      }
    }
    if (i < n) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (c + v < q) sh.kb[i * SKLD + oc + c + v] = acc[v] * scale;
    }
  }
  __syncthreads();
}

// Krylov blocks of R (and R2), their Gram and alpha (d = 1 or 2), in the
// order and scaling of the multi-kernel path; alpha lands in sh.c.alpha.
__device__ void small_alpha(SmallShared& sh, const float* R, const float* R2, int n,
                            const IterCfg& cfg, const AlphaCoef& coef) {
  const int p = cfg.p, d = cfg.degree;
  const double fro = sh.c.fro;
  const float s1 = (float)(1.0 / fro), s2 = (float)(1.0 / (fro * fro));
  if (d == 2) {
    small_skinny(sh, R, n, p, 0, p, s1);           // K1 = R S / s
    small_skinny(sh, R2, n, p, 0, 2 * p, s2);      // K2 = R^2 S / s^2
    small_skinny(sh, R2, n, 2 * p, p, 3 * p, s2);  // [K3 | K4] = R^2 [K1 | K2] / s^2
    small_skinny(sh, R2, n, p, 3 * p, 5 * p, s2);  // K5 = R^2 K3 / s^2
  } else {
    for (int j = 1; j <= 3; ++j) small_skinny(sh, R, n, p, (j - 1) * p, j * p, s1);
  }
  const int J = 2 * d + 1;
  double g[15];
#pragma unroll
  for (int e = 0; e < 15; ++e) g[e] = 0.0;
  for (int e = threadIdx.x; e < n * p; e += SNT) {
    const int i = e / p, c = e - (e / p) * p;
    double v[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int a = 0; a < 5; ++a)
      if (a < J) v[a] = (double)sh.kb[i * SKLD + (a + 1) * p + c];
    int t = 0;
#pragma unroll
    for (int a = 0; a < 5; ++a)
#pragma unroll
      for (int bb = a; bb < 5; ++bb, ++t) g[t] += v[a] * v[bb];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  {
    int t = 0, o = 0;
#pragma unroll
    for (int a = 0; a < 5; ++a)
#pragma unroll
      for (int bb = a; bb < 5; ++bb, ++t) {
        const double sv = wave_sum(g[t]);
        if (a < J && bb < J) {
          if (lane == 0) sh.red[w][o] = sv;
          ++o;
        }
      }
  }
  __syncthreads();
  if (threadIdx.x < J * (J + 1) / 2) {
    const int e = threadIdx.x;
    sh.gsum[e] = ((sh.red[0][e] + sh.red[1][e]) + sh.red[2][e]) + sh.red[3][e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const double alpha = alpha_from_gram(sh.gsum, J, fro, coef, cfg.lo, cfg.hi);
    sh.c.alpha = alpha;
    sh.c.sketch_products += J;
    const int k = sh.c.iter;
    if (cfg.info && k < PMX_TRACE_LEN) cfg.info->alpha[sh.c.stage][k] = (float)alpha;
  }
  __syncthreads();
}

// G = c0 I_n + c1 R + alpha R2 (d = 2) or c0 I_n + alpha R (d = 1), in place of R2.
__device__ void small_poly(float* G, const float* R, int n, int d, float c0, float c1,
                           float alpha) {
  for (int e = threadIdx.x; e < SN * SN; e += SNT) {
    const int i = e >> 6, j = e & 63;
    const float rv = R[i * SLD + j];
    float v = (d == 2) ? c1 * rv + alpha * G[i * SLD + j] : alpha * rv;
    if (i == j && i < n) v += c0;
    G[i * SLD + j] = v;
  }
  __syncthreads();
}

__device__ void small_fill(float* M, int n, float diag) {
  for (int e = threadIdx.x; e < SN * SN; e += SNT) {
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
  // A into Y (zero padded) and ||A||_F
  double acc = 0.0;
  for (int e = threadIdx.x; e < SN * SN; e += SNT) {
    const int i = e >> 6, j = e & 63;
    float v = 0.f;
    if (i < n && j < n) v = A[(int64_t)i * p.lda + j];
    Y[i * SLD + j] = v;
    acc += (double)v * (double)v;
  }
  small_start(sh, cfg.info, block_total(acc, sh), cfg.degree);
  const bool accel = cfg.accelerate != 0;
  const int d = cfg.degree;
  for (int stage = 0; stage < p.stages; ++stage) {
    if (stage == 0) {
      if (small_status(sh) != PMX_RUNNING) break;
      const float fs = (float)(1.0 / sh.c.c);
      for (int e = threadIdx.x; e < SN * SN; e += SNT) {
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
    for (int e = threadIdx.x; e < SN * SN; e += SNT) {
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
      if (accel) small_alpha(sh, R, R2, n, cfg, p.coef);
      small_poly(R2, R, n, d, p.c0, p.c1, (float)sh.c.alpha);
      small_gemm<false, false>(Yn, Y, R2, n, sh);  // Y g
      if (k == 0) {
        for (int e = threadIdx.x; e < SN * SN; e += SNT) {
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
      if (accel && k + 1 < cfg.max_iter)
        small_sketch(sh, n, cfg.p, k + 1, stage, b, cfg.seed_lo, cfg.seed_hi);
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
  for (int e = threadIdx.x; e < SN * SN; e += SNT) {
    const int i = e >> 6, j = e & 63;
    float v = 0.f;
    if (i < rows && j < cols) v = transpose ? load((int64_t)j * ldg + i) : load((int64_t)i * ldg + j);
    X[i * SLD + j] = v;
    acc += (double)v * (double)v;
  }
  small_start(sh, cfg.info, block_total(acc, sh), cfg.degree);
  const bool accel = cfg.accelerate != 0;
  const int d = cfg.degree;
  if (small_status(sh) == PMX_RUNNING) {
    const float fs = (float)(1.0 / sh.c.c);
    for (int e = threadIdx.x; e < SN * SN; e += SNT) {
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
      if (accel) small_alpha(sh, R, R2, cols, cfg, p.coef);
      small_poly(R2, R, cols, d, p.c0, p.c1, (float)sh.c.alpha);
      small_gemm<false, false>(Xn, X, R2, cols, sh);  // X g
      float* t = X;
      X = Xn;
      Xn = t;
      const double f2 = small_gemm<true, true>(R, X, X, cols, sh);  // I - X^T X
      if (accel && k + 1 < cfg.max_iter)
        small_sketch(sh, cols, cfg.p, k + 1, 0, b, cfg.seed_lo, cfg.seed_hi);
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
