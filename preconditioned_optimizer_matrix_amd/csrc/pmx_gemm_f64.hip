// fp64 kernels for the leading updates of an inverse root (pmx_matfn_opts
// fp64_iters): with condition numbers near 1e6 the rounding committed by
// fp32 products in the first updates of a stage, while g is far from I and Z
// grows towards A^{-1/2}, stays in the result (the coupled iteration does not
// damp it); running those updates in fp64 and the rest in fp32 brings the
// result back under 1e-4.  Same steps and control flow as the fp32 path:
// square products only, the polynomial operand formed on load, the residual
// epilogue with the Frobenius reduction and the decision, fp32 copies of R
// and R^2 for the Krylov kernels.
//
// GEMM: 64 x 64 tiles, 256 threads with 4 x 4 fp64 accumulators each, k tiles
// of 16 staged through LDS (A transposed so both operands are read along
// rows), fp64 FMA on the vector ALUs (the gfx950 fp64 vector and matrix rates
// are equal).
#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr int TN = 64, TK = 16, NT = 256;

__device__ __forceinline__ int32_t load_status(const Ctrl* c) {
  return *(const volatile int32_t*)&c->status;
}

// element (i, j) of a plain or polynomial operand
__device__ __forceinline__ double operand(const Gemm64Operand& o, int64_t off, int i, int j,
                                          double c0, double c1, double alpha, int degree) {
  if (!o.poly) return o.p[off];
  const double r = o.p[off];
  double g = degree == 2 ? c1 * r + alpha * o.p2[off] : alpha * r;
  if (i == j) g += c0;
  return g;
}

template <int ROLE>
__global__ __launch_bounds__(NT) void gemm_f64_kernel(Gemm64Params p) {
  constexpr bool RESID = ROLE == ROLE_RESID;
  const int n = p.n;
  const int tiles_1d = (n + TN - 1) / TN;
  const int tiles = tiles_1d * tiles_1d;
  const int pi = blockIdx.y;  // problem
  const int b = blockIdx.z;
  const int tile = blockIdx.x;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const Gemm64Problem& pr = p.prob[pi];
  const int64_t base = (int64_t)b * p.stride;
  if (RESID) sketch_share(p.sketch, b, tile, tiles);
  const double alpha = cb->alpha;
  const int m0 = (tile / tiles_1d) * TN, n0 = (tile % tiles_1d) * TN;
  __shared__ double As[TK][TN + 1];  // As[k][i] = A[m0 + i][k0 + k]
  __shared__ double Bs[TK][TN + 1];  // Bs[k][j] = B[k0 + k][n0 + j]
  __shared__ double red[NT / 64];
  const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int k0 = 0; k0 < n; k0 += TK) {
    // A tile 64 x 16 and B tile 16 x 64: four elements of each per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int idx = t + NT * q;
      const int ai = idx >> 4, ak = idx & 15;  // A: row ai, k ak
      const int gi = m0 + ai, gk = k0 + ak;
      double av = 0.0;
      if (gi < n && gk < n)
        av = operand(pr.a, base + (int64_t)gi * n + gk, gi, gk, p.c0, p.c1, alpha, p.degree);
      As[ak][ai] = av;
      const int bk = idx >> 6, bj = idx & 63;  // B: k bk, column bj
      const int hk = k0 + bk, hj = n0 + bj;
      double bv = 0.0;
      if (hk < n && hj < n)
        bv = operand(pr.b, base + (int64_t)hk * n + hj, hk, hj, p.c0, p.c1, alpha, p.degree);
      Bs[bk][bj] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      double a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] = As[k][ty * 4 + u];
#pragma unroll
      for (int v = 0; v < 4; ++v) bb[v] = Bs[k][tx * 4 + v];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(a[u], bb[v], acc[u][v]);
    }
    __syncthreads();
  }
  double fro = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = m0 + ty * 4 + u;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = n0 + tx * 4 + v;
      if (i < n && j < n) {
        double x = acc[u][v];
        if (RESID) {
          x = (i == j ? 1.0 : 0.0) - x;
          fro += x * x;
        }
        const int64_t o = base + (int64_t)i * n + j;
        pr.c[o] = x;
        if (pr.c32) pr.c32[(int64_t)b * p.stride32 + (int64_t)i * n + j] = (float)x;
      }
    }
  }
  if (RESID) {
    const double bs = block_sum<NT / 64>(fro, red);
    double tot;
    if (last_block_sum<NT / 64>(bs, p.partials + (int64_t)b * p.partial_stride, &cb->counter,
                                tiles, tile, red, &tot)) {
      if (threadIdx.x == 0) {
        if (p.count_update) cb->iter += 1;
        cb->gemms += p.products;
        decide(*cb, p.cfg, p.cfg.info ? p.cfg.info + b : nullptr, tot);
      }
    }
  }
}

// Stage set-up in fp64: Y_0 = scale * src (src fp32: A, or the previous
// stage's Y), R_0 = I - Y_0 (and its fp32 copy), the decision on r_0 and the
// first sketch.  The control flow is that of the fp32 set-up.
__global__ __launch_bounds__(NT) void stage_init_f64_kernel(StageInit64Params p) {
  const int b = blockIdx.y;
  Ctrl* cb = p.ctrl + b;
  if (p.stage == 0) {
    if (load_status(cb) != PMX_RUNNING) return;
  } else {
    const int prev = *(const volatile int32_t*)&cb->status_all;
    if (prev == PMX_NONFINITE || prev == PMX_DIVERGED) return;
  }
  sketch_share(p.sketch, b, blockIdx.x, gridDim.x);
  const int n = p.n;
  double scale;
  const float* src;
  int64_t sld;
  if (p.stage == 0) {
    scale = 1.0 / cb->c;
    src = p.a + (int64_t)b * p.a_stride;
    sld = p.lda;
  } else {
    scale = 1.0;
    const int it = *(const volatile int32_t*)&cb->iter;
    src = p.ybuf32[it & 1] + (int64_t)b * p.stride32;
    sld = n;
  }
  double* y0 = p.y64 + (int64_t)b * p.stride;
  double* R = p.r64 + (int64_t)b * p.stride;
  float* R32 = p.r32 + (int64_t)b * p.stride32;
  double acc = 0.0;
  for (int r = blockIdx.x; r < n; r += gridDim.x)
  for (int c = threadIdx.x; c < n; c += NT) {
    const int64_t e = (int64_t)r * n + c;
    const double y = (double)src[(int64_t)r * sld + c] * scale;
    y0[e] = y;
    const double rv = (r == c ? 1.0 : 0.0) - y;
    R[e] = rv;
    R32[e] = (float)rv;
    acc += rv * rv;
  }
  __shared__ double red[NT / 64];
  const double bs = block_sum<NT / 64>(acc, red);
  double tot;
  if (last_block_sum<NT / 64>(bs, p.partials + (int64_t)b * p.partial_stride, &cb->counter,
                              gridDim.x, blockIdx.x, red, &tot)) {
    if (threadIdx.x == 0) {
      cb->stage = p.stage;
      cb->iter = 0;
      cb->r_prev = 0.0;
      cb->status = PMX_RUNNING;
      cb->degree_next = p.cfg.degree;
      decide(*cb, p.cfg, p.cfg.info ? p.cfg.info + b : nullptr, tot);
    }
  }
}

// Z_1 = g = c0 I + c1 R + alpha R^2 (d = 2) or c0 I + alpha R, in fp64.
__global__ __launch_bounds__(NT) void form_g_f64_kernel(FormG64Params p) {
  const int b = blockIdx.y;
  const Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const double alpha = cb->alpha;
  const int n = p.n;
  const double* R = p.r + (int64_t)b * p.stride;
  const double* R2 = p.r2 ? p.r2 + (int64_t)b * p.stride : nullptr;
  double* G = p.dst + (int64_t)b * p.stride;
  for (int r = blockIdx.x; r < n; r += gridDim.x)
  for (int c = threadIdx.x; c < n; c += NT) {
    const int64_t e = (int64_t)r * n + c;
    double v = p.degree == 1 ? alpha * R[e] : p.c1 * R[e] + alpha * R2[e];
    if (r == c) v += p.c0;
    G[e] = v;
  }
}

// Hand-over to fp32 after the fp64 updates of a stage: Y and Z of the
// current parity (iter & 1) rounded into the fp32 ping-pong buffers.  Runs
// whenever the stage was entered, whether or not it is still iterating.
__global__ __launch_bounds__(NT) void handover_f64_kernel(Handover64Params p) {
  const int b = blockIdx.y;
  const Ctrl* cb = p.ctrl + b;
  if (*(const volatile int32_t*)&cb->stage != p.stage) return;
  const int st = *(const volatile int32_t*)&cb->status_all;
  if (st == PMX_NONFINITE || st == PMX_DIVERGED) return;
  const int it = *(const volatile int32_t*)&cb->iter;
  const int n = p.n;
  const double* Y = p.y64[it & 1] + (int64_t)b * p.stride;
  const double* Z = p.z64[it & 1] + (int64_t)b * p.stride;
  float* Y32 = p.y32[it & 1] + (int64_t)b * p.stride32;
  float* Z32 = p.z32[it & 1] + (int64_t)b * p.stride32;
  for (int r = blockIdx.x; r < n; r += gridDim.x)
  for (int c = threadIdx.x; c < n; c += NT) {
    const int64_t e = (int64_t)r * n + c;
    Y32[e] = (float)Y[e];
    if (it > 0) Z32[e] = (float)Z[e];
  }
}


}  // namespace

hipError_t launch_gemm_f64(const Gemm64Params& p, int role, hipStream_t s) {
  const int t1 = (p.n + TN - 1) / TN;
  const dim3 grid(t1 * t1, p.nprob, p.batch);
  switch (role) {
    case ROLE_POWER: hipLaunchKernelGGL(gemm_f64_kernel<ROLE_POWER>, grid, dim3(NT), 0, s, p); break;
    case ROLE_UPDATE: hipLaunchKernelGGL(gemm_f64_kernel<ROLE_UPDATE>, grid, dim3(NT), 0, s, p); break;
    case ROLE_RESID: hipLaunchKernelGGL(gemm_f64_kernel<ROLE_RESID>, grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_stage_init_f64(const StageInit64Params& p, int batch, hipStream_t s) {
  dim3 grid(blocks_per_matrix(p.n, batch, 1024, kPartialsPerMatrix), batch);
  hipLaunchKernelGGL(stage_init_f64_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_form_g_f64(const FormG64Params& p, int batch, hipStream_t s) {
  dim3 grid(blocks_per_matrix(p.n, batch, 4096, 2048), batch);
  hipLaunchKernelGGL(form_g_f64_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_handover_f64(const Handover64Params& p, int batch, hipStream_t s) {
  dim3 grid(blocks_per_matrix(p.n, batch, 4096, 2048), batch);
  hipLaunchKernelGGL(handover_f64_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace pmx
