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
// GEMM on the fp64 matrix cores (v_mfma_f64_16x16x4_f64): block tiles of
// BT x BT (64 by default, 128 on request), 256 threads in 2 x 2
// waves of (BT/2)^2, each wave holding (BT/32)^2 16 x 16 accumulators; k
// tiles of 16 staged through LDS with both operands stored k-major (A is
// transposed on the LDS store), double buffered with a register prefetch of
// the next k tile: one barrier per k tile.  The symmetric products (R^2 and
// the residual I - Z Y, Z Y = Z A Z^T) run the upper-triangle tiles only and
// store each off-diagonal tile twice.
#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr int TK = 16, NT = 256;

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32_t load_status(const Ctrl* c) {
  return *(const volatile int32_t*)&c->status;
}

// (tile row, tile column) of tile t: full grids row-major, symmetric
// launches the upper triangle row by row
__device__ __forceinline__ void tile_of(int t, int T, bool sym, int& tm, int& tn) {
  if (!sym) {
    tm = t / T;
    tn = t - tm * T;
    return;
  }
  int r = 0;
  while (t >= T - r) {
    t -= T - r;
    ++r;
  }
  tm = r;
  tn = r + t;
}

template <int BT, int ROLE>
__global__ __launch_bounds__(NT) void gemm_f64_kernel(Gemm64Params p) {
  constexpr bool RESID = ROLE == ROLE_RESID;
  constexpr int WT = BT / 2, F = WT / 16, LDT = BT + 2;
  constexpr int PER = BT * TK / NT;  // elements of each operand tile per thread
  const int n = p.n;
  const int T = (n + BT - 1) / BT;
  const bool sym = p.sym != 0;
  const int tiles = sym ? T * (T + 1) / 2 : T * T;
  const int pi = blockIdx.y;  // problem
  const int b = blockIdx.z;
  const int tile = blockIdx.x;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const Gemm64Problem& pr = p.prob[pi];
  const int64_t base = (int64_t)b * p.stride;
  if (RESID) sketch_share(p.sketch, b, tile, tiles);
  int tm, tn;
  tile_of(tile, T, sym, tm, tn);
  const int m0 = tm * BT, n0 = tn * BT;
  __shared__ double As[2][TK][LDT];  // As[k][i] = A[m0 + i][k0 + k]
  __shared__ double Bs[2][TK][LDT];  // Bs[k][j] = B[k0 + k][n0 + j]
  __shared__ double red[NT / 64];
  const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
  const int wm = (wid >> 1) * WT, wn = (wid & 1) * WT;
  const double* __restrict__ A = pr.a.p + base;
  const double* __restrict__ B = pr.b.p + base;
  f64x4 acc[F][F];
#pragma unroll
  for (int u = 0; u < F; ++u)
#pragma unroll
    for (int v = 0; v < F; ++v) acc[u][v] = f64x4{0.0, 0.0, 0.0, 0.0};
  double ra[PER], rb[PER];
  // A: element e = t + NT q -> row e / TK, k e % TK (16 lanes per 128-byte
  // row); B: k e / BT, column e % BT
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + NT * q;
      const int ai = e / TK, ak = e % TK, gi = m0 + ai, gk = k0 + ak;
      ra[q] = (gi < n && gk < n) ? A[(int64_t)gi * n + gk] : 0.0;
      const int bk = e / BT, bj = e % BT, hk = k0 + bk, hj = n0 + bj;
      rb[q] = (hk < n && hj < n) ? B[(int64_t)hk * n + hj] : 0.0;
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + NT * q;
      As[buf][e % TK][e / TK] = ra[q];
      Bs[buf][e / BT][e % BT] = rb[q];
    }
  };
  const int nk = (n + TK - 1) / TK;
  load(0);
  store(0);
  __syncthreads();
  const int li = lane & 15, lk = lane >> 4;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * TK);
#pragma unroll
    for (int ks = 0; ks < TK; ks += 4) {
      double fa[F], fb[F];
#pragma unroll
      for (int u = 0; u < F; ++u) fa[u] = As[cur][ks + lk][wm + 16 * u + li];
#pragma unroll
      for (int v = 0; v < F; ++v) fb[v] = Bs[cur][ks + lk][wn + 16 * v + li];
#pragma unroll
      for (int u = 0; u < F; ++u)
#pragma unroll
        for (int v = 0; v < F; ++v)
          acc[u][v] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[u], fb[v], acc[u][v], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  // lane l of a 16 x 16 fp64 accumulator holds column l % 16 and rows
  // l / 16 + 4 r, r = 0 .. 3 (checked on the device; the fp32 16 x 16 MFMA
  // holds rows 4 (l / 16) + r instead)
  const bool mirror = sym && tm != tn;
  float* c32 = pr.c32 ? pr.c32 + (int64_t)b * p.stride32 : nullptr;
  double* C = pr.c + base;
  double fro = 0.0;
#pragma unroll
  for (int u = 0; u < F; ++u)
#pragma unroll
    for (int v = 0; v < F; ++v) {
      const int j = n0 + wn + 16 * v + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = m0 + wm + 16 * u + lk + 4 * r;
        double x = acc[u][v][r];
        if (RESID) x = (i == j ? 1.0 : 0.0) - x;
        if (i < n && j < n) {
          if (RESID) fro += x * x;
          C[(int64_t)i * n + j] = x;
          if (c32) c32[(int64_t)i * n + j] = (float)x;
          if (mirror) {
            // the transposed tile: C[j][i]
            C[(int64_t)j * n + i] = x;
            if (c32) c32[(int64_t)j * n + i] = (float)x;
          }
        }
      }
    }
  if (RESID) {
    // the tile's Frobenius share; resid_decide_kernel sums them
    if (mirror) fro *= 2.0;  // the tile stands for itself and its transpose
    const double bs = block_sum<NT / 64>(fro, red);
    if (threadIdx.x == 0) p.partials[(int64_t)b * p.partial_stride + tile] = bs;
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

template <int BT>
hipError_t launch_gemm_f64_bt(const Gemm64Params& p, int role, hipStream_t s) {
  const int T = (p.n + BT - 1) / BT;
  const dim3 grid(p.sym ? T * (T + 1) / 2 : T * T, p.nprob, p.batch);
  switch (role) {
    case ROLE_POWER: hipLaunchKernelGGL((gemm_f64_kernel<BT, ROLE_POWER>), grid, dim3(NT), 0, s, p); break;
    case ROLE_UPDATE: hipLaunchKernelGGL((gemm_f64_kernel<BT, ROLE_UPDATE>), grid, dim3(NT), 0, s, p); break;
    case ROLE_RESID: hipLaunchKernelGGL((gemm_f64_kernel<BT, ROLE_RESID>), grid, dim3(NT), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || role != ROLE_RESID) return e;
  ResidDecide d;
  d.ctrl = p.ctrl;
  d.partials = p.partials;
  d.partial_stride = p.partial_stride;
  d.tiles = (int)grid.x;
  d.products = p.products;
  d.count_update = p.count_update;
  d.cfg = p.cfg;
  return launch_resid_decide(d, p.batch, s);
}

hipError_t launch_gemm_f64(const Gemm64Params& p, int role, hipStream_t s) {
  // 64 x 64 tiles by default: four blocks per CU fit in registers (the
  // 128 x 128 tile holds one), and on the 64 x 512^2 blocks the fp64 leading
  // updates took 20.2 ms against 21.9 ms with 128 x 128 tiles
  const int bt = p.tile > 0 ? p.tile : 64;
  return bt == 128 ? launch_gemm_f64_bt<128>(p, role, s) : launch_gemm_f64_bt<64>(p, role, s);
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
