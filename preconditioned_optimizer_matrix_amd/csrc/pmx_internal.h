// Internal declarations shared by the HIP translation units of libpmx.
// Device-side control state, kernel parameter blocks and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pmx.h"

namespace pmx {

// ---------------------------------------------------------------------------
// Per-matrix control block, resident in the workspace.  Written only by the
// library's kernels; every iteration kernel reads `status` first and returns
// at once when the matrix's current stage has finished, so the host can
// enqueue all iterations up front and never wait for the device.
struct Ctrl {
  double c;          // input scale ||A||_F (or ||G||_F)
  double r_prev;     // r_{k-1}
  double fro;        // ||R_k||_F of the current residual (Krylov scaling)
  double alpha;      // alpha_k of the current update
  int32_t status;    // PMX_RUNNING while the current stage iterates
  int32_t status_all;// worst outcome of the finished stages
  int32_t iter;      // updates done in the current stage
  int32_t stage;     // current stage (0 or 1)
  int32_t gemms;
  int32_t sketch_products;
  uint32_t counter;  // arrival counter of the last-block reductions
  int32_t pad;
};

// Static configuration of one iterative call (host-filled, passed by value).
struct IterCfg {
  int n;           // order of the residual matrix
  int degree;      // d
  int p;           // sketch width
  int max_iter;
  int accelerate;
  float lo, hi, tol;
  uint32_t seed_lo, seed_hi;
  pmx_matfn_info* info;  // may be null
};

constexpr double kDivergeLevel = 2.0;
constexpr double kStagLevel = 1e-2;
constexpr double kStagFactor = 0.9;

__device__ __forceinline__ int severity(int s) {
  switch (s) {
    case PMX_CONVERGED: return 0;
    case PMX_STAGNATED: return 1;
    case PMX_MAXITER: return 2;
    case PMX_DIVERGED: return 3;
    default: return 4;  // NONFINITE
  }
}

// Stopping rule applied to r_k = ||R_k||_F / sqrt(n) at the start of update k
// (k = c.iter).  Same order of tests as the fp64 reference iteration:
// non-finite, converged, diverged, stagnated, iteration limit.
__device__ __forceinline__ void decide(Ctrl& c, const IterCfg& cfg, pmx_matfn_info* info,
                                       double fro2) {
  const double r = sqrt(fro2 / (double)cfg.n);
  const int k = c.iter;
  const int s = c.stage;
  int st = PMX_RUNNING;
  if (!isfinite(r)) st = PMX_NONFINITE;
  else if (r <= (double)cfg.tol) st = PMX_CONVERGED;
  else if (r > kDivergeLevel) st = PMX_DIVERGED;
  else if (k >= 1 && c.r_prev < kStagLevel && r > kStagFactor * c.r_prev) st = PMX_STAGNATED;
  else if (k >= cfg.max_iter) st = PMX_MAXITER;
  if (info && k < PMX_TRACE_LEN) info->rtrace[s][k] = (float)r;
  c.r_prev = r;
  c.fro = sqrt(fro2);
  if (st != PMX_RUNNING) {
    if (severity(st) > severity(c.status_all)) c.status_all = st;
    if (info) {
      info->iters[s] = k;
      info->residual[s] = (float)r;
      info->status = c.status_all;
      info->gemms = c.gemms;
      info->sketch_products = c.sketch_products;
      info->stages = s + 1;
    }
  }
  c.status = st;
}

// ---------------------------------------------------------------------------
// Wave (64-lane) and block reductions in fp64, fixed order (deterministic).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Sum over a block of `nwaves` waves; result valid in every thread.
template <int NWAVES>
__device__ __forceinline__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) lds[wid] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) t += lds[w];
  return t;
}

// Last-block-arrives pattern: every block stores its partial, the last block
// (per matrix) to arrive sums them in index order.  Returns true in the
// whole last block; `total` is then valid in every thread of it.
template <int NWAVES>
__device__ __forceinline__ bool last_block_sum(double my_partial, double* partials,
                                               uint32_t* counter, int nparts, int part,
                                               double* lds, double* total) {
  __shared__ int is_last;
  if (threadIdx.x == 0) {
    partials[part] = my_partial;
    __threadfence();
    const uint32_t prev = atomicAdd(counter, 1u);
    is_last = (prev == (uint32_t)(nparts - 1));
  }
  __syncthreads();
  if (!is_last) return false;
  __threadfence();
  double v = 0.0;
  for (int i = threadIdx.x; i < nparts; i += NWAVES * 64)
    v += __hip_atomic_load(&partials[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  *total = block_sum<NWAVES>(v, lds);
  if (threadIdx.x == 0) *counter = 0u;
  return true;
}

// ---------------------------------------------------------------------------
// GEMM parameter block (fp32 MFMA kernel, row-major, optional transposes).
enum Epi : int {
  EPI_STORE = 0,  // C = acc
  EPI_RESID = 1,  // C = I - acc, then ||C||_F^2 -> convergence decision
  EPI_EMA = 2,    // C = beta C + (1 - beta) acc + eps I (in place)
};

struct GemmOperand {
  const float* ptr;
  int64_t ld;
  int64_t stride;  // batch stride in elements
};

struct GemmProblem {
  GemmOperand a, b;
  float* c;
  int64_t ldc;
  int64_t stride_c;
};

struct GemmParams {
  GemmProblem prob[2];
  int nprob;       // problems per launch (the two updates Y g and g Z share one)
  int batch;
  int M, N, K;
  int tiles_m, tiles_n;
  int vec;         // 1: every operand allows 16-byte loads
  Ctrl* ctrl;      // per-matrix control blocks; null = unconditional
  // EPI_EMA
  float beta, omb, eps;
  // EPI_RESID
  double* partials;      // [batch][tiles]
  int64_t partial_stride;
  int products;          // dense products to add to ctrl.gemms on completion
  int count_update;      // 1: this residual ends an update (iter += 1)
  IterCfg cfg;
};

hipError_t launch_gemm_f32(const GemmParams& p, bool ta, bool tb, int epi, hipStream_t s);

}  // namespace pmx
