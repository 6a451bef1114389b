// Internal declarations shared by the HIP translation units of libpmx.
// Device-side control state, kernel parameter blocks and launcher prototypes.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
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
  double inv_s;      // polar factor, estimated scale: 1 / s folded into the first g (0: none)
  int32_t status;    // PMX_RUNNING while the current stage iterates
  int32_t status_all;// worst outcome of the finished stages
  int32_t iter;      // updates done in the current stage
  int32_t stage;     // current stage (0 or 1)
  int32_t gemms;
  int32_t sketch_products;
  uint32_t counter;  // arrival counter of the last-block reductions
  int32_t degree;      // d of the current update (fixed, or the adaptive degree)
  int32_t degree_next; // d of the next update, taken over by decide()
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
  float taylor_d;  // c_d, the coefficient used when accelerate == 0
  int degree_max;  // > degree: adaptive degree (raised up to degree_max)
  float adapt_ratio;
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
  c.degree = c.degree_next;  // a raise decided by the last alpha fit starts here
  c.fro = sqrt(fro2);
  if (st == PMX_RUNNING && !cfg.accelerate) {
    c.alpha = cfg.taylor_d;
    if (info && k < PMX_TRACE_LEN) info->alpha[s][k] = cfg.taylor_d;
  }
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

// Sums of CNT doubles per lane over a 64-lane wave by recursive halving (CNT
// a power of two <= 64): at offset O the lanes with bit O set keep the upper
// half of their values and add the partner's copy of it, so CNT - 1 + log
// exchanges replace CNT full reductions; lane l ends with the wave's sum of
// value l / (64 / CNT) in acc[0].
template <int CNT, int O>
__device__ __forceinline__ void halve_reduce_d(double* acc, int lane) {
  if constexpr (O >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool upper = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const double send = upper ? acc[i] : acc[i + H];
        const double keep = upper ? acc[i + H] : acc[i];
        acc[i] = keep + __shfl_xor(send, O, 64);
      }
      halve_reduce_d<H, O / 2>(acc, lane);
    } else {
      acc[0] += __shfl_xor(acc[0], O, 64);
      halve_reduce_d<1, O / 2>(acc, lane);
    }
  }
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
// Gaussian sketch (shared by every kernel that generates it).
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies, high halves mixed with the other counter words and the key,
// key advanced by two Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// Where and which sketch to generate: S (n x p) of matrix b, stage, iteration
// k goes to columns [0, p) of the Krylov buffer (row stride kld).
struct SketchJob {
  float* kbuf;      // null: no sketch to generate
  int64_t kld, kstride;
  int n, p, k, stage;
  uint32_t seed_lo, seed_hi;
  int col;          // first column of the block written (0: the sketch S_k)
};

// The four standard normals of one Philox call's output words c[0..3]:
// uniforms ((x >> 8) + 1/2) 2^-24, Box-Muller on the word pairs (0,1) and
// (2,3), evaluated in fp64.
__device__ __forceinline__ void philox_normals(const uint32_t (&c)[4], double (&z)[4]) {
  double u[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) u[w] = ((double)(c[w] >> 8) + 0.5) * 0x1p-24;
  const double r01 = sqrt(-2.0 * log(u[0])), r23 = sqrt(-2.0 * log(u[2]));
  double s01, c01, s23, c23;
  sincos(2.0 * M_PI * u[1], &s01, &c01);
  sincos(2.0 * M_PI * u[3], &s23, &c23);
  z[0] = r01 * c01;
  z[1] = r01 * s01;
  z[2] = r23 * c23;
  z[3] = r23 * s23;
}

// Philox calls [q0, q1) of the sketch of matrix b: element e = i p + j takes
// word e % 4 of the call with counter (e / 4, k, stage, b), key = seed; its
// normal (philox_normals) is rounded to fp32.  One call per thread.
__device__ __forceinline__ void sketch_calls(const SketchJob& sj, int b, int64_t q0, int64_t q1) {
  const int64_t total = (int64_t)sj.n * sj.p;
  float* kb = sj.kbuf + (int64_t)b * sj.kstride;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += blockDim.x) {
    uint32_t c[4] = {(uint32_t)q, (uint32_t)sj.k, (uint32_t)sj.stage, (uint32_t)b};
    philox4x32_10(c, sj.seed_lo, sj.seed_hi);
    double z[4];
    philox_normals(c, z);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t e = q * 4 + w;
      if (e < total) {
        const int i = (int)(e / sj.p), j = (int)(e - (int64_t)i * sj.p);
        kb[(int64_t)i * sj.kld + sj.col + j] = (float)z[w];
      }
    }
  }
}

// This block's share [q0, q1) of the ceil(n p / 4) Philox calls when `nblocks`
// blocks split the sketch of one matrix.
__device__ __forceinline__ void sketch_share(const SketchJob& sj, int b, int blk, int nblocks) {
  if (!sj.kbuf) return;
  const int64_t calls = ((int64_t)sj.n * sj.p + 3) / 4;
  const int64_t per = (calls + nblocks - 1) / nblocks;
  const int64_t q0 = (int64_t)blk * per;
  const int64_t q1 = q0 + per < calls ? q0 + per : calls;
  if (q0 < q1) sketch_calls(sj, b, q0, q1);
}

// ---------------------------------------------------------------------------
// GEMM parameter block (fp32 MFMA kernel, row-major, optional transposes).
// The role selects the epilogue and gives every use its own kernel symbol:
enum Role : int {
  ROLE_POWER = 0,   // R^2 = R R                       (plain store)
  ROLE_UPDATE = 1,  // Y g, g Z, X g with g formed on the fly (plain store)
  ROLE_RESID = 2,   // R = I - Z Y or I - X^T X, ||R||_F, convergence decision
  ROLE_STATS = 3,   // C = beta C + (1 - beta) G G^T (or G^T G) + eps I, in place
  ROLE_APPLY = 4,   // L^{-1/4} G and (L^{-1/4} G) R^{-1/4}   (plain store)
};

struct GemmOperand {
  const float* ptr;
  int64_t ld;
  int64_t stride;    // batch stride in elements
  // polynomial operand g = c0 I + c1 R + alpha R2 (d = 2) or c0 I + alpha R
  // (d = 1), formed while loading: ptr = R, ptr2 = R2 (same ld / stride)
  const float* ptr2;
  int poly;
};

struct GemmProblem {
  GemmOperand a, b;
  float* c;
  int64_t ldc;
  int64_t stride_c;
};

// Most split-k workers (and per-tile counters) of one fp32 GEMM launch.
constexpr int kSplitMaxWorkers = 256;

struct GemmParams {
  GemmProblem prob[2];
  int nprob;       // problems per launch (the two updates Y g and g Z share one)
  int batch;
  int M, N, K;
  int tiles_m, tiles_n;
  int vec;         // 1: every operand allows 16-byte loads (and C 16-byte stores when sym)
  int max_blocks;  // persistent grid cap (0: one block per tile)
  int cfg_id;      // tile configuration (-1: chosen from the shape)
  int map_mode;    // tile order: 0 grouped, 1 grouped + XCD rounds, 2 row-major
  int dma;         // bf16: whole-tile variant with direct global-to-LDS loads
  int sym;         // output symmetric, upper-triangle tiles mirrored (M == N)
  int mn;          // bf16 residual: A and Bs given m- / n-contiguous (K x M, K x N)
  int sym_small;   // bf16 symmetric launches: 128 x 128 tiles instead of 256 x 256
  int persist;     // bf16 whole 256 x 256 tiles: persistent blocks, next tile's loads overlapped
  int early;       // bf16 persistent blocks: each k tile's loads issued before the previous tile's barrier
  int ragged_first; // fp32 split-k launches over ragged matrices: edge tiles first (set by the launcher)
  int num_cu;
  Ctrl* ctrl;      // per-matrix control blocks; null = unconditional
  // polynomial operands
  int degree;
  float c0, c1;
  // ROLE_STATS
  float beta, omb, eps;
  // ROLE_RESID
  double* partials;      // [batch][tiles]
  int64_t partial_stride;
  int products;          // dense products to add to ctrl.gemms on completion
  int count_update;      // 1: this residual ends an update (iter += 1)
  int resid_keep;        // 1: the residual also stores the product at prob[1].c
  IterCfg cfg;
  // matrices whose current degree is below min_degree skip the launch
  // (R^3 under the adaptive degree); 0: none
  int min_degree;
  // fp32 split-k tail (null sk_part: every item whole).  The caller provides
  // sk_cap floats of partial-tile slots and kSplitMaxWorkers zeroed per-tile
  // counters (each launch leaves them zero); the launcher fills in the split.
  float* sk_part;
  uint32_t* sk_cnt;
  int64_t sk_cap;
  int sk_dp, sk_rem, sk_workers;
};

hipError_t launch_gemm_f32(const GemmParams& p, bool ta, bool tb, int role, hipStream_t s);
// The convergence decision after a residual product: the product's blocks
// only store their tile's Frobenius share (partials[b][tile], no fence, no
// arrival counter); this kernel, launched right behind it by the GEMM
// launchers, sums the `tiles` shares of every running matrix in tile order
// (fixed order: deterministic), counts the products and the update and runs
// decide().  (A fenced last-block arrival in every tile of the product wrote
// back each XCD's L2 per tile: 65-190 us per launch on batches of small
// matrices.)
struct ResidDecide {
  Ctrl* ctrl;
  const double* partials;
  int64_t partial_stride;
  int tiles;         // shares per matrix
  int products;      // dense products to add to ctrl.gemms
  int count_update;  // 1: this residual ends an update (iter += 1)
  IterCfg cfg;
};
hipError_t launch_resid_decide(const ResidDecide& d, int batch, hipStream_t s);


// The HIP device a handle is bound to (-1 for a null handle).
int handle_device(pmx_handle h);
int gemm_f32_tiles(int M, int N);

}  // namespace pmx
