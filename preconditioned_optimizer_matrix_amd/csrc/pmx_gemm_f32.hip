// fp32 MFMA GEMM for gfx950: C = op(A) op(B) with fused epilogues.
//
// Every dense product of the PRISM Newton-Schulz iteration (the residual
// Z Y, the power R^2, the updates Y g and g Z, the Gram X^T X), of the
// Shampoo statistics (G G^T, G^T G) and of the preconditioned step
// (L^{-1/4} G R^{-1/4}) goes through this kernel.
//
// Design (CDNA4, 64-wide waves):
//  * block tile 128 x 128, k-tile 16, 256 threads = 4 waves in a 2 x 2
//    arrangement, each wave a 64 x 64 sub-tile made of 2 x 2
//    v_mfma_f32_32x32x2_f32 accumulators (64 fp32 accumulator registers).
//  * fp32 MFMA issues one 32x32x2 per 16 passes, so the kernel is bound by
//    matrix-core issue, not by LDS or HBM (arithmetic intensity of a
//    128 x 128 tile is 32 flop per byte of L2 traffic).
//  * Within a k-tile the 16 k values are distributed over the MFMA's two
//    k-lanes as k = 8 * (lane / 32) + step, so an operand stored with k
//    contiguous ("KC", e.g. A not transposed) is read as two 16-byte LDS loads
//    per lane, and an operand stored with m/n contiguous ("MC", e.g. B not
//    transposed) is staged without transposition and read with 4-byte loads
//    along consecutive rows (conflict-free).  Both layouts are written to LDS
//    with 16-byte stores straight from the 16-byte global loads.
//  * LDS is double buffered with a register prefetch of the next k-tile:
//    one barrier per k-tile.
//  * An operand may be the PRISM polynomial g = c0 I + c1 R + alpha R^2
//    (or c0 I + alpha R for d = 1), formed while its tile is loaded from R and
//    R^2, so g is never written to memory.
//  * Epilogues by role: plain store; residual R = I - acc with a deterministic
//    Frobenius reduction and the convergence decision (last block per matrix),
//    while the blocks also generate the next iteration's Gaussian sketch;
//    Shampoo EMA C = beta C + (1 - beta) acc + eps I in place.
#include "pmx_internal.h"

namespace pmx {
namespace {

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_EMA = 2 };

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int KC_LD = BK + 4;    // KC layout: [row][k], row stride 20 floats (80 B)
constexpr int MC_LD = BM + 4;    // MC layout: [k][row], row stride 132 floats
constexpr int NT = 256;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KC_FLOATS = BM * KC_LD;  // 2560
constexpr int MC_FLOATS = BK * MC_LD;  // 2112
constexpr int TILE_FLOATS = KC_FLOATS > MC_FLOATS ? KC_FLOATS : MC_FLOATS;

// Is the operand stored with k contiguous?  A (M x K view): not transposed.
// B (K x N view): transposed.
template <bool IS_A, bool TRANS>
struct Layout {
  static constexpr bool kc = IS_A ? !TRANS : TRANS;
};

// Polynomial operand constants for one block.
struct PolyCtx {
  float c0, c1, alpha;
  int degree;
};

// Global -> register prefetch of one 128 x 16 operand tile: two float4 per thread.
// KC: storage rows are the tile's m/n rows, 16 k values = 4 float4 per row.
// MC: storage rows are k, 128 m/n values = 32 float4 per row.
// With `poly` the element (i, j) of the stored matrix is
// c0 [i == j] + c1 R[i][j] + alpha R2[i][j] (d = 2) or c0 [i == j] + alpha R[i][j].
template <bool KCL>
__device__ __forceinline__ void load_tile(f32x4 (&r)[2], const float* __restrict__ base,
                                          const float* __restrict__ base2, bool poly,
                                          const PolyCtx& pc, int64_t ld, int row0, int nrows,
                                          int k0, int K, bool vec) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + NT * i;
    int srow, scol, lim_row, lim_col;
    if (KCL) {
      srow = row0 + (idx >> 2);
      scol = k0 + ((idx & 3) << 2);
      lim_row = nrows;
      lim_col = K;
    } else {
      srow = k0 + (idx >> 5);
      scol = row0 + ((idx & 31) << 2);
      lim_row = K;
      lim_col = nrows;
    }
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (srow < lim_row) {
      const int64_t off = (int64_t)srow * ld + scol;
      const float* src = base + off;
      const bool full = vec && scol + 3 < lim_col;
      if (!poly) {
        if (full) {
          v = *reinterpret_cast<const f32x4*>(src);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (scol + j < lim_col) v[j] = src[j];
        }
      } else {
        f32x4 r1 = {0.f, 0.f, 0.f, 0.f}, r2 = {0.f, 0.f, 0.f, 0.f};
        const float* src2 = base2 + off;
        if (full) {
          r1 = *reinterpret_cast<const f32x4*>(src);
          if (pc.degree == 2) r2 = *reinterpret_cast<const f32x4*>(src2);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (scol + j < lim_col) {
              r1[j] = src[j];
              if (pc.degree == 2) r2[j] = src2[j];
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float g = (pc.degree == 2) ? (pc.c1 * r1[j] + pc.alpha * r2[j]) : pc.alpha * r1[j];
          if (srow == scol + j) g += pc.c0;
          v[j] = (scol + j < lim_col) ? g : 0.f;
        }
      }
    }
    r[i] = v;
  }
}

template <bool KCL>
__device__ __forceinline__ void store_tile(float* __restrict__ lds, const f32x4 (&r)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = threadIdx.x + NT * i;
    float* dst;
    if (KCL) dst = lds + (idx >> 2) * KC_LD + ((idx & 3) << 2);
    else dst = lds + (idx >> 5) * MC_LD + ((idx & 31) << 2);
    *reinterpret_cast<f32x4*>(dst) = r[i];
  }
}

// Fragment of one 32-row (or 32-column) MFMA operand for the 8 k-steps of a
// k-tile: lane l supplies row (l % 32) at k = 8 * (l / 32) + step.
template <bool KCL>
__device__ __forceinline__ void read_frag(float (&f)[8], const float* __restrict__ lds,
                                          int row_base) {
  const int lane = threadIdx.x & 63;
  const int row = row_base + (lane & 31);
  const int kh = (lane >> 5) << 3;
  if (KCL) {
    const f32x4* p = reinterpret_cast<const f32x4*>(lds + row * KC_LD + kh);
    const f32x4 x0 = p[0], x1 = p[1];
    f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
    f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = lds[(kh + s) * MC_LD + row];
  }
}

template <bool TA, bool TB, int ROLE>
__global__ __launch_bounds__(NT, 2) void gemm_f32_kernel(GemmParams p) {
  constexpr int EPI = ROLE == ROLE_RESID ? EPI_RESID : (ROLE == ROLE_STATS ? EPI_EMA : EPI_STORE);
  const int z = blockIdx.z;
  const int pi = z % p.nprob;
  const int b = z / p.nprob;
  if (p.ctrl) {
    const int st = *(volatile int32_t*)&p.ctrl[b].status;
    if (st != PMX_RUNNING) return;
  }
  const GemmProblem& pr = p.prob[pi];
  const float* __restrict__ A = pr.a.ptr + (int64_t)b * pr.a.stride;
  const float* __restrict__ B = pr.b.ptr + (int64_t)b * pr.b.stride;
  float* __restrict__ C = pr.c + (int64_t)b * pr.stride_c;

  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  PolyCtx pc;
  pc.c0 = p.c0;
  pc.c1 = p.c1;
  pc.degree = p.degree;
  pc.alpha = (p.ctrl && (pr.a.poly || pr.b.poly)) ? (float)p.ctrl[b].alpha : 0.f;
  if (EPI == EPI_RESID) sketch_share(p.sketch, b, tile, gridDim.x);
  const int m0 = tm * BM, n0 = tn * BN;

  constexpr bool AKC = Layout<true, TA>::kc;
  constexpr bool BKC = Layout<false, TB>::kc;

  __shared__ __attribute__((aligned(16))) float smem[2][2][TILE_FLOATS];

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid >> 1) * 64, wn = (wid & 1) * 64;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const bool vec = p.vec != 0;
  const int nk = (p.K + BK - 1) / BK;
  f32x4 ra[2], rb[2];
  const float* __restrict__ A2 = pr.a.poly && pr.a.ptr2 ? pr.a.ptr2 + (int64_t)b * pr.a.stride : A;
  const float* __restrict__ B2 = pr.b.poly && pr.b.ptr2 ? pr.b.ptr2 + (int64_t)b * pr.b.stride : B;
  const bool apoly = pr.a.poly != 0, bpoly = pr.b.poly != 0;
  load_tile<AKC>(ra, A, A2, apoly, pc, pr.a.ld, m0, p.M, 0, p.K, vec);
  load_tile<BKC>(rb, B, B2, bpoly, pc, pr.b.ld, n0, p.N, 0, p.K, vec);
  store_tile<AKC>(smem[0][0], ra);
  store_tile<BKC>(smem[0][1], rb);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_tile<AKC>(ra, A, A2, apoly, pc, pr.a.ld, m0, p.M, (kt + 1) * BK, p.K, vec);
      load_tile<BKC>(rb, B, B2, bpoly, pc, pr.b.ld, n0, p.N, (kt + 1) * BK, p.K, vec);
    }
    float fa[2][8], fb[2][8];
#pragma unroll
    for (int i = 0; i < 2; ++i) read_frag<AKC>(fa[i], smem[cur][0], wm + 32 * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) read_frag<BKC>(fb[j], smem[cur][1], wn + 32 * j);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
    if (more) {
      store_tile<AKC>(smem[cur ^ 1][0], ra);
      store_tile<BKC>(smem[cur ^ 1][1], rb);
    }
    __syncthreads();
  }

  // Epilogue.  Lane l of a 32x32 accumulator holds column (l % 32) and rows
  // 8 * (v / 4) + 4 * (l / 32) + (v % 4), v = 0..15.
  const int hi = lane >> 5, col_in = lane & 31;
  float fro = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + 32 * j + col_in;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * hi + (v & 3);
        if (row < p.M && col < p.N) {
          float* dst = C + (int64_t)row * pr.ldc + col;
          float x = acc[i][j][v];
          if (EPI == EPI_RESID) {
            x = (row == col ? 1.f : 0.f) - x;
            fro += x * x;
          } else if (EPI == EPI_EMA) {
            x = p.beta * *dst + p.omb * x + (row == col ? p.eps : 0.f);
          }
          *dst = x;
        }
      }
    }

  if (EPI == EPI_RESID) {
    __shared__ double red[NT / 64];
    const double blocksum = block_sum<NT / 64>((double)fro, red);
    double total;
    const int nparts = p.tiles_m * p.tiles_n;
    if (last_block_sum<NT / 64>(blocksum, p.partials + (int64_t)b * p.partial_stride,
                                &p.ctrl[b].counter, nparts, tile, red, &total)) {
      if (threadIdx.x == 0) {
        Ctrl& c = p.ctrl[b];
        if (p.count_update) c.iter += 1;
        c.gemms += p.products;
        decide(c, p.cfg, p.cfg.info ? p.cfg.info + b : nullptr, total);
      }
    }
  }
}

#define PMX_GEMM_LAUNCH(TA, TB, ROLE) \
  hipLaunchKernelGGL((gemm_f32_kernel<TA, TB, ROLE>), grid, dim3(NT), 0, s, p)

}  // namespace

int gemm_f32_tiles(int M, int N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

// Instantiated combinations: every NN role, G G^T (NT) and G^T G / X^T X (TN).
hipError_t launch_gemm_f32(const GemmParams& pin, bool ta, bool tb, int role, hipStream_t s) {
  GemmParams p = pin;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  dim3 grid(p.tiles_m * p.tiles_n, 1, p.batch * p.nprob);
  if (!ta && !tb) {
    switch (role) {
      case ROLE_POWER: PMX_GEMM_LAUNCH(false, false, ROLE_POWER); break;
      case ROLE_UPDATE: PMX_GEMM_LAUNCH(false, false, ROLE_UPDATE); break;
      case ROLE_RESID: PMX_GEMM_LAUNCH(false, false, ROLE_RESID); break;
      case ROLE_APPLY: PMX_GEMM_LAUNCH(false, false, ROLE_APPLY); break;
      default: return hipErrorInvalidValue;
    }
  } else if (!ta && tb) {
    if (role != ROLE_STATS) return hipErrorInvalidValue;
    PMX_GEMM_LAUNCH(false, true, ROLE_STATS);
  } else if (ta && !tb) {
    switch (role) {
      case ROLE_STATS: PMX_GEMM_LAUNCH(true, false, ROLE_STATS); break;
      case ROLE_RESID: PMX_GEMM_LAUNCH(true, false, ROLE_RESID); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pmx
