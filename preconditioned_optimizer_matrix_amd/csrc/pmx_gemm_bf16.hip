// bf16 MFMA GEMM for gfx950 (bf16 operands, fp32 accumulation), used by the
// bf16 polar-factor iteration: R = I - X^T X (bf16 X), R^2 (fp32 R rounded to
// bf16 on load) and X <- X g (g = c0 I + c1 R + alpha R^2 formed from fp32 R
// and R^2 while loading, rounded to bf16; bf16 output).
//
// Design (CDNA4):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) and 8
//    consecutive k values 8 (l / 32) .. +7 of a 16-wide k step, so every
//    operand lives in LDS as [row][k] with k contiguous and a fragment is one
//    16-byte LDS read.
//  * Block tile 128 x 128 x 64, 4 waves (64 x 64 each, 2 x 2 accumulators),
//    LDS double buffered with a register prefetch, persistent grid.
//  * Operands stored with k contiguous are copied 8 k values at a time.
//    Operands stored with m/n contiguous (X^T in X^T X, the right operand of
//    every product here) are transposed in registers: each thread loads a
//    4 (k) x 8 (m/n) block and writes eight 8-byte rows of 4 k values; the
//    thread -> block mapping keeps consecutive threads on consecutive k so
//    the LDS writes are conflict-free.
//  * fp32 -> bf16 rounding is round-to-nearest-even everywhere.
#include "pmx_kernels.h"

namespace pmx {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int LDK = BK + 8;          // bf16 per LDS row (144 bytes)
constexpr int TILE = 128 * LDK;      // bf16 per operand tile

enum : int { ST_F32 = 0, ST_BF16 = 1 };

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

struct Poly {
  float c0, c1, alpha;
  int degree;
  int on;
};

// Element value of an fp32-stored operand at storage (row, col), with the
// PRISM polynomial applied when requested.
__device__ __forceinline__ float f32_elem(const float* base, const float* base2, int64_t off,
                                          int row, int col, const Poly& pc) {
  if (!pc.on) return base[off];
  float g = pc.degree == 2 ? pc.c1 * base[off] + pc.alpha * base2[off] : pc.alpha * base[off];
  if (row == col) g += pc.c0;
  return g;
}

// ------------------------------------------------------------ KC operand
// Storage rows = tile rows (m or n), k contiguous.  Tile 128 x 64 = 1024
// chunks of 8 k values, 4 per thread; each chunk becomes one 16-byte LDS row
// segment.
template <int ST>
struct KCLoad {
  u32x4 v[4];
  __device__ __forceinline__ void load(const void* basev, const float* base2, const Poly& pc,
                                       int64_t ld, int row0, int nrows, int k0, int K,
                                       bool vec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + NT * i;
      const int row = row0 + (idx >> 3);
      const int k = k0 + ((idx & 7) << 3);
      u32x4 out = {0u, 0u, 0u, 0u};
      if (row < nrows) {
        const int64_t off = (int64_t)row * ld + k;
        if (ST == ST_BF16) {
          const uint16_t* b = reinterpret_cast<const uint16_t*>(basev) + off;
          if (vec && k + 7 < K) {
            out = *reinterpret_cast<const u32x4*>(b);
          } else {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = (k + j < K) ? b[j] : 0u;
            out = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
          }
        } else {
          const float* b = reinterpret_cast<const float*>(basev);
          float f[8];
          if (vec && k + 7 < K && !pc.on) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(b + off);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(b + off + 4);
            f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
            f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              f[j] = (k + j < K) ? f32_elem(b, base2, off + j, row, k + j, pc) : 0.f;
          }
          out = {pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
        }
      }
      v[i] = out;
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + NT * i;
      *reinterpret_cast<u32x4*>(lds + (idx >> 3) * LDK + ((idx & 7) << 3)) = v[i];
    }
  }
};

// ------------------------------------------------------------ MC operand
// Storage rows = k, contiguous along the tile rows.  Each thread loads a
// 4 (k) x 8 (tile rows) block: k block kb = tid % 16, row block cb = tid / 16.
template <int ST>
struct MCLoad {
  u32x2 v[8];  // per tile row j: 4 bf16 (k0..k0+3)
  __device__ __forceinline__ void load(const void* basev, const float* base2, const Poly& pc,
                                       int64_t ld, int row0, int nrows, int k0, int K,
                                       bool vec) {
    const int kb = threadIdx.x & 15, cb = threadIdx.x >> 4;
    const int kk = k0 + kb * 4;
    const int c0 = row0 + cb * 8;
    uint32_t h[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = kk + r;
#pragma unroll
      for (int j = 0; j < 8; ++j) h[r][j] = 0u;
      if (k < K) {
        const int64_t off = (int64_t)k * ld + c0;
        if (ST == ST_BF16) {
          const uint16_t* b = reinterpret_cast<const uint16_t*>(basev) + off;
          if (vec && c0 + 7 < nrows) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(b);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              h[r][2 * q] = x[q] & 0xFFFFu;
              h[r][2 * q + 1] = x[q] >> 16;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) h[r][j] = (c0 + j < nrows) ? b[j] : 0u;
          }
        } else {
          const float* b = reinterpret_cast<const float*>(basev);
          float f[8];
          if (vec && c0 + 7 < nrows && !pc.on) {
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(b + off);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(b + off + 4);
            f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
            f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
          } else if (vec && c0 + 7 < nrows) {
            // polynomial operand, vector loads of R and R^2
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(b + off);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(b + off + 4);
            f32x4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
            if (pc.degree == 2) {
              y0 = *reinterpret_cast<const f32x4*>(base2 + off);
              y1 = *reinterpret_cast<const f32x4*>(base2 + off + 4);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float r1 = j < 4 ? x0[j] : x1[j - 4];
              const float r2 = j < 4 ? y0[j] : y1[j - 4];
              float g = pc.degree == 2 ? pc.c1 * r1 + pc.alpha * r2 : pc.alpha * r1;
              if (k == c0 + j) g += pc.c0;
              f[j] = g;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
              f[j] = (c0 + j < nrows) ? f32_elem(b, base2, off + j, k, c0 + j, pc) : 0.f;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) h[r][j] = bf16_rne(f[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = {h[0][j] | (h[1][j] << 16), h[2][j] | (h[3][j] << 16)};
  }
  __device__ __forceinline__ void store(uint16_t* lds) const {
    const int kb = threadIdx.x & 15, cb = threadIdx.x >> 4;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x2*>(lds + (cb * 8 + j) * LDK + kb * 4) = v[j];
  }
};

template <bool KC, int ST>
struct Loader;
template <int ST>
struct Loader<true, ST> : KCLoad<ST> {};
template <int ST>
struct Loader<false, ST> : MCLoad<ST> {};

// Work item -> (matrix z, tile m, tile n): tiles of a matrix in groups of 8
// tile-rows per column sweep.
__device__ __forceinline__ void item_tile(int it, int tiles_m, int tiles_n, int* z, int* tm,
                                          int* tn, int* tile) {
  const int tiles = tiles_m * tiles_n;
  *z = it / tiles;
  const int t = it - *z * tiles;
  *tile = t;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in_group = t - group * per_group;
  *tm = first_m + in_group % gsize;
  *tn = in_group / gsize;
}

// A: (AKC ? stored M x K : stored K x M), storage AST; B: (BKC ? stored N x K :
// stored K x N), storage BST; C: M x N, fp32 (OST = ST_F32) or bf16.
template <bool AKC, int AST, bool BKC, int BST, int OST, int ROLE>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmParams p) {
  constexpr bool RESID = ROLE == ROLE_RESID;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][TILE];
  __shared__ double red[NT / 64];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = (wid >> 1) * 64, wn = (wid & 1) * 64;
  const bool vec = p.vec != 0;
  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch;

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    int b, tm, tn, tile;
    item_tile(it, p.tiles_m, p.tiles_n, &b, &tm, &tn, &tile);
    if (p.ctrl) {
      const int st = *(volatile int32_t*)&p.ctrl[b].status;
      if (st != PMX_RUNNING) continue;
    }
    const GemmProblem& pr = p.prob[0];
    const void* A = AST == ST_BF16
                        ? (const void*)(reinterpret_cast<const uint16_t*>(pr.a.ptr) + (int64_t)b * pr.a.stride)
                        : (const void*)(pr.a.ptr + (int64_t)b * pr.a.stride);
    const void* B = BST == ST_BF16
                        ? (const void*)(reinterpret_cast<const uint16_t*>(pr.b.ptr) + (int64_t)b * pr.b.stride)
                        : (const void*)(pr.b.ptr + (int64_t)b * pr.b.stride);
    const float* A2 = pr.a.ptr2 ? pr.a.ptr2 + (int64_t)b * pr.a.stride : nullptr;
    const float* B2 = pr.b.ptr2 ? pr.b.ptr2 + (int64_t)b * pr.b.stride : nullptr;
    Poly pa, pb;
    pa.c0 = pb.c0 = p.c0;
    pa.c1 = pb.c1 = p.c1;
    pa.degree = pb.degree = p.degree;
    const float alpha = (p.ctrl && (pr.a.poly || pr.b.poly)) ? (float)p.ctrl[b].alpha : 0.f;
    pa.alpha = pb.alpha = alpha;
    pa.on = pr.a.poly;
    pb.on = pr.b.poly;
    if (RESID) sketch_share(p.sketch, b, tile, tiles);
    const int m0 = tm * BM, n0 = tn * BN;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    Loader<AKC, AST> la;
    Loader<BKC, BST> lb;
    const int nk = (p.K + BK - 1) / BK;
    __syncthreads();
    la.load(A, A2, pa, pr.a.ld, m0, p.M, 0, p.K, vec);
    lb.load(B, B2, pb, pr.b.ld, n0, p.N, 0, p.K, vec);
    la.store(smem[0][0]);
    lb.store(smem[0][1]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(A, A2, pa, pr.a.ld, m0, p.M, (kt + 1) * BK, p.K, vec);
        lb.load(B, B2, pb, pr.b.ld, n0, p.N, (kt + 1) * BK, p.K, vec);
      }
      const uint16_t* sa = smem[cur][0];
      const uint16_t* sb = smem[cur][1];
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        const int kofs = s * 16 + (lane >> 5) * 8;
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          fa[i] = *reinterpret_cast<const bf16x8*>(sa + (wm + 32 * i + (lane & 31)) * LDK + kofs);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          fb[j] = *reinterpret_cast<const bf16x8*>(sb + (wn + 32 * j + (lane & 31)) * LDK + kofs);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (more) {
        la.store(smem[cur ^ 1][0]);
        lb.store(smem[cur ^ 1][1]);
      }
      __syncthreads();
    }

    // Epilogue (same accumulator layout as the 32x32 fp32 MFMA).
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
            float x = acc[i][j][v];
            if (RESID) {
              x = (row == col ? 1.f : 0.f) - x;
              fro += x * x;
            }
            const int64_t o = (int64_t)b * pr.stride_c + (int64_t)row * pr.ldc + col;
            if (OST == ST_BF16) reinterpret_cast<uint16_t*>(pr.c)[o] = (uint16_t)bf16_rne(x);
            else pr.c[o] = x;
          }
        }
      }
    if (RESID) {
      const double blocksum = block_sum<NT / 64>((double)fro, red);
      double tot;
      if (last_block_sum<NT / 64>(blocksum, p.partials + (int64_t)b * p.partial_stride,
                                  &p.ctrl[b].counter, tiles, tile, red, &tot)) {
        if (threadIdx.x == 0) {
          Ctrl& c = p.ctrl[b];
          if (p.count_update) c.iter += 1;
          c.gemms += p.products;
          decide(c, p.cfg, p.cfg.info ? p.cfg.info + b : nullptr, tot);
        }
      }
    }
  }
}

}  // namespace

// The three products of the bf16 polar iteration:
//   ROLE_RESID : R = I - X^T X   (A = X^T: X stored K x M bf16, B = X stored K x N bf16)
//   ROLE_POWER : R2 = R R        (A = R stored M x K fp32, B = R stored K x N fp32)
//   ROLE_UPDATE: X' = X g        (A = X stored M x K bf16, B = g from R, R2 stored K x N fp32;
//                                 output bf16)
hipError_t launch_gemm_bf16(const GemmParams& pin, int role, hipStream_t s) {
  GemmParams p = pin;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int64_t total = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  int64_t g = total;
  if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
  const dim3 grid((unsigned)g), block(NT);
  switch (role) {
    case ROLE_RESID:
      hipLaunchKernelGGL((gemm_bf16_kernel<false, ST_BF16, false, ST_BF16, ST_F32, ROLE_RESID>),
                         grid, block, 0, s, p);
      break;
    case ROLE_POWER:
      hipLaunchKernelGGL((gemm_bf16_kernel<true, ST_F32, false, ST_F32, ST_F32, ROLE_POWER>),
                         grid, block, 0, s, p);
      break;
    case ROLE_UPDATE:
      hipLaunchKernelGGL((gemm_bf16_kernel<true, ST_BF16, false, ST_F32, ST_BF16, ROLE_UPDATE>),
                         grid, block, 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pmx
