// bf16 MFMA GEMM for gfx950 (bf16 operands, fp32 accumulation), used by the
// bf16 polar-factor iteration.  Every operand is stored with k contiguous:
//   C[i][j] = sum_k A[i][k] * Bs[j][k]
// (A is M x K, Bs is N x K, both row-major bf16).  The polar iteration keeps a
// transposed copy X^T of its iterate and writes R, R^T and g^T in bf16 with a
// tile-transpose kernel, so its three products all take this form:
//   R  = I - X^T X : A = X^T, Bs = X^T
//   R2 = R R       : A = R,   Bs = R^T
//   X' = X g       : A = X,   Bs = g^T   (the epilogue also writes X'^T)
//
// Design (CDNA4):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) and 8 consecutive
//    k values 8 (l / 32) .. +7 of a 16-wide k step: one 16-byte LDS read per
//    fragment.  LDS rows are padded to 72 bf16 (144 bytes) so the 16-byte
//    reads of 8 consecutive rows hit distinct banks.
//  * Block tile 128 x 128 x 64, 4 waves (64 x 64 each, 2 x 2 accumulators),
//    16-byte global loads straight into 16-byte LDS stores, LDS double
//    buffered with a register prefetch, persistent grid over (matrix, tile).
//  * fp32 -> bf16 rounding is round-to-nearest-even.
#include "pmx_kernels.h"

namespace pmx {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int LDK = BK + 8;      // bf16 per LDS row (144 bytes)
constexpr int TILE = 128 * LDK;  // bf16 per operand tile
constexpr int CHUNKS = 128 * BK / 8 / NT;  // 16-byte chunks per thread per operand (4)

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// One 128 x 64 operand tile: chunk idx -> (row idx / 8, k 8 (idx % 8)).
__device__ __forceinline__ void load_chunks(u32x4 (&v)[CHUNKS], const uint16_t* base, int64_t ld,
                                            int row0, int nrows, int k0, int K, bool vec) {
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int idx = threadIdx.x + NT * i;
    const int row = row0 + (idx >> 3);
    const int k = k0 + ((idx & 7) << 3);
    u32x4 out = {0u, 0u, 0u, 0u};
    if (row < nrows) {
      const uint16_t* b = base + (int64_t)row * ld + k;
      if (vec && k + 7 < K) {
        out = *reinterpret_cast<const u32x4*>(b);
      } else {
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = (k + j < K) ? b[j] : 0u;
        out = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    }
    v[i] = out;
  }
}

__device__ __forceinline__ void store_chunks(uint16_t* lds, const u32x4 (&v)[CHUNKS]) {
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int idx = threadIdx.x + NT * i;
    *reinterpret_cast<u32x4*>(lds + (idx >> 3) * LDK + ((idx & 7) << 3)) = v[i];
  }
}

// Tiles of a matrix in groups of 8 tile-rows per column sweep.
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

// ROLE_RESID: C fp32 = I - acc with the Frobenius reduction and decision;
// ROLE_POWER: C fp32 = acc; ROLE_UPDATE: C bf16 = acc and, at ptr2 of the
// output descriptor (prob[1].c), its transpose.
template <int ROLE>
__global__ __launch_bounds__(NT, 2) void gemm_bf16_kernel(GemmParams p) {
  constexpr bool RESID = ROLE == ROLE_RESID;
  constexpr bool BF16_OUT = ROLE == ROLE_UPDATE;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][TILE];
  __shared__ double red[NT / 64];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = (wid >> 1) * 64, wn = (wid & 1) * 64;
  const bool vec = p.vec != 0;
  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch;
  const GemmProblem& pr = p.prob[0];

  for (int it = blockIdx.x; it < total; it += gridDim.x) {
    int b, tm, tn, tile;
    item_tile(it, p.tiles_m, p.tiles_n, &b, &tm, &tn, &tile);
    if (p.ctrl) {
      const int st = *(volatile int32_t*)&p.ctrl[b].status;
      if (st != PMX_RUNNING) continue;
    }
    const uint16_t* A = reinterpret_cast<const uint16_t*>(pr.a.ptr) + (int64_t)b * pr.a.stride;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(pr.b.ptr) + (int64_t)b * pr.b.stride;
    if (RESID) sketch_share(p.sketch, b, tile, tiles);
    const int m0 = tm * BM, n0 = tn * BN;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    u32x4 va[CHUNKS], vb[CHUNKS];
    const int nk = (p.K + BK - 1) / BK;
    __syncthreads();
    load_chunks(va, A, pr.a.ld, m0, p.M, 0, p.K, vec);
    load_chunks(vb, B, pr.b.ld, n0, p.N, 0, p.K, vec);
    store_chunks(smem[0][0], va);
    store_chunks(smem[0][1], vb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        load_chunks(va, A, pr.a.ld, m0, p.M, (kt + 1) * BK, p.K, vec);
        load_chunks(vb, B, pr.b.ld, n0, p.N, (kt + 1) * BK, p.K, vec);
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
        store_chunks(smem[cur ^ 1][0], va);
        store_chunks(smem[cur ^ 1][1], vb);
      }
      __syncthreads();
    }

    // Epilogue (same accumulator layout as the 32x32 fp32 MFMA: lane l holds
    // column l % 32 and rows 8 (v / 4) + 4 (l / 32) + (v % 4)).
    const int hi = lane >> 5, col_in = lane & 31;
    float fro = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn + 32 * j + col_in;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row_base = m0 + wm + 32 * i + 8 * g + 4 * hi;
          uint32_t h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row_base + r;
            float x = acc[i][j][4 * g + r];
            if (RESID) {
              x = (row == col ? 1.f : 0.f) - x;
              if (row < p.M && col < p.N) fro += x * x;
            }
            if (row < p.M && col < p.N) {
              const int64_t o = (int64_t)b * pr.stride_c + (int64_t)row * pr.ldc + col;
              if (BF16_OUT) reinterpret_cast<uint16_t*>(pr.c)[o] = (uint16_t)bf16_rne(x);
              else pr.c[o] = x;
            }
            h[r] = bf16_rne(x);
          }
          if (BF16_OUT && col < p.N) {
            // transposed copy: X'^T[col][row_base .. row_base + 3]
            const GemmProblem& tp = p.prob[1];
            uint16_t* T = reinterpret_cast<uint16_t*>(tp.c) + (int64_t)b * tp.stride_c +
                          (int64_t)col * tp.ldc + row_base;
            if (p.vec && row_base + 3 < p.M) {
              *reinterpret_cast<u32x2*>(T) = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (row_base + r < p.M) T[r] = (uint16_t)h[r];
            }
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

// C = A Bs^T with A (M x K) and Bs (N x K) bf16, k contiguous.  Roles:
// ROLE_RESID (C fp32 = I - A Bs^T, convergence), ROLE_POWER (C fp32),
// ROLE_UPDATE (C bf16 and its transpose at prob[1].c / ldc / stride_c).
hipError_t launch_gemm_bf16(const GemmParams& pin, int role, hipStream_t s) {
  GemmParams p = pin;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const int64_t total = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  int64_t g = total;
  if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
  const dim3 grid((unsigned)g), block(NT);
  switch (role) {
    case ROLE_RESID: hipLaunchKernelGGL((gemm_bf16_kernel<ROLE_RESID>), grid, block, 0, s, p); break;
    case ROLE_POWER: hipLaunchKernelGGL((gemm_bf16_kernel<ROLE_POWER>), grid, block, 0, s, p); break;
    case ROLE_UPDATE: hipLaunchKernelGGL((gemm_bf16_kernel<ROLE_UPDATE>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pmx
