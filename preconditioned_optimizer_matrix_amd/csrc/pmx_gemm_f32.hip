// fp32 MFMA GEMM for gfx950: C = op(A) op(B) with fused epilogues.
//
// Every dense product of the PRISM Newton-Schulz iteration (the residual
// Z Y, the power R^2, the updates Y g and g Z, the Gram X^T X), of the
// Shampoo statistics (G G^T, G^T G) and of the preconditioned step
// (L^{-1/4} G R^{-1/4}) goes through this kernel.
//
// Design (CDNA4, 64-wide waves):
//  * A block tile of BM x BN is split over WGM x WGN waves; every wave owns a
//    (BM/WGM) x (BN/WGN) sub-tile made of 32 x 32 v_mfma_f32_32x32x2_f32
//    accumulators.  fp32 MFMA issues one 32x32x2 per 16 passes, so the
//    kernel is bound by matrix-core issue: a 128 x 128 tile already moves only
//    1/32 byte of L2 traffic per flop.
//  * Within a k-tile of BK values the k index is distributed over the MFMA's
//    two k-lanes as k = (BK/2) * (lane / 32) + step, so an operand stored
//    with k contiguous ("KC", e.g. A not transposed) is read as 16-byte LDS
//    loads, and an operand stored with m/n contiguous ("MC", e.g. B not
//    transposed) is staged without transposition and read with 4-byte loads
//    along consecutive rows.  Both layouts are written to LDS with 16-byte
//    stores straight from 16-byte global loads.
//  * LDS is double buffered with a register prefetch of the next k-tile:
//    one barrier per k-tile.
//  * Persistent grid: at most `max_blocks` blocks loop over (matrix, tile)
//    items, so launches of matrices that have already converged dispatch
//    few workgroups.  Items follow a grouped order (8 tile-rows per column
//    sweep) for L2 reuse.
//  * An operand may be the PRISM polynomial g = c0 I + c1 R + alpha R^2
//    (or c0 I + alpha R for d = 1), formed while its tile is loaded from R and
//    R^2, so g is never written to memory.
//  * Epilogues by role: plain store; residual R = I - acc with a deterministic
//    Frobenius reduction and the convergence decision (last tile per matrix);
//    Shampoo EMA C = beta C + (1 - beta) acc + eps I in place.
//  * Symmetric products (R^2, the residuals Z A Z^T and X^T X, the statistics
//    Grams G G^T and G^T G): with `sym` only the tiles on and above the
//    diagonal are computed and each off-diagonal tile is also stored
//    transposed, about half the products' work.  The statistics' EMA reads
//    the mirrored elements' own old values, so L and R need not be symmetric.
#include <algorithm>
#include <type_traits>

#include "pmx_internal.h"

namespace pmx {
namespace {

enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_EMA = 2 };

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tile configuration: block tile BM x BN x BK over WGM x WGN waves, at least
// MINW waves resident per SIMD (bounds the registers per wave), STAGES LDS
// buffers (2: double buffered, one barrier per k-tile; 1: single buffer with
// the register prefetch written after a second barrier).
template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int MINW_, int STAGES_ = 2>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_, MINW = MINW_;
  static constexpr int STAGES = STAGES_;
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  static constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 accumulators per wave
  static constexpr int KH = BK / 2;                     // k values per MFMA k-lane
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BK % 16 == 0, "k tile");
};

// LDS floats of one operand tile of `rows` (m or n) x BK in layout KC or MC.
template <class C, bool KCL, int ROWS>
struct OpTile {
  static constexpr int LD = KCL ? C::BK + 4 : ROWS + 4;
  static constexpr int FLOATS = KCL ? ROWS * LD : C::BK * LD;
  static constexpr int VEC = ROWS * C::BK / 4;  // float4 per tile
  static constexpr int PER_THREAD = VEC / C::NT;
  static_assert(VEC % C::NT == 0, "tile load split");
};

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

// Global -> register prefetch of one ROWS x BK operand tile.
// KC: storage rows are the tile's m/n rows (BK/4 float4 per row).
// MC: storage rows are k (ROWS/4 float4 per row).
// With `poly` the element (i, j) of the stored matrix is
// c0 [i == j] + c1 R[i][j] + alpha R2[i][j] (d = 2) or c0 [i == j] + alpha R[i][j].
template <class C, bool KCL, int ROWS, int NV>
__device__ __forceinline__ void load_tile(f32x4 (&r)[NV],
                                          const float* __restrict__ base,
                                          const float* __restrict__ base2, bool poly,
                                          const PolyCtx& pc, int64_t ld, int row0, int nrows,
                                          int k0, int K, bool vec) {
  static_assert(NV == OpTile<C, KCL, ROWS>::PER_THREAD, "prefetch registers");
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + C::NT * i;
    int srow, scol, lim_row, lim_col;
    if (KCL) {
      srow = row0 + idx / (C::BK / 4);
      scol = k0 + (idx % (C::BK / 4)) * 4;
      lim_row = nrows;
      lim_col = K;
    } else {
      srow = k0 + idx / (ROWS / 4);
      scol = row0 + (idx % (ROWS / 4)) * 4;
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

template <class C, bool KCL, int ROWS, int NV>
__device__ __forceinline__ void store_tile(float* __restrict__ lds, const f32x4 (&r)[NV]) {
  using T = OpTile<C, KCL, ROWS>;
  static_assert(NV == T::PER_THREAD, "prefetch registers");
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = threadIdx.x + C::NT * i;
    float* dst;
    if (KCL) dst = lds + (idx / (C::BK / 4)) * T::LD + (idx % (C::BK / 4)) * 4;
    else dst = lds + (idx / (ROWS / 4)) * T::LD + (idx % (ROWS / 4)) * 4;
    *reinterpret_cast<f32x4*>(dst) = r[i];
  }
}

// Fragment of one 32-row (or 32-column) MFMA operand for 8 k-steps starting
// at step s0: lane l supplies row (l % 32) at k = KH * (l / 32) + s0 + s.
template <class C, bool KCL, int ROWS>
__device__ __forceinline__ void read_frag(float (&f)[8], const float* __restrict__ lds,
                                          int row_base, int s0) {
  using T = OpTile<C, KCL, ROWS>;
  const int lane = threadIdx.x & 63;
  const int row = row_base + (lane & 31);
  const int kh = (lane >> 5) * C::KH + s0;
  if (KCL) {
    const f32x4* p = reinterpret_cast<const f32x4*>(lds + row * T::LD + kh);
    const f32x4 x0 = p[0], x1 = p[1];
    f[0] = x0[0]; f[1] = x0[1]; f[2] = x0[2]; f[3] = x0[3];
    f[4] = x1[0]; f[5] = x1[1]; f[6] = x1[2]; f[7] = x1[3];
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = lds[(kh + s) * T::LD + row];
  }
}

// Main loop of a whole tile (every load in bounds, K a multiple of BK) with
// A stored k-contiguous and B stored m/n-contiguous, the layout of every
// square product of the iteration.  A k tile is one basic block whose
// schedule is fixed with scheduling-group barriers: the A fragments of the
// whole k tile and the first B fragments are read, and each k step's MFMAs
// are interleaved with the B fragment reads of the following step; the last
// step's MFMAs are interleaved with the LDS stores of the next tile (into
// the other buffer, which no wave reads in this k tile; the polynomial is
// formed as they are stored), and the loads of the tile after it are issued
// right after those stores, before the barrier, so that they have the
// barrier wait and the next tile's first fragment reads as cover (the
// registers hold one tile in flight throughout).
template <int MF, int OPS, int MASK, int PER>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (MF > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int k = OPS < PER ? OPS : PER;
    if constexpr (k > 0) __builtin_amdgcn_sched_group_barrier(MASK, k, 0);
    sched_interleave<MF - 1, OPS - k, MASK, PER>();
  } else if constexpr (OPS > 0) {
    __builtin_amdgcn_sched_group_barrier(MASK, OPS, 0);
  }
}

template <class C, bool APOLY, bool BPOLY, int FM_, int FN_>
__device__ __forceinline__ void mainloop_fast(f32x16 (&acc)[FM_][FN_], float* smem_a0,
                                              float* smem_b0, const float* __restrict__ A,
                                              const float* __restrict__ A2, int64_t lda,
                                              const float* __restrict__ B,
                                              const float* __restrict__ B2, int64_t ldb,
                                              const PolyCtx& pc, int m0, int n0, int kb,
                                              int nk, int lane, int wm, int wn) {
  using TA = OpTile<C, true, C::BM>;
  using TB = OpTile<C, false, C::BN>;
  constexpr int FM = C::FM, FN = C::FN, BK = C::BK, KH = C::KH;
  constexpr int NA = TA::PER_THREAD, NB = TB::PER_THREAD;
  constexpr int MF = FM * FN;
  static_assert(KH == 8, "one A fragment read pair per k tile");
  static_assert(FM_ == FM && FN_ == FN, "accumulator shape");
  auto smem_a = [&](int st) { return smem_a0 + st * TA::FLOATS; };
  auto smem_b = [&](int st) { return smem_b0 + st * TB::FLOATS; };
  const int t = threadIdx.x;
  // A (KC): item idx -> row idx / (BK / 4), k 4 (idx % (BK / 4))
  // B (MC): item idx -> k idx / (BN / 4), column 4 (idx % (BN / 4))
  int64_t aoff[NA], boff[NB];
  int alds[NA], blds[NB], arow[NA], acol[NA], brow[NB], bcol[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int idx = t + C::NT * i;
    arow[i] = idx / (BK / 4);
    acol[i] = (idx % (BK / 4)) * 4;
    aoff[i] = (int64_t)(m0 + arow[i]) * lda + acol[i];
    alds[i] = arow[i] * TA::LD + acol[i];
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int idx = t + C::NT * i;
    brow[i] = idx / (C::BN / 4);
    bcol[i] = (idx % (C::BN / 4)) * 4;
    boff[i] = (int64_t)brow[i] * ldb + n0 + bcol[i];
    blds[i] = brow[i] * TB::LD + bcol[i];
  }
  // polynomial element (i, j) of the stored matrix: c0 [i == j] + c1 R + alpha R2
  auto poly4 = [&](f32x4 r1, f32x4 r2, int i, int j) {
    f32x4 g;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      g[u] = pc.degree == 2 ? pc.c1 * r1[u] + pc.alpha * r2[u] : pc.alpha * r1[u];
      if (i == j + u) g[u] += pc.c0;
    }
    return g;
  };
  f32x4 ra[NA], rb[NB], ra2[NA], rb2[NB];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      ra[i] = *reinterpret_cast<const f32x4*>(A + aoff[i] + k0);
      if (APOLY && pc.degree == 2) ra2[i] = *reinterpret_cast<const f32x4*>(A2 + aoff[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      rb[i] = *reinterpret_cast<const f32x4*>(B + boff[i] + (int64_t)k0 * ldb);
      if (BPOLY && pc.degree == 2)
        rb2[i] = *reinterpret_cast<const f32x4*>(B2 + boff[i] + (int64_t)k0 * ldb);
    }
  };
  auto lstore = [&](int stage, int k0) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const f32x4 v = APOLY ? poly4(ra[i], ra2[i], m0 + arow[i], k0 + acol[i]) : ra[i];
      *reinterpret_cast<f32x4*>(smem_a(stage) + alds[i]) = v;
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const f32x4 v = BPOLY ? poly4(rb[i], rb2[i], k0 + brow[i], n0 + bcol[i]) : rb[i];
      *reinterpret_cast<f32x4*>(smem_b(stage) + blds[i]) = v;
    }
  };
  gload(kb * BK);
  lstore(0, kb * BK);
  gload((kb + (nk > 1 ? 1 : 0)) * BK);  // early: tile 1 in flight
  __syncthreads();
  const int fa_ofs = (wm + (lane & 31)) * TA::LD + (lane >> 5) * KH;
  const int fb_ofs = ((lane >> 5) * KH) * TB::LD + wn + (lane & 31);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const int kn = (kb + (kt + 1 < nk ? kt + 1 : kt)) * BK;  // the last tile reloads itself
    const int kn2 = (kb + (kt + 2 < nk ? kt + 2 : nk - 1)) * BK;  // early: the tile after it
    const float* sa = smem_a(cur) + fa_ofs;
    const float* sb = smem_b(cur) + fb_ofs;
    f32x4 fa[FM][2];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      fa[i][0] = *reinterpret_cast<const f32x4*>(sa + 32 * i * TA::LD);
      fa[i][1] = *reinterpret_cast<const f32x4*>(sa + 32 * i * TA::LD + 4);
    }
    float fb[2][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = sb[32 * j];
#pragma unroll
    for (int s = 0; s < KH; ++s) {
      const int c = s & 1, n = c ^ 1;
      if (s + 1 < KH) {
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[n][j] = sb[(s + 1) * TB::LD + 32 * j];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s >> 2][s & 3], fb[c][j],
                                                           acc[i][j], 0, 0, 0);
    }
    lstore(cur ^ 1, kn);
    gload(kn2);
    // schedule of the k tile
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * FM + FN, 0);  // A, first B fragments
#pragma unroll
    for (int s = 0; s + 1 < KH; ++s) sched_interleave<MF, FN, 0x100, (FN + MF - 1) / MF>();
    sched_interleave<MF, NA + NB, 0x200, (NA + NB + MF - 1) / MF>();
    __builtin_amdgcn_sched_group_barrier(0x020, (NA + NB) * ((APOLY || BPOLY) ? 2 : 1), 0);
    __syncthreads();
  }
}

// Work item -> (matrix-problem z, tile m, tile n).  mode 1 additionally
// permutes every full round of G items so that the blocks resident at the
// same time on one XCD (workgroups go to the 8 XCDs round-robin by block
// index) take neighbouring items; mode 2 keeps row-major tiles; modes 0 and
// 1 order the tiles of a matrix in groups of 8 tile-rows per column sweep.
struct TileCoord {
  int z, tm, tn, tile;
};

__device__ __forceinline__ TileCoord map_item(int it, int G, int total, int tiles_m,
                                              int tiles_n, int mode) {
  int L = it;
  if (mode == 1 && (G & 7) == 0) {
    const int round = it / G;
    if ((round + 1) * G <= total) {
      const int bi = it - round * G;
      L = round * G + (bi & 7) * (G >> 3) + (bi >> 3);
    }
  }
  const int tiles = tiles_m * tiles_n;
  TileCoord c;
  c.z = L / tiles;
  const int t = L - c.z * tiles;
  c.tile = t;
  if (mode == 2) {
    c.tm = t / tiles_n;
    c.tn = t - c.tm * tiles_n;
    return c;
  }
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GM;
  const int gsize = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in_group = t - group * per_group;
  c.tm = first_m + in_group % gsize;
  c.tn = in_group / gsize;
  return c;
}

// Item -> (matrix-problem z, tile) over the T (T + 1) / 2 tiles (tm <= tn) of
// the upper triangle, row by row.
__device__ __forceinline__ TileCoord map_item_sym(int it, int tiles, int T) {
  TileCoord c;
  c.z = it / tiles;
  int t = it - c.z * tiles;
  c.tile = t;
  int tm = 0;
  while (t >= T - tm) {
    t -= T - tm;
    ++tm;
  }
  c.tm = tm;
  c.tn = tm + t;
  return c;
}

// Ragged-first order, for split-k launches over matrices whose order is not
// a multiple of the tile: a matrix's tiles on its ragged last tile-row and
// last tile-column come first, then its whole tiles in row-major order, so
// the last items of the launch (the split-k tail) are whole tiles.  `tile`
// stays the row-major index (the residual's share slot).
__device__ __forceinline__ TileCoord map_item_ragged(int it, int tiles_m, int tiles_n, bool rrow,
                                                     bool rcol) {
  const int tiles = tiles_m * tiles_n;
  TileCoord c;
  c.z = it / tiles;
  const int t = it - c.z * tiles;
  const int nrow = rrow ? tiles_n : 0;                    // the last tile-row
  const int ncol = rcol ? tiles_m - (rrow ? 1 : 0) : 0;  // the last tile-column above it
  if (t < nrow) {
    c.tm = tiles_m - 1;
    c.tn = t;
  } else if (t < nrow + ncol) {
    c.tm = t - nrow;
    c.tn = tiles_n - 1;
  } else {
    const int wn = tiles_n - (rcol ? 1 : 0), u = t - nrow - ncol;
    c.tm = u / wn;
    c.tn = u - c.tm * wn;
  }
  c.tile = c.tm * tiles_n + c.tn;
  return c;
}

// The same for the upper triangle of T x T tiles (tm <= tn): the ragged last
// tile-column first, then the whole tiles row by row; `tile` is the
// row-by-row index of map_item_sym.
__device__ __forceinline__ TileCoord map_item_sym_ragged(int it, int tiles, int T) {
  TileCoord c;
  c.z = it / tiles;
  int t = it - c.z * tiles;
  if (t < T) {
    c.tm = t;
    c.tn = T - 1;
  } else {
    t -= T;
    int tm = 0;
    while (t >= T - 1 - tm) {
      t -= T - 1 - tm;
      ++tm;
    }
    c.tm = tm;
    c.tn = tm + t;
  }
  c.tile = c.tm * T - c.tm * (c.tm - 1) / 2 + (c.tn - c.tm);
  return c;
}

// Split-k tail ("stream-k").  When a launch's tiles do not divide evenly
// over the compute units, the last sk_rem items are not given out whole:
// their k tiles, laid end to end, are cut into sk_workers equal spans, one per
// extra block.  A span's partial accumulators go to a slot of sk_part; the
// block that completes a tile's last span (per-tile arrival counter in
// sk_cnt) adds the tile's slots in k order, so the sum does not depend on the
// order of arrival, resets the counter and runs the epilogue.  The host makes
// spans no longer than a tile, so a worker touches at most two tiles and
// owns slots 2 w and 2 w + 1.
__device__ __forceinline__ int64_t span_start(int w, int64_t U, int W) {
  return (int64_t)w * U / W;
}

// the worker whose span holds k-tile unit u (span_start(w) <= u < span_start(w + 1))
__device__ __forceinline__ int span_owner(int64_t u, int64_t U, int W) {
  int w = (int)(u * W / U);
  while (w + 1 < W && span_start(w + 1, U, W) <= u) ++w;
  while (w > 0 && span_start(w, U, W) > u) --w;
  return w;
}

// SPLIT: 0 every item whole; 1 split-k tail over whole tiles (every tile
// whole); 2 the same on a ragged-first launch (its ragged edge tiles take
// the general loop, so it is a variant of its own: the whole-tile form keeps
// its registers).
template <class C, bool TA, bool TB, int ROLE, int SPLIT>
__global__ __launch_bounds__(C::NT, C::MINW) void gemm_f32_kernel(GemmParams p) {
  constexpr int EPI = ROLE == ROLE_RESID ? EPI_RESID : (ROLE == ROLE_STATS ? EPI_EMA : EPI_STORE);
  constexpr bool AKC = Layout<true, TA>::kc;
  constexpr bool BKC = Layout<false, TB>::kc;
  using TAo = OpTile<C, AKC, C::BM>;
  using TBo = OpTile<C, BKC, C::BN>;
  constexpr int TILE = C::BM * C::BN;

  __shared__ __attribute__((aligned(16))) float smem_a[C::STAGES][TAo::FLOATS];
  __shared__ __attribute__((aligned(16))) float smem_b[C::STAGES][TBo::FLOATS];
  __shared__ double red[C::NW];
  __shared__ int sk_first, sk_pieces;

  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wm = (wid / C::WGN) * C::WTM, wn = (wid % C::WGN) * C::WTN;
  const bool vec = p.vec != 0;
  // symmetric output (C = C^T in exact arithmetic): the upper-triangle tiles
  // only, each off-diagonal one also stored transposed
  const bool sym = p.sym != 0;
  const int tiles = sym ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch * p.nprob;
  const int nk = (p.K + C::BK - 1) / C::BK;
  constexpr bool split = SPLIT;  // launched with sk_part set
  const int dp = split ? p.sk_dp : total;  // items computed whole
  const int G = split ? (int)gridDim.x - p.sk_workers : (int)gridDim.x;

  f32x16 acc[C::FM][C::FN];

  auto coord = [&](int it) __attribute__((always_inline)) {
    if constexpr (SPLIT == 2)
      return sym ? map_item_sym_ragged(it, tiles, p.tiles_m)
                 : map_item_ragged(it, p.tiles_m, p.tiles_n, p.M % C::BM != 0, p.N % C::BN != 0);
    else return sym ? map_item_sym(it, tiles, p.tiles_m)
               : map_item(it, G > 0 ? G : 1, total, p.tiles_m, p.tiles_n, p.map_mode);
  };
  auto running = [&](const TileCoord& tc) __attribute__((always_inline)) {
    if (!p.ctrl) return true;
    const Ctrl* c = p.ctrl + tc.z / p.nprob;
    return *(const volatile int32_t*)&c->status == PMX_RUNNING &&
           (p.min_degree == 0 || *(const volatile int32_t*)&c->degree >= p.min_degree);
  };

  // acc = the product over k tiles [kb, ke) of the tile tc
  auto compute = [&](const TileCoord& tc, int kb, int ke) __attribute__((always_inline)) {
    const int pi = tc.z % p.nprob;
    const int b = tc.z / p.nprob;
    const GemmProblem& pr = p.prob[pi];
    const float* __restrict__ A = pr.a.ptr + (int64_t)b * pr.a.stride;
    const float* __restrict__ B = pr.b.ptr + (int64_t)b * pr.b.stride;
    const float* __restrict__ A2 = pr.a.poly && pr.a.ptr2 ? pr.a.ptr2 + (int64_t)b * pr.a.stride : A;
    const float* __restrict__ B2 = pr.b.poly && pr.b.ptr2 ? pr.b.ptr2 + (int64_t)b * pr.b.stride : B;
    const bool apoly = pr.a.poly != 0, bpoly = pr.b.poly != 0;
    PolyCtx pc;
    pc.c0 = p.c0;
    pc.c1 = p.c1;
    pc.degree = p.degree;
    pc.alpha = (p.ctrl && (apoly || bpoly)) ? (float)p.ctrl[b].alpha : 0.f;
    const int m0 = tc.tm * C::BM, n0 = tc.tn * C::BN;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    __syncthreads();  // the previous item's last LDS reads are done
    if constexpr (SPLIT == 1) {
      // launched only for whole tiles of plain NN operands
      mainloop_fast<C, false, false>(acc, &smem_a[0][0], &smem_b[0][0], A, A2, pr.a.ld, B, B2,
                                     pr.b.ld, pc, m0, n0, kb, ke - kb, lane, wm, wn);
      return;
    } else if constexpr (SPLIT == 2) {
      // plain NN operands; whole tiles (every split-k span is one) take the
      // unchecked loop, the ragged edge tiles the general one below
      if (m0 + C::BM <= p.M && n0 + C::BN <= p.N) {
        mainloop_fast<C, false, false>(acc, &smem_a[0][0], &smem_b[0][0], A, A2, pr.a.ld, B,
                                       B2, pr.b.ld, pc, m0, n0, kb, ke - kb, lane, wm, wn);
        return;
      }
    }
    if constexpr (AKC && !BKC && C::STAGES == 2 && C::KH == 8) {
      if (vec && m0 + C::BM <= p.M && n0 + C::BN <= p.N && p.K % C::BK == 0 &&
          !(apoly && bpoly) && !(apoly && A2 == A && pc.degree == 2) &&
          !(bpoly && B2 == B && pc.degree == 2)) {
        if (apoly)
          mainloop_fast<C, true, false>(acc, &smem_a[0][0], &smem_b[0][0], A, A2, pr.a.ld, B,
                                        B2, pr.b.ld, pc, m0, n0, kb, ke - kb, lane, wm, wn);
        else if (bpoly)
          mainloop_fast<C, false, true>(acc, &smem_a[0][0], &smem_b[0][0], A, A2, pr.a.ld, B,
                                        B2, pr.b.ld, pc, m0, n0, kb, ke - kb, lane, wm, wn);
        else
          mainloop_fast<C, false, false>(acc, &smem_a[0][0], &smem_b[0][0], A, A2, pr.a.ld, B,
                                         B2, pr.b.ld, pc, m0, n0, kb, ke - kb, lane, wm, wn);
        return;
      }
    }
    f32x4 ra[TAo::PER_THREAD], rb[TBo::PER_THREAD];
    load_tile<C, AKC, C::BM>(ra, A, A2, apoly, pc, pr.a.ld, m0, p.M, kb * C::BK, p.K, vec);
    load_tile<C, BKC, C::BN>(rb, B, B2, bpoly, pc, pr.b.ld, n0, p.N, kb * C::BK, p.K, vec);
    store_tile<C, AKC, C::BM>(smem_a[0], ra);
    store_tile<C, BKC, C::BN>(smem_b[0], rb);
    __syncthreads();

    for (int kt = kb; kt < ke; ++kt) {
      const int cur = C::STAGES == 2 ? ((kt - kb) & 1) : 0;
      const bool more = kt + 1 < ke;
      if (more) {
        load_tile<C, AKC, C::BM>(ra, A, A2, apoly, pc, pr.a.ld, m0, p.M, (kt + 1) * C::BK, p.K, vec);
        load_tile<C, BKC, C::BN>(rb, B, B2, bpoly, pc, pr.b.ld, n0, p.N, (kt + 1) * C::BK, p.K, vec);
      }
#pragma unroll
      for (int s0 = 0; s0 < C::KH; s0 += 8) {
        float fa[C::FM][8], fb[C::FN][8];
#pragma unroll
        for (int i = 0; i < C::FM; ++i) read_frag<C, AKC, C::BM>(fa[i], smem_a[cur], wm + 32 * i, s0);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) read_frag<C, BKC, C::BN>(fb[j], smem_b[cur], wn + 32 * j, s0);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][s], fb[j][s], acc[i][j], 0, 0, 0);
      }
      if (C::STAGES == 2) {
        if (more) {
          store_tile<C, AKC, C::BM>(smem_a[cur ^ 1], ra);
          store_tile<C, BKC, C::BN>(smem_b[cur ^ 1], rb);
        }
        __syncthreads();
      } else {
        __syncthreads();
        if (more) {
          store_tile<C, AKC, C::BM>(smem_a[0], ra);
          store_tile<C, BKC, C::BN>(smem_b[0], rb);
          __syncthreads();
        }
      }
    }
  };

  // Epilogue of the tile tc from acc.  Lane l of a 32x32 accumulator holds
  // column (l % 32) and rows 8 * (v / 4) + 4 * (l / 32) + (v % 4), v = 0..15.
  auto epilogue = [&](const TileCoord& tc) __attribute__((always_inline)) {
    const int pi = tc.z % p.nprob;
    const int b = tc.z / p.nprob;
    const GemmProblem& pr = p.prob[pi];
    float* __restrict__ Cm = pr.c + (int64_t)b * pr.stride_c;
    const int m0 = tc.tm * C::BM, n0 = tc.tn * C::BN;
    const int hi = lane >> 5, col_in = lane & 31;
    const bool mirror = sym && tc.tm != tc.tn;
    // resid_keep: the product itself is also stored, at prob[1].c (ld and
    // batch stride of prob[1])
    float* __restrict__ Kp = (EPI == EPI_RESID && p.resid_keep)
                                 ? p.prob[1].c + (int64_t)b * p.prob[1].stride_c : nullptr;
    float fro = 0.f;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int col = n0 + wn + 32 * j + col_in;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row_base = m0 + wm + 32 * i + 8 * g + 4 * hi;
          float xs[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row_base + r;
            float x = acc[i][j][4 * g + r];
            if (row < p.M && col < p.N) {
              float* dst = Cm + (int64_t)row * pr.ldc + col;
              if (EPI == EPI_RESID) {
                if (Kp) Kp[(int64_t)row * p.prob[1].ldc + col] = x;
                x = (row == col ? 1.f : 0.f) - x;
                fro += x * x;
              } else if (EPI == EPI_EMA) {
                x = p.beta * *dst + p.omb * x + (row == col ? p.eps : 0.f);
              }
              *dst = x;
            }
            xs[r] = x;
          }
          if (mirror && col < p.N) {
            // C[col][row_base .. row_base + 3]: four consecutive elements
            float* dst = Cm + (int64_t)col * pr.ldc + row_base;
            if (EPI == EPI_EMA) {
              // the mirrored elements keep their own old values (the caller's
              // statistics need not be symmetric); off the diagonal: no eps
              float old[4] = {0.f, 0.f, 0.f, 0.f};
              if (vec && row_base + 3 < p.M) {
                const f32x4 o = *reinterpret_cast<const f32x4*>(dst);
                old[0] = o[0];
                old[1] = o[1];
                old[2] = o[2];
                old[3] = o[3];
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (row_base + r < p.M) old[r] = dst[r];
              }
#pragma unroll
              for (int r = 0; r < 4; ++r) xs[r] = p.beta * old[r] + p.omb * acc[i][j][4 * g + r];
            }
            if (vec && row_base + 3 < p.M) {
              *reinterpret_cast<f32x4*>(dst) = f32x4{xs[0], xs[1], xs[2], xs[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (row_base + r < p.M) dst[r] = xs[r];
            }
            if (Kp) {
              // the kept product: I - x on the (off-diagonal) mirrored block
              float* kd = Kp + (int64_t)col * p.prob[1].ldc + row_base;
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (row_base + r < p.M) kd[r] = -xs[r];
            }
          }
        }
      }
    if (mirror) fro *= 2.f;  // the tile stands for itself and its transpose

    if (EPI == EPI_RESID) {
      // the tile's Frobenius share; resid_decide_kernel sums them
      const double blocksum = block_sum<C::NW>((double)fro, red);
      if (threadIdx.x == 0) p.partials[(int64_t)b * p.partial_stride + tc.tile] = blocksum;
    }
  };

  if constexpr (!split) {
    for (int it = blockIdx.x; it < total; it += G) {
      const TileCoord tc = coord(it);
      if (!running(tc)) continue;
      compute(tc, 0, nk);
      epilogue(tc);
    }
  } else {
    // Blocks below G take whole items it = blockIdx.x, + G, ... < dp; split-k
    // worker w takes the k-tile units [span_start(w), span_start(w + 1)) of
    // the tail, piece by piece (piece j of its span fills slot 2 w + j).
    const bool worker = (int)blockIdx.x >= G;
    const int W = p.sk_workers;
    const int w = (int)blockIdx.x - G;
    const int64_t U = (int64_t)p.sk_rem * nk;
    int64_t u = worker ? span_start(w, U, W) : 0;
    const int64_t u1 = worker ? span_start(w + 1, U, W) : 0;
    int it = blockIdx.x;
    for (int piece = 0;; ++piece) {
      int t, kb, ke;
      if (!worker) {
        if (it >= dp) break;
        t = it;
        kb = 0;
        ke = nk;
        it += G;
      } else {
        if (u >= u1) break;
        const int tt = (int)(u / nk);
        kb = (int)(u - (int64_t)tt * nk);
        ke = (int)((int64_t)nk < kb + (u1 - u) ? (int64_t)nk : kb + (u1 - u));
        u += ke - kb;
        t = dp + tt;
      }
      const TileCoord tc = coord(t);
      if (!running(tc)) continue;
      compute(tc, kb, ke);
      if (kb != 0 || ke != nk) {
        t -= dp;  // tail tile index
        {
          f32x4* slot = reinterpret_cast<f32x4*>(p.sk_part + (int64_t)(2 * w + piece) * TILE);
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                slot[((i * C::FN + j) * 4 + g) * C::NT + threadIdx.x] =
                    f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                          acc[i][j][4 * g + 3]};
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
          const int wa = span_owner((int64_t)t * nk, U, W);
          const int wb = span_owner((int64_t)t * nk + nk - 1, U, W);
          const uint32_t prev = atomicAdd(&p.sk_cnt[t], 1u);
          sk_first = wa;
          sk_pieces = prev == (uint32_t)(wb - wa) ? wb - wa + 1 : 0;
        }
        __syncthreads();
        const int npc = sk_pieces, wa = sk_first;
        if (npc == 0) continue;
        // the last span of the tile: its slots in k order
        __threadfence();
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        for (int q = 0; q < npc; ++q) {
          const int wq = wa + q;
          // the tile is the first (slot 2 wq) or the second (2 wq + 1) of wq's span
          const int first = (int)(span_start(wq, U, W) / nk);
          const f32x4* slot = reinterpret_cast<const f32x4*>(
              p.sk_part + (int64_t)(2 * wq + (t == first ? 0 : 1)) * TILE);
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const f32x4 x = slot[((i * C::FN + j) * 4 + g) * C::NT + threadIdx.x];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[i][j][4 * g + r] += x[r];
              }
        }
        if (threadIdx.x == 0) p.sk_cnt[t] = 0u;
      }
      epilogue(tc);
    }
  }
}

// Tile configurations.  0: 128 x 128 x 16, 2 x 2 waves (64 x 64 per wave);
// 1: 256 x 128 x 16, 4 x 2 waves; 2: 128 x 256 x 16, 2 x 4 waves;
// 3: 128 x 128 x 32, 2 x 2 waves; 4: 64 x 64 x 16, 2 x 2 waves (32 x 32 per
// wave, for small matrices); 5: 128 x 64 x 16, 2 x 2 waves; 6: 256 x 128 x 16,
// 2 x 2 waves (128 x 64 per wave); 7: 128 x 256 x 16, 2 x 2 waves (64 x 128);
// 8: 128 x 128 x 64, single LDS buffer; 9: 128 x 128 x 32, double buffered.
using C0 = Cfg<128, 128, 16, 2, 2, 3>;
using C1 = Cfg<256, 128, 16, 4, 2, 2>;
using C2 = Cfg<128, 256, 16, 2, 4, 2>;
using C3 = Cfg<128, 128, 32, 2, 2, 2>;
using C4 = Cfg<64, 64, 16, 2, 2, 4>;
using C5 = Cfg<128, 64, 16, 2, 2, 4>;
using C6 = Cfg<256, 128, 16, 2, 2, 2>;
using C7 = Cfg<128, 256, 16, 2, 2, 2>;
using C8 = Cfg<128, 128, 64, 2, 2, 1, 1>;
using C9 = Cfg<128, 128, 32, 2, 2, 1, 2>;

template <class C>
int tiles_of(int M, int N) {
  return ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
}

// Split-k variants: the iteration roles (R^2, updates, residuals) on the
// configurations the automatic choice takes.
template <class C, bool TA, bool TB, int ROLE>
constexpr bool kSplitVariant =
    !TA && !TB &&
    (ROLE == ROLE_POWER || ROLE == ROLE_UPDATE || ROLE == ROLE_RESID || ROLE == ROLE_STATS) &&
    (std::is_same<C, C0>::value || std::is_same<C, C4>::value || std::is_same<C, C5>::value);

template <class C, bool TA, bool TB, int ROLE>
hipError_t launch_role(GemmParams p, hipStream_t s) {
  p.tiles_m = (p.M + C::BM - 1) / C::BM;
  p.tiles_n = (p.N + C::BN - 1) / C::BN;
  if (p.sym && (C::BM != C::BN || p.M != p.N)) return hipErrorInvalidValue;
  const int64_t tiles = p.sym ? (int64_t)p.tiles_m * (p.tiles_m + 1) / 2
                              : (int64_t)p.tiles_m * p.tiles_n;
  const int64_t total = tiles * p.batch * p.nprob;
  // split-k tail when the items leave the last round of the compute units
  // part-filled: the remainder's k tiles are spread over one extra block per
  // CU (at least two k tiles each, so every span is shorter than a tile)
  float* const skp = p.sk_part;
  p.sk_part = nullptr;
  p.sk_dp = (int)total;
  p.sk_rem = p.sk_workers = 0;
  p.ragged_first = 0;
  if (kSplitVariant<C, TA, TB, ROLE>) {
    const int cu = p.num_cu > 0 ? p.num_cu : 256;
    const int64_t nk = (p.K + C::BK - 1) / C::BK;
    const int64_t rem = total % cu;
    const int64_t W = std::min<int64_t>(std::min(cu, kSplitMaxWorkers), rem * nk / 2);
    // split variants take plain operands; the tail (the last rem items) must
    // be whole tiles: on ragged matrices the items go ragged-first (row-major
    // tile order or the triangle), and the tail fits in the last matrix's
    // whole tiles
    const bool rrow = p.M % C::BM != 0, rcol = p.N % C::BN != 0;
    const int64_t whole_tiles =
        p.sym ? (int64_t)(p.tiles_m - rrow) * (p.tiles_m - rrow + 1) / 2
              : (int64_t)(p.tiles_m - rrow) * (p.tiles_n - rcol);
    const bool ragged = rrow || rcol;
    bool whole = p.vec && p.K % C::BK == 0 && rem <= whole_tiles &&
                 (!ragged || p.sym || p.map_mode == 2);
    for (int i = 0; i < p.nprob; ++i) whole = whole && !p.prob[i].a.poly && !p.prob[i].b.poly;
    // only as the tail of at least one whole round, or over long k: a launch
    // with fewer items than CUs runs faster unsplit when k is short (measured
    // on the 1024^2 triangles with k = 1024, 136 tiles: 45 -> 21 us; every
    // span pays the cross-XCD fences of the fix-up), while with k >= 2048
    // (the statistics G G^T of a 1024 x 4096 gradient) the spans are long
    // enough to pay for them
    if (whole && skp && p.sk_cnt && rem > 0 && (total >= cu || nk >= 128) && nk >= 4 &&
        W >= rem && 2 * W * C::BM * C::BN <= p.sk_cap) {
      p.sk_part = skp;
      p.sk_dp = (int)(total - rem);
      p.sk_rem = (int)rem;
      p.sk_workers = (int)W;
      p.ragged_first = ragged ? 1 : 0;
    }
  }
  int64_t g = p.sk_dp;
  if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
  const dim3 grid((unsigned)(g + p.sk_workers)), block(C::NT);
  if (grid.x == 0) return hipSuccess;
  bool launched = false;
  if constexpr (kSplitVariant<C, TA, TB, ROLE>) {
    if (p.sk_part) {
      if (p.ragged_first)
        hipLaunchKernelGGL((gemm_f32_kernel<C, TA, TB, ROLE, 2>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((gemm_f32_kernel<C, TA, TB, ROLE, 1>), grid, block, 0, s, p);
      launched = true;
    }
  }
  if (!launched) hipLaunchKernelGGL((gemm_f32_kernel<C, TA, TB, ROLE, 0>), grid, block, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ROLE != ROLE_RESID) return e;
  ResidDecide d;
  d.ctrl = p.ctrl;
  d.partials = p.partials;
  d.partial_stride = p.partial_stride;
  d.tiles = (int)tiles;
  d.products = p.products;
  d.count_update = p.count_update;
  d.cfg = p.cfg;
  return launch_resid_decide(d, p.batch, s);
}

// Roles instantiated per transpose combination: every role in NN (the
// statistics take G and a transposed copy of G, so G G^T and G^T G are NN
// products too), and the residual I - X^T X of the fp32 polar factor in TN.
template <class C>
hipError_t launch_cfg(const GemmParams& p, bool ta, bool tb, int role, hipStream_t s) {
  if (!ta && !tb) {
    switch (role) {
      case ROLE_POWER: return launch_role<C, false, false, ROLE_POWER>(p, s);
      case ROLE_UPDATE: return launch_role<C, false, false, ROLE_UPDATE>(p, s);
      case ROLE_RESID: return launch_role<C, false, false, ROLE_RESID>(p, s);
      case ROLE_STATS: return launch_role<C, false, false, ROLE_STATS>(p, s);
      case ROLE_APPLY: return launch_role<C, false, false, ROLE_APPLY>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (ta && !tb && role == ROLE_RESID) return launch_role<C, true, false, ROLE_RESID>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace

int gemm_f32_tiles(int M, int N) {
  // upper bound over the configurations: the smallest tile (64 x 64)
  return tiles_of<C4>(M, N);
}

// Configuration choice: p.cfg_id >= 0 forces one; otherwise the largest tile
// that still gives every CU at least one tile of the launch (square tiles for
// symmetric outputs).
hipError_t launch_gemm_f32(const GemmParams& p, bool ta, bool tb, int role, hipStream_t s) {
  int id = p.cfg_id;
  if (p.sym) {
    // square tiles only: the 128 x 128 tile when the split-k tail will spread
    // a long k (>= 2048) over the CUs, or when the triangle gives every CU at
    // least four tiles; else 64 x 64.  (64 batched triangles of order 512,
    // k = 512: 640 tiles of 128, 2.5 per CU, took 162-184 us with the split
    // tail and 111-113 us without; 2304 tiles of 64 took 97-106 us.)
    const int64_t t0 = (p.M + 127) / 128;
    const bool long_split = p.sk_part && p.sk_cnt && p.vec && p.M % 128 == 0 &&
                            p.K % 16 == 0 && p.K >= 2048 && !p.prob[0].a.poly &&
                            !p.prob[0].b.poly;
    const int64_t cu = p.num_cu > 0 ? p.num_cu : 256;
    id = (long_split || t0 * (t0 + 1) / 2 * p.batch * p.nprob >= 4 * cu) ? 0 : 4;
  } else if (id < 0) {
    const int64_t units = (int64_t)p.batch * p.nprob;
    const int cu = p.num_cu > 0 ? p.num_cu : 256;
    if ((int64_t)tiles_of<C0>(p.M, p.N) * units >= cu) id = 0;
    else if ((int64_t)tiles_of<C5>(p.M, p.N) * units >= cu) id = 5;
    else id = 4;
  }
  switch (id) {
    case 0: return launch_cfg<C0>(p, ta, tb, role, s);
    case 1: return launch_cfg<C1>(p, ta, tb, role, s);
    case 2: return launch_cfg<C2>(p, ta, tb, role, s);
    case 3: return launch_cfg<C3>(p, ta, tb, role, s);
    case 4: return launch_cfg<C4>(p, ta, tb, role, s);
    case 5: return launch_cfg<C5>(p, ta, tb, role, s);
    case 6: return launch_cfg<C6>(p, ta, tb, role, s);
    case 7: return launch_cfg<C7>(p, ta, tb, role, s);
    case 8: return launch_cfg<C8>(p, ta, tb, role, s);
    case 9: return launch_cfg<C9>(p, ta, tb, role, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pmx
