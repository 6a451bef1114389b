// bf16 MFMA GEMM for gfx950 (bf16 operands, fp32 accumulation), used by the
// bf16 polar-factor iteration.  Every operand is stored with k contiguous:
//   C[i][j] = sum_k A[i][k] * Bs[j][k]
// (A is M x K, Bs is N x K, both row-major bf16).  The polar iteration keeps a
// transposed copy X^T of its iterate; R and g are symmetric, so their bf16
// copies serve as Bs unchanged and its three products all take this form:
//   R  = I - X^T X : A = X^T, Bs = X^T   (the epilogue also writes R in bf16)
//   R2 = R R       : A = R,   Bs = R
//   X' = X g       : A = X,   Bs = g     (the epilogue also writes X'^T)
//
// Design (CDNA4):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) and 8 consecutive
//    k values 8 (l / 32) .. +7 of a 16-wide k step: one 16-byte LDS read per
//    fragment.  LDS rows are padded to 72 bf16 (144 bytes) so the 16-byte
//    reads of 8 consecutive rows hit distinct banks.
//  * Block tile 256 x 256 x 64 with 8 waves of 128 x 64 (4 x 2 accumulators,
//    one block per CU: 6 fragment reads per 8 MFMAs), or 128 x 128 x 64 with
//    4 waves of 64 x 64 when the problem has fewer large tiles than compute
//    units.  16-byte global loads into 16-byte LDS stores,
//    LDS double buffered with a register prefetch of the next k tile, the
//    fragments of the next 16-wide k step read while the current one
//    multiplies; persistent grid over (matrix, tile).
//  * fp32 -> bf16 rounding is round-to-nearest-even.
#include <type_traits>

#include "pmx_kernels.h"

namespace pmx {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Block tile BM x BN x BK, waves of WM x WN (FM x FN accumulators of
// 32 x 32), MINB blocks resident per CU.  LDS rows hold BK + 8 bf16: the row
// pitch (144 or 80 bytes) is an odd multiple of 16 bytes modulo 128, so the
// 16-byte fragment reads of 8 (or 16) consecutive rows hit distinct banks.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int MINB_>
struct BCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, MINB = MINB_;
  static constexpr int LDK = BK + 8;
  static constexpr int CH = BK / 8;  // 16-byte chunks per LDS row
  static constexpr int WAVES = (BM / WM) * (BN / WN);
  static constexpr int NT = 64 * WAVES;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int CA = BM * CH / NT;  // 16-byte chunks per thread per k tile
  static constexpr int CB = BN * CH / NT;
  static constexpr int LDS = (BM + BN) * LDK;  // bf16 per stage
  static_assert(CA * NT == BM * CH && CB * NT == BN * CH, "tile / thread mismatch");
};
using BSmall = BCfg<128, 128, 64, 64, 64, 2>;   // 4 waves of 64 x 64, 72 KB LDS
using BLarge = BCfg<256, 256, 128, 64, 64, 1>;  // 8 waves of 128 x 64, 144 KB LDS
using BLarge4 = BCfg<256, 256, 128, 128, 64, 1>;  // 4 waves of 128 x 128
using BMid2 = BCfg<256, 128, 128, 64, 32, 2>;   // 4 waves of 128 x 64, 60 KB, 2 per CU

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// One ROWS x BK operand tile: chunk idx -> (row idx / CH, k 8 (idx % CH)).
template <class CF, int C>
__device__ __forceinline__ void load_chunks(u32x4 (&v)[C], const uint16_t* base, int64_t ld,
                                            int row0, int nrows, int k0, int K, bool vec) {
  constexpr int NT = CF::NT, CH = CF::CH;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int idx = threadIdx.x + NT * i;
    const int row = row0 + idx / CH;
    const int k = k0 + (idx % CH) * 8;
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

template <class CF, int C>
__device__ __forceinline__ void store_chunks(uint16_t* lds, const u32x4 (&v)[C]) {
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int idx = threadIdx.x + CF::NT * i;
    *reinterpret_cast<u32x4*>(lds + (idx / CF::CH) * CF::LDK + (idx % CF::CH) * 8) = v[i];
  }
}

// Symmetric outputs: the T (T + 1) / 2 tiles tm <= tn of the upper triangle,
// row by row.
__device__ __forceinline__ void item_tile_sym(int it, int T, int* z, int* tm, int* tn,
                                              int* tile) {
  const int tiles = T * (T + 1) / 2;
  *z = it / tiles;
  int t = it - *z * tiles;
  *tile = t;
  int m = 0;
  while (t >= T - m) {
    t -= T - m;
    ++m;
  }
  *tm = m;
  *tn = m + t;
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

// Main loop of a tile that lies wholly inside A and Bs (16-byte aligned rows,
// K a multiple of 64): no bounds tests, so a k tile is one basic block and
// its schedule is fixed with scheduling-group barriers.  Per k tile: the
// fragments of the first 16-wide step and the next tile's global loads are
// issued first; each step's MFMAs are interleaved one-for-one with the
// fragment reads of the following step; the last step's MFMAs are interleaved
// with the LDS stores of the next tile (into the other LDS buffer, which no
// wave reads in this k tile).
// Scheduling groups: MF MFMAs, each followed by up to PER instructions of
// class MASK (0x100 LDS read, 0x200 LDS write) until OPS are placed.
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

// Operand origins of a whole tile at k tile 0 (wave-uniform) and the
// thread's offsets from them (the same for every tile of a launch), so a
// k tile's loads are uniform base + 32-bit offset.
struct TileBase {
  const uint16_t* a;
  const uint16_t* b;
};

template <class C>
struct FastOffsets {
  uint32_t a, b;    // thread offsets (elements) of chunk 0
  uint32_t sa, sb;  // between a thread's chunks
  int wofs;         // LDS offset of chunk 0
  __device__ FastOffsets(int64_t lda, int64_t ldb) {
    const int t = threadIdx.x;
    constexpr int RS = C::NT / C::CH;  // rows covered by one chunk index step
    a = (uint32_t)((t / C::CH) * lda + (t % C::CH) * 8);
    b = (uint32_t)((t / C::CH) * ldb + (t % C::CH) * 8);
    sa = (uint32_t)(RS * lda);
    sb = (uint32_t)(RS * ldb);
    wofs = (t / C::CH) * C::LDK + (t % C::CH) * 8;
  }
};

// k tile 0 of a tile into LDS buffer `buf`.
template <class C>
__device__ __forceinline__ void fast_stage0(uint16_t (*smem)[C::LDS], int buf, TileBase tb,
                                            const FastOffsets<C>& o) {
  constexpr int CA = C::CA, CB = C::CB, RS = C::NT / C::CH, LDK = C::LDK;
  u32x4 va[CA], vb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(tb.a + (o.a + i * o.sa));
#pragma unroll
  for (int i = 0; i < CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(tb.b + (o.b + i * o.sb));
#pragma unroll
  for (int i = 0; i < CA; ++i)
    *reinterpret_cast<u32x4*>(smem[buf] + o.wofs + i * RS * LDK) = va[i];
#pragma unroll
  for (int i = 0; i < CB; ++i)
    *reinterpret_cast<u32x4*>(smem[buf] + C::BM * LDK + o.wofs + i * RS * LDK) = vb[i];
  __syncthreads();
}

// The k loop of a tile whose k tile 0 is staged in LDS buffer `buf`: k tile
// kt is read from buffer (kt + buf) & 1.  The last k tile's loads fetch k
// tile 0 of `nx` (the next tile of a persistent block, or a reload) into the
// other buffer, so a following tile finds its first k tile staged.
template <class C>
__device__ __forceinline__ void fast_kloop(f32x16 (&acc)[C::FM][C::FN],
                                           uint16_t (*smem)[C::LDS], int buf, TileBase cur,
                                           TileBase nx, const FastOffsets<C>& o, int nk,
                                           int lane, int wm, int wn) {
  constexpr int FM = C::FM, FN = C::FN, CA = C::CA, CB = C::CB;
  constexpr int BK = C::BK, LDK = C::LDK, STEPS = BK / 16;
  constexpr int NF = FM + FN;          // fragment reads per step
  constexpr int RS = C::NT / C::CH;    // rows covered by one chunk index step
  constexpr int MF = FM * FN;          // MFMAs per step
  const int ra = (wm + (lane & 31)) * LDK + (lane >> 5) * 8;
  const int rb = (C::BM + wn + (lane & 31)) * LDK + (lane >> 5) * 8;
  u32x4 va[CA], vb[CB];
  for (int kt = 0; kt < nk; ++kt) {
    const int cb = (kt + buf) & 1;
    const uint16_t* sa = smem[cb] + ra;
    const uint16_t* sb = smem[cb] + rb;
    uint16_t* dst = smem[cb ^ 1] + o.wofs;
    const bool more = kt + 1 < nk;
    const uint16_t* la = more ? cur.a + (kt + 1) * BK : nx.a;
    const uint16_t* lb = more ? cur.b + (kt + 1) * BK : nx.b;
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * LDK);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = *reinterpret_cast<const bf16x8*>(sb + 32 * j * LDK);
#pragma unroll
    for (int i = 0; i < CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(la + (o.a + i * o.sa));
#pragma unroll
    for (int i = 0; i < CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(lb + (o.b + i * o.sb));
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int c = s & 1, n = c ^ 1;
      if (s + 1 < STEPS) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[n][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * LDK + 16 * (s + 1));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          fb[n][j] = *reinterpret_cast<const bf16x8*>(sb + 32 * j * LDK + 16 * (s + 1));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(dst + i * RS * LDK) = va[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(dst + C::BM * LDK + i * RS * LDK) = vb[i];
    // schedule of the k tile
    __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);       // step 0 fragments
    __builtin_amdgcn_sched_group_barrier(0x020, CA + CB, 0);  // next tile, global
#pragma unroll
    for (int s = 0; s + 1 < STEPS; ++s) sched_interleave<MF, NF, 0x100, (NF + MF - 1) / MF>();
    sched_interleave<MF, CA + CB, 0x200, (CA + CB + MF - 1) / MF>();
    __syncthreads();
  }
}

template <class C>
__device__ __forceinline__ void mainloop_fast(f32x16 (&acc)[C::FM][C::FN],
                                              uint16_t (*smem)[C::LDS], const uint16_t* A,
                                              int64_t lda, const uint16_t* B, int64_t ldb,
                                              int m0, int n0, int nk, int lane, int wm, int wn) {
  const FastOffsets<C> o(lda, ldb);
  const TileBase cur = {A + (int64_t)m0 * lda, B + (int64_t)n0 * ldb};
  fast_stage0<C>(smem, 0, cur, o);
  // the last k tile reloads itself
  const TileBase nx = {cur.a + (nk - 1) * C::BK, cur.b + (nk - 1) * C::BK};
  fast_kloop<C>(acc, smem, 0, cur, nx, o, nk, lane, wm, wn);
}

// The same main loop for operands stored m- (n-) contiguous: A is K x M
// (A^T of the C = A Bs^T form, row k holding M values), Bs likewise K x N,
// e.g. C = X^T X straight from the row-major iterate X, with no transposed
// copy.  A k tile is staged untransposed, T[k][i] with row pitch BM + 32
// (576 bytes for 256: 144 dwords = 16 mod 64, so the four rows of a
// transpose read fall on distinct banks), with 16-byte loads and stores.
// The fragments come from gfx950's LDS transpose read ds_read_b64_tr_b16:
// in each group of 16 lanes, lane j receives element j % 4 of the 8 bytes
// read by lanes 4 t + j / 4 (t = 0 .. 3), so a lane that addresses row
// k0 + j / 4, column i0 + 4 (j % 4) gets column i0 + j of rows k0 .. k0 + 3.
// Lane l (group g = l / 16) addresses k0 = 8 (g / 2) (+ 4 for the second
// read) and i0 = 16 (g % 2), which gives it row l % 32 and k = 8 (l / 32)
// .. + 7 of the 32 x 16 MFMA operand: two 8-byte reads per fragment where
// the k-contiguous form reads 16 bytes once.  Only whole 256 x 256 x 64
// tiles (the launcher checks).
typedef short i16x4_tr __attribute__((ext_vector_type(4)));
typedef short i16x8_tr __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* p, int pitch) {
  const i16x4_tr lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_tr*)(p));
  const i16x4_tr hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_tr*)(p + 4 * pitch));
  const i16x8_tr w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

template <class C>
struct MnOffsets {
  static constexpr int PA = C::BM + 32, PB = C::BN + 32;
  static constexpr int CPA = C::BM / 8, CPB = C::BN / 8;  // 16-byte chunks per k row
  static constexpr int RSA = C::NT / CPA, RSB = C::NT / CPB;  // k rows per chunk index step
  uint32_t a, b, sa, sb;
  int wa, wb;
  __device__ MnOffsets(int64_t lda, int64_t ldb) {
    const int t = threadIdx.x;
    a = (uint32_t)((t / CPA) * lda + (t % CPA) * 8);
    b = (uint32_t)((t / CPB) * ldb + (t % CPB) * 8);
    sa = (uint32_t)(RSA * lda);
    sb = (uint32_t)(RSB * ldb);
    wa = (t / CPA) * PA + (t % CPA) * 8;
    wb = C::BK * PA + (t / CPB) * PB + (t % CPB) * 8;
  }
};

template <class C>
__device__ __forceinline__ void mn_stage0(uint16_t (*smem)[C::LDS], int buf, TileBase tb,
                                          const MnOffsets<C>& o) {
  using O = MnOffsets<C>;
  constexpr int CA = C::BK * O::CPA / C::NT, CB = C::BK * O::CPB / C::NT;
  u32x4 va[CA], vb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(tb.a + (o.a + i * o.sa));
#pragma unroll
  for (int i = 0; i < CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(tb.b + (o.b + i * o.sb));
#pragma unroll
  for (int i = 0; i < CA; ++i)
    *reinterpret_cast<u32x4*>(smem[buf] + o.wa + i * O::RSA * O::PA) = va[i];
#pragma unroll
  for (int i = 0; i < CB; ++i)
    *reinterpret_cast<u32x4*>(smem[buf] + o.wb + i * O::RSB * O::PB) = vb[i];
  __syncthreads();
}

// k loop of the m-contiguous form (as fast_kloop: buffer parity `buf`, the
// last k tile's loads fetch k tile 0 of `nx`).  A k tile advances BK rows.
template <class C>
__device__ __forceinline__ void mn_kloop(f32x16 (&acc)[C::FM][C::FN], uint16_t (*smem)[C::LDS],
                                         int buf, TileBase cur, TileBase nx,
                                         const MnOffsets<C>& o, int64_t lda, int64_t ldb,
                                         int nk, int lane, int wm, int wn) {
  using O = MnOffsets<C>;
  constexpr int FM = C::FM, FN = C::FN, BK = C::BK, STEPS = BK / 16;
  constexpr int PA = O::PA, PB = O::PB;
  static_assert(BK * (PA + PB) <= C::LDS, "an m-contiguous k tile fits an LDS stage");
  constexpr int CA = BK * O::CPA / C::NT, CB = BK * O::CPB / C::NT;
  static_assert(CA * C::NT == BK * O::CPA && CB * C::NT == BK * O::CPB, "chunks per thread");
  constexpr int NF = 2 * (FM + FN);  // transpose reads per step
  constexpr int MF = FM * FN;        // MFMAs per step
  const int g = lane >> 4, j = lane & 15;
  const int ra = (8 * (g >> 1) + (j >> 2)) * PA + 16 * (g & 1) + 4 * (j & 3) + wm;
  const int rb = BK * PA + (8 * (g >> 1) + (j >> 2)) * PB + 16 * (g & 1) + 4 * (j & 3) + wn;
  u32x4 va[CA], vb[CB];
  for (int kt = 0; kt < nk; ++kt) {
    const int cb = (kt + buf) & 1;
    const uint16_t* sa = smem[cb] + ra;
    const uint16_t* sb = smem[cb] + rb;
    uint16_t* dst = smem[cb ^ 1];
    const bool more = kt + 1 < nk;
    const uint16_t* la = more ? cur.a + (int64_t)(kt + 1) * BK * lda : nx.a;
    const uint16_t* lb = more ? cur.b + (int64_t)(kt + 1) * BK * ldb : nx.b;
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = frag_tr(sa + 32 * i, PA);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) fb[0][jj] = frag_tr(sb + 32 * jj, PB);
#pragma unroll
    for (int i = 0; i < CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(la + (o.a + i * o.sa));
#pragma unroll
    for (int i = 0; i < CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(lb + (o.b + i * o.sb));
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int c = st & 1, n = c ^ 1;
      if (st + 1 < STEPS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[n][i] = frag_tr(sa + 32 * i + 16 * (st + 1) * PA, PA);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) fb[n][jj] = frag_tr(sb + 32 * jj + 16 * (st + 1) * PB, PB);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
          acc[i][jj] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][jj], acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(dst + o.wa + i * O::RSA * PA) = va[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(dst + o.wb + i * O::RSB * PB) = vb[i];
    // schedule of the k tile (as in fast_kloop)
    __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, CA + CB, 0);
#pragma unroll
    for (int st = 0; st + 1 < STEPS; ++st) sched_interleave<MF, NF, 0x100, (NF + MF - 1) / MF>();
    sched_interleave<MF, CA + CB, 0x200, (CA + CB + MF - 1) / MF>();
    __syncthreads();
  }
}

// Early-load forms of the two k loops (persistent kernel, at least two k
// tiles an item): on entry to k tile kt the registers already hold the loads
// of tile kt + 1, issued at the end of tile kt - 1.  Tile kt + 1 goes from
// the registers into the other LDS buffer during the last 16-wide step, then
// the loads of tile kt + 2 are issued before the barrier, so a load has the
// barrier wait and the next tile's first fragment reads as extra cover.
// Tiles past the item's last are k tiles 0 and 1 of `nx`.
template <class C>
__device__ __forceinline__ void fast_load(u32x4 (&va)[C::CA], u32x4 (&vb)[C::CB], TileBase t,
                                          int kt, const FastOffsets<C>& o) {
  const uint16_t* la = t.a + kt * C::BK;
  const uint16_t* lb = t.b + kt * C::BK;
#pragma unroll
  for (int i = 0; i < C::CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(la + (o.a + i * o.sa));
#pragma unroll
  for (int i = 0; i < C::CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(lb + (o.b + i * o.sb));
}

template <class C>
__device__ __forceinline__ void fast_stage0_early(uint16_t (*smem)[C::LDS], TileBase tb,
                                                  const FastOffsets<C>& o, u32x4 (&va)[C::CA],
                                                  u32x4 (&vb)[C::CB]) {
  constexpr int RS = C::NT / C::CH, LDK = C::LDK;
  fast_load<C>(va, vb, tb, 0, o);
#pragma unroll
  for (int i = 0; i < C::CA; ++i) *reinterpret_cast<u32x4*>(smem[0] + o.wofs + i * RS * LDK) = va[i];
#pragma unroll
  for (int i = 0; i < C::CB; ++i)
    *reinterpret_cast<u32x4*>(smem[0] + C::BM * LDK + o.wofs + i * RS * LDK) = vb[i];
  fast_load<C>(va, vb, tb, 1, o);
  __syncthreads();
}

template <class C>
__device__ __forceinline__ void fast_kloop_early(f32x16 (&acc)[C::FM][C::FN],
                                                 uint16_t (*smem)[C::LDS], int buf, TileBase cur,
                                                 TileBase nx, const FastOffsets<C>& o, int nk,
                                                 int lane, int wm, int wn, u32x4 (&va)[C::CA],
                                                 u32x4 (&vb)[C::CB]) {
  constexpr int FM = C::FM, FN = C::FN, CA = C::CA, CB = C::CB;
  constexpr int BK = C::BK, LDK = C::LDK, STEPS = BK / 16;
  constexpr int NF = FM + FN, RS = C::NT / C::CH, MF = FM * FN;
  const int ra = (wm + (lane & 31)) * LDK + (lane >> 5) * 8;
  const int rb = (C::BM + wn + (lane & 31)) * LDK + (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cb = (kt + buf) & 1;
    const uint16_t* sa = smem[cb] + ra;
    const uint16_t* sb = smem[cb] + rb;
    uint16_t* dst = smem[cb ^ 1] + o.wofs;
    const int j = kt + 2;  // the tile the registers load next
    const TileBase lt = j < nk ? cur : nx;
    const int lk = j < nk ? j : j - nk;
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * LDK);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) fb[0][jj] = *reinterpret_cast<const bf16x8*>(sb + 32 * jj * LDK);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const int c = s & 1, n = c ^ 1;
      if (s + 1 < STEPS) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          fa[n][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * LDK + 16 * (s + 1));
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
          fb[n][jj] = *reinterpret_cast<const bf16x8*>(sb + 32 * jj * LDK + 16 * (s + 1));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][jj], acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(dst + i * RS * LDK) = va[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(dst + C::BM * LDK + i * RS * LDK) = vb[i];
    fast_load<C>(va, vb, lt, lk, o);
    __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);  // step 0 fragments
#pragma unroll
    for (int s = 0; s + 1 < STEPS; ++s) sched_interleave<MF, NF, 0x100, (NF + MF - 1) / MF>();
    sched_interleave<MF, CA + CB, 0x200, (CA + CB + MF - 1) / MF>();
    __builtin_amdgcn_sched_group_barrier(0x020, CA + CB, 0);  // tile kt + 2, global
    __syncthreads();
  }
}

template <class C>
__device__ __forceinline__ void mn_load(u32x4 (&va)[C::BK * MnOffsets<C>::CPA / C::NT],
                                        u32x4 (&vb)[C::BK * MnOffsets<C>::CPB / C::NT],
                                        TileBase t, int kt, const MnOffsets<C>& o, int64_t lda,
                                        int64_t ldb) {
  using O = MnOffsets<C>;
  constexpr int CA = C::BK * O::CPA / C::NT, CB = C::BK * O::CPB / C::NT;
  const uint16_t* la = t.a + (int64_t)kt * C::BK * lda;
  const uint16_t* lb = t.b + (int64_t)kt * C::BK * ldb;
#pragma unroll
  for (int i = 0; i < CA; ++i) va[i] = *reinterpret_cast<const u32x4*>(la + (o.a + i * o.sa));
#pragma unroll
  for (int i = 0; i < CB; ++i) vb[i] = *reinterpret_cast<const u32x4*>(lb + (o.b + i * o.sb));
}

template <class C>
__device__ __forceinline__ void mn_stage0_early(uint16_t (*smem)[C::LDS], TileBase tb,
                                                const MnOffsets<C>& o, int64_t lda, int64_t ldb,
                                                u32x4 (&va)[C::BK * MnOffsets<C>::CPA / C::NT],
                                                u32x4 (&vb)[C::BK * MnOffsets<C>::CPB / C::NT]) {
  using O = MnOffsets<C>;
  constexpr int CA = C::BK * O::CPA / C::NT, CB = C::BK * O::CPB / C::NT;
  mn_load<C>(va, vb, tb, 0, o, lda, ldb);
#pragma unroll
  for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(smem[0] + o.wa + i * O::RSA * O::PA) = va[i];
#pragma unroll
  for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(smem[0] + o.wb + i * O::RSB * O::PB) = vb[i];
  mn_load<C>(va, vb, tb, 1, o, lda, ldb);
  __syncthreads();
}

template <class C>
__device__ __forceinline__ void mn_kloop_early(f32x16 (&acc)[C::FM][C::FN],
                                               uint16_t (*smem)[C::LDS], int buf, TileBase cur,
                                               TileBase nx, const MnOffsets<C>& o, int64_t lda,
                                               int64_t ldb, int nk, int lane, int wm, int wn,
                                               u32x4 (&va)[C::BK * MnOffsets<C>::CPA / C::NT],
                                               u32x4 (&vb)[C::BK * MnOffsets<C>::CPB / C::NT]) {
  using O = MnOffsets<C>;
  constexpr int FM = C::FM, FN = C::FN, BK = C::BK, STEPS = BK / 16;
  constexpr int PA = O::PA, PB = O::PB;
  constexpr int CA = BK * O::CPA / C::NT, CB = BK * O::CPB / C::NT;
  constexpr int NF = 2 * (FM + FN), MF = FM * FN;
  const int g = lane >> 4, jl = lane & 15;
  const int ra = (8 * (g >> 1) + (jl >> 2)) * PA + 16 * (g & 1) + 4 * (jl & 3) + wm;
  const int rb = BK * PA + (8 * (g >> 1) + (jl >> 2)) * PB + 16 * (g & 1) + 4 * (jl & 3) + wn;
  for (int kt = 0; kt < nk; ++kt) {
    const int cb = (kt + buf) & 1;
    const uint16_t* sa = smem[cb] + ra;
    const uint16_t* sb = smem[cb] + rb;
    uint16_t* dst = smem[cb ^ 1];
    const int j = kt + 2;
    const TileBase lt = j < nk ? cur : nx;
    const int lk = j < nk ? j : j - nk;
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = frag_tr(sa + 32 * i, PA);
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) fb[0][jj] = frag_tr(sb + 32 * jj, PB);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int c = st & 1, n = c ^ 1;
      if (st + 1 < STEPS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[n][i] = frag_tr(sa + 32 * i + 16 * (st + 1) * PA, PA);
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) fb[n][jj] = frag_tr(sb + 32 * jj + 16 * (st + 1) * PB, PB);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj)
          acc[i][jj] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][jj], acc[i][jj], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) *reinterpret_cast<u32x4*>(dst + o.wa + i * O::RSA * PA) = va[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *reinterpret_cast<u32x4*>(dst + o.wb + i * O::RSB * PB) = vb[i];
    mn_load<C>(va, vb, lt, lk, o, lda, ldb);
    __builtin_amdgcn_sched_group_barrier(0x100, NF, 0);
#pragma unroll
    for (int st = 0; st + 1 < STEPS; ++st) sched_interleave<MF, NF, 0x100, (NF + MF - 1) / MF>();
    sched_interleave<MF, CA + CB, 0x200, (CA + CB + MF - 1) / MF>();
    __builtin_amdgcn_sched_group_barrier(0x020, CA + CB, 0);
    __syncthreads();
  }
}

template <class C>
__device__ __forceinline__ void mainloop_fast_mn(f32x16 (&acc)[C::FM][C::FN],
                                                 uint16_t (*smem)[C::LDS], const uint16_t* A,
                                                 int64_t lda, const uint16_t* B, int64_t ldb,
                                                 int m0, int n0, int nk, int lane, int wm,
                                                 int wn) {
  const MnOffsets<C> o(lda, ldb);
  const TileBase cur = {A + m0, B + n0};
  mn_stage0<C>(smem, 0, cur, o);
  // the last k tile reloads itself
  const TileBase nx = {cur.a + (int64_t)(nk - 1) * C::BK * lda, cur.b + (int64_t)(nk - 1) * C::BK * ldb};
  mn_kloop<C>(acc, smem, 0, cur, nx, o, lda, ldb, nk, lane, wm, wn);
}

// Epilogue of one tile by role (same accumulator layout as the 32x32 fp32
// MFMA: lane l holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + (v % 4)).
// ROLE_UPDATE's transposed copy goes through LDS when the whole tile is
// inside the output: each wave writes its accumulators transposed into
// Ts[col][row] (pitch BM + 8 bf16, 8-byte stores of 4 consecutive rows), then
// the block stores whole rows of X'^T with 16-byte stores (512 contiguous
// bytes per row of a 256-row tile) instead of 8-byte pieces of 32 different
// rows per instruction (measured 442 -> 381 us for the 32 x 4096 x 1024 x
// 1024 update; staging X' the same way gained nothing).  `lds` is the main
// loop's buffer, free once every wave has passed the main loop's last
// barrier.
template <class C>
constexpr bool kTransposeInLds = C::BN * (C::BM + 8) <= 2 * C::LDS;

// Every loop over the accumulators is unrolled in full (the plain pragma
// left the 4-wave 256 x 256 tile's loops rolled, and the indexed accumulator
// array then went through scratch memory: a kilobyte per lane written and
// read back per tile).
template <class C, int ROLE, int FM, int FN>
__device__ __forceinline__ void bf16_epilogue(f32x16 (&acc)[FM][FN], const GemmParams& p,
                                              const GemmProblem& pr, int b, int m0, int n0,
                                              int tile, int tiles, int lane, int wm, int wn,
                                              double* red, bool mirror, uint16_t* lds) {
  constexpr bool RESID = ROLE == ROLE_RESID;
  constexpr bool BF16_OUT = ROLE == ROLE_UPDATE;
  constexpr int PT = C::BM + 8;  // bf16 per row of the staged transposed tile
  const int hi = lane >> 5, col_in = lane & 31;
  bool t_lds = false;
  if constexpr (BF16_OUT && kTransposeInLds<C>) {
    const GemmProblem& tp = p.prob[1];
    t_lds = lds && tp.c && p.vec && m0 + C::BM <= p.M && n0 + C::BN <= p.N && tp.ldc % 8 == 0 &&
            tp.stride_c % 8 == 0 && ((uintptr_t)tp.c & 15) == 0;
  }
  float fro = 0.f;
#pragma clang loop unroll(full)
  for (int i = 0; i < FM; ++i)
#pragma clang loop unroll(full)
    for (int j = 0; j < FN; ++j) {
      const int col = n0 + wn + 32 * j + col_in;
#pragma clang loop unroll(full)
      for (int g = 0; g < 4; ++g) {
        const int row_base = m0 + wm + 32 * i + 8 * g + 4 * hi;
        uint32_t h[4];
#pragma clang loop unroll(full)
        for (int r = 0; r < 4; ++r) {
          const int row = row_base + r;
          float x = acc[i][j][4 * g + r];
          if (RESID) {
            x = (row == col ? 1.f : 0.f) - x;
            // one rounding per term, as in staged_epilogue (the same shares)
            if (row < p.M && col < p.N) fro = __builtin_fmaf(x, x, fro);
          }
          h[r] = bf16_rne(x);
          if (row < p.M && col < p.N) {
            const int64_t o = (int64_t)b * pr.stride_c + (int64_t)row * pr.ldc + col;
            if (BF16_OUT) reinterpret_cast<uint16_t*>(pr.c)[o] = (uint16_t)h[r];
            else pr.c[o] = x;
            if (RESID && p.prob[1].c) {
              const GemmProblem& hp = p.prob[1];
              reinterpret_cast<uint16_t*>(hp.c)[(int64_t)b * hp.stride_c +
                                                (int64_t)row * hp.ldc + col] = (uint16_t)h[r];
            }
          }
        }
        if (!BF16_OUT && mirror && col < p.N) {
          // symmetric output: the tile's transpose C[col][row_base .. + 3]
          // (off-diagonal tiles only), and of the bf16 copy of a residual
          float xs[4];
#pragma clang loop unroll(full)
          for (int r = 0; r < 4; ++r) {
            const int row = row_base + r;
            const float a = acc[i][j][4 * g + r];
            xs[r] = RESID ? ((row == col ? 1.f : 0.f) - a) : a;
          }
          float* Ct = pr.c + (int64_t)b * pr.stride_c + (int64_t)col * pr.ldc + row_base;
          uint16_t* Ht = (RESID && p.prob[1].c)
                             ? reinterpret_cast<uint16_t*>(p.prob[1].c) +
                                   (int64_t)b * p.prob[1].stride_c +
                                   (int64_t)col * p.prob[1].ldc + row_base
                             : nullptr;
#pragma clang loop unroll(full)
          for (int r = 0; r < 4; ++r)
            if (row_base + r < p.M) {
              Ct[r] = xs[r];
              if (Ht) Ht[r] = (uint16_t)h[r];
            }
        }
        if (BF16_OUT && t_lds) {
          // Ts[col - n0][row_base - m0 .. + 3]
          *reinterpret_cast<u32x2*>(lds + (col - n0) * PT + (row_base - m0)) = {
              h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        } else if (BF16_OUT && col < p.N && p.prob[1].c) {
          // transposed copy: X'^T[col][row_base .. row_base + 3]
          const GemmProblem& tp = p.prob[1];
          uint16_t* T = reinterpret_cast<uint16_t*>(tp.c) + (int64_t)b * tp.stride_c +
                        (int64_t)col * tp.ldc + row_base;
          if (p.vec && row_base + 3 < p.M) {
            *reinterpret_cast<u32x2*>(T) = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          } else {
#pragma clang loop unroll(full)
            for (int r = 0; r < 4; ++r)
              if (row_base + r < p.M) T[r] = (uint16_t)h[r];
          }
        }
      }
    }
  if constexpr (BF16_OUT && kTransposeInLds<C>) {
    if (t_lds) {
      __syncthreads();
      constexpr int CPR = C::BM / 8;  // 16-byte chunks per row of X'^T
      const GemmProblem& tp = p.prob[1];
      uint16_t* T = reinterpret_cast<uint16_t*>(tp.c) + (int64_t)b * tp.stride_c +
                    (int64_t)n0 * tp.ldc + m0;
#pragma unroll 4
      for (int idx = threadIdx.x; idx < C::BN * CPR; idx += C::NT) {
        const int cl = idx / CPR, q = idx - cl * CPR;
        *reinterpret_cast<u32x4*>(T + (int64_t)cl * tp.ldc + 8 * q) =
            *reinterpret_cast<const u32x4*>(lds + cl * PT + 8 * q);
      }
    }
  }
  if (mirror) fro *= 2.f;  // the tile stands for itself and its transpose
  if (RESID) {
    // the tile's Frobenius share; resid_decide_kernel sums them
    const double blocksum = block_sum<C::WAVES>((double)fro, red);
    if (threadIdx.x == 0) p.partials[(int64_t)b * p.partial_stride + tile] = blocksum;
  }
}

// ROLE_RESID: C fp32 = I - acc with the Frobenius share for the decision,
// and a bf16 copy at prob[1].c when set; ROLE_POWER: C fp32 = acc;
// ROLE_UPDATE: C bf16 = acc and its transpose at prob[1].c.
template <class C, int ROLE, bool MN = false>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_bf16_kernel(GemmParams p) {
  constexpr int FM = C::FM, FN = C::FN;
  constexpr int WGN = C::BN / C::WN;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][C::LDS];
  __shared__ double red[C::WAVES];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = (wid / WGN) * C::WM, wn = (wid % WGN) * C::WN;
  const bool vec = p.vec != 0;
  const bool sym = p.sym != 0;  // upper-triangle tiles only, mirrored on store
  const int tiles = sym ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch;
  const GemmProblem& pr = p.prob[0];

  // Workgroups are dealt to the 8 XCDs round-robin; with one block per tile
  // and 8 | total, XCD x takes the contiguous item range [x total / 8, ...),
  // so each XCD's L2 serves whole matrices.
  const bool xcd = p.map_mode != 0 && (int)gridDim.x == total && (total & 7) == 0;
  for (int it0 = blockIdx.x; it0 < total; it0 += gridDim.x) {
    const int it = xcd ? (it0 & 7) * (total >> 3) + (it0 >> 3) : it0;
    int b, tm, tn, tile;
    if (sym) item_tile_sym(it, p.tiles_m, &b, &tm, &tn, &tile);
    else item_tile(it, p.tiles_m, p.tiles_n, &b, &tm, &tn, &tile);
    if (p.ctrl) {
      const int st = *(volatile int32_t*)&p.ctrl[b].status;
      if (st != PMX_RUNNING) continue;
    }
    const uint16_t* A = reinterpret_cast<const uint16_t*>(pr.a.ptr) + (int64_t)b * pr.a.stride;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(pr.b.ptr) + (int64_t)b * pr.b.stride;
    const int m0 = tm * C::BM, n0 = tn * C::BN;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    const int nk = (p.K + C::BK - 1) / C::BK;
    __syncthreads();
    if constexpr (MN) {
      // operands m- / n-contiguous (whole tiles only: the launcher checks)
      mainloop_fast_mn<C>(acc, smem, A, pr.a.ld, B, pr.b.ld, m0, n0, nk, lane, wm, wn);
    } else if (vec && m0 + C::BM <= p.M && n0 + C::BN <= p.N && p.K % C::BK == 0) {
      mainloop_fast<C>(acc, smem, A, pr.a.ld, B, pr.b.ld, m0, n0, nk, lane, wm, wn);
    } else {
    u32x4 va[C::CA], vb[C::CB];
    load_chunks<C>(va, A, pr.a.ld, m0, p.M, 0, p.K, vec);
    load_chunks<C>(vb, B, pr.b.ld, n0, p.N, 0, p.K, vec);
    store_chunks<C>(smem[0], va);
    store_chunks<C>(smem[0] + C::BM * C::LDK, vb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        load_chunks<C>(va, A, pr.a.ld, m0, p.M, (kt + 1) * C::BK, p.K, vec);
        load_chunks<C>(vb, B, pr.b.ld, n0, p.N, (kt + 1) * C::BK, p.K, vec);
      }
      const uint16_t* sa = smem[cur] + (wm + (lane & 31)) * C::LDK + (lane >> 5) * 8;
      const uint16_t* sb = smem[cur] + (C::BM + wn + (lane & 31)) * C::LDK + (lane >> 5) * 8;
      // fragments of the next 16-wide k step are read while this one multiplies
      bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[0][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * C::LDK);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[0][j] = *reinterpret_cast<const bf16x8*>(sb + 32 * j * C::LDK);
#pragma unroll
      for (int s = 0; s < C::BK / 16; ++s) {
        const int c = s & 1, n = c ^ 1;
        if (s + 1 < C::BK / 16) {
#pragma unroll
          for (int i = 0; i < FM; ++i)
            fa[n][i] = *reinterpret_cast<const bf16x8*>(sa + 32 * i * C::LDK + 16 * (s + 1));
#pragma unroll
          for (int j = 0; j < FN; ++j)
            fb[n][j] = *reinterpret_cast<const bf16x8*>(sb + 32 * j * C::LDK + 16 * (s + 1));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
      }
      if (more) {
        store_chunks<C>(smem[cur ^ 1], va);
        store_chunks<C>(smem[cur ^ 1] + C::BM * C::LDK, vb);
      }
      __syncthreads();
    }
    }

    bf16_epilogue<C, ROLE>(acc, p, pr, b, m0, n0, tile, tiles, lane, wm, wn, red,
                           sym && tm != tn, &smem[0][0]);
  }
}

// The epilogue of a whole tile through LDS (`stage`: a free LDS buffer of
// the main loop).  The accumulator layout gives a lane four consecutive rows
// of one column, so direct stores write 2 (bf16) or 4 (fp32) bytes per lane,
// two rows per instruction.  Here the waves write a slice of their values
// row-major into LDS, then the block stores whole rows of the tile with
// 16-byte stores: X' (bf16) in two passes of 128 rows (fragments i = 2 p,
// 2 p + 1 of each wave row), fp32 outputs in four passes of 64 rows
// (fragment i = p), the residual's bf16 copy converted from the staged
// fp32 values.  Values, and the residual's Frobenius share (summed in the
// direct epilogue's order), are the direct epilogue's.
template <class C, int ROLE>
__device__ __forceinline__ void staged_epilogue(f32x16 (&acc)[C::FM][C::FN],
                                                const GemmParams& p, const GemmProblem& pr,
                                                int b, int m0, int n0, int tile, int lane,
                                                int wm, int wn, double* red, uint16_t* stage) {
  static_assert(C::BM == 256 && C::BN == 256 && C::WM == 128 && C::FM == 4, "256 x 256 tiles");
  constexpr bool RESID = ROLE == ROLE_RESID;
  const int hi = lane >> 5, col_in = lane & 31;
  const int wr = wm / 128;  // wave row (0, 1)
  if constexpr (ROLE == ROLE_UPDATE) {
    constexpr int PT = C::BN + 8;  // staged row pitch (bf16): 528 bytes
    static_assert(128 * PT <= C::LDS, "half a tile fits an LDS buffer");
    uint16_t* out = reinterpret_cast<uint16_t*>(pr.c) + (int64_t)b * pr.stride_c;
#pragma clang loop unroll(full)
    for (int pass = 0; pass < 2; ++pass) {
#pragma clang loop unroll(full)
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * pass + ii;
#pragma clang loop unroll(full)
        for (int j = 0; j < C::FN; ++j) {
          const int c = wn + 32 * j + col_in;
#pragma clang loop unroll(full)
          for (int g = 0; g < 4; ++g) {
#pragma clang loop unroll(full)
            for (int r = 0; r < 4; ++r) {
              const int srow = 64 * wr + 32 * ii + 8 * g + 4 * hi + r;
              stage[srow * PT + c] = (uint16_t)bf16_rne(acc[i][j][4 * g + r]);
            }
          }
        }
      }
      __syncthreads();
      // staged row R is tile row 128 (R / 64) + 64 pass + R % 64
#pragma unroll
      for (int q = threadIdx.x; q < 128 * (C::BN / 8); q += C::NT) {
        const int R = q / (C::BN / 8), ch = q % (C::BN / 8);
        const int row = m0 + 128 * (R >> 6) + 64 * pass + (R & 63);
        *reinterpret_cast<u32x4*>(out + (int64_t)row * pr.ldc + n0 + 8 * ch) =
            *reinterpret_cast<const u32x4*>(stage + R * PT + 8 * ch);
      }
      __syncthreads();
    }
  } else {
    constexpr int PF = C::BN + 4;  // staged row pitch (fp32): 1040 bytes
    static_assert(64 * PF * 4 <= C::LDS * 2, "a quarter tile fits an LDS buffer");
    float* st = reinterpret_cast<float*>(stage);
    float* out = pr.c + (int64_t)b * pr.stride_c;
    uint16_t* hout = nullptr;
    int64_t hld = 0;
    if (RESID && p.prob[1].c) {
      hout = reinterpret_cast<uint16_t*>(p.prob[1].c) + (int64_t)b * p.prob[1].stride_c;
      hld = p.prob[1].ldc;
    }
    float fro = 0.f;
#pragma clang loop unroll(full)
    for (int pass = 0; pass < 4; ++pass) {
      const int i = pass;
#pragma clang loop unroll(full)
      for (int j = 0; j < C::FN; ++j) {
        const int c = wn + 32 * j + col_in;
#pragma clang loop unroll(full)
        for (int g = 0; g < 4; ++g) {
#pragma clang loop unroll(full)
          for (int r = 0; r < 4; ++r) {
            float x = acc[i][j][4 * g + r];
            if (RESID) {
              const int row = wm + 32 * i + 8 * g + 4 * hi + r;
              x = (m0 + row == n0 + c ? 1.f : 0.f) - x;
              fro = __builtin_fmaf(x, x, fro);
            }
            st[(32 * wr + 8 * g + 4 * hi + r) * PF + c] = x;
          }
        }
      }
      __syncthreads();
      // staged row R is tile row 128 (R / 32) + 32 pass + R % 32
#pragma unroll
      for (int q = threadIdx.x; q < 64 * (C::BN / 4); q += C::NT) {
        const int R = q / (C::BN / 4), ch = q % (C::BN / 4);
        const int row = m0 + 128 * (R >> 5) + 32 * pass + (R & 31);
        const f32x4 v = *reinterpret_cast<const f32x4*>(st + R * PF + 4 * ch);
        *reinterpret_cast<f32x4*>(out + (int64_t)row * pr.ldc + n0 + 4 * ch) = v;
        if (RESID && hout) {
          *reinterpret_cast<u32x2*>(hout + (int64_t)row * hld + n0 + 4 * ch) = {
              bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
        }
      }
      __syncthreads();
    }
    if (RESID) {
      // the tile's Frobenius share; resid_decide_kernel sums them
      const double blocksum = block_sum<C::WAVES>((double)fro, red);
      if (threadIdx.x == 0) p.partials[(int64_t)b * p.partial_stride + tile] = blocksum;
    }
  }
}

// Persistent form for launches of whole tiles (k-contiguous operands, or the
// m-contiguous residual): one block per CU walks its items, and the last k
// tile of an item loads k tile 0 of the block's next item before the item's
// epilogue stores are issued.  The next item then starts with its first k
// tile staged, and the stores drain under its main loop (loads and stores
// share one in-order counter, so a first load issued after the stores would
// wait for them).  The blocks of one XCD (block index x mod 8) take a
// contiguous range of items, as many at a time as the XCD has blocks.  The
// epilogue goes through the free LDS buffer (staged_epilogue): no transposed
// copy, and output rows that allow 16-byte stores.  EARLY (items of at least
// two k tiles): the k loops issue each k tile's loads before the previous
// tile's barrier (fast_kloop_early, mn_kloop_early): across the epilogue the
// next item's k tile 0 is staged and its k tile 1 in flight.
template <class C, int ROLE, bool MN, bool EARLY = false>
__global__ __launch_bounds__(C::NT, C::MINB) void gemm_bf16_persist_kernel(GemmParams p) {
  constexpr int FM = C::FM, FN = C::FN;
  constexpr int WGN = C::BN / C::WN;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][C::LDS];
  __shared__ double red[C::WAVES];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = (wid / WGN) * C::WM, wn = (wid % WGN) * C::WN;
  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch;
  const GemmProblem& pr = p.prob[0];
  const int nk = p.K / C::BK;
  const int64_t lda = pr.a.ld, ldb = pr.b.ld;
  const bool xcd = p.map_mode != 0 && (gridDim.x & 7) == 0 && (total & 7) == 0;
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3, per = total >> 3, g8 = gridDim.x >> 3;
  int r = 0;
  // the block's next item of a running matrix
  auto next_item = [&](int& b, int& tm, int& tn, int& tile) -> bool {
    for (;;) {
      int L;
      if (xcd) {
        const int jx = q + r * g8;
        if (jx >= per) return false;
        L = x * per + jx;
      } else {
        L = blockIdx.x + r * (int)gridDim.x;
        if (L >= total) return false;
      }
      ++r;
      item_tile(L, p.tiles_m, p.tiles_n, &b, &tm, &tn, &tile);
      if (!p.ctrl || *(volatile int32_t*)&p.ctrl[b].status == PMX_RUNNING) return true;
    }
  };
  auto base_of = [&](int b, int tm, int tn) -> TileBase {
    const uint16_t* A = reinterpret_cast<const uint16_t*>(pr.a.ptr) + (int64_t)b * pr.a.stride;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(pr.b.ptr) + (int64_t)b * pr.b.stride;
    if constexpr (MN) return {A + tm * C::BM, B + tn * C::BN};
    else return {A + (int64_t)(tm * C::BM) * lda, B + (int64_t)(tn * C::BN) * ldb};
  };
  int b, tm, tn, tile;
  if (!next_item(b, tm, tn, tile)) return;
  TileBase cur = base_of(b, tm, tn);
  using Off = std::conditional_t<MN, MnOffsets<C>, FastOffsets<C>>;
  const Off o(lda, ldb);
  int buf = 0;
  using LA = u32x4[MN ? C::BK * MnOffsets<C>::CPA / C::NT : C::CA];
  using LB = u32x4[MN ? C::BK * MnOffsets<C>::CPB / C::NT : C::CB];
  LA va;
  LB vb;
  if constexpr (EARLY) {
    if constexpr (MN) mn_stage0_early<C>(smem, cur, o, lda, ldb, va, vb);
    else fast_stage0_early<C>(smem, cur, o, va, vb);
  } else {
    if constexpr (MN) mn_stage0<C>(smem, buf, cur, o);
    else fast_stage0<C>(smem, buf, cur, o);
  }
  for (;;) {
    int b2 = b, tm2 = tm, tn2 = tn, tile2 = tile;
    const bool more = next_item(b2, tm2, tn2, tile2);
    // without a next item the last k tile loads this item's k tile 0 again
    const TileBase nx = more ? base_of(b2, tm2, tn2) : cur;
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    if constexpr (EARLY) {
      if constexpr (MN) mn_kloop_early<C>(acc, smem, buf, cur, nx, o, lda, ldb, nk, lane, wm, wn, va, vb);
      else fast_kloop_early<C>(acc, smem, buf, cur, nx, o, nk, lane, wm, wn, va, vb);
    } else {
      if constexpr (MN) mn_kloop<C>(acc, smem, buf, cur, nx, o, lda, ldb, nk, lane, wm, wn);
      else fast_kloop<C>(acc, smem, buf, cur, nx, o, nk, lane, wm, wn);
    }
    // the buffer the last k tile was read from is free until the next item's
    // first k tile step stores into it
    staged_epilogue<C, ROLE>(acc, p, pr, b, tm * C::BM, tn * C::BN, tile, lane, wm, wn, red,
                             smem[(buf + nk - 1) & 1]);
    if (!more) break;
    buf = (buf + nk) & 1;
    b = b2;
    tm = tm2;
    tn = tn2;
    tile = tile2;
    cur = nx;
  }
}

// ---------------------------------------------------------------------------
// Whole-tile variant with direct global-to-LDS loads (global_load_lds_dwordx4:
// lane l of a wave writes its 16 bytes at the instruction's LDS base + 16 l).
// 256 x 256 tiles, 8 waves of 128 x 64, k tiles of 32 in a ring of 4 LDS
// stages (32 KB each), so three k tiles are in flight while one is
// multiplied.  No padding is possible inside a wave's contiguous 1 KB, so
// rows are XOR-swizzled instead: the 16-byte chunk kc of row R sits in slot
// 4 R + (kc ^ f(R)), f(R) = ((R >> 1) ^ (R >> 3)) & 3, which keeps the
// fragment reads of 16 consecutive rows on distinct banks.  Waits are
// explicit (vmcnt plus a bare s_barrier, no memory fence): before the
// barrier that starts k tile t + 1 a wave waits for its own loads of that
// tile; after it, the stage of tile t is refilled with tile t + 4 and the
// first fragments of tile t + 1 are read while the last MFMAs of tile t still
// run.  Used when M and N are multiples of 256, K of 32 and rows are
// 16-byte aligned.
constexpr int DBK = 32, DNS = 4;
constexpr int DOPB = 256 * DBK * 2;  // bytes per operand and stage
constexpr int DSTB = 2 * DOPB;       // bytes per stage
using BDma = BCfg<256, 256, 128, 64, 32, 1>;

__device__ __forceinline__ int dma_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int ROLE>
__global__ __launch_bounds__(512, 1) void gemm_bf16_dma_kernel(GemmParams p) {
  using C = BDma;
  constexpr int FM = C::FM, FN = C::FN;  // 4 x 2 accumulators per wave
  __shared__ __attribute__((aligned(16))) unsigned char lds[DNS * DSTB];
  __shared__ double red[C::WAVES];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = (wid >> 2) * 128, wn = (wid & 3) * 64;
  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.batch;
  const GemmProblem& pr = p.prob[0];
  const int nk = p.K / DBK;
  const int sw = dma_swz(lane & 31);
  // this lane's DMA slots: instruction j covers slots (2 wid + j) 64 + lane
  int rowj[2], kcj[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int slot = (2 * wid + j) * 64 + lane;
    rowj[j] = slot >> 2;
    kcj[j] = (slot & 3) ^ dma_swz(slot >> 2);
  }
  const bool xcd = p.map_mode != 0 && (int)gridDim.x == total && (total & 7) == 0;
  for (int it0 = blockIdx.x; it0 < total; it0 += gridDim.x) {
    const int it = xcd ? (it0 & 7) * (total >> 3) + (it0 >> 3) : it0;
    int b, tm, tn, tile;
    item_tile(it, p.tiles_m, p.tiles_n, &b, &tm, &tn, &tile);
    if (p.ctrl) {
      const int st = *(volatile int32_t*)&p.ctrl[b].status;
      if (st != PMX_RUNNING) continue;
    }
    const int m0 = tm * 256, n0 = tn * 256;
    const uint16_t* A = reinterpret_cast<const uint16_t*>(pr.a.ptr) + (int64_t)b * pr.a.stride;
    const uint16_t* B = reinterpret_cast<const uint16_t*>(pr.b.ptr) + (int64_t)b * pr.b.stride;
    const uint16_t* ga[2];
    const uint16_t* gb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ga[j] = A + (int64_t)(m0 + rowj[j]) * pr.a.ld + 8 * kcj[j];
      gb[j] = B + (int64_t)(n0 + rowj[j]) * pr.b.ld + 8 * kcj[j];
    }
    auto issue = [&](int t) {
      const int tc = t < nk ? t : nk - 1;  // past the end: reload the last tile
      unsigned char* st = lds + (t & (DNS - 1)) * DSTB;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(ga[j] + tc * DBK),
                                         (lds_ptr_t)(st + (2 * wid + j) * 1024), 16, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(gb[j] + tc * DBK),
                                         (lds_ptr_t)(st + DOPB + (2 * wid + j) * 1024), 16, 0, 0);
    };
    // fragment i of A / j of B, 16-wide k step s of the k tile in stage st
    auto frag_a = [&](int st, int i, int s) {
      const int r = wm + 32 * i + (lane & 31);
      const int kc = 2 * s + (lane >> 5);
      return *reinterpret_cast<const bf16x8*>(lds + st * DSTB + (r * 4 + (kc ^ sw)) * 16);
    };
    auto frag_b = [&](int st, int j, int s) {
      const int r = wn + 32 * j + (lane & 31);
      const int kc = 2 * s + (lane >> 5);
      return *reinterpret_cast<const bf16x8*>(lds + st * DSTB + DOPB + (r * 4 + (kc ^ sw)) * 16);
    };
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // the previous item's LDS reads are done
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    issue(0);
    issue(1);
    issue(2);
    issue(3);
    __builtin_amdgcn_s_waitcnt(0x3f7c);  // vmcnt(12): tile 0 has landed for this wave
    __builtin_amdgcn_s_barrier();
    bf16x8 fa[2][FM], fb[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[0][i] = frag_a(0, i, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = frag_b(0, j, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & (DNS - 1), nst = (kt + 1) & (DNS - 1);
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[1][i] = frag_a(st, i, 1);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[1][j] = frag_b(st, j, 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0][i], fb[0][j], acc[i][j], 0, 0, 0);
      // step 0: its 8 MFMAs interleaved with the 6 fragment reads of step 1
      sched_interleave<FM * FN, FM + FN, 0x100, 1>();
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1][i], fb[1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, FM * FN, 0);
      // tile kt + 1 landed for this wave, then for every wave; the stage of
      // tile kt is free again
      __builtin_amdgcn_s_waitcnt(0x3f78);  // vmcnt(8)
      __builtin_amdgcn_s_barrier();
      issue(kt + 4);
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[0][i] = frag_a(nst, i, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[0][j] = frag_b(nst, j, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // the trailing reloads are done
    bf16_epilogue<C, ROLE>(acc, p, pr, b, m0, n0, tile, tiles, lane, wm, wn, red, false,
                           nullptr);
  }
}

// After a residual launch: the decision kernel over its `tiles` shares per matrix.
hipError_t after_resid(const GemmParams& p, int role, int tiles, hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || role != ROLE_RESID) return e;
  ResidDecide d;
  d.ctrl = p.ctrl;
  d.partials = p.partials;
  d.partial_stride = p.partial_stride;
  d.tiles = tiles;
  d.products = p.products;
  d.count_update = p.count_update;
  d.cfg = p.cfg;
  return launch_resid_decide(d, p.batch, s);
}

hipError_t launch_dma(GemmParams p, int role, hipStream_t s) {
  p.tiles_m = p.M / 256;
  p.tiles_n = p.N / 256;
  const int64_t total = (int64_t)p.tiles_m * p.tiles_n * p.batch;
  int64_t g = total;
  if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
  const dim3 grid((unsigned)g), block(512);
  switch (role) {
    case ROLE_RESID: hipLaunchKernelGGL(gemm_bf16_dma_kernel<ROLE_RESID>, grid, block, 0, s, p); break;
    case ROLE_POWER: hipLaunchKernelGGL(gemm_bf16_dma_kernel<ROLE_POWER>, grid, block, 0, s, p); break;
    case ROLE_UPDATE: hipLaunchKernelGGL(gemm_bf16_dma_kernel<ROLE_UPDATE>, grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return after_resid(p, role, (int)(total / p.batch), s);
}

// Whole 256 x 256 x 64 tiles of 16-byte aligned rows: the shapes the
// persistent form and the m-contiguous residual take.
template <class C>
bool whole_aligned(const GemmParams& p) {
  return p.vec && p.M % C::BM == 0 && p.N % C::BN == 0 && p.K % C::BK == 0 && p.K >= C::BK &&
         p.prob[0].a.ld % 8 == 0 && p.prob[0].b.ld % 8 == 0 && p.prob[0].a.stride % 8 == 0 &&
         p.prob[0].b.stride % 8 == 0 && ((uintptr_t)p.prob[0].a.ptr & 15) == 0 &&
         ((uintptr_t)p.prob[0].b.ptr & 15) == 0;
}

template <class C>
hipError_t launch_cfg(GemmParams p, int role, hipStream_t s) {
  p.tiles_m = (p.M + C::BM - 1) / C::BM;
  p.tiles_n = (p.N + C::BN - 1) / C::BN;
  if constexpr (C::BM == 256 && C::BN == 256 && C::BK == 64 && C::WM == 128 && C::WN == 64) {
    const GemmProblem& oc = p.prob[0];
    const int cq = role == ROLE_UPDATE ? 8 : 4;  // elements per 16-byte store
    bool out_ok = oc.ldc % cq == 0 && oc.stride_c % cq == 0 && ((uintptr_t)oc.c & 15) == 0;
    if (role == ROLE_UPDATE) out_ok = out_ok && !p.prob[1].c;
    if (role == ROLE_RESID && p.prob[1].c)
      out_ok = out_ok && p.prob[1].ldc % 4 == 0 && p.prob[1].stride_c % 4 == 0 &&
               ((uintptr_t)p.prob[1].c & 7) == 0;
    if (p.persist && !p.sym && whole_aligned<C>(p) && out_ok && (!p.mn || role == ROLE_RESID)) {
      const int64_t total = (int64_t)p.tiles_m * p.tiles_n * p.batch;
      const int64_t cu = p.num_cu > 0 ? p.num_cu : 256;
      const dim3 grid((unsigned)(total < cu ? total : cu)), block(C::NT);
      const bool early = p.early && p.K >= 2 * C::BK;
      if (early) {
        if (p.mn) {
          hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_RESID, true, true>), grid, block, 0, s, p);
        } else {
          switch (role) {
            case ROLE_RESID:
              hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_RESID, false, true>), grid, block, 0, s, p);
              break;
            case ROLE_POWER:
              hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_POWER, false, true>), grid, block, 0, s, p);
              break;
            case ROLE_UPDATE:
              hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_UPDATE, false, true>), grid, block, 0, s, p);
              break;
            default: return hipErrorInvalidValue;
          }
        }
        return after_resid(p, role, (int)(total / p.batch), s);
      }
      if (p.mn) {
        hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_RESID, true>), grid, block, 0, s, p);
      } else {
        switch (role) {
          case ROLE_RESID:
            hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_RESID, false>), grid, block, 0, s, p);
            break;
          case ROLE_POWER:
            hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_POWER, false>), grid, block, 0, s, p);
            break;
          case ROLE_UPDATE:
            hipLaunchKernelGGL((gemm_bf16_persist_kernel<C, ROLE_UPDATE, false>), grid, block, 0, s, p);
            break;
          default: return hipErrorInvalidValue;
        }
      }
      return after_resid(p, role, (int)(total / p.batch), s);
    }
  }
  if (p.mn) {
    // m- / n-contiguous operands: the residual on whole 256 x 256 x 64 tiles
    if constexpr (C::BM == 256 && C::BN == 256 && C::BK == 64 && C::WM == 128 && C::WN == 64) {
      if (role != ROLE_RESID || p.sym || !whole_aligned<C>(p)) return hipErrorInvalidValue;
      const int64_t total = (int64_t)p.tiles_m * p.tiles_n * p.batch;
      int64_t g = total;
      if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
      hipLaunchKernelGGL((gemm_bf16_kernel<C, ROLE_RESID, true>), dim3((unsigned)g),
                         dim3(C::NT), 0, s, p);
      return after_resid(p, role, (int)(total / p.batch), s);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (p.sym && (C::BM != C::BN || p.M != p.N || role == ROLE_UPDATE)) return hipErrorInvalidValue;
  const int64_t total = (p.sym ? (int64_t)p.tiles_m * (p.tiles_m + 1) / 2
                               : (int64_t)p.tiles_m * p.tiles_n) * p.batch;
  int64_t g = total;
  if (p.max_blocks > 0 && g > p.max_blocks) g = p.max_blocks;
  const dim3 grid((unsigned)g), block(C::NT);
  switch (role) {
    case ROLE_RESID: hipLaunchKernelGGL((gemm_bf16_kernel<C, ROLE_RESID>), grid, block, 0, s, p); break;
    case ROLE_POWER: hipLaunchKernelGGL((gemm_bf16_kernel<C, ROLE_POWER>), grid, block, 0, s, p); break;
    case ROLE_UPDATE: hipLaunchKernelGGL((gemm_bf16_kernel<C, ROLE_UPDATE>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return after_resid(p, role, (int)(total / p.batch), s);
}

}  // namespace

// C = A Bs^T with A (M x K) and Bs (N x K) bf16, k contiguous.  Roles:
// ROLE_RESID (C fp32 = I - A Bs^T, convergence, optional bf16 copy at
// prob[1].c / ldc / stride_c), ROLE_POWER (C fp32),
// ROLE_UPDATE (C bf16 and its transpose at prob[1].c / ldc / stride_c).
hipError_t launch_gemm_bf16(const GemmParams& p, int role, hipStream_t s) {
  // the large tile once it still gives every compute unit a tile
  const int64_t large = (int64_t)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.batch;
  int cfg = p.cfg_id;
  if (cfg < 0 || cfg > 3) cfg = (p.M >= 256 && p.N >= 256 && large >= p.num_cu) ? 1 : 0;
  if (p.mn) return launch_cfg<BLarge>(p, role, s);
  if (p.sym) {
    // square tiles (the 256 x 256 tile, or 128 x 128 when forced with 0)
    if (cfg == 2 || cfg == 3) cfg = 1;
    if (cfg == 1 && p.sym_small) cfg = 0;
    if (cfg == 1) return launch_cfg<BLarge>(p, role, s);
    return launch_cfg<BSmall>(p, role, s);
  }
  if (cfg == 2) return launch_cfg<BLarge4>(p, role, s);
  if (cfg == 3) return launch_cfg<BMid2>(p, role, s);
  if (cfg == 1 && p.dma == 1 && p.vec && p.M % 256 == 0 && p.N % 256 == 0 && p.K % DBK == 0 &&
      p.K >= DBK && ((uintptr_t)p.prob[0].a.ptr & 15) == 0 && ((uintptr_t)p.prob[0].b.ptr & 15) == 0)
    return launch_dma(p, role, s);
  return cfg == 1 ? launch_cfg<BLarge>(p, role, s) : launch_cfg<BSmall>(p, role, s);
}

}  // namespace pmx
