// Bandwidth- and latency-bound kernels of the PRISM iteration on gfx950:
// control reset, input scaling, stage set-up, the skinny Krylov products
// R^j S with the fused Gram / alpha fit, the explicit polynomial g for the
// first update, and the scaled outputs.
#include <math.h>

#include "pmx_alpha.h"
#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ int32_t load_status(const Ctrl* c) {
  return *(const volatile int32_t*)&c->status;
}

}  // namespace

// ---------------------------------------------------------------- control
__global__ void ctrl_reset_kernel(Ctrl* ctrl, pmx_matfn_info* info, int batch, int degree,
                                  uint32_t* zero, int nzero) {
  const int b = blockIdx.x;
  for (int i = b * blockDim.x + threadIdx.x; i < nzero; i += gridDim.x * blockDim.x) zero[i] = 0u;
  if (b >= batch) return;
  if (threadIdx.x == 0) {
    Ctrl c;
    c.c = 0.0;
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
    ctrl[b] = c;
  }
  if (info) {
    int32_t* w = reinterpret_cast<int32_t*>(info + b);
    const int words = (int)(sizeof(pmx_matfn_info) / 4);
    for (int i = threadIdx.x; i < words; i += blockDim.x) w[i] = 0;
  }
}

// ---------------------------------------------------------------- scale
// c = ||X||_F over an rows x cols matrix (fp32 or bf16), fp64 accumulation,
// deterministic last-block reduction.  Sets status NONFINITE if c is not a
// positive finite number.
template <typename T>
__global__ __launch_bounds__(NT) void fro_scale_kernel(const T* __restrict__ X, int rows,
                                                       int cols, int64_t ld, int64_t stride,
                                                       int vec, Ctrl* ctrl, double* partials,
                                                       int64_t pstride, pmx_matfn_info* info) {
  const int b = blockIdx.y;
  const T* x = X + (int64_t)b * stride;
  double acc = 0.0;
  // sum of squares of the 4 fp32 or 8 bf16 values of a 16-byte load
  auto sumsq = [](const uint4 w) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (sizeof(T) == 2) {
        const double lo = (double)__uint_as_float(u[i] << 16);
        const double hi = (double)__uint_as_float(u[i] & 0xFFFF0000u);
        a += lo * lo + hi * hi;
      } else {
        const double v = (double)__uint_as_float(u[i]);
        a += v * v;
      }
    }
    return a;
  };
  constexpr int V = 16 / sizeof(T);
  if (vec && ld == cols) {
    // contiguous rows: one stream of 16-byte loads over the whole matrix,
    // four in flight per thread (a row of 1024 bf16 is only 128 loads, so
    // row-by-row left half of the block idle and one load in flight)
    const uint4* v4 = reinterpret_cast<const uint4*>(x);
    const int64_t nv = (int64_t)rows * cols / V;
    const int64_t step = (int64_t)gridDim.x * NT;
    int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    for (; i + 3 * step < nv; i += 4 * step) {
      const uint4 w0 = v4[i], w1 = v4[i + step], w2 = v4[i + 2 * step], w3 = v4[i + 3 * step];
      acc += sumsq(w0) + sumsq(w1) + sumsq(w2) + sumsq(w3);
    }
    for (; i < nv; i += step) acc += sumsq(v4[i]);
  } else if (vec) {
    // 16-byte loads: 8 bf16 or 4 fp32 per load (rows, ld and the base aligned)
    const int cv = cols / V;
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
      const uint4* row = reinterpret_cast<const uint4*>(x + (int64_t)r * ld);
      for (int c = threadIdx.x; c < cv; c += NT) acc += sumsq(row[c]);
    }
  } else {
    for (int r = blockIdx.x; r < rows; r += gridDim.x)
    for (int c = threadIdx.x; c < cols; c += NT) {
      const double v = (double)to_f32(x[(int64_t)r * ld + c]);
      acc += v * v;
    }
  }
  __shared__ double red[NT / 64];
  const double bs = block_sum<NT / 64>(acc, red);
  double tot;
  if (last_block_sum<NT / 64>(bs, partials + (int64_t)b * pstride, &ctrl[b].counter,
                              gridDim.x, blockIdx.x, red, &tot)) {
    if (threadIdx.x == 0) {
      Ctrl& c = ctrl[b];
      const double s = sqrt(tot);
      c.c = s;
      c.fro = s;  // the Krylov scaling of a power estimate on A / c
      if (info) info[b].scale = (float)s;
      if (!(s > 0.0) || !isfinite(s)) {
        c.status = PMX_NONFINITE;
        c.status_all = PMX_NONFINITE;
        if (info) info[b].status = PMX_NONFINITE;
      }
    }
  }
}

// ---------------------------------------------------------------- stage init
// Coupled square-root stage set-up: Y_0 = scale * src (src = A for stage 0,
// the previous stage's Y for stage 1), R_0 = I - Y_0 (Z_0 = I), the
// convergence decision on r_0, and the first sketch S_0.
__global__ __launch_bounds__(NT) void sqrt_stage_init_kernel(StageInitParams p) {
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
    src = p.ybuf[it & 1] + (int64_t)b * p.buf_stride;
    sld = n;
  }
  const float fs = (float)scale;
  float* y0 = p.ybuf[0] + (int64_t)b * p.buf_stride;
  float* R = p.r + (int64_t)b * p.buf_stride;
  double acc = 0.0;
  const bool flat = sld == n && n % 4 == 0 && ((uintptr_t)src & 15) == 0 &&
                    ((uintptr_t)y0 & 15) == 0 && ((uintptr_t)R & 15) == 0;
  if (flat) {
    // contiguous: one stream of 16-byte accesses over the matrix, four
    // loads in flight per thread
    const float4* s4 = reinterpret_cast<const float4*>(src);
    float4* y4 = reinterpret_cast<float4*>(y0);
    float4* r4 = reinterpret_cast<float4*>(R);
    const int64_t nv = (int64_t)n * n / 4;
    const int64_t step = (int64_t)gridDim.x * NT;
    auto put = [&](int64_t i, float4 a) {
      const int64_t e = 4 * i;
      const int r = (int)(e / n), c = (int)(e - (int64_t)r * n);  // 4 | n: one row
      const float y[4] = {a.x * fs, a.y * fs, a.z * fs, a.w * fs};
      float rv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rv[j] = (r == c + j ? 1.f : 0.f) - y[j];
        acc += (double)rv[j] * (double)rv[j];
      }
      y4[i] = make_float4(y[0], y[1], y[2], y[3]);
      r4[i] = make_float4(rv[0], rv[1], rv[2], rv[3]);
    };
    int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    for (; i + 3 * step < nv; i += 4 * step) {
      const float4 a0 = s4[i], a1 = s4[i + step], a2 = s4[i + 2 * step], a3 = s4[i + 3 * step];
      put(i, a0);
      put(i + step, a1);
      put(i + 2 * step, a2);
      put(i + 3 * step, a3);
    }
    for (; i < nv; i += step) put(i, s4[i]);
  } else {
    for (int r = blockIdx.x; r < n; r += gridDim.x)
    for (int c = threadIdx.x; c < n; c += NT) {
      const int64_t e = (int64_t)r * n + c;
      const float y = src[(int64_t)r * sld + c] * fs;
      y0[e] = y;
      const float rv = (r == c ? 1.f : 0.f) - y;
      R[e] = rv;
      acc += (double)rv * (double)rv;
    }
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
      cb->degree_next = p.cfg.degree;  // every stage starts at the configured degree
      decide(*cb, p.cfg, p.cfg.info ? p.cfg.info + b : nullptr, tot);
    }
  }
}

// Polar set-up: X_0 = G / c (transposed when the iteration runs on G^T).
template <typename T>
__global__ __launch_bounds__(NT) void polar_init_kernel(PolarInitParams p) {
  const int b = blockIdx.y;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  sketch_share(p.sketch, b, blockIdx.x, gridDim.x);
  const T* g = reinterpret_cast<const T*>(p.g) + (int64_t)b * p.g_stride;
  T* x = reinterpret_cast<T*>(p.x) + (int64_t)b * p.x_stride;
  const float fs = (float)(1.0 / cb->c);
  for (int r = blockIdx.x; r < p.rows; r += gridDim.x)
  for (int c = threadIdx.x; c < p.cols; c += NT) {
    const int64_t e = (int64_t)r * p.cols + c;
    const float v = p.transpose ? to_f32(g[(int64_t)c * p.ldg + r]) : to_f32(g[(int64_t)r * p.ldg + c]);
    x[e] = from_f32<T>(v * fs);
  }
}

// ---------------------------------------------------------------- skinny products
// Recursive-halving reduction over a 64-lane wave of CNT values per lane
// (CNT a power of two): at the step with offset O the lanes with bit O set
// keep the upper half of their remaining values and add the partner's copy of
// it; once one value is left the remaining offsets add plainly.  Lane l ends
// with the wave-wide sum of value index l / (64 / CNT) in acc[0] (CNT <= 64),
// or of value indices (CNT / 64) l + i in acc[i] (CNT >= 64).
template <int CNT, int O>
__device__ __forceinline__ void halve_reduce(float* acc, int lane) {
  if constexpr (O >= 1) {
    if constexpr (CNT > 1) {
      constexpr int H = CNT / 2;
      const bool upper = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? acc[i] : acc[i + H];
        const float keep = upper ? acc[i + H] : acc[i];
        acc[i] = keep + __shfl_xor(send, O, 64);
      }
      halve_reduce<H, O / 2>(acc, lane);
    } else {
      acc[0] += __shfl_xor(acc[0], O, 64);
      halve_reduce<1, O / 2>(acc, lane);
    }
  }
}

// out[:, oc : oc + q] = ||R||_F^-pow * Mat * in[:, ic : ic + q] for an n x n Mat
// and an n x q block of the Krylov buffer (q <= Q).  HBM-bound on Mat, read
// once with 16-byte loads: a block of 4 waves owns 4 RW rows (RW per wave);
// RW = 2 keeps a single n = 4096 matrix at 512 blocks, RW = 8 serves batches,
// where it cuts the LDS reads of In per byte of Mat by four.  In is staged
// column-major through LDS in chunks of 512 rows (conflict-free 16-byte
// reads) and shared by the block's rows.  Each lane accumulates RW x Q
// partial sums over its columns; the wave's recursive-halving reduction leaves
// the complete sums spread over the lanes.
// GJ != 0 (last Krylov pass, J <= |GJ| Krylov blocks): every block also adds its rows' share of the
// J x J Gram of K_1..K_J in fp64; the last block to arrive reduces the
// shares in block order and solves for alpha.
constexpr int SK_CH = 512;           // In rows per LDS chunk
constexpr int SK_LD = SK_CH + 4;     // column stride of the staged chunk

// Reduction, output and (GJ != 0) Gram share / alpha fit of a skinny product:
// acc holds the lane's RW x Q partial sums for rows row0 .. row0 + RW - 1.
// The output factor of a skinny product: ||R||_F^-pow, 1 for the complement.
__device__ __forceinline__ float skinny_scale(int pow, double fro) {
  return (float)(pow == 1 ? 1.0 / fro : pow == 2 ? 1.0 / (fro * fro) : 1.0);
}

template <int Q, int RW, int GJ, int NW = NT / 64>
__device__ __forceinline__ void skinny_finish(float (&acc)[RW * Q], const SkinnyParams& p,
                                              const SkinnyJob& job, int b, int row0,
                                              float scale, double fro) {
  constexpr int CNT = RW * Q;
  constexpr int NV = CNT > 64 ? CNT / 64 : 1;
  constexpr int SHARE = CNT < 64 ? 64 / CNT : 1;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int n = p.n;
  Ctrl* cb = p.ctrl + b;
  float* kb = p.kbuf + (int64_t)b * p.kstride;
  halve_reduce<CNT, 32>(acc, lane);
  // lane l holds value indices NV l .. NV l + NV - 1 (CNT >= 64) or l / SHARE
  bool valid[NV];
  int vrow[NV], vcol[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = CNT >= 64 ? NV * lane + i : lane / SHARE;
    const int rr = idx / Q, c = idx - rr * Q;
    vrow[i] = row0 + rr;
    vcol[i] = c;
    valid[i] = (lane % SHARE) == 0 && vrow[i] < n && c < p.q;
    acc[i] *= scale;
    if (job.pow == 0 && valid[i]) acc[i] = kb[(int64_t)vrow[i] * p.kld + job.in_col + c] - acc[i];
    if (valid[i]) kb[(int64_t)vrow[i] * p.kld + job.out_col + c] = acc[i];
  }

  if constexpr (GJ != 0) {
    // the block's share of the Gram entries (a, bb), a <= bb < J <= GJ, of
    // K_1..K_J, J = 2 d + 1 for the matrix's current degree d (gram_j when
    // set: 9 for the inverse Newton objective with p = 4); this pass writes
    // K_jo, the others are read back.  gram_alpha_kernel sums the shares.
    constexpr int GA = GJ;
    const int deg = *(const volatile int32_t*)&cb->degree;
    constexpr int NE = GA * (GA + 1) / 2;
    const int J = p.gram_j ? p.gram_j : 2 * deg + 1;
    const int pp = p.cfg.p;
    const int jo = job.out_col / pp;
    double g[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) g[e] = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      double v[GA];
#pragma unroll
      for (int j = 0; j < GA; ++j) v[j] = 0.0;
      if (valid[i]) {
#pragma unroll
        for (int j = 1; j <= GA; ++j)
          if (j <= J)
            v[j - 1] = j == jo ? (double)acc[i]
                               : (double)kb[(int64_t)vrow[i] * p.kld + j * pp + vcol[i]];
      }
      int t = 0;
#pragma unroll
      for (int a = 0; a < GA; ++a)
#pragma unroll
        for (int bb = a; bb < GA; ++bb, ++t) g[t] += v[a] * v[bb];
    }
    // entries of (a, bb) with a <= bb < J, in row order, are packed first
    __shared__ double wsum[NW][NE];
    if constexpr (NE <= 16) {
      // recursive halving over the wave (17 exchanges for 15 sums): lane l
      // ends with the sum of entry l / 4, which lands at its packed index
      // a J - a (a - 1) / 2 + bb - a when a, bb < J
      double h[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) h[e] = e < NE ? g[e] : 0.0;
      halve_reduce_d<16, 32>(h, lane);
      const int t = lane >> 2;
      if ((lane & 3) == 0 && t < NE) {
        int a = 0, rem = t;
        while (rem >= GA - a) {
          rem -= GA - a;
          ++a;
        }
        const int bb = a + rem;
        if (a < J && bb < J) wsum[wid][a * J - a * (a - 1) / 2 + (bb - a)] = h[0];
      }
    } else {
      int t = 0, o = 0;
#pragma unroll
      for (int a = 0; a < GA; ++a)
#pragma unroll
        for (int bb = a; bb < GA; ++bb, ++t) {
          const double sv = wave_sum(g[t]);
          if (a < J && bb < J) {
            if (lane == 0) wsum[wid][o] = sv;
            ++o;
          }
        }
    }
    const int ng = J * (J + 1) / 2;
    __syncthreads();
    double* part = p.gram_partials + (int64_t)b * p.gram_stride;
    if (threadIdx.x < ng)
      part[(int64_t)blockIdx.x * kGramShare + threadIdx.x] =
          [&] {
            double t = wsum[0][threadIdx.x];
            for (int w = 1; w < NW; ++w) t += wsum[w][threadIdx.x];
            return t;
          }();
  }
}

// After a Gram pass (the kernel boundary orders the shares before this): one
// block per matrix sums the pass's `nblocks` shares of every Gram entry with
// a fixed lane assignment and reduction tree (deterministic; one wave for
// J <= 5, one wave per entry above), and solves for alpha: the square-root /
// polar family's quartic, or the inverse Newton objective (newton_p = 4).
// Then the adaptive degree's decision, the product count and the alpha
// trace.
__global__ __launch_bounds__(NT) void gram_alpha_kernel(SkinnyParams p, int nblocks) {
  const int b = blockIdx.x;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int deg = *(const volatile int32_t*)&cb->degree;
  const int J = p.gram_j ? p.gram_j : 2 * deg + 1;
  const int ng = J * (J + 1) / 2;
  const double fro = cb->fro;
  const double* part = p.gram_partials + (int64_t)b * p.gram_stride;
  __shared__ double gsum[kGramShare];
  if (ng <= 16) {
    // one wave: lane l adds the shares of blocks l, l + 64, ... (the 15
    // entries of up to four blocks read together), then the 16 sums are
    // halved across the wave (the same fixed tree every call)
    if (wid == 0) {
      double h[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) h[e] = 0.0;
      for (int i0 = lane; i0 < nblocks; i0 += 256) {
        double v[4][16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + 64 * u;
          const double* row = part + (int64_t)(i < nblocks ? i : 0) * kGramShare;
#pragma unroll
          for (int e = 0; e < 16; ++e) v[u][e] = (i < nblocks && e < ng) ? row[e] : 0.0;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) h[e] += (v[0][e] + v[1][e]) + (v[2][e] + v[3][e]);
      }
      halve_reduce_d<16, 32>(h, lane);
      if ((lane & 3) == 0 && (lane >> 2) < ng) gsum[lane >> 2] = h[0];
    }
  } else {
    for (int e = wid; e < ng; e += NT / 64) {
      double sv = 0.0;
      for (int i = lane; i < nblocks; i += 64) sv += part[(int64_t)i * kGramShare + e];
      sv = wave_sum(sv);
      if (lane == 0) gsum[e] = sv;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double phi = 0.0;
  const bool up = deg > p.cfg.degree;
  double alpha;
  if (p.newton_p == 4) {
    if (J == 9)
      alpha = alpha_from_gram_newton<9, 5>(gsum, fro, p.coef_n, p.cfg.lo, p.cfg.hi, &phi);
    else
      alpha = alpha_from_gram_newton<5, 5>(gsum, fro, p.coef_n, p.cfg.lo, p.cfg.hi, &phi);
  } else {
    alpha = alpha_from_gram(gsum, J, fro, up ? p.coef_up : p.coef, up ? p.lo_up : p.cfg.lo,
                            up ? p.hi_up : p.cfg.hi, &phi);
  }
  cb->alpha = alpha;
  // adaptive degree: the sketch predicts ||R_{k+1} S|| / ||R_k S|| =
  // sqrt(phi_S(alpha)) / ||R S|| (gsum[0] = ||K_1||^2 of the scaled K_1 = R S / s)
  if (deg < p.cfg.degree_max) {
    const double m11 = gsum[0] * fro * fro;
    const double q = m11 > 0.0 ? sqrt(fmax(phi, 0.0) / m11) : 0.0;
    if (q > (double)p.cfg.adapt_ratio) cb->degree_next = deg + 1;
  }
  cb->sketch_products += J;
  const int k = cb->iter;
  if (p.cfg.info && k < PMX_TRACE_LEN) p.cfg.info[b].alpha[cb->stage][k] = (float)alpha;
}

// The same product on the matrix cores, for 16-byte-aligned Mat (n % 4 == 0):
// a block owns 16 rows of Mat and its W waves split the columns into W equal
// slices.  Each wave runs v_mfma_f32_16x16x4_f32 along its slice with 16 x 4
// tiles of Mat as A and the matching 4 x 16 tiles of In as B (columns >= q
// are zero), so one value of In read from L2 serves 16 rows and nothing is
// staged in LDS (the LDS-staged forms above read Q values of In a value of
// Mat).  Lane l holds A[l % 16][k] and B[k][l % 16] for the k-slot l / 16; a
// float4 load of Mat feeds four products.  The W partial 16 x 16 tiles are
// summed through LDS in wave order; wave w then finishes rows w 16/W ..
// (w + 1) 16/W - 1.
typedef float sk_f32x4 __attribute__((ext_vector_type(4)));

template <int Q, int W, int GJ>
__global__ __launch_bounds__(W * 64) void skinny_mfma_kernel(SkinnyParams p) {
  constexpr int RW = 16 / W;  // rows finished by each wave
  constexpr int UN = 4;       // 16-column steps with loads in flight together
  const int b = blockIdx.z;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const SkinnyJob& job = p.job[blockIdx.y];
  const int n = p.n;
  const float* __restrict__ mat = job.mat + (int64_t)b * job.mat_stride;
  float* kb = p.kbuf + (int64_t)b * p.kstride;
  const double fro = cb->fro;
  const float scale = skinny_scale(job.pow, fro);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const bool rok = row0 + r < n;
  const float* arow = mat + (int64_t)(rok ? row0 + r : 0) * job.mat_ld;
  const bool cok = r < p.q;
  const float* xcol = kb + job.in_col + (cok ? r : 0);
  const int kper = (n + 16 * W - 1) / (16 * W) * 16;  // a multiple of 16
  const int kbeg = wid * kper;
  const int kend = n < kbeg + kper ? n : kbeg + kper;  // a multiple of 4
  sk_f32x4 c = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = kbeg; k0 < kend; k0 += 16 * UN) {
    float4 a[UN];
    float x[UN][4];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int k = k0 + 16 * u + 4 * slot;
      const bool kok = k < kend;  // then k + 3 < kend as well
      a[u] = rok && kok ? *reinterpret_cast<const float4*>(arow + k)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = cok && kok ? xcol[(int64_t)(k + i) * p.kld] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].x, x[u][0], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].y, x[u][1], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].z, x[u][2], c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u].w, x[u][3], c, 0, 0, 0);
    }
  }
  // lane l holds D[4 (l / 16) + v][l % 16], v = 0 .. 3
  __shared__ float red[W][16][17];
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wid][4 * slot + v][r] = c[v];
  __syncthreads();
  float tot = 0.f;
  if (lane < RW * Q) {
    const int rr = wid * RW + lane / Q, cc = lane - (lane / Q) * Q;
    for (int w = 0; w < W; ++w) tot += red[w][rr][cc];
  }
  // value (i / Q, i % Q) sits in lane i alone; the finish sums over lanes
  float acc[RW * Q];
#pragma unroll
  for (int i = 0; i < RW * Q; ++i) acc[i] = lane == i ? tot : 0.f;
  skinny_finish<Q, RW, GJ, W>(acc, p, job, b, row0 + wid * RW, scale, fro);
}

// The batched form on the matrix cores (many matrices of a moderate order,
// where one pass must stream every matrix once at HBM speed): a block of
// SB_W = 8 waves owns 128 rows of one matrix and each wave 16 of them over
// the full contraction, so there is no cross-wave reduction.  In (n x q) is
// staged per SB_CH-row chunk in LDS transposed, In^T[c][k] with row stride
// SB_LD (SB_LD = 4 mod 32: the 16-byte reads of eight lanes cover all 32
// banks), so one 16-byte LDS read gives a lane the four values of In that
// match its 16-byte read of Mat: lane (slot = l / 16, r = l % 16) carries
// k = 16 u + 4 slot .. + 3 of row r into v_mfma_f32_16x16x4_f32 as A and
// In[k][r] as B.  Mat is read SB_UN steps at a time into two register sets
// in turn, so one set is in flight while the other is multiplied, and a
// chunk's first reads are issued before In is staged.  (Measured on the 32
// Muon residuals and the 64 blocks of order 512: 8 waves with 4-step sets
// beat 4 waves and 16-step sets, with or without the second set.)  Rows of In beyond n and columns beyond q
// are staged as zero.  GJ = 5 (last Krylov pass, J = 2 d + 1 <= 5 blocks):
// the block's share of the Gram, as in skinny_finish, reduced by recursive
// halving over the wave and then over the waves in order.
constexpr int SB_CH = 1024;
constexpr int SB_LD = SB_CH + 4;
constexpr int SB_W = 8;
constexpr int SB_UN = 4;

template <int Q, int GJ>
__global__ __launch_bounds__(SB_W * 64) void skinny_batch_kernel(SkinnyParams p) {
  static_assert(Q == 8 || Q == 16, "Q");
  static_assert(GJ == 0 || GJ == 5, "GJ");
  const int b = blockIdx.z;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const SkinnyJob& job = p.job[blockIdx.y];
  const int n = p.n;
  const float* __restrict__ mat = job.mat + (int64_t)b * job.mat_stride;
  float* kb = p.kbuf + (int64_t)b * p.kstride;
  const double fro = cb->fro;
  const float scale = skinny_scale(job.pow, fro);
  __shared__ __attribute__((aligned(16))) float inT[Q * SB_LD];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = lane & 15, slot = lane >> 4;
  const int rbase = blockIdx.x * (16 * SB_W) + 16 * wid;
  const int row = rbase + r;
  const bool rok = row < n;
  const float* arow = mat + (int64_t)(rok ? row : 0) * job.mat_ld + 4 * slot;
  // B reads: column r of In^T (rows q .. Q - 1 are staged as zero; for
  // Q = 8 the lanes r >= 8 read row 0: a product's column r depends on B's
  // column r alone, and those columns are not stored)
  const float* brow = inT + (r < Q ? r : 0) * SB_LD + 4 * slot;
  const bool in_vec = (p.kld % 4 == 0) && (job.in_col % 4 == 0) && (p.q == Q) &&
                      ((((uintptr_t)kb) & 15) == 0);
  sk_f32x4 c = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < n; j0 += SB_CH) {
    const int len = n - j0 < SB_CH ? n - j0 : SB_CH;  // a multiple of 4
    const int U = (len + 15) >> 4;  // 16-column steps; the last may be partial
    auto load_a = [&](float4 (&a)[SB_UN], int u0) {
#pragma unroll
      for (int i = 0; i < SB_UN; ++i) {
        const int kk = 16 * (u0 + i) + 4 * slot;  // then kk + 3 < len as well
        a[i] = (rok && kk < len) ? *reinterpret_cast<const float4*>(arow + j0 + 16 * (u0 + i))
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    // In^T beyond len is zero, and the row stride leaves room for the
    // partial last step (16 u + 4 slot + 3 < SB_CH + 4)
    auto mul = [&](const float4 (&a)[SB_UN], int u0) {
#pragma unroll
      for (int i = 0; i < SB_UN; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(brow + 16 * (u0 + i));
        if (u0 + i < U) {
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].x, x.x, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].y, x.y, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].z, x.z, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i].w, x.w, c, 0, 0, 0);
        }
      }
    };
    float4 ba[SB_UN], bb[SB_UN];
    load_a(ba, 0);
    __syncthreads();
    // rows [0, lim) of the chunk are read by the products below
    const int lim = 16 * U;
    if (in_vec) {
      for (int idx = threadIdx.x; idx < lim * (Q / 4); idx += SB_W * 64) {
        const int jj = idx / (Q / 4), cc = 4 * (idx - jj * (Q / 4));
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (jj < len)
          v = *reinterpret_cast<const float4*>(kb + (int64_t)(j0 + jj) * p.kld + job.in_col + cc);
        inT[(cc + 0) * SB_LD + jj] = v.x;
        inT[(cc + 1) * SB_LD + jj] = v.y;
        inT[(cc + 2) * SB_LD + jj] = v.z;
        inT[(cc + 3) * SB_LD + jj] = v.w;
      }
    } else {
      for (int idx = threadIdx.x; idx < lim * Q; idx += SB_W * 64) {
        const int jj = idx / Q, cc = idx - jj * Q;
        float v = 0.f;
        if (jj < len && cc < p.q) v = kb[(int64_t)(j0 + jj) * p.kld + job.in_col + cc];
        inT[cc * SB_LD + jj] = v;
      }
    }
    __syncthreads();
    for (int u0 = 0; u0 < U; u0 += 2 * SB_UN) {
      load_a(bb, u0 + SB_UN);
      mul(ba, u0);
      load_a(ba, u0 + 2 * SB_UN);
      mul(bb, u0 + SB_UN);
    }
  }
  // lane l holds D[4 (l / 16) + v][l % 16]: rows rbase + 4 slot + v, column r
  const int col = r;
  float outv[4];
  bool valid[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int orow = rbase + 4 * slot + v;
    valid[v] = orow < n && col < p.q;
    float a = c[v] * scale;
    if (job.pow == 0 && valid[v]) a = kb[(int64_t)orow * p.kld + job.in_col + col] - a;
    if (valid[v]) kb[(int64_t)orow * p.kld + job.out_col + col] = a;
    outv[v] = a;
  }
  if constexpr (GJ != 0) {
    constexpr int GA = GJ, NE = GA * (GA + 1) / 2;  // 15, reduced as 16
    const int deg = *(const volatile int32_t*)&cb->degree;
    const int J = 2 * deg + 1;
    const int pp = p.cfg.p;
    const int jo = job.out_col / pp;
    double g[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) g[e] = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double x[GA];
#pragma unroll
      for (int j = 0; j < GA; ++j) x[j] = 0.0;
      if (valid[v]) {
        const int orow = rbase + 4 * slot + v;
#pragma unroll
        for (int j = 1; j <= GA; ++j)
          if (j <= J)
            x[j - 1] = j == jo ? (double)outv[v]
                               : (double)kb[(int64_t)orow * p.kld + j * pp + col];
      }
      int t = 0;
#pragma unroll
      for (int a = 0; a < GA; ++a)
#pragma unroll
        for (int bb = a; bb < GA; ++bb, ++t) g[t] += x[a] * x[bb];
    }
    // lane l ends with the wave's sum of value l / 4
    halve_reduce_d<16, 32>(g, lane);
    __shared__ double wsum[SB_W][16];
    if ((lane & 3) == 0) wsum[wid][lane >> 2] = g[0];
    __syncthreads();
    const int ng = J * (J + 1) / 2;
    if (threadIdx.x < ng) {
      // packed index e -> index t of (a, bb) in the GA enumeration
      int t = 0, o = 0, te = 0;
      for (int a = 0; a < GA; ++a)
        for (int bb = a; bb < GA; ++bb, ++t)
          if (a < J && bb < J) {
            if (o == (int)threadIdx.x) te = t;
            ++o;
          }
      double tot = wsum[0][te];
      for (int w = 1; w < SB_W; ++w) tot += wsum[w][te];
      double* part = p.gram_partials + (int64_t)b * p.gram_stride;
      part[(int64_t)blockIdx.x * kGramShare + threadIdx.x] = tot;
    }
    (void)NE;
  }
}

template <int Q, int RW, int GJ>
__global__ __launch_bounds__(NT) void skinny_kernel(SkinnyParams p) {
  constexpr int CNT = RW * Q;  // partial sums per lane
  constexpr int RB = 4 * RW;
  const int b = blockIdx.z;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const SkinnyJob& job = p.job[blockIdx.y];
  const int n = p.n;
  const float* __restrict__ mat = job.mat + (int64_t)b * job.mat_stride;
  float* kb = p.kbuf + (int64_t)b * p.kstride;
  const double fro = cb->fro;
  const float scale = skinny_scale(job.pow, fro);

  __shared__ __attribute__((aligned(16))) float in_lds[Q * SK_LD];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int row0 = blockIdx.x * RB + wid * RW;
  const bool vec = (job.mat_ld % 4 == 0) && ((((uintptr_t)mat) & 15) == 0);
  const bool in_vec = (p.kld % 4 == 0) && (job.in_col % 4 == 0) && (p.q == Q) &&
                      ((((uintptr_t)kb) & 15) == 0);

  float acc[CNT];
#pragma unroll
  for (int i = 0; i < CNT; ++i) acc[i] = 0.f;

  for (int j0 = 0; j0 < n; j0 += SK_CH) {
    __syncthreads();
    // stage In[j0 .. j0 + 512)[0 .. Q) column-major (zero beyond n and q)
    if (in_vec) {
      // one 16-byte load per (row, 4 columns)
      for (int idx = threadIdx.x; idx < SK_CH * (Q / 4); idx += NT) {
        const int jj = idx / (Q / 4), c = 4 * (idx - jj * (Q / 4));
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j0 + jj < n)
          v = *reinterpret_cast<const float4*>(kb + (int64_t)(j0 + jj) * p.kld + job.in_col + c);
        in_lds[(c + 0) * SK_LD + jj] = v.x;
        in_lds[(c + 1) * SK_LD + jj] = v.y;
        in_lds[(c + 2) * SK_LD + jj] = v.z;
        in_lds[(c + 3) * SK_LD + jj] = v.w;
      }
    } else {
      for (int idx = threadIdx.x; idx < SK_CH * Q; idx += NT) {
        const int jj = idx / Q, c = idx - jj * Q;
        float v = 0.f;
        if (j0 + jj < n && c < p.q) v = kb[(int64_t)(j0 + jj) * p.kld + job.in_col + c];
        in_lds[c * SK_LD + jj] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < SK_CH / 256; ++t) {
      const int jj = 256 * t + 4 * lane;
      const int j = j0 + jj;
      if (j >= n) continue;
      float4 m[RW];
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const int row = row0 + rr;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < n) {
          const float* src = mat + (int64_t)row * job.mat_ld + j;
          if (vec && j + 3 < n) {
            v = *reinterpret_cast<const float4*>(src);
          } else {
            v.x = src[0];
            if (j + 1 < n) v.y = src[1];
            if (j + 2 < n) v.z = src[2];
            if (j + 3 < n) v.w = src[3];
          }
        }
        m[rr] = v;
      }
#pragma unroll
      for (int c = 0; c < Q; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(in_lds + c * SK_LD + jj);
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
          acc[rr * Q + c] += m[rr].x * x.x + m[rr].y * x.y + m[rr].z * x.z + m[rr].w * x.w;
      }
    }
  }
  skinny_finish<Q, RW, GJ>(acc, p, job, b, row0, scale, fro);
}

// The same product software-pipelined: while chunk c (CH rows of In, CH
// columns of Mat) is multiplied, the Mat loads and the In staging loads of
// chunk c + 1 are in flight; In is double buffered in LDS, so there is one
// barrier per chunk.
template <int Q, int RW, int CH, int GJ>
__global__ __launch_bounds__(NT) void skinny_pipe_kernel(SkinnyParams p) {
  constexpr int CNT = RW * Q;
  constexpr int RB = 4 * RW;
  constexpr int T = CH / 256;            // 4-column steps per lane per chunk
  constexpr int LD = CH + 4;             // column stride of a staged chunk
  constexpr int IV = CH * Q / 4 / NT;    // 16-byte In loads per thread per chunk
  static_assert(IV >= 1 && IV * NT * 4 == CH * Q, "chunk / thread mismatch");
  const int b = blockIdx.z;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const SkinnyJob& job = p.job[blockIdx.y];
  const int n = p.n;
  const float* __restrict__ mat = job.mat + (int64_t)b * job.mat_stride;
  const float* __restrict__ in = p.kbuf + (int64_t)b * p.kstride + job.in_col;
  const double fro = cb->fro;
  const float scale = skinny_scale(job.pow, fro);
  __shared__ __attribute__((aligned(16))) float in_lds[2][Q * LD];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int row0 = blockIdx.x * RB + wid * RW;
  const bool vec = (job.mat_ld % 4 == 0) && ((((uintptr_t)mat) & 15) == 0) && (n % 4 == 0);
  const bool in_vec = (p.kld % 4 == 0) && (job.in_col % 4 == 0) && (p.q == Q) &&
                      ((((uintptr_t)p.kbuf) & 15) == 0) && (p.kstride % 4 == 0);

  auto load_m = [&](float4 (&m)[T][RW], int j0) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int j = j0 + 256 * t + 4 * lane;
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const int row = row0 + rr;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < n && j < n) {
          const float* src = mat + (int64_t)row * job.mat_ld + j;
          if (vec) {
            v = *reinterpret_cast<const float4*>(src);
          } else {
            v.x = src[0];
            if (j + 1 < n) v.y = src[1];
            if (j + 2 < n) v.z = src[2];
            if (j + 3 < n) v.w = src[3];
          }
        }
        m[t][rr] = v;
      }
    }
  };
  // In chunk rows j0 .. j0 + CH, thread item idx -> (row idx / (Q / 4), 4 columns)
  auto load_in = [&](float4 (&iv)[IV], int j0) {
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int idx = threadIdx.x + NT * i;
      const int jj = idx / (Q / 4), c = 4 * (idx % (Q / 4));
      const int j = j0 + jj;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < n) {
        const float* src = in + (int64_t)j * p.kld + c;
        if (in_vec) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (c + 0 < p.q) v.x = src[0];
          if (c + 1 < p.q) v.y = src[1];
          if (c + 2 < p.q) v.z = src[2];
          if (c + 3 < p.q) v.w = src[3];
        }
      }
      iv[i] = v;
    }
  };
  auto store_in = [&](float* lds, const float4 (&iv)[IV]) {
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int idx = threadIdx.x + NT * i;
      const int jj = idx / (Q / 4), c = 4 * (idx % (Q / 4));
      lds[(c + 0) * LD + jj] = iv[i].x;
      lds[(c + 1) * LD + jj] = iv[i].y;
      lds[(c + 2) * LD + jj] = iv[i].z;
      lds[(c + 3) * LD + jj] = iv[i].w;
    }
  };

  float acc[CNT];
#pragma unroll
  for (int i = 0; i < CNT; ++i) acc[i] = 0.f;
  float4 m[T][RW], mn[T][RW], iv[IV];
  load_m(m, 0);
  load_in(iv, 0);
  store_in(in_lds[0], iv);
  __syncthreads();
  const int nch = (n + CH - 1) / CH;
  for (int c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    if (more) {
      load_m(mn, (c + 1) * CH);
      load_in(iv, (c + 1) * CH);
    }
    const float* lds = in_lds[c & 1];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int jj = 256 * t + 4 * lane;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const float4 x = *reinterpret_cast<const float4*>(lds + q * LD + jj);
#pragma unroll
        for (int rr = 0; rr < RW; ++rr)
          acc[rr * Q + q] += m[t][rr].x * x.x + m[t][rr].y * x.y + m[t][rr].z * x.z + m[t][rr].w * x.w;
      }
    }
    if (more) store_in(in_lds[(c + 1) & 1], iv);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) m[t][rr] = mn[t][rr];
    }
  }
  skinny_finish<Q, RW, GJ>(acc, p, job, b, row0, scale, fro);
}

// The same product without LDS: each lane reads the In rows of its four
// columns directly (16-byte loads, L1/L2 resident: In is n x q) next to the
// RW rows of Mat, so a block has no barriers and keeps its loads in flight.
template <int Q, int RW, int GJ>
__global__ __launch_bounds__(NT) void skinny_stream_kernel(SkinnyParams p) {
  constexpr int CNT = RW * Q;
  constexpr int RB = 4 * RW;
  const int b = blockIdx.z;
  Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const SkinnyJob& job = p.job[blockIdx.y];
  const int n = p.n;
  const float* __restrict__ mat = job.mat + (int64_t)b * job.mat_stride;
  const float* __restrict__ in = p.kbuf + (int64_t)b * p.kstride + job.in_col;
  const double fro = cb->fro;
  const float scale = skinny_scale(job.pow, fro);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int row0 = blockIdx.x * RB + wid * RW;
  const bool vec = (job.mat_ld % 4 == 0) && ((((uintptr_t)mat) & 15) == 0) && (n % 4 == 0) &&
                   (p.kld % 4 == 0) && (job.in_col % 4 == 0) && (p.q == Q) &&
                   ((((uintptr_t)p.kbuf) & 15) == 0) && (p.kstride % 4 == 0);
  float acc[CNT];
#pragma unroll
  for (int i = 0; i < CNT; ++i) acc[i] = 0.f;
  if (vec) {
#pragma unroll 2
    for (int j = 4 * lane; j < n; j += 256) {
      float4 m[RW];
#pragma unroll
      for (int rr = 0; rr < RW; ++rr)
        m[rr] = (row0 + rr < n)
                    ? *reinterpret_cast<const float4*>(mat + (int64_t)(row0 + rr) * job.mat_ld + j)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 x[4][Q / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c4 = 0; c4 < Q / 4; ++c4)
          x[u][c4] = *reinterpret_cast<const float4*>(in + (int64_t)(j + u) * p.kld + 4 * c4);
#pragma unroll
      for (int rr = 0; rr < RW; ++rr)
#pragma unroll
        for (int c4 = 0; c4 < Q / 4; ++c4) {
          float* a = acc + rr * Q + 4 * c4;
          a[0] += m[rr].x * x[0][c4].x + m[rr].y * x[1][c4].x + m[rr].z * x[2][c4].x + m[rr].w * x[3][c4].x;
          a[1] += m[rr].x * x[0][c4].y + m[rr].y * x[1][c4].y + m[rr].z * x[2][c4].y + m[rr].w * x[3][c4].y;
          a[2] += m[rr].x * x[0][c4].z + m[rr].y * x[1][c4].z + m[rr].z * x[2][c4].z + m[rr].w * x[3][c4].z;
          a[3] += m[rr].x * x[0][c4].w + m[rr].y * x[1][c4].w + m[rr].z * x[2][c4].w + m[rr].w * x[3][c4].w;
        }
    }
  } else {
    for (int j = 4 * lane; j < n; j += 256) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j + u >= n) break;
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
          if (row0 + rr >= n) break;
          const float mv = mat[(int64_t)(row0 + rr) * job.mat_ld + j + u];
#pragma unroll
          for (int c = 0; c < Q; ++c)
            if (c < p.q) acc[rr * Q + c] += mv * in[(int64_t)(j + u) * p.kld + c];
        }
      }
    }
  }
  skinny_finish<Q, RW, GJ>(acc, p, job, b, row0, scale, fro);
}

// ---------------------------------------------------------------- polynomial
// g = c_0 I + c_1 R + alpha R^2 (d = 2) or c_0 I + alpha R (d = 1), written
// explicitly: it is Z_1 of the coupled iteration (Z_0 = I).
__global__ __launch_bounds__(NT) void form_g_kernel(FormGParams p) {
  const int b = blockIdx.y;
  const Ctrl* cb = p.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  sketch_share(p.sketch, b, blockIdx.x, gridDim.x);
  // the estimated scale of the polar factor: g / s in the first update
  const float fs = p.first_scale && cb->inv_s > 0.0 ? (float)cb->inv_s : 1.f;
  const float alpha = fs * (float)cb->alpha;
  const int n = p.n;
  const float* R = p.r + (int64_t)b * p.stride;
  const float* R2 = p.r2 ? p.r2 + (int64_t)b * p.stride : nullptr;
  float* G = p.dst_bf16 ? nullptr : reinterpret_cast<float*>(p.dst) + (int64_t)b * p.stride;
  uint16_t* Gh = p.dst_bf16 ? reinterpret_cast<uint16_t*>(p.dst) + (int64_t)b * p.stride : nullptr;
  float* G2 = p.dst2 ? p.dst2 + (int64_t)b * p.stride : nullptr;
  const float* R3 = p.r3 ? p.r3 + (int64_t)b * p.stride : nullptr;
  const float c0 = fs * p.c0, c1 = fs * p.c1, c2 = fs * p.c2;
  const int deg = p.adaptive ? *(const volatile int32_t*)&cb->degree : p.degree;
  const bool d1 = deg == 1, d3 = deg == 3;
  if (p.vec) {
    // four columns per thread (n % 4 == 0, stride % 4 == 0)
    const int nv = n / 4;
    for (int r = blockIdx.x; r < n; r += gridDim.x)
    for (int c4 = threadIdx.x; c4 < nv; c4 += NT) {
      const int64_t e = (int64_t)r * n + 4 * c4;
      const float4 x = *reinterpret_cast<const float4*>(R + e);
      float4 v;
      if (d1) {
        v = make_float4(alpha * x.x, alpha * x.y, alpha * x.z, alpha * x.w);
      } else if (d3) {
        const float4 y = *reinterpret_cast<const float4*>(R2 + e);
        const float4 z = *reinterpret_cast<const float4*>(R3 + e);
        v = make_float4(c1 * x.x + c2 * y.x + alpha * z.x, c1 * x.y + c2 * y.y + alpha * z.y,
                        c1 * x.z + c2 * y.z + alpha * z.z, c1 * x.w + c2 * y.w + alpha * z.w);
      } else {
        const float4 y = *reinterpret_cast<const float4*>(R2 + e);
        v = make_float4(c1 * x.x + alpha * y.x, c1 * x.y + alpha * y.y, c1 * x.z + alpha * y.z,
                        c1 * x.w + alpha * y.w);
      }
      const int dc = r - 4 * c4;
      if (dc == 0) v.x += c0;
      if (dc == 1) v.y += c0;
      if (dc == 2) v.z += c0;
      if (dc == 3) v.w += c0;
      if (Gh) {
        const uint32_t h0 = from_f32<bf16_t>(v.x).bits, h1 = from_f32<bf16_t>(v.y).bits;
        const uint32_t h2 = from_f32<bf16_t>(v.z).bits, h3 = from_f32<bf16_t>(v.w).bits;
        *reinterpret_cast<uint2*>(Gh + e) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
      } else {
        *reinterpret_cast<float4*>(G + e) = v;
      }
      if (G2) *reinterpret_cast<float4*>(G2 + e) = v;
    }
    return;
  }
  for (int r = blockIdx.x; r < n; r += gridDim.x)
  for (int c = threadIdx.x; c < n; c += NT) {
    const int64_t e = (int64_t)r * n + c;
    float v;
    if (d1) v = alpha * R[e];
    else if (d3) v = c1 * R[e] + c2 * R2[e] + alpha * R3[e];
    else v = c1 * R[e] + alpha * R2[e];
    if (r == c) v += c0;
    if (Gh) Gh[e] = from_f32<bf16_t>(v).bits;
    else G[e] = v;
    if (G2) G2[e] = v;
  }
}

// ---------------------------------------------------------------- conversion
template <typename TI, typename TO>
__global__ __launch_bounds__(NT) void convert_kernel(const TI* __restrict__ src, int64_t lds,
                                                     int64_t ss, TO* __restrict__ dst,
                                                     int64_t ldd, int64_t sd, int rows, int cols) {
  const int b = blockIdx.y;
  const TI* x = src + (int64_t)b * ss;
  TO* y = dst + (int64_t)b * sd;
  for (int r = blockIdx.x; r < rows; r += gridDim.x)
  for (int c = threadIdx.x; c < cols; c += NT) {
    y[(int64_t)r * ldd + c] = from_f32<TO>(to_f32(x[(int64_t)r * lds + c]));
  }
}

// ---------------------------------------------------------------- variable-size blocks
// One shape group of large variable-size blocks: blocks[idx[b]] is packed
// into dst[b] (m x n fp32, dense) and, after the batched iteration, src[b]
// goes back to blocks[idx[b]].u (rounded to nearest even for bf16) with the
// group's info record to info[idx[b]].
__global__ __launch_bounds__(NT) void varbatch_gather_kernel(const pmx_polar_block* blocks,
                                                             const int32_t* idx, int bf16,
                                                             float* dst, int m, int n) {
  const int b = blockIdx.y;
  const pmx_polar_block bl = blocks[idx[b]];
  const int64_t total = (int64_t)m * n;
  float* out = dst + (int64_t)b * total;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * NT) {
    const int64_t r = e / n, c = e - r * n;
    const int64_t o = r * bl.ldg + c;
    out[e] = bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(bl.g)[o] << 16)
                  : reinterpret_cast<const float*>(bl.g)[o];
  }
}

__global__ __launch_bounds__(NT) void varbatch_scatter_kernel(const pmx_polar_block* blocks,
                                                              const int32_t* idx, int bf16,
                                                              const float* src, int m, int n,
                                                              const pmx_matfn_info* info_src,
                                                              pmx_matfn_info* info_dst) {
  const int b = blockIdx.y;
  const int id = idx[b];
  const pmx_polar_block bl = blocks[id];
  const int64_t total = (int64_t)m * n;
  const float* in = src + (int64_t)b * total;
  for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * NT) {
    const int64_t r = e / n, c = e - r * n;
    const int64_t o = r * bl.ldu + c;
    if (bf16) reinterpret_cast<uint16_t*>(bl.u)[o] = from_f32<bf16_t>(in[e]).bits;
    else reinterpret_cast<float*>(bl.u)[o] = in[e];
  }
  if (info_dst && blockIdx.x == 0) {
    constexpr int W = (int)(sizeof(pmx_matfn_info) / 4);
    const int32_t* a = reinterpret_cast<const int32_t*>(info_src + b);
    int32_t* z = reinterpret_cast<int32_t*>(info_dst + id);
    for (int w = threadIdx.x; w < W; w += NT) z[w] = a[w];
  }
}

static unsigned varbatch_grid(int64_t total) {
  int64_t g = (total + NT - 1) / NT;
  return (unsigned)(g < 1 ? 1 : (g > 256 ? 256 : g));
}

hipError_t launch_varbatch_gather(const pmx_polar_block* blocks, const int32_t* idx, bool bf16,
                                  float* dst, int m, int n, int count, hipStream_t s) {
  hipLaunchKernelGGL(varbatch_gather_kernel, dim3(varbatch_grid((int64_t)m * n), count),
                     dim3(NT), 0, s, blocks, idx, bf16 ? 1 : 0, dst, m, n);
  return hipGetLastError();
}

hipError_t launch_varbatch_scatter(const pmx_polar_block* blocks, const int32_t* idx, bool bf16,
                                   const float* src, int m, int n, int count,
                                   const pmx_matfn_info* info_src, pmx_matfn_info* info_dst,
                                   hipStream_t s) {
  hipLaunchKernelGGL(varbatch_scatter_kernel, dim3(varbatch_grid((int64_t)m * n), count),
                     dim3(NT), 0, s, blocks, idx, bf16 ? 1 : 0, src, m, n, info_src, info_dst);
  return hipGetLastError();
}

// ---------------------------------------------------------------- residual decision
__global__ __launch_bounds__(NT) void resid_decide_kernel(ResidDecide d) {
  const int b = blockIdx.x;
  Ctrl* cb = d.ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const double* part = d.partials + (int64_t)b * d.partial_stride;
  double v = 0.0;
  for (int i = threadIdx.x; i < d.tiles; i += NT) v += part[i];
  __shared__ double red[NT / 64];
  const double tot = block_sum<NT / 64>(v, red);
  if (threadIdx.x == 0) {
    if (d.count_update) cb->iter += 1;
    // products counts the powers of the configured degree
    cb->gemms += d.products + (cb->degree - d.cfg.degree);
    decide(*cb, d.cfg, d.cfg.info ? d.cfg.info + b : nullptr, tot);
  }
}

hipError_t launch_resid_decide(const ResidDecide& d, int batch, hipStream_t s) {
  hipLaunchKernelGGL(resid_decide_kernel, dim3(batch), dim3(NT), 0, s, d);
  return hipGetLastError();
}

// ---------------------------------------------------------------- statistics operands
// The operands of the statistics products in the layout of the scheduled
// GEMM loop (A with k contiguous, B with n contiguous): G^T (cols x rows,
// fp32, row stride rows) and, for bf16 gradients, G widened to fp32 (rows x
// cols, row stride cols).  64 x 64 tiles through LDS; block (0, 0, 0) also
// zeroes the split-k arrival counters of the products that follow.
template <typename T>
__global__ __launch_bounds__(NT) void stats_operands_kernel(const T* __restrict__ g, int64_t ld,
                                                            int64_t sg, int rows, int cols,
                                                            float* __restrict__ gt,
                                                            float* __restrict__ gn,
                                                            uint32_t* zero, int nzero) {
  const int b = blockIdx.z;
  if (zero && blockIdx.x == 0 && blockIdx.y == 0 && b == 0)
    for (int i = threadIdx.x; i < nzero; i += NT) zero[i] = 0u;
  __shared__ float tile[64][65];
  const T* x = g + (int64_t)b * sg;
  const int64_t plane = (int64_t)rows * cols;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int r = ty + 4 * i, gr = r0 + r, gc = c0 + tx;
    float v = 0.f;
    if (gr < rows && gc < cols) {
      v = to_f32(x[(int64_t)gr * ld + gc]);
      if (gn) gn[(int64_t)b * plane + (int64_t)gr * cols + gc] = v;
    }
    tile[r][tx] = v;
  }
  __syncthreads();
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int c = ty + 4 * i, gc = c0 + c, gr = r0 + tx;
    if (gc < cols && gr < rows) gt[(int64_t)b * plane + (int64_t)gc * rows + gr] = tile[tx][c];
  }
}

hipError_t launch_stats_operands(const void* g, bool bf16, int64_t ld, int64_t sg, int rows,
                                 int cols, int batch, float* gt, float* gn, uint32_t* zero,
                                 int nzero, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  if (bf16)
    hipLaunchKernelGGL(stats_operands_kernel<bf16_t>, grid, dim3(NT), 0, s, (const bf16_t*)g, ld,
                       sg, rows, cols, gt, gn, zero, nzero);
  else
    hipLaunchKernelGGL(stats_operands_kernel<float>, grid, dim3(NT), 0, s, (const float*)g, ld,
                       sg, rows, cols, gt, gn, zero, nzero);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tile transpose
__device__ __forceinline__ uint16_t to_bf16_bits(float x) { return from_f32<bf16_t>(x).bits; }
// two values rounded to bf16, the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
}

__global__ __launch_bounds__(NT) void xpose_kernel(XposeParams p) {
  const int b = blockIdx.z;
  float alpha = 0.f, scale = 1.f;
  if (p.ctrl) {
    if (load_status(p.ctrl + b) != PMX_RUNNING) return;
    alpha = (float)p.ctrl[b].alpha;
    if (p.scale_inv_c) scale = (float)(1.0 / p.ctrl[b].c);
    sketch_share(p.sketch, b, blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  }
  __shared__ float tile[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p.vec4 == 2) {
    // the same with 16-byte accesses (rows, cols and leading dimensions
    // multiples of 8): thread t moves the 8 bf16 chunk t % 8 of rows t / 8
    // and t / 8 + 32 in, and of rows t / 8 and t / 8 + 32 of the transpose
    // out; both reads are issued before either is used
    const uint16_t* ab = reinterpret_cast<const uint16_t*>(p.a) + (int64_t)b * p.sa;
    const int q = threadIdx.x & 7, rr = threadIdx.x >> 3;
    const int gc = c0 + 8 * q;
    uint4 w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gr = r0 + rr + 32 * i;
      w[i] = make_uint4(0u, 0u, 0u, 0u);
      if (gr < p.rows && gc < p.cols)
        w[i] = *reinterpret_cast<const uint4*>(ab + (int64_t)gr * p.lda + gc);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = rr + 32 * i, gr = r0 + r;
      const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(u[j] << 16) * scale;
        v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u) * scale;
      }
      if (p.out_n && gr < p.rows && gc < p.cols)
        *reinterpret_cast<uint4*>(p.out_n + (int64_t)b * p.sn + (int64_t)gr * p.ldn + gc) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      if (p.out_t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[r][8 * q + j] = v[j];
      }
    }
    if (!p.out_t) return;  // (uniform over the block)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = rr + 32 * i, gcol = c0 + c, gr = r0 + 8 * q;
      if (gcol < p.cols && gr < p.rows)
        *reinterpret_cast<uint4*>(p.out_t + (int64_t)b * p.st + (int64_t)gcol * p.ldt + gr) =
            make_uint4(pack_bf16x2(tile[8 * q][c], tile[8 * q + 1][c]),
                       pack_bf16x2(tile[8 * q + 2][c], tile[8 * q + 3][c]),
                       pack_bf16x2(tile[8 * q + 4][c], tile[8 * q + 5][c]),
                       pack_bf16x2(tile[8 * q + 6][c], tile[8 * q + 7][c]));
    }
    return;
  }
  if (p.vec4) {
    // bf16 input without a polynomial: each thread moves four consecutive
    // bf16 (8 bytes) per access, both reading rows and writing the
    // transposed rows (rows and cols multiples of 4)
    const uint16_t* ab = reinterpret_cast<const uint16_t*>(p.a) + (int64_t)b * p.sa;
    const int q = threadIdx.x & 15, rr = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rr + 16 * i, gr = r0 + r, gc = c0 + 4 * q;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (gr < p.rows && gc < p.cols) {
        const uint2 w = *reinterpret_cast<const uint2*>(ab + (int64_t)gr * p.lda + gc);
        v[0] = __uint_as_float(w.x << 16) * scale;
        v[1] = __uint_as_float(w.x & 0xFFFF0000u) * scale;
        v[2] = __uint_as_float(w.y << 16) * scale;
        v[3] = __uint_as_float(w.y & 0xFFFF0000u) * scale;
        if (p.out_n)
          *reinterpret_cast<uint2*>(p.out_n + (int64_t)b * p.sn + (int64_t)gr * p.ldn + gc) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) tile[r][4 * q + j] = v[j];
    }
    __syncthreads();
    if (!p.out_t) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = rr + 16 * i, gc = c0 + c, gr = r0 + 4 * q;
      if (gc < p.cols && gr < p.rows)
        *reinterpret_cast<uint2*>(p.out_t + (int64_t)b * p.st + (int64_t)gc * p.ldt + gr) =
            make_uint2(pack_bf16x2(tile[4 * q][c], tile[4 * q + 1][c]),
                       pack_bf16x2(tile[4 * q + 2][c], tile[4 * q + 3][c]));
    }
    return;
  }
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const float* af = reinterpret_cast<const float*>(p.a) + (int64_t)b * p.sa;
  const uint16_t* ab = reinterpret_cast<const uint16_t*>(p.a) + (int64_t)b * p.sa;
  const float* a2 = p.a2 ? p.a2 + (int64_t)b * p.sa : nullptr;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int r = ty + 4 * i, gr = r0 + r, gc = c0 + tx;
    float v = 0.f;
    if (gr < p.rows && gc < p.cols) {
      const int64_t off = (int64_t)gr * p.lda + gc;
      v = p.a_bf16 ? __uint_as_float((uint32_t)ab[off] << 16) : af[off];
      v *= scale;
      if (p.poly) {
        float g = p.degree == 2 ? p.c1 * v + alpha * a2[off] : alpha * v;
        if (gr == gc) g += p.c0;
        v = g;
      }
      if (p.out_n) p.out_n[(int64_t)b * p.sn + (int64_t)gr * p.ldn + gc] = to_bf16_bits(v);
    }
    tile[r][tx] = v;
  }
  __syncthreads();
  if (!p.out_t) return;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int c = ty + 4 * i, gc = c0 + c, gr = r0 + tx;
    if (gc < p.cols && gr < p.rows)
      p.out_t[(int64_t)b * p.st + (int64_t)gc * p.ldt + gr] = to_bf16_bits(tile[tx][c]);
  }
}

// ---------------------------------------------------------------- outputs
// X = sx * Z_cur, X_aux = sa * Y_cur of the last stage.  Z_0 = I is implicit
// when the stage ended before its first update.  NaN when the call failed.
__global__ __launch_bounds__(NT) void root_finish_kernel(RootFinishParams p) {
  const int b = blockIdx.y;
  const Ctrl* cb = p.ctrl + b;
  const int st = *(const volatile int32_t*)&cb->status_all;
  const bool bad = (st == PMX_NONFINITE || st == PMX_DIVERGED);
  const int it = cb->iter;
  const double c = cb->c;
  const float sx = (float)pow(c, p.expo_x), sa = (float)pow(c, p.expo_aux);
  const float* Z = p.zbuf[it & 1] + (int64_t)b * p.buf_stride;
  const float* Y = p.ybuf[it & 1] + (int64_t)b * p.buf_stride;
  float* X = p.x + (int64_t)b * p.x_stride;
  float* XA = p.aux ? p.aux + (int64_t)b * p.aux_stride : nullptr;
  const int n = p.n;
  const bool flat = !bad && it > 0 && p.ldx == n && (!XA || p.ldaux == n) && n % 4 == 0 &&
                    ((uintptr_t)Z & 15) == 0 && ((uintptr_t)Y & 15) == 0 &&
                    ((uintptr_t)X & 15) == 0 && ((uintptr_t)XA & 15) == 0;
  if (flat) {
    // contiguous outputs: one stream of 16-byte accesses, four loads in
    // flight per thread
    const float4* z4 = reinterpret_cast<const float4*>(Z);
    const float4* y4 = reinterpret_cast<const float4*>(Y);
    float4* x4 = reinterpret_cast<float4*>(X);
    float4* a4 = reinterpret_cast<float4*>(XA);
    const int64_t nv = (int64_t)n * n / 4;
    const int64_t step = (int64_t)gridDim.x * NT;
    auto sc = [](float4 v, float f) { return make_float4(v.x * f, v.y * f, v.z * f, v.w * f); };
    int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    for (; i + 3 * step < nv; i += 4 * step) {
      const float4 z0 = z4[i], z1 = z4[i + step], z2 = z4[i + 2 * step], z3 = z4[i + 3 * step];
      x4[i] = sc(z0, sx);
      x4[i + step] = sc(z1, sx);
      x4[i + 2 * step] = sc(z2, sx);
      x4[i + 3 * step] = sc(z3, sx);
    }
    for (; i < nv; i += step) x4[i] = sc(z4[i], sx);
    if (XA) {
      for (i = (int64_t)blockIdx.x * NT + threadIdx.x; i < nv; i += step) a4[i] = sc(y4[i], sa);
    }
    return;
  }
  for (int r = blockIdx.x; r < n; r += gridDim.x)
  for (int col = threadIdx.x; col < n; col += NT) {
    const int64_t e = (int64_t)r * n + col;
    float zx, ya;
    if (bad) {
      zx = NAN;
      ya = NAN;
    } else {
      zx = ((it == 0) ? (r == col ? 1.f : 0.f) : Z[e]) * sx;
      ya = XA ? Y[e] * sa : 0.f;  // Y is read only for the auxiliary output
    }
    X[(int64_t)r * p.ldx + col] = zx;
    if (XA) XA[(int64_t)r * p.ldaux + col] = ya;
  }
}

template <typename T>
__global__ __launch_bounds__(NT) void polar_finish_kernel(PolarFinishParams p) {
  const int b = blockIdx.y;
  const Ctrl* cb = p.ctrl + b;
  const int st = *(const volatile int32_t*)&cb->status_all;
  const bool bad = (st == PMX_NONFINITE || st == PMX_DIVERGED);
  const int it = cb->iter;
  const T* X = reinterpret_cast<const T*>(p.xbuf[it & 1]) + (int64_t)b * p.buf_stride;
  T* U = reinterpret_cast<T*>(p.u) + (int64_t)b * p.u_stride;
  if (p.vec && !p.transpose) {
    // straight copy, 16 bytes per chunk (cols, ldu and the bases aligned):
    // the matrix's rows x cols / V chunks in a grid-stride loop, four chunks
    // a thread with their reads in flight together
    constexpr int V = 16 / sizeof(T);
    const int cv = p.cols / V;
    const int total = p.rows * cv;
    uint4 nanv;
    {
      const uint32_t w = sizeof(T) == 2 ? 0x7FC07FC0u : 0x7FC00000u;
      nanv = make_uint4(w, w, w, w);
    }
    const int step = gridDim.x * NT;
    for (int e0 = blockIdx.x * NT + threadIdx.x; e0 < total; e0 += 4 * step) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * step;
        if (e < total) {
          const int r = e / cv, c = e - r * cv;
          v[u] = bad ? nanv : reinterpret_cast<const uint4*>(X + (int64_t)r * p.cols)[c];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * step;
        if (e < total) {
          const int r = e / cv, c = e - r * cv;
          reinterpret_cast<uint4*>(U + (int64_t)r * p.ldu)[c] = v[u];
        }
      }
    }
    return;
  }
  for (int r = blockIdx.x; r < p.rows; r += gridDim.x)
  for (int c = threadIdx.x; c < p.cols; c += NT) {
    const int64_t e = (int64_t)r * p.cols + c;
    const T v = bad ? from_f32<T>(NAN) : X[e];
    if (p.transpose) U[(int64_t)c * p.ldu + r] = v;
    else U[(int64_t)r * p.ldu + c] = v;
  }
}

// ---------------------------------------------------------------- launchers
// Row-parallel elementwise kernels: one block per row (grid-stride beyond cap).
static int grid_rows(int rows, int cap) {
  int g = rows < cap ? rows : cap;
  return g < 1 ? 1 : g;
}

hipError_t launch_ctrl_reset(Ctrl* ctrl, pmx_matfn_info* info, int batch, int degree,
                             uint32_t* zero, int nzero, hipStream_t s) {
  hipLaunchKernelGGL(ctrl_reset_kernel, dim3(batch), dim3(NT), 0, s, ctrl, info, batch, degree,
                     zero, nzero);
  return hipGetLastError();
}

hipError_t launch_fro_scale(const void* x, bool bf16, int rows, int cols, int64_t ld,
                            int64_t stride, int batch, Ctrl* ctrl, double* partials,
                            int64_t pstride, pmx_matfn_info* info, hipStream_t s) {
  // about one block per CU over the whole batch: every block pays a fenced
  // arrival in the last-block reduction, so 1024 blocks took 154 us for the
  // 32 Muon matrices (268 MB) and 42 us for one fp32 4096^2 matrix, 256
  // blocks 82 and 19 us, 64 blocks 208 and 29 us
  dim3 grid(blocks_per_matrix(rows, batch, 256, kPartialsPerMatrix), batch);
  const int V = bf16 ? 8 : 4;
  const int vec = (cols % V == 0) && (ld % V == 0) && (batch == 1 || stride % V == 0) &&
                  ((uintptr_t)x % 16 == 0);
  if (bf16)
    hipLaunchKernelGGL(fro_scale_kernel<bf16_t>, grid, dim3(NT), 0, s, (const bf16_t*)x, rows,
                       cols, ld, stride, vec, ctrl, partials, pstride, info);
  else
    hipLaunchKernelGGL(fro_scale_kernel<float>, grid, dim3(NT), 0, s, (const float*)x, rows,
                       cols, ld, stride, vec, ctrl, partials, pstride, info);
  return hipGetLastError();
}

hipError_t launch_sqrt_stage_init(const StageInitParams& p, int batch, hipStream_t s) {
  // one block per CU over the batch, as for the Frobenius scale: at n = 4096
  // the set-up took 74 us with 1024 blocks, 53 with 512 and 44 with 256
  dim3 grid(blocks_per_matrix(p.n, batch, 256, kPartialsPerMatrix), batch);
  hipLaunchKernelGGL(sqrt_stage_init_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_polar_init(const PolarInitParams& p, bool bf16, int batch, hipStream_t s) {
  dim3 grid(blocks_per_matrix(p.rows, batch, 4096, 2048), batch);
  if (bf16) hipLaunchKernelGGL(polar_init_kernel<bf16_t>, grid, dim3(NT), 0, s, p);
  else hipLaunchKernelGGL(polar_init_kernel<float>, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

// Blocks per matrix and job at RW = 2 (the most any launch uses).
int skinny_blocks(int n, int q) {
  (void)q;
  return (n + 7) / 8;
}

// Launches one skinny pass; returns its blocks per matrix and job.
template <int Q, int RW, int GJ>
static int skinny_go_j(const SkinnyParams& p, int njobs, int batch, hipStream_t s) {
  if constexpr (Q == 8 || Q == 16) {
    if (p.mfma) {
      // 16 waves a block
      dim3 g((p.n + 15) / 16, njobs, batch);
      hipLaunchKernelGGL((skinny_mfma_kernel<Q, 16, GJ>), g, dim3(1024), 0, s, p);
      return (int)g.x;
    }
  }
  dim3 grid((p.n + 4 * RW - 1) / (4 * RW), njobs, batch);
  if constexpr (GJ == 9) {
    hipLaunchKernelGGL((skinny_kernel<Q, RW, GJ>), grid, dim3(NT), 0, s, p);
    return (int)grid.x;
  }
  if (p.variant == 1) {
    hipLaunchKernelGGL((skinny_stream_kernel<Q, RW, GJ>), grid, dim3(NT), 0, s, p);
  } else if (p.variant == 2) {
    constexpr int CH = (RW <= 2 && Q <= 8) ? 512 : 256;
    hipLaunchKernelGGL((skinny_pipe_kernel<Q, RW, CH, GJ>), grid, dim3(NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((skinny_kernel<Q, RW, GJ>), grid, dim3(NT), 0, s, p);
  }
  return (int)grid.x;
}

// Gram variants: J = 2d + 1 Krylov blocks, at most 5 (d <= 2) or 7 (d = 3),
// or 9 (the inverse Newton objective for p = 4, d = 2).  The Gram pass is a
// single q = p job (p <= PMX_MAX_SKETCH = 16), followed by gram_alpha_kernel.
template <int Q, int RW>
static void skinny_go(const SkinnyParams& p, int njobs, bool gram, int batch, hipStream_t s) {
  if (!gram) {
    skinny_go_j<Q, RW, 0>(p, njobs, batch, s);
  } else if constexpr (Q <= 16) {
    int blocks;
    if (p.gram_j > 7) blocks = skinny_go_j<Q, RW, 9>(p, njobs, batch, s);
    else if (p.cfg.degree_max == 3 || p.gram_j > 5) blocks = skinny_go_j<Q, RW, 7>(p, njobs, batch, s);
    else blocks = skinny_go_j<Q, RW, 5>(p, njobs, batch, s);
    hipLaunchKernelGGL(gram_alpha_kernel, dim3(batch), dim3(NT), 0, s, p, blocks);
  }
}

hipError_t launch_skinny(const SkinnyParams& pin, int njobs, bool gram, int batch,
                         hipStream_t s) {
  SkinnyParams p = pin;
  if (gram && (njobs != 1 || p.q > 16)) return hipErrorInvalidValue;
  // the matrix-core form: any q <= 16 with 16-byte-aligned rows of Mat, for
  // launches of at most 1024 blocks of 16 rows (single or few large
  // matrices); larger batches of small matrices keep the LDS-staged forms,
  // which measured faster there (their Gram shares cost less a row)
  {
    const int64_t blocks = (int64_t)((p.n + 15) / 16) * njobs * batch;
    bool ok = p.variant == 0 && p.q <= 16 && p.n % 4 == 0 && blocks <= 1024;
    for (int j = 0; j < njobs; ++j)
      ok = ok && p.job[j].mat_ld % 4 == 0 && ((uintptr_t)p.job[j].mat & 15) == 0 &&
           p.job[j].mat_stride % 4 == 0;
    p.mfma = ok ? 1 : 0;
  }
  // batches past the matrix-core form's limit: the batched matrix-core form
  // (Gram passes at degree <= 2 only)
  if (!p.mfma && p.variant == 0 && p.q <= 16 && p.n % 4 == 0 && p.n >= 64 &&
      (!gram || (p.gram_j == 0 && p.cfg.degree_max != 3 && p.cfg.degree <= 2))) {
    bool ok = true;
    for (int j = 0; j < njobs; ++j)
      ok = ok && p.job[j].mat_ld % 4 == 0 && ((uintptr_t)p.job[j].mat & 15) == 0 &&
           p.job[j].mat_stride % 4 == 0;
    if (ok) {
      dim3 g((p.n + 16 * SB_W - 1) / (16 * SB_W), njobs, batch);
      if (p.q <= 8) {
        if (gram) hipLaunchKernelGGL((skinny_batch_kernel<8, 5>), g, dim3(SB_W * 64), 0, s, p);
        else hipLaunchKernelGGL((skinny_batch_kernel<8, 0>), g, dim3(SB_W * 64), 0, s, p);
      } else {
        if (gram) hipLaunchKernelGGL((skinny_batch_kernel<16, 5>), g, dim3(SB_W * 64), 0, s, p);
        else hipLaunchKernelGGL((skinny_batch_kernel<16, 0>), g, dim3(SB_W * 64), 0, s, p);
      }
      if (gram) hipLaunchKernelGGL(gram_alpha_kernel, dim3(batch), dim3(NT), 0, s, p, (int)g.x);
      return hipGetLastError();
    }
  }
  // more rows per wave once that still leaves two blocks per compute unit
  const bool wide = (int64_t)((p.n + 31) / 32) * njobs * batch >= 512;
  if (p.q <= 8) {
    if (wide) skinny_go<8, 8>(p, njobs, gram, batch, s);
    else skinny_go<8, 2>(p, njobs, gram, batch, s);
  } else if (p.q <= 16) {
    if (wide && p.variant != 0) skinny_go<16, 4>(p, njobs, gram, batch, s);
    else if (wide) skinny_go<16, 8>(p, njobs, gram, batch, s);
    else skinny_go<16, 2>(p, njobs, gram, batch, s);
  } else if (p.q <= 32) {
    skinny_go<32, 2>(p, njobs, gram, batch, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ------------------------------------------------------------- power scale
__global__ __launch_bounds__(NT) void sketch_kernel(SketchJob sj, const Ctrl* ctrl) {
  const int b = blockIdx.y;
  if (load_status(ctrl + b) != PMX_RUNNING) return;
  sketch_share(sj, b, blockIdx.x, gridDim.x);
}

// One block per matrix: per column j the fp64 norms of K_{t-1}[:, j] and
// K_t[:, j] (fixed-order block sums), mu = the largest ratio, a lower bound
// of the spectral norm of A / c; c shrinks by min(1, factor mu).
__global__ __launch_bounds__(NT) void power_scale_kernel(Ctrl* ctrl, const float* kbuf,
                                                         int64_t kld, int64_t kstride, int n,
                                                         int p, int col_prev, int col_last,
                                                         double factor, int polar,
                                                         pmx_matfn_info* info) {
  const int b = blockIdx.x;
  Ctrl* cb = ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const float* k = kbuf + (int64_t)b * kstride;
  __shared__ double red[NT / 64];
  double mu = 0.0;
  for (int j = 0; j < p; ++j) {
    double s0 = 0.0, s1 = 0.0;
    for (int i = threadIdx.x; i < n; i += NT) {
      const double a = (double)k[(int64_t)i * kld + col_prev + j];
      const double c = (double)k[(int64_t)i * kld + col_last + j];
      s0 += a * a;
      s1 += c * c;
    }
    s0 = block_sum<NT / 64>(s0, red);
    s1 = block_sum<NT / 64>(s1, red);
    if (s0 > 0.0 && isfinite(s0) && isfinite(s1)) mu = fmax(mu, sqrt(s1 / s0));
  }
  if (threadIdx.x == 0 && mu > 0.0 && isfinite(mu)) {
    const double f = fmin(1.0, factor * mu);
    if (polar) {
      const double sc = sqrt(f);
      cb->inv_s = 1.0 / sc;
      cb->c *= sc;
    } else {
      cb->c *= f;
    }
    if (info) info[b].scale = (float)cb->c;
  }
}

__global__ __launch_bounds__(NT) void polar_rescale_kernel(Ctrl* ctrl, float* r, uint16_t* rh,
                                                           int64_t stride, int n,
                                                           double* partials, int64_t pstride,
                                                           IterCfg cfg) {
  const int b = blockIdx.y;
  Ctrl* cb = ctrl + b;
  if (load_status(cb) != PMX_RUNNING) return;
  const double is = cb->inv_s;
  if (!(is > 1.0)) return;  // uniform over the matrix's blocks
  const float f = (float)(is * is);
  float* R = r + (int64_t)b * stride;
  uint16_t* H = rh ? rh + (int64_t)b * stride : nullptr;
  double acc = 0.0;
  for (int i = blockIdx.x; i < n; i += gridDim.x)
    for (int j = threadIdx.x; j < n; j += NT) {
      const int64_t e = (int64_t)i * n + j;
      const float id = i == j ? 1.f : 0.f;
      const float v = id - (id - R[e]) * f;
      R[e] = v;
      if (H) H[e] = from_f32<bf16_t>(v).bits;
      acc += (double)v * (double)v;
    }
  __shared__ double red[NT / 64];
  const double bs = block_sum<NT / 64>(acc, red);
  double tot;
  if (last_block_sum<NT / 64>(bs, partials + (int64_t)b * pstride, &cb->counter, gridDim.x,
                              blockIdx.x, red, &tot)) {
    if (threadIdx.x == 0) decide(*cb, cfg, cfg.info ? cfg.info + b : nullptr, tot);
  }
}

// The sketch of one (matrix, stage, iteration) as the iterations draw it,
// written to a caller's n x p matrix (row stride lds) and, when `words` is
// set, the Philox output word behind every element (n x p, row stride p).
__global__ __launch_bounds__(NT) void sketch_export_kernel(uint32_t seed_lo, uint32_t seed_hi,
                                                           int b, int stage, int k, int n, int p,
                                                           float* S, int64_t lds,
                                                           uint32_t* words) {
  const int64_t total = (int64_t)n * p, calls = (total + 3) / 4;
  for (int64_t q = (int64_t)blockIdx.x * NT + threadIdx.x; q < calls;
       q += (int64_t)gridDim.x * NT) {
    uint32_t c[4] = {(uint32_t)q, (uint32_t)k, (uint32_t)stage, (uint32_t)b};
    philox4x32_10(c, seed_lo, seed_hi);
    double z[4];
    philox_normals(c, z);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t e = q * 4 + w;
      if (e < total) {
        const int64_t i = e / p, j = e - i * p;
        S[i * lds + j] = (float)z[w];
        if (words) words[e] = c[w];
      }
    }
  }
}

hipError_t launch_sketch_export(uint64_t seed, int b, int stage, int k, int n, int p, float* S,
                                int64_t lds, uint32_t* words, hipStream_t s) {
  const int64_t calls = ((int64_t)n * p + 3) / 4;
  int64_t blocks = (calls + NT - 1) / NT;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
  hipLaunchKernelGGL(sketch_export_kernel, dim3((unsigned)blocks), dim3(NT), 0, s,
                     (uint32_t)(seed & 0xFFFFFFFFull), (uint32_t)(seed >> 32), b, stage, k, n, p,
                     S, lds, words);
  return hipGetLastError();
}

hipError_t launch_sketch(const SketchJob& sj, const Ctrl* ctrl, int batch, hipStream_t s) {
  const int64_t calls = ((int64_t)sj.n * sj.p + 3) / 4;
  int blocks = (int)((calls + NT - 1) / NT);
  blocks = blocks < 1 ? 1 : (blocks > 64 ? 64 : blocks);
  hipLaunchKernelGGL(sketch_kernel, dim3(blocks, batch), dim3(NT), 0, s, sj, ctrl);
  return hipGetLastError();
}

hipError_t launch_power_scale(Ctrl* ctrl, const float* kbuf, int64_t kld, int64_t kstride,
                              int n, int p, int col_prev, int col_last, double factor,
                              int polar, pmx_matfn_info* info, int batch, hipStream_t s) {
  hipLaunchKernelGGL(power_scale_kernel, dim3(batch), dim3(NT), 0, s, ctrl, kbuf, kld, kstride,
                     n, p, col_prev, col_last, factor, polar, info);
  return hipGetLastError();
}

hipError_t launch_polar_rescale(Ctrl* ctrl, float* r, uint16_t* rh, int64_t stride, int n,
                                double* partials, int64_t pstride, IterCfg cfg, int batch,
                                hipStream_t s) {
  dim3 grid(blocks_per_matrix(n, batch, 1024, kPartialsPerMatrix), batch);
  hipLaunchKernelGGL(polar_rescale_kernel, grid, dim3(NT), 0, s, ctrl, r, rh, stride, n,
                     partials, pstride, cfg);
  return hipGetLastError();
}

// One flag for the host: is any matrix of the batch still iterating?
__global__ __launch_bounds__(NT) void publish_running_kernel(const Ctrl* ctrl, int batch,
                                                             int32_t* dst) {
  __shared__ int32_t any;
  if (threadIdx.x == 0) any = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < batch; b += NT)
    if (load_status(ctrl + b) == PMX_RUNNING) any = 1;
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(dst, any, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

hipError_t launch_publish_running(const Ctrl* ctrl, int batch, int32_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(publish_running_kernel, dim3(1), dim3(NT), 0, s, ctrl, batch, dst);
  return hipGetLastError();
}

hipError_t launch_form_g(const FormGParams& pin, int batch, hipStream_t s) {
  FormGParams p = pin;
  if ((p.degree == 3 || p.adaptive) && (!p.r2 || !p.r3)) return hipErrorInvalidValue;
  p.vec = (p.n % 4 == 0) && (p.stride % 4 == 0) && ((uintptr_t)p.r % 16 == 0) &&
          (!p.r2 || (uintptr_t)p.r2 % 16 == 0) && (!p.r3 || (uintptr_t)p.r3 % 16 == 0) &&
          ((uintptr_t)p.dst % 16 == 0) && ((uintptr_t)p.dst2 % 16 == 0);
  const int per = (4096 + batch - 1) / batch;
  dim3 grid(grid_rows(p.n, per < 2048 ? per : 2048), batch);
  hipLaunchKernelGGL(form_g_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_convert(const void* src, bool src_bf16, int64_t lds, int64_t ss, void* dst,
                          bool dst_bf16, int64_t ldd, int64_t sd, int rows, int cols, int batch,
                          hipStream_t s) {
  dim3 grid(grid_rows(rows, 4096), batch);
  if (src_bf16 && !dst_bf16)
    hipLaunchKernelGGL((convert_kernel<bf16_t, float>), grid, dim3(NT), 0, s,
                       (const bf16_t*)src, lds, ss, (float*)dst, ldd, sd, rows, cols);
  else if (!src_bf16 && dst_bf16)
    hipLaunchKernelGGL((convert_kernel<float, bf16_t>), grid, dim3(NT), 0, s,
                       (const float*)src, lds, ss, (bf16_t*)dst, ldd, sd, rows, cols);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_xpose(const XposeParams& pin, int batch, hipStream_t s) {
  XposeParams p = pin;
  auto al8 = [](const void* q) { return ((uintptr_t)q & 7u) == 0; };
  p.vec4 = p.a_bf16 && !p.poly && p.rows % 4 == 0 && p.cols % 4 == 0 && p.lda % 4 == 0 &&
           (batch == 1 || p.sa % 4 == 0) && al8(p.a) &&
           (!p.out_n || (p.ldn % 4 == 0 && (batch == 1 || p.sn % 4 == 0) && al8(p.out_n))) &&
           (!p.out_t || (p.ldt % 4 == 0 && (batch == 1 || p.st % 4 == 0) && al8(p.out_t)));
  auto al16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
  if (p.vec4 && p.rows % 8 == 0 && p.cols % 8 == 0 && p.lda % 8 == 0 &&
      (batch == 1 || p.sa % 8 == 0) && al16(p.a) &&
      (!p.out_n || (p.ldn % 8 == 0 && (batch == 1 || p.sn % 8 == 0) && al16(p.out_n))) &&
      (!p.out_t || (p.ldt % 8 == 0 && (batch == 1 || p.st % 8 == 0) && al16(p.out_t))))
    p.vec4 = 2;
  dim3 grid((p.cols + 63) / 64, (p.rows + 63) / 64, batch);
  hipLaunchKernelGGL(xpose_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_root_finish(const RootFinishParams& p, int batch, hipStream_t s) {
  dim3 grid(blocks_per_matrix(p.n, batch, 4096, 2048), batch);
  hipLaunchKernelGGL(root_finish_kernel, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_polar_finish(const PolarFinishParams& pin, bool bf16, int batch, hipStream_t s) {
  PolarFinishParams p = pin;
  const int V = bf16 ? 8 : 4;
  p.vec = (p.cols % V == 0) && (p.ldu % V == 0) && (p.buf_stride % V == 0) &&
          (batch == 1 || p.u_stride % V == 0) && ((uintptr_t)p.u % 16 == 0) &&
          ((uintptr_t)p.xbuf[0] % 16 == 0) && ((uintptr_t)p.xbuf[1] % 16 == 0) &&
          (int64_t)p.rows * (p.cols / V) < ((int64_t)1 << 31);  // chunk index in int
  const int per = (4096 + batch - 1) / batch;
  dim3 grid(grid_rows(p.rows, per < 2048 ? per : 2048), batch);
  if (p.vec && !p.transpose) {
    // the copy form: enough blocks for four chunks a thread (about 16384
    // blocks over the batch at most)
    const int64_t chunks = (int64_t)p.rows * (p.cols / V);
    const int64_t want = (chunks + 4 * NT - 1) / (4 * NT);
    const int64_t cap = std::max<int64_t>(1, 16384 / batch);
    grid.x = (unsigned)std::max<int64_t>(1, std::min(want, cap));
  }
  if (bf16) hipLaunchKernelGGL(polar_finish_kernel<bf16_t>, grid, dim3(NT), 0, s, p);
  else hipLaunchKernelGGL(polar_finish_kernel<float>, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace pmx
