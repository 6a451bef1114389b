// Host runtime and C ABI of libpmx: argument validation, workspace layout and
// the launch sequences of the four operations.  Every sequence is enqueued
// in full on the caller's stream; iteration kernels skip themselves on the
// device once their matrix has finished, so no call waits for the GPU.
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "pmx_kernels.h"

struct pmx_context {
  int device;
  int num_cu;
  int gemm_blocks_per_cu;  // persistent GEMM grid: blocks per CU (0: one block per tile)
  int gemm_cfg;            // forced tile configuration (-1: by shape)
  int gemm_map;            // tile order mode
  int bf16_cfg;            // bf16 GEMM tile (-1: by shape, 0 128^2, 1 256^2 x 8 waves, 2 x 4)
  int bf16_map;            // bf16 GEMM: 1 deals whole matrices to XCDs, 0 plain order
  int skinny_variant;      // skinny products: 0 In through LDS, 1 In read directly
  int bf16_dma;            // bf16 GEMM: 1 uses direct global-to-LDS loads for whole tiles (measured slower; off)
  int bf16_mn;             // bf16 polar: 1 reads X for I - X^T X via LDS transpose reads (no X^T copy)
  int bf16_persist;        // bf16 GEMM: 1 runs whole-tile launches on persistent blocks, each
                           // loading its next tile's first k tile ahead of the epilogue
  int bf16_early;          // bf16 persistent GEMM: 1 issues each k tile's loads before the previous tile's barrier
  int small_fused;         // 1: one fused launch for orders <= kSmallMaxN
  int split_k;             // 1: split-k tail for the fp32 products of the iterations
  int bf16_sym;            // 1: bf16 X^T X and R^2 run upper-triangle tiles, mirrored
  int bf16_sym_small;      // 1: ... with 128 x 128 tiles
  int f64_tile;            // fp64 GEMM block tile (0: by the launch's size, else 64 or 128)
  // host-polled convergence (pmx_set_host_poll): updates per published point,
  // two pinned host flags (device-mapped) and the events behind them
  int poll_chunk = 0;
  int32_t* poll_host = nullptr;
  int32_t* poll_dev = nullptr;
  hipEvent_t poll_ev[2] = {nullptr, nullptr};
  // launch trace (benchmarking): event pairs recorded around every launch
  bool trace = false;
  struct Rec {
    int cls;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t next_event() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

namespace pmx {
namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxN = 32768;
constexpr int kMaxIter = 1000;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Library-owned scratch of pmx_precond_apply_noalloc: one copy per device,
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (in host code the name is a host-side stand-in): pmx_create resolves
// the device address once per device with hipGetSymbolAddress, and the entry
// point passes that address.
constexpr size_t kScratchBytes = (size_t)PMX_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (the caller made `device` current).
hipError_t resolve_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr || ((uintptr_t)ptr % kAlign) != 0) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void* scratch_of(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch_ptr[device];
}

// Current-device guard: make the handle's device current for the call and
// restore the caller's device afterwards.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      ok = false;
      return;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Byte extent of a (strided batch of) row-major matrices.
struct Extent {
  uintptr_t lo = 0, hi = 0;
  bool valid = false;
};

Extent extent_of(const void* p, int rows, int cols, int64_t ld, int64_t stride, int batch,
                 size_t elem) {
  Extent e;
  if (!p || rows <= 0 || cols <= 0) return e;
  const int64_t last = (int64_t)(batch - 1) * stride + (int64_t)(rows - 1) * ld + cols;
  e.lo = (uintptr_t)p;
  e.hi = e.lo + (uintptr_t)last * elem;
  e.valid = true;
  return e;
}

bool overlap(const Extent& a, const Extent& b) {
  return a.valid && b.valid && a.lo < b.hi && b.lo < a.hi;
}

// Distinct matrices of one batch must not overlap when written.
bool batch_layout_ok(int rows, int cols, int64_t ld, int64_t stride, int batch) {
  if (ld < cols) return false;
  if (batch > 1 && stride < (int64_t)(rows - 1) * ld + cols) return false;
  return stride >= 0;
}

pmx_status from_hip(hipError_t e) { return e == hipSuccess ? PMX_OK : PMX_ERR_HIP; }

// Enqueue helper: runs a launcher on the call's stream, bracketed by trace
// events when the handle's trace is enabled.
struct Enq {
  pmx_context* h;
  hipStream_t s;
  template <typename F>
  hipError_t run(int cls, F&& f) {
    hipEvent_t a = nullptr, b = nullptr;
    if (h && h->trace) {
      a = h->next_event();
      b = h->next_event();
      if (a && b) (void)hipEventRecord(a, s);
    }
    const hipError_t e = f();
    if (a && b) {
      (void)hipEventRecord(b, s);
      h->recs.push_back({cls, a, b});
    }
    return e;
  }
};

// Host-polled convergence of one update loop (pmx_set_host_poll).  At the
// top of update i (i > 0, i a multiple of the chunk) a one-block kernel
// publishes whether any matrix is still iterating, followed by an event; the
// value published one point earlier is then read after its event, so one
// chunk stays queued while the host waits.  When that value is 0 every later
// update of the loop would exit on the device at once, so the loop stops.
struct Poller {
  Enq& q;
  const Ctrl* ctrl;
  int batch;
  int chunk = 0;
  int points = 0;
  Poller(Enq& q_, const Ctrl* c, int b) : q(q_), ctrl(c), batch(b) {
    chunk = q.h ? q.h->poll_chunk : 0;
    if (chunk > 0) {
      hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(q.s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        chunk = 0;
    }
    // a previous loop may have stopped with its newest publish kernel still
    // queued (possibly on another stream): let it land before the flags are
    // reused, so no stale value is read for this loop's points
    if (chunk > 0)
      for (hipEvent_t e : q.h->poll_ev)
        if (hipEventSynchronize(e) != hipSuccess) chunk = 0;
  }
  hipError_t step(int i, bool* stop) {
    *stop = false;
    if (chunk <= 0 || i == 0 || i % chunk != 0) return hipSuccess;
    pmx_context* h = q.h;
    volatile int32_t* flag = h->poll_host;
    const int slot = points & 1;
    flag[slot] = -1;
    hipError_t e = q.run(PMX_KC_OTHER, [&] {
      return launch_publish_running(ctrl, batch, h->poll_dev + slot, q.s);
    });
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(h->poll_ev[slot], q.s)) != hipSuccess) return e;
    if (++points < 2) return hipSuccess;
    if ((e = hipEventSynchronize(h->poll_ev[slot ^ 1])) != hipSuccess) return e;
    *stop = flag[slot ^ 1] == 0;
    return hipSuccess;
  }
};

#define PMX_TRY(expr)                          \
  do {                                         \
    hipError_t _e = (expr);                    \
    if (_e != hipSuccess) return PMX_ERR_HIP;  \
  } while (0)

// Taylor coefficient c_j of (1 - xi)^{-1/2}: c_0 = 1, c_j = c_{j-1} (2j - 1) / (2j).
double taylor(int j) {
  double c = 1.0;
  for (int i = 1; i <= j; ++i) c *= (2.0 * i - 1.0) / (2.0 * i);
  return c;
}

// Polynomials as coefficient arrays (increasing powers), small fixed size.
struct Poly {
  double c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
};
Poly pmul(const Poly& a, const Poly& b) {
  Poly r;
  for (int i = 0; i < 8; ++i)
    for (int j = 0; i + j < 8; ++j) r.c[i + j] += a.c[i] * b.c[j];
  return r;
}

// r(xi; alpha) = 1 - (1 - xi) (f + alpha xi^d)^2 with f = sum_{j<d} c_j xi^j,
// split as A0 + alpha A1 + alpha^2 A2:
//   A0 = 1 - (1 - xi) f^2,  A1 = -2 (1 - xi) f xi^d,  A2 = -(1 - xi) xi^{2d}.
AlphaCoef make_coef(int d) {
  Poly f, om, xd, x2d;
  for (int j = 0; j < d; ++j) f.c[j] = taylor(j);
  om.c[0] = 1.0;
  om.c[1] = -1.0;
  xd.c[d] = 1.0;
  x2d.c[2 * d] = 1.0;
  Poly ff = pmul(f, f);
  Poly A0 = pmul(om, ff);
  for (int i = 0; i < 8; ++i) A0.c[i] = -A0.c[i];
  A0.c[0] += 1.0;
  Poly A1 = pmul(pmul(om, f), xd);
  for (int i = 0; i < 8; ++i) A1.c[i] *= -2.0;
  Poly A2 = pmul(om, x2d);
  for (int i = 0; i < 8; ++i) A2.c[i] = -A2.c[i];
  AlphaCoef co;
  for (int j = 0; j < 8; ++j) {
    co.a[0][j] = A0.c[j];
    co.a[1][j] = A1.c[j];
    co.a[2][j] = A2.c[j];
  }
  co.taylor_d = taylor(d);
  return co;
}

// Effective options after defaults; returns false if invalid.  root_p: the
// root order of an inverse-root call (selects the inverse Newton iteration's
// default interval for p = 4), 0 otherwise.
bool resolve_opts(const pmx_matfn_opts* in, pmx_matfn_opts* out, int root_p = 0) {
  pmx_matfn_opts o;
  pmx_matfn_opts_default(&o);
  if (in) {
    if (in->struct_version == 1) {
      // the 40-byte layout, ending at seed
      memcpy(&o, in, offsetof(pmx_matfn_opts, fp64_iters));
    } else if (in->struct_version == 2) {
      // the 48-byte layout, ending at degree_max (version 2's zero `reserved`)
      memcpy(&o, in, offsetof(pmx_matfn_opts, adapt_ratio));
    } else if (in->struct_version == 3) {
      // the 56-byte layout, ending at method
      memcpy(&o, in, offsetof(pmx_matfn_opts, scale_mode));
    } else if (in->struct_version == PMX_OPTS_VERSION) {
      o = *in;
    } else {
      return false;
    }
    o.struct_version = PMX_OPTS_VERSION;
  }
  if (o.fp64_iters < 0 || o.fp64_iters > o.max_iter) return false;
  if (o.method != PMX_METHOD_NEWTON_SCHULZ && o.method != PMX_METHOD_INVERSE_NEWTON) return false;
  // the inverse Newton iteration: d <= 2, fixed degree, fp32 updates
  if (o.method == PMX_METHOD_INVERSE_NEWTON &&
      (o.degree > 2 || (o.degree_max != 0 && o.degree_max != o.degree) || o.fp64_iters != 0))
    return false;
  if (o.degree < 1 || o.degree > 3) return false;
  // adaptive degree: 2 -> 3 only, with the fitted alpha and fp32 updates
  if (o.degree_max != 0 && o.degree_max != o.degree &&
      !(o.degree == 2 && o.degree_max == 3 && o.accelerate == 1 && o.fp64_iters == 0))
    return false;
  if (!isfinite(o.adapt_ratio)) return false;
  if (o.sketch_p < 1 || o.sketch_p > PMX_MAX_SKETCH) return false;
  if (o.max_iter < 1 || o.max_iter > kMaxIter) return false;
  if (o.accelerate != 0 && o.accelerate != 1) return false;
  if (isnan(o.alpha_lo) != isnan(o.alpha_hi)) return false;
  if (isnan(o.alpha_lo)) {
    // lo = c_d; hi = the interval rule's bound rounded down (1, 1.4722, 2.4686)
    static const float lo_d[4] = {0.f, 0.5f, 0.375f, 0.3125f};
    static const float hi_d[4] = {0.f, 1.0f, 1.47f, 2.46f};
    o.alpha_lo = lo_d[o.degree];
    o.alpha_hi = hi_d[o.degree];
    if (o.method == PMX_METHOD_INVERSE_NEWTON && root_p == 4) {
      // the fourth-root map's rule: lo = b_d (1/4, 5/32), hi 1/2 and 0.6039 -> 0.60
      o.alpha_lo = o.degree == 1 ? 0.25f : 0.15625f;
      o.alpha_hi = o.degree == 1 ? 0.5f : 0.60f;
    }
  }
  if (!isfinite(o.alpha_lo) || !isfinite(o.alpha_hi) || o.alpha_lo > o.alpha_hi) return false;
  if (!isfinite(o.tol) || o.tol < 0.f) return false;
  if (o.scale_mode != PMX_SCALE_FROBENIUS && o.scale_mode != PMX_SCALE_POWER) return false;
  if (o.reserved != 0) return false;
  *out = o;
  return true;
}

IterCfg make_cfg(const pmx_matfn_opts& o, int n, pmx_matfn_info* info) {
  IterCfg c;
  c.n = n;
  c.degree = o.degree;
  c.p = o.sketch_p;
  c.max_iter = o.max_iter;
  c.accelerate = o.accelerate;
  c.lo = o.alpha_lo;
  c.hi = o.alpha_hi;
  c.tol = o.tol;
  c.taylor_d = (float)taylor(o.degree);
  c.degree_max = std::max(o.degree, o.degree_max);
  c.adapt_ratio = o.adapt_ratio;
  c.seed_lo = (uint32_t)(o.seed & 0xFFFFFFFFull);
  c.seed_hi = (uint32_t)(o.seed >> 32);
  c.info = info;
  return c;
}

// ------------------------------------------------------------------ workspace
struct IterLayout {
  size_t ctrl, partials, gram, bufs[10], b64[6], kbuf, skc, skp, total;
  int64_t buf_stride, kstride, kld, pstride, gstride, skcap;
};

// Work buffers of the iterative functions: `nbig` matrices of rows x cols
// (the iterates) and `nsmall` of cols x cols (R, R^2/g), per batch matrix.
IterLayout iter_layout(int rows, int cols, int batch, const pmx_matfn_opts& o, int nbig,
                       int nsmall, size_t big_elem, int nf64 = 0) {
  IterLayout L;
  size_t off = 0;
  L.ctrl = off;
  off = align_up(off + sizeof(Ctrl) * (size_t)batch);
  L.pstride = std::max<int64_t>(kPartialsPerMatrix, gemm_f32_tiles(cols, cols));
  L.partials = off;
  off = align_up(off + sizeof(double) * (size_t)L.pstride * batch);
  L.gstride = (int64_t)kGramShare * (skinny_blocks(cols, 1) + 1);
  L.gram = off;
  off = align_up(off + sizeof(double) * (size_t)L.gstride * batch);
  const int64_t big = (int64_t)rows * cols, small = (int64_t)cols * cols;
  (void)big_elem;
  L.buf_stride = ((std::max(big, small) + 63) / 64) * 64;  // elements (fp32 slots)
  for (int i = 0; i < 10; ++i) {
    L.bufs[i] = 0;
    if (i < nbig + nsmall) {
      L.bufs[i] = off;
      off = align_up(off + sizeof(float) * (size_t)L.buf_stride * batch);
    }
  }
  for (int i = 0; i < 6; ++i) {
    L.b64[i] = 0;
    if (i < nf64) {
      L.b64[i] = off;
      off = align_up(off + sizeof(double) * (size_t)L.buf_stride * batch);
    }
  }
  // Krylov blocks K_0..K_J: J = 2d + 1, or 4d + 1 for the inverse Newton
  // iteration (sized for p = 4)
  const int J = o.method == PMX_METHOD_INVERSE_NEWTON ? 4 * o.degree + 1
                                                      : 2 * std::max(o.degree, o.degree_max) + 1;
  L.kld = (int64_t)(J + 1) * o.sketch_p;
  L.kstride = (((int64_t)cols * L.kld + 63) / 64) * 64;
  L.kbuf = off;
  off = align_up(off + sizeof(float) * (size_t)L.kstride * batch);
  // split-k tail of the fp32 products: counters and two partial-tile slots
  // per worker (128 x 128 tiles from order 512 on, else 64 x 64)
  L.skc = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)kSplitMaxWorkers);
  L.skcap = (int64_t)2 * kSplitMaxWorkers * (cols >= 512 ? 128 * 128 : 64 * 64);
  L.skp = off;
  off = align_up(off + sizeof(float) * (size_t)L.skcap);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(ws) + off);
}

bool ptr_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

GemmParams gemm_base(const pmx_context* h, int M, int N, int K, int batch) {
  GemmParams g;
  memset(&g, 0, sizeof(g));
  g.max_blocks = h->gemm_blocks_per_cu > 0 ? h->num_cu * h->gemm_blocks_per_cu : 0;
  g.cfg_id = h->gemm_cfg;
  g.map_mode = h->gemm_map;
  g.num_cu = h->num_cu;
  g.nprob = 1;
  g.batch = batch;
  g.M = M;
  g.N = N;
  g.K = K;
  return g;
}

GemmParams bf16_base(const pmx_context* h, int M, int N, int K, int batch) {
  GemmParams g = gemm_base(h, M, N, K, batch);
  g.cfg_id = h->bf16_cfg;
  g.map_mode = h->bf16_map;
  g.dma = h->bf16_dma;
  g.persist = h->bf16_persist;
  g.early = h->bf16_early;
  return g;
}

// The split-k tail buffers of an iterative call's workspace.
void use_split(GemmParams& g, void* ws, const IterLayout& L) {
  if (!g.sk_part && g.cfg_id < 0) {
    g.sk_part = at<float>(ws, L.skp);
    g.sk_cnt = at<uint32_t>(ws, L.skc);
    g.sk_cap = L.skcap;
  }
}

void set_vec(GemmParams& g) {
  bool v = true;
  for (int i = 0; i < g.nprob; ++i) {
    const GemmProblem& p = g.prob[i];
    v = v && ptr_aligned16(p.a.ptr) && ptr_aligned16(p.b.ptr) && (p.a.ld % 4 == 0) &&
        (p.b.ld % 4 == 0) && (p.a.stride % 4 == 0) && (p.b.stride % 4 == 0);
    // a symmetric output's mirrored stores are 16-byte stores into C
    if (g.sym)
      v = v && ptr_aligned16(p.c) && (p.ldc % 4 == 0) && (p.stride_c % 4 == 0);
  }
  g.vec = v ? 1 : 0;
}

SketchJob make_sketch(const IterLayout& L, void* ws, const IterCfg& cfg, int n, int k,
                      int stage, bool on) {
  SketchJob sj;
  memset(&sj, 0, sizeof(sj));
  if (!on) return sj;
  sj.kbuf = at<float>(ws, L.kbuf);
  sj.kld = L.kld;
  sj.kstride = L.kstride;
  sj.n = n;
  sj.p = cfg.p;
  sj.k = k;
  sj.stage = stage;
  sj.seed_lo = cfg.seed_lo;
  sj.seed_hi = cfg.seed_hi;
  return sj;
}

// The power estimate of the input scale (scale_mode 1): V_0 = the sketch of
// stage kPowerStage, kPowerPasses skinny passes K_t = (A / c) K_{t-1} that
// alternate between the column blocks [0, p) and [p, 2p) of the Krylov
// buffer, and the update of c from the last two blocks.  The stage set-up
// that follows takes Y_0 = A / c with the new c, and the outputs use it.
hipError_t enqueue_power_scale(Enq& q, void* ws, const IterLayout& L, const IterCfg& cfg,
                               const float* A, int lda, int64_t sa, int n, int batch) {
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  float* kbuf = at<float>(ws, L.kbuf);
  const int pp = cfg.p;
  const SketchJob sj = make_sketch(L, ws, cfg, n, 0, kPowerStage, true);
  hipError_t e = q.run(PMX_KC_OTHER, [&] { return launch_sketch(sj, ctrl, batch, q.s); });
  if (e != hipSuccess) return e;
  SkinnyParams kp;
  memset(&kp, 0, sizeof(kp));
  kp.kbuf = kbuf;
  kp.variant = q.h->skinny_variant;
  kp.kld = L.kld;
  kp.kstride = L.kstride;
  kp.n = n;
  kp.q = pp;
  kp.ctrl = ctrl;
  kp.gram_partials = at<double>(ws, L.gram);
  kp.gram_stride = L.gstride;
  kp.cfg = cfg;
  for (int t = 0; t < kPowerPasses; ++t) {
    SkinnyJob& j = kp.job[0];
    j.mat = A;
    j.mat_ld = lda;
    j.mat_stride = sa;
    j.in_col = (t & 1) ? pp : 0;
    j.out_col = (t & 1) ? 0 : pp;
    j.pow = 1;
    e = q.run(PMX_KC_SKINNY, [&] { return launch_skinny(kp, 1, false, batch, q.s); });
    if (e != hipSuccess) return e;
  }
  const int last = (kPowerPasses & 1) ? pp : 0;
  return q.run(PMX_KC_OTHER, [&] {
    return launch_power_scale(ctrl, kbuf, L.kld, L.kstride, n, pp, pp - last, last,
                              kPowerFactor, 0, cfg.info, batch, q.s);
  });
}

// The estimated scale of the polar factor (scale_mode 1), after the first
// residual R_0 = I - X_0^T X_0: V_0 (the sketch of stage kPowerStage) in the
// Krylov columns [2p, 3p) -- [0, p) holds S_0 --, kPowerPasses complement
// passes K_t = K_{t-1} - R_0 K_{t-1} = X_0^T X_0 K_{t-1} between [2p, 3p) and
// [3p, 4p), s^2 = min(1, 2 mu), then R_0 <- I - (I - R_0) / s^2 in place
// (and its bf16 copy rh) with the decision on r_0 again.  X_0 itself is not
// touched: the first update multiplies by g / s (form_g's first_scale).
hipError_t enqueue_polar_scale(Enq& q, void* ws, const IterLayout& L, const IterCfg& cfg,
                               float* R, uint16_t* rh, int n, int batch) {
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  float* kbuf = at<float>(ws, L.kbuf);
  const int pp = cfg.p;
  const int c0 = 2 * pp, c1 = 3 * pp;
  if ((int64_t)4 * pp > L.kld) return hipErrorInvalidValue;
  SketchJob sj = make_sketch(L, ws, cfg, n, 0, kPowerStage, true);
  sj.col = c0;
  hipError_t e = q.run(PMX_KC_OTHER, [&] { return launch_sketch(sj, ctrl, batch, q.s); });
  if (e != hipSuccess) return e;
  SkinnyParams kp;
  memset(&kp, 0, sizeof(kp));
  kp.kbuf = kbuf;
  kp.variant = q.h->skinny_variant;
  kp.kld = L.kld;
  kp.kstride = L.kstride;
  kp.n = n;
  kp.q = pp;
  kp.ctrl = ctrl;
  kp.gram_partials = at<double>(ws, L.gram);
  kp.gram_stride = L.gstride;
  kp.cfg = cfg;
  for (int t = 0; t < kPowerPasses; ++t) {
    SkinnyJob& j = kp.job[0];
    j.mat = R;
    j.mat_ld = n;
    j.mat_stride = L.buf_stride;
    j.in_col = (t & 1) ? c1 : c0;
    j.out_col = (t & 1) ? c0 : c1;
    j.pow = 0;
    e = q.run(PMX_KC_SKINNY, [&] { return launch_skinny(kp, 1, false, batch, q.s); });
    if (e != hipSuccess) return e;
  }
  const int last = (kPowerPasses & 1) ? c1 : c0;
  const int prev = (kPowerPasses & 1) ? c0 : c1;
  e = q.run(PMX_KC_OTHER, [&] {
    return launch_power_scale(ctrl, kbuf, L.kld, L.kstride, n, pp, prev, last, kPowerFactor, 1,
                              cfg.info, batch, q.s);
  });
  if (e != hipSuccess) return e;
  return q.run(PMX_KC_OTHER, [&] {
    return launch_polar_rescale(ctrl, R, rh, L.buf_stride, n, at<double>(ws, L.partials),
                                L.pstride, cfg, batch, q.s);
  });
}

// The power R^2 (d = 2) and the alpha fit of one PRISM update, shared by the
// square-root and polar sequences (R, R2 are n x n).  The sketch S_k is
// already in the Krylov buffer (generated by the kernel that produced R_k).
//   d = 2: K1 = R S / s, K2 = R^2 S / s^2; [K3 | K4] = R^2 [K1 | K2] / s^2;
//          K5 = R^2 K3 / s^2 (+ Gram, alpha)
//   d = 3: as d = 2, then [K5 | K6] = R^2 [K3 | K4] / s^2 and
//          K7 = R^2 K5 / s^2 (+ Gram, alpha); R^3 = R^2 R is formed for g
//   adaptive degree (2, raised to 3): the d = 3 sequence for every matrix,
//          R^3 only for the matrices at d = 3, and the Gram pass uses
//          K_1..K_5 or K_1..K_7 by each matrix's current degree
//   d = 1: K_j = R K_{j-1} / s, j = 1..3 (+ Gram, alpha on the last pass)
hipError_t enqueue_power_and_alpha(Enq& q, void* ws, const IterLayout& L,
                                   const pmx_matfn_opts& o, const IterCfg& cfg,
                                   const AlphaCoef& coef, int n, int batch, float* R,
                                   float* R2, float* R3, bool power = true) {
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  float* kbuf = at<float>(ws, L.kbuf);
  const int d = o.degree, pp = o.sketch_p;
  const int dmax = cfg.degree_max;  // d = 3, or the adaptive degree's ceiling
  hipError_t e;
  if (d >= 2 && power) {
    GemmParams g = gemm_base(q.h, n, n, n, batch);
    g.prob[0].a = {R, n, L.buf_stride, nullptr, 0};
    g.prob[0].b = {R, n, L.buf_stride, nullptr, 0};
    g.prob[0].c = R2;
    g.prob[0].ldc = n;
    g.prob[0].stride_c = L.buf_stride;
    g.ctrl = ctrl;
    g.sym = 1;  // R symmetric, so R^2 is: upper-triangle tiles, mirrored
    if (q.h->split_k) use_split(g, ws, L);
    set_vec(g);
    e = q.run(PMX_KC_GEMM_POWER, [&] { return launch_gemm_f32(g, false, false, ROLE_POWER, q.s); });
    if (e != hipSuccess) return e;
    if (dmax == 3) {
      // R^3 = R^2 R: symmetric by structure, so its upper triangle is kept and
      // mirrored and g stays exactly symmetric
      g.prob[0].a = {R2, n, L.buf_stride, nullptr, 0};
      g.prob[0].c = R3;
      g.min_degree = 3;  // under the adaptive degree, the matrices at d = 3 only
      e = q.run(PMX_KC_GEMM_POWER, [&] { return launch_gemm_f32(g, false, false, ROLE_POWER, q.s); });
      if (e != hipSuccess) return e;
    }
  }
  if (!o.accelerate) return hipSuccess;
  SkinnyParams kp;
  memset(&kp, 0, sizeof(kp));
  kp.kbuf = kbuf;
  kp.variant = q.h->skinny_variant;
  kp.kld = L.kld;
  kp.kstride = L.kstride;
  kp.n = n;
  kp.ctrl = ctrl;
  kp.gram_partials = at<double>(ws, L.gram);
  kp.gram_stride = L.gstride;
  kp.cfg = cfg;
  kp.coef = coef;
  if (dmax > d) {
    kp.coef_up = make_coef(dmax);
    kp.lo_up = 0.3125f;  // the default interval of d = 3
    kp.hi_up = 2.46f;
  }
  auto job = [&](const float* m, int ic, int oc, int pw) {
    SkinnyJob j;
    j.mat = m;
    j.mat_ld = n;
    j.mat_stride = L.buf_stride;
    j.in_col = ic;
    j.out_col = oc;
    j.pow = pw;
    return j;
  };
  auto pass = [&](int njobs, bool gram) {
    return q.run(gram ? PMX_KC_SKINNY_ALPHA : PMX_KC_SKINNY,
                 [&] { return launch_skinny(kp, njobs, gram, batch, q.s); });
  };
  if (d >= 2) {
    kp.q = pp;
    kp.job[0] = job(R, 0, pp, 1);
    kp.job[1] = job(R2, 0, 2 * pp, 2);
    if ((e = pass(2, false)) != hipSuccess) return e;
    kp.q = 2 * pp;
    kp.job[0] = job(R2, pp, 3 * pp, 2);
    if ((e = pass(1, false)) != hipSuccess) return e;
    if (dmax == 3) {
      kp.job[0] = job(R2, 3 * pp, 5 * pp, 2);
      if ((e = pass(1, false)) != hipSuccess) return e;
    }
    kp.q = pp;
    kp.job[0] = job(R2, (2 * dmax - 1) * pp, (2 * dmax + 1) * pp, 2);
    return pass(1, true);
  }
  kp.q = pp;
  for (int j = 1; j <= 3; ++j) {
    kp.job[0] = job(R, (j - 1) * pp, j * pp, 1);
    if ((e = pass(1, j == 3)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Coefficients a_0..a_p of the inverse Newton residual map
// r(xi; alpha) = 1 - (1 - xi) (f + alpha xi^d)^p = sum_i alpha^i a_i(xi),
// f the Taylor polynomial of (1 - xi)^{-1/p} to degree d - 1:
//   a_0 = 1 - (1 - xi) f^p,  a_i = -binom(p, i) (1 - xi) f^{p-i} xi^{d i}.
double root_coeff(int j, int p) {
  double c = 1.0;
  for (int i = 0; i < j; ++i) c *= (1.0 / p + i) / (i + 1);
  return c;
}

AlphaCoefN make_coef_newton(int d, int p) {
  Poly f, om;
  for (int j = 0; j < d; ++j) f.c[j] = root_coeff(j, p);
  om.c[0] = 1.0;
  om.c[1] = -1.0;
  AlphaCoefN co;
  memset(&co, 0, sizeof(co));
  for (int i = 0; i <= p; ++i) {
    // (1 - xi) f^{p-i} xi^{d i}, in 10 coefficients (p d + 1 <= 9)
    double acc[16] = {0.0};
    double fp[16] = {0.0};
    fp[0] = 1.0;
    for (int t = 0; t < p - i; ++t) {
      double nx[16] = {0.0};
      for (int u = 0; u < 16; ++u)
        for (int v = 0; v < 8 && u + v < 16; ++v) nx[u + v] += fp[u] * f.c[v];
      memcpy(fp, nx, sizeof(fp));
    }
    for (int u = 0; u + 1 < 16; ++u) {
      acc[u] += fp[u];
      acc[u + 1] -= fp[u];
    }
    double binom = 1.0;
    for (int t = 0; t < i; ++t) binom = binom * (p - t) / (t + 1);
    for (int u = 0; u < 10; ++u) {
      const int src = u - d * i;
      co.a[i][u] = (src >= 0 && src < 16) ? -binom * acc[src] : 0.0;
    }
    if (i == 0) co.a[0][0] += 1.0;
  }
  co.taylor_d = root_coeff(d, p);
  return co;
}

// The PRISM coupled inverse Newton iteration for A^{-1/p}, fp32 (the
// iteration and its readings are documented with PMX_METHOD_INVERSE_NEWTON):
//   M_0 = A / c, X_0 = I, R_0 = I - M_0;  per update k:
//   R^2 (d = 2, triangle); Krylov passes K_1..K_{p d + 1} and alpha;
//   g = f(R) + alpha R^d written over R^2 (and into X_1 at k = 0);
//   g^2, g^4 (p = 4) (triangle); X_{k+1} = X_k g (k >= 1);
//   R_{k+1} = I - g^p M_k with M_{k+1} = g^p M_k kept (triangle, convergence).
// The outputs: X = c^{-1/p} X_k, then X_aux = A X^{p-1} from X.
pmx_status enqueue_inverse_newton(Enq& q, void* ws, const IterLayout& L, const pmx_matfn_opts& o,
                                  const IterCfg& cfg, const float* A, int lda, int64_t sa, int n,
                                  int p, float* X, int ldx, int64_t sx, float* XA, int ldaux,
                                  int64_t saux, int batch) {
  Ctrl* ctrl = at<Ctrl>(ws, L.ctrl);
  float* Xb[2] = {at<float>(ws, L.bufs[0]), at<float>(ws, L.bufs[1])};
  float* Mb[2] = {at<float>(ws, L.bufs[2]), at<float>(ws, L.bufs[3])};
  float* Rb = at<float>(ws, L.bufs[4]);
  float* Pb = at<float>(ws, L.bufs[5]);
  float* Tb = at<float>(ws, L.bufs[6]);
  float* Ub = at<float>(ws, L.bufs[7]);
  const int64_t bs = L.buf_stride;
  const int d = o.degree;
  const bool acc = o.accelerate != 0;
  const int J = p * d + 1;
  IterCfg c = cfg;
  c.taylor_d = (float)root_coeff(d, p);  // alpha without the sketch fit
  {
    StageInitParams ip;
    memset(&ip, 0, sizeof(ip));
    ip.a = A;
    ip.lda = lda;
    ip.a_stride = sa;
    ip.ybuf[0] = Mb[0];
    ip.ybuf[1] = Mb[1];
    ip.r = Rb;
    ip.buf_stride = bs;
    ip.n = n;
    ip.stage = 0;
    ip.ctrl = ctrl;
    ip.partials = at<double>(ws, L.partials);
    ip.partial_stride = L.pstride;
    ip.cfg = c;
    ip.sketch = make_sketch(L, ws, c, n, 0, 0, acc);
    PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_sqrt_stage_init(ip, batch, q.s); }));
  }
  auto sym_product = [&](const float* a, const float* b, float* out) {
    GemmParams g = gemm_base(q.h, n, n, n, batch);
    g.prob[0].a = {a, n, bs, nullptr, 0};
    g.prob[0].b = {b, n, bs, nullptr, 0};
    g.prob[0].c = out;
    g.prob[0].ldc = n;
    g.prob[0].stride_c = bs;
    g.ctrl = ctrl;
    g.sym = 1;
    if (q.h->split_k) use_split(g, ws, L);
    set_vec(g);
    return q.run(PMX_KC_GEMM_POWER, [&] { return launch_gemm_f32(g, false, false, ROLE_POWER, q.s); });
  };
  Poller poll(q, ctrl, batch);
  for (int k = 0; k < o.max_iter; ++k) {
    bool stop = false;
    PMX_TRY(poll.step(k, &stop));
    if (stop) break;
    const int cur = k & 1, nxt = cur ^ 1;
    if (d == 2) PMX_TRY(sym_product(Rb, Rb, Pb));
    if (acc) {
      SkinnyParams kp;
      memset(&kp, 0, sizeof(kp));
      kp.kbuf = at<float>(ws, L.kbuf);
      kp.variant = q.h->skinny_variant;
      kp.kld = L.kld;
      kp.kstride = L.kstride;
      kp.n = n;
      kp.ctrl = ctrl;
      kp.gram_partials = at<double>(ws, L.gram);
      kp.gram_stride = L.gstride;
      kp.cfg = c;
      kp.coef = make_coef(d);
      kp.gram_j = J;
      if (p == 4) {
        kp.newton_p = 4;
        kp.coef_n = make_coef_newton(d, 4);
      }
      const int pp = o.sketch_p;
      auto job = [&](const float* m, int ic, int oc, int pw) {
        SkinnyJob j;
        j.mat = m;
        j.mat_ld = n;
        j.mat_stride = bs;
        j.in_col = ic;
        j.out_col = oc;
        j.pow = pw;
        return j;
      };
      auto pass = [&](int njobs, bool gram) {
        return q.run(gram ? PMX_KC_SKINNY_ALPHA : PMX_KC_SKINNY,
                     [&] { return launch_skinny(kp, njobs, gram, batch, q.s); });
      };
      if (d == 2) {
        // K_1 = R S, K_2 = R^2 S; pairs [K_{t+1} | K_{t+2}] = R^2 [K_{t-1} | K_t];
        // the last block K_J = R^2 K_{J-2} with the Gram and alpha (J odd)
        kp.q = pp;
        kp.job[0] = job(Rb, 0, pp, 1);
        kp.job[1] = job(Pb, 0, 2 * pp, 2);
        PMX_TRY(pass(2, false));
        int t = 2;
        while (J - t >= 3) {
          kp.q = 2 * pp;
          kp.job[0] = job(Pb, (t - 1) * pp, (t + 1) * pp, 2);
          PMX_TRY(pass(1, false));
          t += 2;
        }
        kp.q = pp;
        kp.job[0] = job(Pb, (J - 2) * pp, J * pp, 2);
        PMX_TRY(pass(1, true));
      } else {
        kp.q = pp;
        for (int j = 1; j <= J; ++j) {
          kp.job[0] = job(Rb, (j - 1) * pp, j * pp, 1);
          PMX_TRY(pass(1, j == J));
        }
      }
    }
    {
      FormGParams fp;
      memset(&fp, 0, sizeof(fp));
      fp.r = Rb;
      fp.r2 = d == 2 ? Pb : nullptr;
      fp.dst = Pb;
      fp.dst2 = k == 0 ? Xb[1] : nullptr;  // X_1 = X_0 g = g
      fp.stride = bs;
      fp.n = n;
      fp.degree = d;
      fp.c0 = (float)root_coeff(0, p);
      fp.c1 = (float)root_coeff(1, p);
      fp.ctrl = ctrl;
      fp.sketch = make_sketch(L, ws, c, n, k + 1, 0, acc && k + 1 < o.max_iter);
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g(fp, batch, q.s); }));
    }
    PMX_TRY(sym_product(Pb, Pb, Tb));                // g^2
    const float* gp = Tb;
    if (p == 4) {
      PMX_TRY(sym_product(Tb, Tb, Ub));              // g^4
      gp = Ub;
    }
    if (k > 0) {
      GemmParams u = gemm_base(q.h, n, n, n, batch);
      u.ctrl = ctrl;
      u.prob[0].a = {Xb[cur], n, bs, nullptr, 0};
      u.prob[0].b = {Pb, n, bs, nullptr, 0};
      u.prob[0].c = Xb[nxt];
      u.prob[0].ldc = n;
      u.prob[0].stride_c = bs;
      if (q.h->split_k) use_split(u, ws, L);
      set_vec(u);
      PMX_TRY(q.run(PMX_KC_GEMM_UPDATE, [&] { return launch_gemm_f32(u, false, false, ROLE_UPDATE, q.s); }));
    }
    {
      // R_{k+1} = I - g^p M_k, and M_{k+1} = g^p M_k kept (symmetric by
      // construction: g^p and M_k are polynomials in A)
      GemmParams r = gemm_base(q.h, n, n, n, batch);
      r.ctrl = ctrl;
      r.prob[0].a = {gp, n, bs, nullptr, 0};
      r.prob[0].b = {Mb[cur], n, bs, nullptr, 0};
      r.prob[0].c = Rb;
      r.prob[0].ldc = n;
      r.prob[0].stride_c = bs;
      r.prob[1].c = Mb[nxt];
      r.prob[1].ldc = n;
      r.prob[1].stride_c = bs;
      r.resid_keep = 1;
      r.partials = at<double>(ws, L.partials);
      r.partial_stride = L.pstride;
      r.products = (d - 1) + (p == 4 ? 2 : 1) + (k > 0 ? 1 : 0) + 1;
      r.count_update = 1;
      r.cfg = c;
      r.sym = 1;
      if (q.h->split_k) use_split(r, ws, L);
      set_vec(r);
      PMX_TRY(q.run(PMX_KC_GEMM_RESID, [&] { return launch_gemm_f32(r, false, false, ROLE_RESID, q.s); }));
    }
  }
  RootFinishParams fp;
  memset(&fp, 0, sizeof(fp));
  fp.ybuf[0] = Xb[0];
  fp.ybuf[1] = Xb[1];
  fp.zbuf[0] = Xb[0];
  fp.zbuf[1] = Xb[1];
  fp.buf_stride = bs;
  fp.x = X;
  fp.ldx = ldx;
  fp.x_stride = sx;
  fp.n = n;
  fp.expo_x = -1.0 / p;
  fp.ctrl = ctrl;
  PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_root_finish(fp, batch, q.s); }));
  if (XA) {
    // A^{1/p} = A X^{p-1} from the scaled output (no gating: a failed matrix
    // has X = NaN and its auxiliary output follows)
    auto product = [&](const float* a, int64_t la, int64_t sta, const float* b, int64_t lb,
                       int64_t stb, float* out, int64_t lo_, int64_t sto) {
      GemmParams g = gemm_base(q.h, n, n, n, batch);
      g.prob[0].a = {a, la, sta, nullptr, 0};
      g.prob[0].b = {b, lb, stb, nullptr, 0};
      g.prob[0].c = out;
      g.prob[0].ldc = lo_;
      g.prob[0].stride_c = sto;
      set_vec(g);
      return q.run(PMX_KC_OTHER, [&] { return launch_gemm_f32(g, false, false, ROLE_POWER, q.s); });
    };
    if (p == 2) {
      PMX_TRY(product(A, lda, sa, X, ldx, sx, XA, ldaux, saux));
    } else {
      PMX_TRY(product(X, ldx, sx, X, ldx, sx, Tb, n, bs));       // X^2
      PMX_TRY(product(Tb, n, bs, X, ldx, sx, Ub, n, bs));        // X^3
      PMX_TRY(product(A, lda, sa, Ub, n, bs, XA, ldaux, saux));  // A X^3
    }
  }
  return PMX_OK;
}

}  // namespace

int handle_device(pmx_handle h) { return h ? h->device : -1; }

}  // namespace pmx

using namespace pmx;

// ======================================================================= ABI
extern "C" {

const char* pmx_status_string(pmx_status s) {
  switch (s) {
    case PMX_OK: return "PMX_OK";
    case PMX_ERR_INVALID_VALUE: return "PMX_ERR_INVALID_VALUE: invalid argument";
    case PMX_ERR_NOT_SUPPORTED: return "PMX_ERR_NOT_SUPPORTED: not supported by this build";
    case PMX_ERR_WORKSPACE: return "PMX_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case PMX_ERR_ALIAS: return "PMX_ERR_ALIAS: overlapping input/output arguments";
    case PMX_ERR_HIP: return "PMX_ERR_HIP: HIP runtime error";
  }
  return "unknown pmx_status";
}

int pmx_version(void) { return PMX_VERSION_MAJOR * 1000 + PMX_VERSION_MINOR; }

pmx_status pmx_matfn_opts_default(pmx_matfn_opts* o) {
  if (!o) return PMX_ERR_INVALID_VALUE;
  o->struct_version = PMX_OPTS_VERSION;
  o->degree = 2;
  o->sketch_p = 8;
  o->max_iter = 30;
  o->accelerate = 1;
  o->alpha_lo = NAN;
  o->alpha_hi = NAN;
  o->tol = 1e-6f;
  o->seed = 0;
  o->fp64_iters = 0;
  o->degree_max = 0;
  o->adapt_ratio = 0.3f;
  o->method = PMX_METHOD_NEWTON_SCHULZ;
  o->scale_mode = PMX_SCALE_FROBENIUS;
  o->reserved = 0;
  return PMX_OK;
}

pmx_status pmx_create(pmx_handle* handle, int device) {
  if (!handle) return PMX_ERR_INVALID_VALUE;
  *handle = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess) return PMX_ERR_HIP;
  if (device < 0 || device >= count) return PMX_ERR_INVALID_VALUE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return PMX_ERR_HIP;
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return PMX_ERR_NOT_SUPPORTED;
  pmx_context* c = new (std::nothrow) pmx_context;
  if (!c) return PMX_ERR_HIP;
  c->device = device;
  c->num_cu = prop.multiProcessorCount;
  // tuning knobs for experiments (environment, read once per handle)
  c->gemm_blocks_per_cu = 0;
  c->gemm_cfg = -1;
  c->gemm_map = 2;
  if (const char* e = getenv("PMX_GEMM_BLOCKS_PER_CU")) c->gemm_blocks_per_cu = atoi(e);
  if (const char* e = getenv("PMX_GEMM_CFG")) c->gemm_cfg = atoi(e);
  if (const char* e = getenv("PMX_GEMM_MAP")) c->gemm_map = atoi(e);
  c->bf16_cfg = -1;
  c->bf16_map = 1;
  if (const char* e = getenv("PMX_BF16_CFG")) c->bf16_cfg = atoi(e);
  if (const char* e = getenv("PMX_BF16_MAP")) c->bf16_map = atoi(e);
  c->skinny_variant = 0;
  if (const char* e = getenv("PMX_SKINNY")) c->skinny_variant = atoi(e);
  c->bf16_dma = 0;
  if (const char* e = getenv("PMX_BF16_DMA")) c->bf16_dma = atoi(e);
  c->bf16_mn = 1;
  if (const char* e = getenv("PMX_BF16_MN")) c->bf16_mn = atoi(e);
  c->bf16_persist = 1;
  if (const char* e = getenv("PMX_BF16_PERSIST")) c->bf16_persist = atoi(e);
  c->bf16_early = 1;
  if (const char* e = getenv("PMX_BF16_EARLY")) c->bf16_early = atoi(e);
  c->small_fused = 1;
  if (const char* e = getenv("PMX_SMALL")) c->small_fused = atoi(e);
  c->split_k = 1;
  if (const char* e = getenv("PMX_SPLITK")) c->split_k = atoi(e);
  // measured slower for the 32 x 4096 x 1024 polar (320 triangle tiles of 256^2
  // still take two rounds of the compute units, and the mirrored stores cost;
  // a split-k tail that cut the second round to 64 x 4 pieces took the
  // residual from 246 to 204 us, but summing the pieces in a second launch
  // took 96 us on the 64 tail tiles)
  c->bf16_sym = 0;
  if (const char* e = getenv("PMX_BF16_SYM")) c->bf16_sym = atoi(e);
  c->bf16_sym_small = 0;
  if (const char* e = getenv("PMX_BF16_SYM_SMALL")) c->bf16_sym_small = atoi(e);
  c->f64_tile = 0;
  if (const char* e = getenv("PMX_F64_TILE")) c->f64_tile = atoi(e);
  if (c->f64_tile != 64 && c->f64_tile != 128) c->f64_tile = 0;
  {
    // the scratch of pmx_precond_apply_noalloc, resolved once per device
    DeviceGuard dg(device);
    if (!dg.ok || resolve_scratch(device) != hipSuccess) {
      delete c;
      return PMX_ERR_HIP;
    }
  }
  *handle = c;
  return PMX_OK;
}

pmx_status pmx_destroy(pmx_handle h) {
  if (!h) return PMX_ERR_INVALID_VALUE;
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->poll_ev)
    if (e) (void)hipEventDestroy(e);
  if (h->poll_host) (void)hipHostFree(h->poll_host);
  delete h;
  return PMX_OK;
}

pmx_status pmx_set_host_poll(pmx_handle h, int chunk) {
  if (!h || chunk < 0 || chunk > kMaxIter) return PMX_ERR_INVALID_VALUE;
  if (chunk > 0 && !h->poll_host) {
    DeviceGuard dg(h->device);
    if (!dg.ok) return PMX_ERR_HIP;
    void* p = nullptr;
    if (hipHostMalloc(&p, 2 * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent) !=
        hipSuccess)
      return PMX_ERR_HIP;
    void* d = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess ||
        hipEventCreateWithFlags(&e0, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&e1, hipEventDisableTiming) != hipSuccess) {
      if (e0) (void)hipEventDestroy(e0);
      (void)hipHostFree(p);
      return PMX_ERR_HIP;
    }
    h->poll_host = (int32_t*)p;
    h->poll_dev = (int32_t*)d;
    h->poll_ev[0] = e0;
    h->poll_ev[1] = e1;
  }
  h->poll_chunk = chunk;
  return PMX_OK;
}

pmx_status pmx_trace_enable(pmx_handle h, int enable) {
  if (!h || (enable != 0 && enable != 1)) return PMX_ERR_INVALID_VALUE;
  h->trace = enable != 0;
  h->recs.clear();
  h->used = 0;
  return PMX_OK;
}

pmx_status pmx_trace_collect(pmx_handle h, double* ms, int64_t* launches) {
  if (!h || !ms || !launches) return PMX_ERR_INVALID_VALUE;
  for (int i = 0; i < PMX_KC_COUNT; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  pmx_status st = PMX_OK;
  for (const auto& r : h->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) {
      st = PMX_ERR_HIP;
      break;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      st = PMX_ERR_HIP;
      break;
    }
    ms[r.cls] += t;
    launches[r.cls] += 1;
  }
  h->recs.clear();
  h->used = 0;
  return st;
}

// fp32: Y and Z ping-pong, R, R^2; with fp64 leading updates also their fp64
// counterparts (Y, Z ping-pong, R, R^2).
static int inv_root_f64_bufs(const pmx_matfn_opts& o) { return o.fp64_iters > 0 ? 6 : 0; }
// n x n residual buffers: R, R^2 (g is written over R^2), and R^3 for d = 3.
// Inverse Newton: the four big buffers are X and M ping-pong, then R, R^2 / g,
// g^2 and g^4.
static int small_bufs(const pmx_matfn_opts& o) {
  if (o.method == PMX_METHOD_INVERSE_NEWTON) return 4;
  return std::max(o.degree, o.degree_max) == 3 ? 3 : 2;
}
static size_t inv_root_ws(int n, int batch, const pmx_matfn_opts& o) {
  return iter_layout(n, n, batch, o, 4, small_bufs(o), sizeof(float), inv_root_f64_bufs(o)).total;
}
// fp32: X ping-pong, R, R^2 (and R^3 for d = 3).  bf16: X and X^T
// ping-pong, R, R^2 (fp32), and the bf16 operands R and g.
static int polar_bufs(pmx_dtype dt, const pmx_matfn_opts& o) {
  return dt == PMX_BF16 ? 8 : (std::max(o.degree, o.degree_max) == 3 ? 5 : 4);
}
static size_t polar_ws(int m, int n, int batch, const pmx_matfn_opts& o, pmx_dtype dt) {
  const int rows = std::max(m, n), cols = std::min(m, n);
  return iter_layout(rows, cols, batch, o, polar_bufs(dt, o), 0, sizeof(float)).total;
}
static size_t apply_ws(int m, int n, int batch, pmx_dtype dt) {
  // fp32: T = L^{-1/4} G; bf16: G in fp32, T and P in fp32
  const size_t one = align_up(sizeof(float) * (size_t)m * n * batch);
  return dt == PMX_BF16 ? 3 * one : one;
}
// Statistics: G^T in fp32 (and G widened to fp32 for bf16 gradients), then
// the split-k counters and partial-tile slots of the two triangle products.
struct StatsLayout {
  size_t gt, gn, skc, skp, total;
  int64_t skcap;
};
static StatsLayout stats_layout(int m, int n, int batch, pmx_dtype dt) {
  StatsLayout L;
  const size_t one = align_up(sizeof(float) * (size_t)m * n * batch);
  size_t off = 0;
  L.gt = off;
  off += one;
  L.gn = off;
  if (dt == PMX_BF16) off += one;
  L.skc = off;
  off = align_up(off + sizeof(uint32_t) * (size_t)kSplitMaxWorkers);
  L.skcap = (int64_t)2 * kSplitMaxWorkers * (std::max(m, n) >= 512 ? 128 * 128 : 64 * 64);
  L.skp = off;
  off = align_up(off + sizeof(float) * (size_t)L.skcap);
  L.total = off;
  return L;
}
static size_t stats_ws(int m, int n, int batch, pmx_dtype dt) {
  return stats_layout(m, n, batch, dt).total;
}

pmx_status pmx_workspace_size(pmx_handle h, pmx_op op, int m, int n, int batch,
                              pmx_dtype dtype, const pmx_matfn_opts* opts, size_t* bytes) {
  (void)h;  // sizes do not depend on the device; the handle may be NULL
  if (!bytes || batch < 1 || n < 1 || n > kMaxN) return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  pmx_matfn_opts o;
  switch (op) {
    case PMX_OP_STATS:
      if (m < 1 || m > kMaxN) return PMX_ERR_INVALID_VALUE;
      *bytes = stats_ws(m, n, batch, dtype);
      return PMX_OK;
    case PMX_OP_APPLY:
      if (m < 1 || m > kMaxN) return PMX_ERR_INVALID_VALUE;
      *bytes = apply_ws(m, n, batch, dtype);
      return PMX_OK;
    case PMX_OP_INV_ROOT:
      if (!resolve_opts(opts, &o)) return PMX_ERR_INVALID_VALUE;
      *bytes = inv_root_ws(n, batch, o);
      return PMX_OK;
    case PMX_OP_POLAR:
      if (m < 1 || m > kMaxN) return PMX_ERR_INVALID_VALUE;
      if (!resolve_opts(opts, &o)) return PMX_ERR_INVALID_VALUE;
      *bytes = polar_ws(m, n, batch, o, dtype);
      return PMX_OK;
    case PMX_OP_POLAR_VARBATCH:
      // the device copy of the block descriptors
      *bytes = align_up(sizeof(pmx_polar_block) * (size_t)batch);
      return PMX_OK;
  }
  return PMX_ERR_INVALID_VALUE;
}

static pmx_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return PMX_OK;
  if (!ws || have < need || ((uintptr_t)ws % kAlign) != 0) return PMX_ERR_WORKSPACE;
  return PMX_OK;
}

// ------------------------------------------------------------------ stats
pmx_status pmx_shampoo_stats_update_batched(pmx_handle h, const void* G, pmx_dtype dtype,
                                            int m, int n, int ldg, int64_t sg, float* L,
                                            int ldl, int64_t sl, float* R, int ldr,
                                            int64_t sr, float beta, float eps, int batch,
                                            void* ws, size_t ws_bytes, void* stream) {
  if (!h || !G || m < 1 || n < 1 || m > kMaxN || n > kMaxN || batch < 1)
    return PMX_ERR_INVALID_VALUE;
  if (!L && !R) return PMX_ERR_INVALID_VALUE;
  if (!(beta >= 0.f && beta <= 1.f) || !isfinite(eps)) return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  if (!batch_layout_ok(m, n, ldg, sg, 1) || sg < 0) return PMX_ERR_INVALID_VALUE;
  if (batch > 1 && sg < (int64_t)(m - 1) * ldg + n && sg != 0) return PMX_ERR_INVALID_VALUE;
  if (L && !batch_layout_ok(m, m, ldl, sl, batch)) return PMX_ERR_INVALID_VALUE;
  if (R && !batch_layout_ok(n, n, ldr, sr, batch)) return PMX_ERR_INVALID_VALUE;
  const bool bf = dtype == PMX_BF16;
  const size_t need = stats_ws(m, n, batch, dtype);
  pmx_status wst = check_ws(ws, ws_bytes, need);
  if (wst != PMX_OK) return wst;
  const Extent eg = extent_of(G, m, n, ldg, sg, batch, bf ? 2 : 4);
  const Extent el = extent_of(L, m, m, ldl, sl, batch, 4);
  const Extent er = extent_of(R, n, n, ldr, sr, batch, 4);
  Extent ew;
  ew.lo = (uintptr_t)ws;
  ew.hi = ew.lo + need;
  ew.valid = need > 0;
  if (overlap(eg, el) || overlap(eg, er) || overlap(el, er) || overlap(ew, eg) ||
      overlap(ew, el) || overlap(ew, er))
    return PMX_ERR_ALIAS;
  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  // G^T (and G in fp32 for bf16 gradients) once, so that both Grams are
  // NN products; they run as upper-triangle tiles, mirrored (SYRK)
  const int nb = sg == 0 ? 1 : batch;
  const StatsLayout SL = stats_layout(m, n, nb, dtype);
  const int64_t plane = (int64_t)m * n;
  float* gt = at<float>(ws, SL.gt);
  float* gn = bf ? at<float>(ws, SL.gn) : nullptr;
  uint32_t* skc = at<uint32_t>(ws, SL.skc);
  PMX_TRY(q.run(PMX_KC_OTHER, [&] {
    return launch_stats_operands(G, bf, ldg, sg, m, n, nb, gt, gn, skc, kSplitMaxWorkers, q.s);
  }));
  const float* g = bf ? gn : (const float*)G;
  const int64_t ldgf = bf ? n : ldg;
  const int64_t sgf = sg == 0 ? 0 : (bf ? plane : sg);
  const int64_t sgt = sg == 0 ? 0 : plane;
  const float omb = 1.f - beta;
  auto stats = [&](int dim, int k, GemmOperand a, GemmOperand b, float* C, int ldc, int64_t sc) {
    GemmParams p = gemm_base(q.h, dim, dim, k, batch);
    p.prob[0].a = a;
    p.prob[0].b = b;
    p.prob[0].c = C;
    p.prob[0].ldc = ldc;
    p.prob[0].stride_c = sc;
    p.beta = beta;
    p.omb = omb;
    p.eps = eps;
    p.sym = 1;
    p.sk_part = at<float>(ws, SL.skp);
    p.sk_cnt = skc;
    p.sk_cap = SL.skcap;
    set_vec(p);
    return q.run(PMX_KC_GEMM_STATS, [&] { return launch_gemm_f32(p, false, false, ROLE_STATS, q.s); });
  };
  // L = G G^T: A = G (m x n), B = G^T (n x m);  R = G^T G: A = G^T, B = G
  if (L) PMX_TRY(stats(m, n, {g, ldgf, sgf, nullptr, 0}, {gt, m, sgt, nullptr, 0}, L, ldl, sl));
  if (R) PMX_TRY(stats(n, m, {gt, m, sgt, nullptr, 0}, {g, ldgf, sgf, nullptr, 0}, R, ldr, sr));
  return PMX_OK;
}

pmx_status pmx_shampoo_stats_update(pmx_handle h, const void* G, pmx_dtype dtype, int m,
                                    int n, int ldg, float* L, int ldl, float* R, int ldr,
                                    float beta, float eps, void* ws, size_t ws_bytes,
                                    void* stream) {
  return pmx_shampoo_stats_update_batched(h, G, dtype, m, n, ldg, 0, L, ldl, 0, R, ldr, 0,
                                          beta, eps, 1, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ inverse roots
pmx_status pmx_matfn_inv_root_batched(pmx_handle h, const float* A, int n, int lda,
                                      int64_t sa, int p, float* X, int ldx, int64_t sx,
                                      float* XA, int ldaux, int64_t saux, int batch,
                                      const pmx_matfn_opts* opts, pmx_matfn_info* info,
                                      void* ws, size_t ws_bytes, void* stream) {
  if (!h || !A || !X || n < 1 || n > kMaxN || batch < 1) return PMX_ERR_INVALID_VALUE;
  if (p != 2 && p != 4) return PMX_ERR_INVALID_VALUE;
  pmx_matfn_opts o;
  if (!resolve_opts(opts, &o, p)) return PMX_ERR_INVALID_VALUE;
  if (lda < n || sa < 0 || (batch > 1 && sa != 0 && sa < (int64_t)(n - 1) * lda + n))
    return PMX_ERR_INVALID_VALUE;
  if (!batch_layout_ok(n, n, ldx, sx, batch)) return PMX_ERR_INVALID_VALUE;
  if (XA && !batch_layout_ok(n, n, ldaux, saux, batch)) return PMX_ERR_INVALID_VALUE;
  // d = 3 runs the fp32 updates only
  if (o.degree == 3 && o.fp64_iters > 0) return PMX_ERR_NOT_SUPPORTED;
  const IterLayout Lw =
      iter_layout(n, n, batch, o, 4, small_bufs(o), sizeof(float), inv_root_f64_bufs(o));
  pmx_status st = check_ws(ws, ws_bytes, Lw.total);
  if (st != PMX_OK) return st;
  const Extent ea = extent_of(A, n, n, lda, sa, batch, 4);
  const Extent ex = extent_of(X, n, n, ldx, sx, batch, 4);
  const Extent eaux = extent_of(XA, n, n, ldaux, saux, batch, 4);
  Extent ew;
  ew.lo = (uintptr_t)ws;
  ew.hi = ew.lo + Lw.total;
  ew.valid = true;
  Extent ei = extent_of(info, 1, (int)sizeof(pmx_matfn_info), 0, sizeof(pmx_matfn_info), batch, 1);
  if (overlap(ea, ex) || overlap(ea, eaux) || overlap(ex, eaux) || overlap(ew, ea) ||
      overlap(ew, ex) || overlap(ew, eaux) || overlap(ei, ea) || overlap(ei, ex) ||
      overlap(ei, eaux) || overlap(ei, ew))
    return PMX_ERR_ALIAS;

  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  Ctrl* ctrl = at<Ctrl>(ws, Lw.ctrl);
  double* partials = at<double>(ws, Lw.partials);
  float* Yb[2] = {at<float>(ws, Lw.bufs[0]), at<float>(ws, Lw.bufs[1])};
  float* Zb[2] = {at<float>(ws, Lw.bufs[2]), at<float>(ws, Lw.bufs[3])};
  float* Rb = at<float>(ws, Lw.bufs[4]);
  float* R2b = at<float>(ws, Lw.bufs[5]);
  float* R3b = small_bufs(o) == 3 ? at<float>(ws, Lw.bufs[6]) : nullptr;
  const IterCfg cfg = make_cfg(o, n, info);
  const AlphaCoef coef = make_coef(o.degree);
  const int d = o.degree;
  const bool acc = o.accelerate != 0;

  const int stages = (p == 4) ? 2 : 1;
  if (n <= kSmallMaxN && h->small_fused && o.fp64_iters == 0 &&
      std::max(o.degree, o.degree_max) <= 2 && o.method == PMX_METHOD_NEWTON_SCHULZ &&
      o.scale_mode == PMX_SCALE_FROBENIUS) {
    SmallRootParams sp;
    memset(&sp, 0, sizeof(sp));
    sp.a = A;
    sp.lda = lda;
    sp.a_stride = sa;
    sp.x = X;
    sp.ldx = ldx;
    sp.x_stride = sx;
    sp.aux = XA;
    sp.ldaux = ldaux;
    sp.aux_stride = saux;
    sp.n = n;
    sp.stages = stages;
    sp.expo_x = -1.0 / p;
    sp.expo_aux = 1.0 / p;
    sp.c0 = (float)taylor(0);
    sp.c1 = (float)taylor(1);
    sp.cfg = cfg;
    sp.coef = coef;
    PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_small_root(sp, batch, q.s); }));
    return PMX_OK;
  }
  PMX_TRY(q.run(PMX_KC_OTHER, [&] {
    return launch_ctrl_reset(ctrl, info, batch, o.degree, at<uint32_t>(ws, Lw.skc),
                             kSplitMaxWorkers, q.s);
  }));
  PMX_TRY(q.run(PMX_KC_OTHER, [&] {
    return launch_fro_scale(A, false, n, n, lda, sa, batch, ctrl, partials, Lw.pstride, info, q.s);
  }));
  if (o.scale_mode == PMX_SCALE_POWER)
    PMX_TRY(enqueue_power_scale(q, ws, Lw, cfg, A, lda, sa, n, batch));
  if (o.method == PMX_METHOD_INVERSE_NEWTON)
    return enqueue_inverse_newton(q, ws, Lw, o, cfg, A, lda, sa, n, p, X, ldx, sx, XA, ldaux,
                                  saux, batch);
  const int k64 = std::min(o.fp64_iters, o.max_iter);
  double* Y64[2] = {at<double>(ws, Lw.b64[0]), at<double>(ws, Lw.b64[1])};
  double* Z64[2] = {at<double>(ws, Lw.b64[2]), at<double>(ws, Lw.b64[3])};
  double* R64 = at<double>(ws, Lw.b64[4]);
  double* R264 = at<double>(ws, Lw.b64[5]);
  auto gemm64 = [&](int nprob) {
    Gemm64Params g;
    memset(&g, 0, sizeof(g));
    g.nprob = nprob;
    g.n = n;
    g.batch = batch;
    g.stride = Lw.buf_stride;
    g.stride32 = Lw.buf_stride;
    g.ctrl = ctrl;
    g.degree = d;
    g.c0 = taylor(0);
    g.c1 = taylor(1);
    g.num_cu = q.h->num_cu;
    g.tile = q.h->f64_tile;
    return g;
  };
  auto plain64 = [](const double* m) { return Gemm64Operand{m}; };
  for (int stage = 0; stage < stages; ++stage) {
    if (k64 > 0) {
      // leading updates in fp64 (same sequence as the fp32 loop below)
      StageInit64Params ip;
      memset(&ip, 0, sizeof(ip));
      ip.a = A;
      ip.lda = lda;
      ip.a_stride = sa;
      ip.ybuf32[0] = Yb[0];
      ip.ybuf32[1] = Yb[1];
      ip.stride32 = Lw.buf_stride;
      ip.y64 = Y64[0];
      ip.r64 = R64;
      ip.r32 = Rb;
      ip.stride = Lw.buf_stride;
      ip.n = n;
      ip.stage = stage;
      ip.ctrl = ctrl;
      ip.partials = partials;
      ip.partial_stride = Lw.pstride;
      ip.cfg = cfg;
      ip.sketch = make_sketch(Lw, ws, cfg, n, 0, stage, acc);
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_stage_init_f64(ip, batch, q.s); }));
      for (int k = 0; k < k64; ++k) {
        if (d == 2) {
          Gemm64Params g = gemm64(1);
          g.sym = 1;
          g.prob[0].a = plain64(R64);
          g.prob[0].b = plain64(R64);
          g.prob[0].c = R264;
          g.prob[0].c32 = R2b;
          PMX_TRY(q.run(PMX_KC_GEMM_POWER, [&] { return launch_gemm_f64(g, ROLE_POWER, q.s); }));
        }
        PMX_TRY(enqueue_power_and_alpha(q, ws, Lw, o, cfg, coef, n, batch, Rb, R2b, nullptr, false));
        const int cur = k & 1, nxt = cur ^ 1;
        Gemm64Params u = gemm64(k == 0 ? 1 : 2);
        // g = f_{d-1}(R) + alpha R^d in fp64: into Z_1 at k = 0, else over
        // R^2 (the Krylov passes have read its fp32 copy)
        FormG64Params fp;
        memset(&fp, 0, sizeof(fp));
        fp.r = R64;
        fp.r2 = (d == 2) ? R264 : nullptr;
        fp.dst = k == 0 ? Z64[1] : R264;
        fp.stride = Lw.buf_stride;
        fp.n = n;
        fp.degree = d;
        fp.c0 = taylor(0);
        fp.c1 = taylor(1);
        fp.ctrl = ctrl;
        PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g_f64(fp, batch, q.s); }));
        if (k == 0) {
          u.prob[0].a = plain64(Y64[0]);
          u.prob[0].b = plain64(Z64[1]);
          u.prob[0].c = Y64[1];
        } else {
          u.prob[0].a = plain64(Y64[cur]);
          u.prob[0].b = plain64(R264);
          u.prob[0].c = Y64[nxt];
          u.prob[1].a = plain64(R264);
          u.prob[1].b = plain64(Z64[cur]);
          u.prob[1].c = Z64[nxt];
        }
        PMX_TRY(q.run(PMX_KC_GEMM_UPDATE, [&] { return launch_gemm_f64(u, ROLE_UPDATE, q.s); }));
        Gemm64Params r = gemm64(1);
        r.sym = 1;
        r.prob[0].a = plain64(Z64[nxt]);
        r.prob[0].b = plain64(Y64[nxt]);
        r.prob[0].c = R64;
        r.prob[0].c32 = Rb;
        r.partials = partials;
        r.partial_stride = Lw.pstride;
        r.products = (d - 1) + 1 + (k > 0 ? 1 : 0) + 1;
        r.count_update = 1;
        r.cfg = cfg;
        r.sketch = make_sketch(Lw, ws, cfg, n, k + 1, stage, acc && k + 1 < o.max_iter);
        PMX_TRY(q.run(PMX_KC_GEMM_RESID, [&] { return launch_gemm_f64(r, ROLE_RESID, q.s); }));
      }
      Handover64Params hp;
      memset(&hp, 0, sizeof(hp));
      hp.y64[0] = Y64[0];
      hp.y64[1] = Y64[1];
      hp.z64[0] = Z64[0];
      hp.z64[1] = Z64[1];
      hp.y32[0] = Yb[0];
      hp.y32[1] = Yb[1];
      hp.z32[0] = Zb[0];
      hp.z32[1] = Zb[1];
      hp.stride = Lw.buf_stride;
      hp.stride32 = Lw.buf_stride;
      hp.n = n;
      hp.stage = stage;
      hp.ctrl = ctrl;
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_handover_f64(hp, batch, q.s); }));
    } else {
      StageInitParams ip;
      ip.a = A;
      ip.lda = lda;
      ip.a_stride = sa;
      ip.ybuf[0] = Yb[0];
      ip.ybuf[1] = Yb[1];
      ip.r = Rb;
      ip.buf_stride = Lw.buf_stride;
      ip.n = n;
      ip.stage = stage;
      ip.ctrl = ctrl;
      ip.partials = partials;
      ip.partial_stride = Lw.pstride;
      ip.cfg = cfg;
      ip.sketch = make_sketch(Lw, ws, cfg, n, 0, stage, acc);
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_sqrt_stage_init(ip, batch, q.s); }));
    }
    Poller poll(q, ctrl, batch);
    for (int k = k64; k < o.max_iter; ++k) {
      bool stop = false;
      PMX_TRY(poll.step(k - k64, &stop));
      if (stop) break;
      PMX_TRY(enqueue_power_and_alpha(q, ws, Lw, o, cfg, coef, n, batch, Rb, R2b, R3b));
      const int cur = k & 1, nxt = cur ^ 1;
      GemmParams u = gemm_base(q.h, n, n, n, batch);
      u.ctrl = ctrl;
      u.degree = d;
      u.c0 = (float)taylor(0);
      u.c1 = (float)taylor(1);
      // the sketch of update k + 1 is generated with g (after the Krylov
      // passes of update k have read S_k)
      const SketchJob next_sketch = make_sketch(Lw, ws, cfg, n, k + 1, stage, acc && k + 1 < o.max_iter);
      if (k == 0) {
        // Z_1 = g Z_0 = g is written explicitly; Y_1 = Y_0 g reads it back.
        FormGParams fp;
        memset(&fp, 0, sizeof(fp));
        fp.r = Rb;
        fp.r2 = (d >= 2) ? R2b : nullptr;
        fp.r3 = R3b;
        fp.c2 = (float)taylor(2);
        fp.adaptive = cfg.degree_max > d;
        fp.dst = Zb[1];
        fp.stride = Lw.buf_stride;
        fp.n = n;
        fp.degree = d;
        fp.c0 = (float)taylor(0);
        fp.c1 = (float)taylor(1);
        fp.ctrl = ctrl;
        fp.sketch = next_sketch;
        PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g(fp, batch, q.s); }));
        u.prob[0].a = {Yb[0], n, Lw.buf_stride, nullptr, 0};
        u.prob[0].b = {Zb[1], n, Lw.buf_stride, nullptr, 0};
        u.prob[0].c = Yb[1];
        u.prob[0].ldc = n;
        u.prob[0].stride_c = Lw.buf_stride;
      } else {
        // g written once (in place of R^2, which the Krylov passes have read),
        // then Y_{k+1} = Y_k g and Z_{k+1} = g Z_k
        FormGParams fp;
        memset(&fp, 0, sizeof(fp));
        fp.r = Rb;
        fp.r2 = (d >= 2) ? R2b : nullptr;
        fp.r3 = R3b;
        fp.c2 = (float)taylor(2);
        fp.adaptive = cfg.degree_max > d;
        fp.dst = R2b;
        fp.stride = Lw.buf_stride;
        fp.n = n;
        fp.degree = d;
        fp.c0 = (float)taylor(0);
        fp.c1 = (float)taylor(1);
        fp.ctrl = ctrl;
        fp.sketch = next_sketch;
        PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g(fp, batch, q.s); }));
        u.nprob = 2;
        u.prob[0].a = {Yb[cur], n, Lw.buf_stride, nullptr, 0};
        u.prob[0].b = {R2b, n, Lw.buf_stride, nullptr, 0};
        u.prob[0].c = Yb[nxt];
        u.prob[0].ldc = n;
        u.prob[0].stride_c = Lw.buf_stride;
        u.prob[1].a = {R2b, n, Lw.buf_stride, nullptr, 0};
        u.prob[1].b = {Zb[cur], n, Lw.buf_stride, nullptr, 0};
        u.prob[1].c = Zb[nxt];
        u.prob[1].ldc = n;
        u.prob[1].stride_c = Lw.buf_stride;
      }
      // Y g and g Z are left whole: the full products keep Y_k = A Z_k^T as
      // computed, which keeps Z Y symmetric by structure; mirroring their
      // upper triangles would mix Y g with g Y and lose that (measurably
      // less accurate on ill-conditioned inputs)
      if (q.h->split_k) use_split(u, ws, Lw);
      set_vec(u);
      PMX_TRY(q.run(PMX_KC_GEMM_UPDATE, [&] { return launch_gemm_f32(u, false, false, ROLE_UPDATE, q.s); }));
      GemmParams r = gemm_base(q.h, n, n, n, batch);
      r.ctrl = ctrl;
      r.prob[0].a = {Zb[nxt], n, Lw.buf_stride, nullptr, 0};
      r.prob[0].b = {Yb[nxt], n, Lw.buf_stride, nullptr, 0};
      r.prob[0].c = Rb;
      r.prob[0].ldc = n;
      r.prob[0].stride_c = Lw.buf_stride;
      r.partials = partials;
      r.partial_stride = Lw.pstride;
      r.products = (d - 1) + 1 + (k > 0 ? 1 : 0) + 1;
      r.count_update = 1;
      r.cfg = cfg;
      // Z Y = Z A Z^T is symmetric by structure: its upper triangle is kept
      // and mirrored, so R and every g formed from it stay exactly symmetric
      r.sym = 1;
      if (q.h->split_k) use_split(r, ws, Lw);
      set_vec(r);
      PMX_TRY(q.run(PMX_KC_GEMM_RESID, [&] { return launch_gemm_f32(r, false, false, ROLE_RESID, q.s); }));
    }
  }
  RootFinishParams fp;
  fp.ybuf[0] = Yb[0];
  fp.ybuf[1] = Yb[1];
  fp.zbuf[0] = Zb[0];
  fp.zbuf[1] = Zb[1];
  fp.buf_stride = Lw.buf_stride;
  fp.x = X;
  fp.ldx = ldx;
  fp.x_stride = sx;
  fp.aux = XA;
  fp.ldaux = ldaux;
  fp.aux_stride = saux;
  fp.n = n;
  fp.expo_x = -1.0 / p;
  fp.expo_aux = 1.0 / p;
  fp.ctrl = ctrl;
  PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_root_finish(fp, batch, q.s); }));
  return PMX_OK;
}

pmx_status pmx_matfn_inv_root(pmx_handle h, const float* A, int n, int lda, int p, float* X,
                              int ldx, float* XA, int ldaux, const pmx_matfn_opts* opts,
                              pmx_matfn_info* info, void* ws, size_t ws_bytes, void* stream) {
  return pmx_matfn_inv_root_batched(h, A, n, lda, 0, p, X, ldx, 0, XA, ldaux, 0, 1, opts,
                                    info, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ polar
pmx_status pmx_matfn_polar_batched(pmx_handle h, const void* G, pmx_dtype dtype, int m, int n,
                                   int ldg, int64_t sg, void* U, int ldu, int64_t su,
                                   int batch, const pmx_matfn_opts* opts,
                                   pmx_matfn_info* info, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!h || !G || !U || m < 1 || n < 1 || m > kMaxN || n > kMaxN || batch < 1)
    return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  pmx_matfn_opts o;
  if (!resolve_opts(opts, &o)) return PMX_ERR_INVALID_VALUE;
  if (ldg < n || sg < 0 || (batch > 1 && sg != 0 && sg < (int64_t)(m - 1) * ldg + n))
    return PMX_ERR_INVALID_VALUE;
  if (!batch_layout_ok(m, n, ldu, su, batch)) return PMX_ERR_INVALID_VALUE;
  const bool bf = dtype == PMX_BF16;
  const int rows = std::max(m, n), cols = std::min(m, n);
  const bool tr = m < n;
  // d = 3 and the adaptive degree: fp32 only
  if (bf && std::max(o.degree, o.degree_max) == 3) return PMX_ERR_NOT_SUPPORTED;
  const bool pscale = o.scale_mode == PMX_SCALE_POWER;
  // the estimated scale is fp32 only: with X in bf16 it diverged on one of the
  // 32 Muon matrices (the top eigenvalues of R sit in the overshoot band near
  // xi = -0.25 from the first update on, where r(xi; alpha) at the upper alpha
  // bound expands perturbations about 1.8x per update, and bf16 rounding of X
  // is large enough to be driven past it)
  if (bf && pscale) return PMX_ERR_NOT_SUPPORTED;
  const IterLayout Lw = iter_layout(rows, cols, batch, o, polar_bufs(dtype, o), 0, sizeof(float));
  pmx_status st = check_ws(ws, ws_bytes, Lw.total);
  if (st != PMX_OK) return st;
  const Extent eg = extent_of(G, m, n, ldg, sg, batch, bf ? 2 : 4);
  const Extent eu = extent_of(U, m, n, ldu, su, batch, bf ? 2 : 4);
  Extent ew;
  ew.lo = (uintptr_t)ws;
  ew.hi = ew.lo + Lw.total;
  ew.valid = true;
  Extent ei = extent_of(info, 1, (int)sizeof(pmx_matfn_info), 0, sizeof(pmx_matfn_info), batch, 1);
  if (overlap(eg, eu) || overlap(ew, eg) || overlap(ew, eu) || overlap(ei, eg) ||
      overlap(ei, eu) || overlap(ei, ew))
    return PMX_ERR_ALIAS;

  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  Ctrl* ctrl = at<Ctrl>(ws, Lw.ctrl);
  double* partials = at<double>(ws, Lw.partials);
  float* Xb[2] = {at<float>(ws, Lw.bufs[0]), at<float>(ws, Lw.bufs[1])};
  float* Rb = at<float>(ws, Lw.bufs[2]);
  float* R2b = at<float>(ws, Lw.bufs[3]);
  float* R3b = (!bf && polar_bufs(dtype, o) == 5) ? at<float>(ws, Lw.bufs[4]) : nullptr;
  const IterCfg cfg = make_cfg(o, cols, info);
  const AlphaCoef coef = make_coef(o.degree);
  const int d = o.degree;
  const bool acc = o.accelerate != 0;
  const int64_t bs = Lw.buf_stride;

  if (!bf && rows <= kSmallMaxN && h->small_fused && std::max(o.degree, o.degree_max) <= 2 &&
      !pscale) {
    SmallPolarParams sp;
    memset(&sp, 0, sizeof(sp));
    sp.g = (const float*)G;
    sp.ldg = ldg;
    sp.g_stride = sg;
    sp.u = (float*)U;
    sp.ldu = ldu;
    sp.u_stride = su;
    sp.rows = rows;
    sp.cols = cols;
    sp.transpose = tr ? 1 : 0;
    sp.c0 = (float)taylor(0);
    sp.c1 = (float)taylor(1);
    sp.cfg = cfg;
    sp.coef = coef;
    PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_small_polar(sp, batch, q.s); }));
    return PMX_OK;
  }
  PMX_TRY(q.run(PMX_KC_OTHER, [&] {
    return launch_ctrl_reset(ctrl, info, batch, o.degree, at<uint32_t>(ws, Lw.skc),
                             kSplitMaxWorkers, q.s);
  }));
  PMX_TRY(q.run(PMX_KC_OTHER, [&] {
    return launch_fro_scale(G, bf, m, n, ldg, sg, batch, ctrl, partials, Lw.pstride, info, q.s);
  }));
  if (!bf) {
    PolarInitParams pi;
    pi.g = G;
    pi.ldg = ldg;
    pi.g_stride = sg;
    pi.x = Xb[0];
    pi.x_stride = bs;
    pi.rows = rows;
    pi.cols = cols;
    pi.transpose = tr ? 1 : 0;
    pi.ctrl = ctrl;
    pi.sketch = make_sketch(Lw, ws, cfg, cols, 0, 0, acc);
    PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_polar_init(pi, false, batch, q.s); }));
    auto residual = [&](float* Xc, int products, int count) {
      GemmParams r = gemm_base(q.h, cols, cols, rows, batch);
      r.ctrl = ctrl;
      r.prob[0].a = {Xc, cols, bs, nullptr, 0};
      r.prob[0].b = {Xc, cols, bs, nullptr, 0};
      r.prob[0].c = Rb;
      r.prob[0].ldc = cols;
      r.prob[0].stride_c = bs;
      r.partials = partials;
      r.partial_stride = Lw.pstride;
      r.products = products;
      r.count_update = count;
      r.cfg = cfg;
      r.sym = 1;  // X^T X: upper-triangle tiles, mirrored
      if (q.h->split_k) use_split(r, ws, Lw);
      set_vec(r);
      return q.run(PMX_KC_GEMM_RESID, [&] { return launch_gemm_f32(r, true, false, ROLE_RESID, q.s); });
    };
    PMX_TRY(residual(Xb[0], 1, 0));
    if (pscale) PMX_TRY(enqueue_polar_scale(q, ws, Lw, cfg, Rb, nullptr, cols, batch));
    Poller poll(q, ctrl, batch);
    for (int k = 0; k < o.max_iter; ++k) {
      bool stop = false;
      PMX_TRY(poll.step(k, &stop));
      if (stop) break;
      PMX_TRY(enqueue_power_and_alpha(q, ws, Lw, o, cfg, coef, cols, batch, Rb, R2b, R3b));
      const int cur = k & 1, nxt = cur ^ 1;
      GemmParams u = gemm_base(q.h, rows, cols, cols, batch);
      u.ctrl = ctrl;
      u.degree = d;
      u.c0 = (float)taylor(0);
      u.c1 = (float)taylor(1);
      u.prob[0].a = {Xb[cur], cols, bs, nullptr, 0};
      u.prob[0].b = {Rb, cols, bs, R2b, 1};
      {
        // g written once in place of R^2 (read by the Krylov passes already),
        // with the sketch of the next update
        FormGParams fp;
        memset(&fp, 0, sizeof(fp));
        fp.r = Rb;
        fp.r2 = (d >= 2) ? R2b : nullptr;
        fp.r3 = R3b;
        fp.c2 = (float)taylor(2);
        fp.adaptive = cfg.degree_max > d;
        fp.dst = R2b;
        fp.stride = bs;
        fp.n = cols;
        fp.degree = d;
        fp.c0 = (float)taylor(0);
        fp.c1 = (float)taylor(1);
        fp.ctrl = ctrl;
        fp.first_scale = pscale && k == 0;
        fp.sketch = make_sketch(Lw, ws, cfg, cols, k + 1, 0, acc && k + 1 < o.max_iter);
        PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g(fp, batch, q.s); }));
        u.prob[0].b = {R2b, cols, bs, nullptr, 0};
      }
      u.prob[0].c = Xb[nxt];
      u.prob[0].ldc = cols;
      u.prob[0].stride_c = bs;
      if (q.h->split_k) use_split(u, ws, Lw);
      set_vec(u);
      PMX_TRY(q.run(PMX_KC_GEMM_UPDATE, [&] { return launch_gemm_f32(u, false, false, ROLE_UPDATE, q.s); }));
      PMX_TRY(residual(Xb[nxt], (d - 1) + 1 + 1, 1));
    }
  } else {
    // bf16: every product is k-contiguous x k-contiguous (pmx_gemm_bf16.hip).
    // X and X^T are kept in bf16 (the update writes both); R is symmetric, so
    // its bf16 copy Rh (written by the residual) is both operands of R^2, and
    // the bf16 polynomial g is the update's second operand as it stands.
    float* Xt[2] = {at<float>(ws, Lw.bufs[4]), at<float>(ws, Lw.bufs[5])};
    float* Rh = at<float>(ws, Lw.bufs[6]);  // R in bf16
    float* Gh = at<float>(ws, Lw.bufs[7]);  // g in bf16
    const bool vec = (cols % 8 == 0) && (rows % 8 == 0) && (bs % 8 == 0);
    // Where the residual's tiles are whole 256 x 256 x 64 ones (and the
    // large tile is the launcher's choice), I - X^T X reads the row-major
    // iterate itself through the LDS transpose reads, and no transposed copy
    // of X is written (by the update or the set-up).
    const bool mn = !tr && q.h->bf16_mn && vec && cols % 256 == 0 && rows % 64 == 0 &&
                    (int64_t)(cols / 256) * (cols / 256) * batch >= q.h->num_cu &&
                    q.h->bf16_cfg < 0 && !q.h->bf16_sym;
    auto residual = [&](int it, int products, int count) {
      GemmParams r = bf16_base(q.h, cols, cols, rows, batch);
      r.ctrl = ctrl;
      if (mn) {
        r.prob[0].a = {Xb[it], cols, bs, nullptr, 0};
        r.prob[0].b = {Xb[it], cols, bs, nullptr, 0};
        r.mn = 1;
      } else {
        r.prob[0].a = {Xt[it], rows, bs, nullptr, 0};
        r.prob[0].b = {Xt[it], rows, bs, nullptr, 0};
      }
      r.prob[0].c = Rb;
      r.prob[0].ldc = cols;
      r.prob[0].stride_c = bs;
      r.prob[1].c = (d == 2) ? Rh : nullptr;  // bf16 copy for the power R^2
      r.prob[1].ldc = cols;
      r.prob[1].stride_c = bs;
      r.partials = partials;
      r.partial_stride = Lw.pstride;
      r.products = products;
      r.count_update = count;
      r.cfg = cfg;
      r.vec = vec ? 1 : 0;
      r.sym = q.h->bf16_sym;  // X^T X: upper-triangle tiles, mirrored
      r.sym_small = q.h->bf16_sym_small;
      return q.run(PMX_KC_GEMM_RESID, [&] { return launch_gemm_bf16(r, ROLE_RESID, q.s); });
    };
    {
      // X_0 = G / ||G||_F and its transpose, in one pass over G
      XposeParams x;
      memset(&x, 0, sizeof(x));
      x.a = G;
      x.a_bf16 = 1;
      x.lda = ldg;
      x.sa = sg;
      x.rows = m;
      x.cols = n;
      x.scale_inv_c = 1;
      x.ctrl = ctrl;
      x.out_n = (uint16_t*)(tr ? Xt[0] : Xb[0]);
      x.ldn = n;
      x.sn = bs;
      x.out_t = mn ? nullptr : (uint16_t*)(tr ? Xb[0] : Xt[0]);
      x.ldt = m;
      x.st = bs;
      x.sketch = make_sketch(Lw, ws, cfg, cols, 0, 0, acc);
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_xpose(x, batch, q.s); }));
    }
    PMX_TRY(residual(0, 1, 0));
    Poller poll(q, ctrl, batch);
    for (int k = 0; k < o.max_iter; ++k) {
      bool stop = false;
      PMX_TRY(poll.step(k, &stop));
      if (stop) break;
      if (d == 2) {
        GemmParams g = bf16_base(q.h, cols, cols, cols, batch);
        g.ctrl = ctrl;
        g.prob[0].a = {Rh, cols, bs, nullptr, 0};
        g.prob[0].b = {Rh, cols, bs, nullptr, 0};
        g.prob[0].c = R2b;
        g.prob[0].ldc = cols;
        g.prob[0].stride_c = bs;
        g.vec = vec ? 1 : 0;
        g.sym = q.h->bf16_sym;  // R^2 with R exactly symmetric: triangle, mirrored
        g.sym_small = q.h->bf16_sym_small;
        PMX_TRY(q.run(PMX_KC_GEMM_POWER, [&] { return launch_gemm_bf16(g, ROLE_POWER, q.s); }));
      }
      PMX_TRY(enqueue_power_and_alpha(q, ws, Lw, o, cfg, coef, cols, batch, Rb, R2b, nullptr, false));
      FormGParams fg;
      memset(&fg, 0, sizeof(fg));
      fg.r = Rb;
      fg.r2 = (d == 2) ? R2b : nullptr;
      fg.dst = Gh;
      fg.dst_bf16 = 1;
      fg.stride = bs;
      fg.n = cols;
      fg.degree = d;
      fg.c0 = (float)taylor(0);
      fg.c1 = (float)taylor(1);
      fg.ctrl = ctrl;
      fg.sketch = make_sketch(Lw, ws, cfg, cols, k + 1, 0, acc && k + 1 < o.max_iter);
      PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_form_g(fg, batch, q.s); }));
      const int cur = k & 1, nxt = cur ^ 1;
      GemmParams u = bf16_base(q.h, rows, cols, cols, batch);
      u.ctrl = ctrl;
      u.nprob = 1;
      u.prob[0].a = {Xb[cur], cols, bs, nullptr, 0};
      u.prob[0].b = {Gh, cols, bs, nullptr, 0};
      u.prob[0].c = Xb[nxt];
      u.prob[0].ldc = cols;
      u.prob[0].stride_c = bs;
      u.prob[1].c = mn ? nullptr : Xt[nxt];  // transposed copy of the new iterate
      u.prob[1].ldc = rows;
      u.prob[1].stride_c = bs;
      u.vec = vec ? 1 : 0;
      PMX_TRY(q.run(PMX_KC_GEMM_UPDATE, [&] { return launch_gemm_bf16(u, ROLE_UPDATE, q.s); }));
      PMX_TRY(residual(nxt, (d - 1) + 1 + 1, 1));
    }
  }
  PolarFinishParams fp;
  memset(&fp, 0, sizeof(fp));
  if (bf && tr) {
    // U = X^T is the kept transposed iterate: a straight copy
    fp.xbuf[0] = at<float>(ws, Lw.bufs[4]);
    fp.xbuf[1] = at<float>(ws, Lw.bufs[5]);
    fp.rows = cols;
    fp.cols = rows;
    fp.transpose = 0;
  } else {
    fp.xbuf[0] = Xb[0];
    fp.xbuf[1] = Xb[1];
    fp.rows = rows;
    fp.cols = cols;
    fp.transpose = tr ? 1 : 0;
  }
  fp.buf_stride = bs;
  fp.u = U;
  fp.ldu = ldu;
  fp.u_stride = su;
  fp.ctrl = ctrl;
  PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_polar_finish(fp, bf, batch, q.s); }));
  return PMX_OK;
}

// ------------------------------------------------------------------ variable-size polar
// The plan of a variable-size polar call: the descriptor table (every
// block, in order; the fused kernel skips the large ones), then the indices
// of the blocks above kSmallMaxN grouped by shape, then one scratch area
// reused by every shape group in turn: the packed fp32 input and output, the
// group's info records and the batched polar factor's workspace.
struct VarGroup {
  int m, n, first, count;  // shape; idx[first, first + count)
};
struct VarPlan {
  std::vector<int32_t> idx;
  std::vector<VarGroup> groups;
  size_t table = 0, idx_off = 0, scratch = 0, total = 0;
  bool small = false;  // any block for the fused kernel
};

static size_t var_group_bytes(const VarGroup& g, const pmx_matfn_opts& o) {
  const size_t mat = align_up(sizeof(float) * (size_t)g.m * g.n * g.count);
  return 2 * mat + align_up(sizeof(pmx_matfn_info) * (size_t)g.count) +
         polar_ws(g.m, g.n, g.count, o, PMX_F32);
}

static bool var_plan(const pmx_polar_block* blocks, int count, const pmx_matfn_opts& o,
                     VarPlan* P) {
  std::vector<std::pair<std::pair<int, int>, int32_t>> big;
  for (int i = 0; i < count; ++i) {
    const pmx_polar_block& bl = blocks[i];
    if (bl.m < 1 || bl.n < 1 || bl.m > PMX_VARBATCH_MAX_SIDE || bl.n > PMX_VARBATCH_MAX_SIDE)
      return false;
    if (bl.m > kSmallMaxN || bl.n > kSmallMaxN) big.push_back({{bl.m, bl.n}, (int32_t)i});
    else P->small = true;
  }
  std::stable_sort(big.begin(), big.end(),
                   [](const auto& x, const auto& y) { return x.first < y.first; });
  for (size_t i = 0; i < big.size(); ++i) {
    if (i == 0 || big[i].first != big[i - 1].first)
      P->groups.push_back({big[i].first.first, big[i].first.second, (int)i, 0});
    P->groups.back().count += 1;
    P->idx.push_back(big[i].second);
  }
  P->table = align_up(sizeof(pmx_polar_block) * (size_t)count);
  P->idx_off = P->table;
  P->scratch = P->idx_off + (P->idx.empty() ? 0 : align_up(sizeof(int32_t) * P->idx.size()));
  size_t g = 0;
  for (const VarGroup& gr : P->groups) g = std::max(g, var_group_bytes(gr, o));
  P->total = P->scratch + g;
  return true;
}

pmx_status pmx_polar_varbatch_workspace_size(const pmx_polar_block* blocks, int count,
                                             pmx_dtype dtype, const pmx_matfn_opts* opts,
                                             size_t* bytes) {
  if (!blocks || count < 1 || !bytes) return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  pmx_matfn_opts o;
  if (!resolve_opts(opts, &o)) return PMX_ERR_INVALID_VALUE;
  VarPlan P;
  if (!var_plan(blocks, count, o, &P)) return PMX_ERR_INVALID_VALUE;
  *bytes = P.total;
  return PMX_OK;
}

pmx_status pmx_matfn_polar_varbatch(pmx_handle h, const pmx_polar_block* blocks, int count,
                                    pmx_dtype dtype, const pmx_matfn_opts* opts,
                                    pmx_matfn_info* info, void* ws, size_t ws_bytes,
                                    void* stream) {
  if (!h || !blocks || count < 1) return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  pmx_matfn_opts o;
  if (!resolve_opts(opts, &o)) return PMX_ERR_INVALID_VALUE;
  if (std::max(o.degree, o.degree_max) > 2) return PMX_ERR_NOT_SUPPORTED;
  if (o.scale_mode != PMX_SCALE_FROBENIUS) return PMX_ERR_NOT_SUPPORTED;
  const int esz = dtype == PMX_BF16 ? 2 : 4;
  VarPlan P;
  if (!var_plan(blocks, count, o, &P)) return PMX_ERR_INVALID_VALUE;
  const size_t need = P.total;
  pmx_status st = check_ws(ws, ws_bytes, need);
  if (st != PMX_OK) return st;
  Extent ew;
  ew.lo = (uintptr_t)ws;
  ew.hi = ew.lo + need;
  ew.valid = true;
  const Extent ei =
      extent_of(info, 1, (int)sizeof(pmx_matfn_info), 0, sizeof(pmx_matfn_info), count, 1);
  if (overlap(ei, ew)) return PMX_ERR_ALIAS;
  for (int i = 0; i < count; ++i) {
    const pmx_polar_block& bl = blocks[i];
    if (!bl.g || !bl.u || bl.ldg < bl.n || bl.ldu < bl.n) return PMX_ERR_INVALID_VALUE;
    const Extent eg = extent_of(bl.g, bl.m, bl.n, bl.ldg, 0, 1, esz);
    const Extent eu = extent_of(bl.u, bl.m, bl.n, bl.ldu, 0, 1, esz);
    if (overlap(eg, eu) || overlap(eu, ew) || overlap(eg, ew) || overlap(eu, ei))
      return PMX_ERR_ALIAS;
  }
  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  // the descriptor copy below reads the caller's host array, which may be
  // gone when a captured graph is replayed: refuse capture
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(q.s, &cs) != hipSuccess) return PMX_ERR_HIP;
  if (cs != hipStreamCaptureStatusNone) return PMX_ERR_NOT_SUPPORTED;
  // descriptors and the grouped indices to the device on the call's stream,
  // staged from host memory before the copy calls return
  if (hipMemcpyAsync(ws, blocks, sizeof(pmx_polar_block) * (size_t)count, hipMemcpyHostToDevice,
                     q.s) != hipSuccess)
    return PMX_ERR_HIP;
  if (!P.idx.empty() && hipMemcpyAsync(at<void>(ws, P.idx_off), P.idx.data(),
                                       sizeof(int32_t) * P.idx.size(), hipMemcpyHostToDevice,
                                       q.s) != hipSuccess)
    return PMX_ERR_HIP;
  const pmx_polar_block* table = reinterpret_cast<const pmx_polar_block*>(ws);
  if (P.small) {
    SmallPolarParams sp;
    memset(&sp, 0, sizeof(sp));
    sp.blocks = table;
    sp.bf16 = dtype == PMX_BF16;
    sp.c0 = (float)taylor(0);
    sp.c1 = (float)taylor(1);
    sp.cfg = make_cfg(o, PMX_VARBATCH_MAX_DIM, info);
    sp.coef = make_coef(o.degree);
    PMX_TRY(q.run(PMX_KC_OTHER, [&] { return launch_small_polar(sp, count, q.s); }));
  }
  // the large blocks, one shape group at a time through the batched fp32 path
  const int32_t* idx = at<int32_t>(ws, P.idx_off);
  for (const VarGroup& g : P.groups) {
    const size_t mat = align_up(sizeof(float) * (size_t)g.m * g.n * g.count);
    float* in = at<float>(ws, P.scratch);
    float* out = at<float>(ws, P.scratch + mat);
    pmx_matfn_info* ginfo = at<pmx_matfn_info>(ws, P.scratch + 2 * mat);
    const size_t woff = P.scratch + 2 * mat + align_up(sizeof(pmx_matfn_info) * (size_t)g.count);
    const size_t wbytes = polar_ws(g.m, g.n, g.count, o, PMX_F32);
    const int32_t* gi = idx + g.first;
    PMX_TRY(q.run(PMX_KC_OTHER, [&] {
      return launch_varbatch_gather(table, gi, dtype == PMX_BF16, in, g.m, g.n, g.count, q.s);
    }));
    const int64_t plane = (int64_t)g.m * g.n;
    st = pmx_matfn_polar_batched(h, in, PMX_F32, g.m, g.n, g.n, plane, out, g.n, plane, g.count,
                                 &o, info ? ginfo : nullptr, at<void>(ws, woff), wbytes, stream);
    if (st != PMX_OK) return st;
    PMX_TRY(q.run(PMX_KC_OTHER, [&] {
      return launch_varbatch_scatter(table, gi, dtype == PMX_BF16, out, g.m, g.n, g.count,
                                     info ? ginfo : nullptr, info, q.s);
    }));
  }
  return PMX_OK;
}

pmx_status pmx_matfn_polar(pmx_handle h, const void* G, pmx_dtype dtype, int m, int n, int ldg,
                           void* U, int ldu, const pmx_matfn_opts* opts, pmx_matfn_info* info,
                           void* ws, size_t ws_bytes, void* stream) {
  return pmx_matfn_polar_batched(h, G, dtype, m, n, ldg, 0, U, ldu, 0, 1, opts, info, ws,
                                 ws_bytes, stream);
}

// ------------------------------------------------------------------ apply
// The preconditioned step with the workspace `ws` (caller's, or the
// library's scratch for the allocation-free entry point).
static pmx_status precond_apply_impl(pmx_handle h, const float* Linv, int ldl, int64_t sl,
                                     const void* G, pmx_dtype dtype, int m, int n, int ldg,
                                     int64_t sg, const float* Rinv, int ldr, int64_t sr,
                                     void* P, int ldp, int64_t sp, int batch, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!h || !Linv || !G || !Rinv || !P || m < 1 || n < 1 || m > kMaxN || n > kMaxN ||
      batch < 1)
    return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  if (ldl < m || ldg < n || ldr < n || sl < 0 || sg < 0 || sr < 0)
    return PMX_ERR_INVALID_VALUE;
  if (!batch_layout_ok(m, n, ldp, sp, batch)) return PMX_ERR_INVALID_VALUE;
  const bool bf = dtype == PMX_BF16;
  const size_t need = apply_ws(m, n, batch, dtype);
  pmx_status st = check_ws(ws, ws_bytes, need);
  if (st != PMX_OK) return st;
  const Extent ep = extent_of(P, m, n, ldp, sp, batch, bf ? 2 : 4);
  const Extent el = extent_of(Linv, m, m, ldl, sl, batch, 4);
  const Extent eg = extent_of(G, m, n, ldg, sg, batch, bf ? 2 : 4);
  const Extent er = extent_of(Rinv, n, n, ldr, sr, batch, 4);
  Extent ew;
  ew.lo = (uintptr_t)ws;
  ew.hi = ew.lo + need;
  ew.valid = true;
  if (overlap(ep, el) || overlap(ep, eg) || overlap(ep, er) || overlap(ew, ep) ||
      overlap(ew, el) || overlap(ew, eg) || overlap(ew, er))
    return PMX_ERR_ALIAS;
  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  const size_t one = align_up(sizeof(float) * (size_t)m * n * batch);
  float* T = (float*)ws;
  const int64_t st_t = (int64_t)m * n;
  const float* gf = (const float*)G;
  if (bf) {
    float* Gw = at<float>(ws, one);
    PMX_TRY(q.run(PMX_KC_OTHER, [&] {
      return launch_convert(G, true, ldg, sg, Gw, false, n, st_t, m, n, batch, q.s);
    }));
    gf = Gw;
    ldg = n;
    sg = st_t;
  }
  GemmParams a = gemm_base(q.h, m, n, m, batch);
  a.prob[0].a = {Linv, ldl, sl, nullptr, 0};
  a.prob[0].b = {gf, ldg, sg, nullptr, 0};
  a.prob[0].c = T;
  a.prob[0].ldc = n;
  a.prob[0].stride_c = st_t;
  set_vec(a);
  PMX_TRY(q.run(PMX_KC_GEMM_APPLY, [&] { return launch_gemm_f32(a, false, false, ROLE_APPLY, q.s); }));
  GemmParams b = gemm_base(q.h, m, n, n, batch);
  float* Pw = bf ? at<float>(ws, 2 * one) : (float*)P;
  b.prob[0].a = {T, n, st_t, nullptr, 0};
  b.prob[0].b = {Rinv, ldr, sr, nullptr, 0};
  b.prob[0].c = Pw;
  b.prob[0].ldc = bf ? n : ldp;
  b.prob[0].stride_c = bf ? st_t : sp;
  set_vec(b);
  PMX_TRY(q.run(PMX_KC_GEMM_APPLY, [&] { return launch_gemm_f32(b, false, false, ROLE_APPLY, q.s); }));
  if (bf) {
    PMX_TRY(q.run(PMX_KC_OTHER, [&] {
      return launch_convert(Pw, false, n, st_t, P, true, ldp, sp, m, n, batch, q.s);
    }));
  }
  return PMX_OK;
}

pmx_status pmx_precond_apply_batched(pmx_handle h, const float* Linv, int ldl, int64_t sl,
                                     const void* G, pmx_dtype dtype, int m, int n, int ldg,
                                     int64_t sg, const float* Rinv, int ldr, int64_t sr,
                                     void* P, int ldp, int64_t sp, int batch, void* ws,
                                     size_t ws_bytes, void* stream) {
  return precond_apply_impl(h, Linv, ldl, sl, G, dtype, m, n, ldg, sg, Rinv, ldr, sr, P, ldp, sp,
                            batch, ws, ws_bytes, stream);
}

pmx_status pmx_precond_apply_noalloc(pmx_handle h, const float* Linv, int ldl, int64_t sl,
                                     const void* G, pmx_dtype dtype, int m, int n, int ldg,
                                     int64_t sg, const float* Rinv, int ldr, int64_t sr,
                                     void* P, int ldp, int64_t sp, int batch, void* stream) {
  if (!h || m < 1 || n < 1 || m > kMaxN || n > kMaxN || batch < 1) return PMX_ERR_INVALID_VALUE;
  if (dtype != PMX_F32 && dtype != PMX_BF16) return PMX_ERR_INVALID_VALUE;
  const size_t need = apply_ws(m, n, batch, dtype);
  if (need > kScratchBytes) return PMX_ERR_WORKSPACE;
  void* ws = scratch_of(h->device);
  if (!ws) return PMX_ERR_HIP;
  return precond_apply_impl(h, Linv, ldl, sl, G, dtype, m, n, ldg, sg, Rinv, ldr, sr, P, ldp, sp,
                            batch, ws, kScratchBytes, stream);
}

pmx_status pmx_precond_apply(pmx_handle h, const float* Linv, int ldl, const void* G,
                             pmx_dtype dtype, int m, int n, int ldg, const float* Rinv, int ldr,
                             void* P, int ldp, void* ws, size_t ws_bytes, void* stream) {
  return pmx_precond_apply_batched(h, Linv, ldl, 0, G, dtype, m, n, ldg, 0, Rinv, ldr, 0, P,
                                   ldp, 0, 1, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ sketch
pmx_status pmx_sketch_gaussian(pmx_handle h, uint64_t seed, int matrix, int stage, int k, int n,
                               int p, float* S, int lds, uint32_t* words, void* stream) {
  if (!h || !S || n <= 0 || n > kMaxN || p < 1 || p > PMX_MAX_SKETCH || lds < p || matrix < 0 ||
      stage < 0 || k < 0)
    return PMX_ERR_INVALID_VALUE;
  if (words) {
    const Extent es = extent_of(S, n, p, lds, 0, 1, sizeof(float));
    const Extent ew = extent_of(words, n, p, p, 0, 1, sizeof(uint32_t));
    if (overlap(es, ew)) return PMX_ERR_ALIAS;
  }
  DeviceGuard dg(h->device);
  if (!dg.ok) return PMX_ERR_HIP;
  Enq q{h, (hipStream_t)stream};
  return from_hip(q.run(PMX_KC_OTHER, [&] {
    return launch_sketch_export(seed, matrix, stage, k, n, p, S, lds, words, q.s);
  }));
}

}  // extern "C"
