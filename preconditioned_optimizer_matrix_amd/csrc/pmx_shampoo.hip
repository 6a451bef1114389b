// A whole Shampoo optimizer step over the layers of a model ([Shampoo blog]
// sections 2.3, 3.2, 5.1, 5.2, 5.3): block-diagonal statistics, roots every
// `root_every` steps, momentum and the weight update, with blocks of equal
// shape batched through the library's own entry points.
//
// The plan (host) cuts every layer's matrix view into blocks of at most
// block x block and groups equal shapes.  Device memory:
//   state     -- per group L, R, L^{-1/4}, R^{-1/4} (square, batched), M
//                (rows x cols, batched); the block and layer tables; the
//                running sum of ||G||_F^2 and the current step size.
//   workspace -- the layer pointers of the step, the gathered gradient
//                blocks and their preconditioned steps (one buffer each, laid
//                out like M), the norm partials, and the workspace of the
//                library calls (the largest any group needs).
// Per step: one gather launch (gradient blocks into the batch buffers, with
// the squared norm), the norm/step-size launch (adaptive_lr), per group the
// statistics, roots (t % root_every == 0) and apply calls, and one update
// launch (M <- momentum M + P, W -= eta M through the layers' index maps).
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "pmx_kernels.h"

namespace pmx {
namespace {

constexpr size_t kAlignS = 256;
size_t up(size_t x) { return (x + kAlignS - 1) / kAlignS * kAlignS; }

// Matrix view of a layer: rows x cols; a c_out x c_in x kh x kw kernel is the
// (c_out kh kw) x c_in matrix K'[(o kh + y) kw + x][i] = K[o][i][y][x].
struct LayerDev {
  int dims;
  int cin, kh, kw;  // dims == 4
  int64_t rows, cols;
};

struct BlockDev {
  int layer, row0, col0, rows, cols;
  int pad;
  int64_t off;  // element offset of the block in the batch buffers (and M)
};

__device__ __forceinline__ int64_t layer_offset(const LayerDev& L, int64_t r, int64_t c) {
  if (L.dims == 2) return r * L.cols + c;
  const int64_t hw = (int64_t)L.kh * L.kw;
  const int64_t o = r / hw, rem = r - o * hw;  // rem = y kw + x
  return (o * L.cin + c) * hw + rem;
}

constexpr int ST = 256;  // threads per block of the plan kernels
constexpr int RT = 16;   // block rows per workgroup

// Gradient blocks into the batch buffer (block b at off_b, row-major rows x
// cols), with the workgroup's share of sum ||G||^2 (fp64) in part[].
__global__ __launch_bounds__(ST) void gather_kernel(const BlockDev* __restrict__ blocks,
                                                    const LayerDev* __restrict__ layers,
                                                    const float* const* __restrict__ G,
                                                    float* __restrict__ out,
                                                    double* __restrict__ part) {
  const BlockDev bk = blocks[blockIdx.y];
  const LayerDev L = layers[bk.layer];
  const float* g = G[bk.layer];
  double acc = 0.0;
  const int r0 = blockIdx.x * RT;
  for (int r = r0; r < r0 + RT && r < bk.rows; ++r)
    for (int c = threadIdx.x; c < bk.cols; c += ST) {
      const float v = g[layer_offset(L, bk.row0 + r, bk.col0 + c)];
      out[bk.off + (int64_t)r * bk.cols + c] = v;
      acc += (double)v * (double)v;
    }
  __shared__ double red[ST / 64];
  const double t = block_sum<ST / 64>(acc, red);
  if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
}

// running += sum of the partials (fixed order); eta = lr / sqrt(1 + running).
__global__ __launch_bounds__(ST) void step_size_kernel(const double* __restrict__ part,
                                                       int64_t nparts, double* running,
                                                       float* eta, float lr) {
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < nparts; i += ST) acc += part[i];
  __shared__ double red[ST / 64];
  const double t = block_sum<ST / 64>(acc, red);
  if (threadIdx.x == 0) {
    const double run = *running + t;
    *running = run;
    *eta = (float)(lr / sqrt(1.0 + run));
  }
}

// M <- momentum M + P (M = P when momentum is 0), W -= eta M through the
// layer maps; eta from *eta_dev when set, else eta.
__global__ __launch_bounds__(ST) void update_kernel(const BlockDev* __restrict__ blocks,
                                                    const LayerDev* __restrict__ layers,
                                                    float* const* __restrict__ W,
                                                    const float* __restrict__ P,
                                                    float* __restrict__ M, float momentum,
                                                    const float* eta_dev, float eta) {
  const BlockDev bk = blocks[blockIdx.y];
  const LayerDev L = layers[bk.layer];
  float* w = W[bk.layer];
  const float e = eta_dev ? *eta_dev : eta;
  const int r0 = blockIdx.x * RT;
  for (int r = r0; r < r0 + RT && r < bk.rows; ++r)
    for (int c = threadIdx.x; c < bk.cols; c += ST) {
      const int64_t i = bk.off + (int64_t)r * bk.cols + c;
      const float m = momentum != 0.f ? momentum * M[i] + P[i] : P[i];
      M[i] = m;
      w[layer_offset(L, bk.row0 + r, bk.col0 + c)] -= e * m;
    }
}

// n x n matrices of a batch set to value * I, or all of x zeroed (diag < 0).
__global__ __launch_bounds__(ST) void fill_kernel(float* __restrict__ x, int64_t count,
                                                  int64_t n, float value) {
  for (int64_t i = (int64_t)blockIdx.x * ST + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * ST) {
    float v = 0.f;
    if (n > 0) {
      const int64_t e = i % (n * n);
      if (e / n == e % n) v = value;
    }
    x[i] = v;
  }
}

__global__ void zero_scalars_kernel(double* running, float* eta, float lr) {
  if (threadIdx.x == 0) {
    *running = 0.0;
    *eta = lr;
  }
}

struct Group {
  int rows, cols, count;
  int64_t first;       // index of the group's first block (blocks are group-ordered)
  size_t L, R, Li, Ri;  // state offsets (bytes)
  int64_t off;         // element offset of the group in the batch buffers and M
};

}  // namespace
}  // namespace pmx

using namespace pmx;

struct pmx_shampoo_plan_t {
  pmx_handle h;
  int device;
  pmx_shampoo_config cfg;
  std::vector<LayerDev> layers;
  std::vector<BlockDev> blocks;
  std::vector<Group> groups;
  int64_t elems;  // elements of all blocks
  int64_t tiles;  // workgroups of the gather / update launches (norm partials)
  int max_rows;   // largest block side, for the launch grids
  // state layout
  size_t s_M, s_blocks, s_layers, s_running, s_eta, state_bytes;
  // workspace layout
  size_t w_ptrs, w_G, w_P, w_part, w_lib, lib_bytes, ws_bytes;
};

namespace {

struct Guard {
  int prev = -1;
  bool ok = true;
  explicit Guard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) {
      ok = false;
      return;
    }
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~Guard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// True while `s` is being captured into a graph (or its status is unknown).
bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone;
}


template <typename T>
T* at_(void* base, size_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

pmx_status pmx_shampoo_config_default(pmx_shampoo_config* c) {
  if (!c) return PMX_ERR_INVALID_VALUE;
  memset(c, 0, sizeof(*c));
  c->struct_version = 1;
  c->block = 1024;
  c->root_every = 1;
  c->adaptive_lr = 0;
  c->beta = 0.95f;
  c->eps = 1e-6f;
  c->lr = 1e-3f;
  c->momentum = 0.f;
  return pmx_matfn_opts_default(&c->root_opts);
}

pmx_status pmx_shampoo_plan_create(pmx_handle h, const pmx_shampoo_config* cfg,
                                   const pmx_layer* layers, int nlayers,
                                   pmx_shampoo_plan* out) {
  if (!out) return PMX_ERR_INVALID_VALUE;
  *out = nullptr;
  if (!h || !cfg || !layers || nlayers < 1) return PMX_ERR_INVALID_VALUE;
  if (cfg->struct_version != 1 || cfg->block < 1 || cfg->block > 32768 || cfg->root_every < 1 ||
      (cfg->adaptive_lr != 0 && cfg->adaptive_lr != 1) || !(cfg->beta >= 0.f && cfg->beta <= 1.f) ||
      !(cfg->eps >= 0.f) || !isfinite(cfg->lr) || !isfinite(cfg->momentum))
    return PMX_ERR_INVALID_VALUE;
  // the root options are checked by a workspace query of a 1 x 1 root
  {
    size_t b = 0;
    if (pmx_workspace_size(nullptr, PMX_OP_INV_ROOT, 1, 1, 1, PMX_F32, &cfg->root_opts, &b) !=
        PMX_OK)
      return PMX_ERR_INVALID_VALUE;
  }
  pmx_shampoo_plan_t* P = new (std::nothrow) pmx_shampoo_plan_t;
  if (!P) return PMX_ERR_HIP;
  P->h = h;
  P->device = handle_device(h);
  P->cfg = *cfg;
  for (int l = 0; l < nlayers; ++l) {
    const pmx_layer& ly = layers[l];
    LayerDev d;
    memset(&d, 0, sizeof(d));
    d.dims = ly.dims;
    if (ly.dims == 2) {
      d.rows = ly.shape[0];
      d.cols = ly.shape[1];
    } else if (ly.dims == 4) {
      d.cin = ly.shape[1];
      d.kh = ly.shape[2];
      d.kw = ly.shape[3];
      d.rows = (int64_t)ly.shape[0] * ly.shape[2] * ly.shape[3];
      d.cols = ly.shape[1];
    } else {
      delete P;
      return PMX_ERR_INVALID_VALUE;
    }
    for (int k = 0; k < ly.dims; ++k)
      if (ly.shape[k] < 1) {
        delete P;
        return PMX_ERR_INVALID_VALUE;
      }
    if (d.rows > (int64_t)1 << 30 || d.cols > (int64_t)1 << 30) {
      delete P;
      return PMX_ERR_INVALID_VALUE;
    }
    P->layers.push_back(d);
  }
  // blocks: rows and columns cut into pieces of at most `block`
  struct Raw {
    int layer, row0, col0, rows, cols;
  };
  std::vector<Raw> raw;
  const int B = cfg->block;
  for (int l = 0; l < nlayers; ++l) {
    const LayerDev& d = P->layers[l];
    for (int64_t r = 0; r < d.rows; r += B)
      for (int64_t c = 0; c < d.cols; c += B)
        raw.push_back({l, (int)r, (int)c, (int)std::min<int64_t>(B, d.rows - r),
                       (int)std::min<int64_t>(B, d.cols - c)});
  }
  if (raw.size() > 65535) {  // one grid row per block in the gather / update launches
    delete P;
    return PMX_ERR_INVALID_VALUE;
  }
  // groups of equal shape, in order of first appearance; blocks group-ordered
  std::vector<std::pair<int, int>> shapes;
  for (const Raw& b : raw) {
    const std::pair<int, int> s{b.rows, b.cols};
    if (std::find(shapes.begin(), shapes.end(), s) == shapes.end()) shapes.push_back(s);
  }
  size_t soff = 0;
  int64_t eoff = 0;
  P->max_rows = 0;
  for (const auto& s : shapes) {
    Group g;
    g.rows = s.first;
    g.cols = s.second;
    g.count = 0;
    g.first = (int64_t)P->blocks.size();
    g.off = eoff;
    for (const Raw& b : raw)
      if (b.rows == g.rows && b.cols == g.cols) {
        BlockDev bd;
        bd.layer = b.layer;
        bd.row0 = b.row0;
        bd.col0 = b.col0;
        bd.rows = b.rows;
        bd.cols = b.cols;
        bd.pad = 0;
        bd.off = eoff;
        eoff += (int64_t)b.rows * b.cols;
        P->blocks.push_back(bd);
        ++g.count;
      }
    const size_t sq_r = sizeof(float) * (size_t)g.rows * g.rows * g.count;
    const size_t sq_c = sizeof(float) * (size_t)g.cols * g.cols * g.count;
    g.L = soff;
    soff = up(soff + sq_r);
    g.R = soff;
    soff = up(soff + sq_c);
    g.Li = soff;
    soff = up(soff + sq_r);
    g.Ri = soff;
    soff = up(soff + sq_c);
    P->max_rows = std::max(P->max_rows, g.rows);
    P->groups.push_back(g);
  }
  P->elems = eoff;
  P->s_M = soff;
  soff = up(soff + sizeof(float) * (size_t)eoff);
  P->s_blocks = soff;
  soff = up(soff + sizeof(BlockDev) * P->blocks.size());
  P->s_layers = soff;
  soff = up(soff + sizeof(LayerDev) * P->layers.size());
  P->s_running = soff;
  soff = up(soff + sizeof(double));
  P->s_eta = soff;
  soff = up(soff + sizeof(float));
  P->state_bytes = soff;
  // workspace: pointers, gathered G, P, norm partials, library calls
  P->tiles = (int64_t)((P->max_rows + RT - 1) / RT) * (int64_t)P->blocks.size();
  size_t w = 0;
  P->w_ptrs = w;
  w = up(w + 2 * sizeof(void*) * P->layers.size());
  P->w_G = w;
  w = up(w + sizeof(float) * (size_t)eoff);
  P->w_P = w;
  w = up(w + sizeof(float) * (size_t)eoff);
  P->w_part = w;
  w = up(w + sizeof(double) * (size_t)P->tiles);
  P->w_lib = w;
  size_t lib = 0;
  for (const Group& g : P->groups) {
    size_t b = 0;
    const pmx_matfn_opts* ro = &cfg->root_opts;
    if (pmx_workspace_size(nullptr, PMX_OP_INV_ROOT, g.rows, g.rows, g.count, PMX_F32, ro, &b) != PMX_OK ||
        (lib = std::max(lib, b), pmx_workspace_size(nullptr, PMX_OP_INV_ROOT, g.cols, g.cols,
                                                     g.count, PMX_F32, ro, &b)) != PMX_OK ||
        (lib = std::max(lib, b), pmx_workspace_size(nullptr, PMX_OP_APPLY, g.rows, g.cols,
                                                     g.count, PMX_F32, nullptr, &b)) != PMX_OK ||
        (lib = std::max(lib, b), pmx_workspace_size(nullptr, PMX_OP_STATS, g.rows, g.cols,
                                                     g.count, PMX_F32, nullptr, &b)) != PMX_OK) {
      delete P;
      return PMX_ERR_INVALID_VALUE;
    }
    lib = std::max(lib, b);
  }
  P->lib_bytes = up(lib);
  P->ws_bytes = w + P->lib_bytes;
  *out = P;
  return PMX_OK;
}

pmx_status pmx_shampoo_plan_destroy(pmx_shampoo_plan plan) {
  delete plan;
  return PMX_OK;
}

pmx_status pmx_shampoo_plan_sizes(pmx_shampoo_plan P, size_t* state_bytes, size_t* ws_bytes) {
  if (!P || !state_bytes || !ws_bytes) return PMX_ERR_INVALID_VALUE;
  *state_bytes = P->state_bytes;
  *ws_bytes = P->ws_bytes;
  return PMX_OK;
}

pmx_status pmx_shampoo_plan_init(pmx_shampoo_plan P, void* state, size_t state_bytes,
                                 void* stream) {
  if (!P) return PMX_ERR_INVALID_VALUE;
  if (!state || state_bytes < P->state_bytes || ((uintptr_t)state % kAlignS) != 0)
    return PMX_ERR_WORKSPACE;
  Guard dg(P->device);
  if (!dg.ok) return PMX_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  // the block tables are copied from the plan's host memory: not captured
  if (capturing(s)) return PMX_ERR_NOT_SUPPORTED;
  auto fill = [&](size_t off, int64_t count, int64_t n, float v) {
    if (count == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((count + ST - 1) / ST, 65536);
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(ST), 0, s,
                       at_<float>(state, off), count, n, v);
    return hipGetLastError();
  };
  for (const Group& g : P->groups) {
    const int64_t rr = (int64_t)g.rows * g.rows * g.count, cc = (int64_t)g.cols * g.cols * g.count;
    if (fill(g.L, rr, g.rows, P->cfg.eps) != hipSuccess || fill(g.R, cc, g.cols, P->cfg.eps) != hipSuccess ||
        fill(g.Li, rr, g.rows, 1.f) != hipSuccess || fill(g.Ri, cc, g.cols, 1.f) != hipSuccess)
      return PMX_ERR_HIP;
  }
  if (fill(P->s_M, P->elems, 0, 0.f) != hipSuccess) return PMX_ERR_HIP;
  hipLaunchKernelGGL(zero_scalars_kernel, dim3(1), dim3(64), 0, s,
                     at_<double>(state, P->s_running), at_<float>(state, P->s_eta), P->cfg.lr);
  if (hipGetLastError() != hipSuccess) return PMX_ERR_HIP;
  if (hipMemcpyAsync(at_<void>(state, P->s_blocks), P->blocks.data(),
                     sizeof(BlockDev) * P->blocks.size(), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(at_<void>(state, P->s_layers), P->layers.data(),
                     sizeof(LayerDev) * P->layers.size(), hipMemcpyHostToDevice, s) != hipSuccess)
    return PMX_ERR_HIP;
  return PMX_OK;
}

pmx_status pmx_shampoo_plan_step(pmx_shampoo_plan P, float* const* W, const float* const* G,
                                 int64_t step, void* state, size_t state_bytes, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!P || !W || !G || step < 0) return PMX_ERR_INVALID_VALUE;
  const int nl = (int)P->layers.size();
  for (int l = 0; l < nl; ++l)
    if (!W[l] || !G[l]) return PMX_ERR_INVALID_VALUE;
  if (!state || state_bytes < P->state_bytes || ((uintptr_t)state % kAlignS) != 0)
    return PMX_ERR_WORKSPACE;
  if (!ws || ws_bytes < P->ws_bytes || ((uintptr_t)ws % kAlignS) != 0) return PMX_ERR_WORKSPACE;
  Guard dg(P->device);
  if (!dg.ok) return PMX_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  // the pointer table below is copied from host memory that is gone once the
  // call returns, so a captured graph could not replay it: refuse capture
  if (capturing(s)) return PMX_ERR_NOT_SUPPORTED;
  const pmx_shampoo_config& c = P->cfg;
  // the step's layer pointers (W then G)
  std::vector<const void*> ptrs(2 * (size_t)nl);
  for (int l = 0; l < nl; ++l) {
    ptrs[l] = W[l];
    ptrs[nl + l] = G[l];
  }
  if (hipMemcpyAsync(at_<void>(ws, P->w_ptrs), ptrs.data(), sizeof(void*) * ptrs.size(),
                     hipMemcpyHostToDevice, s) != hipSuccess)
    return PMX_ERR_HIP;
  float* const* Wd = at_<float* const>(ws, P->w_ptrs);
  const float* const* Gd = at_<const float* const>(ws, P->w_ptrs + sizeof(void*) * nl);
  const BlockDev* bd = at_<const BlockDev>(state, P->s_blocks);
  const LayerDev* ld = at_<const LayerDev>(state, P->s_layers);
  float* Gb = at_<float>(ws, P->w_G);
  float* Pb = at_<float>(ws, P->w_P);
  float* M = at_<float>(state, P->s_M);
  double* part = at_<double>(ws, P->w_part);
  const dim3 grid((unsigned)((P->max_rows + RT - 1) / RT), (unsigned)P->blocks.size());
  hipLaunchKernelGGL(gather_kernel, grid, dim3(ST), 0, s, bd, ld, Gd, Gb, part);
  if (hipGetLastError() != hipSuccess) return PMX_ERR_HIP;
  if (c.adaptive_lr) {
    hipLaunchKernelGGL(step_size_kernel, dim3(1), dim3(ST), 0, s, part, P->tiles,
                       at_<double>(state, P->s_running), at_<float>(state, P->s_eta), c.lr);
    if (hipGetLastError() != hipSuccess) return PMX_ERR_HIP;
  }
  void* lib = at_<void>(ws, P->w_lib);
  const bool roots = step % c.root_every == 0;
  for (const Group& g : P->groups) {
    const int m = g.rows, n = g.cols, cnt = g.count;
    const int64_t smn = (int64_t)m * n;
    float* L = at_<float>(state, g.L);
    float* R = at_<float>(state, g.R);
    float* Li = at_<float>(state, g.Li);
    float* Ri = at_<float>(state, g.Ri);
    const float* gg = Gb + g.off;
    float* pg = Pb + g.off;
    pmx_status st = pmx_shampoo_stats_update_batched(P->h, gg, PMX_F32, m, n, n, smn, L, m,
                                                     (int64_t)m * m, R, n, (int64_t)n * n,
                                                     c.beta, c.eps, cnt, lib, P->lib_bytes, s);
    if (st != PMX_OK) return st;
    if (roots) {
      st = pmx_matfn_inv_root_batched(P->h, L, m, m, (int64_t)m * m, 4, Li, m, (int64_t)m * m,
                                      nullptr, m, 0, cnt, &c.root_opts, nullptr, lib,
                                      P->lib_bytes, s);
      if (st != PMX_OK) return st;
      st = pmx_matfn_inv_root_batched(P->h, R, n, n, (int64_t)n * n, 4, Ri, n, (int64_t)n * n,
                                      nullptr, n, 0, cnt, &c.root_opts, nullptr, lib,
                                      P->lib_bytes, s);
      if (st != PMX_OK) return st;
    }
    st = pmx_precond_apply_batched(P->h, Li, m, (int64_t)m * m, gg, PMX_F32, m, n, n, smn, Ri, n,
                                   (int64_t)n * n, pg, n, smn, cnt, lib, P->lib_bytes, s);
    if (st != PMX_OK) return st;
  }
  hipLaunchKernelGGL(update_kernel, grid, dim3(ST), 0, s, bd, ld, Wd, Pb, M, c.momentum,
                     c.adaptive_lr ? at_<const float>(state, P->s_eta) : nullptr, c.lr);
  if (hipGetLastError() != hipSuccess) return PMX_ERR_HIP;
  return PMX_OK;
}

}  // extern "C"
