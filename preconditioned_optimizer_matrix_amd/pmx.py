"""ctypes binding of libpmx.so (the C ABI declared in include/pmx.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in libpmx's kernels.
Importing this module raises if the built library is missing, so no caller
can silently fall back to another implementation.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PMX_LIBRARY selects another build of the same library (the host-sanitized
# libpmx_san.so of build.py's --sanitize); there is no other implementation
LIB_PATH = os.environ.get("PMX_LIBRARY") or os.path.join(_HERE, "libpmx.so")

OK, ERR_INVALID_VALUE, ERR_NOT_SUPPORTED, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP = range(6)
RUNNING, CONVERGED, MAXITER, STAGNATED, NONFINITE, DIVERGED = -1, 0, 1, 2, 3, 4
F32, BF16 = 0, 1
OP_STATS, OP_INV_ROOT, OP_POLAR, OP_APPLY, OP_POLAR_VARBATCH = range(5)
VARBATCH_MAX_DIM = 64
VARBATCH_MAX_SIDE = 8192
OPTS_VERSION = 4
METHOD_NEWTON_SCHULZ, METHOD_INVERSE_NEWTON = 0, 1
SCALE_FROBENIUS, SCALE_POWER = 0, 1
TRACE_LEN = 64
MAX_SKETCH = 16
STATUS_NAMES = {RUNNING: "RUNNING", CONVERGED: "CONVERGED", MAXITER: "MAXITER",
                STAGNATED: "STAGNATED", NONFINITE: "NONFINITE", DIVERGED: "DIVERGED"}

EXPORTS = [
    "pmx_create", "pmx_destroy", "pmx_status_string", "pmx_version",
    "pmx_matfn_opts_default", "pmx_workspace_size",
    "pmx_shampoo_stats_update", "pmx_shampoo_stats_update_batched",
    "pmx_matfn_inv_root", "pmx_matfn_inv_root_batched",
    "pmx_matfn_polar", "pmx_matfn_polar_batched", "pmx_matfn_polar_varbatch",
    "pmx_precond_apply", "pmx_precond_apply_batched",
    "pmx_trace_enable", "pmx_trace_collect", "pmx_set_host_poll",
    "pmx_shampoo_config_default", "pmx_shampoo_plan_create", "pmx_shampoo_plan_destroy",
    "pmx_shampoo_plan_sizes", "pmx_shampoo_plan_init", "pmx_shampoo_plan_step",
    "pmx_sketch_gaussian", "pmx_precond_apply_noalloc", "pmx_polar_varbatch_workspace_size",
]

# kernel classes of the launch trace (pmx_kernel_class)
KERNEL_CLASSES = ["gemm_power", "gemm_update", "gemm_resid", "gemm_stats", "gemm_apply",
                  "skinny", "skinny_alpha", "other"]


class Opts(ctypes.Structure):
    _fields_ = [("struct_version", ctypes.c_int32), ("degree", ctypes.c_int32),
                ("sketch_p", ctypes.c_int32), ("max_iter", ctypes.c_int32),
                ("accelerate", ctypes.c_int32), ("alpha_lo", ctypes.c_float),
                ("alpha_hi", ctypes.c_float), ("tol", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("fp64_iters", ctypes.c_int32),
                ("degree_max", ctypes.c_int32), ("adapt_ratio", ctypes.c_float),
                ("method", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ShampooConfig(ctypes.Structure):
    _fields_ = [("struct_version", ctypes.c_int32), ("block", ctypes.c_int32),
                ("root_every", ctypes.c_int32), ("adaptive_lr", ctypes.c_int32),
                ("beta", ctypes.c_float), ("eps", ctypes.c_float), ("lr", ctypes.c_float),
                ("momentum", ctypes.c_float), ("root_opts", Opts)]


class Layer(ctypes.Structure):
    _fields_ = [("dims", ctypes.c_int32), ("shape", ctypes.c_int32 * 4)]


class PolarBlock(ctypes.Structure):
    _fields_ = [("g", ctypes.c_void_p), ("u", ctypes.c_void_p), ("m", ctypes.c_int32),
                ("n", ctypes.c_int32), ("ldg", ctypes.c_int32), ("ldu", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("iters", ctypes.c_int32 * 2),
                ("gemms", ctypes.c_int32), ("sketch_products", ctypes.c_int32),
                ("stages", ctypes.c_int32), ("scale", ctypes.c_float),
                ("residual", ctypes.c_float * 2),
                ("alpha", (ctypes.c_float * TRACE_LEN) * 2),
                ("rtrace", (ctypes.c_float * TRACE_LEN) * 2)]


INFO_DTYPE = np.dtype([("status", "<i4"), ("iters", "<i4", (2,)), ("gemms", "<i4"),
                       ("sketch_products", "<i4"), ("stages", "<i4"), ("scale", "<f4"),
                       ("residual", "<f4", (2,)), ("alpha", "<f4", (2, TRACE_LEN)),
                       ("rtrace", "<f4", (2, TRACE_LEN))])
assert INFO_DTYPE.itemsize == ctypes.sizeof(Info)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpmx.so is not built (%s); run "
                          "`python -m preconditioned_optimizer_matrix_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "pmx_create": (_i32, [ctypes.POINTER(_vp), _i32]),
        "pmx_destroy": (_i32, [_vp]),
        "pmx_status_string": (ctypes.c_char_p, [_i32]),
        "pmx_version": (_i32, []),
        "pmx_matfn_opts_default": (_i32, [ctypes.POINTER(Opts)]),
        "pmx_workspace_size": (_i32, [_vp, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(Opts),
                                      ctypes.POINTER(_sz)]),
        "pmx_shampoo_stats_update": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp,
                                            _i32, _f32, _f32, _vp, _sz, _vp]),
        "pmx_shampoo_stats_update_batched": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i64, _vp,
                                                    _i32, _i64, _vp, _i32, _i64, _f32, _f32,
                                                    _i32, _vp, _sz, _vp]),
        "pmx_matfn_inv_root": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _i32,
                                      ctypes.POINTER(Opts), _vp, _vp, _sz, _vp]),
        "pmx_matfn_inv_root_batched": (_i32, [_vp, _vp, _i32, _i32, _i64, _i32, _vp, _i32, _i64,
                                              _vp, _i32, _i64, _i32, ctypes.POINTER(Opts), _vp,
                                              _vp, _sz, _vp]),
        "pmx_matfn_polar": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32,
                                   ctypes.POINTER(Opts), _vp, _vp, _sz, _vp]),
        "pmx_matfn_polar_batched": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i64, _vp, _i32,
                                           _i64, _i32, ctypes.POINTER(Opts), _vp, _vp, _sz,
                                           _vp]),
        "pmx_matfn_polar_varbatch": (_i32, [_vp, ctypes.POINTER(PolarBlock), _i32, _i32,
                                            ctypes.POINTER(Opts), _vp, _vp, _sz, _vp]),
        "pmx_precond_apply": (_i32, [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _i32,
                                     _vp, _i32, _vp, _sz, _vp]),
        "pmx_precond_apply_batched": (_i32, [_vp, _vp, _i32, _i64, _vp, _i32, _i32, _i32, _i32,
                                             _i64, _vp, _i32, _i64, _vp, _i32, _i64, _i32, _vp,
                                             _sz, _vp]),
        "pmx_polar_varbatch_workspace_size": (_i32, [ctypes.POINTER(PolarBlock), _i32, _i32,
                                                     ctypes.POINTER(Opts),
                                                     ctypes.POINTER(_sz)]),
        "pmx_precond_apply_noalloc": (_i32, [_vp, _vp, _i32, _i64, _vp, _i32, _i32, _i32, _i32,
                                             _i64, _vp, _i32, _i64, _vp, _i32, _i64, _i32,
                                             _vp]),
        "pmx_trace_enable": (_i32, [_vp, _i32]),
        "pmx_set_host_poll": (_i32, [_vp, _i32]),
        "pmx_shampoo_config_default": (_i32, [ctypes.POINTER(ShampooConfig)]),
        "pmx_shampoo_plan_create": (_i32, [_vp, ctypes.POINTER(ShampooConfig),
                                           ctypes.POINTER(Layer), _i32,
                                           ctypes.POINTER(ctypes.c_void_p)]),
        "pmx_shampoo_plan_destroy": (_i32, [_vp]),
        "pmx_shampoo_plan_sizes": (_i32, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "pmx_shampoo_plan_init": (_i32, [_vp, _vp, _sz, _vp]),
        "pmx_shampoo_plan_step": (_i32, [_vp, ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.POINTER(ctypes.c_void_p), _i64, _vp, _sz, _vp,
                                         _sz, _vp]),
        "pmx_sketch_gaussian": (_i32, [_vp, ctypes.c_uint64, _i32, _i32, _i32, _i32, _i32, _vp,
                                       _i32, _vp, _vp]),
        "pmx_trace_collect": (_i32, [_vp, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class PmxError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        msg = lib.pmx_status_string(code).decode()
        super().__init__("%s: %s" % (where, msg))


def check(code, where=""):
    if code != OK:
        raise PmxError(code, where)


def default_opts(**kw):
    """pmx_matfn_opts with the library defaults, fields overridden by kw."""
    o = Opts()
    check(lib.pmx_matfn_opts_default(ctypes.byref(o)), "opts_default")
    for k, v in kw.items():
        if not hasattr(o, k):
            raise KeyError(k)
        setattr(o, k, v)
    return o


# ---------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


_handles = {}


def handle(device=None):
    torch = _torch()
    dev = torch.cuda.current_device() if device is None else int(device)
    h = _handles.get(dev)
    if h is None:
        hv = _vp()
        check(lib.pmx_create(ctypes.byref(hv), dev), "pmx_create")
        h = _handles[dev] = hv
    return h


def _stream(t):
    torch = _torch()
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _stream_of(device):
    torch = _torch()
    return _vp(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s" % t.dtype)


def _mat(t):
    """(rows, cols, ld, batch_stride, batch) of a 2-D or 3-D row-major tensor."""
    if t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("matrices must have unit column stride")
        return t.shape[0], t.shape[1], t.stride(0), 0, 1
    if t.dim() == 3:
        if t.stride(2) != 1:
            raise ValueError("matrices must have unit column stride")
        return t.shape[1], t.shape[2], t.stride(1), t.stride(0), t.shape[0]
    raise ValueError("expected a 2-D matrix or a 3-D batch")


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def workspace_bytes(op, m, n, batch=1, dtype=F32, opts=None):
    sz = _sz()
    check(lib.pmx_workspace_size(None, op, m, n, batch, dtype,
                                 ctypes.byref(opts) if opts is not None else None,
                                 ctypes.byref(sz)), "workspace_size")
    return sz.value


def workspace(nbytes, device):
    """Workspace tensor (256-byte aligned: torch's caching allocator aligns to 512 B)."""
    torch = _torch()
    t = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t


def new_info(batch, device):
    torch = _torch()
    return torch.zeros(batch * INFO_DTYPE.itemsize, dtype=torch.uint8, device=device)


def parse_info(info_tensor):
    """Device info buffer -> numpy structured array (synchronises via .cpu())."""
    raw = info_tensor.detach().cpu().numpy().tobytes()
    return np.frombuffer(raw, dtype=INFO_DTYPE)


def shampoo_stats_update(G, L, R, beta, eps, ws=None):
    """In place: L <- beta L + (1-beta) G G^T + eps I, R <- beta R + (1-beta) G^T G + eps I."""
    m, n, ldg, sg, batch = _mat(G)
    if L is not None and L.dim() == 3:
        batch = L.shape[0]
    elif R is not None and R.dim() == 3:
        batch = R.shape[0]
    if L is not None:
        _, _, ldl, sl, _ = _mat(L)
    else:
        ldl, sl = m, 0
    if R is not None:
        _, _, ldr, sr, _ = _mat(R)
    else:
        ldr, sr = n, 0
    dt = _dtype_code(G)
    need = workspace_bytes(OP_STATS, m, n, batch, dt, None)
    if need and (ws is None or ws.numel() < need):
        ws = workspace(need, G.device)
    check(lib.pmx_shampoo_stats_update_batched(
        handle(G.device.index), _ptr(G), dt, m, n, ldg, sg, _ptr(L), ldl, sl,
        _ptr(R), ldr, sr, float(beta), float(eps), batch, _ptr(ws) if need else None,
        ws.numel() if need else 0, _stream(G)), "shampoo_stats_update")
    return L, R


def inv_root(A, p, opts=None, aux=True, out=None, out_aux=None, info=None, ws=None):
    """A^{-1/p} (and A^{1/p} if aux) of an SPD matrix or a batch of them.
    Returns (X, X_aux or None, info_tensor)."""
    torch = _torch()
    n, n2, lda, sa, batch = _mat(A)
    if n != n2:
        raise ValueError("A must be square")
    if opts is None:
        opts = default_opts()
    X = out if out is not None else torch.empty_like(A, memory_format=torch.contiguous_format)
    XA = None
    if aux:
        XA = out_aux if out_aux is not None else torch.empty_like(X)
    _, _, ldx, sx, _ = _mat(X)
    ldaux, saux = (n, 0)
    if XA is not None:
        _, _, ldaux, saux, _ = _mat(XA)
    if info is None:
        info = new_info(batch, A.device)
    need = workspace_bytes(OP_INV_ROOT, n, n, batch, F32, opts)
    if ws is None or ws.numel() < need:
        ws = workspace(need, A.device)
    check(lib.pmx_matfn_inv_root_batched(
        handle(A.device.index), _ptr(A), n, lda, sa, int(p), _ptr(X), ldx, sx, _ptr(XA),
        ldaux, saux, batch, ctypes.byref(opts), _ptr(info), _ptr(ws), ws.numel(),
        _stream(A)), "matfn_inv_root")
    return X, XA, info


def polar(G, opts=None, out=None, info=None, ws=None):
    """Polar factor of G (m x n) or a batch; returns (U, info_tensor)."""
    torch = _torch()
    m, n, ldg, sg, batch = _mat(G)
    if opts is None:
        opts = default_opts()
    U = out if out is not None else torch.empty_like(G, memory_format=torch.contiguous_format)
    _, _, ldu, su, _ = _mat(U)
    if info is None:
        info = new_info(batch, G.device)
    dt = _dtype_code(G)
    need = workspace_bytes(OP_POLAR, m, n, batch, dt, opts)
    if ws is None or ws.numel() < need:
        ws = workspace(need, G.device)
    check(lib.pmx_matfn_polar_batched(
        handle(G.device.index), _ptr(G), dt, m, n, ldg, sg, _ptr(U), ldu, su, batch,
        ctypes.byref(opts), _ptr(info), _ptr(ws), ws.numel(), _stream(G)), "matfn_polar")
    return U, info


class VarBlocks:
    """The descriptor table of a variable-size polar call: the addresses,
    shapes and row strides of the blocks Gs (2-D, unit column stride, one
    dtype) and of their outputs Us (allocated when not given).  Built once and
    passed to polar_varbatch(blocks=...) on every call over the same tensors,
    so a call marshals nothing per block; valid while those tensors live."""

    def __init__(self, Gs, Us=None):
        torch = _torch()
        self.Gs = list(Gs)
        if not self.Gs:
            raise ValueError("no blocks")
        self.Us = (list(Us) if Us is not None else
                   [torch.empty_like(g, memory_format=torch.contiguous_format) for g in self.Gs])
        if len(self.Us) != len(self.Gs):
            raise ValueError("one output per block")
        self.count = len(self.Gs)
        self.arr = (PolarBlock * self.count)()
        for i, (g, u) in enumerate(zip(self.Gs, self.Us)):
            if g.dim() != 2 or u.dim() != 2:
                raise ValueError("blocks are 2-D matrices")
            m, n, ldg, _, _ = _mat(g)
            _, _, ldu, _, _ = _mat(u)
            self.arr[i] = PolarBlock(_ptr(g), _ptr(u), m, n, ldg, ldu)
        self.dtype = _dtype_code(self.Gs[0])
        self.device = self.Gs[0].device


def polar_varbatch(Gs=None, opts=None, outs=None, info=None, ws=None, blocks=None):
    """Polar factors of a list of 2-D blocks of different shapes (sides up to
    VARBATCH_MAX_SIDE, one dtype) in one call: blocks of sides up to
    VARBATCH_MAX_DIM in one fused launch, larger ones grouped by shape;
    returns (list of U, info_tensor).  `blocks` (a VarBlocks) replaces Gs and
    outs with a descriptor table built beforehand."""
    if opts is None:
        opts = default_opts()
    if blocks is None:
        blocks = VarBlocks(Gs, outs)
    count, dev = blocks.count, blocks.device
    if info is None:
        info = new_info(count, dev)
    sz = _sz()
    check(lib.pmx_polar_varbatch_workspace_size(blocks.arr, count, blocks.dtype,
                                                ctypes.byref(opts), ctypes.byref(sz)),
          "polar_varbatch_workspace_size")
    need = sz.value
    if ws is None or ws.numel() < need:
        ws = workspace(need, dev)
    check(lib.pmx_matfn_polar_varbatch(handle(dev.index), blocks.arr, count, blocks.dtype,
                                       ctypes.byref(opts), _ptr(info), _ptr(ws), ws.numel(),
                                       _stream(blocks.Gs[0])), "matfn_polar_varbatch")
    return blocks.Us, info


def shampoo_config(root_opts=None, **kw):
    """pmx_shampoo_config with the library defaults, fields overridden by kw."""
    c = ShampooConfig()
    check(lib.pmx_shampoo_config_default(ctypes.byref(c)), "shampoo_config_default")
    for k, v in kw.items():
        if not hasattr(c, k):
            raise KeyError(k)
        setattr(c, k, v)
    if root_opts is not None:
        c.root_opts = root_opts
    return c


def _layer(shape):
    ly = Layer()
    ly.dims = len(shape)
    if ly.dims not in (2, 4):
        # passed on: the library rejects it (PMX_ERR_INVALID_VALUE)
        return ly
    for i, v in enumerate(shape[:4]):
        ly.shape[i] = int(v)
    return ly


class ShampooPlan:
    """A whole Shampoo step over a list of layer shapes (2-D or 4-D), with its
    device state and workspace (torch tensors on `device`)."""

    def __init__(self, shapes, device, config=None):
        torch = _torch()
        self.device = torch.device(device)
        self.config = config if config is not None else shampoo_config()
        arr = (Layer * len(shapes))(*[_layer(s) for s in shapes])
        self.nlayers = len(shapes)
        plan = ctypes.c_void_p()
        check(lib.pmx_shampoo_plan_create(handle(self.device.index), ctypes.byref(self.config),
                                          arr, len(shapes), ctypes.byref(plan)),
              "shampoo_plan_create")
        self.plan = plan
        sb, wb = _sz(), _sz()
        check(lib.pmx_shampoo_plan_sizes(plan, ctypes.byref(sb), ctypes.byref(wb)),
              "shampoo_plan_sizes")
        self.state = workspace(sb.value, self.device)
        self.ws = workspace(wb.value, self.device)
        check(lib.pmx_shampoo_plan_init(plan, _ptr(self.state), self.state.numel(),
                                        _stream_of(self.device)), "shampoo_plan_init")

    def step(self, Ws, Gs, t):
        if len(Ws) != self.nlayers or len(Gs) != self.nlayers:
            raise ValueError("one weight and one gradient per layer")
        for w, g in zip(Ws, Gs):
            if w.dtype != _torch().float32 or g.dtype != _torch().float32:
                raise TypeError("fp32 weights and gradients")
            if not (w.is_contiguous() and g.is_contiguous()):
                raise ValueError("contiguous weights and gradients")
        wp = (ctypes.c_void_p * self.nlayers)(*[w.data_ptr() for w in Ws])
        gp = (ctypes.c_void_p * self.nlayers)(*[g.data_ptr() for g in Gs])
        check(lib.pmx_shampoo_plan_step(self.plan, wp, gp, int(t), _ptr(self.state),
                                        self.state.numel(), _ptr(self.ws), self.ws.numel(),
                                        _stream_of(self.device)), "shampoo_plan_step")

    def __del__(self):
        if getattr(self, "plan", None) is not None and lib is not None:
            lib.pmx_shampoo_plan_destroy(self.plan)
            self.plan = None


def precond_apply(Linv, G, Rinv, out=None, ws=None):
    """P = Linv G Rinv (single or batched)."""
    torch = _torch()
    m, n, ldg, sg, batch = _mat(G)
    _, _, ldl, sl, _ = _mat(Linv)
    _, _, ldr, sr, _ = _mat(Rinv)
    P = out if out is not None else torch.empty_like(G, memory_format=torch.contiguous_format)
    _, _, ldp, sp, _ = _mat(P)
    dt = _dtype_code(G)
    need = workspace_bytes(OP_APPLY, m, n, batch, dt, None)
    if ws is None or ws.numel() < need:
        ws = workspace(need, G.device)
    check(lib.pmx_precond_apply_batched(
        handle(G.device.index), _ptr(Linv), ldl, sl, _ptr(G), dt, m, n, ldg, sg, _ptr(Rinv),
        ldr, sr, _ptr(P), ldp, sp, batch, _ptr(ws), ws.numel(), _stream(G)),
        "precond_apply")
    return P


def sketch_gaussian(seed, matrix, stage, k, n, p, device=None, words=True):
    """The iterations' Gaussian sketch S_k (n x p fp32) of (matrix, stage, k)
    and, if words, the raw Philox words behind it (n x p int32 tensor holding
    the uint32 bits); returns (S, words or None)."""
    torch = _torch()
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else int(device))
    S = torch.empty((n, p), dtype=torch.float32, device=dev)
    Wd = torch.empty((n, p), dtype=torch.int32, device=dev) if words else None
    check(lib.pmx_sketch_gaussian(handle(dev.index), ctypes.c_uint64(int(seed)), int(matrix),
                                  int(stage), int(k), int(n), int(p), _ptr(S), int(p), _ptr(Wd),
                                  _stream_of(dev)), "sketch_gaussian")
    return S, Wd


NOALLOC_SCRATCH_BYTES = 32 << 20


def precond_apply_noalloc(Linv, G, Rinv, out=None):
    """P = Linv G Rinv through the allocation-free entry point (the library's
    scratch holds the intermediate; no workspace)."""
    torch = _torch()
    m, n, ldg, sg, batch = _mat(G)
    _, _, ldl, sl, _ = _mat(Linv)
    _, _, ldr, sr, _ = _mat(Rinv)
    P = out if out is not None else torch.empty_like(G, memory_format=torch.contiguous_format)
    _, _, ldp, sp, _ = _mat(P)
    check(lib.pmx_precond_apply_noalloc(
        handle(G.device.index), _ptr(Linv), ldl, sl, _ptr(G), _dtype_code(G), m, n, ldg, sg,
        _ptr(Rinv), ldr, sr, _ptr(P), ldp, sp, batch, _stream(G)), "precond_apply_noalloc")
    return P


def set_host_poll(chunk, device=None):
    """Host-polled convergence for this device's handle: after every `chunk`
    updates the iteration loops publish whether any matrix still iterates and
    stop enqueuing once none does (0 turns it off: all max_iter updates are
    enqueued and the surplus ones exit on the device).  Same results either
    way; the calling thread waits on the published points."""
    check(lib.pmx_set_host_poll(handle(device), int(chunk)), "set_host_poll")


def trace_enable(enable=True, device=None):
    """Bracket every launch of this device's handle with HIP events."""
    check(lib.pmx_trace_enable(handle(device), 1 if enable else 0), "trace_enable")


def trace_collect(device=None):
    """{kernel class: (total ms, launches)} of the launches since trace_enable
    or the previous collect (waits for the recorded events)."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    check(lib.pmx_trace_collect(handle(device), ms, cnt), "trace_collect")
    return {KERNEL_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}
