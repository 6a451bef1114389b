"""Host-side checks of libpmx.so that need no GPU: the library loads, exports
every entry point include/pmx.h declares, and validates options and sizes."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pmx.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pmx_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from preconditioned_optimizer_matrix_amd import pmx
    names = _declared()
    assert len(names) >= 16
    raw = ctypes.CDLL(pmx.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name
    assert set(pmx.EXPORTS) == set(names)


def test_struct_layouts_match_header():
    from preconditioned_optimizer_matrix_amd import pmx
    # pmx_matfn_opts: 5 int32 + 3 float + uint64 (8-aligned) + 2 int32 + float
    # + 3 int32 + reserved = 64 bytes (version 3 ended at method, version 2 at
    # degree_max, version 1 at seed)
    assert ctypes.sizeof(pmx.Opts) == 64
    assert pmx.Opts.method.offset == 52 and pmx.Opts.scale_mode.offset == 56
    assert pmx.Opts.fp64_iters.offset == 40
    assert pmx.Opts.degree_max.offset == 44 and pmx.Opts.adapt_ratio.offset == 48
    # pmx_matfn_info: 6 int32 + 3 float + 4 * 64 float
    assert ctypes.sizeof(pmx.Info) == 4 * (6 + 3 + 4 * pmx.TRACE_LEN)
    src = open(HEADER).read()
    assert "#define PMX_TRACE_LEN %d" % pmx.TRACE_LEN in src
    assert "#define PMX_OPTS_VERSION %d" % pmx.OPTS_VERSION in src


def test_host_only_calls():
    from preconditioned_optimizer_matrix_amd import pmx
    assert pmx.lib.pmx_version() == 1
    for code in range(6):
        assert pmx.lib.pmx_status_string(code)
    o = pmx.default_opts()
    assert (o.degree, o.sketch_p, o.max_iter, o.accelerate) == (2, 8, 30, 1)
    assert math.isnan(o.alpha_lo) and math.isnan(o.alpha_hi)
    assert o.tol == pytest.approx(1e-6)
    assert (o.fp64_iters, o.method, o.struct_version) == (0, 0, pmx.OPTS_VERSION)
    assert (o.scale_mode, o.reserved) == (pmx.SCALE_FROBENIUS, 0)
    assert o.degree_max == 0 and o.adapt_ratio == pytest.approx(0.3)
    assert pmx.lib.pmx_matfn_opts_default(None) == pmx.ERR_INVALID_VALUE


def test_workspace_sizes_and_option_validation():
    from preconditioned_optimizer_matrix_amd import pmx
    o = pmx.default_opts()
    n = 4096
    b = pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, 1, pmx.F32, o)
    # six n x n fp32 work matrices, then the split-k slots (two 128 x 128
    # fp32 tiles for each of 256 workers)
    sk = 2 * 256 * 128 * 128 * 4
    assert 6 * 4 * n * n + sk <= b < 6 * 4 * n * n + sk + (1 << 20)
    bb = pmx.workspace_bytes(pmx.OP_INV_ROOT, 512, 512, 64, pmx.F32, o)
    assert bb >= 64 * 6 * 4 * 512 * 512
    # statistics: G^T in fp32 (bf16: and G widened), counters, split-k slots
    st = pmx.workspace_bytes(pmx.OP_STATS, 1024, 4096, 1, pmx.F32, None)
    assert 4 * 1024 * 4096 + sk <= st < 4 * 1024 * 4096 + sk + (1 << 20)
    stb = pmx.workspace_bytes(pmx.OP_STATS, 1024, 4096, 1, pmx.BF16, None)
    assert stb - st == 4 * 1024 * 4096
    # variable-size polar: the descriptors (32 bytes each), 256-byte aligned
    assert ctypes.sizeof(pmx.PolarBlock) == 32
    assert pmx.workspace_bytes(pmx.OP_POLAR_VARBATCH, 1, 1, 100, pmx.F32, None) == 3328
    # with blocks above the fused order: descriptors, grouped indices, and one
    # shape group's scratch (packed input and output, info, batched workspace)
    blk = (pmx.PolarBlock * 3)(pmx.PolarBlock(None, None, 8, 8, 8, 8),
                               pmx.PolarBlock(None, None, 100, 30, 30, 30),
                               pmx.PolarBlock(None, None, 100, 30, 30, 30))
    sz = ctypes.c_size_t()
    assert pmx.lib.pmx_polar_varbatch_workspace_size(blk, 1, pmx.F32, None,
                                                     ctypes.byref(sz)) == pmx.OK
    assert sz.value == 256
    assert pmx.lib.pmx_polar_varbatch_workspace_size(blk, 3, pmx.F32, None,
                                                     ctypes.byref(sz)) == pmx.OK
    grp = pmx.workspace_bytes(pmx.OP_POLAR, 100, 30, 2, pmx.F32, o)
    assert sz.value >= 256 + 256 + 2 * 4 * 100 * 30 * 2 + 2 * ctypes.sizeof(pmx.Info) + grp
    blk[1].m = pmx.VARBATCH_MAX_SIDE + 1
    assert pmx.lib.pmx_polar_varbatch_workspace_size(blk, 3, pmx.F32, None,
                                                     ctypes.byref(sz)) == pmx.ERR_INVALID_VALUE
    assert pmx.workspace_bytes(pmx.OP_APPLY, 1024, 4096, 1, pmx.F32, None) >= 4 * 1024 * 4096
    pb = pmx.workspace_bytes(pmx.OP_POLAR, 4096, 1024, 1, pmx.F32, o)
    assert pb >= 2 * 4 * 4096 * 1024 + 2 * 4 * 1024 * 1024

    def ws(**kw):
        sz = ctypes.c_size_t()
        oo = pmx.default_opts(**kw)
        return pmx.lib.pmx_workspace_size(None, pmx.OP_INV_ROOT, 64, 64, 1, pmx.F32,
                                          ctypes.byref(oo), ctypes.byref(sz))

    assert ws() == pmx.OK
    assert ws(degree=3) == pmx.OK
    assert ws(degree=4) == pmx.ERR_INVALID_VALUE
    assert ws(degree=0) == pmx.ERR_INVALID_VALUE
    # d = 3 adds the n x n buffer of R^3
    b2 = pmx.workspace_bytes(pmx.OP_INV_ROOT, 512, 512, 1, pmx.F32, pmx.default_opts())
    b3 = pmx.workspace_bytes(pmx.OP_INV_ROOT, 512, 512, 1, pmx.F32, pmx.default_opts(degree=3))
    assert b3 - b2 >= 4 * 512 * 512
    assert ws(sketch_p=0) == pmx.ERR_INVALID_VALUE
    assert ws(sketch_p=pmx.MAX_SKETCH + 1) == pmx.ERR_INVALID_VALUE
    assert ws(max_iter=0) == pmx.ERR_INVALID_VALUE
    assert ws(tol=-1.0) == pmx.ERR_INVALID_VALUE
    assert ws(alpha_lo=0.9, alpha_hi=0.5) == pmx.ERR_INVALID_VALUE
    assert ws(alpha_lo=0.4, alpha_hi=float("nan")) == pmx.ERR_INVALID_VALUE
    assert ws(struct_version=99) == pmx.ERR_INVALID_VALUE
    assert ws(alpha_lo=0.5, alpha_hi=0.5) == pmx.OK
    assert ws(fp64_iters=-1) == pmx.ERR_INVALID_VALUE
    assert ws(fp64_iters=31) == pmx.ERR_INVALID_VALUE  # more than max_iter
    assert ws(method=2) == pmx.ERR_INVALID_VALUE
    assert ws(method=1) == pmx.OK
    assert ws(method=1, degree=3) == pmx.ERR_INVALID_VALUE
    assert ws(method=1, fp64_iters=2) == pmx.ERR_INVALID_VALUE
    assert ws(method=1, degree_max=3) == pmx.ERR_INVALID_VALUE
    assert ws(fp64_iters=4) == pmx.OK
    # the 40-byte version-1 layout is still accepted (fp64_iters = 0)
    assert ws(struct_version=1, fp64_iters=7, method=5) == pmx.OK
    # version 2 (48 bytes): the fields after degree_max are not read
    assert ws(struct_version=2, adapt_ratio=float("nan"), method=5) == pmx.OK
    # version 3 (56 bytes): scale_mode and reserved are not read
    assert ws(struct_version=3, scale_mode=7, reserved=3) == pmx.OK
    # the input scale: Frobenius or the power estimate
    assert ws(scale_mode=pmx.SCALE_POWER) == pmx.OK
    assert ws(scale_mode=pmx.SCALE_POWER, method=1) == pmx.OK
    assert ws(scale_mode=2) == pmx.ERR_INVALID_VALUE
    assert ws(scale_mode=-1) == pmx.ERR_INVALID_VALUE
    assert ws(reserved=1) == pmx.ERR_INVALID_VALUE
    # adaptive degree: 2 -> 3 with the fitted alpha and fp32 updates only
    assert ws(degree_max=3) == pmx.OK
    assert ws(degree_max=2) == pmx.OK
    assert ws(degree=1, degree_max=3) == pmx.ERR_INVALID_VALUE
    assert ws(degree_max=3, accelerate=0) == pmx.ERR_INVALID_VALUE
    assert ws(degree_max=3, fp64_iters=2) == pmx.ERR_INVALID_VALUE
    assert ws(degree_max=4) == pmx.ERR_INVALID_VALUE
    assert ws(degree_max=3, adapt_ratio=float("inf")) == pmx.ERR_INVALID_VALUE
    # fp64 leading updates add six n x n fp64 buffers
    o4 = pmx.default_opts(fp64_iters=4)
    b4 = pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, 1, pmx.F32, o4)
    assert b4 - b >= 6 * 8 * n * n
    sz = ctypes.c_size_t()
    assert pmx.lib.pmx_workspace_size(None, pmx.OP_INV_ROOT, 0, 0, 1, pmx.F32, None,
                                      ctypes.byref(sz)) == pmx.ERR_INVALID_VALUE
    assert pmx.lib.pmx_workspace_size(None, 9, 8, 8, 1, pmx.F32, None,
                                      ctypes.byref(sz)) == pmx.ERR_INVALID_VALUE


def test_calls_without_handle_enqueue_nothing():
    from preconditioned_optimizer_matrix_amd import pmx
    L = pmx.lib
    assert L.pmx_matfn_inv_root(None, None, 8, 8, 4, None, 8, None, 8, None, None, None, 0,
                                None) == pmx.ERR_INVALID_VALUE
    assert L.pmx_matfn_polar(None, None, pmx.F32, 8, 4, 4, None, 4, None, None, None, 0,
                             None) == pmx.ERR_INVALID_VALUE
    assert L.pmx_precond_apply(None, None, 8, None, pmx.F32, 8, 4, 4, None, 4, None, 4,
                               None, 0, None) == pmx.ERR_INVALID_VALUE
    assert L.pmx_shampoo_stats_update(None, None, pmx.F32, 8, 4, 4, None, 8, None, 4, 0.9,
                                      1e-6, None, 0, None) == pmx.ERR_INVALID_VALUE
    h = ctypes.c_void_p()
    assert L.pmx_create(None, 0) == pmx.ERR_INVALID_VALUE
    assert L.pmx_destroy(None) == pmx.ERR_INVALID_VALUE


def test_product_path_has_no_oracle_or_cpu_fallback():
    # the package never imports the oracle and its binding fails loudly
    pkg = os.path.join(ROOT, "preconditioned_optimizer_matrix_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "numpy.linalg" not in txt and "np.linalg" not in txt, f


def test_shampoo_plan_host_side():
    # plan creation, grouping and sizes need no GPU (a null handle is refused)
    from preconditioned_optimizer_matrix_amd import pmx
    c = pmx.shampoo_config()
    assert (c.block, c.root_every, c.adaptive_lr) == (1024, 1, 0)
    assert c.beta == pytest.approx(0.95) and c.root_opts.degree == 2
    arr = (pmx.Layer * 1)(pmx._layer((8, 8)))
    plan = ctypes.c_void_p()
    assert pmx.lib.pmx_shampoo_plan_create(None, ctypes.byref(c), arr, 1,
                                           ctypes.byref(plan)) == pmx.ERR_INVALID_VALUE


def test_varblocks_descriptor_table():
    # the reusable descriptor table of the variable-size polar call: one
    # 32-byte entry per block with its addresses, shape and row strides
    # (host tensors: the table is only built, nothing is launched)
    import torch
    from preconditioned_optimizer_matrix_amd import pmx
    Gs = [torch.zeros(3, 5), torch.zeros(64, 64), torch.zeros(10, 40)[:, :7]]
    Us = [torch.zeros(3, 5), torch.zeros(64, 64), torch.zeros(10, 7)]
    vb = pmx.VarBlocks(Gs, Us)
    assert vb.count == 3 and vb.dtype == pmx.F32
    for e, g, u in zip(vb.arr, Gs, Us):
        assert (e.m, e.n, e.ldg, e.ldu) == (g.shape[0], g.shape[1], g.stride(0), u.stride(0))
        assert e.g == g.data_ptr() and e.u == u.data_ptr()
    # outputs allocated when not given, contiguous, one per block
    vb2 = pmx.VarBlocks(Gs)
    assert [tuple(u.shape) for u in vb2.Us] == [(3, 5), (64, 64), (10, 7)]
    assert all(u.is_contiguous() for u in vb2.Us)
    with pytest.raises(ValueError):
        pmx.VarBlocks(Gs, Us[:2])
    with pytest.raises(ValueError):
        pmx.VarBlocks([torch.zeros(2, 3, 4)])
    with pytest.raises(ValueError):
        pmx.VarBlocks([])
