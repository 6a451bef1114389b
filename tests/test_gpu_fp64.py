"""The fp64 leading updates (opts.fp64_iters) against the oracle's eigh roots.

The fp64 products run on the fp64 matrix cores with 64 x 64 or 128 x 128
block tiles, the symmetric ones (R^2, I - Z Y) as upper-triangle tiles.
Orders that leave ragged edges in both tile sizes, batches, and a call whose
every update runs in fp64 (so that only the final fp32 rounding separates it
from the oracle) pin them; the inverse 4th root is the chained coupled
Newton-Schulz iteration ([Shampoo blog] section 3.1; [PRISM synthesis]
Part I), its closed form Q Lambda^{-1/4} Q^T.
"""
import numpy as np
import pytest

import workloads as W
from oracle import closed_form as cf

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from preconditioned_optimizer_matrix_amd import pmx
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, pmx, dev


def _spd_batch(n, batch, seed):
    # the power-law spectrum of the 64 x 512 blocks workload (kappa = 1e6),
    # where the first four updates in fp64 bring fp32 back under 1e-4
    return W.spd_power_batch(batch, n, seed)[0]


@pytest.mark.parametrize("n,batch,tile", [(100, 3, 0), (300, 2, 64), (300, 2, 128), (700, 1, 0)])
def test_fp64_leading_updates(env, margin, monkeypatch, n, batch, tile):
    torch, pmx, dev = env
    print("fp64 leading updates n=%d batch=%d tile=%s" % (n, batch, tile or "auto"), flush=True)
    As = _spd_batch(n, batch, 900 + n)
    A = torch.from_numpy(As).to(dev)
    refs = [cf.inv_root(As[b], 4)[0] for b in range(batch)]
    h = None
    if tile:
        # a handle of its own with the tile forced (read at handle creation)
        import ctypes
        monkeypatch.setenv("PMX_F64_TILE", str(tile))
        h = ctypes.c_void_p()
        pmx.check(pmx.lib.pmx_create(ctypes.byref(h), 0), "create")
        monkeypatch.delenv("PMX_F64_TILE")
    try:
        for name, opts in (("4 fp64 updates", pmx.default_opts(fp64_iters=4)),
                           ("all fp64", pmx.default_opts(fp64_iters=30, tol=1e-7))):
            X = torch.empty_like(A)
            info = pmx.new_info(batch, dev)
            need = pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, batch, pmx.F32, opts)
            ws = pmx.workspace(need, dev)
            if h is None:
                pmx.inv_root(A, 4, opts=opts, aux=False, out=X, info=info, ws=ws)
            else:
                pmx.check(pmx.lib.pmx_matfn_inv_root_batched(
                    h, pmx._ptr(A), n, n, n * n, 4, pmx._ptr(X), n, n * n, None, n, 0, batch,
                    pmx.ctypes.byref(opts), pmx._ptr(info), pmx._ptr(ws), ws.numel(),
                    pmx._stream(A)), "inv_root")
            torch.cuda.synchronize()
            inf = pmx.parse_info(info)
            Xn = X.cpu().numpy()
            errs = [cf.rel_fro(Xn[b], refs[b]) for b in range(batch)]
            print("  %s: iters %s, worst rel err %.2e" % (
                name, [list(int(x) for x in i) for i in inf["iters"]], max(errs)), flush=True)
            for i in inf:
                assert int(i["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
            bound = 1e-4 if name == "4 fp64 updates" else 1e-5
            margin("fp64 %s, n=%d tile=%s" % (name, n, tile or "auto"), max(errs), bound)
            assert max(errs) < bound
    finally:
        if h is not None:
            pmx.lib.pmx_destroy(h)
