"""The library's calls captured into a HIP graph and replayed.

Every launch goes to the caller's stream, no call allocates or clears memory
with a memset node (the control blocks are reset by a kernel), and host
polling switches itself off while the stream is being captured, so a whole
matrix-function call can be captured once and replayed.  Each replay is
checked bit for bit against the eager result, with eager work and
synchronisations between the replays.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    from preconditioned_optimizer_matrix_amd import pmx
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    return torch, pmx, dev


def _say(*a):
    print(*a, flush=True)


def _bytes(t):
    # raw bytes of any dtype (bf16 has no numpy type)
    import torch
    return t.contiguous().view(-1).view(torch.uint8).cpu().numpy().tobytes()


def _replays(torch, dev, graph, outs, refs, n=3):
    for rep in range(n):
        for o in outs:
            o.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert _bytes(o) == r, rep
        # eager work of the program between replays
        a = torch.randn(300, 300, device=dev)
        float((a @ a).sum())


def test_capture_inv_root_and_polar(env):
    torch, pmx, dev = env
    As = np.stack([W.spd_logu(384, 60 + b, 0.3, 1.0)[0] for b in range(2)])
    A = torch.from_numpy(As).to(dev)
    opts = pmx.default_opts(scale_mode=pmx.SCALE_POWER, max_iter=12)
    ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, 384, 384, 2, pmx.F32, opts), dev)
    X, XA = torch.empty_like(A), torch.empty_like(A)
    info = pmx.new_info(2, dev)
    call = lambda: pmx.inv_root(A, 4, opts=opts, out=X, out_aux=XA, info=info, ws=ws)
    Gb = torch.from_numpy(W.gaussian(512, 128, 3)).to(torch.bfloat16).to(dev)
    popts = pmx.default_opts(tol=1e-2, max_iter=12)
    pws = pmx.workspace(pmx.workspace_bytes(pmx.OP_POLAR, 512, 128, 1, pmx.BF16, popts), dev)
    U = torch.empty_like(Gb)
    pinfo = pmx.new_info(1, dev)
    pcall = lambda: pmx.polar(Gb, opts=popts, out=U, info=pinfo, ws=pws)
    _say("graph: eager references")
    call()
    pcall()
    torch.cuda.synchronize()
    refs = [_bytes(t) for t in (X, XA, info, U, pinfo)]
    assert int(pmx.parse_info(info)[0]["status"]) == pmx.CONVERGED
    # host polling on: it turns itself off under capture
    pmx.set_host_poll(2)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
            pcall()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        _say("graph: capture")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call()
            pcall()
    finally:
        pmx.set_host_poll(0)
    _say("graph: replays")
    _replays(torch, dev, g, [X, XA, info, U, pinfo], refs)


def test_capture_refused_where_host_tables_are_copied(env):
    """The variable-size polar call and the whole Shampoo step copy a host
    table to the device on the call's stream; a replay could not rely on
    that host memory, so both refuse capture (PMX_ERR_NOT_SUPPORTED) and
    enqueue nothing."""
    torch, pmx, dev = env
    Gs = [torch.from_numpy(W.gaussian(12, 7, 5)).to(dev)]
    plan = pmx.ShampooPlan([(48, 80)], dev, pmx.shampoo_config(block=64))
    Wt = torch.zeros(48, 80, device=dev)
    Gt = torch.from_numpy(W.gaussian(48, 80, 6)).to(dev)
    torch.cuda.synchronize()
    codes = []
    g = torch.cuda.CUDAGraph()
    x = torch.zeros(4, device=dev)
    with torch.cuda.graph(g):
        for fn in (lambda: pmx.polar_varbatch(Gs), lambda: plan.step([Wt], [Gt], 0)):
            try:
                fn()
                codes.append(pmx.OK)
            except pmx.PmxError as e:
                codes.append(e.code)
        x.add_(1.0)
    _say("capture refused with codes", codes)
    assert codes == [pmx.ERR_NOT_SUPPORTED, pmx.ERR_NOT_SUPPORTED]
    g.replay()
    torch.cuda.synchronize()
    assert float(x.sum()) == 4.0
    # outside capture both run
    pmx.polar_varbatch(Gs)
    plan.step([Wt], [Gt], 0)
    torch.cuda.synchronize()
