"""Host-polled convergence (pmx_set_host_poll) against full enqueue-ahead.

With polling the update loops stop enqueuing once a published flag says that
no matrix of the batch is still iterating; every update left out would have
returned at once on the device.  So the outputs and the info records must be
bit-identical to the run without polling, with fewer launches.
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


def _calls(env):
    """Every fp32 update loop of the library (coupled roots with one and two
    stages, with the Frobenius and the estimated scale, the inverse Newton
    method, fp32 and bf16 polar), batched so that
    the matrices converge at different updates; orders above the fused
    small-matrix path."""
    torch, pmx, dev = env
    As = np.stack([W.spd_logu(200, 40 + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(3)])
    Gs = np.stack([W.gaussian(160, 96, 9 + b) for b in range(2)])
    Gb = torch.from_numpy(W.gaussian(300, 128, 4)).to(torch.bfloat16)
    out = []
    for p in (2, 4):
        X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), p)
        out += [X, XA, info]
    X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), 4,
                               opts=pmx.default_opts(method=pmx.METHOD_INVERSE_NEWTON))
    out += [X, XA, info]
    X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), 4,
                               opts=pmx.default_opts(scale_mode=pmx.SCALE_POWER))
    out += [X, XA, info]
    for G in (torch.from_numpy(Gs), Gb):
        U, info = pmx.polar(G.to(dev))
        out += [U, info]
    torch.cuda.synchronize()
    return [t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
            for t in out]


def test_host_poll_same_results(env):
    torch, pmx, dev = env
    _say("host poll: baseline")
    pmx.trace_enable(True)
    try:
        base = _calls(env)
        launches0 = sum(c for _, c in pmx.trace_collect().values())
        for chunk in (1, 2, 3):
            _say("host poll: chunk", chunk)
            pmx.set_host_poll(chunk)
            try:
                got = _calls(env)
                launches = sum(c for _, c in pmx.trace_collect().values())
            finally:
                pmx.set_host_poll(0)
            for i, (a, b) in enumerate(zip(base, got)):
                assert a.dtype == b.dtype and a.shape == b.shape, i
                assert a.tobytes() == b.tobytes(), (chunk, i)
            assert launches < launches0, (chunk, launches, launches0)
    finally:
        pmx.trace_enable(False)
    info = np.frombuffer(base[2].tobytes(), dtype=pmx.INFO_DTYPE)
    for b in range(3):
        assert int(info[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b


def test_host_poll_arguments(env):
    torch, pmx, dev = env
    with pytest.raises(pmx.PmxError):
        pmx.set_host_poll(-1)
    with pytest.raises(pmx.PmxError):
        pmx.set_host_poll(1001)
    pmx.set_host_poll(0)


def test_host_poll_across_streams(env):
    # consecutive polled calls on different streams, no synchronisation in
    # between: each loop first lets the previous loop's last publish land, so
    # no stale flag ends a loop early
    torch, pmx, dev = env
    As = [np.stack([W.spd_logu(256, 900 + 10 * i + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(2)])
          for i in range(3)]

    def run(streams):
        outs = []
        for i, A in enumerate(As):
            with torch.cuda.stream(streams[i % len(streams)]):
                X, _, info = pmx.inv_root(torch.from_numpy(A).to(dev), 4, aux=False)
            outs.append((X, info))
        torch.cuda.synchronize()
        return [(X.cpu().numpy().tobytes(), info.cpu().numpy().tobytes()) for X, info in outs]

    base = run([torch.cuda.current_stream()])
    pmx.set_host_poll(1)
    try:
        got = run([torch.cuda.Stream(), torch.cuda.Stream()])
    finally:
        pmx.set_host_poll(0)
    assert got == base
