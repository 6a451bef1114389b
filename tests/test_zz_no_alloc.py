"""pmx_precond_apply_noalloc (the library's scratch array instead of a
workspace) against pmx_precond_apply_batched on the same inputs, through the
C ABI: two calls in a row, the second smaller, fp32 and bf16 gradients, and
the size limit.  Both run the same kernels, so the results must agree bit
for bit; both are also checked against the oracle's L^{-1/4} G R^{-1/4}
product ([Shampoo blog] section 2.3, step 4) to the fp32 tolerance.
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


def _case(torch, dev, batch, m, n, seed):
    Ls = np.stack([W.spd_logu(m, seed + 3 * b)[0] for b in range(batch)])
    Rs = np.stack([W.spd_logu(n, seed + 3 * b + 1)[0] for b in range(batch)])
    Gs = np.stack([W.gaussian(m, n, seed + 3 * b + 2) for b in range(batch)])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return Ls, Rs, Gs, t(Ls), t(Rs), t(Gs)


@pytest.mark.parametrize("bf16", [False, True])
def test_noalloc_matches_workspace_call(env, bf16):
    torch, pmx, dev = env
    # the first call larger than the second, both ragged against the tiles
    for batch, m, n, seed in ((2, 1000, 1100, 11), (3, 130, 77, 29)):
        print("noalloc apply batch=%d m=%d n=%d bf16=%s" % (batch, m, n, bf16), flush=True)
        Ls, Rs, Gs, L, R, G = _case(torch, dev, batch, m, n, seed)
        if bf16:
            G = G.to(torch.bfloat16)
            Gs = G.float().cpu().numpy()
        P_ref = pmx.precond_apply(L, G, R)
        P_na = pmx.precond_apply_noalloc(L, G, R)
        torch.cuda.synchronize()
        assert torch.equal(P_ref.view(torch.int16) if bf16 else P_ref,
                           P_na.view(torch.int16) if bf16 else P_na)
        Pn = P_na.float().cpu().numpy()
        worst = max(cf.rel_fro(Pn[b], cf.precond_apply(Ls[b], Gs[b], Rs[b]))
                    for b in range(batch))
        print("  bit-identical to the workspace call; worst rel err vs oracle %.2e" % worst,
              flush=True)
        assert worst < (1e-2 if bf16 else 1e-5)


def test_noalloc_rejects_oversize(env):
    torch, pmx, dev = env
    m, n, batch = 2048, 4096, 2  # 64 MiB of fp32 intermediate > the scratch
    need = pmx.workspace_bytes(pmx.OP_APPLY, m, n, batch, pmx.F32)
    assert need > pmx.NOALLOC_SCRATCH_BYTES
    h = pmx.handle(0)
    st = pmx._stream_of(dev)
    dummy = torch.empty(16, device=dev)
    rc = pmx.lib.pmx_precond_apply_noalloc(h, pmx._ptr(dummy), m, 0, pmx._ptr(dummy), pmx.F32, m,
                                          n, n, 0, pmx._ptr(dummy), n, 0, pmx._ptr(dummy), n, 0,
                                          batch, st)
    assert rc == pmx.ERR_WORKSPACE
    # the largest fp32 case that fits is accepted by the size check
    assert pmx.workspace_bytes(pmx.OP_APPLY, 1024, 4096, 2, pmx.F32) <= pmx.NOALLOC_SCRATCH_BYTES
