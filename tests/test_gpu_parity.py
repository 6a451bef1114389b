"""GPU parity of libpmx against the fp64 oracle on small and ragged shapes.

Tolerances: the fp32 path is held to a relative Frobenius error of 1e-4
against the exact (eigendecomposition / SVD) results; single GEMM-based
operations (statistics, apply) to 1e-5, which covers fp32 accumulation over
K <= 512 (worst case K u ~ 3e-5, typical sqrt(K) u ~ 1e-6).
"""
import numpy as np
import pytest

import workloads as W
from oracle import closed_form as cf
from oracle import inv_newton as inw
from oracle import prism

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


@pytest.mark.parametrize("m,n", [(17, 33), (64, 32), (130, 200), (256, 384), (1, 5)])
def test_precond_apply(env, m, n):
    torch, pmx, dev = env
    _say("apply", m, n)
    rng = np.random.default_rng(m * 1000 + n)
    Li = rng.standard_normal((m, m)).astype(np.float32)
    Ri = rng.standard_normal((n, n)).astype(np.float32)
    G = rng.standard_normal((m, n)).astype(np.float32)
    P = pmx.precond_apply(torch.from_numpy(Li).to(dev), torch.from_numpy(G).to(dev),
                          torch.from_numpy(Ri).to(dev))
    torch.cuda.synchronize()
    assert cf.rel_fro(P.cpu().numpy(), cf.precond_apply(Li, G, Ri)) < 1e-5


@pytest.mark.parametrize("m,n", [(17, 45), (100, 260), (128, 128), (3, 1)])
def test_stats_update(env, m, n):
    torch, pmx, dev = env
    _say("stats", m, n)
    rng = np.random.default_rng(m + n)
    Gs = [rng.standard_normal((m, n)).astype(np.float32) for _ in range(3)]
    L0 = (1e-3 * np.eye(m)).astype(np.float32)
    R0 = (1e-3 * np.eye(n)).astype(np.float32)
    L = torch.from_numpy(L0).to(dev)
    R = torch.from_numpy(R0).to(dev)
    for G in Gs:
        pmx.shampoo_stats_update(torch.from_numpy(G).to(dev), L, R, 0.95, 1e-4)
    torch.cuda.synchronize()
    Lr, Rr = cf.stats_sequence(L0, R0, Gs, 0.95, 1e-4)
    assert cf.rel_fro(L.cpu().numpy(), Lr) < 1e-5
    assert cf.rel_fro(R.cpu().numpy(), Rr) < 1e-5


def _run_root(env, A, p, **kw):
    torch, pmx, dev = env
    opts = pmx.default_opts(**kw)
    X, XA, info = pmx.inv_root(torch.from_numpy(A).to(dev), p, opts=opts)
    torch.cuda.synchronize()
    return X.cpu().numpy(), XA.cpu().numpy(), pmx.parse_info(info)


@pytest.mark.parametrize("n", [17, 64, 65, 200, 517, 600])
@pytest.mark.parametrize("p", [2, 4])
def test_inv_root_matches_closed_form(env, n, p):
    _, pmx, _ = env
    _say("inv_root", n, p)
    A, Q, lam = W.spd_logu(n, 1000 + n)
    X, XA, info = _run_root(env, A, p, seed=11)
    ref, ref_aux = cf.inv_root(A, p)
    # fp32 floors the measured residual near u sqrt(n); reaching it is success
    assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
    assert cf.rel_fro(X, ref) < 1e-4
    assert cf.rel_fro(XA, ref_aux) < 1e-4


@pytest.mark.parametrize("p", [2, 4])
def test_inv_root_iterations_and_alpha_follow_reference(env, p):
    # same sketches on both sides: alpha traces agree while the residual is
    # large enough for alpha to be well determined, iteration counts within 1
    _, pmx, _ = env
    A, _, _ = W.spd_logu(96, 77)
    _say("alpha trace", p)
    X, XA, info = _run_root(env, A, p, seed=5)
    _, _, ref = prism.inv_root(A.astype(np.float64), p=p,
                               sketch_fn=prism.make_sketch_fn(5, b=0, p=8))
    inf = info[0]
    assert int(inf["gemms"]) > 0
    for s, st in enumerate(ref["stages"]):
        it = int(inf["iters"][s])
        assert abs(it - st.iters) <= 1, (s, it, st.iters)
        for k in range(min(it, st.iters)):
            if st.r[k] >= 1e-3:
                assert abs(inf["alpha"][s][k] - st.alpha[k]) < 1e-3, (s, k)
                assert inf["rtrace"][s][k] == pytest.approx(st.r[k], rel=1e-3)
    total_ref = sum(st.gemms for st in ref["stages"])
    assert abs(int(inf["gemms"]) - total_ref) <= 4 * len(ref["stages"])


@pytest.mark.parametrize("d", [1, 2, 3])
def test_taylor_and_degree_variants(env, d):
    _, pmx, _ = env
    A, _, _ = W.spd_logu(80, 3, 1e-2, 1.0)
    _say("variants d", d)
    ref, _ = cf.inv_root(A, 2)
    for acc in (0, 1):
        X, _, info = _run_root(env, A, 2, degree=d, accelerate=acc)
        assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
        assert cf.rel_fro(X, ref) < 1e-4
        _, _, r = prism.inv_root(A.astype(np.float64), p=2, d=d, accelerate=bool(acc),
                                 sketch_fn=prism.make_sketch_fn(0))
        assert abs(int(info[0]["iters"][0]) - r["stages"][0].iters) <= 1


@pytest.mark.parametrize("p", [2, 4])
def test_degree_three(env, p):
    # d = 3: g = 1 + R/2 + 3R^2/8 + alpha R^3 with alpha in [5/16, 2.46]; R^3 is a
    # fourth (symmetric) product per update and the alpha fit uses K_1..K_7
    torch, pmx, dev = env
    for n in (64, 100, 256, 517):
        _say("degree 3 root", p, n)
        A, _, _ = W.spd_logu(n, 3000 + n)
        X, XA, info = _run_root(env, A, p, degree=3, seed=4)
        ref, ref_aux = cf.inv_root(A, p)
        assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), n
        assert cf.rel_fro(X, ref) < 1e-4 and cf.rel_fro(XA, ref_aux) < 1e-4, n
    # alpha traces and iteration counts against the oracle with the same sketches
    A, _, _ = W.spd_logu(96, 77)
    _say("degree 3 alpha trace", p)
    X, XA, info = _run_root(env, A, p, degree=3, seed=5)
    _, _, ref = prism.inv_root(A.astype(np.float64), p=p, d=3,
                               sketch_fn=prism.make_sketch_fn(5, b=0, p=8))
    inf = info[0]
    for s, st in enumerate(ref["stages"]):
        it = int(inf["iters"][s])
        assert abs(it - st.iters) <= 1, (s, it, st.iters)
        for k in range(min(it, st.iters)):
            if st.r[k] >= 1e-3:
                assert abs(inf["alpha"][s][k] - st.alpha[k]) < 1e-3, (s, k)
                assert inf["rtrace"][s][k] == pytest.approx(st.r[k], rel=1e-3)
    # batched, mixed conditioning
    As = np.stack([W.spd_logu(200, 40 + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(3)])
    Xb, _, infb = pmx.inv_root(torch.from_numpy(As).to(dev), p, opts=pmx.default_opts(degree=3))
    torch.cuda.synchronize()
    for b in range(3):
        assert cf.rel_fro(Xb[b].cpu().numpy(), cf.inv_root(As[b], p)[0]) < 1e-4, b
    if p == 2:
        # fp32 polar factor with d = 3
        for m, n in ((64, 32), (150, 150), (300, 17)):
            _say("degree 3 polar", m, n)
            G = W.gaussian(m, n, m + 7 * n)
            U, pinfo = pmx.polar(torch.from_numpy(G).to(dev), opts=pmx.default_opts(degree=3))
            torch.cuda.synchronize()
            assert int(pmx.parse_info(pinfo)[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
            assert cf.rel_fro(U.cpu().numpy(), cf.polar(G)[0]) < 1e-4
        # d = 3 is an fp32 path: the bf16 polar and the fp64 leading updates refuse it
        Gb = _bf16(torch, W.gaussian(64, 32, 5)).to(dev)
        with pytest.raises(pmx.PmxError):
            pmx.polar(Gb, opts=pmx.default_opts(degree=3))
        with pytest.raises(pmx.PmxError):
            pmx.inv_root(torch.from_numpy(A).to(dev), 2, opts=pmx.default_opts(degree=3, fp64_iters=2))
        torch.cuda.synchronize()


@pytest.mark.parametrize("p", [2, 4])
def test_adaptive_degree(env, p):
    # degree 2 raised to 3 per matrix after an update whose sketched
    # contraction exceeds adapt_ratio (0.3)
    torch, pmx, dev = env
    for n in (100, 256, 517):
        _say("adaptive degree root", p, n)
        # (at kappa = 1e4 and n = 517 an fp32 emulation of the fixed d = 2
        # iteration already floors near 1.1e-4 for A^{1/4}, so kappa = 1e3 here)
        A, _, _ = W.spd_logu(n, 5000 + n, 1e-3, 1.0)
        X, XA, info = _run_root(env, A, p, degree_max=3, seed=6)
        ref, ref_aux = cf.inv_root(A, p)
        assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), n
        assert cf.rel_fro(X, ref) < 1e-4 and cf.rel_fro(XA, ref_aux) < 1e-4, n
    # same sketches as the oracle: iteration counts, alphas and products
    A, _, _ = W.spd_logu(96, 77)
    _say("adaptive degree alpha trace", p)
    X, XA, info = _run_root(env, A, p, degree_max=3, seed=5)
    _, _, ref = prism.inv_root(A.astype(np.float64), p=p, d=2, degree_max=3,
                               sketch_fn=prism.make_sketch_fn(5, b=0, p=8))
    inf = info[0]
    assert any(3 in st.degree for st in ref["stages"])
    for s, st in enumerate(ref["stages"]):
        it = int(inf["iters"][s])
        assert abs(it - st.iters) <= 1, (s, it, st.iters)
        for k in range(min(it, st.iters)):
            if st.r[k] >= 1e-3:
                assert abs(inf["alpha"][s][k] - st.alpha[k]) < 1e-3, (s, k)
    total_ref = sum(st.gemms for st in ref["stages"])
    assert abs(int(inf["gemms"]) - total_ref) <= 5 * len(ref["stages"])
    # batched, mixed conditioning: each matrix keeps its own degree
    As = np.stack([W.spd_logu(200, 60 + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(3)])
    Xb, _, infb = pmx.inv_root(torch.from_numpy(As).to(dev), p,
                               opts=pmx.default_opts(degree_max=3))
    torch.cuda.synchronize()
    for b in range(3):
        assert cf.rel_fro(Xb[b].cpu().numpy(), cf.inv_root(As[b], p)[0]) < 1e-4, b
    if p == 2:
        for m, n in ((150, 150), (300, 17), (96, 200)):
            _say("adaptive degree polar", m, n)
            G = W.gaussian(m, n, 3 * m + n)
            U, pinfo = pmx.polar(torch.from_numpy(G).to(dev), opts=pmx.default_opts(degree_max=3))
            torch.cuda.synchronize()
            assert int(pmx.parse_info(pinfo)[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
            assert cf.rel_fro(U.cpu().numpy(), cf.polar(G)[0]) < 1e-4
        with pytest.raises(pmx.PmxError):
            pmx.polar(_bf16(torch, W.gaussian(64, 32, 5)).to(dev),
                      opts=pmx.default_opts(degree_max=3))
        torch.cuda.synchronize()


@pytest.mark.parametrize("p", [2, 4])
def test_inverse_newton(env, p):
    # method 1: X <- X g, M <- g^p M with the PRISM alpha (degree-2p objective)
    torch, pmx, dev = env
    M1 = pmx.METHOD_INVERSE_NEWTON
    for d in (1, 2):
        for n in (64, 100, 256, 517):
            _say("inverse newton", p, d, n)
            A, _, _ = W.spd_logu(n, 7000 + n, 1e-3, 1.0)
            X, XA, info = _run_root(env, A, p, method=M1, degree=d, seed=2, max_iter=40)
            ref, ref_aux = cf.inv_root(A, p)
            assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (d, n)
            assert cf.rel_fro(X, ref) < 1e-4 and cf.rel_fro(XA, ref_aux) < 1e-4, (d, n)
        # iteration counts, alphas and products against the oracle (same sketches)
        A, _, _ = W.spd_logu(96, 77)
        _say("inverse newton alpha trace", p, d)
        X, XA, info = _run_root(env, A, p, method=M1, degree=d, seed=5, max_iter=40)
        _, _, ref = inw.inv_root(A.astype(np.float64), p=p, d=d, max_iter=40,
                                 sketch_fn=prism.make_sketch_fn(5, b=0, p=8))
        inf, st = info[0], ref["stages"][0]
        it = int(inf["iters"][0])
        assert abs(it - st.iters) <= 1, (it, st.iters)
        for k in range(min(it, st.iters)):
            if st.r[k] >= 1e-3:
                assert abs(inf["alpha"][0][k] - st.alpha[k]) < 1e-3, (d, k)
                assert inf["rtrace"][0][k] == pytest.approx(st.r[k], rel=1e-3)
        per = (d - 1) + (1 if p == 2 else 2) + 1
        assert abs(int(inf["gemms"]) - st.gemms) <= per + 1
    # the Taylor coefficient with d = 1 is the classical coupled inverse Newton
    A, _, _ = W.spd_logu(80, 3, 1e-2, 1.0)
    X, _, info = _run_root(env, A, p, method=M1, degree=1, accelerate=0, max_iter=60)
    _, _, r = inw.inv_root(A.astype(np.float64), p=p, d=1, accelerate=False, max_iter=60)
    assert cf.rel_fro(X, cf.inv_root(A, p)[0]) < 1e-4
    assert abs(int(info[0]["iters"][0]) - r["stages"][0].iters) <= 1
    # batched, and a non-finite input
    As = np.stack([W.spd_logu(200, 80 + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(3)])
    As[2, 5, 7] = np.nan
    Xb, _, infb = pmx.inv_root(torch.from_numpy(As).to(dev), p,
                               opts=pmx.default_opts(method=M1))
    torch.cuda.synchronize()
    inf = pmx.parse_info(infb)
    for b in range(2):
        assert cf.rel_fro(Xb[b].cpu().numpy(), cf.inv_root(As[b], p)[0]) < 1e-4, b
    assert int(inf[2]["status"]) == pmx.NONFINITE
    assert np.all(np.isnan(Xb[2].cpu().numpy()))


def test_power_scale(env):
    # scale_mode 1: c = ||A||_F min(1, 2 mu) from eight power passes; the scale,
    # the iteration counts and the roots against the oracle with the same
    # start block (the sketch of stage 2)
    torch, pmx, dev = env
    P = pmx.SCALE_POWER
    for n, lo in ((64, 0.5), (200, 0.5), (517, 0.2), (1024, 0.5)):
        for p in (2, 4):
            _say("power scale", n, p)
            A, _, _ = W.spd_logu(n, 9000 + n, lo, 1.0)
            X, XA, info = _run_root(env, A, p, seed=4, scale_mode=P)
            _, _, ref_info = prism.inv_root(A.astype(np.float64), p,
                                            sketch_fn=prism.make_sketch_fn(4, b=0, p=8),
                                            scale="power")
            ref, ref_aux = cf.inv_root(A, p)
            assert int(info[0]["status"]) == pmx.CONVERGED, (n, p)
            assert cf.rel_fro(X, ref) < 1e-4 and cf.rel_fro(XA, ref_aux) < 1e-4, (n, p)
            assert float(info[0]["scale"]) == pytest.approx(ref_info["c"], rel=1e-5), (n, p)
            for s_, st in enumerate(ref_info["stages"]):
                assert abs(int(info[0]["iters"][s_]) - st.iters) <= 1, (n, p, s_)
            # never more updates than the Frobenius scale
            _, _, inf_f = _run_root(env, A, p, seed=4)
            assert int(info[0]["iters"].sum()) <= int(inf_f[0]["iters"].sum()), (n, p)
    # batched, a shared start block stream per matrix; the inverse Newton
    # iteration and fp64 leading updates take the same scale
    As = np.stack([W.spd_logu(300, 70 + b, 10.0 ** -b, 1.0)[0] for b in range(3)])
    for kw in ({}, {"method": pmx.METHOD_INVERSE_NEWTON}, {"fp64_iters": 2}):
        _say("power scale batched", kw)
        Xb, _, infb = pmx.inv_root(torch.from_numpy(As).to(dev), 4,
                                   opts=pmx.default_opts(scale_mode=P, seed=9, **kw))
        torch.cuda.synchronize()
        inf = pmx.parse_info(infb)
        for b in range(3):
            c_ref = prism.input_scale(As[b].astype(np.float64), "power",
                                      prism.make_sketch_fn(9, b=b, p=8))
            assert float(inf[b]["scale"]) == pytest.approx(c_ref, rel=1e-5), (kw, b)
            assert cf.rel_fro(Xb[b].cpu().numpy(), cf.inv_root(As[b], 4)[0]) < 1e-4, (kw, b)
    # the variable-size polar factor does not take it
    with pytest.raises(pmx.PmxError):
        pmx.polar_varbatch([torch.from_numpy(W.gaussian(16, 8, 1)).to(dev)],
                           opts=pmx.default_opts(scale_mode=P))


def _spd_from(lam, seed):
    n = lam.size
    Q = W.random_orthogonal(np.random.default_rng(seed), n)
    return ((Q * lam) @ Q.T).astype(np.float32)


def test_power_scale_spectra(env):
    # spectra that stress the estimate: an isolated top eigenvalue over a bulk
    # just below half of it (the estimate's worst case), two clusters, a
    # single large eigenvalue, geometric decay; every one converges to the
    # eigendecomposition result with the estimated scale, in both iterations
    torch, pmx, dev = env
    P = pmx.SCALE_POWER
    for n in (512, 1000):
        cases = {
            "isolated top": np.concatenate([[1.0], np.full(n - 1, 0.45)]),
            "two clusters": np.concatenate([np.full(n // 2, 1.0), np.full(n - n // 2, 0.05)]),
            "one large": np.concatenate([[50.0], np.linspace(0.5, 1.0, n - 1)]),
            "geometric 1e-3": np.geomspace(1e-3, 1.0, n),
            "flat": np.linspace(0.8, 1.0, n),
        }
        for k, (name, lam) in enumerate(cases.items()):
            A = _spd_from(lam, 100 * n + k)
            for method in (pmx.METHOD_NEWTON_SCHULZ, pmx.METHOD_INVERSE_NEWTON):
                _say("power scale spectrum", n, name, method)
                X, XA, info = _run_root(env, A, 4, scale_mode=P, method=method, max_iter=40)
                ref, ref_aux = cf.inv_root(A, 4)
                assert int(info[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (n, name, method)
                assert cf.rel_fro(X, ref) < 1e-4 and cf.rel_fro(XA, ref_aux) < 1e-4, (n, name, method)
                # the scale covers the spectrum and never exceeds ||A||_F
                assert float(lam.max()) <= float(info[0]["scale"]) <= float(np.linalg.norm(lam)) * 1.0001


def _spread(m, n, seed, lo):
    # m x n with singular values geomspace(lo, 1) and random singular vectors
    rng = np.random.default_rng(seed)
    U0 = np.linalg.qr(rng.standard_normal((max(m, n), min(m, n))))[0]
    V0 = np.linalg.qr(rng.standard_normal((min(m, n), min(m, n))))[0]
    G = (U0 * np.geomspace(lo, 1.0, min(m, n))) @ V0.T
    return np.ascontiguousarray(G if m >= n else G.T, dtype=np.float32)


def test_polar_power_scale(env):
    # scale_mode 1 for the polar factor: s from eight complement passes on
    # I - R_0, R_0 rewritten, 1 / s folded into the first g
    torch, pmx, dev = env
    P = pmx.SCALE_POWER
    for (m, n) in ((512, 256), (256, 512), (300, 172)):
        _say("polar power scale fp32", m, n)
        G = _spread(m, n, m + n, 1e-3)
        U, info = pmx.polar(torch.from_numpy(G).to(dev), opts=pmx.default_opts(scale_mode=P, seed=3))
        Uf, info_f = pmx.polar(torch.from_numpy(G).to(dev), opts=pmx.default_opts(seed=3))
        torch.cuda.synchronize()
        inf, inf_f = pmx.parse_info(info)[0], pmx.parse_info(info_f)[0]
        _, ref = prism.polar(G.astype(np.float64), sketch_fn=prism.make_sketch_fn(3, b=0, p=8),
                             scale="power")
        assert int(inf["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (m, n)
        assert cf.rel_fro(U.cpu().numpy(), cf.polar(G)[0]) < 1e-4, (m, n)
        assert float(inf["scale"]) == pytest.approx(ref["c"], rel=1e-5), (m, n)
        assert abs(int(inf["iters"][0]) - ref["stages"][0].iters) <= 1, (m, n)
        assert int(inf["iters"][0]) <= int(inf_f["iters"][0]), (m, n)
    # fp32, batched (each matrix its own start block and scale); smallest
    # singular values 1e-1 .. 1e-3: at 1e-4 the fp32 factor itself floors
    # near the 1e-4 bar, with either scale
    _say("polar power scale fp32 batched")
    Gs = np.stack([_spread(512, 256, 40 + b, 10.0 ** -(b + 1)) for b in range(3)])
    U, info = pmx.polar(torch.from_numpy(Gs).to(dev), opts=pmx.default_opts(scale_mode=P, seed=5))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)
    for b in range(3):
        _, ref = prism.polar(Gs[b].astype(np.float64), sketch_fn=prism.make_sketch_fn(5, b=b, p=8),
                             scale="power")
        assert int(inf[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b
        assert cf.rel_fro(U[b].cpu().numpy(), cf.polar(Gs[b])[0]) < 1e-4, b
        assert float(inf[b]["scale"]) == pytest.approx(ref["c"], rel=1e-5), b
    # bf16: not supported (its rounding, amplified while the top singular
    # values overshoot under the largest alpha, made the iteration diverge)
    with pytest.raises(pmx.PmxError):
        pmx.polar(_bf16(torch, Gs).to(dev), opts=pmx.default_opts(scale_mode=P))


def test_polar_varbatch(env):
    # many small blocks of different shapes (tall, wide, square, 1 x 1, the
    # 64 limit) in one fused launch, against the SVD polar factor and, for a
    # few blocks, the oracle's iteration with the block's own sketch stream
    torch, pmx, dev = env
    rng = np.random.default_rng(44)
    shapes = [(1, 1), (64, 64), (64, 1), (1, 64), (3, 5), (40, 17), (17, 40)]
    shapes += [tuple(int(x) for x in rng.integers(1, 65, 2)) for _ in range(33)]
    Gs = [W.gaussian(m, n, 100 + i) for i, (m, n) in enumerate(shapes)]
    _say("polar varbatch fp32", len(Gs))
    Us, info = pmx.polar_varbatch([torch.from_numpy(g).to(dev) for g in Gs],
                                  opts=pmx.default_opts(seed=9))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)
    for i, (g, u) in enumerate(zip(Gs, Us)):
        assert int(inf[i]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (i, shapes[i])
        assert cf.rel_fro(u.cpu().numpy(), cf.polar(g)[0]) < 1e-4, (i, shapes[i])
    for i in (1, 5, 6):
        _, ref = prism.polar(Gs[i].astype(np.float64), sketch_fn=prism.make_sketch_fn(9, b=i, p=8))
        st = ref["stages"][0]
        assert abs(int(inf[i]["iters"][0]) - st.iters) <= 1
        for k in range(min(int(inf[i]["iters"][0]), st.iters)):
            if st.r[k] >= 1e-3:
                assert abs(inf[i]["alpha"][0][k] - st.alpha[k]) < 1e-3, (i, k)
    # a descriptor table built once and reused: two calls, the same factors
    # bit for bit as the call that built its own table
    Gd = [torch.from_numpy(g).to(dev) for g in Gs]
    vb = pmx.VarBlocks(Gd)
    for _ in range(2):
        vb.Us[0].fill_(float("nan"))
        Ur, _ = pmx.polar_varbatch(blocks=vb, opts=pmx.default_opts(seed=9))
        torch.cuda.synchronize()
        for u, ur in zip(Us, Ur):
            assert torch.equal(u, ur)
    # bf16 blocks: fp32 inside, the factor rounded once on store
    Gb = [_bf16(torch, g).to(dev) for g in Gs[:12]]
    Ub, _ = pmx.polar_varbatch(Gb)
    torch.cuda.synchronize()
    for g, u in zip(Gb, Ub):
        gq = g.float().cpu().numpy()
        assert cf.rel_fro(u.float().cpu().numpy(), cf.polar(gq)[0]) < 1e-2
    # argument errors: a block above the limit, an output overlapping its input
    big = torch.zeros(pmx.VARBATCH_MAX_SIDE + 1, 2, device=dev)
    with pytest.raises(pmx.PmxError):
        pmx.polar_varbatch([torch.from_numpy(Gs[0]).to(dev), big])
    g0 = torch.from_numpy(Gs[5]).to(dev)
    with pytest.raises(pmx.PmxError):
        pmx.polar_varbatch([g0], outs=[g0])
    with pytest.raises(pmx.PmxError):
        pmx.polar_varbatch([g0], opts=pmx.default_opts(degree=3))
    torch.cuda.synchronize()


def test_polar_varbatch_large_blocks(env, margin):
    # blocks above the fused order (grouped by shape, packed, batched fp32
    # iteration, scattered back) mixed with small ones in one call, against
    # the SVD polar factor; sides up to 512, tall and wide, repeated shapes
    torch, pmx, dev = env
    shapes = [(65, 40), (100, 300), (300, 100), (512, 512), (128, 128), (7, 9),
              (128, 128), (200, 64), (64, 200), (128, 128), (40, 65), (384, 96), (33, 1)]
    Gs = [W.gaussian(m, n, 900 + i) for i, (m, n) in enumerate(shapes)]
    _say("polar varbatch with large blocks", len(Gs))
    Us, info = pmx.polar_varbatch([torch.from_numpy(g).to(dev) for g in Gs],
                                  opts=pmx.default_opts(seed=5))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)
    worst = 0.0
    for i, (g, u) in enumerate(zip(Gs, Us)):
        assert int(inf[i]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (i, shapes[i])
        e = cf.rel_fro(u.cpu().numpy(), cf.polar(g)[0])
        worst = max(worst, e)
        assert e < 1e-4, (i, shapes[i], e)
        # a single column is orthonormal after the scaling: no update
        assert (int(inf[i]["iters"][0]) > 0) == (min(shapes[i]) > 1), (i, shapes[i])
    margin("varbatch blocks up to 512 vs SVD factor (fp32)", worst, 1e-4)
    # bf16: fp32 inside, one rounding on store
    Gb = [_bf16(torch, g).to(dev) for g in Gs[:6]]
    Ub, _ = pmx.polar_varbatch(Gb)
    torch.cuda.synchronize()
    for g, u in zip(Gb, Ub):
        gq = g.float().cpu().numpy()
        assert cf.rel_fro(u.float().cpu().numpy(), cf.polar(gq)[0]) < 1e-2
    # the same large block alone through the batched call: identical factor
    # (same kernels; the sketch of group position 0 equals batch position 0)
    U1, _ = pmx.polar(torch.from_numpy(Gs[3]).to(dev), opts=pmx.default_opts(seed=5))
    torch.cuda.synchronize()
    assert torch.equal(U1, Us[3])


def test_rank_deficient_statistics(env):
    # Shampoo's first step: one 48 x 80 gradient on eps I statistics leaves
    # 32 eigenvalues of R at the damping (kappa = 2.3e4).  The pure fp32
    # chain floors near 2e-4 on R^{-1/4} there (a float32 emulation of the
    # same iteration lands at 2.1e-4); with the fp64 leading updates the
    # root and the preconditioned step are within 1e-4.  Pure fp32 bounds:
    # the measured floors with margin, so a loss of accuracy shows.
    torch, pmx, dev = env
    Gs = W.gaussian(48, 80, 7)
    Lr, Rr = cf.stats_update(1e-3 * np.eye(48), 1e-3 * np.eye(80), Gs, 0.9, 1e-4)
    lam = np.linalg.eigvalsh(Rr)
    assert lam[31] < 1.1e-3 and lam[32] > 0.4  # the 32-fold eigenvalue at the damping
    Lx, Rx = cf.inv_root(Lr, 4)[0], cf.inv_root(Rr, 4)[0]
    Pr = cf.precond_apply(Lx, Gs, Rx)
    G = torch.from_numpy(Gs).to(dev)
    for kw, root_bound, apply_bound in (({}, 4e-4, 8e-4), ({"fp64_iters": 4}, 1e-4, 1e-4)):
        _say("rank-deficient statistics", kw)
        o = pmx.default_opts(**kw)
        Li, _, il = pmx.inv_root(torch.from_numpy(Lr.astype(np.float32)).to(dev), 4, aux=False,
                                 opts=o)
        Ri, _, ir = pmx.inv_root(torch.from_numpy(Rr.astype(np.float32)).to(dev), 4, aux=False,
                                 opts=o)
        P = pmx.precond_apply(Li, G, Ri)
        torch.cuda.synchronize()
        eL = cf.rel_fro(Li.cpu().numpy(), Lx)
        eR = cf.rel_fro(Ri.cpu().numpy(), Rx)
        eP = cf.rel_fro(P.cpu().numpy(), Pr)
        _say("  L^-1/4 %.2e, R^-1/4 %.2e, P %.2e" % (eL, eR, eP))
        for info in (il, ir):
            assert int(pmx.parse_info(info)[0]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
        assert eL < 1e-4 and eR < root_bound and eP < apply_bound, kw


def test_inv_root_batched(env):
    torch, pmx, dev = env
    _say("batched inv_root")
    As = np.stack([W.spd_logu(72, 50 + b, 10.0 ** -(b + 1), 1.0)[0] for b in range(4)])
    X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), 4)
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)
    Xn = X.cpu().numpy()
    for b in range(4):
        assert int(inf[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
        assert cf.rel_fro(Xn[b], cf.inv_root(As[b], 4)[0]) < 1e-4
    # matrices converge in different numbers of iterations
    assert len(set(int(i) for i in inf["iters"][:, 0])) > 1


@pytest.mark.parametrize("p", [2, 4])
def test_fp64_leading_updates(env, p):
    # kappa = 1e6 power-law blocks (ragged n = 100 and n = 256): fp32 alone
    # floors near 2e-4; with the first four updates of each stage in fp64 the
    # result is within 1e-4 of the oracle
    torch, pmx, dev = env
    _say("fp64 leading updates", p)
    for n, k64 in ((100, 4), (256, 4)):
        As, _, _ = W.spd_power_batch(3, n, 1100 + n)
        opts = pmx.default_opts(fp64_iters=k64)
        X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), p, opts=opts)
        torch.cuda.synchronize()
        inf = pmx.parse_info(info)
        Xn, XAn = X.cpu().numpy(), XA.cpu().numpy()
        for b in range(3):
            ref, ref_aux = cf.inv_root(As[b], p)
            assert int(inf[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), (n, b)
            assert cf.rel_fro(Xn[b], ref) < 1e-4, (n, b, cf.rel_fro(Xn[b], ref))
            assert cf.rel_fro(XAn[b], ref_aux) < 1e-4
            assert int(inf[b]["iters"][0]) > k64  # the fp32 updates continued the stage
    # a NaN input through the fp64 path
    A = np.eye(80, dtype=np.float32)
    A[3, 5] = np.nan
    X, _, info = _run_root(env, A, 4, fp64_iters=2)
    assert int(info[0]["status"]) == pmx.NONFINITE
    assert np.all(np.isnan(X))
    # a stage that converges inside the fp64 updates (well conditioned input)
    A, _, _ = W.spd_logu(90, 4242, 0.5, 1.0)
    X, XA, info = _run_root(env, A, p, fp64_iters=12)
    ref, ref_aux = cf.inv_root(A, p)
    assert int(info[0]["iters"][0]) < 12
    assert cf.rel_fro(X, ref) < 1e-6 and cf.rel_fro(XA, ref_aux) < 1e-6


def test_small_fused_batched(env):
    # orders up to 64 run as one fused launch per call (one workgroup per
    # matrix): a batch of mixed conditioning, ragged order 40, both roots
    torch, pmx, dev = env
    _say("small fused batch")
    As = np.stack([W.spd_logu(40, 900 + b, 10.0 ** -(b % 4 + 1), 1.0)[0] for b in range(6)])
    for p in (2, 4):
        X, XA, info = pmx.inv_root(torch.from_numpy(As).to(dev), p)
        torch.cuda.synchronize()
        inf = pmx.parse_info(info)
        Xn, XAn = X.cpu().numpy(), XA.cpu().numpy()
        for b in range(6):
            ref, ref_aux = cf.inv_root(As[b], p)
            assert int(inf[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
            assert cf.rel_fro(Xn[b], ref) < 1e-4
            assert cf.rel_fro(XAn[b], ref_aux) < 1e-4
            assert int(inf[b]["stages"]) == (2 if p == 4 else 1)
        assert len(set(int(i) for i in inf["iters"][:, 0])) > 1


@pytest.mark.parametrize("m,n", [(64, 32), (32, 48), (33, 70), (150, 150), (300, 17)])
def test_polar_fp32(env, m, n):
    torch, pmx, dev = env
    _say("polar", m, n)
    G = W.gaussian(m, n, m + 7 * n)
    U, info = pmx.polar(torch.from_numpy(G).to(dev))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)[0]
    Un = U.cpu().numpy()
    ref, _ = cf.polar(G)
    assert int(inf["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
    assert cf.rel_fro(Un, ref) < 1e-4
    k = min(m, n)
    gram = Un.T.astype(np.float64) @ Un if m >= n else Un.astype(np.float64) @ Un.T
    assert np.linalg.norm(gram - np.eye(k)) / np.sqrt(k) < 1e-5


def test_status_codes(env):
    _, pmx, _ = env
    _say("status codes")
    A = np.diag([1.0, 0.5, -0.3, 0.2]).astype(np.float32)
    X, _, info = _run_root(env, A, 2)
    assert int(info[0]["status"]) == pmx.DIVERGED
    assert np.all(np.isnan(X))
    A = np.eye(6, dtype=np.float32)
    A[1, 2] = np.nan
    _, _, info = _run_root(env, A, 4)
    assert int(info[0]["status"]) == pmx.NONFINITE
    _, _, info = _run_root(env, np.zeros((5, 5), np.float32), 2)
    assert int(info[0]["status"]) == pmx.NONFINITE
    # the same with the estimated scale (orders above the fused kernel's 64):
    # the power passes skip a non-finite or zero input, and an indefinite
    # input still diverges
    P = pmx.SCALE_POWER
    big = np.diag(np.concatenate([[1.0, 0.5, -0.3], np.full(97, 0.2)])).astype(np.float32)
    X, _, info = _run_root(env, big, 2, scale_mode=P)
    assert int(info[0]["status"]) == pmx.DIVERGED and np.all(np.isnan(X))
    Anan = np.eye(100, dtype=np.float32)
    Anan[3, 7] = np.nan
    _, _, info = _run_root(env, Anan, 4, scale_mode=P)
    assert int(info[0]["status"]) == pmx.NONFINITE
    _, _, info = _run_root(env, np.zeros((100, 100), np.float32), 4, scale_mode=P)
    assert int(info[0]["status"]) == pmx.NONFINITE
    X, XA, info = _run_root(env, 3.0 * np.eye(100, dtype=np.float32), 4, scale_mode=P)
    assert int(info[0]["status"]) == pmx.CONVERGED
    assert np.allclose(X, 3.0 ** -0.25 * np.eye(100), atol=1e-6)
    # the estimate of a I is c = 2 a (every column grows by exactly a / ||A||_F)
    assert float(info[0]["scale"]) == pytest.approx(6.0, rel=1e-6)
    A64 = W.spd_64()["A"]
    _, _, info = _run_root(env, A64, 2, max_iter=1)
    assert int(info[0]["status"]) == pmx.MAXITER and int(info[0]["iters"][0]) == 1
    _, _, info = _run_root(env, A64, 2, tol=0.0)
    assert int(info[0]["status"]) == pmx.STAGNATED
    # 1 x 1 and identity inputs
    X, XA, info = _run_root(env, np.array([[4.0]], np.float32), 4)
    assert int(info[0]["status"]) == pmx.CONVERGED
    assert X[0, 0] == pytest.approx(4.0 ** -0.25, rel=1e-5)


def test_argument_errors_enqueue_nothing(env):
    import ctypes
    torch, pmx, dev = env
    h = pmx.handle()
    A = torch.eye(8, device=dev)
    X = torch.empty_like(A)
    ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, 8, 8), dev)
    L = pmx.lib
    args = lambda **o: dict(dict(A=A.data_ptr(), n=8, lda=8, p=4, X=X.data_ptr(), ldx=8,
                                 ws=ws.data_ptr(), wsb=ws.numel()), **o)

    def call(a):
        return L.pmx_matfn_inv_root(h, a["A"], a["n"], a["lda"], a["p"], a["X"], a["ldx"],
                                    None, 8, None, None, a["ws"], a["wsb"], None)

    assert call(args()) == pmx.OK
    assert call(args(p=3)) == pmx.ERR_INVALID_VALUE
    assert call(args(lda=4)) == pmx.ERR_INVALID_VALUE
    assert call(args(n=0)) == pmx.ERR_INVALID_VALUE
    assert call(args(X=A.data_ptr())) == pmx.ERR_ALIAS
    assert call(args(wsb=16)) == pmx.ERR_WORKSPACE
    assert call(args(ws=ws.data_ptr() + 4)) == pmx.ERR_WORKSPACE
    assert call(args(ws=None)) == pmx.ERR_WORKSPACE
    torch.cuda.synchronize()


def _bf16(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("m,n", [(256, 64), (64, 200), (300, 40), (130, 37)])
def test_polar_bf16(env, m, n):
    # bf16 iterates: orthogonality to the bf16 floor, U^T G close to the exact
    # H = V Sigma V^T of the (bf16-valued) input, and U close to the exact factor
    # for this well-conditioned Gaussian input
    torch, pmx, dev = env
    _say("polar bf16", m, n)
    Gt = _bf16(torch, W.gaussian(m, n, 5 * m + n))
    G = Gt.float().numpy().astype(np.float64)
    U, info = pmx.polar(Gt.to(dev), opts=pmx.default_opts(tol=1e-2))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)[0]
    assert U.dtype == torch.bfloat16
    Un = U.float().cpu().numpy().astype(np.float64)
    Up, H = cf.polar(G if m >= n else G.T)
    if m < n:
        Un_t, G_t = Un.T, G.T
    else:
        Un_t, G_t = Un, G
    k = min(m, n)
    assert int(inf["status"]) in (pmx.CONVERGED, pmx.STAGNATED)
    assert np.linalg.norm(Un_t.T @ Un_t - np.eye(k)) / np.sqrt(k) < 1e-2
    assert cf.rel_fro(Un_t.T @ G_t, H) < 3e-2
    assert cf.rel_fro(Un_t, Up) < 3e-2


@pytest.mark.parametrize("m,n", [(640, 264), (300, 600)])
def test_polar_bf16_batched_large_tiles(env, m, n):
    # 64 matrices: enough 256 x 256 tiles for the large bf16 GEMM tile, with
    # ragged edges (264 = 256 + 8, 300 = 256 + 44, 600 = 2 * 256 + 88) and
    # whole interior tiles
    torch, pmx, dev = env
    _say("polar bf16 batched", m, n)
    vals, bits, _ = W.polar_batch(64, max(m, n), min(m, n), 7 * m + n, smin=1e-2)
    if m < n:
        vals = np.ascontiguousarray(vals.transpose(0, 2, 1))
        bits = np.ascontiguousarray(bits.transpose(0, 2, 1))
    Gt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    U, info = pmx.polar(Gt.to(dev), opts=pmx.default_opts(tol=1e-2))
    torch.cuda.synchronize()
    infs = pmx.parse_info(info)
    Un = U.float().cpu().numpy().astype(np.float64)
    k = min(m, n)
    for b in (0, 1, 31, 63):
        assert int(infs[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b
        G = vals[b].astype(np.float64)
        Up, _ = cf.polar(G if m >= n else G.T)
        Ub = Un[b] if m >= n else Un[b].T
        assert np.linalg.norm(Ub.T @ Ub - np.eye(k)) / np.sqrt(k) < 1e-2, b
        assert cf.rel_fro(Ub, Up) < 3e-2, b


def test_polar_bf16_transpose_reads(env, monkeypatch):
    # 64 matrices of 1024 x 512: whole 256 x 256 x 64 residual tiles and
    # enough of them, so I - X^T X reads the row-major iterate through the
    # LDS transpose reads (no transposed copy); a handle created with
    # PMX_BF16_MN=0 runs the transposed-copy form on the same input.  Both
    # against the SVD factor, and against each other.
    import ctypes
    torch, pmx, dev = env
    _say("polar bf16 transpose reads 64 x 1024 x 512")
    vals, bits, _ = W.polar_batch(64, 1024, 512, 9001, smin=1e-2)
    Gt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    opts = pmx.default_opts(tol=1e-2)
    U, info = pmx.polar(Gt, opts=opts)
    monkeypatch.setenv("PMX_BF16_MN", "0")
    h = ctypes.c_void_p()
    pmx.check(pmx.lib.pmx_create(ctypes.byref(h), 0), "create")
    monkeypatch.delenv("PMX_BF16_MN")
    try:
        U0 = torch.empty_like(Gt)
        info0 = pmx.new_info(64, dev)
        need = pmx.workspace_bytes(pmx.OP_POLAR, 1024, 512, 64, pmx.BF16, opts)
        ws = pmx.workspace(need, dev)
        pmx.check(pmx.lib.pmx_matfn_polar_batched(
            h, pmx._ptr(Gt), pmx.BF16, 1024, 512, 512, 1024 * 512, pmx._ptr(U0), 512,
            1024 * 512, 64, ctypes.byref(opts), pmx._ptr(info0), pmx._ptr(ws), ws.numel(),
            pmx._stream(Gt)), "polar")
        torch.cuda.synchronize()
    finally:
        pmx.lib.pmx_destroy(h)
    infs, infs0 = pmx.parse_info(info), pmx.parse_info(info0)
    Un = U.float().cpu().numpy().astype(np.float64)
    U0n = U0.float().cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in (0, 1, 17, 40, 63):
        assert int(infs[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b
        assert int(infs0[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b
        Up, _ = cf.polar(vals[b].astype(np.float64))
        for X in (Un[b], U0n[b]):
            assert np.linalg.norm(X.T @ X - np.eye(512)) / np.sqrt(512) < 1e-2, b
            assert cf.rel_fro(X, Up) < 3e-2, b
        worst = max(worst, cf.rel_fro(Un[b], U0n[b]))
    print("  transpose reads vs transposed copy: worst rel diff %.2e, iters %s / %s" % (
        worst, [int(i["iters"][0]) for i in infs[:4]], [int(i["iters"][0]) for i in infs0[:4]]),
        flush=True)
    assert worst < 1e-2


def test_polar_bf16_persistent_mixed_convergence(env, monkeypatch):
    # 64 matrices of 1024 x 512, alternately well conditioned (sigma_min 0.1)
    # and ill conditioned (1e-3), so they converge after different numbers of
    # updates and the later products skip the converged matrices' tiles, also
    # inside the persistent blocks' item walk (whose last k tile prefetches
    # the next running item).  The persistent kernel runs each tile's k loop
    # in the same order and stores the same values as the one-block-per-tile
    # kernel (a handle created with PMX_BF16_PERSIST=0) and as the persistent
    # kernel without the early loads (PMX_BF16_EARLY=0), so the calls must
    # agree bit for bit; all against the SVD factor.
    import ctypes
    torch, pmx, dev = env
    _say("polar bf16 persistent blocks, mixed convergence 64 x 1024 x 512")
    va, ba, _ = W.polar_batch(32, 1024, 512, 4242, smin=1e-1)
    vb, bb, _ = W.polar_batch(32, 1024, 512, 4243, smin=1e-3)
    vals = np.empty((64, 1024, 512), np.float32)
    bits = np.empty((64, 1024, 512), np.uint16)
    vals[0::2], vals[1::2] = va, vb
    bits[0::2], bits[1::2] = ba, bb
    Gt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    opts = pmx.default_opts(tol=1e-2)
    U, info = pmx.polar(Gt, opts=opts)

    def with_env(var):
        # the same call on a handle created with `var` = 0
        monkeypatch.setenv(var, "0")
        h = ctypes.c_void_p()
        pmx.check(pmx.lib.pmx_create(ctypes.byref(h), 0), "create")
        monkeypatch.delenv(var)
        try:
            Uo = torch.empty_like(Gt)
            info_o = pmx.new_info(64, dev)
            need = pmx.workspace_bytes(pmx.OP_POLAR, 1024, 512, 64, pmx.BF16, opts)
            ws = pmx.workspace(need, dev)
            pmx.check(pmx.lib.pmx_matfn_polar_batched(
                h, pmx._ptr(Gt), pmx.BF16, 1024, 512, 512, 1024 * 512, pmx._ptr(Uo), 512,
                1024 * 512, 64, ctypes.byref(opts), pmx._ptr(info_o), pmx._ptr(ws), ws.numel(),
                pmx._stream(Gt)), "polar")
            torch.cuda.synchronize()
        finally:
            pmx.lib.pmx_destroy(h)
        return Uo, info_o

    U0, info0 = with_env("PMX_BF16_PERSIST")
    # persistent blocks whose loads are issued after each k tile's barrier
    # (the early loads switched off): the same values again
    U1, _ = with_env("PMX_BF16_EARLY")
    assert torch.equal(U.view(torch.int16), U1.view(torch.int16))
    infs, infs0 = pmx.parse_info(info), pmx.parse_info(info0)
    iters = [int(i["iters"][0]) for i in infs]
    print("  updates: well conditioned %s, ill conditioned %s" % (
        sorted(set(iters[0::2])), sorted(set(iters[1::2]))), flush=True)
    assert max(iters[0::2]) < min(iters[1::2])
    assert torch.equal(U.view(torch.int16), U0.view(torch.int16))
    for b in range(64):
        assert int(infs[b]["status"]) == int(infs0[b]["status"]), b
        assert iters[b] == int(infs0[b]["iters"][0]), b
        assert np.array_equal(infs[b]["alpha"], infs0[b]["alpha"]), b
    # against the SVD: the factor itself for the well-conditioned matrices;
    # for sigma_min 1e-3 at tol 1e-2 in bf16 the directions of the smallest
    # singular values are resolved only coarsely, so there (as for the Muon
    # workload) orthogonality and the symmetric factor U^T G = H
    Un = U.float().cpu().numpy().astype(np.float64)
    for b in (0, 1, 2, 33, 62, 63):
        assert int(infs[b]["status"]) in (pmx.CONVERGED, pmx.STAGNATED), b
        G = vals[b].astype(np.float64)
        Up, H = cf.polar(G)
        assert np.linalg.norm(Un[b].T @ Un[b] - np.eye(512)) / np.sqrt(512) < 1e-2, b
        assert cf.rel_fro(Un[b].T @ G, H) < 3e-2, b
        if b % 2 == 0:
            assert cf.rel_fro(Un[b], Up) < 3e-2, b


def test_polar_bf16_iterations_follow_reference(env):
    torch, pmx, dev = env
    Gt = _bf16(torch, W.polar_batch(1, 512, 128, 9, smin=1e-2)[0][0])
    _say("polar bf16 trace")
    U, info = pmx.polar(Gt.to(dev), opts=pmx.default_opts(tol=1e-2, seed=3))
    torch.cuda.synchronize()
    inf = pmx.parse_info(info)[0]
    _, ref = prism.polar(Gt.float().numpy().astype(np.float64), tol=1e-2,
                         sketch_fn=prism.make_sketch_fn(3, b=0, p=8))
    st = ref["stages"][0]
    assert abs(int(inf["iters"][0]) - st.iters) <= 1
    for kk in range(min(int(inf["iters"][0]), st.iters)):
        if st.r[kk] >= 3e-2:
            assert abs(inf["alpha"][0][kk] - st.alpha[kk]) < 2e-2, kk


@pytest.mark.parametrize("m,n", [(64, 96), (33, 17)])
def test_stats_and_apply_bf16(env, m, n):
    torch, pmx, dev = env
    _say("stats/apply bf16", m, n)
    Gt = _bf16(torch, W.gaussian(m, n, m * n))
    G = Gt.float().numpy().astype(np.float64)
    L = torch.eye(m, device=dev) * 1e-2
    R = torch.eye(n, device=dev) * 1e-2
    pmx.shampoo_stats_update(Gt.to(dev), L, R, 0.9, 1e-3)
    Lr, Rr = cf.stats_update(1e-2 * np.eye(m), 1e-2 * np.eye(n), G, 0.9, 1e-3)
    torch.cuda.synchronize()
    assert cf.rel_fro(L.cpu().numpy(), Lr) < 1e-5
    assert cf.rel_fro(R.cpu().numpy(), Rr) < 1e-5
    rng = np.random.default_rng(m)
    Li = rng.standard_normal((m, m)).astype(np.float32)
    Ri = rng.standard_normal((n, n)).astype(np.float32)
    P = pmx.precond_apply(torch.from_numpy(Li).to(dev), Gt.to(dev), torch.from_numpy(Ri).to(dev))
    torch.cuda.synchronize()
    assert P.dtype == torch.bfloat16
    # fp32 products, one bf16 rounding of the output (relative 2^-8)
    assert cf.rel_fro(P.float().cpu().numpy(), cf.precond_apply(Li, G, Ri)) < 5e-3


def test_shampoo_plan_step(env):
    # a small model: two dense layers cut into blocks of 48 (ragged edges), a
    # convolution kernel, roots every 2 steps, momentum and the adaptive rate;
    # the weights after four steps against the fp64 reference
    from oracle import shampoo_step as ss
    torch, pmx, dev = env
    shapes = [(100, 70), (48, 130), (16, 8, 3, 3)]
    rng = np.random.default_rng(5)
    W0 = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    Gs = [[(0.1 * rng.standard_normal(s)).astype(np.float32) for s in shapes] for _ in range(4)]
    for momentum, adaptive in ((0.0, 0), (0.9, 1)):
        _say("shampoo plan step", momentum, adaptive)
        cfg = pmx.shampoo_config(block=48, root_every=2, beta=0.9, eps=1e-3, lr=0.05,
                                 momentum=momentum, adaptive_lr=adaptive)
        plan = pmx.ShampooPlan(shapes, dev, cfg)
        Wd = [torch.from_numpy(w.copy()).to(dev) for w in W0]
        st = ss.ShampooState(shapes, block=48, eps=1e-3)
        Wr = [w.astype(np.float64) for w in W0]
        for t in range(4):
            plan.step(Wd, [torch.from_numpy(g).to(dev) for g in Gs[t]], t)
            Wr = ss.step(st, Wr, Gs[t], t, 0.9, 1e-3, 0.05, momentum=momentum, root_every=2,
                         adaptive_lr=bool(adaptive))
        torch.cuda.synchronize()
        for l in range(len(shapes)):
            dW = Wd[l].cpu().numpy().astype(np.float64) - W0[l]
            dWr = Wr[l] - W0[l]
            assert cf.rel_fro(dW, dWr) < 1e-4, (l, cf.rel_fro(dW, dWr))
        del plan
    # argument errors
    with pytest.raises(pmx.PmxError):
        pmx.ShampooPlan([(4, 4, 4)], dev)
    with pytest.raises(pmx.PmxError):
        pmx.ShampooPlan([(8, 8)], dev, pmx.shampoo_config(block=0))
