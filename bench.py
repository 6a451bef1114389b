"""Benchmark of the PRISM Shampoo hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

One step = one Shampoo step for one 1024 x 4096 layer (fp32): restore the
statistics after nine warm-up updates, the tenth statistics update
L <- beta L + (1 - beta) G G^T + eps I, R <- beta R + (1 - beta) G^T G + eps I,
the inverse 4th roots L^{-1/4} (n = 1024) and R^{-1/4} (n = 4096) by PRISM
coupled Newton-Schulz, and the preconditioned step L^{-1/4} G R^{-1/4}.
Inputs are seeded synthetic gradients (workloads.shampoo_1024x4096), resident
in HBM before timing starts.  Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ms per inverse-4th-root (n=4096) + MFMA TFLOP/s vs peak; GEMMs to converge"
PEAK_FP32_MFMA = 157.3  # TFLOP/s, MI355X dense fp32 matrix
PEAK_HBM = 8000.0       # GB/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--max-iter", type=int, default=30)
    ap.add_argument("--degree", type=int, default=2,
                    help="polynomial degree d of the fp32 inverse roots and polar factors "
                         "(the bf16 polar factor always runs d = 2)")
    ap.add_argument("--degree-max", type=int, default=0,
                    help="3 with --degree 2: adaptive degree (fp32 paths)")
    ap.add_argument("--method", type=int, default=0,
                    help="inverse roots: 0 coupled Newton-Schulz (chained for p = 4), "
                         "1 coupled inverse Newton")
    ap.add_argument("--scale", choices=["frobenius", "power"], default="power",
                    help="input scale of the inverse roots: the power estimate of the "
                         "top eigenvalue (opts.scale_mode 1), or ||A||_F (the library's "
                         "default, also reported beside the headline)")
    ap.add_argument("--host-poll", type=int, default=2,
                    help="updates per host-polled convergence point (0: enqueue all "
                         "max_iter updates; the surplus ones exit on the device)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads (n = 64 roots, 64 x 512 blocks, 10^4 "
                         "square root, 32 Muon matrices) in the default run")
    ap.add_argument("--no-trace", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 256 MiB fp32 buffer 4 times (a plain copy kernel of "
                         "known traffic, for scaling HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=5,
                    metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE", "BENCH_JSON"),
                    help="only write the update GEMM's HBM traffic record from four "
                         "rocprofv3 --pmc output folders (FETCH_SIZE and WRITE_SIZE of "
                         "'--steps 1 --warmup 0 --no-cpu-baseline --no-trace --no-secondary "
                         "--host-poll 0', "
                         "then of --calibrate-copy) and the JSON line that profiled bench "
                         "run printed (for its R^-1/4 update counts)")
    ap.add_argument("--sweep", choices=["sketch", "sigma"],
                    help="only a measurement sweep: the sketch width p on three "
                         "workloads, or sigma_min of the polar factor (PRISM against "
                         "the Taylor coefficient)")
    ap.add_argument("--workload", default="shampoo_1024x4096",
                    choices=["shampoo_1024x4096", "spd_64", "blocks_64x512",
                             "muon_32x4096x1024", "mp_10000", "varblocks_4096",
                             "model_step"])
    return ap.parse_args()


SCALE_MODES = {"frobenius": 0, "power": 1}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(G, L0, R0, beta, eps, updates=0):
    """The fp64 oracle (closed forms: eigendecomposition roots) for one full
    step at the full size, timed on the host cores."""
    from oracle import closed_form as cf
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count()
    t0 = time.perf_counter()
    L, R = cf.stats_update(L0, R0, G, beta, eps)
    t1 = time.perf_counter()
    Linv, _ = cf.inv_root(L, 4)
    t2 = time.perf_counter()
    Rinv, _ = cf.inv_root(R, 4)
    t3 = time.perf_counter()
    cf.precond_apply(Linv, G, Rinv)
    t4 = time.perf_counter()
    out = dict(value=round((t3 - t2) * 1e3, 1), unit="ms per inverse-4th-root (n=4096)",
               cores=int(threads), kind="oracle",
               sample="one full step at full size (fp64 stats update, eigh-based L^-1/4 and "
                      "R^-1/4, apply) = %.1f s; value is the R^-1/4 part" % (t4 - t0),
               step_s=round(t4 - t0, 2))
    if updates:
        # like for like: the oracle's PRISM iteration itself (fp64, the same
        # sketch generator) on the same R, two updates of the first coupled
        # square-root stage from Y_0 = R / ||R||_F, per update times the
        # updates the device call ran
        from oracle import prism
        Y0 = R / np.linalg.norm(R)
        t5 = time.perf_counter()
        _, _, tr = prism.coupled_sqrt_stage(Y0, d=2, tol=0.0, max_iter=2,
                                            sketch_fn=prism.make_sketch_fn(0))
        t6 = time.perf_counter()
        per = (t6 - t5) / max(tr.iters, 1)
        out["prism_like_for_like"] = dict(
            value=round(per * updates * 1e3, 1), unit="ms per inverse-4th-root (n=4096)",
            kind="oracle (PRISM iteration, fp64)", cores=int(threads),
            sample="%d updates of the first stage timed (%.1f s, %d products), scaled by the "
                   "%d updates of the device call" % (tr.iters, t6 - t5, tr.gemms, updates),
            ms_per_update=round(per * 1e3, 1))
    return out


def root_exec_flops(n, batch, iters, gemms, method=0):
    """Launched tile arithmetic of one fp32 inverse-root sequence of order n
    (batch matrices per launch) from its update counts and dense products: a
    stage of k updates runs 2 k - 1 full update products (Y g, g Z; the
    inverse Newton iteration k - 1, X g); the rest (residuals, powers of R and
    g, g^p M) are symmetric and run the upper-triangle tiles only."""
    bm = 128
    T = -(-n // bm)
    if T * (T + 1) // 2 * batch < 256:
        bm = 64
        T = -(-n // bm)
    tf = -(-n // 128)
    full = tf * tf * 2.0 * 128 * 128 * n if tf * tf * batch >= 256 else 2.0 * n ** 3
    sym = T * (T + 1) // 2 * 2.0 * bm * bm * n
    nfull = sum((2 * int(k) - 1) if method == 0 else (int(k) - 1) for k in iters if int(k) > 0)
    return nfull * full + (int(gemms) - nfull) * sym


def timed(torch, fn, steps, warmup):
    """Mean ms of `fn` over `steps` calls after `warmup` calls (HIP events on
    the current stream, synchronised on both sides)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def other_workload(args):
    """Secondary workloads (one JSON line each; the headline is the Shampoo layer)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out = measure(args.workload, args)
    print(json.dumps(out), flush=True)


def measure(wl, args, inputs=None):
    """One secondary workload's measurement as a dict (the JSON line of
    `--workload wl`).  `inputs` may hold the workload's host arrays, made
    beforehand."""
    import copy

    import torch

    import workloads as W
    from preconditioned_optimizer_matrix_amd import pmx
    args = copy.copy(args)
    dev = torch.device("cuda:0")
    pmx.set_host_poll(args.host_poll)
    # the power scale applies to the fp32 calls above order 64 (order 64 runs
    # the fused single-launch kernel, which scales by ||A||_F; the bf16 polar
    # factor takes only the Frobenius scale)
    scale = args.scale if wl in ("blocks_64x512", "mp_10000", "model_step") else "frobenius"
    args.scale = scale
    opts = pmx.default_opts(max_iter=args.max_iter, degree=args.degree,
                            degree_max=args.degree_max, method=args.method,
                            scale_mode=SCALE_MODES[scale])
    taylor = pmx.default_opts(max_iter=60, accelerate=0, degree=args.degree, method=args.method,
                              scale_mode=SCALE_MODES[scale])
    out = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
           "higher_is_better": False, "scaling": "weak", "vs_baseline": None}

    def traced(fn):
        # one more call with the launch trace: per-class kernel ms and launches
        if args.no_trace:
            return None
        pmx.trace_enable(True)
        fn()
        tr = pmx.trace_collect()
        pmx.trace_enable(False)
        return {k: [round(v[0], 3), v[1]] for k, v in tr.items()}

    if wl == "spd_64":
        c = W.spd_64()
        A = torch.from_numpy(c["A"]).to(dev)
        G = torch.from_numpy(c["G"]).to(dev)
        res = {}
        for name, fn in (("inv_sqrt_p2", lambda o: pmx.inv_root(A, 2, opts=o)),
                         ("inv_root_p4", lambda o: pmx.inv_root(A, 4, opts=o)),
                         ("polar_64x32", lambda o: pmx.polar(G, opts=o))):
            ms = timed(torch, lambda: fn(opts), args.steps, args.warmup)
            info = pmx.parse_info(fn(opts)[-1])[0]
            tinfo = pmx.parse_info(fn(taylor)[-1])[0]
            # one workgroup (one compute unit) runs each call: the matrix-core
            # bound is that CU's share of the fp32 MFMA peak
            fl = int(info["gemms"]) * 2.0 * 64 * (64 if name != "polar_64x32" else 32) ** 2
            tf = fl / (ms * 1e-3) / 1e12
            res[name] = {"us": round(ms * 1e3, 1), "gemms": int(info["gemms"]),
                         "gemms_taylor": int(tinfo["gemms"]),
                         "iters": [int(x) for x in info["iters"]],
                         "roofline": {"bound": "latency (one CU)", "achieved": round(tf, 4),
                                      "peak": round(PEAK_FP32_MFMA / 256, 4), "unit": "TFLOP/s",
                                      "frac": round(tf / (PEAK_FP32_MFMA / 256), 4)}}
        out.update(metric="us per matrix function (n=64)", value=res["inv_root_p4"]["us"],
                   unit="us", dtype="f32", config={"workload": wl}, calls=res)
    elif wl == "model_step":
        # a whole Shampoo step over a synthetic model: four 1024 x 4096 and
        # four 4096 x 1024 dense layers and two 256 x 128 x 3 x 3 convolution
        # kernels, blocks of 1024, gradients N(0, 1e-2) (seed 701); roots
        # every step and every 10 steps (momentum 0.9)
        shapes = [(1024, 4096)] * 4 + [(4096, 1024)] * 4 + [(256, 128, 3, 3)] * 2
        rng = np.random.default_rng(701)
        Ws = [torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(dev) for s in shapes]
        Gs = [torch.from_numpy((0.1 * rng.standard_normal(s)).astype(np.float32)).to(dev)
              for s in shapes]
        res = {}
        for every in (1, 10):
            cfg = pmx.shampoo_config(block=1024, root_every=every, momentum=0.9,
                                     root_opts=pmx.default_opts(max_iter=args.max_iter,
                                                                method=args.method,
                                                                scale_mode=SCALE_MODES[args.scale]))
            plan = pmx.ShampooPlan(shapes, dev, cfg)
            t = [0]

            def one():
                plan.step(Ws, Gs, t[0])
                t[0] += 1
            n_steps = max(args.steps, every)
            ms = timed(torch, one, n_steps, max(args.warmup, 1))
            res["root_every_%d" % every] = round(ms, 3)
            del plan
        params = sum(int(np.prod(s)) for s in shapes)
        out.update(metric="ms per Shampoo step over a 10-layer model (blocks of 1024)",
                   value=res["root_every_1"], unit="ms", dtype="f32",
                   config={"workload": wl, "layers": [list(s) for s in shapes], "block": 1024,
                           "momentum": 0.9, "method": args.method},
                   ms_per_step=res, parameters=params)
    elif wl == "varblocks_4096":
        # 4096 Gaussian blocks with sides uniform in [8, 64] (seed 601), fp32,
        # polar factors in one variable-size call
        Gs = [torch.from_numpy(g).to(dev) for g in W.irregular_blocks(4096, 601)]
        Us = [torch.empty_like(g) for g in Gs]
        info = pmx.new_info(len(Gs), dev)
        ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_POLAR_VARBATCH, 1, 1, len(Gs)), dev)
        # the descriptor table is built once, outside the timed calls
        vb = pmx.VarBlocks(Gs, Us)
        fn = lambda o: pmx.polar_varbatch(blocks=vb, opts=o, info=info, ws=ws)
        ms = timed(torch, lambda: fn(opts), args.steps, args.warmup)
        inf = pmx.parse_info(info)
        flops = sum(2.0 * max(g.shape) * min(g.shape) ** 2 * (2 * int(i) + 1) +
                    2.0 * min(g.shape) ** 3 * int(i) for g, i in zip(Gs, inf["iters"][:, 0]))
        out.update(metric="ms per variable-size batched polar (4096 blocks, sides 8..64)",
                   value=round(ms, 3), unit="ms", dtype="f32", config={"workload": wl},
                   blocks_per_s=round(len(Gs) / (ms * 1e-3), 1),
                   iters_mean=round(float(inf["iters"][:, 0].mean()), 2),
                   status_counts={pmx.STATUS_NAMES[int(k)]: int(v) for k, v in
                                  zip(*np.unique(inf["status"], return_counts=True))},
                   tflops=round(flops / (ms * 1e-3) / 1e12, 2))
    elif wl == "blocks_64x512":
        # fp32 throughout, and with the first four updates of each stage in
        # fp64 (the setting that meets 1e-4 at kappa = 1e6); value is the latter
        c = W.blocks_64x512()
        A = torch.from_numpy(c["A"]).to(dev)
        o64 = pmx.default_opts(max_iter=args.max_iter, fp64_iters=4,
                               scale_mode=SCALE_MODES[args.scale])
        ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, 512, 512, 64, pmx.F32, o64), dev)
        X = torch.empty_like(A)
        info = pmx.new_info(64, dev)
        fn = lambda o: pmx.inv_root(A, 4, opts=o, aux=False, out=X, info=info, ws=ws)
        ms32 = timed(torch, lambda: fn(opts), args.steps, args.warmup)
        inf32 = pmx.parse_info(info)
        gemms = int(inf32["gemms"].sum())
        flops32 = sum(root_exec_flops(512, 64, inf32["iters"][b], inf32["gemms"][b], args.method)
                      for b in range(64))
        ms = timed(torch, lambda: fn(o64), args.steps, args.warmup)
        gemms64 = int(pmx.parse_info(info)["gemms"].sum())
        out["kernel_trace_ms"] = traced(lambda: fn(o64))
        fn(taylor)
        tg = int(pmx.parse_info(info)["gemms"].sum())
        tf = flops32 / (ms32 * 1e-3) / 1e12
        out.update(metric="ms per batched inverse-4th-root (64 x 512)", value=round(ms, 3),
                   unit="ms", dtype="f64 leading 4 updates per stage, then f32",
                   config={"workload": wl, "fp64_iters": 4},
                   fp32_only_ms=round(ms32, 3), gemms_total=gemms64, gemms_total_fp32_only=gemms,
                   gemms_taylor_total=tg, mfma_tflops_fp32_only=round(tf, 2),
                   mfma_frac_fp32_only=round(tf / PEAK_FP32_MFMA, 4))
    elif wl == "muon_32x4096x1024":
        c = inputs if inputs is not None else W.muon_32x4096x1024()
        G = torch.from_numpy(c["G_bits"].view(np.int16)).view(torch.bfloat16).to(dev)
        o = pmx.default_opts(max_iter=args.max_iter, tol=c["tol"], scale_mode=SCALE_MODES[scale])
        ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_POLAR, 4096, 1024, 32, pmx.BF16, o), dev)
        U = torch.empty_like(G)
        info = pmx.new_info(32, dev)
        fn = lambda oo: pmx.polar(G, opts=oo, out=U, info=info, ws=ws)
        ms = timed(torch, lambda: fn(o), args.steps, args.warmup)
        inf = pmx.parse_info(info)
        it = int(inf["iters"][:, 0].max())
        out["kernel_trace_ms"] = traced(lambda: fn(o))
        fn(pmx.default_opts(max_iter=60, tol=c["tol"], accelerate=0, scale_mode=SCALE_MODES[scale]))
        tit = int(pmx.parse_info(info)["iters"][:, 0].max())
        # per update: X^T X (4096 x 1024 x 1024), R^2 (1024^3), X g (4096 x 1024 x 1024)
        flops = 32 * (2.0 * 4096 * 1024 * 1024 * (2 * it + 1) + 2.0 * 1024 ** 3 * it)
        tf = flops / (ms * 1e-3) / 1e12
        out.update(metric="ms per batched polar factor (32 x 4096 x 1024, bf16)",
                   value=round(ms, 3), unit="ms", dtype="bf16", config={"workload": wl},
                   iters=it, iters_taylor=tit, gemms_per_matrix=int(inf["gemms"][0]),
                   mfma_tflops=round(tf, 1), mfma_frac=round(tf / 2516.6, 4))
        # each product on its own, from the traced call: algorithmic flops of
        # the launches that ran (X g and R^2 once per update, I - X^T X once
        # more) over the class's event-to-event time, which also holds the few
        # early-exit launches after convergence
        tr = out["kernel_trace_ms"]
        if tr:
            per = {"gemm_update": (it, 2.0 * 4096 * 1024 * 1024),
                   "gemm_resid": (it + 1, 2.0 * 1024 * 1024 * 4096),
                   "gemm_power": (it, 2.0 * 1024 ** 3)}
            prod = {}
            for k, (cnt, fl) in per.items():
                t = tr.get(k, [0.0, 0])[0]
                if t > 0:
                    pf = 32 * fl * cnt / (t * 1e-3) / 1e15
                    prod[k] = {"pflops": round(pf, 3), "frac": round(pf * 1e3 / 2516.6, 4)}
            out["bf16_products"] = prod
    elif wl == "mp_10000":
        A = W.mp_square_device(device=dev)
        ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, 10000, 10000, 1, pmx.F32, opts), dev)
        X, XA = torch.empty_like(A), torch.empty_like(A)
        info = pmx.new_info(1, dev)
        fn = lambda o: pmx.inv_root(A, 2, opts=o, out=X, out_aux=XA, info=info, ws=ws)
        ms = timed(torch, lambda: fn(opts), args.steps, args.warmup)
        inf = pmx.parse_info(info)[0]
        gemms = int(inf["gemms"])
        out["kernel_trace_ms"] = traced(lambda: fn(opts))
        fn(taylor)
        tg = int(pmx.parse_info(info)[0]["gemms"])
        tf = root_exec_flops(10000, 1, inf["iters"], inf["gemms"], args.method) / (ms * 1e-3) / 1e12
        out.update(metric="ms per square root (n=10^4, A^1/2 and A^-1/2)", value=round(ms, 2),
                   unit="ms", dtype="f32", config={"workload": wl}, gemms=gemms,
                   gemms_taylor=tg, gemm_ratio_taylor_over_prism=round(tg / gemms, 3),
                   iters=int(inf["iters"][0]), mfma_tflops=round(tf, 2),
                   mfma_frac=round(tf / PEAK_FP32_MFMA, 4))
    out["config"]["host_poll"] = args.host_poll
    out["config"]["scale"] = args.scale
    return out


def sweep_sketch(args):
    """Sketch width p in {2, 4, 8, 16} on the 4096 statistics root (R^-1/4 of
    the Shampoo layer after ten updates), the 64 x 512 power-law blocks
    (A^-1/4, fp32) and the 10^4 square root: updates, dense products, skinny
    sketch products, ms and the first stage's alpha trace.  Library scale
    (||A||_F), host polling at chunk 2 (same results as enqueue-ahead)."""
    import torch

    import workloads as W
    from preconditioned_optimizer_matrix_amd import pmx
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pmx.set_host_poll(2)
    cfg = W.shampoo_1024x4096()
    R = torch.from_numpy(cfg["R0"]).to(dev)
    L = torch.from_numpy(cfg["L0"]).to(dev)
    for g in cfg["Gs"]:
        pmx.shampoo_stats_update(torch.from_numpy(g).to(dev), L, R, cfg["beta"], cfg["eps"])
    del L
    blocks = torch.from_numpy(W.blocks_64x512()["A"]).to(dev)
    mp = W.mp_square_device(device=dev)
    cases = (("shampoo_R_4096", R, 4, 1), ("blocks_64x512", blocks, 4, 64),
             ("mp_10000", mp, 2, 1))
    rows = []
    for name, A, root, batch in cases:
        n = A.shape[-1]
        for sp in (2, 4, 8, 16):
            o = pmx.default_opts(sketch_p=sp, max_iter=args.max_iter)
            ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, batch, pmx.F32, o), dev)
            X = torch.empty_like(A)
            info = pmx.new_info(batch, dev)
            fn = lambda: pmx.inv_root(A, root, opts=o, aux=False, out=X, info=info, ws=ws)
            steps = 3 if n >= 10000 else args.steps
            ms = timed(torch, fn, steps, 1)
            inf = pmx.parse_info(info)
            it = inf["iters"]
            row = dict(workload=name, p=sp, ms=round(ms, 3),
                       iters=[int(x) for x in it.max(axis=0)],
                       updates_total=int(it.sum()), gemms_total=int(inf["gemms"].sum()),
                       sketch_products_total=int(inf["sketch_products"].sum()),
                       status=sorted(set(pmx.STATUS_NAMES[int(x)] for x in inf["status"])),
                       alpha_stage1=[round(float(a), 4) for a in inf["alpha"][0][0][:int(it[0][0])]])
            log(json.dumps(row))
            rows.append(row)
            del ws
            torch.cuda.empty_cache()
    print(json.dumps({"sweep": "sketch_p", "host_poll": 2, "scale": "frobenius", "rows": rows}),
          flush=True)


def sweep_sigma(args):
    """Polar factors of 8 fp32 matrices 2048 x 512 with singular values in
    [sigma_min, 1] for sigma_min = 1e-1 .. 1e-5, log-uniform ("geometric") or
    the Marchenko-Pastur shape of a 2048 x 512 Gaussian's singular values
    mapped onto the interval ("mp"): PRISM (fitted alpha) against the Taylor
    coefficient (alpha = c_d), tol 1e-5 on ||I - X^T X||_F / sqrt(n)."""
    import torch

    import workloads as W
    from preconditioned_optimizer_matrix_amd import pmx
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pmx.set_host_poll(2)
    m, n, batch = 2048, 512, 8
    shape = W.mp_shape(m, n, 811)
    rows = []
    for fam in ("geometric", "mp"):
        for k, smin in enumerate((1e-1, 1e-2, 1e-3, 1e-4, 1e-5)):
            sig = np.geomspace(smin, 1.0, n) if fam == "geometric" else smin + (1 - smin) * shape
            G = torch.from_numpy(W.polar_spectrum_batch(batch, m, n, 820 + k, sig)).to(dev)
            row = dict(spectrum=fam, sigma_min=smin)
            for meth, acc in (("prism", 1), ("taylor", 0)):
                o = pmx.default_opts(tol=1e-5, max_iter=100, accelerate=acc)
                ws = pmx.workspace(pmx.workspace_bytes(pmx.OP_POLAR, m, n, batch, pmx.F32, o), dev)
                U = torch.empty_like(G)
                info = pmx.new_info(batch, dev)
                fn = lambda: pmx.polar(G, opts=o, out=U, info=info, ws=ws)
                ms = timed(torch, fn, args.steps, 1)
                inf = pmx.parse_info(info)
                row[meth] = dict(ms=round(ms, 3), iters_max=int(inf["iters"][:, 0].max()),
                                 gemms_per_matrix=int(inf["gemms"].max()),
                                 status=sorted(set(pmx.STATUS_NAMES[int(x)]
                                                   for x in inf["status"])))
            row["gemm_ratio_taylor_over_prism"] = round(
                row["taylor"]["gemms_per_matrix"] / max(row["prism"]["gemms_per_matrix"], 1), 3)
            log(json.dumps(row))
            rows.append(row)
    print(json.dumps({"sweep": "sigma_min", "shape": [batch, m, n], "dtype": "f32",
                      "tol": 1e-5, "rows": rows}), flush=True)


UPDATE_KERNEL = ("gemm_f32_kernel<pmx::(anonymous namespace)::Cfg<128, 128, 16, 2, 2, 3, 2>, "
                 "false, false, 1, 0>")


def write_traffic(dirs):
    """profiles/update_gemm_traffic.json from rocprofv3 counter folders: HBM
    bytes per update product of the n = 4096 update GEMM, summed over the
    first 60 dispatches (the first step's R^-1/4 call without host polling:
    30 updates a stage, early exits included) and divided by that call's
    products (2 k - 1 a stage of k updates, from the profiled run's JSON
    line); each counter scaled by what it reads for the plain 256 MiB copy of
    calibrate_copy()."""
    import csv
    import glob

    def per_dispatch(d, pick):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(f)):
            if pick(r["Kernel_Name"]):
                k = int(r["Dispatch_Id"])
                vals[k] = vals.get(k, 0.0) + float(r["Counter_Value"])
        return [vals[k] for k in sorted(vals)]

    upd = lambda name: UPDATE_KERNEL in name
    cpy = lambda name: "copyBuffer" in name
    n_launch = 60
    fetch = per_dispatch(dirs[0], upd)[:n_launch]
    write = per_dispatch(dirs[1], upd)[:n_launch]
    run = json.loads(open(dirs[4]).read().strip().splitlines()[-1])
    products = sum(2 * int(k) - 1 for k in run["iters"]["R"] if int(k) > 0)
    cf = per_dispatch(dirs[2], cpy)
    cw = per_dispatch(dirs[3], cpy)
    true_kib = 256 * 1024.0
    fs, ws = true_kib / np.mean(cf), true_kib / np.mean(cw)
    f_raw, w_raw = float(np.sum(fetch)), float(np.sum(write))
    rec = {
        "kernel": "gemm_f32_kernel<Cfg<128,128,16,2,2,3>,NN,ROLE_UPDATE> (n=4096 updates of R^-1/4)",
        "source_sha256": source_digest(),
        "source_files": ["preconditioned_optimizer_matrix_amd/csrc/pmx_gemm_f32.hip",
                         "preconditioned_optimizer_matrix_amd/csrc/pmx_api.hip"],
        "dispatches": n_launch,
        "products": products,
        "fetch_kib_raw": round(f_raw, 1),
        "write_kib_raw": round(w_raw, 1),
        "copy_kib_true": true_kib,
        "copy_fetch_kib_raw": round(float(np.mean(cf)), 1),
        "copy_write_kib_raw": round(float(np.mean(cw)), 1),
        "fetch_scale": round(fs, 5),
        "write_scale": round(ws, 5),
        "hbm_bytes_per_product": int(round((f_raw * fs + w_raw * ws) * 1024 / products)),
        "commands": [
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o p -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-trace --no-secondary --host-poll 0 > <json>",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o p -- python3 bench.py --steps 1 --warmup 0 --no-cpu-baseline --no-trace --no-secondary --host-poll 0",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o p -- python3 bench.py --calibrate-copy",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o p -- python3 bench.py --calibrate-copy",
            "python3 bench.py --traffic-from <four dirs> <json>",
        ],
        "reduction": "per counter: sum over the first 60 dispatches of the kernel (the first "
                     "step's R^-1/4 call, early exits included) over that call's update "
                     "products; copy: mean over the 4 __amd_rocclr_copyBuffer dispatches "
                     "of 256 MiB",
    }
    path = os.path.join(ROOT, "profiles", "update_gemm_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec), flush=True)


def calibrate_copy():
    """A plain device copy of known size: 4 launches, each reading and writing
    256 MiB, so FETCH_SIZE / WRITE_SIZE per launch should read 262144 KiB."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": a.numel() * 4, "launches": 4}), flush=True)


def source_digest():
    """SHA-256 over the sources that decide what the update GEMM launches read
    and write: the GEMM kernel and the launch sequence."""
    import hashlib
    h = hashlib.sha256()
    for f in ("pmx_gemm_f32.hip", "pmx_api.hip"):
        h.update(open(os.path.join(ROOT, "preconditioned_optimizer_matrix_amd", "csrc", f),
                      "rb").read())
    return h.hexdigest()


def update_traffic(products, launches):
    """HBM bytes per update-GEMM launch of a call with `products` update
    products in `launches` launches, from the bytes per product measured with
    rocprofv3 counters (profiles/update_gemm_traffic.json; the early exits
    move no matrix data), or None when the GEMM kernel or its launch sequence
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "update_gemm_traffic.json")
    try:
        rec = json.load(open(path))
        digest = source_digest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != digest or "hbm_bytes_per_product" not in rec:
        return None
    return int(round(rec["hbm_bytes_per_product"] * products / max(launches, 1)))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: every GPU box here has one GPU, and the path "
              "has no multi-GPU implementation (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        return calibrate_copy()
    if args.traffic_from:
        return write_traffic(args.traffic_from)
    if args.sweep == "sketch":
        return sweep_sketch(args)
    if args.sweep == "sigma":
        return sweep_sigma(args)
    if args.workload != "shampoo_1024x4096":
        return other_workload(args)
    import torch

    import workloads as W
    from preconditioned_optimizer_matrix_amd import pmx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pmx.set_host_poll(args.host_poll)
    cfg = W.shampoo_1024x4096()
    m, n = cfg["Gs"][0].shape
    beta, eps = cfg["beta"], cfg["eps"]
    Gs = [torch.from_numpy(g).to(dev) for g in cfg["Gs"]]
    L = torch.from_numpy(cfg["L0"]).to(dev)
    R = torch.from_numpy(cfg["R0"]).to(dev)
    for g in Gs[:-1]:
        pmx.shampoo_stats_update(g, L, R, beta, eps)
    L9, R9 = L.clone(), R.clone()
    G = Gs[-1]
    opts = pmx.default_opts(max_iter=args.max_iter, degree=args.degree,
                            degree_max=args.degree_max, method=args.method,
                            scale_mode=SCALE_MODES[args.scale])
    wsL = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, m, m, 1, pmx.F32, opts), dev)
    wsR = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, 1, pmx.F32, opts), dev)
    wsA = pmx.workspace(pmx.workspace_bytes(pmx.OP_APPLY, m, n, 1, pmx.F32, None), dev)
    Li, Ri, P = torch.empty_like(L), torch.empty_like(R), torch.empty_like(G)
    infoL, infoR = pmx.new_info(1, dev), pmx.new_info(1, dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    r_ev = [(ev(), ev()) for _ in range(args.steps)]

    def step(i=None):
        L.copy_(L9)
        R.copy_(R9)
        pmx.shampoo_stats_update(G, L, R, beta, eps)
        pmx.inv_root(L, 4, opts=opts, aux=False, out=Li, info=infoL, ws=wsL)
        if i is not None:
            r_ev[i][0].record()
        pmx.inv_root(R, 4, opts=opts, aux=False, out=Ri, info=infoR, ws=wsR)
        if i is not None:
            r_ev[i][1].record()
        pmx.precond_apply(Li, G, Ri, out=P, ws=wsA)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = ev(), ev()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    r_steps = [a.elapsed_time(b) for a, b in r_ev]
    r_ms = float(np.mean(r_steps))
    iL, iR = pmx.parse_info(infoL)[0], pmx.parse_info(infoR)[0]
    gemmsR, gemmsL = int(iR["gemms"]), int(iL["gemms"])
    tflops_r = root_exec_flops(n, 1, iR["iters"], iR["gemms"], args.method) / (r_ms * 1e-3) / 1e12
    dense_tflops_r = gemmsR * 2.0 * n ** 3 / (r_ms * 1e-3) / 1e12
    log("step %.3f ms, R^-1/4 %.3f ms, gemms R %d L %d, iters R %s L %s, status R %s L %s"
        % (ms_step, r_ms, gemmsR, gemmsL, list(iR["iters"]), list(iL["iters"]),
           pmx.STATUS_NAMES[int(iR["status"])], pmx.STATUS_NAMES[int(iL["status"])]))

    # ablation: the same R^-1/4 with the Taylor coefficient (classical Newton-Schulz)
    infoT = pmx.new_info(1, dev)
    pmx.inv_root(R, 4, opts=pmx.default_opts(max_iter=60, accelerate=0,
                                             scale_mode=SCALE_MODES[args.scale]), aux=False,
                 out=torch.empty_like(R), info=infoT, ws=wsR)
    gemmsR_taylor = int(pmx.parse_info(infoT)[0]["gemms"])

    # property check at full size: || X^4 R e_j - e_j || on sampled columns (fp64)
    cols = torch.arange(0, n, n // 8, device=dev)
    E = torch.zeros(n, len(cols), dtype=torch.float64, device=dev)
    E[cols, torch.arange(len(cols), device=dev)] = 1.0

    def prop_of(Xr):
        V = R.double() @ E
        Xd = Xr.double()
        for _ in range(4):
            V = Xd @ V
        return float((V - E).norm(dim=0).max())

    prop = prop_of(Ri)
    log("max_j ||R^{-1/4}^4 R e_j - e_j|| over 8 sampled columns: %.2e" % prop)

    # the other inverse-root family on the same R: the coupled inverse Newton
    # iteration (method 1), timed the same way
    newton = None
    if args.method == 0:
        oN = pmx.default_opts(max_iter=args.max_iter, method=1,
                              scale_mode=SCALE_MODES[args.scale])
        wsN = pmx.workspace(pmx.workspace_bytes(pmx.OP_INV_ROOT, n, n, 1, pmx.F32, oN), dev)
        infoN = pmx.new_info(1, dev)
        XN = torch.empty_like(R)
        fnN = lambda: pmx.inv_root(R, 4, opts=oN, aux=False, out=XN, info=infoN, ws=wsN)
        msN = timed(torch, fnN, args.steps, args.warmup)
        iN = pmx.parse_info(infoN)[0]
        newton = dict(ms=round(msN, 3), gemms=int(iN["gemms"]), iters=int(iN["iters"][0]),
                      status=pmx.STATUS_NAMES[int(iN["status"])],
                      tflops_launched=round(root_exec_flops(n, 1, iN["iters"], iN["gemms"], 1)
                                            / (msN * 1e-3) / 1e12, 2),
                      property_x4r_minus_i=prop_of(XN))
        log("inverse Newton R^-1/4:", newton)

    # the same R^-1/4 with the other input scale, timed the same way
    other_scale = None
    if args.method == 0:
        alt = "frobenius" if args.scale == "power" else "power"
        oS = pmx.default_opts(max_iter=args.max_iter, degree=args.degree,
                              degree_max=args.degree_max, scale_mode=SCALE_MODES[alt])
        infoS = pmx.new_info(1, dev)
        XS = torch.empty_like(R)
        fnS = lambda: pmx.inv_root(R, 4, opts=oS, aux=False, out=XS, info=infoS, ws=wsR)
        msS = timed(torch, fnS, args.steps, args.warmup)
        iS = pmx.parse_info(infoS)[0]
        other_scale = dict(scale=alt, ms=round(msS, 3), gemms=int(iS["gemms"]),
                           iters=[int(x) for x in iS["iters"]],
                           status=pmx.STATUS_NAMES[int(iS["status"])],
                           property_x4r_minus_i=prop_of(XS))
        log("R^-1/4 with the %s scale:" % alt, other_scale)

    roofline = None
    trace = None
    if not args.no_trace and args.method == 0:
        # one more step with the launch trace: per-class kernel time and
        # launches; the R^-1/4 call is collected on its own for the roofline of
        # its update GEMM (the n = 4096 instantiation, one kernel).
        pmx.trace_enable(True)
        L.copy_(L9)
        R.copy_(R9)
        pmx.shampoo_stats_update(G, L, R, beta, eps)
        pmx.inv_root(L, 4, opts=opts, aux=False, out=Li, info=infoL, ws=wsL)
        tr_pre = pmx.trace_collect()
        pmx.inv_root(R, 4, opts=opts, aux=False, out=Ri, info=infoR, ws=wsR)
        tr_r = pmx.trace_collect()
        pmx.precond_apply(Li, G, Ri, out=P, ws=wsA)
        tr_post = pmx.trace_collect()
        pmx.trace_enable(False)
        trace = {k: (tr_pre[k][0] + tr_r[k][0] + tr_post[k][0],
                     tr_pre[k][1] + tr_r[k][1] + tr_post[k][1]) for k in tr_r}
        t_ms, launches = tr_r["gemm_update"]
        iR2 = pmx.parse_info(infoR)[0]
        # update products of a stage with k iterations: 2 k - 1 (Z_1 = g is formed directly)
        products = sum(2 * int(it) - 1 for it in iR2["iters"] if int(it) > 0)
        flops = products * 2.0 * n ** 3
        avg_ms = t_ms / max(launches, 1)
        achieved = flops / launches / (avg_ms * 1e-3) / 1e12
        roofline = dict(bound="mfma",
                        kernel="gemm_f32_kernel<Cfg<128,128,16,2,2,3>,NN,ROLE_UPDATE> (n=4096)",
                        achieved=round(achieved, 2), peak=PEAK_FP32_MFMA, unit="TFLOP/s",
                        frac=round(achieved / PEAK_FP32_MFMA, 4),
                        traffic=update_traffic(products, int(launches)),
                        launches=int(launches), avg_launch_ms=round(avg_ms, 4),
                        products=products, algorithmic_flops_per_launch=round(flops / launches, 1))
        log("trace:", {k: (round(v[0], 3), v[1]) for k, v in trace.items()})

    # the library's defaults: Frobenius scale, every update enqueued up front
    # (the surplus ones exit on the device), the host never waits
    pmx.set_host_poll(0)
    oD = pmx.default_opts()
    infoD = pmx.new_info(1, dev)
    XD = torch.empty_like(R)
    fnD = lambda: pmx.inv_root(R, 4, opts=oD, aux=False, out=XD, info=infoD, ws=wsR)
    msD = timed(torch, fnD, args.steps, args.warmup)
    iD = pmx.parse_info(infoD)[0]
    lib_default = dict(scale="frobenius", host_poll=0, ms=round(msD, 3), gemms=int(iD["gemms"]),
                       iters=[int(x) for x in iD["iters"]],
                       status=pmx.STATUS_NAMES[int(iD["status"])],
                       mfma_tflops=round(root_exec_flops(n, 1, iD["iters"], iD["gemms"])
                                         / (msD * 1e-3) / 1e12, 2),
                       property_x4r_minus_i=prop_of(XD))
    log("R^-1/4 with the library defaults:", lib_default)
    pmx.set_host_poll(args.host_poll)

    secondary = None
    if not args.no_secondary:
        secondary = {}
        keep = {
            "spd_64": lambda r: {"us": {k: v["us"] for k, v in r["calls"].items()},
                                 "gemms": {k: v["gemms"] for k, v in r["calls"].items()},
                                 "gemms_taylor": {k: v["gemms_taylor"] for k, v in r["calls"].items()},
                                 "roofline": r["calls"]["inv_root_p4"]["roofline"]},
            "blocks_64x512": lambda r: {
                "ms_fp64_leading": r["value"], "ms_fp32_only": r["fp32_only_ms"],
                "gemms_total": r["gemms_total"], "gemms_taylor_total": r["gemms_taylor_total"],
                "roofline": {"bound": "mfma", "achieved": r["mfma_tflops_fp32_only"],
                             "peak": PEAK_FP32_MFMA, "unit": "TFLOP/s",
                             "frac": r["mfma_frac_fp32_only"], "of": "fp32-only call"}},
            "mp_10000": lambda r: {
                "ms": r["value"], "gemms": r["gemms"], "gemms_taylor": r["gemms_taylor"],
                "gemm_ratio_taylor_over_prism": r["gemm_ratio_taylor_over_prism"],
                "iters": r["iters"],
                "roofline": {"bound": "mfma", "achieved": r["mfma_tflops"],
                             "peak": PEAK_FP32_MFMA, "unit": "TFLOP/s", "frac": r["mfma_frac"]}},
            "muon_32x4096x1024": lambda r: {
                "ms": r["value"], "iters": r["iters"], "iters_taylor": r["iters_taylor"],
                "gemms_per_matrix": r["gemms_per_matrix"],
                "roofline": {"bound": "mfma", "achieved": r["mfma_tflops"], "peak": 2516.6,
                             "unit": "TFLOP/s", "frac": r["mfma_frac"], "of": "whole call"},
                "bf16_products": r.get("bf16_products")},
        }
        for wl in ("spd_64", "blocks_64x512", "mp_10000", "muon_32x4096x1024"):
            t0 = time.perf_counter()
            # (the Muon inputs, QR of 64 Gaussians, are built here with the
            # GPU idle: built on a host thread during the other measurements
            # they took the host-polled headline from 28.3 to 28-36 ms a step)
            r = measure(wl, args)
            secondary[wl] = dict(keep[wl](r), metric=r["metric"], unit=r["unit"],
                                 dtype=r["dtype"], host_poll=r["config"]["host_poll"],
                                 scale=r["config"]["scale"])
            log("%s (%.1f s): %s" % (wl, time.perf_counter() - t0, json.dumps(secondary[wl])))
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg["Gs"][-1], L9.cpu().numpy(), R9.cpu().numpy(), beta, eps,
                           updates=sum(int(x) for x in iR["iters"]))
        log("cpu baseline:", cpu)

    out = {
        "metric": METRIC, "value": round(r_ms, 3), "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "shampoo_1024x4096", "m": m, "n": n, "beta": beta, "eps": eps,
                   "warmup_updates": 9, "degree": args.degree,
                   "degree_max": args.degree_max, "method": args.method, "sketch_p": 8,
                   "tol": 1e-6,
                   "max_iter": args.max_iter, "host_poll": args.host_poll,
                   "scale": args.scale,
                   "step": "restore L,R; stats update; L^-1/4; R^-1/4; apply"},
        "r_ms_per_step": [round(x, 3) for x in r_steps],
        "gemms_to_converge": {"R": gemmsR, "L": gemmsL, "R_taylor": gemmsR_taylor},
        "iters": {"R": [int(x) for x in iR["iters"]], "L": [int(x) for x in iL["iters"]]},
        "status": {"R": pmx.STATUS_NAMES[int(iR["status"])],
                   "L": pmx.STATUS_NAMES[int(iL["status"])]},
        "mfma_tflops_r_root": round(tflops_r, 2),
        "mfma_frac_r_root": round(tflops_r / PEAK_FP32_MFMA, 4),
        "dense_equiv_tflops_r_root": round(dense_tflops_r, 2),
        "property_x4r_minus_i": prop,
        "library_default_r_root": lib_default,
        "inverse_newton_r_root": newton,
        "r_root_other_scale": other_scale,
        "secondary": secondary,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if trace is not None:
        out["kernel_trace_ms"] = {k: [round(v[0], 3), v[1]] for k, v in trace.items()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
