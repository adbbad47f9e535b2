"""Benchmark: GPTQ-2D two-sided adaptive rounding of one 4096x4096 4-bit layer on one GPU.

One step = the whole hot path on inputs already resident in HBM: factor A, factor B,
anti-diagonal sweep (gptq2d_quantize).  Prints one JSON line with
  value = quantized weight entries / second (m*n / seconds per layer),
  roofline = the dominant kernel (the persistent sweep) against its MI355X peak: the
             recurrence's flops m n (m + n - 2) over the launch duration from HIP events
             recorded on the launch stream by the library's hook,
  cpu_baseline = the CPU oracle on a bounded sample of the same layer.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"hbm_gbs": 8000.0, "fp32_tflops": 157.3, "fp64_tflops": 78.6}
# Kernel sources whose text the stored HBM-traffic counters belong to.
TRAFFIC_SOURCES = ("two_sided_adaptive_amd/csrc/sweep.hip", "two_sided_adaptive_amd/csrc/common.hpp",
                   "two_sided_adaptive_amd/csrc/schedule.hpp")
METRIC = "quantized weight entries/sec and s/layer, 4096x4096 4-bit GPTQ-2D, 1 MI355X"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload, dtype):
    """HBM bytes per launch of the sweep kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy kernel), or None when the summary
    is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"pmc_sweep_{workload.lower()}_{dtype}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(("#", "|", " ")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """A plain elementwise copy of known size (reads and writes `mib` MiB once each), for
    scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "kernel": "torch.neg (elementwise)", "dispatches": 3}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, W, A, B, s, z_gpu, rows, rows_1core):
    """Oracle (plain fp64 CPU) timed on this host, on the same arrays as the GPU run.

    All cores: both LAPACK factors in full with BLAS on every core, then the C sweep of the
    first `rows` rows (an exact sub-problem: rows only feed rows below them) with one OpenMP
    thread per core.  One core: the same with BLAS and OpenMP pinned to one thread and the
    first `rows_1core` rows.  Each sweep sample is scaled to the whole layer by the sweep's
    multiply-add count, k (n + k) / 2 over rows k < m; the factors are timed in full."""
    import numpy as np
    import oracle
    oracle.build_library(force=False)
    try:
        import threadpoolctl
    except Exception:  # pragma: no cover
        threadpoolctl = None
    ncores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    m, n = W.shape
    work_full = m * n * (m + n) / 2.0

    def timed(threads, r):
        import contextlib
        ctx = (threadpoolctl.threadpool_limits(limits=threads) if threadpoolctl
               else contextlib.nullcontext())
        with ctx:
            t0 = time.perf_counter()
            Ua = oracle.factor_unit_upper(A)
            Ub = oracle.factor_unit_upper(B)
            t1 = time.perf_counter()
            out = oracle.sweep(W[:r], Ua[:r, :r], Ub, s[:r], wl.bits, nthreads=threads)
            t2 = time.perf_counter()
        work = r * n * (r + n) / 2.0
        return t1 - t0, t2 - t1, work_full / work, out

    f_all, s_all, x_all, out = timed(ncores, rows)
    t_all = f_all + s_all * x_all
    agree = float(np.mean(out["Z"] == z_gpu[:rows]))
    f_one, s_one, x_one, out1 = timed(1, rows_1core)
    t_one = f_one + s_one * x_one
    return {
        "value": m * n / t_all, "unit": "entries/s", "cores": int(out["threads"]),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"LAPACK factors of A and B ({m}x{m}, {n}x{n}) in full in {f_all:.2f} s + C "
                   f"sweep of the first {rows} rows in {s_all:.2f} s, both on {out['threads']} "
                   f"threads, the sweep scaled to all {m} rows by its multiply-add count "
                   f"(x{x_all:.1f}): {t_all:.1f} s/layer"),
        "seconds_per_layer": t_all,
        "gpu_code_agreement_on_sample": agree,
        "single_core": {"value": m * n / t_one, "unit": "entries/s", "cores": 1,
                        "seconds_per_layer": t_one,
                        "sample": (f"factors {f_one:.2f} s + sweep of the first {rows_1core} rows "
                                   f"{s_one:.2f} s on one thread, scaled x{x_one:.1f}")},
    }


def kron3_leg(steps, warmup, cpu, peak):
    """Three Kronecker factors on the 16 x 1024 x 1024 tensor K2 (fp64): time per call,
    per-class kernel figures, and the oracle on its first two slabs."""
    import numpy as np
    import torch

    import two_sided_adaptive_amd as g2d
    from synthetic import make3

    wl = make3("K2")
    m1, m2, m3 = wl.W.shape
    dev = torch.device("cuda:0")
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(dev)
         for x in (wl.W, wl.A1, wl.A2, wl.A3, wl.scales)]
    codes = torch.empty((m1, m2, m3), dtype=torch.int8, device=dev)
    Q = torch.empty_like(t[0])
    ws = torch.empty(g2d.load_library().gptq2d_workspace3_bytes(m1, m2, m3, 1),
                     dtype=torch.uint8, device=dev)

    def call(check=False):
        g2d.quantize3(t[0], t[1], t[2], t[3], wl.bits, t[4], check=check, workspace=ws,
                      out=(codes, Q))

    for _ in range(warmup):
        call()
    call(check=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    g2d.profile_enable(True)
    g2d.profile_read()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    prof = g2d.profile_read()
    g2d.profile_enable(False)
    kernels = {}
    for name, (ms, launches, flops, byts) in prof.items():
        if launches == 0 or name == "band_gemm":
            continue
        sec = ms / 1e3
        kernels[name] = {"ms_per_call": ms / steps, "launches_per_call": launches / steps,
                         "avg_launch_us": 1e3 * ms / launches,
                         "tflops": flops / sec / 1e12 if sec > 0 else None,
                         "gbs": byts / sec / 1e9 if sec > 0 else None}
    out = {"workload": f"K2: {m1}x{m2}x{m3} {wl.bits}-bit tensor under A1 (x) A2 (x) A3, fp64",
           "recipe": wl.recipe, "ms_per_call": dt * 1e3, "value": wl.W.size / dt,
           "unit": "entries/s", "kernels": kernels}
    sw, fb = kernels.get("sweep"), kernels.get("slab_feedback")
    if sw and sw["tflops"]:
        # algorithmic flops of the three-factor definition: every slab's two-sided sweep,
        # m2 m3 (m2 + m3), plus the mode-1 feedback, 2 m2 m3 per earlier slab.  The stacked
        # route's sweep runs the (m1 m2) x m3 problem, whose U1' (x) U2' products are mostly
        # zero or repeated: its counted rate is reported beside it as executed flops.
        algo = m1 * m2 * m3 * (m2 + m3) + m1 * (m1 - 1) * m2 * m3
        ach = algo / (sw["ms_per_call"] * 1e-3) / 1e12
        out["roofline_sweep"] = {"bound": "mfma", "achieved": ach,
                                 "peak": peak["fp64_tflops"], "unit": "TFLOP/s",
                                 "frac": ach / peak["fp64_tflops"],
                                 "algorithmic_flops": algo,
                                 "executed_tflops": sw["tflops"]}
    if fb and fb["gbs"]:
        out["roofline_slab_feedback"] = {"bound": "hbm", "achieved": fb["gbs"],
                                         "peak": peak["hbm_gbs"], "unit": "GB/s",
                                         "frac": fb["gbs"] / peak["hbm_gbs"]}
    if cpu:
        import oracle
        oracle.build_library(force=False)
        k = 2
        t0 = time.perf_counter()
        U1, U2, U3 = (oracle.factor_unit_upper(a) for a in (wl.A1, wl.A2, wl.A3))
        t1 = time.perf_counter()
        # the first k slabs are an exact sub-problem (slabs only feed later slabs), with the
        # leading k x k block of the full U1'
        ref = oracle.quantize3_factored(wl.W[:k], U1[:k, :k], U2, U3, wl.scales[:k], wl.bits)
        t2 = time.perf_counter()
        t_full = (t1 - t0) + (t2 - t1) * m1 / k
        out["cpu_baseline"] = {
            "value": wl.W.size / t_full, "unit": "entries/s", "kind": "oracle",
            "sample": f"LAPACK factors of A1, A2, A3 in {t1 - t0:.2f} s + nested sweep of the "
                      f"first {k} slabs in {t2 - t1:.2f} s, scaled by {m1 // k} to {m1} slabs: "
                      f"est. {t_full:.1f} s/tensor",
            "gpu_code_agreement_on_sample": float(
                np.mean(ref["Z"] == codes[:k].cpu().numpy().astype(np.int32)))}
    return out


def packed_leg(codes, scales, bits, reps, peak):
    """Packed storage of the layer's codes: pack, unpack to Q, and a batch-1 and batch-8
    GEMV on the packed rows, each timed with the library's event hook over `reps` calls."""
    import torch

    import two_sided_adaptive_amd as g2d

    rows, n = codes.shape
    dev = codes.device
    P = g2d.pack(codes, bits)
    X8 = torch.randn((8, n), dtype=scales.dtype, device=dev,
                     generator=torch.Generator(device=dev).manual_seed(11))
    Y = torch.empty((8, rows), dtype=scales.dtype, device=dev)
    out = {"workload": f"{rows}x{n} {bits}-bit codes of the layer, {scales.dtype}",
           "packed_bytes": int(P.numel() * 4)}
    calls = {"pack": lambda: g2d.pack(codes, bits),
             "unpack": lambda: g2d.unpack(P, n, bits, scales),
             "gemv_b1": lambda: g2d.packed_gemv(P, n, bits, scales, X8[:1], out=Y[:1]),
             "gemv_b8": lambda: g2d.packed_gemv(P, n, bits, scales, X8, out=Y)}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        g2d.profile_enable(True)
        g2d.profile_read()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        ms, launches, fl, by = g2d.profile_read()["packed"]
        g2d.profile_enable(False)
        us = 1e3 * ms / launches
        gbs = by / launches / (us * 1e-6) / 1e9
        out[name] = {"avg_launch_us": us, "bytes_per_launch": by / launches,
                     "roofline": {"bound": "hbm", "achieved": gbs, "peak": peak["hbm_gbs"],
                                  "unit": "GB/s", "frac": gbs / peak["hbm_gbs"]}}
    return out


def gram_leg(reps, peak):
    """Kronecker factor accumulation A += X^T X / N at the layer's width (p = 4096) from
    N = 8192 synthetic activation samples, fp64, timed with the event hook."""
    import torch

    import two_sided_adaptive_amd as g2d

    p, N = 4096, 8192
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(12)
    X = torch.randn((N, p), dtype=torch.float64, device=dev, generator=gen)
    A = torch.zeros((p, p), dtype=torch.float64, device=dev)
    g2d.gram_accumulate(A, X, 1.0 / N)
    torch.cuda.synchronize()
    g2d.profile_enable(True)
    g2d.profile_read()
    for _ in range(reps):
        g2d.gram_accumulate(A, X, 1.0 / N)
    torch.cuda.synchronize()
    ms, launches, fl, by = g2d.profile_read()["gram"]
    g2d.profile_enable(False)
    sec = ms / 1e3 / launches
    tf = fl / launches / sec / 1e12
    return {"workload": f"A += X^T X / N, p={p}, N={N} samples, fp64",
            "ms_per_call": sec * 1e3, "flops_per_call": fl / launches,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": peak["fp64_tflops"],
                         "unit": "TFLOP/s", "frac": tf / peak["fp64_tflops"]}}


def _fp32_factor(A):
    """U' of an SPD matrix with every step in fp32 on the device (torch: Cholesky of the
    index-reversed matrix, triangular inverse, unit rows): the alternative factor of the
    precision study (measurement only; the library's factor stage is fp64)."""
    import torch
    a = torch.flip(A.float(), dims=(0, 1))
    L = torch.linalg.cholesky(a)
    X = torch.linalg.solve_triangular(L, torch.eye(L.shape[0], dtype=L.dtype, device=L.device),
                                      upper=False)
    U = torch.flip(X, dims=(0, 1))
    return (U / torch.diagonal(U)[:, None]).contiguous()


def precision_leg():
    """Finite-precision study: the fp32 sweep against the exact fp64 one (both with fp64
    factors), and the exact fp64 sweep with fp32-computed factors, on 1024-wide layers of
    two metric families: U diag(k^-1.5) U^T + damp I (condition number about 1/damp), and
    Wishart matrices of 1024 samples with the 14336- and 8192-wide layers' k^-1 and k^-1.2
    spectra plus damping.  Reports the share of codes equal to the exact ones and the
    relative change of the objective tr(A E B E^T) (evaluated in fp64 with torch:
    measurement only)."""
    import numpy as np
    import torch

    import two_sided_adaptive_amd as g2d
    from synthetic import make_conditioned, make_powerlaw

    dev = torch.device("cuda:0")

    def study(wls, label):
        eq, rel, kap, eqf, relf = [], [], [], [], []
        for wl in wls:
            W, A, B, s = (torch.from_numpy(np.ascontiguousarray(x)).to(dev)
                          for x in (wl.W, wl.A, wl.B, wl.scales))
            z64, _ = g2d.quantize(W, A, B, wl.bits, s)
            z32, _ = g2d.quantize(W.float(), A.float(), B.float(), wl.bits, s.float())
            zf, _ = g2d.quantize_factored(W, _fp32_factor(A).double(), _fp32_factor(B).double(),
                                          wl.bits, s)

            def obj(z):
                E = W - s[:, None] * z.to(torch.float64)
                return float(torch.sum((A @ E) * (E @ B)).item())

            f64 = obj(z64)
            ev = torch.linalg.eigvalsh(A)
            kap.append(float((ev.max() / ev.min()).item()))
            eq.append(float((z64 == z32).float().mean().item()))
            rel.append((obj(z32) - f64) / f64)
            eqf.append(float((z64 == zf).float().mean().item()))
            relf.append((obj(zf) - f64) / f64)
        return {"metric": label, "kappa_A": float(np.mean(kap)), "seeds": len(wls),
                "fp32_sweep": {"codes_equal_mean": float(np.mean(eq)),
                               "codes_equal_min": float(min(eq)),
                               "seeds_departed": int(sum(e < 1.0 for e in eq)),
                               "objective_rel_change_max": float(max(rel, key=abs))},
                "fp32_factor": {"codes_equal_mean": float(np.mean(eqf)),
                                "codes_equal_min": float(min(eqf)),
                                "seeds_departed": int(sum(e < 1.0 for e in eqf)),
                                "objective_rel_change_max": float(max(relf, key=abs))}}

    rows = []
    for damp in (1e-1, 1e-2, 1e-3, 1e-4):
        wls = [make_conditioned(1024, damp, seed=10 * int(round(-np.log10(damp))) + k)
               for k in range(3)]
        rows.append(dict(study(wls, f"U diag(k^-1.5) U^T + {damp:g} I"), damp=damp))
    for power in (1.0, 1.2):
        for damp in (1e-2, 1e-3):
            wls = [make_powerlaw(1024, power, damp, bits=4 if power == 1.0 else 3,
                                 seed=100 * int(power * 10) + 10 * int(round(-np.log10(damp))) + k)
                   for k in range(3)]
            rows.append(dict(study(wls, f"Wishart of 1024 samples, k^-{power:g} spectrum + "
                                        f"{damp:g} damping"), damp=damp, power=power))
    return {"workload": "1024x1024 layers (4-bit; 3-bit for the k^-1.2 family)", "rows": rows}


def kernel_table(prof, steps):
    """Per kernel class from the event hook (launches timed with HIP events on their
    stream).  The band-update tasks are not kernels and are reported by task_table."""
    kernels = {}
    for name, (ms, launches, flops, byts) in prof.items():
        if launches == 0 or name == "band_gemm":
            continue
        sec = ms / 1e3
        kernels[name] = {
            "ms_per_step": ms / steps, "launches_per_step": launches / steps,
            "avg_launch_us": 1e3 * ms / launches,
            "tflops": flops / sec / 1e12 if sec > 0 else None,
            "gbs": byts / sec / 1e9 if sec > 0 else None,
            "bytes_per_launch": byts / launches, "flops_per_launch": flops / launches,
        }
    return kernels


def task_table(classes, steps, ncu, dtype):
    """Band-update tasks inside the sweep kernel, by task class, from the kernel's own
    accounting while the hook is on: the summed busy wall-clock time of the workgroups that
    ran them (CU-milliseconds, not kernel time) and their dense GEMM flops.  The rate is
    per busy CU, against one CU's share of the MFMA peak of the dtype."""
    peak_cu = (PEAK["fp32_tflops"] if dtype == "f32" else PEAK["fp64_tflops"]) / ncu
    out = {"what": "band-update GEMM tasks inside k_sweep; cu_ms = summed busy time of the "
                   "workgroups running them (CU-milliseconds), not a kernel duration",
           "peak_tflops_per_cu": peak_cu}
    tot_ms = tot_fl = 0.0
    tot_n = 0
    for name, (cu_ms, n, fl) in classes.items():
        tot_ms += cu_ms
        tot_fl += fl
        tot_n += n
        if n == 0:
            continue
        rate = fl / (cu_ms / 1e3) / 1e12 if cu_ms > 0 else None
        out[name] = {"cu_ms_per_step": cu_ms / steps, "tasks_per_step": n / steps,
                     "us_per_task": 1e3 * cu_ms / n, "flops_per_task": fl / n,
                     "tflops_per_busy_cu": rate,
                     "frac_of_cu_peak": rate / peak_cu if rate is not None else None}
    if tot_ms > 0:
        rate = tot_fl / (tot_ms / 1e3) / 1e12
        out["all"] = {"cu_ms_per_step": tot_ms / steps, "tasks_per_step": tot_n / steps,
                      "tflops_per_busy_cu": rate, "frac_of_cu_peak": rate / peak_cu}
    return out


def configs_leg(names, steps, warmup, ncu):
    """Every layer of the workload list, both sweep dtypes: seconds per layer (whole call,
    inputs resident), the sweep and factor kernels from the event hook, and the fp32 codes'
    agreement with the exact fp64 codes (those equal the oracle's: tests/test_gpu_large.py)."""
    import numpy as np
    import torch

    import two_sided_adaptive_amd as g2d
    from synthetic import make

    dev = torch.device("cuda:0")
    out = {}
    for name in names:
        t0 = time.perf_counter()
        wl = make(name)
        gen = time.perf_counter() - t0
        rec = {"m": wl.m, "n": wl.n, "bits": wl.bits, "recipe": wl.recipe,
               "generated_s": gen}
        z64 = None
        for dt in ("f64", "f32"):
            tW, tA, tB, ts = (torch.from_numpy(np.array(x)).to(dev) for x in wl.cast(dt))
            codes = torch.empty((wl.m, wl.n), dtype=torch.int8, device=dev)
            Q = torch.empty_like(tW)
            ws = torch.empty(g2d.workspace_bytes(wl.m, wl.n, tW.dtype), dtype=torch.uint8,
                             device=dev)

            def call(check=False):
                g2d.quantize(tW, tA, tB, wl.bits, ts, check=check, workspace=ws, out=(codes, Q))

            call(check=True)
            for _ in range(max(0, warmup - 1)):
                call()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / steps
            g2d.profile_enable(True)
            g2d.profile_read()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            prof = g2d.profile_read()
            g2d.profile_enable(False)
            ks = kernel_table(prof, steps)
            peak = PEAK["fp32_tflops"] if dt == "f32" else PEAK["fp64_tflops"]
            r = {"ms_per_layer": sec * 1e3, "entries_per_s": wl.m * wl.n / sec}
            if "sweep" in ks:
                r["sweep_ms"] = ks["sweep"]["ms_per_step"]
                r["sweep_tflops"] = ks["sweep"]["tflops"]
                r["sweep_frac_of_mfma_peak"] = ks["sweep"]["tflops"] / peak
            if "factor" in ks:
                r["factor_ms"] = ks["factor"]["ms_per_step"]
                r["factor_tflops"] = ks["factor"]["tflops"]
            bt = task_table(g2d.profile_task_classes(), steps, ncu, dt).get("all")
            if bt:
                r["band_update_tflops_per_busy_cu"] = bt["tflops_per_busy_cu"]
                r["band_update_frac_of_cu_peak"] = bt["frac_of_cu_peak"]
            z = codes.cpu().numpy()
            if dt == "f64":
                z64 = z
            else:
                r["codes_equal_to_f64"] = float(np.mean(z == z64))
            rec[dt] = r
            log(f"[bench] {name} {dt}: {sec * 1e3:.2f} ms/layer")
            del tW, tA, tB, ts, codes, Q, ws
            torch.cuda.empty_cache()
        out[name] = rec
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C3")
    ap.add_argument("--dtype", default="f64", choices=["f32", "f64"],
                    help="sweep arithmetic: f64 reproduces the oracle exactly (default); "
                         "f32 is faster but its trajectory departs after fp32 near-ties")
    ap.add_argument("--no-alt", action="store_true", help="skip timing the other sweep dtype")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="rows of the oracle's all-core sweep sample")
    ap.add_argument("--cpu-rows-1core", type=int, default=96,
                    help="rows of the oracle's one-core sweep sample")
    ap.add_argument("--configs", default="C1,C2,C3,C4,C4T,C5",
                    help="layers timed (both dtypes) for the per-layer table; '' for none")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-precision", action="store_true",
                    help="skip the precision study (its 1024-wide sweeps would mix into a "
                         "profile of the headline sweep)")
    ap.add_argument("--no-kron3", action="store_true",
                    help="skip the three-factor tensor leg (K2, 16x1024x1024)")
    ap.add_argument("--kron3-only", action="store_true",
                    help="run only the three-factor leg and print its JSON object")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the layer is a single-GPU problem and no "
              "multi-GPU path is built (layers would be spread over GPUs independently).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import two_sided_adaptive_amd as g2d
    from synthetic import make

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    g2d.load_library()
    if args.kron3_only:
        print(json.dumps(kron3_leg(args.steps, args.warmup, not args.no_cpu_baseline, PEAK)),
              flush=True)
        return
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    wl = make(args.workload, cache_dir=os.environ.get("GPTQ2D_CACHE"))
    W, A, B, s = wl.cast(args.dtype)
    log(f"[bench] workload {wl.name} {wl.m}x{wl.n} {wl.bits}-bit {args.dtype} generated in "
        f"{time.perf_counter() - t0:.1f} s")
    tW, tA, tB, ts = (torch.from_numpy(x).to(dev) for x in (W, A, B, s))
    m, n = wl.m, wl.n
    codes = torch.empty((m, n), dtype=torch.int8, device=dev)
    Q = torch.empty_like(tW)
    ws = torch.empty(g2d.workspace_bytes(m, n, tW.dtype), dtype=torch.uint8, device=dev)

    def step():
        g2d.quantize(tW, tA, tB, wl.bits, ts, check=False, workspace=ws, out=(codes, Q))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    log(f"[bench] timed {args.steps} steps: {dt * 1e3:.2f} ms/step")
    # validity of the last result
    g2d.quantize(tW, tA, tB, wl.bits, ts, check=True, workspace=ws, out=(codes, Q))

    # per-kernel durations: the same K steps again with the library's event hook on
    g2d.profile_enable(True)
    g2d.profile_read()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = g2d.profile_read()
    g2d.profile_enable(False)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    kernels = kernel_table(prof, args.steps)
    tasks = task_table(g2d.profile_task_classes(), args.steps, ncu, args.dtype)
    log("[bench] per-kernel: " + json.dumps(kernels))
    gemm_peak = PEAK["fp32_tflops"] if args.dtype == "f32" else PEAK["fp64_tflops"]
    dominant = max((k for k in kernels if k != "other"), key=lambda k: kernels[k]["ms_per_step"])

    def roof(name):
        k = kernels[name]
        if name == "sweep":
            # the whole sweep kernel: algorithmic flops of the recurrence per launch over
            # the launch's event-timed duration, against the MFMA peak of its dtype
            return {"kernel": name, "bound": "mfma", "achieved": k["tflops"], "peak": gemm_peak,
                    "unit": "TFLOP/s", "frac": k["tflops"] / gemm_peak,
                    "traffic": stored_traffic(wl.name, args.dtype),
                    "algorithmic_flops_per_launch": k["flops_per_launch"],
                    "algorithmic_bytes_per_launch": k["bytes_per_launch"]}
        return {"kernel": name, "bound": "mfma", "achieved": k["tflops"],
                "peak": PEAK["fp64_tflops"], "unit": "TFLOP/s",
                "frac": k["tflops"] / PEAK["fp64_tflops"], "traffic": None}

    z_gpu = codes.cpu().numpy().astype(np.int32)
    alt = None
    # the headline's codes are compared with the oracle on the CPU-baseline sample below
    # (gpu_code_agreement_on_sample); the full-size parity tests compare every code
    if not args.no_alt:
        adt = "f32" if args.dtype == "f64" else "f64"
        aW, aA, aB, a_s = (torch.from_numpy(np.array(x)).to(dev) for x in wl.cast(adt))
        acodes = torch.empty((m, n), dtype=torch.int8, device=dev)
        aQ = torch.empty_like(aW)
        aws = torch.empty(g2d.workspace_bytes(m, n, aW.dtype), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            g2d.quantize(aW, aA, aB, wl.bits, a_s, check=False, workspace=aws, out=(acodes, aQ))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g2d.quantize(aW, aA, aB, wl.bits, a_s, check=False, workspace=aws, out=(acodes, aQ))
        torch.cuda.synchronize()
        adt_s = (time.perf_counter() - t0) / args.steps
        alt = {"dtype": adt, "ms_per_step": adt_s * 1e3, "value": m * n / adt_s,
               "codes_equal_to_headline": float((acodes == codes).float().mean().item())}
        # the same steps with the event hook on: the sweep kernel and the band-update tasks
        # of this dtype against its own MFMA peak
        g2d.profile_enable(True)
        g2d.profile_read()
        for _ in range(args.steps):
            g2d.quantize(aW, aA, aB, wl.bits, a_s, check=False, workspace=aws, out=(acodes, aQ))
        torch.cuda.synchronize()
        aprof = g2d.profile_read()
        g2d.profile_enable(False)
        sw = aprof.get("sweep")
        if sw is not None and sw[1] > 0 and sw[0] > 0:
            alt["sweep_ms_per_launch"] = sw[0] / sw[1]
            alt["sweep_tflops"] = sw[2] / (sw[0] / 1e3) / 1e12
        alt["band_update_tasks"] = task_table(g2d.profile_task_classes(), args.steps, ncu, adt)
        log(f"[bench] {adt} sweep: {adt_s * 1e3:.2f} ms/step")
        del aW, aA, aB, a_s, acodes, aQ, aws
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle factors + the first {args.cpu_rows} rows "
            f"(all cores), {args.cpu_rows_1core} rows (one core)")
        cpu = cpu_baseline(wl, W.astype(np.float64), A.astype(np.float64),
                           B.astype(np.float64), s.astype(np.float64), z_gpu, args.cpu_rows,
                           args.cpu_rows_1core)
    log("[bench] packed codes leg")
    pk = packed_leg(codes, ts, wl.bits, 50, PEAK)
    log("[bench] factor accumulation leg")
    gr = gram_leg(5, PEAK)
    prec = None
    if not args.no_precision:
        log("[bench] precision study leg")
        prec = precision_leg()
    cfg = None
    if args.configs:
        log("[bench] per-layer table: " + args.configs)
        cfg = configs_leg([c for c in args.configs.split(",") if c], 3, 1, ncu)
    k3 = None
    if not args.no_kron3:
        log("[bench] three-factor leg (K2)")
        k3 = kron3_leg(max(1, min(args.steps, 5)), 1, not args.no_cpu_baseline, PEAK)
    out = {
        "metric": METRIC, "value": m * n / dt, "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": dt * 1e3,
        "s_per_layer": dt, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.m}x{wl.n} {wl.bits}-bit GPTQ-2D layer, "
                               f"{args.dtype} sweep, fp64 factor", "m": m, "n": n,
                   "bits": wl.bits, "recipe": wl.recipe},
        "roofline": roof(dominant),
        "rooflines": [roof(k) for k in sorted(kernels, key=lambda k: -kernels[k]["ms_per_step"])
                      if k != "other"],
        "kernels": kernels,
        "band_update_tasks": tasks,
        "configs": cfg,
        "cpu_baseline": cpu,
        "other_dtype": alt,
        "kron3": k3,
        "packed": pk,
        "gram": gr,
        "precision": prec,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
