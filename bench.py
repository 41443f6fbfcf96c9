"""Benchmark of the TensorGRaD optimizer step on one MI355X.

Workload: the bf16 3-D FNO spectral-weight gradient of shape (64, 64, 48, 48, 25)
(235,929,600 elements), Tucker ranks (32, 32, 24, 24, 13), 5% top-k sparse part
(11,796,480 COO entries), Adam lr 1e-3, betas (0.9, 0.999), eps 1e-8, refresh every
T = 200 steps; synthetic seeded inputs (Tucker low-rank signal + N(0, 0.01) noise + 1%
Laplace(5) outliers, see synth/gen.py).

A timed step is one tgrad_step on a fresh gradient buffer already resident in HBM
(every buffer is staged before timing starts, so no step re-reads a gradient another
step has left in the caches; the step only reads its gradient). The refresh (top-k + Gram + eigensolver) runs before step 1 during warm-up
and is timed on its own with tgrad_refresh. Per-kernel durations come from HIP events
that the library records on the launch stream around every launch in the timed region.

Beside the headline it reports, in "multi_tensor", the 4-layer fp16 (64,64,64,64)
workload stepped layer after layer and as one tgrad_step_many call.

Prints ONE JSON line. --gpus N with N > 1 exits: the step is measured on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_MFMA_PEAK_TFS = 157.3     # MI355X dense fp32 matrix


def esize(dtype):
    return {"f32": 4, "f16": 2, "bf16": 2, "c64": 8}[dtype]


def unfused_step_bytes(wl):
    """The step's algorithmic bytes with one launch per kernel of the path and fp32
    intermediates, no fusion (the whole-step roofline's definition): the COO gather (k
    indices, k values read, k fp32 values written, k zeros written), one mode product per
    compressed mode in each chain (input read once, output written once), Adam over core
    and sparse values (24 B a value), and the last reconstruction's weight update (W read
    and written, the k indices and k sparse updates read)."""
    P = 2 if wl.dtype == "c64" else 1
    es = esize(wl.dtype)
    N, k = wl.numel, wl.k
    fmodes = [n for n, (I, r) in enumerate(zip(wl.shape, wl.ranks)) if r < I]
    cur = list(wl.shape)
    size, total = N, 0
    for j, n in enumerate(reversed(fmodes)):
        out = size // cur[n] * wl.ranks[n]
        total += size * P * (es if j == 0 else 4) + out * P * 4
        cur[n] = wl.ranks[n]
        size = out
    ncore = size
    for j, n in enumerate(fmodes):
        out = size // cur[n] * wl.shape[n]
        total += size * P * 4
        total += (2 * N * es + k * 4 + k * P * 4) if j + 1 == len(fmodes) else out * P * 4
        cur[n] = wl.shape[n]
        size = out
    gather = k * (4 + es + 4 * P + es) if k else 0
    return total + gather + (ncore + k) * P * 24, ncore


def by_kernel(launches):
    """{kernel name: (launches, bytes read + written, flops)} from a launch record."""
    out = {}
    for name, _modes, br, bw, fl in launches:
        n, b, f = out.get(name, (0, 0, 0))
        out[name] = (n + 1, b + br + bw, f + fl)
    return out


def counter_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (scaled by the plain-copy calibration), or None when the kernel's
    source has changed since the counters were taken."""
    import glob
    import hashlib
    for f in glob.glob(os.path.join(ROOT, "profiles", "counters_*.json")):
        with open(f) as fh:
            rec = json.load(fh)
        if rec.get("kernel") != kernel:
            continue
        src = os.path.join(ROOT, rec["source"])
        if not os.path.exists(src):
            return None
        with open(src, "rb") as fh:
            sha = hashlib.sha256(fh.read()).hexdigest()
        return rec["traffic_bytes"] if sha.startswith(rec["source_sha256_prefix"]) else None
    return None


def multi_tensor(dev, stream, steps=10, warmup=3):
    """The 4-layer fp16 (64,64,64,64) workload: one optimizer step of all four layers,
    issued layer after layer with tgrad_step on one stream, and as one tgrad_step_many
    call (the layers' kernels overlap on internal streams). Milliseconds per 4-layer
    step, after the warm-up steps (step 1 refreshes every layer)."""
    import torch
    import tensor_gradient_compression_amd as tg
    from synth import (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, BF16_64x64x48x48x25,
                   GradStream, init_weights)
    wl = F16_4x64x64x64x64
    L = wl.layers
    out = {"workload": f"fp16 {L} x (64,64,64,64), Tucker ranks (32,32,32,32), 5% sparse"}
    for mode in ("sequential", "step_many"):
        libs = [tg.TGrad(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, wl.betas,
                         wl.eps) for _ in range(L)]
        G = [tg.to_device(GradStream(wl, seed=0, layer=l).next(), wl.dtype, dev) for l in range(L)]
        W = [tg.to_device(init_weights(wl, seed=0, layer=l), wl.dtype, dev) for l in range(L)]

        def one():
            if mode == "sequential":
                for l in range(L):
                    libs[l].step(W[l], G[l], stream)
            else:
                tg.step_many(libs, W, G, stream)
        for _ in range(warmup):
            one()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            one()
        torch.cuda.synchronize()
        out[mode + "_ms"] = round((time.perf_counter() - t0) * 1e3 / steps, 4)
        for lib in libs:
            lib.close()
        del G, W
    return out


def cpu_baseline(wl, seed=0):
    """The oracle (numpy, fp64 contractions) timed on this host on bounded samples:
    * one non-refresh step of the full workload on all available cores, with Omega a
      seeded random index set of size k and seeded random orthonormal factors (the
      step's cost does not depend on which indices or which subspace it uses) -- the
      reported value;
    * the same step with numpy's BLAS held to one thread, on the first 8 of the 64
      leading indices (1/8 of the elements, ranks capped at the slice's sizes);
    * one refresh (top-k by a full sort of the keys, five fp64 Grams, eigh) on the first
      4 leading indices (1/16 of the elements), all cores.
    Each figure is scaled to gradient elements per second of its own sample."""
    import oracle as O
    from synth import GradStream, init_weights
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:
        threadpool_limits = None
    g = GradStream(wl, seed=seed).next()
    W = init_weights(wl, seed=seed)

    def timed_step(shape, gs, Ws):
        ranks = tuple(min(r, I) for I, r in zip(shape, wl.ranks))
        n = int(np.prod(shape, dtype=np.int64))
        k = int(np.floor(wl.sparse_ratio * n))
        orc = O.TGradOracle(shape, ranks, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, *wl.betas, wl.eps)
        rng = np.random.default_rng(seed + 99)
        orc.omega = np.sort(rng.choice(n, k, replace=False)).astype(np.uint32)
        orc.factors = [np.linalg.qr(rng.standard_normal((I, r)))[0].astype(np.float32) if r < I else None
                       for I, r in zip(shape, ranks)]
        orc.t = 1
        orc.refreshed_for = 2
        t0 = time.perf_counter()
        orc.step(np.ascontiguousarray(Ws), np.ascontiguousarray(gs))
        return n, time.perf_counter() - t0

    n_all, dt = timed_step(wl.shape, g, W)
    one = None
    if threadpool_limits is not None:
        sl = (8,) + tuple(wl.shape[1:])
        with threadpool_limits(limits=1):
            n1, dt1 = timed_step(sl, g[:8], W[:8])
        one = {"value": n1 / dt1, "unit": "grad elems/s", "cores": 1, "seconds": dt1,
               "sample": f"1 non-refresh step on the first 8 leading indices {sl} ({n1} elements), "
                         f"numpy BLAS held to one thread"}
    sr = (4,) + tuple(wl.shape[1:])
    ranks_r = tuple(min(r, I) for I, r in zip(sr, wl.ranks))
    orc = O.TGradOracle(sr, ranks_r, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, *wl.betas, wl.eps)
    gr = np.ascontiguousarray(g[:4])
    t0 = time.perf_counter()
    orc.refresh(gr, 1)
    dtr = time.perf_counter() - t0
    nr = int(np.prod(sr, dtype=np.int64))
    refresh = {"value": nr / dtr, "unit": "grad elems/s", "seconds": dtr,
               "sample": f"1 refresh (sort-based top-k, fp64 Grams, eigh) on the first 4 leading "
                         f"indices {sr} ({nr} elements), all cores"}
    threads = len(os.sched_getaffinity(0))
    cpu_model, blas = None, None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"].get("name")
    except Exception:
        pass
    return {"value": n_all / dt, "unit": "grad elems/s", "cores": threads, "kind": "oracle",
            "sample": f"1 non-refresh step of the full workload ({n_all} elements), "
                      f"{dt:.1f} s; numpy BLAS threads = available cores",
            "seconds": dt, "one_thread": one, "refresh": refresh,
            "cpu_model": cpu_model, "blas": blas}


def kernel_table(timed, work, reps):
    """Per kernel: launches, ms, and from the launch record its algorithmic bytes, flops,
    achieved GB/s and TFLOP/s (bytes and flops of all its launches in one step or refresh
    over their total time)."""
    out = {}
    for name, (n, ms) in timed.items():
        per = n // reps if n % reps == 0 else n / reps
        entry = {"launches": per, "avg_ms": round(ms / n, 5), "ms": round(ms / reps, 5)}
        if name in work:
            _, byts, fl = work[name]
            t = ms / reps * 1e-3
            entry.update({"alg_bytes": int(byts), "achieved_GBs": round(byts / t / 1e9, 1),
                          "hbm_frac": round(byts / t / 1e9 / HBM_PEAK_GBS, 4)})
            if fl:
                entry.update({"flops": int(fl), "achieved_TFs": round(fl / t / 1e12, 2)})
        out[name] = entry
    return out


def other_configs(dev, stream, steps=10, warmup=3, refresh_reps=3):
    """The other workloads, one tensor each: ms per step (K steps, no events inside), the
    per-kernel table (K more steps with an event pair around every launch, bytes and
    flops from the launch record), and the refresh alone (median of refresh_reps) with
    its per-kernel table."""
    import torch
    import tensor_gradient_compression_amd as tg
    from synth import F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, GradStream, init_weights
    out = {}
    for key, wl, desc in (
            ("fp16_64x64x64x64", F16_4x64x64x64x64,
             "fp16 (64,64,64,64), Tucker ranks (32,32,32,32), 5% sparse (one of the 4 layers)"),
            ("c64_64x64x64x33", C64_64x64x64x33,
             "complex64 (64,64,64,33), Tucker ranks (32,32,32,16), 5% sparse"),
            ("fp32_32x32x16x16", F32_32x32x16x16,
             "fp32 (32,32,16,16), Tucker ranks (16,16,8,8), 5% sparse")):
        # refresh period beyond the run: the steps timed are plain steps (step 1 refreshes)
        lib = tg.TGrad(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, 10 ** 6, wl.lr, wl.betas,
                       wl.eps)
        gs = GradStream(wl, seed=0)
        G = [tg.to_device(gs.next(), wl.dtype, dev) for _ in range(2)]
        W = tg.to_device(init_weights(wl, seed=0), wl.dtype, dev)
        for i in range(warmup):
            lib.step(W, G[i % 2], stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            lib.step(W, G[i % 2], stream)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        lib.timing_enable(True, 100000)
        for i in range(steps):
            lib.step(W, G[i % 2], stream)
        rec = lib.timing_read()
        kb = by_kernel(lib.last_launches())
        rt = []
        for _ in range(refresh_reps):
            torch.cuda.synchronize()
            r0 = time.perf_counter()
            lib.refresh(G[0], stream)
            torch.cuda.synchronize()
            rt.append((time.perf_counter() - r0) * 1e3)
        rrec = lib.timing_read()
        rkb = by_kernel(lib.last_launches())
        lib.timing_enable(False, 0)
        step_bytes, _ = unfused_step_bytes(wl)
        out[key] = {"workload": desc, "numel": wl.numel, "ms_per_step": round(ms, 4),
                    "grad_elems_per_s": wl.numel / (ms * 1e-3),
                    "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "kernels": kernel_table(rec, kb, steps),
                    "refresh_ms": round(float(np.median(rt)), 3),
                    "refresh_kernels": kernel_table(rrec, rkb, refresh_reps)}
        lib.close()
        del G, W
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--refresh-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the per-kernel measurement of the other workloads")
    ap.add_argument("--other-configs-only", action="store_true",
                    help="run only the other workloads' per-kernel measurement (for a profiler "
                         "run of those kernels) and print their table as one JSON line")
    ap.add_argument("--no-multi-tensor", action="store_true",
                    help="skip the 4-layer fp16 sequential vs tgrad_step_many measurement")
    ap.add_argument("--plan", type=int, default=None,
                    help="launch plan (tgrad_set_fusion value); default: the library's")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the step is measured on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import tensor_gradient_compression_amd as tg
    from synth import (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, BF16_64x64x48x48x25,
                   GradStream, init_weights)

    wl = BF16_64x64x48x48x25
    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if args.other_configs_only:
        print(json.dumps({"other_configs": other_configs(dev, stream, steps=args.steps,
                                                          refresh_reps=args.refresh_reps)}))
        return
    K, Wm = args.steps, args.warmup

    # inputs: two distinct synthetic gradients, staged into one buffer per step
    gs = GradStream(wl, seed=0)
    bases = [tg.to_device(gs.next(), wl.dtype, dev) for _ in range(2)]
    W = tg.to_device(init_weights(wl, seed=0), wl.dtype, dev)
    nbuf = 2 * K + Wm
    grads = [bases[i % 2].clone() for i in range(nbuf)]
    pristine = bases[0]
    torch.cuda.synchronize()

    lib = tg.TGrad(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, wl.betas, wl.eps)
    if args.plan is not None and not lib.set_fusion(args.plan):
        raise SystemExit(f"launch plan {args.plan} does not apply to this workload")
    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for i in range(Wm):                      # step 1 refreshes (t = 1)
        lib.step(W, grads[i], stream)
    torch.cuda.synchronize()

    # per-kernel breakdown: K steps with every launch bracketed by HIP events (an event
    # pair per launch lengthens the step, so these steps are not the timed ones); the
    # algorithmic bytes and flops of each launch come from the library's record of the
    # launches the step made
    lib.timing_enable(True, 100000)
    for i in range(K):
        lib.step(W, grads[Wm + i], stream)
    torch.cuda.synchronize()
    rec = lib.timing_read()
    step_launches = lib.last_launches()
    kb = by_kernel(step_launches)
    # the dominant kernel: the largest share of the step among kernels with one launch
    # per step (a unique symbol for the profiler)
    single = {n: ms for n, (c, ms) in rec.items() if c == K and n in kb and kb[n][0] == 1}
    dom = max(single, key=single.get)

    # the timed steps: events around the dominant kernel's launches only
    lib.timing_only(dom)
    lib.timing_enable(True, 100000)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        lib.step(W, grads[Wm + K + i], stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    drec = lib.timing_read()
    lib.timing_only(None)
    ms_step = (t1 - t0) * 1e3 / K

    # refresh timed alone (reads the gradient only)
    rt = []
    lib.timing_enable(True, 100000)
    for _ in range(args.refresh_reps):
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        lib.refresh(pristine, stream)
        torch.cuda.synchronize()
        rt.append((time.perf_counter() - r0) * 1e3)
    rrec = lib.timing_read()
    refresh_launches = by_kernel(lib.last_launches())
    lib.timing_enable(False, 0)
    refresh_ms = float(np.median(rt))

    # the rate of a plain 1 GiB device copy on this machine (read + write bytes): what a pure
    # streaming kernel reaches, beside the 8 TB/s peak
    ncp = (1 << 30) // 4
    ca = torch.empty(ncp, dtype=torch.float32, device=dev).fill_(1.0)
    cb = torch.empty_like(ca)
    cb.copy_(ca)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(5):
        cb.copy_(ca)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * ncp * 4 * 5 / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    del ca, cb

    kernels = kernel_table(rec, kb, K)
    refresh_kernels = kernel_table(rrec, refresh_launches, args.refresh_reps)

    # the dominant kernel's launches inside the timed steps
    dn, dms = drec[dom]
    dom_bytes = kb[dom][1]
    dom_gbs = dom_bytes / (dms / dn * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(dom), "avg_ms": round(dms / dn, 5),
                "launches": dn, "alg_bytes": int(dom_bytes)}
    # whole-step roofline: the step's algorithmic bytes counted kernel by kernel without
    # fusion, over the measured step time; beside it the bytes the launched (fused)
    # kernels move by their own algorithmic count
    moved_bytes = sum(b for _, b, _ in kb.values())
    step_bytes, ncore = unfused_step_bytes(wl)
    step_frac = step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    moved_frac = moved_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS

    del grads
    torch.cuda.empty_cache()
    multi = None if args.no_multi_tensor else multi_tensor(dev, stream)
    others = None if args.no_other_configs else other_configs(dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        cpu = cpu_baseline(wl)

    out = {
        "metric": "TensorGRaD step ms + grad elems/s, % of HBM/MFMA roofline; refresh ms",
        "value": wl.numel / (ms_step * 1e-3),
        "unit": "grad elems/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 FNO spectral-weight gradient (64,64,48,48,25), Tucker ranks "
                               "(32,32,24,24,13), 5% top-k sparse, T=200",
                   "numel": wl.numel, "k": wl.k, "core_numel": ncore,
                   "launch_plan": "library default" if args.plan is None else args.plan,
                   "parallelism": "single GPU"},
        "refresh_ms": round(refresh_ms, 3),
        "step_alg_bytes": int(step_bytes),
        "step_hbm_frac": round(step_frac, 4),
        "step_moved_bytes": int(moved_bytes),
        "step_moved_hbm_frac": round(moved_frac, 4),
        "roofline": roofline,
        "hbm_copy_GBs": round(copy_gbs, 1),
        "kernels": kernels,
        "kernels_note": "per-kernel table from K extra steps with every launch timed (bytes "
                        "and flops: the library's record of the launches one step made); the "
                        "timed steps carry events around the roofline kernel only",
        "refresh_kernels": refresh_kernels,
        "multi_tensor": multi,
        "other_configs": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
