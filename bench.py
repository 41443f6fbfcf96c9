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

Prints ONE JSON line. --gpus N with N > 1 exits: this build runs on one GPU.
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


def kernel_bytes(wl, proj3=False):
    """Algorithmic HBM bytes per launch of every step kernel, keyed by kernel name
    (proj3: the projection's first launch takes the last three modes).
    Mode products: the input tile read once and the output written once (the operand
    matrix is negligible); apply: + W read and written, membership bitmask (N/8 B),
    per-word ranks (N/16 B) and the k sparse updates. Gather: k indices, k gradient
    values read, k fp32 values written, k zeros written. Adam: g, m, v read and m, v, u
    written, 4 B each, over core + k values."""
    P = 2 if wl.dtype == "c64" else 1
    es = esize(wl.dtype)
    N, k = wl.numel, wl.k
    fmodes = [n for n, (I, r) in enumerate(zip(wl.shape, wl.ranks)) if r < I]
    cur = list(wl.shape)
    proj, rec = [], []
    psizes = [N]        # tensor size after each projection mode
    size = N
    for j, n in enumerate(reversed(fmodes)):
        out = size // cur[n] * wl.ranks[n]
        inb = size * P * (es if j == 0 else 4)
        proj.append(inb + out * P * 4)
        cur[n] = wl.ranks[n]
        size = out
        psizes.append(size)
    ncore = size
    rsizes = [ncore]    # tensor size after each reconstruction mode
    for j, n in enumerate(fmodes):
        out = size // cur[n] * wl.shape[n]
        b = size * P * 4
        if j + 1 == len(fmodes):
            # W read + written, membership mask, per-word ranks, the k sparse updates and
            # (contiguous output tiles) their k Omega indices
            b += 2 * N * es + N // 8 + N // 16 + k * P * 4 + k * 4
        else:
            b += out * P * 4
        rec.append(b)
        cur[n] = wl.shape[n]
        size = out
        rsizes.append(size)
    # two trailing modes per launch: input read once, output written once; the first
    # projection launch also performs the COO gather (k indices read and k fp32 values
    # written; the gradient values come with the input tile, which is zeroed at Omega in
    # LDS only)
    d = len(wl.shape)
    I1, I2, R1, R2 = wl.shape[d - 2], wl.shape[d - 1], wl.ranks[d - 2], wl.ranks[d - 1]
    A = N // (I1 * I2)
    proj2 = A * I1 * I2 * P * es + A * R1 * R2 * P * 4 + k * (4 + 4 * P)
    # three trailing modes: the same, with the output R0 R1 R2 per index of the leading modes
    R0 = wl.ranks[d - 3] if d >= 3 else 1
    U = A // wl.shape[d - 3] if d >= 3 else A
    proj3_b = A * I1 * I2 * P * es + U * R0 * R1 * R2 * P * 4 + k * (4 + 4 * P)
    rec2 = A * R1 * R2 * P * 4 + 2 * N * es + N // 8 + N // 16 + k * P * 4 + k * 4
    flops_proj = []
    size = N
    cur = list(wl.shape)
    for n in reversed(fmodes):
        flops_proj.append(2 * size * P * wl.ranks[n] * P)
        size = size // cur[n] * wl.ranks[n]
        cur[n] = wl.ranks[n]
    return {
        "gather_residual": [k * (4 + es + 4 * P + es)],
        "modeprod_project_first": proj[:1],
        "modeprod_project": proj[2:] if proj3 else proj[1:],
        "adam_fused": [(ncore + k) * P * 24],
        "modeprod_reconstruct": rec[:-1],
        "modeprod_reconstruct_apply": rec[-1:],
        "modeprod2_project_first": [proj2],
        "modeprod3_project_first": [proj3_b],
        "modeprod2_reconstruct_apply": [rec2],
        # the projection's last two modes in one launch (fp32 in, core out), and the
        # reconstruction's first two
        "modeprod_pair_project": [(psizes[-3] + ncore) * P * 4] if len(psizes) >= 3 else [],
        "modeprod_pair_reconstruct": [(ncore + rsizes[2]) * P * 4] if len(rsizes) >= 3 else [],
        "_flops_project": flops_proj,
        "_ncore": ncore,
        # the step's work as one launch per kernel of the path, fp32 intermediates and no
        # fusion: gather, projection chain, Adam, reconstruction chain with the apply
        "_unfused_step": k * (4 + es + 4 * P + es) * (1 if k else 0) + sum(proj)
                         + (ncore + k) * P * 24 + sum(rec),
    }


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
    """The oracle (numpy, fp64 contractions) timed on this host on a bounded sample: one
    non-refresh step of the full workload, with Omega a seeded random index set of size
    k and seeded random orthonormal factors (the step's cost does not depend on which
    indices or which subspace it uses). The refresh (a 236M-key sort and fp64 Grams)
    is left out of the sample."""
    import oracle as O
    from synth import GradStream, init_weights
    g = GradStream(wl, seed=seed).next()
    W = init_weights(wl, seed=seed)
    orc = O.TGradOracle(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, *wl.betas, wl.eps)
    rng = np.random.default_rng(seed + 99)
    orc.omega = np.sort(rng.choice(wl.numel, wl.k, replace=False)).astype(np.uint32)
    orc.factors = [np.linalg.qr(rng.standard_normal((I, r)))[0].astype(np.float32) if r < I else None
                   for I, r in zip(wl.shape, wl.ranks)]
    orc.t = 1
    orc.refreshed_for = 2
    t0 = time.perf_counter()
    orc.step(W, g)
    dt = time.perf_counter() - t0
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
    return {"value": wl.numel / dt, "unit": "grad elems/s", "cores": threads, "kind": "oracle",
            "sample": f"1 non-refresh step of the full workload ({wl.numel} elements), "
                      f"{dt:.1f} s; numpy BLAS threads = available cores; refresh excluded",
            "seconds": dt, "cpu_model": cpu_model, "blas": blas}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--refresh-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-multi-tensor", action="store_true",
                    help="skip the 4-layer fp16 sequential vs tgrad_step_many measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
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
    # pair per launch lengthens the step, so these steps are not the timed ones)
    lib.timing_enable(True, 100000)
    for i in range(K):
        lib.step(W, grads[Wm + i], stream)
    torch.cuda.synchronize()
    rec = lib.timing_read()
    kb = kernel_bytes(wl, proj3="modeprod3_project_first" in rec)
    # the dominant kernel: the largest share of the step among kernels with one launch
    # per step (a unique symbol for the profiler) and a byte count
    single = {n: ms for n, (c, ms) in rec.items() if c == K and n in kb and kb[n]}
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

    kernels = {}
    for name, (n, ms) in rec.items():
        per_step = n // K if n % K == 0 else n / K
        avg_ms = ms / n
        entry = {"launches_per_step": per_step, "avg_ms": round(avg_ms, 5),
                 "ms_per_step": round(ms / K, 5)}
        if name in kb and kb[name]:
            byts = sum(kb[name]) / len(kb[name])           # mean algorithmic bytes per launch
            gbs = byts / (avg_ms * 1e-3) / 1e9
            entry.update({"alg_bytes_per_launch": int(byts), "achieved_GBs": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        kernels[name] = entry
    refresh_kernels = {name: {"launches": n, "ms": round(ms / args.refresh_reps, 4)}
                       for name, (n, ms) in rrec.items()}

    # the dominant kernel's launches inside the timed steps
    dn, dms = drec[dom]
    dom_bytes = sum(kb[dom]) / len(kb[dom])
    dom_gbs = dom_bytes / (dms / dn * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": counter_traffic(dom), "avg_ms": round(dms / dn, 5),
                "launches": dn}
    # whole-step roofline: the step's algorithmic bytes counted kernel by kernel without
    # fusion, over the measured step time; the bytes the launched (fused) kernels move
    # are reported beside it
    moved_bytes = sum(sum(kb[name]) / len(kb[name]) * v["launches_per_step"]
                      for name, v in kernels.items() if name in kb and kb[name])
    step_bytes = kb["_unfused_step"]
    step_frac = step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    moved_frac = moved_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS

    del grads
    torch.cuda.empty_cache()
    multi = None if args.no_multi_tensor else multi_tensor(dev, stream)

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
                   "numel": wl.numel, "k": wl.k, "core_numel": kb["_ncore"],
                   "parallelism": "single GPU"},
        "refresh_ms": round(refresh_ms, 3),
        "step_alg_bytes": int(step_bytes),
        "step_hbm_frac": round(step_frac, 4),
        "step_moved_bytes": int(moved_bytes),
        "step_moved_hbm_frac": round(moved_frac, 4),
        "roofline": roofline,
        "hbm_copy_GBs": round(copy_gbs, 1),
        "kernels": kernels,
        "kernels_note": "per-kernel table from K extra steps with every launch timed; the "
                        "timed steps carry events around the roofline kernel only",
        "refresh_kernels": refresh_kernels,
        "multi_tensor": multi,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
