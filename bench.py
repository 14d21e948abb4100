#!/usr/bin/env python3
"""Benchmark: the direct-palette fused GEMV (lossless BF16 weights rebuilt on chip) on a
Llama-3.1-8B gate_proj-shaped matrix (14336 x 4096, N(0, 0.02^2), 0.05 % rows with a
planted out-of-palette exponent), M = 1, one MI355X.

One step = one uw_gemm(direct palette) call: reads the resident compressed matrix
(sign+mantissa bytes, 4-bit palette indices, verbatim flags and exponents) and X, writes
Y = X W^T in fp32.  Inputs are resident in HBM before timing starts.  Launches rotate over
R distinct copies of the matrix so the working set exceeds twice the 256 MB Infinity
Cache and every step reads HBM.

Prints one JSON line (stdout).  Diagnostics go to stderr.
    python bench.py [--gpus 1] [--steps 500] [--warmup 50]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode GEMM eff. weight GB/s & % HBM peak; bits/weight (8B MLP, M=1-64)"
HBM_PEAK_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X (no sparsity)
ROTATE_BYTES = 512e6
PMC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_direct_palette_gate14336x4096_m1_pmc.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("uw_gemm.hip", "uw_device.h", "uw_internal.h"):
        h.update(open(os.path.join(ROOT, "lossless_bf16_weight_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was taken on the
    current kernel source; else None."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m_hash = re.search(r"kernel source sha256\[:16\]:\s*([0-9a-f]{16})", text)
    m_bytes = re.search(r"HBM bytes per launch \(fetch \+ write, calibrated\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def device_info():
    """Current GPU clock levels from sysfs (the amdgpu driver's pp_dpm_* files, the starred
    line) and the host CPU model; read from files, so no program is started (a process that
    has touched the GPU, e.g. under a profiler's preload, must not exec another).  Fields are
    None where a read fails."""
    info = {"gpu": None, "clocks": None, "cpu_model": None}
    clocks = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device"))[:4]:
        for f in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(dev, f)) as fh:
                    cur = [ln.strip() for ln in fh if ln.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                clocks.append("%s %s %s" % (dev.split("/")[-2], f[7:], cur[0]))
    info["clocks"] = clocks or None
    try:
        with open("/proc/cpuinfo") as f:
            m = re.search(r"^model name\s*:\s*(.+)$", f.read(), re.M)
        info["cpu_model"] = m.group(1).strip() if m else None
    except OSError:
        pass
    return info


def _rate(fn, seconds):
    """Repeat fn() for at least `seconds`; returns (calls, elapsed seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def rows_within_bound(y, x, w, rows):
    """Sanity check of a timed configuration (not the parity tests, which compare with the
    oracle): the sampled output columns against y = x W^T evaluated in fp64 from the BF16 bits,
    within 1e-3 * sum_k |x_k w_k|."""
    def f64(b):
        return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xf, wf = f64(x), f64(w[rows])
    ref, mag = xf @ wf.T, np.abs(xf) @ np.abs(wf).T
    return np.abs(np.asarray(y, np.float64)[:, rows] - ref) <= 1e-3 * mag


def cpu_baseline(w, x, seconds=2.5):
    """The oracle (numpy, as it stands) on a bounded row sample of the same workload, on this
    host's cores: the step itself (rebuild W from the direct-palette format, fp64 GEMV) and,
    separately, oracle encode, oracle decode (Huffman bundle -> W) and the fp64 GEMV, each at
    every core of this process's affinity set and again at one thread (BLAS threads limited
    with threadpoolctl; the oracle's own loops are numpy, single-threaded).  Rates are
    uncompressed-equivalent bytes of the sample (2 B a weight) per second."""
    from threadpoolctl import threadpool_limits
    from oracle import codec, gemm
    rows = 448                                   # 28 tiles of 16 rows
    ws = w[:rows]
    k = ws.shape[1]
    nbytes = 2.0 * rows * k
    enc = codec.encode(ws, rows, k)
    blob = codec.serialize(enc)
    d = codec.parse(blob)
    idx = codec.transcode_blob(blob)
    cores = len(os.sched_getaffinity(0))

    def step():
        wr = codec.reconstruct_from_palette(d["sm"], idx, d["flags"], d["vprefix"], d["vexp"], d["palette"], rows, k)
        return gemm.gemm_ref(x, wr)

    parts = {"step": step,
             "encode": lambda: codec.serialize(codec.encode(ws, rows, k)),
             "decode": lambda: codec.decode_blob(blob),
             "gemm_fp64": lambda: gemm.gemm_ref(x, ws)}
    detail = {}
    for threads in (cores, 1):
        with threadpool_limits(limits=threads):
            for name, fn in parts.items():
                reps, el = _rate(fn, seconds)
                detail["%s_%dt" % (name, threads)] = {"gb_s": round(nbytes * reps / el / 1e9, 4), "calls": reps,
                                                      "s": round(el, 2)}
    assert np.array_equal(codec.decode_blob(blob), ws)
    return dict(value=detail["step_%dt" % cores]["gb_s"], unit="GB/s", cores=cores, kind="oracle",
                sample="%d of 14336 rows (%d tiles) x %d of the same matrix and X: the oracle's step (direct-palette "
                       "rebuild + fp64 GEMV) at all %d cores of the affinity set; detail: oracle encode, decode and "
                       "fp64 GEMV at %d cores and at 1 thread, %.1f s each; uncompressed-equivalent bytes"
                       % (rows, rows // 16, k, cores, cores, seconds),
                cpu_model=device_info()["cpu_model"], threads=[cores, 1], detail=detail)


class ClockSampler:
    """Samples the GPU's current sclk/mclk (sysfs pp_dpm_*, the starred line) in a thread
    while the GPU runs the measured kernel; reports min / median / max MHz over the samples."""

    def __init__(self, period_s=0.002):
        import threading
        self.period = period_s
        self.counts = {}      # clock name -> MHz samples
        self._stop = threading.Event()
        self._files = [os.path.join(dev, f) for dev in sorted(glob.glob("/sys/class/drm/card*/device"))[:1]
                       for f in ("pp_dpm_sclk", "pp_dpm_mclk")]
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        out = {}
        for path in self._files:
            try:
                with open(path) as fh:
                    cur = [ln.strip() for ln in fh if ln.strip().endswith("*")]
            except OSError:
                continue
            m = re.search(r"(\d+)\s*Mhz", cur[0], re.I) if cur else None
            if m:
                out[path.split("_")[-1]] = int(m.group(1))
        return out

    def _run(self):
        while not self._stop.is_set():
            for name, mhz in self._read().items():
                self.counts.setdefault(name, []).append(mhz)
            self._stop.wait(self.period)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        """{clock: {min, median, max MHz, samples}} over the sampled run, or None."""
        out = {}
        for name, v in self.counts.items():
            v = sorted(v)
            out[name + "_mhz"] = {"min": v[0], "median": v[len(v) // 2], "max": v[-1], "samples": len(v)}
        return out or None


SETTLE_MS = 50.0


def settle(fn, copies, stream, ms=SETTLE_MS):
    """Untimed launches of fn until `ms` of GPU time has passed.  The GPU's clocks drop while
    the host works between measurements and take a few milliseconds of load to come back; a
    few dozen warm-up launches of a 16 us kernel are not enough for that."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    done, i = 0.0, 0
    while done < ms:
        for _ in range(64):
            fn(i % copies)
            i += 1
        e1.record(stream)
        e1.synchronize()
        done = e0.elapsed_time(e1)


def time_launches(fn, copies, steps, warmup, stream):
    """fn(i) launches on `stream`.  Returns (total_ms, per-launch ms list).  The clocks are
    settled first; then, from an idle synchronised GPU, `warmup` untimed launches immediately
    followed by exactly `steps` timed ones between two events.  The untimed launches are the
    runway: the GPU is busy with them while the host queues the first timed launches, so the
    timed region holds back-to-back kernels and not the host's latency to queue the first one
    (with few steps that latency would otherwise be a visible share of the region)."""
    import torch
    settle(fn, copies, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(warmup):
        fn(i % copies)
    e0.record(stream)
    for i in range(steps):
        fn((warmup + i) % copies)
    e1.record(stream)
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1)
    # individual launches (for the spread)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(min(steps, 200))]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i % copies)
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return total, per


def time_torch_bf16(w, xs, steps, warmup):
    """torch.matmul (hipBLASLt) on the uncompressed BF16 matrix, rotated copies, per batch."""
    import torch
    n, k = w.shape
    copies = max(2, int(np.ceil(ROTATE_BYTES / (2 * n * k))))
    wd = [torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16) for _ in range(copies)]
    out = {}
    for m, xd in xs.items():
        xb = xd.view(torch.bfloat16)
        tot, _ = time_launches(lambda i: torch.matmul(xb, wd[i].t()), copies, steps, warmup,
                               torch.cuda.current_stream())
        out[m] = tot * 1e3 / steps
    del wd
    return out


def diagnostic(args):
    """Diagnostic lines (not the headline): every pipeline autotuned per batch size on the
    down_proj shape (4096 x 14336, M = 1..64), the heavy-tail 8192^2 matrix (M = 128), the
    1024^2 matrix (M = 1) or the gate_proj shape at large batches (14336 x 4096, M = 256..1024),
    timed against torch BF16; the decode entry points; or the 32-layer MLP stack at M = 16
    (plain, with hard layers, tuned end to end)."""
    import torch
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import autotune, synth
    assert torch.cuda.is_available(), "no GPU"
    steps, warmup = min(args.steps, 200), min(args.warmup, 20)
    if args.workload == "stack":
        return stack_step(args, steps, warmup)
    if args.workload == "stack-hard":
        return stack_hard_step(args, steps, warmup)
    if args.workload == "stack-tune":
        return stack_tune(args, steps, warmup)
    if args.workload == "decode":
        return decode_step(args, steps, warmup)
    if args.workload == "large":
        # gate_proj shape at prefill-sized batches: X drawn like the other configs' X.
        c = synth.config2()
        c["x"] = synth.gaussian_bf16(np.random.default_rng(11), (1024, c["w"].shape[1]), 1.0)
    else:
        c = {"down": synth.config3, "heavy": synth.config5, "small": synth.config1}[args.workload]()
    ms = {"down": (1, 8, 16, 32, 64), "heavy": (128,), "small": (1,), "large": (256, 512, 1024)}[args.workload]
    w, x_all = c["w"], c["x"]
    n, k = w.shape
    tuner = autotune.Tuner(w, rotate_bytes=ROTATE_BYTES)
    table = tuner.tune(ms, log=log)
    table.apply()
    info = uw.uw_blob_info(tuner.blob)
    resident = int(info["resident_bytes"])
    xs = {m: torch.from_numpy(np.ascontiguousarray(x_all[:m]).view(np.int16)).cuda() for m in ms}
    rows = np.random.default_rng(0).choice(n, 256, replace=False)
    res = []
    torch_us = time_torch_bf16(w, xs, steps, warmup)
    for m in ms:
        best = table.best_pipeline(n, k, m)
        ws = torch.zeros(uw.uw_workspace_size(tuner.mats[0], m, best.pipeline), dtype=torch.uint8, device="cuda")
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        step = lambda i: uw.uw_gemm(tuner.mats[i], xs[m], y, m, uw.UW_PIPE_AUTO, ws)
        step(0)
        torch.cuda.synchronize()
        assert rows_within_bound(y.cpu().numpy(), x_all[:m], w, rows).all(), "result outside the GEMM bound"
        tot, _ = time_launches(step, tuner.copies, steps, warmup, torch.cuda.current_stream())
        us = tot * 1e3 / steps
        bf = table.best_variant.get((n, k, m, uw.UW_PIPE_BF16))
        res.append({"m": m, "pipeline": autotune.PIPELINE_NAMES[best.pipeline],
                    "variant": uw.uw_variant_name(best.variant), "us": round(us, 3),
                    "compressed_tb_s": round((resident + 2 * m * k + 4 * m * n) / us / 1e6, 3),
                    "eff_weight_gb_s": round(2.0 * n * k / us / 1e3, 1),
                    "tflop_s": round(2.0 * m * n * k / us / 1e6, 1),
                    "frac_of_bf16_mfma_peak": round(2.0 * m * n * k / us / 1e6 / PEAK_MFMA_BF16_TFLOPS, 4),
                    "torch_bf16_us": round(torch_us[m], 3),
                    "own_bf16_us": round(bf.us, 3) if bf else None,
                    "speedup_vs_torch_bf16": round(torch_us[m] / us, 3)})
        log("m=%d: %s" % (m, res[-1]))
    out = {"diagnostic": args.workload, "n": n, "k": k, "bits_per_weight": round(8 * resident / (n * k), 4),
           "results": res}
    if args.workload == "small":
        # The 1024^2 case is launch/L2 sized (1.6 MB): microseconds only, no roofline claim.
        err = torch.zeros(64, dtype=torch.int32, device="cuda")
        wout = torch.empty((n, k), dtype=torch.int16, device="cuda")
        idx = [m_.idx for m_ in tuner.mats]
        tot, _ = time_launches(lambda i: uw.uw_transcode_palette(tuner.mats[i], idx[i], err), tuner.copies,
                               steps, warmup, torch.cuda.current_stream())
        out["transcode_us"] = round(tot * 1e3 / steps, 3)
        tot, _ = time_launches(lambda i: uw.uw_decode_full(tuner.mats[i], wout, err), tuner.copies, steps, warmup,
                               torch.cuda.current_stream())
        out["decode_full_us"] = round(tot * 1e3 / steps, 3)
        uw.uw_check(err)
        assert np.array_equal(wout.cpu().numpy().view(np.uint16), w), "decode not bit-exact"
    return out


def decode_step(args, steps, warmup):
    """The three Huffman decode entry points (load-time transcode to 4-bit indices, exponent
    bytes, full BF16 W) on gate_proj 14336 x 4096, down_proj 4096 x 14336 and the heavy-tail
    8192^2 matrix, each encoded with 512-symbol (default) and 256-symbol chunks; cache-cold
    rotation.  Checks: the full decode equals W bit for bit, and both chunkings give the same
    index and exponent streams."""
    import torch
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import synth
    res = {}
    for name, cfg in (("gate", synth.config2), ("down", synth.config3), ("heavy", synth.config5)):
        w = cfg()["w"]
        n, k = w.shape
        outs = {}
        for chunk in (512, 256):
            blob = uw.uw_encode(w, chunk)
            info = uw.uw_blob_info(blob)
            copies = max(2, int(np.ceil(ROTATE_BYTES / blob.size)))
            mats = [uw.DMat(blob, torch.from_numpy(blob).cuda(),
                            torch.empty(int(info["idx_bytes"]), dtype=torch.uint8, device="cuda")) for _ in range(copies)]
            err = torch.zeros(64, dtype=torch.int32, device="cuda")
            ex = [torch.empty(int(info["np"]) * k, dtype=torch.uint8, device="cuda") for _ in range(2)]
            wout = [torch.empty((n, k), dtype=torch.int16, device="cuda") for _ in range(2)]
            fns = {"transcode": lambda i: uw.uw_transcode_palette(mats[i], mats[i].idx, err),
                   "exponents": lambda i: uw.uw_decode_exponents(mats[i], ex[i % 2], err),
                   "full": lambda i: uw.uw_decode_full(mats[i], wout[i % 2], err)}
            row = {"bundle_bits_per_weight": round(8 * blob.size / (n * k), 4)}
            for op, fn in fns.items():
                tot, _ = time_launches(fn, copies, min(steps, 50), min(warmup, 5), torch.cuda.current_stream())
                uw.uw_check(err)
                us = tot * 1e3 / min(steps, 50)
                row[op + "_us"] = round(us, 2)
            assert np.array_equal(wout[0].cpu().numpy().view(np.uint16), w), "full decode is not W"
            outs[chunk] = (mats[0].idx.cpu().numpy(), ex[0].cpu().numpy())
            res["%s_chunk%d" % (name, chunk)] = row
            log("decode %s chunk %d: %s" % (name, chunk, row))
            del mats, ex, wout
            torch.cuda.empty_cache()
        assert all(np.array_equal(a, b) for a, b in zip(outs[512], outs[256])), "chunkings disagree"
    return {"diagnostic": "decode", "results": res}


def stack_step(args, steps, warmup):
    """One decode step at M = 16 through the 32-layer MLP stack (96 compressed matrices, SwiGLU
    and RMS norm between), timed against the same step with torch BF16 matmuls."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import synth
    from lossless_bf16_weight_amd.stack import MLPStack
    meta = synth.config4_meta()
    layers = len(meta["stds"])
    st = MLPStack(16, 4096, 14336)
    bf = []
    t0 = time.time()
    jobs = [(l, j) for l in range(layers) for j in range(3)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        mats = ex.map(lambda lj: synth.config4_matrix(meta, *lj), jobs)
        pending = []
        for (l, j), w in zip(jobs, mats):
            pending.append(uw.CompressedMatrix(w))
            bf.append(torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16))
            if j == 2:
                st.add_layer(*pending)
                pending = []
    log("stack built in %.1fs" % (time.time() - t0))
    # Kernel variant per matrix shape at M = 16 chosen by measurement (the library's autotuner,
    # once, as an engine would at load time); gate and up share a shape.
    from lossless_bf16_weight_amd import autotune
    for lj in ((0, 0), (0, 2)):
        tuner = autotune.Tuner(synth.config4_matrix(meta, *lj), bf16=False)
        tuner.tune([16], pipelines=(uw.UW_PIPE_DIRECT_PALETTE,), bf16=False, log=log).apply()
        del tuner
    torch.cuda.empty_cache()
    x = torch.from_numpy(meta["x"].view(np.int16)).cuda()
    step = lambda i: st.step(x, pipeline=uw.UW_PIPE_DIRECT_PALETTE, check=False)
    tot, _ = time_launches(step, 1, steps, warmup, torch.cuda.current_stream())
    us = tot * 1e3 / steps
    xb = x.view(torch.bfloat16)

    def step_bf16(i):
        h = xb
        for l in range(layers):
            g = torch.matmul(h, bf[3 * l].t()).float()
            u = torch.matmul(h, bf[3 * l + 1].t()).float()
            a = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
            yy = torch.matmul(a, bf[3 * l + 2].t()).float()
            h = (yy * torch.rsqrt((yy * yy).mean(dim=1, keepdim=True) + 1e-5)).to(torch.bfloat16)
        return h

    tot_b, _ = time_launches(step_bf16, 1, steps, warmup, torch.cuda.current_stream())
    us_b = tot_b * 1e3 / steps
    nparams = st.weight_count()
    return {"diagnostic": "stack", "layers": layers, "m": 16, "us_per_step": round(us, 1),
            "tokens_per_s": round(16 / (us * 1e-6), 1), "eff_weight_gb_s": round(2.0 * nparams / us / 1e3, 1),
            "compressed_tb_s": round(st.resident_bytes() / us / 1e6, 3),
            "torch_bf16_us_per_step": round(us_b, 1), "speedup_vs_torch_bf16": round(us_b / us, 3)}


def stack_hard_step(args, steps, warmup):
    """The 32-layer stack at M = 16 with hard layers (bundle only resident, index streams decoded
    ahead on a side stream by libuw's scheduler) and easy layers (direct-palette form): step time
    and weight footprint for 0, 1/4, 1/2 and all layers hard, each step checked bit-identical to
    the plain fused step; and the same with the decodes on the main stream (no overlap)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import autotune, synth
    from lossless_bf16_weight_amd.stack import HardEasyStack, MLPStack
    meta = synth.config4_meta()
    layers = len(meta["stds"])
    t0 = time.time()
    jobs = [(l, j) for l in range(layers) for j in range(3)]
    easy, bundles = [], []
    # Hard layers keep the bundle only; it is encoded with args.hard_chunk-symbol chunks (more,
    # shorter chunks: more independent decode chains) -- the same weights, palette and index
    # stream as the easy form, so every step must still equal the plain step bit for bit.
    with ThreadPoolExecutor(max_workers=8) as ex:
        for w in ex.map(lambda lj: synth.config4_matrix(meta, *lj), jobs):
            cm = uw.CompressedMatrix(w)
            easy.append(cm)
            bundles.append(uw.uw_encode(w, args.hard_chunk) if args.hard_chunk else cm.blob)
    log("stack built in %.1fs" % (time.time() - t0))
    for lj in ((0, 0), (0, 2)):
        tuner = autotune.Tuner(synth.config4_matrix(meta, *lj), bf16=False)
        tuner.tune([16], pipelines=(uw.UW_PIPE_DIRECT_PALETTE,), bf16=False, log=log).apply()
        del tuner
    torch.cuda.empty_cache()
    x = torch.from_numpy(meta["x"].view(np.int16)).cuda()
    plain = MLPStack(16, 4096, 14336)
    for l in range(layers):
        plain.add_layer(*easy[3 * l:3 * l + 3])
    ref = plain.step(x, pipeline=uw.UW_PIPE_DIRECT_PALETTE, check=True).clone()
    tot, _ = time_launches(lambda i: plain.step(x, pipeline=uw.UW_PIPE_DIRECT_PALETTE, check=False), 1, steps, warmup,
                           torch.cuda.current_stream())
    res = {"plain_us": round(tot * 1e3 / steps, 1), "plain_bits_per_weight": round(8 * plain.resident_bytes() /
                                                                                  plain.weight_count(), 4)}
    del plain
    hard_cms = {}
    for name, hard in (("none", []), ("quarter", [l for l in range(layers) if l % 4 == 3]),
                       ("half", [l for l in range(layers) if l % 2 == 1]), ("all", list(range(layers)))):
        for l in hard:
            for j in range(3):
                if (l, j) not in hard_cms:
                    hard_cms[(l, j)] = uw.CompressedMatrix(None, blob=bundles[3 * l + j], keep_index=False)
        mats = [tuple(hard_cms[(l, j)] if l in hard else easy[3 * l + j] for j in range(3)) for l in range(layers)]
        row = {"hard_layers": len(hard)}
        # (overlap, decoder workgroups): side-stream decode on the whole chip, on a persistent
        # grid of 32 / 64 / 128 workgroups (the rest of the chip left to the GEMMs), and the
        # decodes on the main stream.
        runs = [(True, 0)] + ([(True, 32), (True, 64), (True, 128), (False, 0)] if hard else [])
        for overlap, split in runs:
            st = HardEasyStack(16, 4096, 14336, mats, hard_layers=hard, overlap=overlap, decode_workgroups=split)
            out = st.step(x, check=True)
            assert torch.equal(out, ref), "scheduled step (%s, overlap=%s, split=%d) differs from the plain step" % (
                name, overlap, split)
            tot, _ = time_launches(lambda i: st.step(x, check=False), 1, steps, warmup, torch.cuda.current_stream())
            torch.cuda.synchronize()
            uw.uw_check(st.dws)
            key = ("us_overlap" if overlap else "us_main_stream") + ("_split%d" % split if split else "")
            row[key] = round(tot * 1e3 / steps, 1)
            row["bits_per_weight"] = round(8 * st.resident_bytes() / st.weight_count(), 4)
            row["weight_gb"] = round(st.resident_bytes() / 1e9, 3)
            st.close()
            del st
        res[name] = row
        log("stack-hard %s: %s" % (name, row))
    return {"diagnostic": "stack-hard", "layers": layers, "m": 16, "hard_bundle_chunk": args.hard_chunk or 512,
            "results": res}


def stack_tune(args, steps, warmup):
    """End-to-end tuning of the 32-layer stack's step at M = 1 and M = 16: coordinate descent over
    (pipeline, kernel variant) per projection on the measured step time, the tuned step checked
    bit-identical to the same configuration's traced step, written to a per-model file
    (--config-out, one file per M)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import autotune, synth
    from lossless_bf16_weight_amd.stack import MLPStack
    meta = synth.config4_meta()
    layers = len(meta["stds"])
    t0 = time.time()
    jobs = [(l, j) for l in range(layers) for j in range(3)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        cms = list(ex.map(lambda lj: uw.CompressedMatrix(synth.config4_matrix(meta, *lj)), jobs))
    log("stack built in %.1fs" % (time.time() - t0))
    res = {}
    for m in (1, 16):
        st = MLPStack(m, 4096, 14336)
        for l in range(layers):
            st.add_layer(*cms[3 * l:3 * l + 3])
        x = torch.from_numpy(np.ascontiguousarray(meta["x"][:m]).view(np.int16)).cuda()
        tuner = autotune.StepTuner(st, x, pipelines=(uw.UW_PIPE_TRANSCODE, uw.UW_PIPE_DIRECT_PALETTE),
                                   steps=8, rounds=3)
        t0 = time.time()
        r = tuner.tune(max_sweeps=3, log=log)
        cfg = r["config"]
        trace = []
        st.step(x, config=cfg, trace=trace)
        out = st.step(x, config=cfg)
        assert np.array_equal(out.cpu().numpy(), trace[-1][5]), "tuned fused step differs from its traced step"
        tot, _ = time_launches(lambda i: st.step(x, config=cfg, check=False), 1, steps, warmup,
                               torch.cuda.current_stream())
        row = {"us_per_step": round(tot * 1e3 / steps, 1), "tuner_us": round(r["us"], 1),
               "default_us": round(r["default_us"], 1), "sweeps": r["sweeps"], "evals": len(tuner.evals),
               "tune_s": round(time.time() - t0, 1),
               "config": {k: [autotune.PIPELINE_NAMES[p], uw.uw_variant_name(v) if v >= 0 else "library default"]
                          for k, (p, v) in cfg.items()}}
        if args.config_out:
            path = args.config_out.replace(".json", "") + "_m%d.json" % m
            autotune.save_model_config(path, "llama-3.1-8b-mlp-32x(14336x4096,4096x14336)", m, r)
            row["file"] = path
        res["m%d" % m] = row
        log("stack-tune m=%d: %s" % (m, row))
        del st, tuner
    return {"diagnostic": "stack-tune", "layers": layers, "results": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--variant", type=int, default=-1,
                    help="fused-kernel variant id (default: autotuned); given, nothing is autotuned")
    ap.add_argument("--bf16-variant", type=int, default=-1,
                    help="BF16 GEMV variant with --variant (default: the library's choice for the shape)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three device copies of 512 MiB (HBM counter calibration) and exit")
    ap.add_argument("--workload", default="gate",
                    choices=("gate", "down", "heavy", "stack", "stack-hard", "stack-tune", "small", "large",
                             "decode"),
                    help="gate (default: the headline line); down, heavy, stack, stack-hard, stack-tune, small, "
                         "large, decode: diagnostic lines for the down_proj batch sweep, the 8192^2 heavy-tail matrix at "
                         "M=128, the 32-layer stack, the same stack with hard (bundle-only) layers decoded ahead on a "
                         "side stream (whole chip or a persistent decoder grid), the stack's step tuned end to end "
                         "per projection, the 1024^2 single-matrix case, gate_proj at M = 256, 512, 1024, and the "
                         "three decode entry points on the MLP shapes at two chunk lengths")
    ap.add_argument("--hard-chunk", type=int, default=256,
                    help="stack-hard: chunk length (symbols) of the hard layers' bundles (0: the default encode)")
    ap.add_argument("--config-out", default="",
                    help="stack-tune: per-model configuration file prefix (written as <prefix>_m<M>.json)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda:0").fill_(1)
        for _ in range(3):
            src.clone()
        torch.cuda.synchronize()
        print("copied 3 x 512 MiB", file=sys.stderr)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    if args.workload != "gate":
        print(json.dumps(diagnostic(args)), flush=True)
        return

    dinfo = device_info()   # GPU name filled in below; clocks again after the timed region
    import torch
    import lossless_bf16_weight_amd as uw
    from lossless_bf16_weight_amd import autotune, synth

    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    dinfo["gpu"] = "%s (%s)" % (torch.cuda.get_device_name(0), torch.cuda.get_device_properties(0).gcnArchName)
    stream = torch.cuda.current_stream()
    t0 = time.time()
    c = synth.config2()
    w, x = c["w"], c["x"]
    n, k = w.shape
    log("generated c2 %dx%d in %.1fs, sha %s" % (n, k, time.time() - t0, synth.digest(w, x)))
    t0 = time.time()
    blob = uw.uw_encode(w)
    enc_s = time.time() - t0
    info = uw.uw_blob_info(blob)
    resident = int(info["resident_bytes"])
    # Rotated device copies (compressed and uncompressed), each cache-cold per launch, and the
    # per-(shape, M) variant choice by measurement for both the fused kernel and the BF16 GEMV.
    tuner = autotune.Tuner(w, blob=blob, rotate_bytes=ROTATE_BYTES)
    copies, mats = tuner.copies, tuner.mats
    log("encoded in %.2fs: bundle %.3f b/w, resident %.3f b/w, %d copies" % (
        enc_s, 8 * blob.size / (n * k), 8 * resident / (n * k), copies))
    if args.variant < 0:
        table = tuner.tune([1], pipelines=(uw.UW_PIPE_DIRECT_PALETTE,), bf16=True)
        table.apply()
        pal_variant = uw.uw_autotune_get_variant(n, k, 1, uw.UW_PIPE_DIRECT_PALETTE)
        bf16_variant = uw.uw_autotune_get_variant(n, k, 1, uw.UW_PIPE_BF16)
    else:                      # fixed variants, no tuning launches (profiling runs)
        pal_variant, bf16_variant = args.variant, args.bf16_variant
    log("autotuned: direct palette variant %d (%s), bf16 variant %d (%s)" % (
        pal_variant, uw.uw_variant_name(pal_variant), bf16_variant, uw.uw_variant_name(bf16_variant)))
    # load-time transcode (Huffman -> 4-bit indices), timed on the copies
    t_tc = []
    ws = torch.zeros(64, dtype=torch.int32, device=dev)
    for d in mats:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        uw.uw_transcode_palette(d, d.idx, ws)
        e1.record(stream)
        uw.uw_check(ws)
        t_tc.append(e0.elapsed_time(e1))
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)

    calls = [0]   # launches of the headline kernel so far (locates the timed ones in a kernel trace)

    def step(i):
        uw.uw_gemm_variant(mats[i], xd, y, 1, uw.UW_PIPE_DIRECT_PALETTE, pal_variant)
        calls[0] += 1

    # parity of the timed configuration on sampled rows
    step(0)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(n, 2048, replace=False)
    rows = np.union1d(rows, c["planted"])
    assert rows_within_bound(y.cpu().numpy(), x, w, rows).all(), "timed configuration outside the GEMM bound"

    before = calls[0]
    total_ms, per = time_launches(step, copies, args.steps, args.warmup, stream)
    # time_launches: settling launches, `warmup` untimed, `steps` timed, then single-event ones
    first_timed = before + (calls[0] - before - args.steps - min(args.steps, 200))
    log("timed launches: the headline kernel's dispatches %d .. %d (0-based, in launch order)" % (
        first_timed, first_timed + args.steps - 1))
    # Clocks under the same load, sampled right after the timed region (a sampling thread
    # during it would take the interpreter lock between launches and open gaps on the GPU).
    with ClockSampler() as clk:
        settle(step, copies, stream, ms=100.0)
    us = total_ms * 1e3 / args.steps
    med, p10, p90 = per[len(per) // 2] * 1e3, per[len(per) // 10] * 1e3, per[(9 * len(per)) // 10] * 1e3
    eff_gbs = 2.0 * n * k / (us * 1e-6) / 1e9
    alg_bytes = resident + 2 * k + 4 * n          # compressed W + X + Y per launch
    achieved = alg_bytes / (us * 1e-6) / 1e9

    # uncompressed comparators: own BF16 GEMV and torch (hipBLASLt) on BF16 W
    wcopies, wd = tuner.wcopies, tuner.wd
    yb = torch.empty((1, n), dtype=torch.float32, device=dev)

    def step_bf16(i):
        uw.uw_gemm_bf16(wd[i], xd, yb, 1, bf16_variant)

    tot_b, per_b = time_launches(step_bf16, wcopies, args.steps, args.warmup, stream)
    us_b = tot_b * 1e3 / args.steps
    wbf = [t.view(torch.bfloat16) for t in wd]
    xbf = xd.view(torch.bfloat16)

    def step_torch(i):
        torch.matmul(xbf, wbf[i].t())

    tot_t, _ = time_launches(step_torch, wcopies, args.steps, args.warmup, stream)
    us_t = tot_t * 1e3 / args.steps
    best_bf16_us = min(us_b, us_t)
    log("direct palette %.2f us (median %.2f, p10 %.2f, p90 %.2f); own bf16 %.2f us; torch %.2f us" % (
        us, med, p10, p90, us_b, us_t))

    cpu = None if args.no_cpu else cpu_baseline(w, x)
    traffic = traffic_from_profile()
    dinfo.update({k: v for k, v in device_info().items() if k != "gpu" and v is not None})
    dinfo["clocks_under_load_after_timed_region"] = clk.summary()
    out = {
        "metric": METRIC,
        "value": round(eff_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B gate_proj 14336x4096 N(0,0.02^2), 0.05% rows planted, "
                               "direct-palette fused GEMV M=1, fp32 out",
                   "n": n, "k": k, "m": 1, "pipeline": "direct_palette",
                   "variant": uw.uw_variant_name(pal_variant), "bf16_variant": uw.uw_variant_name(bf16_variant),
                   "rotation_copies": copies, "global_batch": 1, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "traffic_source": ("FETCH_SIZE + WRITE_SIZE from the committed rocprofv3 --pmc summary "
                                        "(%s), taken on this kernel source (sha256[:16] %s); not measured in this run"
                                        % (os.path.relpath(PMC_SUMMARY, ROOT), kernel_source_hash()))
                                       if traffic is not None else None},
        "cpu_baseline": cpu,
        "us_per_gemm": round(us, 3),
        "us_per_gemm_single_launch": {"median": round(med, 3), "p10": round(p10, 3), "p90": round(p90, 3)},
        "bits_per_weight": {"resident_direct_palette": round(8 * resident / (n * k), 4),
                            "huffman_bundle": round(8 * blob.size / (n * k), 4)},
        "compressed_bytes_per_launch": alg_bytes,
        "verbatim_segment_fraction": round(info["n_verb"] / (n * k / 64), 5),
        "bf16_gemv_us": {"own_hip": round(us_b, 3), "torch_hipblaslt": round(us_t, 3)},
        "bf16_eff_gbs_best": round(2.0 * n * k / (best_bf16_us * 1e-6) / 1e9, 1),
        "speedup_vs_best_bf16": round(best_bf16_us / us, 4),
        "load_time_transcode_us": round(1e3 * float(np.median(t_tc)), 2),
        "host_encode_s": round(enc_s, 3),
        "device": dinfo,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
