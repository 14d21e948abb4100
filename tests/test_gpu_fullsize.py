"""GPU parity at the full workload sizes, through the C ABI.

Byte work is compared whole: the device decode must return W itself, and the load-time
transcode and the exponent-only stream must hash to the digests the oracle produced for the
same seeded matrix (tests/golden/fullsize_digests.txt, written by make_fullsize_digests.py).
GEMMs are compared with the oracle (fp64) on every output element: every pipeline at each
batch size of the workload, and every kernel variant of the direct-palette path and of the
BF16 GEMM (so whatever variant the autotuner picks for the benchmark is covered).  The oracle
product is computed once per (workload, M).

The 32-layer stack (four of the five workloads are single matrices; this one is the model)
checks each matrix's decode bit-exactly, and every output of each layer's GEMMs and glue
against the oracle on the inputs the device actually fed that layer.
"""
import hashlib
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import synth
from lossless_bf16_weight_amd.stack import MLPStack, as_bf16_bits
from oracle import gemm

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize_digests.txt")
ALL_PIPES = [uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE, uw.UW_PIPE_EXP_ONLY, uw.UW_PIPE_FULL_DECODE]
M_SETS = {"c2": (1,), "c3": (1, 8, 32, 64), "c5": (128,)}
MAKERS = {"c2": synth.config2, "c3": synth.config3, "c5": synth.config5}


def torch():
    import torch as t
    return t


def log(msg):
    print(msg, flush=True)


def digests():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, wd, blob, tc, ex, size = line.split()
        out[name] = dict(w=wd, blob=blob, transcode=tc, exp=ex, size=int(size))
    return out


def sha(t_):
    return hashlib.sha256(t_.cpu().numpy().tobytes()).hexdigest()


def check_all(y_dev, y_ref, s, what):
    y = y_dev.cpu().numpy().astype(np.float64)
    assert y.shape == y_ref.shape
    ok = gemm.within_bound(y, y_ref, s)
    bad = np.argwhere(~ok)
    assert ok.all(), "%s: %d/%d outside bound, first %s: gpu %r ref %r S %r" % (
        what, len(bad), ok.size, bad[:3].tolist(), y[tuple(bad[0])], y_ref[tuple(bad[0])], s[tuple(bad[0])])


@pytest.fixture(scope="module")
def golden():
    return digests()


@pytest.mark.parametrize("name", ["c2", "c3", "c5"])
def test_fullsize_matrix(name, golden):
    t = torch()
    t0 = time.time()
    c = MAKERS[name]()
    w, x_all = c["w"], c["x"]
    n, k = w.shape
    ref = golden[name]
    assert synth.digest(w) == ref["w"], "seeded generator changed"
    blob = uw.uw_encode(w)
    assert hashlib.sha256(blob.tobytes()).hexdigest() == ref["blob"]
    cm = uw.CompressedMatrix(w, blob=blob)
    log("%s: generated, encoded (%d B, equals the oracle's) and uploaded in %.1fs" % (name, blob.size, time.time() - t0))
    ws = t.zeros(64, dtype=t.int32, device="cuda")
    assert sha(cm.idx) == ref["transcode"]
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w)
    del out
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert sha(ex) == ref["exp"]
    del ex
    wbits = t.from_numpy(w.view(np.int16)).cuda()
    refs = gemm.gemm_ref_multi([x_all[:m] for m in M_SETS[name]], w)
    for m, (y_ref, s) in zip(M_SETS[name], refs):
        x = x_all[:m]
        xd = t.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        for pipe in ALL_PIPES:
            wsp = cm.workspace(m, pipe)
            variants = range(uw.uw_variant_count()) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (-1,)
            for v in variants:
                y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
                uw.uw_gemm_variant(cm.d, xd, y, m, pipe, v, wsp)
                if wsp is not None:
                    uw.uw_check(wsp)
                check_all(y, y_ref, s, "%s m=%d pipeline %d variant %d" % (name, m, pipe, v))
        for v in range(uw.uw_variant_count()):
            y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_bf16(wbits, xd, y, m, v)
            check_all(y, y_ref, s, "%s m=%d bf16 variant %d" % (name, m, v))
        log("%s m=%d: every pipeline and variant within bound on all %d outputs" % (name, m, m * n))


@pytest.fixture(scope="module")
def stack4():
    """The 32-layer MLP stack at M = 16, every matrix decoded and checked as it is loaded;
    each W kept on the host for the GEMM checks (11.3 GB)."""
    t0 = time.time()
    meta = synth.config4_meta()
    layers = len(meta["stds"])
    st = MLPStack(16, 4096, 14336)
    keep = {}
    buf = {0: torch().empty((14336, 4096), dtype=torch().int16, device="cuda"),
           2: torch().empty((4096, 14336), dtype=torch().int16, device="cuda")}
    ws = torch().zeros(64, dtype=torch().int32, device="cuda")
    jobs = [(l, j) for l in range(layers) for j in range(3)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        futs = [ex.submit(synth.config4_matrix, meta, l, j) for (l, j) in jobs[:8]]
        pending = []
        for i, (l, j) in enumerate(jobs):
            w = futs[i].result()
            futs[i] = None
            if i + 8 < len(jobs):
                futs.append(ex.submit(synth.config4_matrix, meta, *jobs[i + 8]))
            cm = uw.CompressedMatrix(w)
            out = buf[2 if j == 2 else 0]
            uw.uw_decode_full(cm.d, out, ws)
            uw.uw_check(ws)
            assert np.array_equal(out.cpu().numpy().view(np.uint16), w), "layer %d matrix %d" % (l, j)
            keep[(l, j)] = w
            pending.append(cm)
            if j == 2:
                st.add_layer(*pending)
                pending = []
            if j == 2 and l % 8 == 7:
                log("c4: %d layers generated, encoded, uploaded and decoded bit-exactly (%.0fs)" % (l + 1,
                                                                                                   time.time() - t0))
    return st, meta, keep


def test_c4_stack_step(stack4):
    """One decode step through all 96 compressed matrices; every output of each GEMM checked
    against the oracle fed the device's own layer input, the glue within 1 BF16 ulp."""
    t = torch()
    st, meta, keep = stack4
    assert st.weight_count() == 32 * 3 * 14336 * 4096
    x = t.from_numpy(meta["x"].view(np.int16)).cuda()
    pipes = (uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE)
    traces = {}
    for pipe in pipes:
        trace = []
        st.step(x, pipeline=pipe, trace=trace)
        traces[pipe] = trace
        fused = st.step(x, pipeline=pipe, fused=True)   # SwiGLU in the up GEMM's epilogue
        assert np.array_equal(as_bf16_bits(fused), as_bf16_bits(trace[-1][5])), "fused step differs"
        log("c4 pipeline %d: step traced, fused step bit-identical" % pipe)
    t0 = time.time()
    for l in range(len(traces[pipes[0]])):
        for j in range(3):
            ios = [((xi, g), (xi, u), (h, y))[j] for (xi, g, u, h, y, xo) in (traces[p][l] for p in pipes)]
            refs = gemm.gemm_ref_multi([as_bf16_bits(inp) for inp, _ in ios], keep[(l, j)])
            for pipe, (_, out), (y_ref, s) in zip(pipes, ios, refs):
                ok = gemm.within_bound(out.astype(np.float64), y_ref, s)
                assert ok.all(), "pipeline %d layer %d matrix %d: %d outside bound" % (pipe, l, j, (~ok).sum())
        for pipe in pipes:
            xi, g, u, h, y, xo = traces[pipe][l]
            xi, h, xo = as_bf16_bits(xi), as_bf16_bits(h), as_bf16_bits(xo)
            if l == 0:
                assert np.array_equal(xi, meta["x"])
            assert np.abs(h.astype(np.int32) - gemm.swiglu_ref(g, u).astype(np.int32)).max() <= 1
            assert np.abs(xo.astype(np.int32) - gemm.rmsnorm_ref(y).astype(np.int32)).max() <= 1
            assert np.isfinite(y).all()
        if l % 8 == 7:
            log("c4: layers 0..%d, every GEMM output within bound for both pipelines (%.0fs)" % (l, time.time() - t0))
