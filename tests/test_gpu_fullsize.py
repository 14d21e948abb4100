"""GPU parity at the full workload sizes, through the C ABI.

Byte work is compared whole: the device decode must return W itself, and the load-time
transcode and the exponent-only stream must hash to the digests the oracle produced for the
same seeded matrix (tests/golden/fullsize_digests.txt, written by make_fullsize_digests.py).
GEMMs are compared with the oracle (fp64) on sampled output columns: the first and last
rows of W, rows in tiles holding verbatim segments, and a seeded random sample; every
pipeline at each batch size of the workload, and every kernel variant of the direct-palette
path (so whatever variant the autotuner picks for the benchmark is covered).

The 32-layer stack (four of the five workloads are single matrices; this one is the model)
checks each matrix's decode bit-exactly, and each layer's GEMMs and glue against the oracle
on the inputs the device actually fed that layer.
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
from oracle import codec, gemm

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


def sample_rows(w, flags_tiles, count=256, seed=0):
    n = w.shape[0]
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows |= {0, n - 1}
    vt = np.nonzero(flags_tiles)[0][:64]                       # tiles with verbatim segments
    for t in vt:
        rows |= {r for r in range(16 * t, min(16 * t + 16, n))}
    return np.array(sorted(rows))


def check_rows(y_dev, y_ref, s, rows, what):
    y = y_dev.cpu().numpy().astype(np.float64)[:, rows]
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
    flags = codec.parse(blob.tobytes())["flags"].reshape(-1, k // 64)
    rows = sample_rows(w, flags.any(axis=1))
    wbits = t.from_numpy(w.view(np.int16)).cuda()
    for m in M_SETS[name]:
        x = x_all[:m]
        y_ref, s = gemm.gemm_ref_rows(x, w, rows)
        xd = t.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        for pipe in ALL_PIPES:
            wsp = cm.workspace(m, pipe)
            variants = range(uw.uw_variant_count()) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (-1,)
            for v in variants:
                y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
                uw.uw_gemm_variant(cm.d, xd, y, m, pipe, v, wsp)
                if wsp is not None:
                    uw.uw_check(wsp)
                check_rows(y, y_ref, s, rows, "%s m=%d pipeline %d variant %d" % (name, m, pipe, v))
        for v in range(uw.uw_variant_count()):
            y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_bf16(wbits, xd, y, m, v)
            check_rows(y, y_ref, s, rows, "%s m=%d bf16 variant %d" % (name, m, v))
        log("%s m=%d: every pipeline and variant within bound on %d sampled rows" % (name, m, len(rows)))


@pytest.fixture(scope="module")
def stack4():
    """The 32-layer MLP stack at M = 16, every matrix decoded and checked as it is loaded;
    sampled rows of each W kept on the host for the GEMM checks."""
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
            flags = codec.parse(cm.blob.tobytes())["flags"].reshape(-1, w.shape[1] // 64)
            rows = sample_rows(w, flags.any(axis=1), count=48, seed=l * 3 + j)
            keep[(l, j)] = (rows, w[rows].copy())
            pending.append(cm)
            if j == 2:
                st.add_layer(*pending)
                pending = []
            if j == 2 and l % 8 == 7:
                log("c4: %d layers generated, encoded, uploaded and decoded bit-exactly (%.0fs)" % (l + 1,
                                                                                                   time.time() - t0))
    return st, meta, keep


def test_c4_stack_step(stack4):
    """One decode step through all 96 compressed matrices; each GEMM checked on sampled
    rows against the oracle fed the device's own layer input, the glue within 1 BF16 ulp."""
    t = torch()
    st, meta, keep = stack4
    assert st.weight_count() == 32 * 3 * 14336 * 4096
    x = t.from_numpy(meta["x"].view(np.int16)).cuda()
    for pipe in (uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE):
        trace = []
        st.step(x, pipeline=pipe, trace=trace)
        for l, (xi, g, u, h, y, xo) in enumerate(trace):
            xi, h, xo = as_bf16_bits(xi), as_bf16_bits(h), as_bf16_bits(xo)
            if l == 0:
                assert np.array_equal(xi, meta["x"])
            for j, (inp, out) in enumerate(((xi, g), (xi, u), (h, y))):
                rows, wr = keep[(l, j)]
                y_ref, s = gemm.gemm_ref(inp, wr)
                ok = gemm.within_bound(out.astype(np.float64)[:, rows], y_ref, s)
                assert ok.all(), "pipeline %d layer %d matrix %d: %d outside bound" % (pipe, l, j, (~ok).sum())
            assert np.abs(h.astype(np.int32) - gemm.swiglu_ref(g, u).astype(np.int32)).max() <= 1
            assert np.abs(xo.astype(np.int32) - gemm.rmsnorm_ref(y).astype(np.int32)).max() <= 1
            assert np.isfinite(y).all()
        log("c4 pipeline %d: 32 layers, 96 GEMMs + glue within bound" % pipe)
        fused = st.step(x, pipeline=pipe, fused=True)   # SwiGLU in the up GEMM's epilogue
        assert np.array_equal(as_bf16_bits(fused), as_bf16_bits(trace[-1][5])), "fused step differs"
        log("c4 pipeline %d: fused step bit-identical" % pipe)
