"""GPU tests of the per-(shape, M) pipeline choice (UW_PIPE_AUTO) and the tuner that fills it.

The Unweight post's autotuning paragraphs choose the pipeline and kernel per weight matrix and
batch size by measurement.  Here: the tuner times every pipeline x variant through the C ABI;
its table must name, for each measured batch size, exactly the argmin of its own medians
(the uncompressed BF16 key is recorded but never chosen for uw_gemm); the table installed in
the library (directly, or saved and reloaded through uw_autotune_load) must be what the
dispatcher reads; and uw_gemm(UW_PIPE_AUTO) -- at a measured batch size and at ones between --
must give the oracle's product within the GEMM bound, bit-identical to calling the chosen
pipeline and variant by hand (so the dispatch ran that choice)."""
import numpy as np
import pytest

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import autotune, synth
from oracle import gemm

pytestmark = pytest.mark.gpu

N, K = 512, 4096
TUNED_M = (1, 8, 64)
BETWEEN_M = (3, 20, 40, 100)


def torch():
    import torch as t
    return t


@pytest.fixture(scope="module")
def tuned():
    t = torch()
    w = synth.small_gaussian(N, K, seed=41, plant_frac=0.02)["w"]
    tuner = autotune.Tuner(w, rotate_bytes=24e6)
    table = tuner.tune(TUNED_M, launches=6, rounds=2)
    t.cuda.synchronize()
    return w, tuner, table


def test_table_is_the_argmin_of_its_own_timings(tuned):
    _, _, table = tuned
    for m in TUNED_M:
        cand = [e for e in table.all_times if (e.n, e.k, e.m) == (N, K, m)]
        assert {e.pipeline for e in cand} == set(autotune.PIPELINES) | {uw.UW_PIPE_BF16}
        assert len(cand) == 5 * uw.uw_variant_count()
        comp = [e for e in cand if e.pipeline != uw.UW_PIPE_BF16]
        best = table.best_pipeline(N, K, m)
        assert best.us == min(e.us for e in comp) and best.pipeline != uw.UW_PIPE_BF16
        for p in autotune.PIPELINES + (uw.UW_PIPE_BF16,):
            e = table.best_variant[(N, K, m, p)]
            assert e.us == min(c.us for c in cand if c.pipeline == p)


def _installed(m):
    return uw.uw_autotune_get(N, K, m)


def test_installed_and_reloaded_table_drive_the_dispatcher(tuned, tmp_path):
    _, _, table = tuned
    uw.uw_autotune_clear()
    try:
        table.apply()
        got = {m: _installed(m) for m in TUNED_M}
        for m in TUNED_M:
            b = table.best_pipeline(N, K, m)
            assert got[m] == (b.pipeline, b.variant)
            for p in autotune.PIPELINES + (uw.UW_PIPE_BF16,):
                assert uw.uw_autotune_get_variant(N, K, m, p) == table.best_variant[(N, K, m, p)].variant
        path = tmp_path / "table.txt"
        table.save(str(path))
        uw.uw_autotune_clear()
        assert _installed(1) == (uw.UW_PIPE_DIRECT_PALETTE, -1)
        uw.uw_autotune_load(str(path))
        assert {m: _installed(m) for m in TUNED_M} == got
    finally:
        uw.uw_autotune_clear()


@pytest.mark.parametrize("source", ["apply", "file"])
def test_auto_dispatch_against_oracle(tuned, source, tmp_path):
    t = torch()
    w, tuner, table = tuned
    uw.uw_autotune_clear()
    try:
        if source == "apply":
            table.apply()
        else:
            path = tmp_path / "table.txt"
            table.save(str(path))
            uw.uw_autotune_load(str(path))
        d = tuner.mats[0]
        rng = np.random.default_rng(42)
        for m in TUNED_M + BETWEEN_M:
            pipe, var = _installed(m)
            x = synth.gaussian_bf16(rng, (m, K), 1.0)
            xd = t.from_numpy(x.view(np.int16)).cuda()
            need = uw.uw_workspace_size(d, m, uw.UW_PIPE_AUTO)
            assert need >= uw.uw_workspace_size(d, m, pipe)       # AUTO's size covers the chosen pipeline
            ws = t.zeros(max(need, 256), dtype=t.uint8, device="cuda")
            y = t.full((m, N), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm(d, xd, y, m, uw.UW_PIPE_AUTO, ws)
            uw.uw_check(ws)
            y_ref, s = gemm.gemm_ref(x, w)
            ok = gemm.within_bound(y.cpu().numpy().astype(np.float64), y_ref, s)
            assert ok.all(), "m=%d (pipeline %d variant %d): %d outside bound" % (m, pipe, var, (~ok).sum())
            y2 = t.full((m, N), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(d, xd, y2, m, pipe, var, ws)
            uw.uw_check(ws)
            assert t.equal(y, y2), "m=%d: AUTO did not run pipeline %d variant %d" % (m, pipe, var)
    finally:
        uw.uw_autotune_clear()
