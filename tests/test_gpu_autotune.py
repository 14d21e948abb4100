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


# ----------------------------------------------------------------------------------------------
# End-to-end coordinate descent over an MLP stack's step (per projection), and the decode/GEMM
# split coordinate of a stack with hard layers.
# ----------------------------------------------------------------------------------------------
def _small_stack(m, layers=3, seed=61):
    from lossless_bf16_weight_amd.stack import MLPStack
    rng = np.random.default_rng(seed)
    hidden, inter = 256, 704
    mats = [(synth.small_gaussian(inter, hidden, seed=seed + 3 * l, plant_frac=0.01)["w"],
             synth.gaussian_bf16(rng, (inter, hidden), 0.03),
             synth.student_t_bf16(rng, (hidden, inter), 3, 0.02)) for l in range(layers)]
    st = MLPStack(m, hidden, inter)
    for lay in mats:
        st.add_layer(*lay)
    x = synth.gaussian_bf16(rng, (m, hidden), 1.0)
    return st, mats, x


@pytest.mark.parametrize("m", [1, 16])
def test_step_tuner_coordinate_descent(m, tmp_path):
    """The tuned configuration is the fastest of everything the descent measured, no slower than
    its start (the default), and the step it runs equals the oracle-checked step bit for bit:
    every GEMM of the traced (unfused) step under the tuned configuration within the oracle
    bound on the device's own inputs, and the fused step ending in the same bits.  The per-model
    file round-trips."""
    t = torch()
    from lossless_bf16_weight_amd.stack import PROJECTIONS, as_bf16_bits
    st, mats, x = _small_stack(m)
    xd = t.from_numpy(x.view(np.int16)).cuda()
    tuner = autotune.StepTuner(st, xd, variants=[-1, 5, 9, 10, 14], steps=4, rounds=3)
    res = tuner.tune(max_sweeps=3)
    assert res["us"] == min(us for _, us in tuner.evals)
    assert res["us"] <= res["default_us"]
    assert res["sweeps"] >= 1 and len(tuner.evals) >= 1 + 3 * (len(tuner.candidates()) - 1)
    cfg = res["config"]
    trace = []
    st.step(xd, config=cfg, trace=trace)
    for l, (xi, g, u, h, y, xo) in enumerate(trace):
        xi, h = as_bf16_bits(xi), as_bf16_bits(h)
        for (inp, out), wm in zip(((xi, g), (xi, u), (h, y)), mats[l]):
            y_ref, s_ = gemm.gemm_ref(inp, wm)
            ok = gemm.within_bound(out.astype(np.float64), y_ref, s_)
            assert ok.all(), "layer %d: %d outside bound under %s" % (l, (~ok).sum(), cfg)
    fused = st.step(xd, config=cfg)
    assert np.array_equal(as_bf16_bits(fused), as_bf16_bits(trace[-1][5]))
    path = tmp_path / "model.json"
    autotune.save_model_config(str(path), "test-mlp", m, res)
    cfg2, split = autotune.load_model_config(str(path))
    assert cfg2 == {k: tuple(cfg[k]) for k in PROJECTIONS} and split == 0


def test_step_tuner_split_coordinate():
    """The decode/GEMM split of a stack with hard layers: the chosen decoder workgroup count is
    the argmin of its own measurements, and every split gives the plain step's bits."""
    t = torch()
    from lossless_bf16_weight_amd.stack import HardEasyStack
    st, mats, x = _small_stack(16, layers=4, seed=71)
    xd = t.from_numpy(x.view(np.int16)).cuda()
    ref = st.step(xd, pipeline=uw.UW_PIPE_DIRECT_PALETTE).clone()
    outs = {}

    def make(split):
        hs = HardEasyStack(16, 256, 704, mats, hard_layers=(1, 3), decode_workgroups=split)
        outs[split] = hs.step(xd).clone()
        return hs

    res = autotune.StepTuner.tune_split(make, xd, splits=(0, 1, 4), steps=4, rounds=3)
    assert res["us"] == min(res["all"].values()) and res["all"][res["decode_workgroups"]] == res["us"]
    for sp, o in outs.items():
        assert t.equal(o, ref), "split %d" % sp
