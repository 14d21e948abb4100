"""The allocation-free GEMM entry point (uw_gemm_noalloc, include/uw.h): through the C ABI,
against the workspace entry point (uw_gemm_variant with a uw_workspace_size workspace) and the
oracle, on two calls in a row, the second with a smaller input; and its refusal of a call whose
partial sums would not fit its device scratch (nothing launched)."""
import numpy as np
import pytest

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import synth
from oracle import gemm

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


def run_pair(cm, w, m, variant, seed):
    t = torch()
    n, k = w.shape
    x = synth.gaussian_bf16(np.random.default_rng(seed), (m, k), 1.0)
    xd = t.from_numpy(x.view(np.int16)).cuda()
    y_ws = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
    ws = cm.workspace(m, uw.UW_PIPE_DIRECT_PALETTE)
    uw.uw_gemm_variant(cm.d, xd, y_ws, m, uw.UW_PIPE_DIRECT_PALETTE, variant, ws)
    y_na = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
    uw.uw_gemm_noalloc(cm.d, xd, y_na, m, variant)
    t.cuda.synchronize()
    assert t.equal(y_na, y_ws), "m=%d variant %d: differs from the workspace entry point" % (m, variant)
    y_ref, s = gemm.gemm_ref(x, w)
    ok = gemm.within_bound(y_na.cpu().numpy().astype(np.float64), y_ref, s)
    assert ok.all(), "m=%d variant %d: %d outside the oracle bound" % (m, variant, (~ok).sum())


@pytest.mark.parametrize("variant", [-1, 10, 12, 16])
def test_noalloc_matches_workspace_entry_two_calls(variant):
    """First a call that uses the scratch (a K-split multi-tile or wide-tile launch at m = 64
    on a long-k matrix), then a smaller one (fewer rows, m = 8) that leaves part of the
    previous call's partial sums in the scratch."""
    big = synth.small_gaussian(600, 8192, seed=51, plant_frac=0.02)["w"]
    small = synth.small_gaussian(200, 2048, seed=52, plant_frac=0.02)["w"]
    cm_big, cm_small = uw.CompressedMatrix(big), uw.CompressedMatrix(small)
    run_pair(cm_big, big, 64, variant, 1)
    run_pair(cm_small, small, 8, variant, 2)


def test_noalloc_refuses_what_does_not_fit():
    """n = 20000 at m = 1024 needs at least 20000 * 1024 * 4 B = 81.9 MB of partial sums, more
    than the 64 MiB scratch: refused on the host before any launch."""
    t = torch()
    w = synth.small_gaussian(20000, 64, seed=53)["w"]
    cm = uw.CompressedMatrix(w)
    x = t.zeros((1024, 64), dtype=t.int16, device="cuda")
    y = t.full((1024, 20000), 7.0, dtype=t.float32, device="cuda")
    with pytest.raises(uw.UwError) as ei:
        uw.uw_gemm_noalloc(cm.d, x, y, 1024)
    assert ei.value.status == uw.UW_E_WORKSPACE
    t.cuda.synchronize()
    assert bool((y == 7.0).all())
