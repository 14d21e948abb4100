"""The C++ encoder at the full workload sizes: its blob must be byte-identical to the oracle's
(compared through the SHA-256 digests the oracle wrote into tests/golden/fullsize_digests.txt),
and the seeded generators must still produce the matrices those digests were taken on."""
import hashlib
import os

import numpy as np
import pytest

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize_digests.txt")
MAKERS = {"c1": synth.config1, "c2": synth.config2, "c3": synth.config3, "c5": synth.config5}


def golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, wd, blob, _tc, _ex, size = line.split()
        out[name] = (wd, blob, int(size))
    return out


@pytest.mark.parametrize("name", list(MAKERS))
def test_host_encoder_matches_oracle_full_size(name):
    wd, blob_sha, size = golden()[name]
    w = MAKERS[name]()["w"]
    assert synth.digest(w) == wd, "seeded generator changed"
    blob = uw.uw_encode(w)
    assert blob.size == size
    assert hashlib.sha256(blob.tobytes()).hexdigest() == blob_sha


def test_config4_streams_match_whole_stack_generation():
    """Per-matrix generation of the MLP stack equals the all-at-once generator, whatever
    the thread count (small shapes)."""
    kw = dict(seed=3, layers=2, m=4, hidden=128, inter=192)
    a = synth.config4(threads=1, **kw)
    b = synth.config4(threads=4, **kw)
    meta = synth.config4_meta(3, 2, 4, 128)
    shapes = ((192, 128), (192, 128), (128, 192))
    assert np.array_equal(a["x"], meta["x"]) and np.array_equal(a["stds"], meta["stds"])
    for l in range(2):
        for j in range(3):
            w = synth.config4_matrix(meta, l, j, shapes)
            assert w.shape == shapes[j]
            assert np.array_equal(a["layers"][l][j], w) and np.array_equal(b["layers"][l][j], w)
    assert 0.01 <= meta["stds"].min() and meta["stds"].max() <= 0.03
