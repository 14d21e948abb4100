"""GPU parity: every device entry point of libuw against the CPU oracle, through the C ABI.

Bar: bit-exact for decode / transcode / exponent streams (byte work); for GEMMs
|y_gpu - y_ref| <= 1e-3 * sum_k |x_k w_k| per element (y_ref accumulated in fp64);
SwiGLU / RMS-norm glue within one BF16 ulp of the oracle."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import synth
from oracle import codec, gemm

from generated import finite, matrices

pytestmark = pytest.mark.gpu

ALL_PIPES = [uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE, uw.UW_PIPE_EXP_ONLY, uw.UW_PIPE_FULL_DECODE]


def torch():
    import torch as t
    return t


def dev_u16(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda()


def host_u16(t_):
    return t_.cpu().numpy().view(np.uint16)


def check_gemm(y_dev, x, w, rows=None):
    y = y_dev.cpu().numpy().astype(np.float64)
    if rows is None:
        y_ref, s = gemm.gemm_ref(x, w)
    else:
        y_ref, s = gemm.gemm_ref_rows(x, w, rows)
        y = y[:, rows]
    ok = gemm.within_bound(y, y_ref, s)
    bad = np.argwhere(~ok)
    assert ok.all(), "%d/%d outside bound, first %s: gpu %r ref %r S %r" % (
        len(bad), ok.size, bad[:3].tolist(), y[tuple(bad[0])], y_ref[tuple(bad[0])], s[tuple(bad[0])])


def err_ws():
    return torch().zeros(64, dtype=torch().int32, device="cuda")


CASES = {
    "ragged_37x192": lambda: synth.small_gaussian(37, 192, seed=1, plant_frac=0.05)["w"],
    "tiles_160x1024": lambda: synth.small_gaussian(160, 1024, seed=4, plant_frac=0.02)["w"],
    "student_t_48x1024": lambda: synth.student_t_bf16(np.random.default_rng(5), (48, 1024), 3, 0.02),
    "one_row_1x64": lambda: synth.small_gaussian(1, 64, seed=3)["w"],
    "all_verbatim_20x128": lambda: every_segment_verbatim(20, 128, 8),
    "single_exponent_16x128": lambda: np.full((16, 128), 0x3F80, np.uint16) | (np.arange(128, dtype=np.uint16)[None, :] & 0x7F),
    "bimodal_lut_96x512": lambda: bimodal(96, 512, 6),
    "all_zero_32x128": lambda: np.zeros((32, 128), np.uint16),
    "subnormal_48x256": lambda: synth.subnormal_bf16(np.random.default_rng(7), (48, 256)),
}


# Non-finite patterns (NaN payloads, +-Inf) only go through the byte-exact decoders.
DECODE_ONLY = {
    "every_bit_pattern_1024x64": lambda: np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1024, 64),
}


def every_segment_verbatim(n, k, seed):
    """Gaussian weights with one rare (finite, large) exponent planted in every segment:
    each planted exponent is used once, so none enters the palette."""
    rng = np.random.default_rng(seed)
    w = synth.gaussian_bf16(rng, (n, k), 0.02)
    e = 140
    for r in range(n):
        for b in range(k // 64):
            w[r, 64 * b + int(rng.integers(0, 64))] = (e << 7) | int(rng.integers(0, 128))
            e = 140 + (e - 139) % 100
    return w


def bimodal(n, k, seed):
    """Two magnitude scales far apart: the top-16 exponents are not consecutive, so the
    palette is not affine and the kernels take the table-lookup path."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, k)).astype(np.float32)
    scale = np.where(rng.random((n, k)) < 0.5, np.float32(1e-4), np.float32(30.0))
    return synth.f32_to_bf16_bits(a * scale)


@pytest.mark.parametrize("name", list(CASES) + list(DECODE_ONLY))
@pytest.mark.parametrize("chunk", [64, 512, 1024])
def test_decoders_bit_exact(name, chunk):
    t = torch()
    w = {**CASES, **DECODE_ONLY}[name]()
    n, k = w.shape
    blob = uw.uw_encode(w, chunk)
    ref_blob = codec.serialize(codec.encode(w, n, k, chunk=chunk))
    assert blob.tobytes() == ref_blob
    cm = uw.CompressedMatrix(w, chunk=chunk, blob=blob)
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    idx = t.empty(int(cm.info["idx_bytes"]), dtype=t.uint8, device="cuda")
    uw.uw_transcode_palette(cm.d, idx, ws)
    uw.uw_check(ws)
    assert idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    assert cm.idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()


@pytest.mark.parametrize("name", ["tiles_160x1024", "student_t_48x1024", "ragged_37x192"] + list(DECODE_ONLY))
@pytest.mark.parametrize("chunk", [256, 512])
@pytest.mark.parametrize("in_kernel", [True, False])
def test_row_decoder_table_source(name, chunk, in_kernel, monkeypatch):
    """The row decoder's lookup table either comes from the table built on the host at bind
    time (LDS-DMA) or is built by each workgroup (UW_ROW_TABLE_IN_KERNEL, also the path when the
    per-device table cache is full): both decode bit-exact against the oracle."""
    if in_kernel:
        monkeypatch.setenv("UW_ROW_TABLE_IN_KERNEL", "1")
    else:
        monkeypatch.delenv("UW_ROW_TABLE_IN_KERNEL", raising=False)
    t = torch()
    w = {**CASES, **DECODE_ONLY}[name]()
    n, k = w.shape
    blob = uw.uw_encode(w, chunk)
    ref_blob = codec.serialize(codec.encode(w, n, k, chunk=chunk))
    cm = uw.CompressedMatrix(w, chunk=chunk, blob=blob)
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    idx = t.empty(int(cm.info["idx_bytes"]), dtype=t.uint8, device="cuda")
    uw.uw_transcode_palette(cm.d, idx, ws)
    uw.uw_check(ws)
    assert idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()


@pytest.mark.parametrize("name", ["tiles_160x1024", "ragged_37x192"])
@pytest.mark.parametrize("chunk", [256, 512, 1024])
@pytest.mark.parametrize("in_kernel", [True, False])
def test_decoders_13_bit_codes(name, chunk, in_kernel, monkeypatch):
    """The encoders limit codes to 12 bits, but a blob may hold codes of up to 13 (the format's
    limit).  Oracle blobs written at that limit hold 13-bit codes for these inputs; every decoder
    (the row decoder through its secondary table entries, with either table source; the general
    decoder at 1024-symbol chunks) decodes them bit-exact."""
    if in_kernel:
        monkeypatch.setenv("UW_ROW_TABLE_IN_KERNEL", "1")
    else:
        monkeypatch.delenv("UW_ROW_TABLE_IN_KERNEL", raising=False)
    t = torch()
    w = CASES[name]()
    n, k = w.shape
    enc = codec.encode(w, n, k, chunk=chunk, lmax=13)
    assert max(enc["lengths"]) == 13
    ref_blob = codec.serialize(enc)
    cm = uw.CompressedMatrix(w, chunk=chunk, blob=np.frombuffer(ref_blob, np.uint8).copy())
    assert cm.info["lmax"] == 13
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    idx = t.empty(int(cm.info["idx_bytes"]), dtype=t.uint8, device="cuda")
    uw.uw_transcode_palette(cm.d, idx, ws)
    uw.uw_check(ws)
    assert idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()


@settings(max_examples=25, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(matrices(max_rows=70, max_blocks=8), st.sampled_from([64, 256, 512]), st.integers(1, 40))
def test_generated_matrices(w, chunk, m):
    """Generated matrices (random shapes; Gaussian, few-exponent, many-exponent and raw-bit
    values with signed zeros, subnormals, infinities and NaN payloads sprinkled in): the three
    device decoders bit-exact against the oracle, and the direct-palette GEMM of the same matrix
    with its non-finite values replaced within the bound at a random batch size."""
    t = torch()
    n, k = w.shape
    ref_blob = codec.serialize(codec.encode(w, n, k, chunk=chunk))
    cm = uw.CompressedMatrix(w, chunk=chunk)
    assert cm.blob.tobytes() == ref_blob
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    assert cm.idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()
    wf = finite(w)
    cf = uw.CompressedMatrix(wf, chunk=chunk)
    x = synth.gaussian_bf16(np.random.default_rng(m), (m, k), 1.0)
    y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
    uw.uw_gemm(cf.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, cf.workspace(m, uw.UW_PIPE_DIRECT_PALETTE))
    check_gemm(y, x, wf)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("m", [1, 5, 16, 17, 40, 128, 200])
def test_gemm_all_pipelines(name, m):
    t = torch()
    w = CASES[name]()
    n, k = w.shape
    x = synth.gaussian_bf16(np.random.default_rng(100 + m), (m, k), 1.0)
    cm = uw.CompressedMatrix(w, chunk=128)
    xd = dev_u16(x)
    for pipe in ALL_PIPES:
        ws = cm.workspace(m, pipe)
        y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm(cm.d, xd, y, m, pipe, ws)
        if ws is not None:
            uw.uw_check(ws)
        check_gemm(y, x, w)


def _other_palette(w, shift, swap=0):
    """Another matrix's palette: W's own top 16 moved by `shift` octaves; with swap > 0 its
    `swap` smallest exponents are replaced by distant large ones (a gap makes the palette
    non-affine, so the kernels take the table-lookup path)."""
    n, k = w.shape
    own = sorted(int(x) for x in codec.analyse(w, n, k)["palette"])
    own = own[swap:] + [200 + i for i in range(swap)]
    return sorted({min(255, max(0, x + shift)) for x in own})


@pytest.mark.parametrize("shift,swap", [(5, 0), (0, 3), (-1, 0)], ids=["shift5", "gap_lut", "shift-1"])
def test_caller_palette_end_to_end(shift, swap):
    """uw_encode with a caller palette (another matrix's, so a large share of segments is
    verbatim): the blob is the oracle's, every decoder is bit-exact, and every pipeline's GEMM
    is within the oracle bound."""
    t = torch()
    w = synth.small_gaussian(200, 1024, seed=17, plant_frac=0.02)["w"]
    n, k = w.shape
    pal = _other_palette(w, shift, swap)
    blob = uw.uw_encode(w, 256, palette=pal)
    ref_blob = codec.serialize(codec.encode(w, n, k, chunk=256, palette=pal))
    assert blob.tobytes() == ref_blob
    info = uw.uw_blob_info(blob)
    assert list(info["palette"][: len(pal)]) == pal and 0 < info["n_verb"] < n * k // 64
    assert bool(info["affine"]) == (swap == 0)
    cm = uw.CompressedMatrix(w, blob=blob)
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    assert cm.idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()
    for m in (1, 16, 64):
        x = synth.gaussian_bf16(np.random.default_rng(300 + m), (m, k), 1.0)
        for pipe in ALL_PIPES:
            wsp = cm.workspace(m, pipe)
            y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm(cm.d, dev_u16(x), y, m, pipe, wsp)
            if wsp is not None:
                uw.uw_check(wsp)
            check_gemm(y, x, w)


N_VARIANTS = 21
SHARED_X_VARIANTS = (14, 15)   # kind 2: whole tiles per wave, X rows shared in LDS
WIDE_VARIANTS = (16, 17)       # kind 3: tile pairs per wave, 32x32 MFMAs (palette sources)
BIG_VARIANTS = (18, 19, 20)    # kinds 4, 5: W rebuilt once a block into LDS, 32x32 MFMAs (palette sources)


def test_variant_count():
    assert uw.uw_variant_count() == N_VARIANTS


@pytest.mark.parametrize("variant", range(N_VARIANTS))
def test_gemm_every_variant(variant):
    """Every kernel variant, with and without a workspace (the multi-tile kernel splits K
    over workgroups only when it has room for the partial sums), at batch sizes that take
    1, 2, 4 and 8 MFMA column tiles and a second column group."""
    t = torch()
    w = synth.small_gaussian(200, 2048, seed=11, plant_frac=0.05)["w"]
    cm = uw.CompressedMatrix(w)
    for m in (1, 24, 70, 128, 200):
        x = synth.gaussian_bf16(np.random.default_rng(m), (m, 2048), 1.0)
        for ws in (None, cm.workspace(m, uw.UW_PIPE_DIRECT_PALETTE)):
            y = t.full((m, 200), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, variant, ws)
            check_gemm(y, x, w)
        yb = t.full((m, 200), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm_bf16(dev_u16(w), dev_u16(x), yb, m, variant)
        check_gemm(yb, x, w)


@pytest.mark.parametrize("variant", range(N_VARIANTS))
def test_gemm_long_k_every_variant(variant):
    """k = 9216 (144 blocks: more than one flag register of blocks, so the multi-tile kernel
    needs several K slices), ragged rows, verbatim segments; the exponent and transcode
    pipelines too."""
    t = torch()
    w = synth.small_gaussian(70, 9216, seed=13, plant_frac=0.1)["w"]
    cm = uw.CompressedMatrix(w)
    for m in (3, 40):
        x = synth.gaussian_bf16(np.random.default_rng(m), (m, 9216), 1.0)
        for pipe in (uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_EXP_ONLY, uw.UW_PIPE_TRANSCODE):
            ws = cm.workspace(m, pipe)
            y = t.full((m, 70), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, pipe, variant, ws)
            uw.uw_check(ws)
            check_gemm(y, x, w)
        y = t.full((m, 70), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, variant, None)
        check_gemm(y, x, w)
        yb = t.full((m, 70), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm_bf16(dev_u16(w), dev_u16(x), yb, m, variant)
        check_gemm(yb, x, w)


@pytest.mark.parametrize("variant", WIDE_VARIANTS)
@pytest.mark.parametrize("case", ["odd_pairs", "lut_palette", "long_k"])
def test_gemm_wide_tiles(variant, case):
    """The wide-tile kernel (a wave rebuilds two row tiles, 32x32 MFMAs): an odd tile count
    (the last pair holds one tile) and ragged rows, the table-lookup palette, and k = 9216
    (several K slices, flag words past the first 64 blocks), with and without room for the
    partial sums, across 1, 2 and 3 column chunks of 128 X rows and a ragged last chunk."""
    t = torch()
    w = {"odd_pairs": lambda: synth.small_gaussian(200, 2048, seed=19, plant_frac=0.05)["w"],
         "lut_palette": lambda: bimodal(96, 512, 6),
         "long_k": lambda: synth.small_gaussian(70, 9216, seed=23, plant_frac=0.1)["w"]}[case]()
    n, k = w.shape
    cm = uw.CompressedMatrix(w)
    assert uw.uw_variant_name(variant).startswith("wide ")
    for m in (17, 128, 129, 300):
        x = synth.gaussian_bf16(np.random.default_rng(900 + m), (m, k), 1.0)
        for pipe in (uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE):
            for ws in (None, cm.workspace(m, pipe)):
                if pipe == uw.UW_PIPE_TRANSCODE and ws is None:
                    continue
                y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
                uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, pipe, variant, ws)
                if ws is not None:
                    uw.uw_check(ws)
                check_gemm(y, x, w)


@pytest.mark.parametrize("variant", BIG_VARIANTS)
@pytest.mark.parametrize("case", ["ragged_rows", "lut_palette", "long_k", "odd_blocks"])
def test_gemm_big_tiles(variant, case):
    """The big-tile kernel (the workgroup rebuilds each block's weight rows once into LDS,
    32x32 MFMAs on LDS operands, two or three blocks in flight): a row count that leaves the
    last workgroup's rows partly empty and ragged, the table-lookup palette, k = 9216 (several
    K slices and flag words past the first 64 blocks), and k = 1216 (19 blocks: every
    remainder of a slice's block count modulo the pipeline depth, slices of one and two
    blocks), with and without room for the partial sums, across one, two and three column
    chunks of 256 X rows and ragged last chunks."""
    t = torch()
    w = {"ragged_rows": lambda: synth.small_gaussian(200, 2048, seed=29, plant_frac=0.05)["w"],
         "lut_palette": lambda: bimodal(96, 512, 6),
         "long_k": lambda: synth.small_gaussian(70, 9216, seed=31, plant_frac=0.1)["w"],
         "odd_blocks": lambda: synth.small_gaussian(150, 1216, seed=37, plant_frac=0.05)["w"]}[case]()
    n, k = w.shape
    cm = uw.CompressedMatrix(w)
    assert uw.uw_variant_name(variant).startswith("big ")
    for m in (17, 256, 257, 600):
        x = synth.gaussian_bf16(np.random.default_rng(700 + m), (m, k), 1.0)
        for pipe in (uw.UW_PIPE_DIRECT_PALETTE, uw.UW_PIPE_TRANSCODE):
            for ws in (None, cm.workspace(m, pipe)):
                if pipe == uw.UW_PIPE_TRANSCODE and ws is None:
                    continue
                y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
                uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, pipe, variant, ws)
                if ws is not None:
                    uw.uw_check(ws)
                check_gemm(y, x, w)


@pytest.mark.parametrize("variant", SHARED_X_VARIANTS)
@pytest.mark.parametrize("shape", [(200, 4096), (1000, 1024), (37, 2048)], ids=["200x4096", "1000x1024", "37x2048"])
def test_gemm_shared_x(variant, shape):
    """The shared-X per-tile kernel (each wave a whole tile, the workgroup's X rows staged once
    in LDS) at every batch size it takes, 1..16: ragged tile counts (the last workgroup holds
    tiles past n), verbatim segments, up to 131 KB of X in LDS at k = 4096, M = 16."""
    t = torch()
    n, k = shape
    w = synth.small_gaussian(n, k, seed=17, plant_frac=0.05)["w"]
    cm = uw.CompressedMatrix(w)
    assert uw.uw_variant_name(variant).startswith("shared-x ")
    for m in (1, 2, 5, 8, 16):
        x = synth.gaussian_bf16(np.random.default_rng(500 + m), (m, k), 1.0)
        y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, variant, None)
        check_gemm(y, x, w)
        y2 = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm_variant(cm.d, dev_u16(x), y2, m, uw.UW_PIPE_TRANSCODE, variant, cm.workspace(m, uw.UW_PIPE_TRANSCODE))
        check_gemm(y2, x, w)


def test_shared_workspace_across_calls():
    """One zeroed workspace serves a sequence of calls on different matrices, batch sizes and
    pipelines (each call must leave the K-split counters as it found them), and repeating the
    sequence reproduces every output bit for bit (partial sums are added in slice order)."""
    t = torch()
    mats = [synth.small_gaussian(200, 2048, seed=31, plant_frac=0.05)["w"],
            synth.small_gaussian(70, 9216, seed=32, plant_frac=0.1)["w"]]
    cms = [uw.CompressedMatrix(w) for w in mats]
    calls = [(i, m, p) for i in range(2) for m in (24, 70, 128, 200) for p in ALL_PIPES]
    size = max(uw.uw_workspace_size(cms[i].d, m, p) for i, m, p in calls)
    ws = t.zeros(size, dtype=t.uint8, device="cuda")
    first = {}
    for rep in range(2):
        for i, m, p in calls:
            w = mats[i]
            x = synth.gaussian_bf16(np.random.default_rng(1000 + m), (m, w.shape[1]), 1.0)
            y = t.full((m, w.shape[0]), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(cms[i].d, dev_u16(x), y, m, p, 13 if m > 16 else -1, ws)
            uw.uw_check(ws)
            out = y.cpu().numpy()
            if rep == 0:
                check_gemm(y, x, w)
                first[(i, m, p)] = out
            else:
                assert np.array_equal(out, first[(i, m, p)]), (i, m, p)


def test_bf16_gemm_ragged_rows():
    t = torch()
    w = synth.small_gaussian(45, 320, seed=2)["w"]
    x = synth.gaussian_bf16(np.random.default_rng(3), (3, 320), 1.0)
    y = t.empty((3, 45), dtype=t.float32, device="cuda")
    uw.uw_gemm_bf16(dev_u16(w), dev_u16(x), y, 3)
    check_gemm(y, x, w)


def test_config1_end_to_end():
    """Config 1: encode -> decode (bit-exact) -> GEMV, fp32 output."""
    t = torch()
    c = synth.config1()
    w, x = c["w"], c["x"]
    cm = uw.CompressedMatrix(w)
    ws = err_ws()
    out = t.empty((1024, 1024), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    for pipe in ALL_PIPES:
        y = cm.gemm(dev_u16(x), pipeline=pipe)
        check_gemm(y, x, w)
    assert cm.info["n_verb"] > 0 and cm.info["affine"] == 1


@pytest.mark.parametrize("name", ["ragged_37x192", "tiles_160x1024", "bimodal_lut_96x512", "all_verbatim_20x128"])
@pytest.mark.parametrize("m", [256, 300, 1024])
def test_gemm_large_batch(name, m):
    """Batches up to the largest M the library takes: every pipeline against the fp64
    oracle bound, M split into several column chunks (and a ragged last chunk at 300)."""
    t = torch()
    w = CASES[name]()
    n, k = w.shape
    x = synth.gaussian_bf16(np.random.default_rng(7 + m), (m, k), 1.0)
    cm = uw.CompressedMatrix(w, chunk=256)
    xd = dev_u16(x)
    for pipe in ALL_PIPES:
        ws = cm.workspace(m, pipe)
        y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
        uw.uw_gemm(cm.d, xd, y, m, pipe, ws)
        if ws is not None:
            uw.uw_check(ws)
        check_gemm(y, x, w)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_every_entry_point(seed):
    """Seeded random sweep: row counts 1..300 (ragged tiles), k = 64..1536, chunk 64..1024,
    Gaussian / Student-t / two-scale values with 0-20 % planted outlier rows.  The blob equals
    the oracle's byte for byte; the three decoders equal the oracle's decodes; every pipeline
    (and the wide-tile variant for M > 16) is within the oracle's GEMM bound."""
    t = torch()
    rng = np.random.default_rng(1000 + seed)
    n, k = int(rng.integers(1, 301)), 64 * int(rng.integers(1, 25))
    chunk = 64 * int(rng.integers(1, 17))
    kind = seed % 3
    if kind == 0:
        w = synth.gaussian_bf16(rng, (n, k), float(rng.uniform(0.005, 0.05)))
    elif kind == 1:
        w = synth.student_t_bf16(rng, (n, k), 3, 0.02)
    else:
        w = bimodal(n, k, 3000 + seed)
    synth.plant_outliers(rng, w, float(rng.choice([0.0, 0.01, 0.2])))
    blob = uw.uw_encode(w, chunk)
    ref_blob = codec.serialize(codec.encode(w, n, k, chunk=chunk))
    assert blob.tobytes() == ref_blob, "n=%d k=%d chunk=%d" % (n, k, chunk)
    cm = uw.CompressedMatrix(w, chunk=chunk, blob=blob)
    ws = err_ws()
    out = t.empty((n, k), dtype=t.int16, device="cuda")
    uw.uw_decode_full(cm.d, out, ws)
    uw.uw_check(ws)
    assert np.array_equal(host_u16(out), w)
    assert cm.idx.cpu().numpy().tobytes() == codec.transcode_blob(ref_blob).tobytes()
    ex = t.empty(int(cm.info["np"]) * k, dtype=t.uint8, device="cuda")
    uw.uw_decode_exponents(cm.d, ex, ws)
    uw.uw_check(ws)
    assert ex.cpu().numpy().tobytes() == codec.exponent_stream_blob(ref_blob).tobytes()
    for m in (1, int(rng.integers(2, 17)), int(rng.integers(17, 200))):
        x = synth.gaussian_bf16(rng, (m, k), 1.0)
        for pipe in ALL_PIPES:
            wsp = cm.workspace(m, pipe)
            y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm(cm.d, dev_u16(x), y, m, pipe, wsp)
            if wsp is not None:
                uw.uw_check(wsp)
            check_gemm(y, x, w)
        if m > 16:
            y = t.full((m, n), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, WIDE_VARIANTS[-1],
                               cm.workspace(m, uw.UW_PIPE_DIRECT_PALETTE))
            check_gemm(y, x, w)


def test_corrupt_stream_matches_oracle():
    """Flipped stream bits (tables intact, every read in bounds).  Where the oracle's
    chunk-end check detects the corruption the GPU must report UW_E_DATA; where a flip
    resynchronises undetected, the GPU must produce exactly the oracle's decode of the
    corrupted blob."""
    t = torch()
    w = synth.small_gaussian(64, 1024, seed=21)["w"]
    blob = uw.uw_encode(w, 256)
    info = uw.uw_blob_info(blob)
    wo = int(info["sec_off"][6])
    seen = {True: 0, False: 0}
    for pos, bit in [(40, 0x10), (41, 0x01), (300, 0x80), (1000, 0x04), (1501, 0x40), (2222, 0x02), (3000, 0x08)]:
        bad = blob.copy()
        bad[wo + pos] ^= bit
        try:
            ref = codec.decode_blob(bad.tobytes())
            detected = False
        except ValueError:
            detected = True
        seen[detected] += 1
        d = uw.DMat(bad, t.from_numpy(bad).cuda())
        ws = err_ws()
        out = t.empty((64, 1024), dtype=t.int16, device="cuda")
        uw.uw_decode_full(d, out, ws)
        if detected:
            with pytest.raises(uw.UwError) as ei:
                uw.uw_check(ws)
            assert ei.value.status == uw.UW_E_DATA
            uw.uw_check(ws)  # the error word was cleared
        else:
            uw.uw_check(ws)
            assert np.array_equal(host_u16(out), ref)
    assert seen[True] >= 1


def test_argument_errors_launch_nothing():
    t = torch()
    w = synth.small_gaussian(32, 128, seed=1)["w"]
    cm = uw.CompressedMatrix(w)
    x = dev_u16(synth.gaussian_bf16(np.random.default_rng(1), (1, 128), 1.0))
    y = t.empty((1, 32), dtype=t.float32, device="cuda")
    for m in (0, uw.UW_MAX_M + 1):
        with pytest.raises(uw.UwError) as ei:
            uw.uw_gemm(cm.d, x, y, m, uw.UW_PIPE_DIRECT_PALETTE)
        assert ei.value.status == uw.UW_E_SHAPE
    with pytest.raises(uw.UwError) as ei:
        uw.uw_gemm(cm.d, x, y, 1, uw.UW_PIPE_TRANSCODE, None)
    assert ei.value.status == uw.UW_E_WORKSPACE
    d2 = uw.DMat(cm.blob, cm.blob_dev, None)
    with pytest.raises(uw.UwError) as ei:
        uw.uw_gemm(d2, x, y, 1, uw.UW_PIPE_DIRECT_PALETTE)
    assert ei.value.status == uw.UW_E_ARG


def test_binding_refuses_wrong_buffers():
    """Short, non-contiguous or wrongly typed device buffers are refused by the binding
    (ValueError) before a kernel could read or write past them."""
    t = torch()
    w = synth.small_gaussian(32, 128, seed=1)["w"]
    cm = uw.CompressedMatrix(w)
    x = dev_u16(synth.gaussian_bf16(np.random.default_rng(1), (4, 128), 1.0))
    y = t.empty((4, 32), dtype=t.float32, device="cuda")
    with pytest.raises(ValueError, match="needs at least"):
        uw.uw_gemm(cm.d, x, y[:2], 4, uw.UW_PIPE_DIRECT_PALETTE)             # y too short for m = 4
    with pytest.raises(ValueError, match="needs at least"):
        uw.uw_gemm(cm.d, x[:1], y, 4, uw.UW_PIPE_DIRECT_PALETTE)             # x too short
    with pytest.raises(ValueError, match="contiguous"):
        uw.uw_gemm(cm.d, x, t.empty((32, 4), dtype=t.float32, device="cuda").t(), 4, uw.UW_PIPE_DIRECT_PALETTE)
    with pytest.raises(ValueError, match="dtype"):
        uw.uw_gemm(cm.d, x.float(), y, 4, uw.UW_PIPE_DIRECT_PALETTE)
    with pytest.raises(ValueError, match="needs at least"):
        uw.uw_decode_full(cm.d, t.empty((16, 128), dtype=t.int16, device="cuda"), err_ws())
    with pytest.raises(ValueError, match="needs at least"):
        uw.DMat(cm.blob, cm.blob_dev[:100])
    with pytest.raises(ValueError, match="needs at least"):
        uw.uw_swiglu(t.zeros(64, device="cuda"), t.zeros(32, device="cuda"), t.zeros(64, dtype=t.int16, device="cuda"))
    # the right buffers still work after the refusals
    uw.uw_gemm(cm.d, x, y, 4, uw.UW_PIPE_DIRECT_PALETTE)
    check_gemm(y, host_u16(x), w)


@pytest.mark.parametrize("shape", [(16, 1000), (7, 333), (1, 4)])
def test_swiglu(shape):
    """SwiGLU glue within one BF16 ulp of the oracle: the 4-wide path (element count a
    multiple of 4) and the scalar path."""
    t = torch()
    rng = np.random.default_rng(4)
    g = (rng.standard_normal(shape) * 3).astype(np.float32)
    u = rng.standard_normal(shape).astype(np.float32)
    h = t.empty(shape, dtype=t.int16, device="cuda")
    uw.uw_swiglu(t.from_numpy(g).cuda(), t.from_numpy(u).cuda(), h)
    ref = gemm.swiglu_ref(g, u).astype(np.int32)
    assert np.abs(host_u16(h).astype(np.int32) - ref).max() <= 1


@pytest.mark.parametrize("shape", [(16, 4096), (2, 6000), (2, 12000), (3, 1001), (1, 20000), (5, 4)])
def test_rmsnorm(shape):
    """Weightless RMS norm within one BF16 ulp of the oracle: one, two and four vectors a
    thread, and the scalar kernel (row length not a multiple of 4, or past 16384)."""
    t = torch()
    rng = np.random.default_rng(5)
    y = (rng.standard_normal(shape) * 5).astype(np.float32)
    xo = t.empty(shape, dtype=t.int16, device="cuda")
    uw.uw_rmsnorm(t.from_numpy(y).cuda(), xo)
    ref = gemm.rmsnorm_ref(y).astype(np.int32)
    assert np.abs(host_u16(xo).astype(np.int32) - ref).max() <= 1


@pytest.mark.parametrize("name", ["ragged_37x192", "tiles_160x1024", "bimodal_lut_96x512"])
def test_gemm_swiglu_equals_unfused(name):
    """uw_gemm_swiglu gives exactly uw_gemm_variant then uw_swiglu: every variant and pipeline,
    per-tile and multi-tile kernels, with the K-slice reduction (workspace) and without."""
    t = torch()
    w = CASES[name]()
    n, k = w.shape
    cm = uw.CompressedMatrix(w)
    rng = np.random.default_rng(11)
    for m in (1, 5, 16, 17, 40, 128):
        x = dev_u16(synth.gaussian_bf16(rng, (m, k), 1.0))
        gate = t.from_numpy((rng.standard_normal((m, n)) * 2).astype(np.float32)).cuda()
        y = t.empty((m, n), dtype=t.float32, device="cuda")
        h_ref = t.empty((m, n), dtype=t.int16, device="cuda")
        h = t.empty((m, n), dtype=t.int16, device="cuda")
        for pipe in ALL_PIPES:
            ws_full = cm.workspace(m, pipe)
            variants = range(N_VARIANTS) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (-1,)
            for variant in variants:
                for ws in ((ws_full, None) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (ws_full,)):
                    uw.uw_gemm_variant(cm.d, x, y, m, pipe, variant, ws)
                    uw.uw_swiglu(gate, y, h_ref)
                    h.fill_(0x7FFF)
                    uw.uw_gemm_swiglu(cm.d, x, gate, h, m, pipe, variant, ws)
                    assert t.equal(h, h_ref), "m=%d pipeline %d variant %d ws %s" % (
                        m, pipe, variant, "yes" if ws is not None else "no")
        if m == 1:
            check_gemm(y, host_u16(x), w)
    x1 = dev_u16(synth.gaussian_bf16(rng, (1, k), 1.0))
    g1 = t.zeros(n + 4, dtype=t.float32, device="cuda")
    with pytest.raises(uw.UwError) as ei:   # gate must be 16-byte aligned
        uw.uw_gemm_swiglu(cm.d, x1, g1[1:], h, 1, uw.UW_PIPE_DIRECT_PALETTE)
    assert ei.value.status == uw.UW_E_ARG


def test_stack_fused_equals_unfused():
    """A two-layer MLP stack: the fused step (SwiGLU in the up GEMM's epilogue, the RMS norm
    with the down GEMM) ends in the same bits as the unfused one."""
    t = torch()
    from lossless_bf16_weight_amd.stack import MLPStack
    rng = np.random.default_rng(12)
    hidden, inter, m = 256, 704, 16
    st = MLPStack(m, hidden, inter)
    for _ in range(2):
        st.add_layer(synth.gaussian_bf16(rng, (inter, hidden), 0.03), synth.gaussian_bf16(rng, (inter, hidden), 0.03),
                     synth.gaussian_bf16(rng, (hidden, inter), 0.02))
    x = dev_u16(synth.gaussian_bf16(rng, (m, hidden), 1.0))
    a = st.step(x, pipeline=uw.UW_PIPE_DIRECT_PALETTE, fused=False).clone()
    b = st.step(x, pipeline=uw.UW_PIPE_DIRECT_PALETTE, fused=True).clone()
    assert t.equal(a, b)


@pytest.mark.parametrize("name", ["ragged_37x192", "tiles_160x1024", "student_t_48x1024"])
def test_gemm_rmsnorm_equals_unfused(name):
    """uw_gemm_rmsnorm gives exactly uw_gemm_variant then uw_rmsnorm (y and the normed rows):
    every variant and pipeline, with the K-slice reduction (the norm fused into it) and without."""
    t = torch()
    w = CASES[name]()
    n, k = w.shape
    cm = uw.CompressedMatrix(w)
    rng = np.random.default_rng(13)
    for m in (1, 16, 17, 40, 128):
        x = dev_u16(synth.gaussian_bf16(rng, (m, k), 1.0))
        y_ref = t.empty((m, n), dtype=t.float32, device="cuda")
        xn_ref = t.empty((m, n), dtype=t.int16, device="cuda")
        y = t.empty((m, n), dtype=t.float32, device="cuda")
        xn = t.empty((m, n), dtype=t.int16, device="cuda")
        for pipe in ALL_PIPES:
            ws_full = cm.workspace(m, pipe)
            variants = range(N_VARIANTS) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (-1,)
            for variant in variants:
                for ws in ((ws_full, None) if pipe == uw.UW_PIPE_DIRECT_PALETTE else (ws_full,)):
                    uw.uw_gemm_variant(cm.d, x, y_ref, m, pipe, variant, ws)
                    uw.uw_rmsnorm(y_ref, xn_ref, 1e-5)
                    y.fill_(float("nan"))
                    xn.fill_(0x7FFF)
                    uw.uw_gemm_rmsnorm(cm.d, x, y, xn, m, 1e-5, pipe, variant, ws)
                    what = "m=%d pipeline %d variant %d ws %s" % (m, pipe, variant, "yes" if ws is not None else "no")
                    assert t.equal(y, y_ref), what
                    assert t.equal(xn, xn_ref), what


@pytest.mark.parametrize("split", [0, 2])
@pytest.mark.parametrize("m", [1, 16])
@pytest.mark.parametrize("hard", [(), (0,), (1, 2), (3,), (0, 1, 2, 3)], ids=["none", "first", "middle", "last", "all"])
def test_hard_easy_stack_equals_plain(m, hard, split):
    """The hard/easy scheduler (uw_sched_*: hard layers keep only their bundle, their index
    streams decoded on a side stream into two alternating slot sets ahead of use) gives the
    same bits as the plain fused step on the same matrices, for three steps in a row (each
    step's first decodes reuse slots the previous step's last hard layers used)."""
    t = torch()
    from lossless_bf16_weight_amd.stack import HardEasyStack, MLPStack
    rng = np.random.default_rng(21)
    hidden, inter, layers = 256, 704, 4
    mats = [(synth.gaussian_bf16(rng, (inter, hidden), 0.03), synth.gaussian_bf16(rng, (inter, hidden), 0.03),
             synth.gaussian_bf16(rng, (hidden, inter), 0.02)) for _ in range(layers)]
    plain = MLPStack(m, hidden, inter)
    for lay in mats:
        plain.add_layer(*lay)
    sched = HardEasyStack(m, hidden, inter, mats, hard_layers=hard, decode_workgroups=split)
    for l, lay in enumerate(sched.layers):
        assert all((cm.idx is None) == (l in hard) for cm in lay)
    x = dev_u16(synth.gaussian_bf16(rng, (m, hidden), 1.0))
    xa, xb = x.clone(), x.clone()
    for step in range(3):
        a = plain.step(xa, pipeline=uw.UW_PIPE_DIRECT_PALETTE, fused=True).clone()
        b = sched.step(xb).clone()
        assert t.equal(a, b), "m=%d hard=%s step %d" % (m, hard, step)
        xa, xb = a, b
    assert sched.resident_bytes() < plain.resident_bytes() + 6 * sched.slot_bytes + 1
    sched.close()


@pytest.mark.parametrize("chunk,split", [(64, 0), (128, 2), (256, 0), (256, 3)])
def test_hard_easy_stack_short_chunks(chunk, split):
    """Hard layers whose bundles use shorter chunks (more, shorter decode chains: the decoder's
    16-wave workgroups at 256-symbol chunks), on the whole chip or a persistent grid of `split`
    workgroups: the same bits as the plain step of the default encoding, two steps in a row."""
    t = torch()
    from lossless_bf16_weight_amd.stack import HardEasyStack, MLPStack
    rng = np.random.default_rng(23)
    hidden, inter, layers, m = 256, 704, 3, 16
    mats = [(synth.small_gaussian(inter, hidden, seed=300 + 3 * l, plant_frac=0.02)["w"],
             synth.gaussian_bf16(rng, (inter, hidden), 0.03),
             synth.student_t_bf16(rng, (hidden, inter), 3, 0.02)) for l in range(layers)]
    plain = MLPStack(m, hidden, inter)
    for lay in mats:
        plain.add_layer(*lay)
    sched = HardEasyStack(m, hidden, inter, mats, hard_layers=(0, 1, 2), chunk=chunk, decode_workgroups=split)
    assert all(uw.uw_blob_info(cm.blob)["chunk"] == chunk for lay in sched.layers for cm in lay)
    x = dev_u16(synth.gaussian_bf16(rng, (m, hidden), 1.0))
    xa, xb = x.clone(), x.clone()
    for step in range(2):
        a = plain.step(xa, pipeline=uw.UW_PIPE_DIRECT_PALETTE, fused=True).clone()
        b = sched.step(xb).clone()
        assert t.equal(a, b), "chunk=%d split=%d step %d" % (chunk, split, step)
        xa, xb = a, b
    sched.close()


def bf16_key(bits):
    """Monotone integer key of BF16 bit patterns (adjacent keys = adjacent values; +0 and -0
    share key 0)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_swiglu_through_gemm_bound(h, g, x_in, w_up):
    """The fused up GEMM + SwiGLU epilogue, checked on the device's own g and x: for every u
    within the GEMM bound of the oracle's (|u - u_ref| <= 1e-3 S), silu(g) * u lies between
    silu(g) * (u_ref -+ 1e-3 S); h must be within one BF16 step of the rounded ends of that
    interval (the step covers the fp32 silu)."""
    u_ref, s = gemm.gemm_ref(x_in, w_up)
    g64 = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):                          # exp(-g) = inf for g << 0: silu -> -0
        silu = g64 / (1.0 + np.exp(-g64))
    a, b = silu * (u_ref - 1e-3 * s), silu * (u_ref + 1e-3 * s)
    lo = bf16_key(gemm.f64_to_bf16_rne(np.minimum(a, b)))
    hi = bf16_key(gemm.f64_to_bf16_rne(np.maximum(a, b)))
    k = bf16_key(h)
    ok = (k >= lo - 1) & (k <= hi + 1)
    assert ok.all(), "%d of %d SwiGLU outputs outside the interval" % ((~ok).sum(), ok.size)


@pytest.mark.parametrize("m,hard,split", [(1, (0, 2), 0), (16, (0, 2), 0), (1, (0, 1, 2, 3), 0), (16, (0, 1, 2, 3), 0),
                                          (16, (0, 2), 1), (1, (0, 1, 2, 3), 3)],
                         ids=["alternate-1", "alternate-16", "all-1", "all-16", "alternate-16-split1", "all-1-split3"])
def test_hard_easy_stack_against_oracle(m, hard, split):
    """Each GEMM of a scheduled step (hard layers decoded on the side stream) against the
    oracle on the inputs the device fed it (teacher-forced, from the library's per-layer
    trace): gate y = x W^T and down y = h W^T within the GEMM bound, the up GEMM through its
    fused SwiGLU epilogue within the bound's interval, the RMS norm within one BF16 ulp; two
    steps in a row, the second from the first's output.  split > 0: the hard layers' decodes
    run on that many decoder workgroups, which take the decode units in turn."""
    from lossless_bf16_weight_amd.stack import HardEasyStack
    rng = np.random.default_rng(31)
    hidden, inter, layers = 256, 704, 4
    mats = [(synth.small_gaussian(inter, hidden, seed=100 + 3 * l, plant_frac=0.01)["w"],
             synth.gaussian_bf16(rng, (inter, hidden), 0.03),
             synth.student_t_bf16(rng, (hidden, inter), 3, 0.02)) for l in range(layers)]
    sched = HardEasyStack(m, hidden, inter, mats, hard_layers=hard, decode_workgroups=split)
    x = dev_u16(synth.gaussian_bf16(rng, (m, hidden), 1.0))
    for step in range(2):
        trace = []
        out = sched.step(x, trace=trace).clone()
        assert len(trace) == layers
        for l, (xi, g, h, y, xo) in enumerate(trace):
            wg, wu, wd = mats[l]
            xi, h, xo = xi.view(np.uint16), h.view(np.uint16), xo.view(np.uint16)
            check_gemm_host(g, xi, wg, "step %d layer %d gate" % (step, l))
            check_swiglu_through_gemm_bound(h, g, xi, wu)
            check_gemm_host(y, h, wd, "step %d layer %d down" % (step, l))
            assert np.abs(xo.astype(np.int32) - gemm.rmsnorm_ref(y).astype(np.int32)).max() <= 1
        assert np.array_equal(host_u16(out), trace[-1][4].view(np.uint16))
        x = out
    sched.close()


def check_gemm_host(y, x, w, what):
    y_ref, s = gemm.gemm_ref(x, w)
    ok = gemm.within_bound(np.asarray(y, np.float64), y_ref, s)
    assert ok.all(), "%s: %d outside bound" % (what, (~ok).sum())


@pytest.mark.parametrize("k", [28672, 32768], ids=["28_blocks_a_slice", "32_blocks_a_slice"])
def test_gemm_multitile_two_batches_deep(k):
    """The multi-tile kernel's two-batch-deep pipeline (three X buffers, taken when every K
    slice holds 28 or 32 blocks): 16 K slices of a long row, ragged row count, verbatim
    segments, 1, 2 and 4 MFMA column tiles, every multi-tile variant, against the oracle."""
    t = torch()
    w = synth.small_gaussian(300, k, seed=23, plant_frac=0.05)["w"]
    cm = uw.CompressedMatrix(w)
    for m in (8, 17, 40, 64):
        x = synth.gaussian_bf16(np.random.default_rng(900 + m), (m, k), 1.0)
        ws = cm.workspace(m, uw.UW_PIPE_DIRECT_PALETTE)
        for variant in (10, 11, 12, 13):
            y = t.full((m, 300), float("nan"), dtype=t.float32, device="cuda")
            uw.uw_gemm_variant(cm.d, dev_u16(x), y, m, uw.UW_PIPE_DIRECT_PALETTE, variant, ws)
            check_gemm(y, x, w)
