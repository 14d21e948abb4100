"""CPU tests of libuw's host side: every declared symbol is exported, the C++ encoder's
blob is byte-identical to the oracle's, the palette matches, and malformed inputs are
rejected with the documented status codes.  No GPU needed (nothing here launches)."""
import os
import re

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from generated import matrices

import lossless_bf16_weight_amd as uw
from lossless_bf16_weight_amd import synth
from oracle import codec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "uw.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(uw_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = uw.lib()
    names = declared_functions()
    assert len(names) >= 20
    for name in names:
        assert hasattr(L, name), name
    assert sorted(uw.EXPORTS) == names
    assert uw.uw_version() == 10000


def oracle_blob(w, chunk=512):
    n, k = w.shape
    return np.frombuffer(codec.serialize(codec.encode(w, n, k, chunk=chunk)), np.uint8)


CASES = [
    ("gauss_ragged", lambda: synth.small_gaussian(37, 192, seed=1, plant_frac=0.05)["w"]),
    ("gauss_tiles", lambda: synth.small_gaussian(160, 512, seed=4, plant_frac=0.02)["w"]),
    ("specials", lambda: np.random.default_rng(2).choice(
        np.array([0, 0x8000, 1, 0x807F, 0x7F80, 0xFF80, 0x7FC0, 0xFFFF, 0x3F80, 0x0080], np.uint16), size=(19, 256))),
    ("single_exponent", lambda: np.full((16, 64), 0x3F80, np.uint16) | np.arange(64, dtype=np.uint16)[None, :]),
    ("all_verbatim", lambda: (np.arange(20 * 64, dtype=np.uint32) * 251).astype(np.uint16).reshape(20, 64)),
    ("one_row", lambda: synth.small_gaussian(1, 64, seed=3)["w"]),
    ("student_t", lambda: synth.student_t_bf16(np.random.default_rng(5), (48, 1024), 3, 0.02)),
    ("uniform_bits", lambda: np.random.default_rng(6).integers(0, 65536, size=(33, 320)).astype(np.uint16)),
    ("all_zero", lambda: np.zeros((32, 128), np.uint16)),
    ("subnormal", lambda: synth.subnormal_bf16(np.random.default_rng(7), (48, 256))),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("chunk", [64, 512, 4096])
def test_encoder_blob_equals_oracle(name, make, chunk):
    w = make()
    blob = uw.uw_encode(w, chunk)
    ref = oracle_blob(w, chunk)
    assert blob.size == ref.size
    assert np.array_equal(blob, ref)


@settings(max_examples=40, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(matrices(), st.sampled_from([64, 128, 512]))
def test_encoder_blob_equals_oracle_generated(w, chunk):
    """Generated matrices (random shapes; Gaussian, few-exponent, many-exponent and raw-bit
    values; signed zeros, subnormals, infinities and NaN payloads sprinkled in): the C++ blob
    equals the oracle's byte for byte, and the oracle decodes it back to W."""
    blob = uw.uw_encode(w, chunk)
    ref = oracle_blob(w, chunk)
    assert np.array_equal(blob, ref)
    assert np.array_equal(codec.decode_blob(ref.tobytes()), w)


@pytest.mark.parametrize("threads", ["1", "3", "8"])
def test_encoder_independent_of_thread_count(threads, monkeypatch):
    monkeypatch.setenv("UW_HOST_THREADS", threads)
    w = synth.small_gaussian(257, 1024, seed=9, plant_frac=0.01)["w"]
    assert np.array_equal(uw.uw_encode(w, 256), oracle_blob(w, 256))


def test_config1_blob_equals_oracle():
    w = synth.config1()["w"]
    assert np.array_equal(uw.uw_encode(w), oracle_blob(w))


def _other_palette(w, shift):
    """Another matrix's palette: W's own top 16 moved by `shift` octaves (oracle's choice)."""
    n, k = w.shape
    own = [int(x) for x in codec.analyse(w, n, k)["palette"]]
    return sorted({min(255, max(0, x + shift)) for x in own})


@pytest.mark.parametrize("name,make", CASES[:2] + CASES[6:7], ids=[CASES[i][0] for i in (0, 1, 6)])
@pytest.mark.parametrize("shift", [0, 1, 5])
@pytest.mark.parametrize("chunk", [64, 512])
def test_encoder_caller_palette_equals_oracle(name, make, shift, chunk):
    """uw_encode with a caller palette (another matrix's, so part of W becomes verbatim) writes
    the oracle's blob byte for byte; with W's own palette (shift 0) the blob equals the
    palette-less encode."""
    w = make()
    n, k = w.shape
    pal = _other_palette(w, shift)
    blob = uw.uw_encode(w, chunk, palette=pal)
    ref = np.frombuffer(codec.serialize(codec.encode(w, n, k, chunk=chunk, palette=pal)), np.uint8)
    assert np.array_equal(blob, ref)
    if shift == 0:
        assert np.array_equal(blob, uw.uw_encode(w, chunk))
        assert np.array_equal(uw.uw_encode(w, chunk, palette=uw.uw_build_palette(w)), blob)


def test_encoder_rejects_bad_caller_palettes():
    import ctypes
    w = synth.small_gaussian(32, 128, seed=1)["w"]
    good = uw._palette_struct([100, 110, 120])
    L = uw.lib()
    used = ctypes.c_size_t()

    def status(p):
        return L.uw_encode(w.ctypes.data, 32, 128, ctypes.byref(p), 0, None, 0, ctypes.byref(used))

    assert status(good) == uw.UW_OK
    for mutate in (lambda p: setattr(p, "n", 0), lambda p: setattr(p, "n", 17),
                   lambda p: p.exp.__setitem__(1, 100),                 # not strictly ascending
                   lambda p: p.index_of.__setitem__(7, 0),              # index_of not the inverse
                   lambda p: p.index_of.__setitem__(110, 2)):
        p = uw._palette_struct([100, 110, 120])
        mutate(p)
        assert status(p) == uw.UW_E_ARG
        assert "palette" in uw.lib().uw_last_error().decode()


def test_palette_matches_oracle():
    w = synth.small_gaussian(64, 640, seed=7, plant_frac=0.1)["w"]
    p = uw.uw_build_palette(w)
    e, _ = codec.split_fields(w)
    hist = codec.exponent_histogram(e)
    pal, index_of = codec.build_palette(hist)
    assert p["exp"] == list(pal) and p["n"] == len(pal)
    assert np.array_equal(p["index_of"], index_of)
    assert np.array_equal(p["hist"], hist)


def test_blob_info_fields():
    w = synth.small_gaussian(50, 256, seed=3, plant_frac=0.05)["w"]
    blob = uw.uw_encode(w)
    info = uw.uw_blob_info(blob)
    enc = codec.encode(w, 50, 256)
    assert info["n"] == 50 and info["k"] == 256 and info["np"] == 64 and info["tiles"] == 4 and info["kb"] == 4
    assert info["n_verb"] == enc["n_verb"] and info["n_coded"] == enc["n_coded"]
    assert info["total_bits"] == enc["total_bits"]
    assert info["palette"][: info["n_pal"]] == list(enc["palette"])
    assert info["resident_bytes"] == codec.resident_palette_bytes(enc)
    assert info["idx_bytes"] == 64 * 256 // 2
    assert info["blob_bytes"] == blob.size
    assert info["affine"] == int(all(enc["palette"][i] == enc["palette"][0] + i for i in range(len(enc["palette"]))))


def test_code_length_limits():
    """The encoders limit codes to 12 bits (every code fits the decoder's 2^12-entry table); a
    blob may hold codes up to the format's 13 bits, and such a blob (the oracle writes one when
    asked for that limit) parses with its limit reported."""
    w = synth.small_gaussian(160, 1024, seed=4, plant_frac=0.02)["w"]
    blob = uw.uw_encode(w)
    info = uw.uw_blob_info(blob)
    assert info["lmax"] == 12 and max(codec.parse(blob)["lengths"]) <= 12
    enc13 = codec.encode(w, 160, 1024, lmax=13)
    assert max(enc13["lengths"]) == 13
    info13 = uw.uw_blob_info(np.frombuffer(codec.serialize(enc13), np.uint8).copy())
    assert info13["lmax"] == 13 and info13["total_bits"] == enc13["total_bits"]


def test_encode_bound_covers_worst_case():
    for w in (CASES[7][1](), CASES[4][1](), synth.small_gaussian(40, 128, seed=1)["w"]):
        n, k = w.shape
        assert uw.uw_encode(w).size <= uw.uw_encode_bound(n, k)


# ------------------------------------------------------------------ error paths
def status_of(fn, *args):
    with pytest.raises(uw.UwError) as ei:
        fn(*args)
    return ei.value.status


def test_shape_errors():
    assert status_of(uw.uw_encode, np.zeros((4, 100), np.uint16)) == uw.UW_E_SHAPE
    assert status_of(uw.uw_encode, np.zeros((4, 32), np.uint16)) == uw.UW_E_ARG
    assert status_of(uw.uw_encode, np.zeros((4, 64), np.uint16), 100) == uw.UW_E_ARG
    assert status_of(uw.uw_build_palette, np.zeros((4, 130), np.uint16)) == uw.UW_E_SHAPE


def corrupt(blob, offset, data):
    b = blob.copy()
    b[offset: offset + len(data)] = np.frombuffer(bytes(data), np.uint8)
    return b


def test_blob_validation_rejects_corruption():
    w = synth.small_gaussian(40, 256, seed=5, plant_frac=0.1)["w"]
    blob = uw.uw_encode(w, 128)
    info = uw.uw_blob_info(blob)
    bad = [
        corrupt(blob, 0, b"XXXX"),                                        # magic
        corrupt(blob, 4, (2).to_bytes(4, "little")),                       # version
        corrupt(blob, 12, (100).to_bytes(4, "little")),                    # k not a multiple of 64
        corrupt(blob, 24, (100).to_bytes(4, "little")),                    # chunk
        corrupt(blob, 80, bytes([1, 1, 1] + [0] * 13)),                     # Kraft violated
        corrupt(blob, 28, (14).to_bytes(4, "little")),                     # limit above the format's 13
        corrupt(blob, 28, (2).to_bytes(4, "little")),                      # a code above the stated limit
        corrupt(blob, 96, (5).to_bytes(2, "little")),                      # non-canonical code
        corrupt(blob, 128 + 16 * 6 + 8, (10 ** 9).to_bytes(8, "little")),  # words section size
        blob[: blob.size - 512],                                           # truncated
    ]
    vp = int(info["sec_off"][2])
    bad.append(corrupt(blob, vp + 4, (999).to_bytes(4, "little")))         # vprefix vs flags
    off = int(info["sec_off"][5])
    bad.append(corrupt(blob, off + 4, (3).to_bytes(4, "little")))           # chunk offset span
    cb = int(info["sec_off"][4])
    bad.append(corrupt(blob, cb + 4, (77).to_bytes(4, "little")))          # cbase
    fl = int(info["sec_off"][1])
    last_tile_flags = fl + 2 * 4 * (info["tiles"] - 1)
    bad.append(corrupt(blob, last_tile_flags, (0x8000).to_bytes(2, "little")))  # flag on a padding row
    for b in bad:
        assert status_of(uw.uw_blob_info, b) == uw.UW_E_FORMAT


def test_autotune_table_roundtrip(tmp_path):
    uw.uw_autotune_clear()
    assert uw.uw_autotune_get(14336, 4096, 1) == (uw.UW_PIPE_DIRECT_PALETTE, -1)
    uw.uw_autotune_set(14336, 4096, 1, uw.UW_PIPE_TRANSCODE, 3)
    assert uw.uw_autotune_get(14336, 4096, 1) == (uw.UW_PIPE_TRANSCODE, 3)
    p = tmp_path / "tune.txt"
    p.write_text("# n k m pipeline variant\n4096 14336 8 1 2\n\n4096 14336 64 4 -1  # comment\n")
    uw.uw_autotune_clear()
    uw.uw_autotune_load(str(p))
    assert uw.uw_autotune_get(4096, 14336, 8) == (uw.UW_PIPE_FULL_DECODE, 2)
    assert uw.uw_autotune_get(4096, 14336, 64) == (uw.UW_PIPE_DIRECT_PALETTE, -1)
    p.write_text("4096 14336 8 9 0\n")
    assert status_of(uw.uw_autotune_load, str(p)) == uw.UW_E_ARG
    assert status_of(uw.uw_autotune_set, 1, 64, 1, uw.UW_PIPE_AUTO, 0) == uw.UW_E_ARG
    uw.uw_autotune_clear()


def test_autotune_model_table_merge(tmp_path):
    """A model's projection shapes tuned separately merge into one table file that the C ABI
    loads: per (n, k, m) the fastest compressed pipeline becomes the AUTO entry, every
    pipeline keeps its own best variant, and a slower later measurement changes nothing."""
    from lossless_bf16_weight_amd import autotune as at
    gate, down = at.Table(), at.Table()
    gate.add(at.Entry(14336, 4096, 16, uw.UW_PIPE_DIRECT_PALETTE, 14, 17.9))
    gate.add(at.Entry(14336, 4096, 16, uw.UW_PIPE_DIRECT_PALETTE, 10, 23.1))
    gate.add(at.Entry(14336, 4096, 16, uw.UW_PIPE_TRANSCODE, 10, 80.0))
    gate.add(at.Entry(14336, 4096, 16, uw.UW_PIPE_BF16, 3, 25.0))
    down.add(at.Entry(4096, 14336, 16, uw.UW_PIPE_EXP_ONLY, 11, 40.0))
    down.add(at.Entry(4096, 14336, 16, uw.UW_PIPE_DIRECT_PALETTE, 12, 18.8))
    model = at.Table().merge(gate).merge(down)
    model.add(at.Entry(4096, 14336, 16, uw.UW_PIPE_DIRECT_PALETTE, 13, 19.5))   # slower: ignored
    assert model.shapes() == [(4096, 14336, 16), (14336, 4096, 16)]
    p = tmp_path / "model.txt"
    model.save(str(p))
    uw.uw_autotune_clear()
    uw.uw_autotune_load(str(p))
    assert uw.uw_autotune_get(14336, 4096, 16) == (uw.UW_PIPE_DIRECT_PALETTE, 14)
    assert uw.uw_autotune_get(4096, 14336, 16) == (uw.UW_PIPE_DIRECT_PALETTE, 12)
    assert uw.uw_autotune_get_variant(14336, 4096, 16, uw.UW_PIPE_TRANSCODE) == 10
    assert uw.uw_autotune_get_variant(14336, 4096, 16, uw.UW_PIPE_BF16) == 3
    assert uw.uw_autotune_get_variant(4096, 14336, 16, uw.UW_PIPE_EXP_ONLY) == 11
    uw.uw_autotune_clear()


def test_autotune_variant_entries(tmp_path):
    uw.uw_autotune_clear()
    assert uw.uw_autotune_get_variant(14336, 4096, 1, uw.UW_PIPE_BF16) == -1
    # an AUTO entry also records the variant of its pipeline
    uw.uw_autotune_set(14336, 4096, 1, uw.UW_PIPE_DIRECT_PALETTE, 6)
    assert uw.uw_autotune_get_variant(14336, 4096, 1, uw.UW_PIPE_DIRECT_PALETTE) == 6
    assert uw.uw_autotune_get_variant(14336, 4096, 1, uw.UW_PIPE_TRANSCODE) == -1
    uw.uw_autotune_set_variant(14336, 4096, 1, uw.UW_PIPE_BF16, 2)
    assert uw.uw_autotune_get_variant(14336, 4096, 1, uw.UW_PIPE_BF16) == 2
    assert uw.uw_autotune_get(14336, 4096, 1) == (uw.UW_PIPE_DIRECT_PALETTE, 6)   # AUTO entry untouched
    uw.uw_autotune_set_variant(14336, 4096, 1, uw.UW_PIPE_BF16, -1)                # deletes
    assert uw.uw_autotune_get_variant(14336, 4096, 1, uw.UW_PIPE_BF16) == -1
    assert status_of(uw.uw_autotune_set_variant, 1, 64, 1, uw.UW_PIPE_AUTO, 0) == uw.UW_E_ARG
    assert status_of(uw.uw_autotune_set_variant, 1, 64, 1, 6, 0) == uw.UW_E_ARG
    assert status_of(uw.uw_autotune_set_variant, 1, 64, 1, uw.UW_PIPE_BF16, uw.uw_variant_count()) == uw.UW_E_ARG
    p = tmp_path / "tune.txt"
    p.write_text("4096 14336 8 2 1\nvariant 4096 14336 8 5 3\nvariant 4096 14336 8 4 0  # palette\n")
    uw.uw_autotune_clear()
    uw.uw_autotune_load(str(p))
    assert uw.uw_autotune_get(4096, 14336, 8) == (uw.UW_PIPE_EXP_ONLY, 1)
    assert uw.uw_autotune_get_variant(4096, 14336, 8, uw.UW_PIPE_EXP_ONLY) == 1
    assert uw.uw_autotune_get_variant(4096, 14336, 8, uw.UW_PIPE_BF16) == 3
    assert uw.uw_autotune_get_variant(4096, 14336, 8, uw.UW_PIPE_DIRECT_PALETTE) == 0
    # a bad line anywhere rejects the whole file and applies nothing
    uw.uw_autotune_clear()
    for bad in ("variant 4096 14336 8 0 1\n", "variant 4096 14336 8 5\n", "4096 14336 8 4 1 7\n",
                "4096x 14336 8 4 1\n", "4096 14336 8 4 1\nvariant 1 64 1 5 99\n"):
        p.write_text(bad)
        assert status_of(uw.uw_autotune_load, str(p)) == uw.UW_E_ARG, bad
        assert uw.uw_autotune_get(4096, 14336, 8) == (uw.UW_PIPE_DIRECT_PALETTE, -1)
    uw.uw_autotune_clear()


def test_variant_names():
    n = uw.uw_variant_count()
    assert n >= 4
    assert all(uw.uw_variant_name(v).startswith(("waves=", "multitile ", "shared-x ", "wide ", "big ")) for v in range(n))
    assert any(uw.uw_variant_name(v).startswith("multitile ") for v in range(n))
    assert uw.uw_variant_name(n) == ""


def test_binding_refuses_host_buffers():
    """Device entry points take raw pointers the library cannot bound-check: the binding
    refuses host arrays and CPU tensors before anything reaches the C ABI."""
    import torch
    w = synth.small_gaussian(32, 128, seed=1)["w"]
    blob = uw.uw_encode(w)
    with pytest.raises(ValueError, match="CUDA tensor"):
        uw.DMat(blob, blob)                       # numpy "device" copy
    with pytest.raises(ValueError, match="CUDA tensor"):
        uw.DMat(blob, torch.from_numpy(blob))     # CPU tensor
    g = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="CUDA tensor"):
        uw.uw_swiglu(g, g, torch.zeros(16, dtype=torch.int16))
    with pytest.raises(ValueError, match="CUDA tensor"):
        uw.uw_rmsnorm(torch.zeros((2, 8), dtype=torch.float32), torch.zeros((2, 8), dtype=torch.int16))
    with pytest.raises(ValueError, match="CUDA tensor"):
        uw.uw_gemm_bf16(torch.zeros((16, 64), dtype=torch.int16), torch.zeros((1, 64), dtype=torch.int16),
                        torch.zeros((1, 16), dtype=torch.float32), 1)


def test_autotune_nearest_batch_size():
    """A batch size without an entry takes the entry of the nearest measured one for the same
    shape (by ratio, the smaller on a tie); another shape or pipeline is never borrowed."""
    uw.uw_autotune_clear()
    try:
        n, k = 4096, 14336
        uw.uw_autotune_set(n, k, 1, uw.UW_PIPE_DIRECT_PALETTE, 6)
        uw.uw_autotune_set(n, k, 16, uw.UW_PIPE_DIRECT_PALETTE, 13)
        uw.uw_autotune_set(n, k, 64, uw.UW_PIPE_TRANSCODE, 10)
        assert uw.uw_autotune_get(n, k, 1) == (uw.UW_PIPE_DIRECT_PALETTE, 6)
        assert uw.uw_autotune_get(n, k, 3) == (uw.UW_PIPE_DIRECT_PALETTE, 6)     # 3/1 = 3 < 16/3
        assert uw.uw_autotune_get(n, k, 4) == (uw.UW_PIPE_DIRECT_PALETTE, 6)     # 4/1 = 16/4: tie -> 1
        assert uw.uw_autotune_get(n, k, 5) == (uw.UW_PIPE_DIRECT_PALETTE, 13)
        assert uw.uw_autotune_get(n, k, 32) == (uw.UW_PIPE_DIRECT_PALETTE, 13)   # 32/16 = 64/32: tie -> 16
        assert uw.uw_autotune_get(n, k, 48) == (uw.UW_PIPE_TRANSCODE, 10)
        assert uw.uw_autotune_get(n, k, 256) == (uw.UW_PIPE_TRANSCODE, 10)
        assert uw.uw_autotune_get_variant(n, k, 40, uw.UW_PIPE_DIRECT_PALETTE) == 13  # only 1 and 16 measured
        assert uw.uw_autotune_get_variant(n, k, 2, uw.UW_PIPE_TRANSCODE) == 10       # only 64 measured
        assert uw.uw_autotune_get_variant(n, k, 2, uw.UW_PIPE_EXP_ONLY) == -1        # none for this pipeline
        assert uw.uw_autotune_get(k, n, 16) == (uw.UW_PIPE_DIRECT_PALETTE, -1)   # other shape: default
        with pytest.raises(uw.UwError):
            uw.uw_autotune_get(n, k, 0)
    finally:
        uw.uw_autotune_clear()


def test_sched_rejects_bad_arguments_before_any_launch():
    """uw_sched_init validates on the host (null buffers, shapes, the side error word) and
    uw_sched_step refuses a scheduler that was never initialised; neither touches a GPU."""
    import ctypes
    L = uw.lib()
    buf = ctypes.create_string_buffer(L.uw_sched_size())
    one = (ctypes.c_void_p * 3)()
    hard = (ctypes.c_uint8 * 3)()
    p = ctypes.c_void_p(256)   # never dereferenced: validation fails first
    args = [buf, 1, 1, 64, 64, one, hard, None, 0, p, p, p, p, None, 0, p, 256, 1e-5, None, None]
    assert L.uw_sched_init(*args) == uw.UW_E_ARG          # views are null: check_dmat refuses
    bad = list(args)
    bad[9] = None                                             # g
    assert L.uw_sched_init(*bad) == uw.UW_E_ARG
    bad = list(args)
    bad[2] = 0                                                # m
    assert L.uw_sched_init(*bad) == uw.UW_E_SHAPE
    bad = list(args)
    bad[16] = 16                                              # side error word too small
    assert L.uw_sched_init(*bad) == uw.UW_E_WORKSPACE
    out = ctypes.c_void_p()
    assert L.uw_sched_step(buf, p, ctypes.byref(out)) == uw.UW_E_ARG
    assert L.uw_sched_release(buf) == uw.UW_E_ARG
