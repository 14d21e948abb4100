"""Lossless BF16 weight compression fused into the decode-time GEMM, for MI355X (gfx950).

Thin ctypes binding over libuw.so (include/uw.h): every function marshals arguments and
calls the C ABI of the same name; all computation happens in the library (host codec in
C++, everything on the device in hand-written HIP kernels).  PyTorch supplies device
memory and streams only.  The library must be built first
(``python -m lossless_bf16_weight_amd.build``); calls fail loudly when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import synth  # noqa: F401  (seeded workloads; no method arithmetic)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libuw.so")

UW_OK, UW_E_ARG, UW_E_SHAPE, UW_E_FORMAT, UW_E_NOMEM, UW_E_WORKSPACE, UW_E_HIP, UW_E_DATA = 0, -1, -2, -3, -4, -5, -6, -7
UW_PIPE_AUTO, UW_PIPE_FULL_DECODE, UW_PIPE_EXP_ONLY, UW_PIPE_TRANSCODE, UW_PIPE_DIRECT_PALETTE = 0, 1, 2, 3, 4
UW_PIPE_BF16 = 5
UW_OP_DECODE_FULL, UW_OP_TRANSCODE, UW_OP_DECODE_EXP = 16, 17, 18
UW_MAX_M = 1024
PIPELINES = {"full": UW_PIPE_FULL_DECODE, "exp": UW_PIPE_EXP_ONLY, "transcode": UW_PIPE_TRANSCODE,
             "direct": UW_PIPE_DIRECT_PALETTE}

# Every symbol include/uw.h declares (checked by the CPU tests).
EXPORTS = ("uw_last_error", "uw_version", "uw_build_palette", "uw_encode_bound", "uw_encode", "uw_blob_info",
           "uw_dmat_size", "uw_dmat_bind", "uw_dmat_get_info", "uw_workspace_size", "uw_decode_full",
           "uw_transcode_palette", "uw_decode_exponents", "uw_gemm", "uw_gemm_variant", "uw_gemm_noalloc",
           "uw_gemm_bf16",
           "uw_variant_count", "uw_variant_name", "uw_check", "uw_autotune_load", "uw_autotune_set",
           "uw_autotune_get", "uw_autotune_set_variant", "uw_autotune_get_variant", "uw_autotune_clear", "uw_swiglu",
           "uw_gemm_swiglu", "uw_gemm_rmsnorm", "uw_rmsnorm", "uw_sched_size", "uw_sched_init", "uw_sched_step",
           "uw_sched_trace", "uw_sched_split", "uw_sched_release")


class UwError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("uw status %d: %s" % (status, msg))
        self.status = status


class Palette(ctypes.Structure):
    _fields_ = [("n", ctypes.c_uint32), ("exp", ctypes.c_uint8 * 16), ("index_of", ctypes.c_uint8 * 256),
                ("hist", ctypes.c_uint64 * 256)]


class Info(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("np", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("kb", ctypes.c_int64), ("chunk", ctypes.c_int32), ("lmax", ctypes.c_int32),
                ("n_pal", ctypes.c_int32), ("affine", ctypes.c_int32), ("n_verb", ctypes.c_int64),
                ("n_coded", ctypes.c_int64), ("total_bits", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("n_words", ctypes.c_int64), ("palette", ctypes.c_uint8 * 16), ("code_len", ctypes.c_uint8 * 16),
                ("code", ctypes.c_uint16 * 16), ("sec_off", ctypes.c_uint64 * 7), ("sec_size", ctypes.c_uint64 * 7),
                ("blob_bytes", ctypes.c_uint64), ("resident_bytes", ctypes.c_uint64), ("idx_bytes", ctypes.c_uint64)]

    def as_dict(self):
        out = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            out[name] = list(v) if hasattr(v, "__len__") else v
        return out


_lib = None
_P, _S, _I32, _I64, _F = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float


def lib():
    """Load libuw.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libuw.so is not built (%s); run: python -m lossless_bf16_weight_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "uw_last_error": (ctypes.c_char_p, []),
        "uw_version": (_I32, []),
        "uw_build_palette": (_I32, [_P, _I64, _I64, ctypes.POINTER(Palette)]),
        "uw_encode_bound": (_I32, [_I64, _I64, _I32, ctypes.POINTER(_S)]),
        "uw_encode": (_I32, [_P, _I64, _I64, ctypes.POINTER(Palette), _I32, _P, _S, ctypes.POINTER(_S)]),
        "uw_blob_info": (_I32, [_P, _S, ctypes.POINTER(Info)]),
        "uw_dmat_size": (_S, []),
        "uw_dmat_bind": (_I32, [_P, _P, _S, _P, _P]),
        "uw_dmat_get_info": (_I32, [_P, ctypes.POINTER(Info)]),
        "uw_workspace_size": (_I32, [_P, _I32, _I32, ctypes.POINTER(_S)]),
        "uw_decode_full": (_I32, [_P, _P, _P, _S, _P]),
        "uw_transcode_palette": (_I32, [_P, _P, _P, _S, _P]),
        "uw_decode_exponents": (_I32, [_P, _P, _P, _S, _P]),
        "uw_gemm": (_I32, [_P, _P, _P, _I32, _I32, _P, _S, _P]),
        "uw_gemm_variant": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _S, _P]),
        "uw_gemm_noalloc": (_I32, [_P, _P, _P, _I32, _I32, _P]),
        "uw_gemm_bf16": (_I32, [_P, _I64, _I64, _P, _P, _I32, _I32, _P]),
        "uw_variant_count": (_I32, []),
        "uw_variant_name": (ctypes.c_char_p, [_I32]),
        "uw_check": (_I32, [_P, _P]),
        "uw_autotune_load": (_I32, [ctypes.c_char_p]),
        "uw_autotune_set": (_I32, [_I64, _I64, _I32, _I32, _I32]),
        "uw_autotune_get": (_I32, [_I64, _I64, _I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
        "uw_autotune_set_variant": (_I32, [_I64, _I64, _I32, _I32, _I32]),
        "uw_autotune_get_variant": (_I32, [_I64, _I64, _I32, _I32, ctypes.POINTER(_I32)]),
        "uw_autotune_clear": (_I32, []),
        "uw_swiglu": (_I32, [_P, _P, _P, _I64, _P]),
        "uw_gemm_swiglu": (_I32, [_P, _P, _P, _P, _I32, _I32, _I32, _P, _S, _P]),
        "uw_gemm_rmsnorm": (_I32, [_P, _P, _P, _P, _I32, _F, _I32, _I32, _P, _S, _P]),
        "uw_rmsnorm": (_I32, [_P, _P, _I32, _I32, _F, _P]),
        "uw_sched_size": (_S, []),
        "uw_sched_init": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P, _P, _S, _P, _P, _P, _P, _P, _S, _P, _S, _F,
                                 _P, _P]),
        "uw_sched_step": (_I32, [_P, _P, ctypes.POINTER(ctypes.c_void_p)]),
        "uw_sched_trace": (_I32, [_P, _P, _S]),
        "uw_sched_split": (_I32, [_P, _I32]),
        "uw_sched_release": (_I32, [_P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status):
    if status != UW_OK:
        raise UwError(status, lib().uw_last_error().decode(errors="replace"))


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _dev(t, name, min_bytes, dtypes=None, optional=False):
    """Device address of a contiguous CUDA tensor holding at least min_bytes (the C ABI takes
    raw pointers it cannot bound-check, so a wrong buffer is refused here, not faulted on)."""
    if t is None:
        if optional:
            return None
        raise ValueError("%s: a CUDA tensor is required" % name)
    if isinstance(t, np.ndarray) or not getattr(t, "is_cuda", False):
        raise ValueError("%s: must be a CUDA tensor (got %s)" % (name, type(t).__name__))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)
    if dtypes is not None and str(t.dtype).replace("torch.", "") not in dtypes:
        raise ValueError("%s: dtype %s, expected one of %s" % (name, t.dtype, "/".join(dtypes)))
    if _nbytes(t) < min_bytes:
        raise ValueError("%s: %d bytes, the call needs at least %d" % (name, _nbytes(t), min_bytes))
    return t.data_ptr()


_U16 = ("int16", "uint16", "bfloat16")


# ----------------------------------------------------------------------------------------
# Host encoder
# ----------------------------------------------------------------------------------------
def uw_version():
    return lib().uw_version()


def uw_build_palette(w):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    p = Palette()
    _check(lib().uw_build_palette(w.ctypes.data, w.shape[0], w.shape[1], ctypes.byref(p)))
    return dict(n=p.n, exp=list(p.exp)[: p.n], index_of=np.array(p.index_of, np.uint8),
                hist=np.array(p.hist, np.int64))


def uw_encode_bound(n, k, chunk=0):
    out = ctypes.c_size_t()
    _check(lib().uw_encode_bound(n, k, chunk, ctypes.byref(out)))
    return out.value


def _palette_struct(palette):
    """uw_palette from a uw_build_palette() dict, or from a list of exponents (index_of is the
    list's inverse; the library checks the result)."""
    if palette is None:
        return None
    p = Palette()
    exps = list(palette["exp"]) if isinstance(palette, dict) else [int(v) for v in palette]
    if not 1 <= len(exps) <= 16:
        raise ValueError("a palette holds 1..16 exponents (got %d)" % len(exps))
    p.n = len(exps)
    for i, e in enumerate(exps):
        p.exp[i] = e
    if isinstance(palette, dict) and "index_of" in palette:
        for x in range(256):
            p.index_of[x] = int(palette["index_of"][x])
    else:
        for x in range(256):
            p.index_of[x] = 0xFF
        for i, e in enumerate(exps):
            p.index_of[e] = i
    return p


def uw_encode(w, chunk=0, palette=None):
    """Encode a [n, k] uint16 BF16 matrix; returns the blob as a uint8 numpy array.
    palette: None (W's own top-16), a uw_build_palette() dict, or ascending exponents."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    used = ctypes.c_size_t()
    p = _palette_struct(palette)
    pp = ctypes.byref(p) if p is not None else None
    _check(lib().uw_encode(w.ctypes.data, n, k, pp, chunk, None, 0, ctypes.byref(used)))
    blob = np.zeros(used.value, np.uint8)
    _check(lib().uw_encode(w.ctypes.data, n, k, pp, chunk, blob.ctypes.data, blob.size, ctypes.byref(used)))
    return blob


def uw_blob_info(blob):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    info = Info()
    _check(lib().uw_blob_info(blob.ctypes.data, blob.size, ctypes.byref(info)))
    return info.as_dict()


# ----------------------------------------------------------------------------------------
# Device view and kernels
# ----------------------------------------------------------------------------------------
class DMat:
    """A bound uw_dmat plus the tensors it borrows (kept alive here).  blob_dev: a device copy
    of the whole host blob; idx_dev: the direct-palette index stream (info idx_bytes) or None."""

    def __init__(self, blob_host, blob_dev, idx_dev=None):
        self.buf = ctypes.create_string_buffer(lib().uw_dmat_size())
        self.blob_host = np.ascontiguousarray(blob_host, dtype=np.uint8)
        info = uw_blob_info(self.blob_host)
        self.blob_dev = blob_dev
        self.idx = idx_dev
        _check(lib().uw_dmat_bind(self.buf, self.blob_host.ctypes.data, self.blob_host.size,
                                  _dev(blob_dev, "blob_dev", self.blob_host.size),
                                  _dev(idx_dev, "idx_dev", int(info["idx_bytes"]), optional=True)))
        info = Info()
        _check(lib().uw_dmat_get_info(self.buf, ctypes.byref(info)))
        self.info = info.as_dict()

    @property
    def handle(self):
        return self.buf


def uw_dmat_bind(blob_host, blob_dev, idx_dev=None):
    return DMat(blob_host, blob_dev, idx_dev)


def uw_workspace_size(d, m, op):
    out = ctypes.c_size_t()
    _check(lib().uw_workspace_size(d.handle, m, op, ctypes.byref(out)))
    return out.value


def uw_decode_full(d, w_out, ws, stream=None):
    n, k = int(d.info["n"]), int(d.info["k"])
    _check(lib().uw_decode_full(d.handle, _dev(w_out, "w_out", 2 * n * k), _dev(ws, "ws", 0, optional=True),
                                _nbytes(ws), _stream(stream)))


def uw_transcode_palette(d, idx_out, ws, stream=None):
    _check(lib().uw_transcode_palette(d.handle, _dev(idx_out, "idx_out", int(d.info["idx_bytes"])),
                                      _dev(ws, "ws", 0, optional=True), _nbytes(ws), _stream(stream)))


def uw_decode_exponents(d, exp_out, ws, stream=None):
    need = int(d.info["np"]) * int(d.info["k"])
    _check(lib().uw_decode_exponents(d.handle, _dev(exp_out, "exp_out", need), _dev(ws, "ws", 0, optional=True),
                                     _nbytes(ws), _stream(stream)))


def _gemm_ptrs(n, k, x, y, m, ws):
    mm = int(m) if 1 <= int(m) <= UW_MAX_M else 0   # other m: the library refuses them (UW_E_SHAPE)
    return (_dev(x, "x", 2 * mm * k, _U16), _dev(y, "y", 4 * mm * n, ("float32",)),
            _dev(ws, "ws", 0, optional=True))


def uw_gemm(d, x, y, m, pipeline=UW_PIPE_AUTO, ws=None, stream=None):
    px, py, pw = _gemm_ptrs(int(d.info["n"]), int(d.info["k"]), x, y, m, ws)
    _check(lib().uw_gemm(d.handle, px, py, m, pipeline, pw, _nbytes(ws), _stream(stream)))


def uw_gemm_variant(d, x, y, m, pipeline, variant, ws=None, stream=None):
    px, py, pw = _gemm_ptrs(int(d.info["n"]), int(d.info["k"]), x, y, m, ws)
    _check(lib().uw_gemm_variant(d.handle, px, py, m, pipeline, variant, pw, _nbytes(ws), _stream(stream)))


def uw_gemm_noalloc(d, x, y, m, variant=-1, stream=None):
    """Direct-palette GEMM with no workspace: the library's own device scratch holds the K-slice
    partial sums (calls overlapping on one GPU race; see include/uw.h)."""
    px, py, _ = _gemm_ptrs(int(d.info["n"]), int(d.info["k"]), x, y, m, None)
    _check(lib().uw_gemm_noalloc(d.handle, px, py, m, variant, _stream(stream)))


def uw_gemm_swiglu(d, x, gate, h, m, pipeline=UW_PIPE_AUTO, variant=-1, ws=None, stream=None):
    """h = bf16(silu(gate) * (x W^T)): the up projection with the SwiGLU glue in its epilogue."""
    n, k = int(d.info["n"]), int(d.info["k"])
    mm = int(m) if 1 <= int(m) <= UW_MAX_M else 0
    px = _dev(x, "x", 2 * mm * k, _U16)
    pg = _dev(gate, "gate", 4 * mm * n, ("float32",))
    ph = _dev(h, "h", 2 * mm * n, _U16)
    _check(lib().uw_gemm_swiglu(d.handle, px, pg, ph, m, pipeline, variant, _dev(ws, "ws", 0, optional=True),
                                _nbytes(ws), _stream(stream)))


def uw_gemm_rmsnorm(d, x, y, xn, m, eps=1e-5, pipeline=UW_PIPE_AUTO, variant=-1, ws=None, stream=None):
    """y = x W^T (fp32) and xn = bf16(RMS-normed rows of y): the down projection with the norm
    fused into its K-slice reduction when it runs one."""
    n, k = int(d.info["n"]), int(d.info["k"])
    px, py, pw = _gemm_ptrs(n, k, x, y, m, ws)
    mm = int(m) if 1 <= int(m) <= UW_MAX_M else 0
    pn = _dev(xn, "xn", 2 * mm * n, _U16)
    _check(lib().uw_gemm_rmsnorm(d.handle, px, py, pn, m, eps, pipeline, variant, pw, _nbytes(ws), _stream(stream)))


def uw_gemm_bf16(w, x, y, m, variant=-1, stream=None):
    n, k = w.shape
    pw = _dev(w, "w", 2 * n * k, _U16)
    px, py, _ = _gemm_ptrs(n, k, x, y, m, None)
    _check(lib().uw_gemm_bf16(pw, n, k, px, py, m, variant, _stream(stream)))


def uw_variant_count():
    return lib().uw_variant_count()


def uw_variant_name(v):
    return lib().uw_variant_name(v).decode()


def uw_check(ws, stream=None):
    _check(lib().uw_check(_dev(ws, "ws", 0, optional=True), _stream(stream)))


def uw_autotune_load(path):
    _check(lib().uw_autotune_load(path.encode()))


def uw_autotune_set(n, k, m, pipeline, variant):
    _check(lib().uw_autotune_set(n, k, m, pipeline, variant))


def uw_autotune_get(n, k, m):
    p, v = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().uw_autotune_get(n, k, m, ctypes.byref(p), ctypes.byref(v)))
    return p.value, v.value


def uw_autotune_set_variant(n, k, m, pipeline, variant):
    _check(lib().uw_autotune_set_variant(n, k, m, pipeline, variant))


def uw_autotune_get_variant(n, k, m, pipeline):
    v = ctypes.c_int32()
    _check(lib().uw_autotune_get_variant(n, k, m, pipeline, ctypes.byref(v)))
    return v.value


def uw_autotune_clear():
    _check(lib().uw_autotune_clear())


def uw_swiglu(g, u, h, stream=None):
    """h = bf16(silu(g) * u); g, u fp32, h BF16 bits (int16), all of g.numel() elements."""
    count = g.numel()
    _check(lib().uw_swiglu(_dev(g, "g", 4 * count, ("float32",)), _dev(u, "u", 4 * count, ("float32",)),
                           _dev(h, "h", 2 * count, _U16), count, _stream(stream)))


def uw_rmsnorm(y, x, eps=1e-5, stream=None):
    """x = bf16(y / sqrt(mean(y^2, rows) + eps)); y fp32 [m, n], x BF16 bits [m, n]."""
    m, n = y.shape
    _check(lib().uw_rmsnorm(_dev(y, "y", 4 * m * n, ("float32",)), _dev(x, "x", 2 * m * n, _U16), m, n, eps,
                            _stream(stream)))


class Sched:
    """A bound uw_sched (hard/easy MLP step) plus the tensors it borrows.  mats: 3*layers DMat
    (gate, up, down per layer); hard: 3*layers flags; buffers as uw_sched_init documents."""

    def __init__(self, mats, hard, m, hidden, inter, slots, slot_bytes, g, h, y, xo, ws, dws, eps=1e-5,
                 main_stream=None, side_stream=None):
        layers = len(mats) // 3
        if len(mats) != 3 * layers or len(hard) != len(mats) or layers < 1:
            raise ValueError("mats and hard must hold 3 entries a layer")
        self.keep = (mats, slots, g, h, y, xo, ws, dws)
        self.buf = ctypes.create_string_buffer(lib().uw_sched_size())
        self.views = (ctypes.c_void_p * len(mats))(*[ctypes.addressof(d.handle) for d in mats])
        self.hard = (ctypes.c_uint8 * len(hard))(*[1 if f else 0 for f in hard])
        nslot = 6 * slot_bytes if any(hard) else 0
        _check(lib().uw_sched_init(
            self.buf, layers, m, hidden, inter, self.views, self.hard,
            _dev(slots, "slots", nslot, optional=not any(hard)), slot_bytes,
            _dev(g, "g", 4 * m * inter, ("float32",)), _dev(h, "h", 2 * m * inter, _U16),
            _dev(y, "y", 4 * m * hidden, ("float32",)), _dev(xo, "xo", 4 * m * hidden, _U16),
            _dev(ws, "ws", 0, optional=True), _nbytes(ws), _dev(dws, "dws", 256), _nbytes(dws), eps,
            _stream(main_stream), _stream(side_stream)))
        self.live = True

    def step(self, x):
        """Returns the device address of the last layer's output (inside xo)."""
        out = ctypes.c_void_p()
        m_hidden = self.keep[5].numel() // 2
        _check(lib().uw_sched_step(self.buf, _dev(x, "x", 2 * m_hidden, _U16), ctypes.byref(out)))
        return out.value

    def trace(self, buf):
        """Record g, h, y and the output of every layer of the following steps into buf (a
        device tensor of layers * m * (6 * inter + 6 * hidden) bytes), or stop with None."""
        self.trace_buf = buf
        _check(lib().uw_sched_trace(self.buf, _dev(buf, "trace", 0, optional=True), _nbytes(buf)))

    def split(self, decode_workgroups):
        """At most `decode_workgroups` decoder workgroups for hard-layer decodes (0: whole chip)."""
        _check(lib().uw_sched_split(self.buf, int(decode_workgroups)))

    def release(self):
        if self.live:
            _check(lib().uw_sched_release(self.buf))
            self.live = False

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


# ----------------------------------------------------------------------------------------
# Convenience: a compressed matrix resident on the GPU
# ----------------------------------------------------------------------------------------
class CompressedMatrix:
    """Encode W on the host (C++), copy the blob to the device, bind it and run the
    load-time transcode to the direct-palette index stream (a device kernel)."""

    def __init__(self, w, chunk=0, device="cuda", blob=None, keep_index=True, palette=None):
        import torch
        self.blob = uw_encode(w, chunk, palette) if blob is None else np.ascontiguousarray(blob, np.uint8)
        self.blob_dev = torch.from_numpy(self.blob).to(device)
        info = uw_blob_info(self.blob)
        self.idx = torch.empty(int(info["idx_bytes"]), dtype=torch.uint8, device=device) if keep_index else None
        self.d = DMat(self.blob, self.blob_dev, self.idx)
        self.info = self.d.info
        self.n, self.k = int(info["n"]), int(info["k"])
        self.err = torch.zeros(64, dtype=torch.int32, device=device)
        self._ws = {}
        if keep_index:
            uw_transcode_palette(self.d, self.idx, self.err)
            uw_check(self.err)   # load time: a corrupt bitstream is reported here

    def workspace(self, m, pipeline):
        """A zeroed workspace of uw_workspace_size bytes (error word, decoded operand of
        pipelines 1-3, K-slice partial sums of the multi-tile kernel)."""
        import torch
        size = uw_workspace_size(self.d, m, pipeline)
        return torch.zeros(max(size, 256), dtype=torch.uint8, device=self.blob_dev.device) if size else None

    def gemm(self, x, y=None, pipeline=UW_PIPE_DIRECT_PALETTE, ws=None, variant=-1, stream=None):
        import torch
        m = x.shape[0]
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        if ws is None:
            key = (m, pipeline)
            if key not in self._ws:
                self._ws[key] = self.workspace(m, pipeline)
            ws = self._ws[key]
        uw_gemm_variant(self.d, x, y, m, pipeline, variant, ws, stream)
        return y

    def resident_bytes(self):
        return int(self.info["resident_bytes"])

    def bundle_bytes(self):
        return int(self.blob.size)
