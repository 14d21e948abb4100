"""Oracle GEMM and the glue of a decode step through an MLP stack.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Cloudflare blog post "Unweight", the four-pipeline and reconstructive-matmul
paragraphs: the compressed weights feed an ordinary matrix multiply whose output must be
the one the uncompressed BF16 weights give.  Orientation (a reading; the post is silent):
W is [N, K] (output x input, like a Linear layer's weight), X is [M, K], Y = X W^T is
[M, N] in fp32.

Every BF16 x BF16 product is exact in fp64 (8-bit significands), so the fp64 sum differs
from the exact dot product by at most K * 2**-53 * sum|x w|; that is far below the
acceptance bound |y - y_ref| <= 1e-3 * sum|x w| the GPU results are held to.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits):
    """BF16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def gemm_ref(x_bits, w_bits):
    """Y = X W^T accumulated in fp64, and the error scale S = |X| |W|^T.

    x_bits: uint16 [M, K]; w_bits: uint16 [N, K].  Returns (y, s), both float64 [M, N]."""
    x = bf16_to_f64(x_bits)
    w = bf16_to_f64(w_bits)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def gemm_ref_multi(xs_bits, w_bits):
    """gemm_ref of several inputs X against one W (W converted to fp64 once): a list of
    (y, s) pairs, one per X."""
    w = bf16_to_f64(w_bits)
    aw = np.abs(w)
    out = []
    for xb in xs_bits:
        x = bf16_to_f64(xb)
        out.append((x @ w.T, np.abs(x) @ aw.T))
    return out


def gemm_ref_rows(x_bits, w_bits, rows):
    """gemm_ref restricted to the output columns `rows` (rows of W), for sampled checks."""
    w = np.asarray(w_bits)[np.asarray(rows)]
    return gemm_ref(x_bits, w)


def within_bound(y, y_ref, s, rel=1e-3):
    """Acceptance test per element: |y - y_ref| <= rel * S; S == 0 requires y == 0."""
    y = np.asarray(y, dtype=np.float64)
    return np.abs(y - y_ref) <= rel * s


def f64_to_bf16_rne(a):
    """Round float64 to the nearest BF16 (ties to even), via fp32 (finite inputs)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def swiglu_ref(g, u):
    """h = bf16(silu(g) * u), silu(g) = g / (1 + exp(-g)); g, u are the fp32 outputs of
    the gate and up matmuls (SwiGLU between the up/gate and down projections)."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return f64_to_bf16_rne(g / (1.0 + np.exp(-g)) * u)


def rmsnorm_ref(y, eps=1e-5):
    """Weightless RMS norm of each row of the down-projection output, rounded to BF16:
    the next layer's input (a reading: keeps a 32-layer stack finite)."""
    y = np.asarray(y, dtype=np.float64)
    scale = 1.0 / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    return f64_to_bf16_rne(y * scale)
