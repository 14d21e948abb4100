"""Seeded synthetic workloads (weights and activations as BF16 bit patterns).

This module is the only code shared by the GPU path's tests/bench and the CPU oracle.
It draws random numbers and rounds them to BF16; it contains none of the compression
method's arithmetic.

The post measures on Llama-3.1-8B trained weights, which are not available here; these
generators stand in for them with the model's MLP shapes (gate/up 14336 x 4096,
down 4096 x 14336) and Gaussian or heavy-tailed entries.

Recipe (one numpy PCG64 generator per workload unless stated):
  * values are drawn in fp32 (Student-t in fp64, then rounded to fp32), multiplied by the
    fp32 standard deviation, then rounded to BF16 (round to nearest, ties to even);
  * draw order: weights, then planted outliers, then activations;
  * planted outliers: max(1, round(frac * N)) distinct rows chosen without replacement,
    one uniformly random column each, value +-2**(+-20) with sign and exponent sign
    uniform (exactly representable in BF16).
"""
from __future__ import annotations

import hashlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def f32_to_bf16_bits(a):
    """fp32 -> BF16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = b >> np.uint32(16)                # in place from here: one temporary for any size
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def gaussian_bf16(rng, shape, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def student_t_bf16(rng, shape, df, scale):
    return f32_to_bf16_bits(rng.standard_t(df, size=shape).astype(np.float32) * np.float32(scale))


def subnormal_bf16(rng, shape):
    """Edge case: BF16 bit patterns with exponent field 0 (zeros and subnormals, 70 %) or the two
    smallest normal exponents 1 and 2; random sign and mantissa."""
    e = rng.choice(np.array([0, 1, 2], np.uint16), size=shape, p=[0.7, 0.2, 0.1])
    m = rng.integers(0, 128, size=shape).astype(np.uint16)
    s = rng.integers(0, 2, size=shape).astype(np.uint16)
    return (s << 15) | (e << 7) | m


def plant_outliers(rng, w, frac):
    """Give max(1, round(frac*N)) distinct rows one value of +-2**(+-20); returns the rows."""
    n, k = w.shape
    count = max(1, int(round(frac * n)))
    rows = rng.choice(n, size=count, replace=False)
    cols = rng.integers(0, k, size=count)
    sign = rng.integers(0, 2, size=count)
    up = rng.integers(0, 2, size=count)
    biased = np.where(up == 1, 127 + 20, 127 - 20)
    w[rows, cols] = ((sign << 15) | (biased << 7)).astype(np.uint16)
    return np.sort(rows)


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------------------
CONFIGS = {
    "c1": "single 1024x1024, N(0,0.02^2), 0.1% rows with a +-2^+-20 outlier, X 1x1024",
    "c2": "Llama-3.1-8B gate_proj 14336x4096, N(0,0.02^2), 0.05% rows planted, X M=1",
    "c3": "Llama-3.1-8B down_proj 4096x14336, N(0,0.015^2), X M in {1,8,32,64}",
    "c4": "32-layer Llama-3.1-8B MLP stack, per-layer std U[0.01,0.03], X M=16",
    "c5": "heavy tail 8192x8192, Student-t(3)*0.02, X M=128",
}


def config1(seed=0):
    rng = np.random.default_rng(seed)
    w = gaussian_bf16(rng, (1024, 1024), 0.02)
    planted = plant_outliers(rng, w, 0.001)
    x = gaussian_bf16(rng, (1, 1024), 1.0)
    return dict(w=w, x=x, planted=planted)


def config2(seed=1):
    rng = np.random.default_rng(seed)
    w = gaussian_bf16(rng, (14336, 4096), 0.02)
    planted = plant_outliers(rng, w, 0.0005)
    x = gaussian_bf16(rng, (1, 4096), 1.0)
    return dict(w=w, x=x, planted=planted)


def config3(seed=2, m_max=64):
    rng = np.random.default_rng(seed)
    w = gaussian_bf16(rng, (4096, 14336), 0.015)
    x = gaussian_bf16(rng, (m_max, 14336), 1.0)   # X for M is the first M rows
    return dict(w=w, x=x)


def config5(seed=4):
    rng = np.random.default_rng(seed)
    w = student_t_bf16(rng, (8192, 8192), 3, 0.02)
    x = gaussian_bf16(rng, (128, 8192), 1.0)
    return dict(w=w, x=x)


C4_SHAPES = ((14336, 4096), (14336, 4096), (4096, 14336))   # gate, up [inter, hidden]; down [hidden, inter]


def config4_meta(seed=3, layers=32, m=16, hidden=4096):
    """Per-layer std and X of the MLP stack.  SeedSequence(seed) spawns 1 + 3*layers children:
    child 0 draws the per-layer std (U[0.01, 0.03]) then X; child 1 + 3l + j draws matrix j
    (0 gate, 1 up, 2 down) of layer l (config4_matrix)."""
    kids = np.random.SeedSequence(seed).spawn(1 + 3 * layers)
    rng0 = np.random.default_rng(kids[0])
    stds = rng0.uniform(0.01, 0.03, size=layers)
    x = gaussian_bf16(rng0, (m, hidden), 1.0)
    return dict(stds=stds, x=x, kids=kids)


def config4_matrix(meta, l, j, shapes=C4_SHAPES):
    """Matrix j (0 gate, 1 up, 2 down) of layer l, from its own child generator."""
    return gaussian_bf16(np.random.default_rng(meta["kids"][1 + 3 * l + j]), shapes[j], meta["stds"][l])


def config4(seed=3, layers=32, m=16, threads=16, hidden=4096, inter=14336):
    """The whole stack at once (about 11 GB of BF16 at full size): matrices are drawn in
    parallel threads, each from its own child generator, so the values do not depend on
    the thread count."""
    meta = config4_meta(seed, layers, m, hidden)
    shapes = ((inter, hidden), (inter, hidden), (hidden, inter))

    def make(i):
        return config4_matrix(meta, i // 3, i % 3, shapes)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        mats = list(ex.map(make, range(3 * layers)))
    return dict(stds=meta["stds"], x=meta["x"], layers=[tuple(mats[3 * l: 3 * l + 3]) for l in range(layers)])


def small_gaussian(n, k, m=1, std=0.02, seed=0, plant_frac=0.0):
    """Small seeded case for parity tests (any shape)."""
    rng = np.random.default_rng(seed)
    w = gaussian_bf16(rng, (n, k), std)
    if plant_frac > 0:
        plant_outliers(rng, w, plant_frac)
    x = gaussian_bf16(rng, (m, k), 1.0)
    return dict(w=w, x=x)
