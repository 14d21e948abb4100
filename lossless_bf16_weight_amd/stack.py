"""A stack of LLM MLP layers served from compressed weights: one decode step.

Per layer l with input x_l [m, hidden] (BF16):
    g = x_l gate^T, u = x_l up^T        (fused reconstruct GEMMs, fp32 out)
    h = bf16(silu(g) * u)               (SwiGLU: in the up GEMM's epilogue, uw_gemm_swiglu;
                                         or uw_gemm + uw_swiglu when u itself is wanted)
    y = h down^T                        (fused reconstruct GEMM, fp32 out)
    x_{l+1} = bf16(y / sqrt(mean(y^2) + eps))   (weightless RMS norm: in the down GEMM's slice
                                                 reduction, uw_gemm_rmsnorm; or uw_rmsnorm)

The Unweight post compresses the MLP projections of Llama-3.1-8B (gate, up, down) and runs
them through its reconstructive matmul; the SwiGLU and the norm between layers are the
model's own glue, kept here so a multi-layer step stays finite.  Every step runs in libuw's
kernels on one stream; this class only holds the buffers and issues the calls.
"""
from __future__ import annotations

import numpy as np

from . import (UW_PIPE_AUTO, UW_PIPE_DIRECT_PALETTE, CompressedMatrix, Sched, uw_check, uw_gemm_rmsnorm, uw_gemm_swiglu,
               uw_gemm_variant, uw_rmsnorm, uw_swiglu, uw_workspace_size)

PROJECTIONS = ("gate", "up", "down")


class MLPStack:
    def __init__(self, m, hidden, inter, device="cuda:0", eps=1e-5):
        import torch
        self.m, self.hidden, self.inter, self.eps = m, hidden, inter, eps
        self.dev = torch.device(device)
        self.layers = []                                  # [(gate, up, down) CompressedMatrix]
        self.g = torch.empty((m, inter), dtype=torch.float32, device=self.dev)
        self.u = torch.empty((m, inter), dtype=torch.float32, device=self.dev)
        self.h = torch.empty((m, inter), dtype=torch.int16, device=self.dev)
        self.y = torch.empty((m, hidden), dtype=torch.float32, device=self.dev)
        self.xs = [torch.empty((m, hidden), dtype=torch.int16, device=self.dev) for _ in range(2)]
        self.ws = None
        self.ws_bytes = 0

    def add_layer(self, gate, up, down, chunk=0):
        """gate, up: [inter, hidden]; down: [hidden, inter] BF16 bit patterns (host uint16),
        or CompressedMatrix objects already on this device."""
        mats = []
        for w, shape in ((gate, (self.inter, self.hidden)), (up, (self.inter, self.hidden)),
                         (down, (self.hidden, self.inter))):
            cm = w if isinstance(w, CompressedMatrix) else CompressedMatrix(w, chunk=chunk, device=self.dev)
            if (cm.n, cm.k) != shape:
                raise ValueError("layer matrix is %dx%d, expected %dx%d" % (cm.n, cm.k, *shape))
            mats.append(cm)
        self.layers.append(tuple(mats))

    def _workspace(self, pipelines):
        """A zeroed workspace that serves every matrix under `pipelines` (one per projection)."""
        import torch
        need = max(uw_workspace_size(cm.d, self.m, p) for lay in self.layers for cm, p in zip(lay, pipelines))
        if need > self.ws_bytes:
            self.ws = torch.zeros(need, dtype=torch.uint8, device=self.dev)
            self.ws_bytes = need
        return self.ws if need else None

    def step(self, x, pipeline=UW_PIPE_AUTO, trace=None, check=True, fused=None, config=None):
        """x: device int16 [m, hidden] (BF16 bits).  Returns the device tensor holding the last
        layer's output (one of two ping-pong buffers).  trace: optional list that receives,
        per layer, host copies (x_in, g, u, h, y, x_out) -- for tests; it synchronises.
        check: wait for the step and report a corrupt stream found by a decode pipeline
        (UwError); pass False to keep the step asynchronous.  fused: SwiGLU in the up GEMM's
        epilogue and the RMS norm after the down GEMM in one call (default unless tracing,
        which needs u itself); the outputs are identical.  config: per projection
        {"gate"|"up"|"down": (pipeline, variant)} (e.g. a tuned per-model file), overriding
        `pipeline` and the autotuned variants."""
        fused = trace is None if fused is None else fused
        if fused and trace is not None:
            raise ValueError("a traced step needs u: use fused=False")
        cfg = [(pipeline, -1)] * 3 if config is None else [tuple(config[k]) for k in PROJECTIONS]
        (pg, vg), (pu, vu), (pd, vd) = cfg
        ws = self._workspace((pg, pu, pd))
        cur = x
        for i, (gate, up, down) in enumerate(self.layers):
            out = self.xs[i % 2]
            uw_gemm_variant(gate.d, cur, self.g, self.m, pg, vg, ws)
            if fused:
                uw_gemm_swiglu(up.d, cur, self.g, self.h, self.m, pu, vu, ws)
            else:
                uw_gemm_variant(up.d, cur, self.u, self.m, pu, vu, ws)
                uw_swiglu(self.g, self.u, self.h)
            if fused:
                uw_gemm_rmsnorm(down.d, self.h, self.y, out, self.m, self.eps, pd, vd, ws)
            else:
                uw_gemm_variant(down.d, self.h, self.y, self.m, pd, vd, ws)
                uw_rmsnorm(self.y, out, self.eps)
            if trace is not None:
                trace.append(tuple(t.cpu().numpy().copy() for t in (cur, self.g, self.u, self.h, self.y, out)))
            cur = out
        if ws is not None and check:
            uw_check(ws)
        return cur

    def resident_bytes(self):
        return sum(cm.resident_bytes() for lay in self.layers for cm in lay)

    def weight_count(self):
        return sum(cm.n * cm.k for lay in self.layers for cm in lay)


def as_bf16_bits(t):
    """Host uint16 view of a device or host int16 tensor/array."""
    a = t if isinstance(t, np.ndarray) else t.cpu().numpy()
    return a.view(np.uint16)


class HardEasyStack:
    """The same MLP stack with hard and easy layers (hard/easy-layer paragraphs of the Unweight
    post): an easy matrix holds its direct-palette index stream (resident 12.06 bits a weight on
    the MLP shapes); a hard one holds only its Huffman bundle (10.70 bits a weight) and its index
    stream is decoded into one of two slot sets on a side stream while the main stream computes
    the layers before it (libuw's uw_sched_*: the ordering lives in the library, events between
    the streams).  Outputs are bit-identical to MLPStack.step (same kernels on the same index
    bits).  hard_layers: the layer indices whose three matrices are hard."""

    def __init__(self, m, hidden, inter, matrices, hard_layers=(), device="cuda:0", eps=1e-5, chunk=0,
                 overlap=True, decode_workgroups=0):
        import torch
        self.m, self.hidden, self.inter, self.eps = m, hidden, inter, eps
        self.dev = torch.device(device)
        self.hard_layers = sorted(set(int(l) for l in hard_layers))
        self.layers = []
        hard = []
        for l, (gw, uw_, dw) in enumerate(matrices):
            is_hard = l in self.hard_layers
            mats = []
            for w in (gw, uw_, dw):
                if isinstance(w, CompressedMatrix):
                    if is_hard and w.idx is not None:
                        raise ValueError("layer %d is hard: give its matrices without an index stream" % l)
                    mats.append(w)
                else:
                    mats.append(CompressedMatrix(w, chunk=chunk, device=self.dev, keep_index=not is_hard))
            self.layers.append(tuple(mats))
            hard += [is_hard] * 3
        for l in self.hard_layers:
            if l >= len(self.layers):
                raise ValueError("hard layer %d past the %d layers" % (l, len(self.layers)))
        flat = [cm for lay in self.layers for cm in lay]
        self.slot_bytes = max([int(cm.info["idx_bytes"]) for cm, f in zip(flat, hard) if f] or [0])
        self.slot_bytes = (self.slot_bytes + 255) // 256 * 256
        self.slots = torch.empty(6 * self.slot_bytes, dtype=torch.uint8, device=self.dev) if self.slot_bytes else None
        self.g = torch.empty((m, inter), dtype=torch.float32, device=self.dev)
        self.h = torch.empty((m, inter), dtype=torch.int16, device=self.dev)
        self.y = torch.empty((m, hidden), dtype=torch.float32, device=self.dev)
        self.xo = torch.empty((2, m, hidden), dtype=torch.int16, device=self.dev)
        need = max(uw_workspace_size(cm.d, m, UW_PIPE_DIRECT_PALETTE) for cm in flat)
        self.ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.dev) if need else None
        self.dws = torch.zeros(64, dtype=torch.int32, device=self.dev)
        # overlap=False decodes on the main stream (the same ordering, no concurrency): the
        # baseline the side stream is measured against.  Streams keep the default priority.
        self.side = torch.cuda.Stream(device=self.dev) if overlap else torch.cuda.current_stream(self.dev)
        self.sched = Sched([cm.d for cm in flat], hard, m, hidden, inter, self.slots, self.slot_bytes, self.g, self.h,
                           self.y, self.xo, self.ws, self.dws, eps, torch.cuda.current_stream(self.dev), self.side)
        if decode_workgroups:
            self.sched.split(decode_workgroups)

    def step(self, x, check=True, trace=None):
        """One decode step from x (device int16 [m, hidden], BF16 bits) on the current stream
        (the one bound at construction).  Returns the output half of xo.  trace: optional list
        that receives, per layer, host copies (x_in, g, h, y, x_out) recorded by the library
        during the step (uw_sched_trace) -- for tests; it synchronises."""
        import torch
        m, hid, inter = self.m, self.hidden, self.inter
        per = m * (6 * inter + 6 * hid)
        if trace is not None:
            buf = torch.empty(len(self.layers) * per, dtype=torch.uint8, device=self.dev)
            self.sched.trace(buf)
        addr = self.sched.step(x)
        out = self.xo[0] if addr == self.xo[0].data_ptr() else self.xo[1]
        if trace is not None:
            self.sched.trace(None)
            torch.cuda.synchronize(self.dev)
            host = buf.cpu().numpy()
            cur = x.cpu().numpy()
            for l in range(len(self.layers)):
                rec = host[l * per:(l + 1) * per]
                o = 0
                parts = []
                for cnt, dt in ((m * inter, np.float32), (m * inter, np.int16), (m * hid, np.float32),
                                (m * hid, np.int16)):
                    nb = cnt * np.dtype(dt).itemsize
                    parts.append(rec[o:o + nb].view(dt).reshape(m, -1).copy())
                    o += nb
                trace.append((cur,) + tuple(parts))
                cur = parts[3]
        if check:
            torch.cuda.synchronize(self.dev)
            uw_check(self.dws)
        return out

    def resident_bytes(self):
        """Device bytes the weights need: the resident direct-palette form of easy matrices, the
        bundle of hard ones, and the two slot sets."""
        easy = sum(cm.resident_bytes() for l, lay in enumerate(self.layers) if l not in self.hard_layers for cm in lay)
        hard = sum(cm.bundle_bytes() for l, lay in enumerate(self.layers) if l in self.hard_layers for cm in lay)
        return easy + hard + (0 if self.slots is None else self.slots.numel())

    def weight_count(self):
        return sum(cm.n * cm.k for lay in self.layers for cm in lay)

    def close(self):
        self.sched.release()
