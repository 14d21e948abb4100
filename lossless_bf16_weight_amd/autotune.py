"""Per-(n, k, m) choice of pipeline and kernel variant by measurement.

Method: Cloudflare blog post "Unweight", autotuning paragraphs -- which of the four pipelines
(full decode, exponent-only, palette transcode, direct palette) is fastest depends on the
weight shape and the batch size, so it is measured per shape and M rather than set by rule;
the result is a table the runtime reads.

Timing is cache-cold: launches rotate over enough copies of the compressed matrix that the
working set is at least twice the 256 MB Infinity Cache, so every launch streams its weights
from HBM.  Each candidate is timed over several rounds, interleaved with the other candidates
(so slow drift of clocks or temperature does not favour one), and scored by its median
per-launch time.  Every launch goes through the C ABI; this module only orchestrates.

Table format: the text file of uw_autotune_load ("n k m pipeline variant" for the pipeline
UW_PIPE_AUTO runs, "variant n k m pipeline variant" for each pipeline's own best variant,
pipeline 5 = the uncompressed BF16 GEMM).
"""
from __future__ import annotations

import argparse
import dataclasses
import sys

import numpy as np

from . import (UW_PIPE_BF16, UW_PIPE_DIRECT_PALETTE, UW_PIPE_EXP_ONLY, UW_PIPE_FULL_DECODE, UW_PIPE_TRANSCODE,
               DMat, uw_autotune_set, uw_autotune_set_variant, uw_blob_info, uw_encode, uw_gemm_bf16, uw_gemm_variant,
               uw_transcode_palette, uw_variant_count, uw_variant_name, uw_workspace_size)

PIPELINES = (UW_PIPE_FULL_DECODE, UW_PIPE_EXP_ONLY, UW_PIPE_TRANSCODE, UW_PIPE_DIRECT_PALETTE)
PIPELINE_NAMES = {UW_PIPE_FULL_DECODE: "full_decode", UW_PIPE_EXP_ONLY: "exp_only", UW_PIPE_TRANSCODE: "transcode",
                  UW_PIPE_DIRECT_PALETTE: "direct_palette", UW_PIPE_BF16: "bf16"}
ROTATE_BYTES = 512e6
SETTLE_MS = 50.0      # untimed load before timing, for the clocks to come up


@dataclasses.dataclass
class Entry:
    n: int
    k: int
    m: int
    pipeline: int
    variant: int
    us: float                      # median per-launch time of this (pipeline, variant)


@dataclasses.dataclass
class Table:
    """Best variant per (n, k, m, pipeline) and the best pipeline per (n, k, m)."""
    best_variant: dict = dataclasses.field(default_factory=dict)   # (n, k, m, pipeline) -> Entry
    all_times: list = dataclasses.field(default_factory=list)      # every Entry measured

    def add(self, e: Entry):
        self.all_times.append(e)
        key = (e.n, e.k, e.m, e.pipeline)
        if key not in self.best_variant or e.us < self.best_variant[key].us:
            self.best_variant[key] = e

    def merge(self, other: "Table"):
        """Add every measurement of another table (e.g. another weight shape of the same model)."""
        for e in other.all_times:
            self.add(e)
        return self

    def best_pipeline(self, n, k, m):
        """Fastest compressed pipeline at (n, k, m) (the uncompressed key is not a choice of uw_gemm)."""
        c = [e for (a, b, mm, p), e in self.best_variant.items() if (a, b, mm) == (n, k, m) and p != UW_PIPE_BF16]
        return min(c, key=lambda e: e.us) if c else None

    def shapes(self):
        return sorted({(n, k, m) for (n, k, m, _) in self.best_variant})

    def apply(self):
        """Install the table in the library (AUTO entries and per-pipeline variants)."""
        for e in self.best_variant.values():
            uw_autotune_set_variant(e.n, e.k, e.m, e.pipeline, e.variant)
        for n, k, m in self.shapes():
            b = self.best_pipeline(n, k, m)
            if b is not None:
                uw_autotune_set(n, k, m, b.pipeline, b.variant)

    def text(self):
        lines = ["# n k m pipeline variant  (pipeline UW_PIPE_AUTO runs)",
                 "# variant n k m pipeline variant  (best variant of each pipeline; 5 = uncompressed BF16)"]
        for n, k, m in self.shapes():
            b = self.best_pipeline(n, k, m)
            if b is not None:
                lines.append("%d %d %d %d %d  # %s %.2f us" % (n, k, m, b.pipeline, b.variant,
                                                                PIPELINE_NAMES[b.pipeline], b.us))
            for p in sorted(PIPELINE_NAMES):
                e = self.best_variant.get((n, k, m, p))
                if e is not None:
                    lines.append("variant %d %d %d %d %d  # %s %s %.2f us" % (
                        n, k, m, p, e.variant, PIPELINE_NAMES[p], uw_variant_name(e.variant), e.us))
        return "\n".join(lines) + "\n"

    def save(self, path):
        with open(path, "w") as f:
            f.write(self.text())


def _time_interleaved(cands, launches, rounds, stream):
    """cands: {key: (fn, copies)}; fn(i) launches one step on copy i (0 <= i < copies).
    Returns {key: median us per launch}."""
    import torch
    per = {key: [] for key in cands}
    for fn, copies in cands.values():               # warm-up: code objects
        for i in range(copies):
            fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Clocks: the GPU needs a few milliseconds of load after an idle host phase before it runs
    # at speed; without this the first round's candidates would be timed at a lower clock.
    fn, copies = next(iter(cands.values()))
    e0.record(stream)
    i = 0
    while True:
        for _ in range(32):
            fn(i % copies)
            i += 1
        e1.record(stream)
        e1.synchronize()
        if e0.elapsed_time(e1) >= SETTLE_MS:
            break
    for r in range(rounds):
        for key, (fn, copies) in cands.items():
            e0.record(stream)
            for i in range(launches):
                fn((r * launches + i) % copies)
            e1.record(stream)
            e1.synchronize()
            per[key].append(1e3 * e0.elapsed_time(e1) / launches)
    return {key: float(np.median(v)) for key, v in per.items()}


class Tuner:
    """Times pipelines x variants for one weight matrix and a set of batch sizes.

    The matrix is encoded once on the host and copied `copies` times to the device (rotation
    keeps each launch cache-cold); the direct-palette index stream is transcoded on the device
    for each copy.  The uncompressed BF16 baseline gets its own rotated copies of W.
    """

    def __init__(self, w, device="cuda:0", blob=None, rotate_bytes=ROTATE_BYTES, bf16=True):
        import torch
        self.w = w
        self.n, self.k = w.shape
        self.dev = torch.device(device)
        self.blob = uw_encode(w) if blob is None else blob
        info = uw_blob_info(self.blob)
        self.resident = int(info["resident_bytes"])
        self.copies = max(2, int(np.ceil(rotate_bytes / self.resident)))
        self.mats = []
        err = torch.zeros(64, dtype=torch.int32, device=self.dev)
        for _ in range(self.copies):
            bd = torch.from_numpy(self.blob).to(self.dev)
            idx = torch.empty(int(info["idx_bytes"]), dtype=torch.uint8, device=self.dev)
            d = DMat(self.blob, bd, idx)
            uw_transcode_palette(d, idx, err)
            self.mats.append(d)
        self.wcopies = max(2, int(np.ceil(rotate_bytes / (2 * self.n * self.k)))) if bf16 else 0
        self.wd = [torch.from_numpy(w.view(np.int16)).to(self.dev) for _ in range(self.wcopies)]
        torch.cuda.synchronize()

    def tune(self, ms, pipelines=PIPELINES, variants=None, bf16=True, launches=40, rounds=5, log=None):
        import torch
        variants = list(range(uw_variant_count())) if variants is None else list(variants)
        stream = torch.cuda.current_stream()
        table = Table()
        g = torch.Generator(device="cpu").manual_seed(0)
        for m in ms:
            x = torch.randn((m, self.k), generator=g).to(torch.bfloat16).view(torch.int16).to(self.dev)
            y = torch.empty((m, self.n), dtype=torch.float32, device=self.dev)
            cands = {}
            for p in pipelines:
                need = uw_workspace_size(self.mats[0], m, p)
                ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.dev) if need else None
                for v in variants:
                    cands[(p, v)] = (lambda i, p=p, v=v, ws=ws, x=x, y=y:
                                     uw_gemm_variant(self.mats[i], x, y, m, p, v, ws), self.copies)
            if bf16 and self.wd:
                for v in variants:
                    cands[(UW_PIPE_BF16, v)] = (lambda i, v=v, x=x, y=y: uw_gemm_bf16(self.wd[i], x, y, m, v),
                                                self.wcopies)
            res = _time_interleaved(cands, launches, rounds, stream)
            for (p, v), us in res.items():
                table.add(Entry(self.n, self.k, m, p, v, us))
            if log:
                b = table.best_pipeline(self.n, self.k, m)
                log("tuned n=%d k=%d m=%d: %s variant %d %.2f us" % (self.n, self.k, m, PIPELINE_NAMES[b.pipeline],
                                                                     b.variant, b.us))
        return table


class StepTuner:
    """End-to-end choice of pipeline and kernel variant per projection of an MLP stack, by
    coordinate descent on the measured time of whole decode steps (autotuning paragraphs of the
    Unweight post: the choices are made by end-to-end throughput, per projection and batch size,
    and written to a per-model configuration file).

    Starting from a configuration (default: every projection on the direct-palette pipeline with
    the library's variant choice), each sweep takes gate, then up, then down: with the other two
    fixed, every candidate (pipeline, variant) of that projection is timed on the full step and the
    fastest kept.  Sweeps repeat until one changes nothing (or max_sweeps).  Timing: `steps`
    back-to-back steps per measurement after a warm-up, the median of `rounds` measurements.
    The step's weights are the stack's own resident matrices (a model's working set: gate, up and
    down of every layer, not cache-resident between steps at the MLP sizes).

    A stack with hard (bundle-only) layers adds one more coordinate, the decode/GEMM split of the
    chip (uw_sched_split): `tune_split` sweeps the decoder workgroup count on a HardEasyStack."""

    def __init__(self, stack, x, pipelines=PIPELINES, variants=None, steps=8, rounds=3):
        self.stack, self.x = stack, x
        self.pipelines = tuple(pipelines)
        self.variants = list(range(uw_variant_count())) if variants is None else list(variants)
        self.steps, self.rounds = steps, rounds
        self.evals = []                              # (config, us) of every measurement

    def candidates(self):
        return [(p, v) for p in self.pipelines for v in self.variants]

    def time_config(self, cfg):
        import torch
        st, x = self.stack, self.x
        for _ in range(2):
            st.step(x, config=cfg, check=False)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per = []
        for _ in range(self.rounds):
            e0.record()
            for _ in range(self.steps):
                st.step(x, config=cfg, check=False)
            e1.record()
            e1.synchronize()
            per.append(1e3 * e0.elapsed_time(e1) / self.steps)
        us = float(np.median(per))
        self.evals.append((dict(cfg), us))
        return us

    def tune(self, start=None, max_sweeps=4, log=None):
        """Returns {"config": {proj: (pipeline, variant)}, "us": tuned us per step,
        "default_us": the starting configuration's, "sweeps": sweeps run}."""
        from .stack import PROJECTIONS
        cfg = dict(start) if start else {k: (UW_PIPE_DIRECT_PALETTE, -1) for k in PROJECTIONS}
        best = self.time_config(cfg)
        default_us = best
        sweeps = 0
        for sweeps in range(1, max_sweeps + 1):
            changed = False
            for proj in PROJECTIONS:
                for cand in self.candidates():
                    if cand == tuple(cfg[proj]):
                        continue
                    trial = dict(cfg)
                    trial[proj] = cand
                    us = self.time_config(trial)
                    if us < best:
                        best, cfg, changed = us, trial, True
                if log:
                    log("sweep %d %s: %s variant %d, %.1f us a step" % (sweeps, proj, PIPELINE_NAMES[cfg[proj][0]],
                                                                      cfg[proj][1], best))
            if not changed:
                break
        return {"config": {k: tuple(v) for k, v in cfg.items()}, "us": best, "default_us": default_us,
                "sweeps": sweeps}

    @staticmethod
    def tune_split(make_stack, x, splits, steps=8, rounds=3, log=None):
        """The decode/GEMM split coordinate of a stack with hard layers: make_stack(split) builds a
        HardEasyStack with that many decoder workgroups (0: the whole chip); returns
        {"decode_workgroups": best, "us": its us per step, "all": {split: us}}."""
        import torch
        res = {}
        for sp in splits:
            st = make_stack(sp)
            try:
                for _ in range(2):
                    st.step(x, check=False)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                per = []
                for _ in range(rounds):
                    e0.record()
                    for _ in range(steps):
                        st.step(x, check=False)
                    e1.record()
                    e1.synchronize()
                    per.append(1e3 * e0.elapsed_time(e1) / steps)
                res[sp] = float(np.median(per))
                if log:
                    log("split %d decoder workgroups: %.1f us a step" % (sp, res[sp]))
            finally:
                st.close()
        best = min(res, key=res.get)
        return {"decode_workgroups": best, "us": res[best], "all": res}


def save_model_config(path, model, m, result, split=None):
    """Per-model configuration file (JSON): per projection the pipeline and variant, the
    decode/GEMM split, and the measured step times."""
    import json
    from . import uw_variant_name
    out = {"model": model, "m": m,
           "projections": {k: {"pipeline": PIPELINE_NAMES[p], "pipeline_id": p, "variant": v,
                               "variant_name": uw_variant_name(v) if v >= 0 else "library default"}
                           for k, (p, v) in result["config"].items()},
           "us_per_step": round(result["us"], 2), "default_us_per_step": round(result["default_us"], 2),
           "sweeps": result["sweeps"]}
    if split is not None:
        out["decode_workgroups"] = split["decode_workgroups"]
        out["split_us_per_step"] = {str(k): round(v, 2) for k, v in split["all"].items()}
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def load_model_config(path):
    """{proj: (pipeline, variant)} and the decode/GEMM split of a per-model configuration file."""
    import json
    d = json.load(open(path))
    cfg = {k: (int(v["pipeline_id"]), int(v["variant"])) for k, v in d["projections"].items()}
    return cfg, int(d.get("decode_workgroups", 0))


def main(argv=None):
    ap = argparse.ArgumentParser(description="Autotune pipelines and kernel variants for one or more weight shapes "
                                             "(synthetic N(0, std^2) BF16 weights of each shape) into one table "
                                             "file, e.g. every projection shape of a model.")
    ap.add_argument("--shape", required=True,
                    help="NxK, or several comma-separated, e.g. 14336x4096,4096x14336 (a Llama-3.1-8B MLP layer)")
    ap.add_argument("--m", default="1,8,32,64", help="comma-separated batch sizes")
    ap.add_argument("--std", type=float, default=0.02)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--out", required=True, help="table file to write (uw_autotune_load format)")
    ap.add_argument("--launches", type=int, default=40)
    ap.add_argument("--rounds", type=int, default=5)
    a = ap.parse_args(argv)
    from . import synth
    rng = np.random.default_rng(a.seed)
    table = Table()
    for shape in a.shape.split(","):
        n, k = (int(v) for v in shape.lower().split("x"))
        w = synth.gaussian_bf16(rng, (n, k), a.std)
        t = Tuner(w)
        table.merge(t.tune([int(v) for v in a.m.split(",")], launches=a.launches, rounds=a.rounds,
                           log=lambda s: print(s, file=sys.stderr, flush=True)))
        del t   # its rotated device copies
    table.save(a.out)
    sys.stdout.write(table.text())


if __name__ == "__main__":
    main()
