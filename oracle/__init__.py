"""Plain CPU oracle for lossless BF16 weight compression (Unweight-style).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link this
package: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg use it.  It shares no code, tables or constants generator with the HIP library; the
two meet only through the seeded input generator (``lossless_bf16_weight_amd.synth``),
which holds none of the method's arithmetic.

The oracle is written from the Cloudflare blog post "Unweight" (unweight-tensor-compression):
the BF16 anatomy paragraph, the exponent-distribution paragraph and its figure, the Huffman
paragraph, the rare-exponent (verbatim row) paragraph and the four-pipeline paragraphs.
Where that post is silent the oracle states its reading in the docstring of the function
that takes it.

Modules
-------
codec  -- field split, exponent histogram, top-16 palette, verbatim segments,
          length-limited Huffman code, chunked bitstream, tiled layouts, blob,
          decoders (sequential and chunk-lockstep), palette reconstruction.
gemm   -- fp64-accumulate reference GEMM, error scale sum |x*w|, SwiGLU/RMSNorm glue.

Pins (tests/test_oracle_*.py) tie every function to something other than itself.
Parity unpinned: nothing in ``codec`` or ``gemm``; the compression *ratios* against the
post's trained-model figures are only loose bands (synthetic weights stand in).
"""
from . import codec, gemm  # noqa: F401
