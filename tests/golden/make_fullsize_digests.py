"""Write tests/golden/fullsize_digests.txt: SHA-256 digests of what the oracle produces for the
full-size workloads (the encoded blob, the direct-palette index stream of the load-time
transcode, the exponent-only stream), so tests can compare the C++ encoder and the device
decoders with the oracle bit for bit at full size without re-running the slow oracle.

Calls only the oracle and the seeded input generators.  Takes several minutes:
    python tests/golden/make_fullsize_digests.py
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from lossless_bf16_weight_amd import synth  # noqa: E402
from oracle import codec  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fullsize_digests.txt")
CONFIGS = {"c1": synth.config1, "c2": synth.config2, "c3": synth.config3, "c5": synth.config5}


def sha(b):
    return hashlib.sha256(np.ascontiguousarray(b).tobytes()).hexdigest()


def main():
    lines = ["# Oracle digests at full size (written by make_fullsize_digests.py from oracle/ only).",
             "# config w_digest blob_sha256 transcode_sha256 exponent_stream_sha256 blob_bytes"]
    for name, make in CONFIGS.items():
        t0 = time.time()
        w = make()["w"]
        n, k = w.shape
        blob = codec.serialize(codec.encode(w, n, k))
        assert np.array_equal(codec.decode_blob(blob), w), name
        lines.append("%s %s %s %s %s %d" % (name, synth.digest(w), sha(np.frombuffer(blob, np.uint8)),
                                            sha(codec.transcode_blob(blob)), sha(codec.exponent_stream_blob(blob)),
                                            len(blob)))
        print(lines[-1], "(%.0f s)" % (time.time() - t0), flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
