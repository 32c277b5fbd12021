"""Write input_fingerprints.txt: SHA-256 prefixes of the seeded synthetic
inputs of every workload, so that a change of the recipe (seeds, lengths,
outlier channels, block layout) or of the random streams it draws from shows
up as a failing CPU test instead of silently changing every measurement.

Per workload: the context lengths and the block tables of the full-size
layout (host block manager, shuffled free list), and the fp16 K, V and Q of
layer 0 drawn on the CPU for 4,096 unique tokens.  Only the input module is
called (it holds none of the method's arithmetic).  Run from the repository
root: python tests/golden/make_input_fingerprints.py
"""
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from paged_quantized_kv_cache_amd import workloads as W  # noqa: E402

NTOK = 4096


def _h(b: bytes) -> str:
    return hashlib.sha256(b).hexdigest()[:16]


def fingerprints(name: str) -> dict:
    s = W.spec(name)
    rng = np.random.default_rng(s.seed)
    lens = W.draw_lengths(s, rng)
    layout = W.build_layout(s, lens, rng)
    d = W.gen_layer(s, NTOK, 0, device="cpu")
    return {"lens": _h(lens.astype(np.int64).tobytes()),
            "tables": _h(layout.block_tables.astype(np.int32).tobytes()),
            "k": _h(d.k.numpy().tobytes()), "v": _h(d.v.numpy().tobytes()),
            "q": _h(d.q.numpy().tobytes())}


def main() -> None:
    lines = ["# SHA-256 prefixes of the seeded inputs (written by make_input_fingerprints.py)",
             "# workload lens tables k v q"]
    for name in sorted(W.SPECS):
        f = fingerprints(name)
        lines.append(" ".join([name] + [f[k] for k in ("lens", "tables", "k", "v", "q")]))
    with open(os.path.join(HERE, "input_fingerprints.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
