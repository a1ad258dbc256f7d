"""Writes tests/golden/tiny_f32_oracle.json from the CPU oracle alone.

The pages print no worked example with values, so this fixture is not a pin of
the oracle: it freezes the oracle's output on the seeded tiny fp32 workload
(batch 1, seqlen 256, 4 heads, headdim 16, d_state 16, chunk 64) so that a
later change to the oracle or to the input recipe shows up as a diff.  Run:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from mamba_ssd_chunked_scan_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.json")


def sample_indices(shape, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(count)]


def main():
    spec = synth.WORKLOADS["tiny_f32"]
    inp = synth.scan_inputs(spec)
    y, fin = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init"], nthreads=1)
    yi = sample_indices(y.shape, 64, 100)
    fi = sample_indices(fin.shape, 32, 101)
    doc = {
        "workload": spec.name,
        "what": "oracle outputs at sampled indices of y [B,L,H,P] and final_state [B,H,P,N]",
        "source": "written by tests/golden/make_golden.py from oracle.scan only",
        "y": [[list(i), float(y[i])] for i in yi],
        "final": [[list(i), float(fin[i])] for i in fi],
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
