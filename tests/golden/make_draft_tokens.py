"""Write the drafted tokens x[b, i] ~ filtered q_i of every named workload.

The tokens are inputs of the verification step (the draft model's samples);
they are drawn here with the fp64 oracle's inverse CDF from the workload's
seeded draft logits and draft-sampling uniforms, so that the benchmark can
load them without running the oracle.  Calls only oracle/ and synth/.

    python tests/golden/make_draft_tokens.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import WORKLOADS, make_inputs  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "draft_tokens")


def main():
    os.makedirs(OUT, exist_ok=True)
    for name, w in WORKLOADS.items():
        d = make_inputs(w)
        x = np.zeros((w.B, w.K), dtype=np.int64)
        for i in range(w.K):
            x[:, i] = oracle.sample_tokens(oracle.widen(d["draft"][:, i], w.dtype), w.temperature, w.top_k,
                                           w.top_p, d["draft_u"][:, i])
        path = os.path.join(OUT, f"{name}.txt")
        with open(path, "w") as f:
            f.write(f"# drafted tokens [B={w.B}, K={w.K}] of workload {name}, one sequence per line\n")
            for b in range(w.B):
                f.write(" ".join(str(int(v)) for v in x[b]) + "\n")
        print(path)


if __name__ == "__main__":
    main()
