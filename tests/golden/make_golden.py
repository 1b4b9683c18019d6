"""Write tests/golden/osr_tiny.json from the fp64 oracle (and nothing else).

The pages print no worked numeric example of the recurrence, so this fixture
is a regression guard for the oracle itself: small seeded inputs and the
oracle's outputs for both objectives, at C = 1 (exact) and C = 4 (chunked).
Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from compressed_memory_linear_amd import synth  # noqa: E402


def main():
    cases = []
    for mode, C in ((oracle.MODE_DEC, 1), (oracle.MODE_DEC, 4), (oracle.MODE_SIM, 1),
                    (oracle.MODE_SIM, 4)):
        inp = synth.make_inputs(1, 8, 2, 3, 4, seed=77, in_dtype=synth.F32)
        q, k, v, g, mu, S0 = inp.values_f64()
        y, S = oracle.osr_forward(q, k, v, g, mu, S0, chunk_size=C, mode=mode)
        cases.append(dict(mode=mode, chunk_size=C, q=q.tolist(), k=k.tolist(), v=v.tolist(),
                          gamma=g.tolist(), mu=mu.tolist(), state_in=S0.tolist(),
                          y=y.tolist(), state_out=S.tolist()))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "osr_tiny.json")
    with open(out, "w") as f:
        json.dump({"source": "oracle/osr_oracle.c via tests/golden/make_golden.py",
                   "cases": cases}, f, indent=0)
    print(out)


if __name__ == "__main__":
    main()
