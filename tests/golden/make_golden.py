"""Write the oracle's regression fixture for the small fp32 workload
(B=1, T=64, H=1, N=64, zero initial state, seed 0).

The pages print no input/output values for the recurrence, so this fixture
is not a page value: it freezes what the pinned oracle computes, so that any
later change to the oracle's arithmetic shows up as a diff of this file.
It calls only oracle/ and the seeded input generator.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from oracle import oracle as O  # noqa: E402
from linear_recurrent_lm_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "wkv7_small_f32.json")


def compute():
    inp = synth.make_inputs(1, 64, 1, 64, seed=0, dtype="f32")
    f = O.forward(*inp.streams(), checkpoints=True)
    rng = np.random.Generator(np.random.PCG64(100))
    dy = rng.standard_normal((1, 64, 1, 64))
    g = O.backward(*inp.streams(), dy=dy)
    y = f["y"][0, :, 0]
    S = f["s_out"][0, 0]
    return {
        "workload": "B=1 T=64 H=1 N=64 f32, zero initial state, seed 0; dy ~ N(0,1) from PCG64(100)",
        "y_first_tokens": y[:2].tolist(),
        "y_last_token": y[-1].tolist(),
        "s_out_row0": S[0].tolist(),
        "s_out_diag": np.diag(S).tolist(),
        "ckpt2_row5": f["ckpt"][2, 0, 5].tolist(),
        "y_sum": float(y.sum()), "y_sumsq": float((y ** 2).sum()),
        "s_out_sum": float(S.sum()), "s_out_sumsq": float((S ** 2).sum()),
        "grad_sums": {n: float(g[n].sum()) for n in ("dr", "dw", "dk", "dv", "da", "db")},
        "grad_sumsq": {n: float((g[n] ** 2).sum()) for n in ("dr", "dw", "dk", "dv", "da", "db")},
    }


if __name__ == "__main__":
    with open(OUT, "w") as fh:
        json.dump(compute(), fh, indent=1)
    print("wrote", OUT)
