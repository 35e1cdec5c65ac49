"""Write tests/golden/tiny_greedy.json from the CPU oracle alone.

    python tests/golden/make_golden.py

The pages print no worked values for the decode step, so this fixture is not
a value of theirs: it is the oracle's own greedy run of the tiny decoder
(2 layers, hidden 256, 4 query / 2 kv heads of 64, SwiGLU 1024, vocab 4096,
tied, RMSNorm eps 1e-5, RoPE theta 1e4, seed-0 weights with jittered gains,
the seeded 16-token prompt, then 8 greedy steps from position 16).  It pins
the oracle to its committed behaviour: a later change to the oracle's
arithmetic shows up as a changed token or logit here.  Only oracle/ and the
seeded input generators are called.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_greedy.json")
PROMPT_LEN, STEPS, TOPK, GAIN_JITTER = 16, 8, 5, 0.1


def compute() -> dict:
    import oracle as orc
    from synth_inputs import TINY, make_prompt, make_weights

    ora = orc.Oracle(TINY, make_weights(TINY, master=0, gain_jitter=GAIN_JITTER))
    k, v = ora.new_cache(PROMPT_LEN + STEPS + 1)
    prompt = [int(t) for t in make_prompt(TINY, PROMPT_LEN, master=0)]
    logits = ora.prefill(prompt, k, v)
    first = orc.argmax_first(logits)
    toks, all_logits = ora.greedy(first, PROMPT_LEN, STEPS, k, v)
    steps = []
    for lg in [logits] + list(all_logits):
        lg = np.asarray(lg, dtype=np.float64)
        top = np.argsort(-lg, kind="stable")[:TOPK]
        steps.append({"argmax": int(top[0]), "top": [[int(i), round(float(lg[i]), 6)] for i in top],
                      "max_abs": round(float(np.abs(lg).max()), 6)})
    return {
        "what": "oracle greedy run of the tiny decoder (not a value printed by the pages)",
        "written_by": "tests/golden/make_golden.py (oracle/ and synth_inputs/ only)",
        "model": "tiny: 2L, H256, 4q/2kv x64, SwiGLU 1024, V4096, tied, eps 1e-5, theta 1e4, gains 1+N(0,0.1), seed 0",
        "prompt": prompt,
        "greedy_tokens": [first] + [int(t) for t in toks],
        "steps": steps,
    }


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(compute(), f, indent=1)
        f.write("\n")
    print(OUT)
