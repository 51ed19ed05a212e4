"""Writes tests/golden/oracle_4b_bench_config.json: the oracle's outputs, sampled, for the
benchmark's headline workload on the ~4B shapes (d = 3072, 24/8 heads of 128, FFN 8192,
V = 131072, stacks 8/20/8, window 4096, bf16 storage points): the seeded random weights
(seed 0), the seeded 2560-token prompt, k = 2, last-loop KV, then two greedy decode steps.

For the prefill's last row and each decode step it stores the oracle's greedy id, its final
hidden row (all 3072 values) and its logits at a sample of the vocabulary: the row's 64 largest
and every 64th entry, to 8 significant digits (far below the comparison bars). Only the oracle
and the seeded input generators run here (about three minutes on 16 cores); the GPU test
replays the same calls and compares at the sampled entries.

    python tests/golden/make_4b_bench_config.py
"""
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from looped_ngpt_language_amd import synth  # noqa: E402
from oracle import OracleModel  # noqa: E402

PROMPT, K, STEPS, TOP, STRIDE = 2560, 2, 2, 64, 64
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_4b_bench_config.json")


def row_record(logits, token_id, hidden):
    top = np.argsort(-logits, kind="stable")[:TOP]
    idx = np.union1d(top, np.arange(0, logits.shape[0], STRIDE)).astype(np.int64)
    return {"id": int(token_id), "sample_idx": idx.tolist(),
            "logits": [float(f"{v:.8g}") for v in logits[idx]], "hidden": [float(f"{v:.8g}") for v in hidden]}


def main():
    t0 = time.time()
    w = synth.make_weights(synth.DORY4B, seed=0)
    prompt = synth.prompt_tokens(synth.DORY4B, PROMPT)
    om = OracleModel(synth.DORY4B, w, "last_loop", K)
    lg, ids = om.prefill(0, prompt, 1)
    rows = [row_record(lg[0], ids[0], om.last_hidden[-1])]
    print(f"prefill of {PROMPT} tokens: {time.time() - t0:.0f} s", flush=True)
    tok = int(ids[0])
    for _ in range(STEPS):
        lg, ids = om.decode([0], [tok])
        rows.append(row_record(lg[0], ids[0], om.last_hidden[0]))
        tok = int(ids[0])
    doc = {"what": "oracle outputs for the ~4B model: seeded weights (seed 0), seeded 2560-token prompt, "
                   "k = 2, last-loop KV; the prefill's last row, then 2 greedy decode steps",
           "prompt_tokens": PROMPT, "loops": K, "kv_mode": "last_loop", "weights_seed": 0,
           "sample": f"the {TOP} largest logits of each row and every {STRIDE}th vocabulary entry",
           "rows": rows}
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
    print(f"wrote {OUT} ({os.path.getsize(OUT) / 1e3:.0f} KB) in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
