"""Writes tests/golden/oracle_4b_batched_config.json: the oracle's outputs, sampled, for the
benchmark's batched-decode workload on the ~4B shapes: 128 sequences with seeded prompt
lengths uniform in [256, 4096] (seed 2) and seeded prompts (seed 1), the seeded random weights
(seed 0), k = 2, last-loop KV. Rows of a batch do not interact, so the oracle runs only three
of the 128 sequences: the longest (4069 tokens), the shortest (404) and sequence 64 (2261).

For each of them it stores, for the prefill's last row and two greedy decode steps, the greedy
id, the final hidden row (all 3072 values) and the logits at the row's 64 largest and every
64th vocabulary entry, to 8 significant digits. Only the oracle and the seeded input
generators run here (about eight minutes on 16 cores).

    python tests/golden/make_4b_batched_config.py
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

N_SEQ, MIN_LEN, MAX_LEN, K, STEPS, TOP, STRIDE = 128, 256, 4096, 2, 2, 64, 64
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_4b_batched_config.json")


def row_record(logits, token_id, hidden):
    top = np.argsort(-logits, kind="stable")[:TOP]
    idx = np.union1d(top, np.arange(0, logits.shape[0], STRIDE)).astype(np.int64)
    return {"id": int(token_id), "sample_idx": idx.tolist(),
            "logits": [float(f"{v:.8g}") for v in logits[idx]], "hidden": [float(f"{v:.8g}") for v in hidden]}


class Progress(dict):
    """Trace sink for the oracle's forward pass: reports each stage as the oracle records it
    (the input stack's output, then every core loop's state)."""

    def __init__(self, tag, t0):
        super().__init__()
        self.tag, self.t0 = tag, t0

    def __setitem__(self, key, value):
        print(f"  {self.tag}: {key} recorded at {time.time() - self.t0:.0f} s", flush=True)
        super().__setitem__(key, value)

    def setdefault(self, key, default=None):
        out = super().setdefault(key, default)
        print(f"  {self.tag}: {key}[{len(out)}] at {time.time() - self.t0:.0f} s", flush=True)
        return out


def main():
    t0 = time.time()
    w = synth.make_weights(synth.DORY4B, seed=0)
    lens = synth.batch_prompt_lengths(N_SEQ, MIN_LEN, MAX_LEN, seed=2)
    prompts = synth.batch_prompts(synth.DORY4B, lens, seed=1)
    picked = sorted({int(np.argmax(lens)), int(np.argmin(lens)), N_SEQ // 2})
    om = OracleModel(synth.DORY4B, w, "last_loop", K)
    seqs = {}
    toks = []
    for s in picked:
        lg, ids = om.prefill(s, prompts[s], 1, trace=Progress(f"sequence {s}", t0))
        seqs[s] = [row_record(lg[0], ids[0], om.last_hidden[-1])]
        toks.append(int(ids[0]))
        print(f"sequence {s}: {len(prompts[s])}-token prefill done at {time.time() - t0:.0f} s", flush=True)
    for _ in range(STEPS):
        lg, ids = om.decode(picked, toks)
        for i, s in enumerate(picked):
            seqs[s].append(row_record(lg[i], ids[i], om.last_hidden[i]))
        toks = [int(v) for v in ids]
    doc = {"what": "oracle outputs for the ~4B model's batched-decode workload: seeded weights (seed 0), "
                   "128 sequences, prompt lengths uniform in [256, 4096] (seed 2), prompts seed 1, k = 2, "
                   "last-loop KV; per sampled sequence the prefill's last row and 2 greedy decode steps",
           "n_seq": N_SEQ, "loops": K, "kv_mode": "last_loop", "weights_seed": 0,
           "sample": f"the {TOP} largest logits of each row and every {STRIDE}th vocabulary entry",
           "sequences": {str(s): {"prompt_tokens": int(len(prompts[s])), "rows": seqs[s]} for s in picked}}
    with open(OUT, "w") as f:
        json.dump(doc, f, separators=(",", ":"))
    print(f"wrote {OUT} ({os.path.getsize(OUT) / 1e3:.0f} KB) in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
