"""Consistency of the stored oracle outputs the full-size GPU tests compare against
(tests/golden/oracle_4b_*_config.json, written by the make_4b_*_config.py scripts beside them,
which run only the oracle). Checked here without a GPU: every stored hidden row is a final
state of the model, so it has unit L2 norm (up to the 8 stored digits); every row's greedy id is
among its sampled entries and has the largest sampled logit (the sample holds the row's 64
largest logits); the sampled indices are sorted, unique and inside the vocabulary."""
import json
import os

import numpy as np
import pytest

from looped_ngpt_language_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows_of(name):
    doc = json.load(open(os.path.join(GOLDEN, name)))
    if "rows" in doc:
        return doc, doc["rows"]
    return doc, [r for s in doc["sequences"].values() for r in s["rows"]]


@pytest.mark.parametrize("name", ["oracle_4b_bench_config.json", "oracle_4b_batched_config.json"])
def test_golden_rows_are_consistent(name):
    doc, rows = rows_of(name)
    assert doc["kv_mode"] == "last_loop" and doc["loops"] == 2
    for r in rows:
        idx = np.array(r["sample_idx"])
        lg = np.array(r["logits"])
        h = np.array(r["hidden"])
        assert h.shape == (synth.DORY4B.d_model,)
        assert abs(float(np.linalg.norm(h)) - 1.0) < 1e-6
        assert idx.shape == lg.shape and idx.size >= 64
        assert np.all(np.diff(idx) > 0) and idx[0] >= 0 and idx[-1] < synth.DORY4B.vocab
        assert r["id"] in set(idx.tolist())
        assert int(idx[np.argmax(lg)]) == r["id"]


def test_batched_golden_picks_the_workload_sequences():
    doc, _ = rows_of("oracle_4b_batched_config.json")
    lens = synth.batch_prompt_lengths(doc["n_seq"], 256, 4096, seed=2)
    picked = sorted(int(s) for s in doc["sequences"])
    assert picked == sorted({int(np.argmax(lens)), int(np.argmin(lens)), doc["n_seq"] // 2})
    for s in picked:
        assert doc["sequences"][str(s)]["prompt_tokens"] == int(lens[s])
