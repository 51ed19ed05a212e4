"""Greedy argmax ties on the GPU: the lowest id among the largest logits.

The LM head's rows are copies of 7 distinct unit rows (each id draws its row from a seeded
random group), so every logit of a row ties exactly with the other ids of its group and the
argmax is always a tie. Checked through the C ABI on the tiny fp32 model (ids bit-exact with the
oracle, which takes the lowest id in float32) and on a bf16 model with a 131072-token
vocabulary, where the two-pass argmax splits a row into 64 parts and ties straddle parts:
  * the GPU's logits of one group are bitwise equal (tied rows give tied logits);
  * the GPU's id is the lowest id attaining the GPU's own maximum;
  * against the oracle: bf16 logits within 5e-2, ids equal except near-ties.
"""
import dataclasses
import sys

import numpy as np
import pytest

from looped_ngpt_language_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from looped_ngpt_language_amd import dory  # noqa: E402
from oracle import OracleModel  # noqa: E402

NARROW_V = dataclasses.replace(synth.MID, d_model=384, n_heads=3, n_kv_heads=1, d_ff=768, vocab=131072, n_in=1,
                               n_rec=2, n_out=1, window=64)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tied_weights(shape, seed):
    w = synth.make_weights(shape, seed=seed)
    rng = np.random.default_rng(99)
    group = rng.integers(0, 7, shape.vocab)
    w.lm_head = np.ascontiguousarray(w.lm_head[:7][group])
    return w, group


def check_gpu_ties(lg, ids, group):
    """Within a row: logits of one group bitwise equal; id = lowest index of the row maximum."""
    for r in range(lg.shape[0]):
        row = lg[r]
        for gi in range(7):
            vals = row[group == gi]
            assert np.all(vals == vals[0]), f"row {r}: group {gi} logits differ on the GPU"
        top = np.flatnonzero(row == row.max())
        assert int(ids[r]) == int(top[0]), (r, int(ids[r]), top[:4])
        assert len(top) > 1           # the maximum is a tie


def test_argmax_ties_fp32_tiny():
    shape = synth.TINY
    w, group = tied_weights(shape, 0)
    m = dory.Model(shape, w, kv_mode="last_loop", max_loops=2, max_seqs=4, max_model_len=64, max_tokens=32)
    m.set_loops(2)
    om = OracleModel(shape, w, "last_loop", 2)
    say("[tiny fp32] argmax ties: 20-token prompt, all-row logits, then 4 batched decode rows")
    prompt = synth.prompt_tokens(shape, 20)
    lg, ids = m.prefill(0, prompt, 20)
    olg, oids = om.prefill(0, prompt, 20)
    lg, ids = lg.cpu().numpy(), ids.cpu().numpy()
    check_gpu_ties(lg, ids, group)
    assert np.max(np.abs(lg - olg)) <= 1e-4
    np.testing.assert_array_equal(ids, oids)
    for s in (1, 2, 3):
        m.prefill(s, prompt[:5 + s], 1)
        om.prefill(s, prompt[:5 + s], 1)
    toks = [3, 17, 256, 900]
    lg, ids = m.decode([0, 1, 2, 3], torch.tensor(toks, dtype=torch.int32, device=m.device))
    olg, oids = om.decode([0, 1, 2, 3], toks)
    lg, ids = lg.cpu().numpy(), ids.cpu().numpy()
    check_gpu_ties(lg, ids, group)
    assert np.max(np.abs(lg - olg)) <= 1e-4
    np.testing.assert_array_equal(ids, oids)
    say(f"  ids {list(ids)} (oracle {list(oids)})")
    m.close()


def test_argmax_ties_bf16_wide_vocab():
    shape = NARROW_V
    w, group = tied_weights(shape, 1)
    m = dory.Model(shape, w, kv_mode="last_loop", max_loops=2, max_seqs=20, max_model_len=64, max_tokens=32)
    m.set_loops(2)
    om = OracleModel(shape, w, "last_loop", 2)
    say("[narrow bf16, V=131072] argmax ties: batch-1 decode and 20 batched rows")
    prompts = synth.batch_prompts(shape, synth.batch_prompt_lengths(20, 3, 30, seed=4), seed=5)
    firsts = []
    for s, p in enumerate(prompts):
        lg, ids = m.prefill(s, p, 1)
        olg, oids = om.prefill(s, p, 1)
        lg, ids = lg.cpu().numpy(), ids.cpu().numpy()
        check_gpu_ties(lg, ids, group)
        assert np.max(np.abs(lg - olg)) <= 5e-2
        if ids[0] != oids[0]:
            assert olg[0][oids[0]] - olg[0][ids[0]] < 2 * np.max(np.abs(lg - olg))
        firsts.append(int(oids[0]))
    lg, ids = m.decode([0], torch.tensor(firsts[:1], dtype=torch.int32, device=m.device))   # batch 1
    check_gpu_ties(lg.cpu().numpy(), ids.cpu().numpy(), group)
    lg, ids = m.decode(list(range(1, 20)), torch.tensor(firsts[1:], dtype=torch.int32, device=m.device))
    olg, oids = om.decode(list(range(1, 20)), firsts[1:])
    lg, ids = lg.cpu().numpy(), ids.cpu().numpy()
    check_gpu_ties(lg, ids, group)
    err = np.max(np.abs(lg - olg))
    say(f"  19 rows: logits max-abs {err:.2e}, ids equal {int(np.sum(ids == oids))}/19")
    assert err <= 5e-2
    for r in range(19):
        if ids[r] != oids[r]:
            assert olg[r][oids[r]] - olg[r][ids[r]] < 2 * np.max(np.abs(lg[r] - olg[r]))
    m.close()
