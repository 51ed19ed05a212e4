"""Run-twice determinism: no reduction on the GPU path uses floating-point atomics or an order that
depends on scheduling (split-K partials and split-attention partials are summed in a fixed order;
the sampler's masses are integers), so the same calls on fresh contexts give bitwise-identical
logits, hidden rows and ids. Covers batch-1 decode with split attention and the fused GEMV
path, a prefill chunk of 5 rows (multi-row attention, 3..8-row GEMV), and batched decode of 20
rows (VALU split kernel, split-K projections)."""
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

NARROW3 = dataclasses.replace(synth.MID, d_model=384, n_heads=3, n_kv_heads=1, d_ff=768, vocab=4096, n_in=2,
                              n_rec=4, n_out=2, window=1000)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_mid(w):
    m = dory.Model(synth.MID, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=1400, max_tokens=1200)
    m.set_loops(2)
    prompt = synth.prompt_tokens(synth.MID, 1200)
    out = []
    lg, ids = m.prefill(0, prompt, 1)
    out.append(lg.cpu().numpy())
    tok = ids
    for _ in range(4):
        lg, tok = m.decode([0], tok)
        out.append(lg.cpu().numpy())
        out.append(m.last_hidden(1).cpu().numpy())
    lg, _ = m.prefill(0, synth.prompt_tokens(synth.MID, 5, seed=9), 5)
    out.append(lg.cpu().numpy())
    m.close()
    return out


def run_batched(w):
    n = 20
    lens = synth.batch_prompt_lengths(n, 300, 2500, seed=3)
    prompts = synth.batch_prompts(NARROW3, lens, seed=4)
    m = dory.Model(NARROW3, w, kv_mode="per_loop", max_loops=2, max_seqs=n, max_model_len=2600, max_tokens=2500)
    m.set_loops(2)
    firsts = [m.prefill(s, p, 1)[1] for s, p in enumerate(prompts)]
    tok = torch.cat(firsts)
    out = []
    for _ in range(3):
        lg, tok = m.decode(list(range(n)), tok)
        out.append(lg.cpu().numpy())
        out.append(m.last_hidden(n).cpu().numpy())
    m.close()
    return out


def test_bs1_and_chunk_bitwise_repeatable():
    w = synth.make_weights(synth.MID, seed=0)
    a, b = run_mid(w), run_mid(w)
    same = all(np.array_equal(x, y) for x, y in zip(a, b))
    say(f"[determinism] mid bs1 decode + 5-row chunk: bitwise equal {same}")
    assert same


def test_batched_bitwise_repeatable():
    w = synth.make_weights(NARROW3, seed=0)
    a, b = run_batched(w), run_batched(w)
    same = all(np.array_equal(x, y) for x, y in zip(a, b))
    say(f"[determinism] narrow3 20-row batched decode: bitwise equal {same}")
    assert same
