"""Long prompts in one chunk: properties that hold at any size, at 32768, 131072 and 262144 tokens.

Under the chunk semantics (a call's keys/values are written before its queries read them, in
every block application), per-loop results do not depend on how a prompt is split into chunks,
and for a prompt prefilled as one chunk last-loop and per-loop give the same activations (every
loop's queries see that loop's keys of the same chunk). Neither the oracle nor a page prints
values at these lengths, so the GPU is checked against these identities:

  * narrow bf16 model (128-wide heads, 3 query heads per KV head), 32768 tokens, k = 2:
    last-loop in one chunk == per-loop in one chunk == per-loop in 8192-token chunks;
  * the ~4B model, 131072 tokens, k = 4 (the long-context workload): last-loop in one chunk ==
    per-loop in 8192-token chunks, on the last row's logits and final hidden state;
  * the ~4B model, 262144 tokens (the longest context the pages give), k = 1: one chunk == two
    131072-token chunks.

The GEMM tiles, split-K choices and flash row blocks differ between one chunk and several, so
the results agree to bf16 rounding noise, not bitwise: 1e-3 on logits, 1e-3 on hidden rows.
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

NARROW3 = dataclasses.replace(synth.MID, d_model=384, n_heads=3, n_kv_heads=1, d_ff=768, vocab=4096, n_in=2,
                              n_rec=4, n_out=2, window=1000)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def prefill_chunks(m, prompt, chunk):
    for a in range(0, len(prompt), chunk):
        lg, ids = m.prefill(0, prompt[a:a + chunk], 1)
    return lg[0].cpu().numpy(), m.last_hidden(1)[0].cpu().numpy(), int(ids[0].item())


def compare(tag, a, b, bar=1e-3):
    el = float(np.max(np.abs(a[0] - b[0])))
    eh = float(np.max(np.abs(a[1] - b[1])))
    say(f"  {tag}: logits max-abs {el:.2e}, hidden max-abs {eh:.2e}, ids {a[2]} / {b[2]}")
    assert np.isfinite(a[0]).all() and np.isfinite(b[0]).all()
    assert el <= bar and eh <= bar


def test_narrow_32k_one_chunk_equals_chunks():
    T, k = 32768, 2
    w = synth.make_weights(NARROW3, seed=0)
    prompt = torch.from_numpy(synth.prompt_tokens(NARROW3, T)).to("cuda:0")
    say(f"[narrow3 bf16] {T}-token prompt, k={k}: one chunk vs 8192-token chunks")
    res = {}
    for mode, chunk in (("last_loop", T), ("per_loop", T), ("per_loop", 8192)):
        m = dory.Model(NARROW3, w, kv_mode=mode, max_loops=k, max_seqs=1, max_model_len=T + 16, max_tokens=chunk)
        m.set_loops(k)
        res[(mode, chunk)] = prefill_chunks(m, prompt, chunk)
        m.close()
        del m
    compare("last-loop one chunk vs per-loop one chunk", res[("last_loop", T)], res[("per_loop", T)], bar=1e-6)
    compare("per-loop one chunk vs 8192-token chunks", res[("per_loop", T)], res[("per_loop", 8192)])


def test_4b_131072_one_chunk_last_loop_equals_per_loop_chunks():
    T, k = 131072, 4
    say(f"[4B] {T}-token prompt, k={k}: last-loop one chunk vs per-loop 8192-token chunks")
    w = synth.make_weights(synth.DORY4B, seed=0)
    prompt = torch.from_numpy(synth.prompt_tokens(synth.DORY4B, T, seed=1)).to("cuda:0")
    m1 = dory.Model(synth.DORY4B, w, kv_mode="last_loop", max_loops=k, max_seqs=1, max_model_len=T + 16,
                    max_tokens=T)
    del w
    m1.set_loops(k)
    one = prefill_chunks(m1, prompt, T)
    say("  one-chunk prefill done")
    m2 = dory.Model(synth.DORY4B, None, kv_mode="per_loop", max_loops=k, max_seqs=1, max_model_len=T + 16,
                    max_tokens=8192, share_weights_from=m1)
    m2.set_loops(k)
    chunked = prefill_chunks(m2, prompt, 8192)
    compare("last-loop one chunk vs per-loop 8192-token chunks", one, chunked)
    m2.close()
    m1.close()


def test_4b_262144_one_chunk_equals_two_chunks():
    """The pages' longest context (256K = 262144 tokens) prefilled as one chunk, k = 1: the down
    projection's activation operand (262144 x 8192 bf16) passes 4 GiB, so its GEMM runs in row
    blocks. At k = 1 the result does not depend on the chunking (the last-loop cache is the
    per-loop one), so the one-chunk last row equals that of two 131072-token chunks."""
    T, k = 262144, 1
    say(f"[4B] {T}-token prompt, k={k}: one chunk vs two {T // 2}-token chunks")
    w = synth.make_weights(synth.DORY4B, seed=0)
    prompt = torch.from_numpy(synth.prompt_tokens(synth.DORY4B, T, seed=1)).to("cuda:0")
    m1 = dory.Model(synth.DORY4B, w, kv_mode="last_loop", max_loops=k, max_seqs=1, max_model_len=T,
                    max_tokens=T)
    del w
    m1.set_loops(k)
    one = prefill_chunks(m1, prompt, T)
    say("  one-chunk prefill done")
    m1.close()
    m1.pool = m1.ws = None          # the weights stay, shared with the second context
    torch.cuda.empty_cache()
    m2 = dory.Model(synth.DORY4B, None, kv_mode="last_loop", max_loops=k, max_seqs=1, max_model_len=T,
                    max_tokens=T // 2, share_weights_from=m1)
    m2.set_loops(k)
    chunked = prefill_chunks(m2, prompt, T // 2)
    compare("one chunk vs two chunks", one, chunked)
    m2.close()
