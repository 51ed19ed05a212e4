"""GPU: a context created on a side stream (dory_create's stream argument) computes what a
context on torch's current stream does, bit for bit, with the binding's device tensors
allocated on the current stream and used on the side stream.

Prefill of a 40-token prompt (all rows' logits), then 6 greedy decode steps that feed each
context its own ids, on the tiny fp32 model and on a narrow bf16 shape with 128-wide heads
(MFMA GEMM tiles, flash prefill over a 24-token window, MFMA decode attention); the sampler on a side stream
against the sampler on the current stream.
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

NARROW = dataclasses.replace(synth.MID, d_model=256, n_heads=2, n_kv_heads=1, d_ff=512, vocab=2048, n_in=1,
                             n_rec=2, n_out=1, window=24)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(shape, w, stream):
    m = dory.Model(shape, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=96, max_tokens=64,
                   stream=stream)
    m.set_loops(2)
    prompt = synth.prompt_tokens(shape, 40)
    lg, ids = m.prefill(0, prompt, 40)
    logits, hidden = [lg], [m.last_hidden(1)]
    tok = ids[-1:]
    for _ in range(6):
        lg, tok = m.decode([0], tok)   # the previous call's device ids, on the context's stream
        logits.append(lg)
        hidden.append(m.last_hidden(1))
    torch.cuda.synchronize()
    out = ([t.cpu().numpy() for t in logits], [t.cpu().numpy() for t in hidden])
    m.close()
    return out


@pytest.mark.parametrize("name,shape", [("tiny", synth.TINY), ("narrow-bf16", NARROW)])
def test_side_stream_context_equals_current_stream(name, shape):
    say(f"[{name}] context on a side stream vs on the current stream")
    w = synth.make_weights(shape, seed=3)
    side = torch.cuda.Stream(device="cuda:0")
    lg0, h0 = run(shape, w, None)
    lg1, h1 = run(shape, w, side)
    for a, b in zip(lg0, lg1):
        assert np.array_equal(a, b)
    for a, b in zip(h0, h1):
        assert np.array_equal(a, b)


def test_sampler_on_side_stream():
    say("[sampler] 3 rows of 131072 logits on a side stream vs the current stream")
    g = torch.Generator(device="cpu").manual_seed(7)
    logits = (torch.randn(3, 131072, generator=g) * 4).to("cuda:0")
    u = torch.rand(3, generator=g).to("cuda:0")
    want = dory.sample(logits, u, temperature=1.0, top_p=0.95)
    side = torch.cuda.Stream(device="cuda:0")
    side.wait_stream(torch.cuda.current_stream())
    got = dory.sample(logits, u, temperature=1.0, top_p=0.95, stream=side)
    side.synchronize()
    assert torch.equal(want.cpu(), got.cpu())
