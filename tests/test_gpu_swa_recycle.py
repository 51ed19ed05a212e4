"""GPU parity of sliding-window page recycling (DORY_FLAG_SWA_RECYCLE): the same calls with and
without recycling give bit-identical logits and ids (only the physical pages differ), while the
window pages in use stay bounded; and a recycled tiny-model run matches the oracle."""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def mid_weights():
    return synth.make_weights(synth.MID, seed=0)


def run_chunks_and_decode(m, mode, prompt, chunk, steps, k=2):
    m.set_kv_mode(mode)
    m.set_loops(k)
    logs, ids = [], []
    for i in range(0, len(prompt), chunk):
        lg, gid = m.prefill(0, prompt[i:i + chunk], 1)
        logs.append(lg[0].cpu().numpy().copy())
        ids.append(int(gid[0].item()))
    tok = ids[-1]
    swa_max = 0
    for _ in range(steps):
        lg, gid = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        logs.append(lg[0].cpu().numpy().copy())
        tok = int(gid[0].item())
        ids.append(tok)
        swa_max = max(swa_max, m.stats()["swa_pages_in_use"])
    m.release(0)
    return np.array(logs), ids, swa_max


@pytest.mark.parametrize("mode", ["last_loop", "per_loop"])
def test_mid_recycling_is_bit_exact(mid_weights, mode):
    prompt = synth.prompt_tokens(synth.MID, 2048)
    kw = dict(max_loops=2, max_seqs=1, max_model_len=2048 + 64, max_tokens=512)
    say(f"[swa] mid {mode} k=2: 2048-token prompt in 512-token chunks, 48 decode steps")
    a = dory.Model(synth.MID, mid_weights, kv_mode=mode, **kw)
    la, ia, _ = run_chunks_and_decode(a, mode, prompt, 512, 48)
    a.close()
    b = dory.Model(synth.MID, mid_weights, kv_mode=mode, swa_recycle=True, **kw)
    lb, ib, swa_max = run_chunks_and_decode(b, mode, prompt, 512, 48)
    b.close()
    bound = (1024 + 64 + 512) // 16 + 3
    say(f"  ids equal {ia == ib}, max |logit diff| {np.max(np.abs(la - lb)):.3e}, window pages held <= {swa_max} "
        f"(bound {bound}, without recycling {-(-(2048 + 48) // 16)})")
    assert ia == ib
    np.testing.assert_array_equal(la, lb)
    assert swa_max <= bound


def test_mid_two_sequences_reuse_recycled_pages(mid_weights):
    """Two sequences decoded in one call per step: pages one releases by recycling serve the other,
    and a rollback inside the reserve still reproduces the run without recycling."""
    kw = dict(kv_mode="last_loop", max_loops=2, max_seqs=2, max_model_len=2048 + 64, max_tokens=1024)
    prompts = [synth.prompt_tokens(synth.MID, 1600), synth.prompt_tokens(synth.MID, 1100)[::-1].copy()]
    outs = []
    for rec in (False, True):
        m = dory.Model(synth.MID, mid_weights, swa_recycle=rec, **kw)
        m.set_loops(2)
        toks = []
        for s_, p in enumerate(prompts):
            for i in range(0, len(p), 1024):
                _, gid = m.prefill(s_, p[i:i + 1024], 1)
            toks.append(int(gid[0].item()))
        seq = []
        for step in range(40):
            lg, gid = m.decode([0, 1], torch.tensor(toks, dtype=torch.int32, device=m.device))
            seq.append(lg.cpu().numpy().copy())
            toks = [int(x) for x in gid.cpu().numpy()]
            if step == 20:
                m.truncate(0, m.seq_len(0) - 8)          # roll sequence 0 back by 8 tokens
        outs.append((np.array(seq), m.stats()))
        m.close()
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    say(f"[swa] two sequences: bit-exact; window pages in use {outs[1][1]['swa_pages_in_use']} of "
        f"{outs[1][1]['swa_pages_total']}")


def test_tiny_recycled_decode_matches_oracle():
    """fp32 tiny model, window 16: 64-token prompt then 300 greedy steps with recycling, against
    the oracle (max-abs 1e-4 on logits, ids equal)."""
    w = synth.make_weights(synth.TINY, seed=0)
    m = dory.Model(synth.TINY, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=512, max_tokens=64,
                   swa_recycle=True)
    m.set_loops(2)
    om = OracleModel(synth.TINY, w, "last_loop", 2)
    prompt = synth.prompt_tokens(synth.TINY, 64)
    lg, gid = m.prefill(0, prompt, 1)
    olg, oid = om.prefill(0, prompt, 1)
    err = float(np.max(np.abs(lg[0].cpu().numpy() - olg[0])))
    tok = int(oid[0])
    for _ in range(300):
        lg, gid = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        olg, oid = om.decode([0], [tok])
        err = max(err, float(np.max(np.abs(lg[0].cpu().numpy() - olg[0]))))
        assert int(gid[0].item()) == int(oid[0])
        tok = int(oid[0])
    st = m.stats()
    say(f"[swa] tiny fp32 recycled: 300 steps, logits max-abs {err:.2e}, window pages held {st['swa_pages_in_use']}")
    assert err <= 1e-4
    assert st["swa_pages_in_use"] <= (16 + 64 + 64) // 16 + 3
