"""Decode-attention parity at the key-split depths the benchmark runs, against the oracle.

The ~4B benchmark decodes at batch 1 after a 2560-token prompt: the split-key MFMA kernel then
takes 21..23 splits per (row, KV head) (128 keys per split), and the split merge runs two groups
(16 + the rest). Batched decode of 128 ragged sequences and 131072-token contexts take up to 32
splits, on the VALU kernel (longest row first) and on the MFMA kernel respectively. A narrow bf16 model with the ~4B
attention geometry per KV head (128-wide heads, 3 query heads per KV head, scale sqrt(128)) and
a window of 1000 (not a page multiple) reaches those depths at sizes the oracle computes in
about a minute:

  * batch 1 after 2560- and 4400-token prompts: 21 and 32 splits (MFMA kernel, both merge
    groups);
  * 20 rows of 300..6000 keys decoded together: up to 24 splits (VALU kernel), ragged rows,
    empty trailing splits for the short rows, window edges inside pages.

Oracle side: one whole-prompt prefill of a 6000-token prompt (k = 2, last-loop). Within one
chunk, row i depends only on tokens 0..i (causal attention, every loop reading the chunk's own
keys), so the cache and logits a whole-prompt prefill of the prefix P[:L] produces are the first
L rows of the long prefill's. Each sequence's oracle state is that prefix, copied; its decode
steps then run on the oracle as usual.

Bars: bf16 (logits 5e-2, final hidden rows 3e-2 max-abs), teacher-forced on the oracle's ids;
a differing id must be a near-tie (oracle margin below twice that step's max logit error).
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
from oracle.model import _Seq  # noqa: E402

NARROW3 = dataclasses.replace(synth.MID, d_model=384, n_heads=3, n_kv_heads=1, d_ff=768, vocab=4096, n_in=2,
                              n_rec=4, n_out=2, window=1000)
LONG = 6000
K = 2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def fork(om, src, dst, n):
    """Oracle sequence dst = the first n positions of sequence src (cache rows copied)."""
    s = om.seqs[src]
    t = _Seq(s.hk, s.dh)
    for sl in s.K:
        t.K[sl] = s.K[sl][:n].copy()
        t.V[sl] = s.V[sl][:n].copy()
        t.written[sl] = s.written[sl][:n].copy()
    t.len = n
    om.seqs[dst] = t


@pytest.fixture(scope="module")
def narrow():
    say(f"[narrow3 bf16] oracle: one {LONG}-token prefill, k={K}, last-loop")
    w = synth.make_weights(NARROW3, seed=0)
    prompt = synth.prompt_tokens(NARROW3, LONG)
    om = OracleModel(NARROW3, w, "last_loop", K)
    om.prefill(0, prompt, 1)
    hidden = om.last_hidden.copy()
    say("  oracle prefill done")
    return w, prompt, om, hidden


def near_tie_ok(g_id, o_id, g_lg, o_lg):
    if g_id == o_id:
        return True
    return o_lg[o_id] - o_lg[g_id] < 2 * np.max(np.abs(g_lg - o_lg))


def check_rows(tag, g_lg, g_ids, o_lg, o_ids, g_h=None, o_h=None):
    err = float(np.max(np.abs(g_lg - o_lg)))
    err_h = float(np.max(np.abs(g_h - o_h))) if g_h is not None else 0.0
    agree = int(np.sum(g_ids == o_ids))
    say(f"  {tag}: logits max-abs {err:.2e}, hidden max-abs {err_h:.2e}, ids {agree}/{len(o_ids)}")
    assert err <= 5e-2
    assert err_h <= 3e-2
    for i in range(len(o_ids)):
        assert near_tie_ok(int(g_ids[i]), int(o_ids[i]), g_lg[i], o_lg[i]), (tag, i)


def test_bs1_decode_21_and_32_splits(narrow):
    """Batch-1 decode (split-key MFMA kernel) after a 2560-token prompt (2561..2563 keys: 21
    splits, merge groups 16 + 5) and after a 4400-token prompt (32 splits, two full merge
    groups), k = 2, last-loop, 3 teacher-forced steps."""
    w, prompt, om, hidden = narrow
    n_dec = 3
    m = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=K, max_seqs=2, max_model_len=4600, max_tokens=4400)
    m.set_loops(K)
    for sid, (L, want_splits) in enumerate(((2560, 21), (4400, 32))):
        say(f"[narrow3 bf16] bs1 decode at {L} keys, expect {want_splits} splits")
        fork(om, 0, 10 + sid, L)
        o_lg0, o_id0 = om.lm_head(hidden[L - 1:L])
        lg, ids = m.prefill(sid, prompt[:L], 1)
        check_rows(f"prefill {L}", lg.cpu().numpy(), ids.cpu().numpy(), o_lg0, o_id0,
                   m.last_hidden(1).cpu().numpy(), hidden[L - 1:L])
        tok = int(o_id0[0])
        g_lg, g_ids, o_lg, o_ids, g_h, o_h = [], [], [], [], [], []
        for _ in range(n_dec):
            l1, i1 = m.decode([sid], torch.tensor([tok], dtype=torch.int32, device=m.device))
            ol, oi = om.decode([10 + sid], [tok])
            g_lg.append(l1[0].cpu().numpy())
            g_ids.append(int(i1[0].item()))
            g_h.append(m.last_hidden(1)[0].cpu().numpy())
            o_lg.append(ol[0])
            o_ids.append(int(oi[0]))
            o_h.append(om.last_hidden[0])
            tok = int(oi[0])
        check_rows(f"decode at {L}", np.array(g_lg), np.array(g_ids), np.array(o_lg), np.array(o_ids),
                   np.array(g_h), np.array(o_h))
        got = m.stats()["max_attn_splits"]
        say(f"  largest split count so far: {got}")
        assert got == want_splits
        del om.seqs[10 + sid]
    m.close()


def test_batched_decode_20_ragged_rows_deep_splits(narrow):
    """20 sequences of 300..6000 tokens decoded together (VALU split kernel, rows longest first,
    up to 24 splits, short rows with empty trailing splits), k = 2, last-loop, 3 steps."""
    w, prompt, om, hidden = narrow
    n_seq, n_dec = 20, 3
    lens = np.concatenate([[300], synth.batch_prompt_lengths(n_seq - 1, 2048, LONG, seed=7)]).astype(int)
    say(f"[narrow3 bf16] batched decode, {n_seq} rows, k={K}, last-loop, lengths {list(lens)}")
    m = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=K, max_seqs=n_seq, max_model_len=LONG + 16,
                   max_tokens=LONG)
    m.set_loops(K)
    o_lg0, o_id0 = om.lm_head(hidden[lens - 1])
    g_lg0, g_id0 = [], []
    for s, L in enumerate(lens):
        fork(om, 0, 100 + s, int(L))
        lg, ids = m.prefill(s, prompt[:L], 1)
        g_lg0.append(lg[0].cpu().numpy())
        g_id0.append(int(ids[0].item()))
    check_rows("prefill rows", np.array(g_lg0), np.array(g_id0), o_lg0, o_id0)
    toks = [int(t) for t in o_id0]
    for step in range(n_dec):
        lg, ids = m.decode(list(range(n_seq)), torch.tensor(toks, dtype=torch.int32, device=m.device))
        g_h = m.last_hidden(n_seq).cpu().numpy()
        o_lg, o_ids, o_h = [], [], []
        for s in range(n_seq):
            ol, oi = om.decode([100 + s], [toks[s]])
            o_lg.append(ol[0])
            o_ids.append(int(oi[0]))
            o_h.append(om.last_hidden[0])
        check_rows(f"step {step}", lg.cpu().numpy(), ids.cpu().numpy(), np.array(o_lg), np.array(o_ids), g_h,
                   np.array(o_h))
        toks = o_ids
    splits = m.stats()["max_attn_splits"]
    say(f"  largest split count: {splits}")
    assert splits >= 17
    for s in range(n_seq):
        del om.seqs[100 + s]
    m.close()


def test_6000_token_prefill_all_rows(narrow):
    """The whole 6000-token prompt prefilled as one chunk on the GPU, every row's final hidden
    state and logits against the oracle's whole-prompt prefill (the module's fixture): 47 row
    blocks of the flash prefill kernel on three query heads per KV head (the last block ragged,
    112 rows), causal and 1000-token-window edges inside pages, k = 2 last-loop."""
    w, prompt, om, hidden = narrow
    m = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=K, max_seqs=1, max_model_len=LONG + 16,
                   max_tokens=LONG)
    m.set_loops(K)
    say(f"[narrow3 bf16] {LONG}-token prefill in one chunk, all rows against the oracle")
    lg, ids = m.prefill(0, torch.from_numpy(prompt).to(m.device), LONG)
    g_h = m.last_hidden(LONG).cpu().numpy()
    o_lg, o_ids = om.lm_head(hidden)
    check_rows(f"{LONG} rows", lg.cpu().numpy(), ids.cpu().numpy(), o_lg, o_ids, g_h, hidden)
    m.close()


def test_16384_token_prefill_and_decode():
    """16384 positions in one chunk (128 flash row blocks per head; RoPE phases and
    full-attention keys out to 16K): every row's final hidden state and the last 256 rows' logits
    against the oracle's whole-prompt prefill, then 2 teacher-forced decode steps at that context
    on the split MFMA kernel (32 splits, both merge groups), k = 2, last-loop."""
    T = 16384
    w = synth.make_weights(NARROW3, seed=0)
    prompt = synth.prompt_tokens(NARROW3, T, seed=5)
    say(f"[narrow3 bf16] oracle: {T}-token prefill, k={K}, last-loop")
    om = OracleModel(NARROW3, w, "last_loop", K)
    o_lg, o_ids = om.prefill(0, prompt, 256)
    o_h = om.last_hidden.copy()
    m = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=K, max_seqs=1, max_model_len=T + 16, max_tokens=T)
    m.set_loops(K)
    lg, ids = m.prefill(0, torch.from_numpy(prompt).to(m.device), 256)
    g_h = m.last_hidden(T).cpu().numpy()
    check_rows(f"{T}-token prefill (hidden: all rows; logits: last 256)", lg.cpu().numpy(), ids.cpu().numpy(),
               o_lg, o_ids, g_h, o_h)
    tok = int(o_ids[-1])
    for step in range(2):
        l1, i1 = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        ol, oi = om.decode([0], [tok])
        check_rows(f"decode step {step} at {T + step + 1} keys", l1.cpu().numpy(), i1.cpu().numpy(), np.array(ol),
                   np.array(oi), m.last_hidden(1).cpu().numpy(), om.last_hidden)
        tok = int(oi[0])
    assert m.stats()["max_attn_splits"] == 32
    m.close()
