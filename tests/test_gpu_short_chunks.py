"""Short prefill chunks whose keys / values the MFMA decode-attention kernel writes itself (at
most min(16, 32 / G) consecutive positions, G query heads per KV head, all in one workgroup per
key split), against the oracle fed the same chunks. Last-loop KV (every loop overwrites the
chunk's positions before its queries read them) and per-loop KV; G = 1..4 on a 5-block bf16
model (d = 512, two KV heads of 128, window 256; blocks 0-2 and 4 sliding-window, block 3 full)
so that the oracle runs past 900 positions in seconds.

The schedule after an 860-token prompt has chunks that straddle a page boundary, and one
(positions 895..902) whose two pages fall in different key splits of the full-attention layer
under the runtime's split rule (min(ceil(2048 / (rows * H_kv)), ceil(keys / 128), 32) splits of
ceil(pages / splits) pages: 8 splits of 8 pages at 903 keys), so two workgroups each write
their share of the chunk. Two decode steps follow. Bars: logits 5e-2, hidden rows 3e-2 max-abs;
ids equal except near-ties."""
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

PROMPT = 860
SCHEDULE = [3, 5, 8, 2, 7, 4, 6, 8, 5, 3, 8]   # 860..918; 895..902 crosses a split boundary
WINDOW = 256


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def shape_for(G: int) -> synth.ModelShape:
    return synth.ModelShape(d_model=512, n_heads=2 * G, n_kv_heads=2, head_dim=128, d_ff=1024, vocab=4096,
                            n_in=1, n_rec=3, n_out=1, window=WINDOW, dtype=synth.BF16)


def split_crossings(n_kv: int):
    """Chunks of the schedule whose first and last page fall in different key splits of the
    full-attention layer (the runtime's rule for the MFMA decode kernel)."""
    out, p = [], PROMPT
    for n in SCHEDULE:
        keys = p + n
        s = max(1, min(-(-2048 // (n * n_kv)), -(-keys // 128), 32))
        pl = (p + n - 1) >> 4
        pps = -(-(pl + 1) // s)
        if (p >> 4) // pps != pl // pps:
            out.append((p, n))
        p += n
    return out


def near_ok(g_ids, o_ids, g_lg, o_lg):
    for i in range(len(o_ids)):
        if g_ids[i] != o_ids[i]:
            assert o_lg[i][o_ids[i]] - o_lg[i][g_ids[i]] < 2 * np.max(np.abs(g_lg[i] - o_lg[i])), i


def test_schedule_crosses_a_split_boundary():
    assert split_crossings(2) == [(895, 8)]


@pytest.mark.parametrize("kv_mode", ["last_loop", "per_loop"])
@pytest.mark.parametrize("G", [1, 2, 3, 4])
def test_short_chunks_write_their_own_keys(G, kv_mode):
    shape = shape_for(G)
    assert max(SCHEDULE) <= min(16, 32 // G)   # every chunk takes the kernel's own KV write
    w = synth.make_weights(shape, seed=G)
    total = PROMPT + sum(SCHEDULE)
    m = dory.Model(shape, w, kv_mode=kv_mode, max_loops=3, max_seqs=1, max_model_len=total + 8,
                   max_tokens=PROMPT)
    m.set_loops(3)
    om = OracleModel(shape, w, kv_mode, 3)
    prompt = synth.prompt_tokens(shape, total, seed=30 + G)
    say(f"[G={G} {kv_mode}] prompt of {PROMPT}, then chunks {SCHEDULE}, k=3")
    m.prefill(0, torch.from_numpy(prompt[:PROMPT]).to(m.device), 1)
    om.prefill(0, prompt[:PROMPT], 1)
    p = PROMPT
    for n in SCHEDULE:
        lg, ids = m.prefill(0, torch.from_numpy(prompt[p:p + n]).to(m.device), n)
        g_h = m.last_hidden(n).cpu().numpy()
        olg, oids = om.prefill(0, prompt[p:p + n], n)
        g_lg, g_ids = lg.cpu().numpy(), ids.cpu().numpy()
        err = float(np.max(np.abs(g_lg - olg)))
        err_h = float(np.max(np.abs(g_h - om.last_hidden)))
        say(f"  chunk {p}..{p + n - 1}: logits max-abs {err:.2e}, hidden {err_h:.2e}, "
            f"ids {int(np.sum(g_ids == oids))}/{n}")
        assert err <= 5e-2 and err_h <= 3e-2
        near_ok(g_ids, oids, g_lg, olg)
        p += n
    tok = int(oids[-1])
    for step in range(2):
        lg, ids = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        olg, oids = om.decode([0], [tok])
        err = float(np.max(np.abs(lg.cpu().numpy() - olg)))
        say(f"  decode step {step}: logits max-abs {err:.2e}")
        assert err <= 5e-2
        near_ok(ids.cpu().numpy(), oids, lg.cpu().numpy(), olg)
        tok = int(oids[0])
    m.release(0)
