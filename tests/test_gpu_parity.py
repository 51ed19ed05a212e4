"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars (written in each test):
  * fp32 model: logits and final hidden states within 1e-4 max-abs; greedy ids bit-exact
    (free-running: the GPU feeds its own ids).
  * bf16 model: teacher-forced on the oracle's ids; logits within 5e-2 and final hidden
    states within 3e-2 max-abs; the GPU's argmax equals the oracle's except at steps whose
    oracle margin between the two ids is below twice the step's max logit error (near-ties,
    counted and reported).
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
from oracle import OracleModel, greedy  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tiny():
    w = synth.make_weights(synth.TINY, seed=0)
    gpu = dory.Model(synth.TINY, w, kv_mode="per_loop", max_loops=4, max_seqs=4, max_model_len=256, max_tokens=128)
    return w, gpu


def run_gpu_greedy(m, seq, prompt, n_steps, teacher=None):
    """Prefill + n_steps decode steps; feeds the GPU's own ids unless teacher ids are given."""
    lg, ids = m.prefill(seq, prompt, 1)
    logits = [lg[0].cpu().numpy()]
    out = [int(ids[0].item())]
    hidden = [m.last_hidden(1)[0].cpu().numpy()]
    for i in range(n_steps):
        tok = out[-1] if teacher is None else int(teacher[i])
        lg, ids = m.decode([seq], torch.tensor([tok], dtype=torch.int32, device=m.device))
        logits.append(lg[0].cpu().numpy())
        out.append(int(ids[0].item()))
        hidden.append(m.last_hidden(1)[0].cpu().numpy())
    return np.array(out, dtype=np.int32), np.array(logits), np.array(hidden)


def oracle_greedy(shape, w, mode, k, prompt, n_steps):
    om = OracleModel(shape, w, mode, k)
    lg, ids = om.prefill(0, prompt, 1)
    out, logits, hidden = [int(ids[0])], [lg[0]], [om.last_hidden[-1]]
    for _ in range(n_steps):
        lg, ids = om.decode([0], [out[-1]])
        out.append(int(ids[0]))
        logits.append(lg[0])
        hidden.append(om.last_hidden[0])
    return np.array(out, dtype=np.int32), np.array(logits), np.array(hidden)


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_tiny_fp32_end_to_end(tiny, mode, k):
    w, m = tiny
    say(f"[tiny fp32] mode={mode} k={k} prompt=64 decode=16")
    for s in range(4):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode(mode)
    m.set_loops(k)
    prompt = synth.prompt_tokens(synth.TINY, 64)
    g_ids, g_lg, g_h = run_gpu_greedy(m, 0, prompt, 16)
    o_ids, o_lg, o_h = oracle_greedy(synth.TINY, w, mode, k, prompt, 16)
    err_l = np.max(np.abs(g_lg - o_lg))
    err_h = np.max(np.abs(g_h - o_h))
    say(f"  logits max-abs {err_l:.3e}  hidden max-abs {err_h:.3e}  ids equal {np.array_equal(g_ids, o_ids)}")
    assert err_l <= 1e-4
    assert err_h <= 1e-4
    np.testing.assert_array_equal(g_ids, o_ids)


def test_tiny_fp32_all_rows_and_chunks(tiny):
    """Logits of every prompt row; a prompt in ragged chunks (per-loop: chunking invariant)."""
    w, m = tiny
    say("[tiny fp32] all-row logits, chunked per-loop prefill, k=2")
    for s in range(4):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode("per_loop")
    m.set_loops(2)
    prompt = synth.prompt_tokens(synth.TINY, 77)
    lg, ids = m.prefill(0, prompt, 77)
    om = OracleModel(synth.TINY, w, "per_loop", 2)
    olg, oids = om.prefill(0, prompt, 77)
    assert np.max(np.abs(lg.cpu().numpy() - olg)) <= 1e-4
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    outs = []
    for a, b in ((0, 1), (1, 18), (18, 50), (50, 77)):
        l2, _ = m.prefill(1, prompt[a:b], b - a)
        outs.append(l2.cpu().numpy())
    assert np.max(np.abs(np.concatenate(outs) - olg)) <= 1e-4


@pytest.fixture(scope="module")
def mid():
    w = synth.make_weights(synth.MID, seed=0)
    gpu = dory.Model(synth.MID, w, kv_mode="per_loop", max_loops=4, max_seqs=2, max_model_len=1280, max_tokens=1024)
    return w, gpu


def bf16_check(tag, g_ids, g_lg, g_h, o_ids, o_lg, o_h):
    err_l = np.max(np.abs(g_lg - o_lg))
    err_h = np.max(np.abs(g_h - o_h))
    rel_h = np.linalg.norm(g_h - o_h) / np.linalg.norm(o_h)
    near, wrong = 0, 0
    for i in range(len(g_ids)):
        if g_ids[i] == o_ids[i]:
            continue
        step_err = np.max(np.abs(g_lg[i] - o_lg[i]))
        margin = o_lg[i][o_ids[i]] - o_lg[i][g_ids[i]]
        if margin < 2 * step_err:
            near += 1
        else:
            wrong += 1
    say(f"  {tag}: logits max-abs {err_l:.3e}  hidden max-abs {err_h:.3e} rel-L2 {rel_h:.2e}  "
        f"ids {np.sum(g_ids == o_ids)}/{len(g_ids)} equal, near-ties {near}, wrong {wrong}")
    assert err_l <= 5e-2
    assert err_h <= 3e-2
    assert wrong == 0


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_mid_bf16_end_to_end(mid, mode, k):
    w, m = mid
    n_dec = 6
    say(f"[mid bf16] mode={mode} k={k} prompt=512 decode={n_dec} (teacher-forced)")
    for s in range(2):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode(mode)
    m.set_loops(k)
    prompt = synth.prompt_tokens(synth.MID, 512)
    o_ids, o_lg, o_h = oracle_greedy(synth.MID, w, mode, k, prompt, n_dec)
    g_ids, g_lg, g_h = run_gpu_greedy(m, 0, prompt, n_dec, teacher=o_ids)
    bf16_check(f"mid k={k} {mode}", g_ids, g_lg, g_h, o_ids, o_lg, o_h)


def test_mid_bf16_sliding_window_and_chunks(mid):
    """W = 1024 binds (1200-token prompt); per-loop prompt in ragged chunks through the
    short-chunk attention path (rows <= 16) and the flash path, checked against the oracle."""
    w, m = mid
    say("[mid bf16] window binds: 1200-token prompt, k=1, chunks 700 + 1 + 5 + 16 + 17 + 461")
    for s in range(2):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode("per_loop")
    m.set_loops(1)
    prompt = synth.prompt_tokens(synth.MID, 1200)
    om = OracleModel(synth.MID, w, "per_loop", 1)
    olg, oids = om.prefill(0, prompt, 1)
    bounds = [0, 700, 701, 706, 722, 739, 1200]
    for a, b in zip(bounds[:-1], bounds[1:]):
        l2, i2 = m.prefill(0, prompt[a:b], 1)
    err = float(np.max(np.abs(l2.cpu().numpy() - olg)))
    h = m.last_hidden(1)[0].cpu().numpy()
    err_h = float(np.max(np.abs(h - om.last_hidden[-1])))
    say(f"  chunked 1200-token prompt: logits max-abs {err:.3e}, hidden {err_h:.3e}, id {int(i2[0])} vs {int(oids[0])}")
    assert err <= 5e-2 and err_h <= 3e-2


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_tiny_fp32_self_speculative(tiny, mode):
    """dory_spec_decode (k=1 draft of 4, k=4 verify) against the oracle's driver, ids bit-exact;
    in per-loop mode both also equal plain k=4 greedy."""
    from oracle import self_speculative
    w, m = tiny
    say(f"[tiny fp32] self-speculative decoding, {mode}")
    for s in range(4):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode(mode)
    m.set_loops(4)
    prompt = synth.prompt_tokens(synth.TINY, 30)
    _, ids = m.prefill(0, prompt, 1)
    first = int(ids[0].item())
    got = m.spec_decode(0, first, 20, gamma=4, k_draft=1, k_verify=4)
    om = OracleModel(synth.TINY, w, mode, 4)
    want = self_speculative(om, 0, prompt, 21, gamma=4, k_draft=1, k_verify=4)
    say(f"  gpu {list(got[:20])}\n  oracle {list(want[1:21])}")
    assert first == int(want[0])
    np.testing.assert_array_equal(got[:20], want[1:21])
    assert m.loops() == 4
    if mode == "per_loop":
        ref = oracle_greedy(synth.TINY, w, mode, 4, prompt, 20)[0]
        np.testing.assert_array_equal(want[:21], ref[:21])


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_tiny_fp32_self_speculative_reuse(tiny, mode):
    """dory_spec_decode with reuse (the verify pass takes the k=1 draft's input-stack output,
    loop-1 state and cache) against the oracle's reuse driver, ids bit-exact; the same ids as
    without reuse."""
    from oracle import self_speculative_reuse
    w, m = tiny
    say(f"[tiny fp32] self-speculative decoding with reuse, {mode}")
    for s in range(4):
        if m.seq_len(s) >= 0:
            m.release(s)
    m.set_kv_mode(mode)
    m.set_loops(4)
    prompt = synth.prompt_tokens(synth.TINY, 30)
    _, ids = m.prefill(0, prompt, 1)
    first = int(ids[0].item())
    got = m.spec_decode(0, first, 20, gamma=4, k_draft=1, k_verify=4, reuse=True)
    m.release(0)
    _, ids = m.prefill(0, prompt, 1)
    plain = m.spec_decode(0, first, 20, gamma=4, k_draft=1, k_verify=4, reuse=False)
    om = OracleModel(synth.TINY, w, mode, 4)
    want = self_speculative_reuse(om, 0, prompt, 21, gamma=4, k_verify=4)
    say(f"  gpu {list(got[:20])}\n  oracle {list(want[1:21])}")
    np.testing.assert_array_equal(got[:20], want[1:21])
    np.testing.assert_array_equal(got[:20], plain[:20])
    with pytest.raises(dory.DoryError):
        m.spec_decode(0, int(plain[-1]), 4, gamma=4, k_draft=2, k_verify=4, reuse=True)


def test_mid_bf16_self_speculative_reuse_matches_plain():
    """bf16 mid model, last-loop KV: speculative decoding with and without reuse produce the same
    ids (the reused rows' states come from the decode kernels instead of the chunk kernels)."""
    w = synth.make_weights(synth.MID, seed=0)
    m = dory.Model(synth.MID, w, kv_mode="last_loop", max_loops=4, max_seqs=1, max_model_len=512, max_tokens=256)
    m.set_loops(4)
    prompt = synth.prompt_tokens(synth.MID, 200)
    out = []
    for reuse in (False, True):
        _, ids = m.prefill(0, prompt, 1)
        out.append(m.spec_decode(0, int(ids[0].item()), 24, gamma=4, k_draft=1, k_verify=4, reuse=reuse)[:24])
        m.release(0)
    agree = int(np.argmin(np.append(out[0] == out[1], False)))
    say(f"[mid bf16] self-speculative with / without reuse: first {agree} of 24 ids agree")
    np.testing.assert_array_equal(out[0], out[1])


# bf16 with 128-wide heads (the batched split-attention kernels need them) but narrow and
# shallow, so the oracle runs 20 sequences of ~300 tokens in seconds; the window sits
# inside the prompts
NARROW = dataclasses.replace(synth.MID, d_model=256, n_heads=2, n_kv_heads=1, d_ff=512, vocab=2048, n_in=2, n_rec=4,
                             n_out=2, window=192)
# attention scale above the fixed-offset limit (40): the running-maximum prefill and batched
# decode kernels
NARROW60 = dataclasses.replace(NARROW, attn_scale=60.0)


@pytest.mark.parametrize("shape_name,mode,n_seq,min_len,max_len",
                         [("mid", "per_loop", 6, 17, 300), ("mid", "last_loop", 6, 17, 300),
                          ("narrow", "last_loop", 20, 257, 360), ("narrow", "per_loop", 20, 257, 360),
                          ("narrow60", "last_loop", 20, 257, 360), ("narrow", "last_loop", 100, 17, 60)])
def test_bf16_batched_decode(shape_name, mode, n_seq, min_len, max_len):
    """Serving-style batched decode: sequences with ragged prompt lengths decode together
    (one call per step, rows = sequences); every sequence against its own oracle run,
    teacher-forced. Exercises the split-K small-M GEMM and multi-row split attention (the
    MFMA kernel up to 16 rows, the VALU kernel above; prompts over 256 tokens give it two
    key splits per row); 100 rows take the 64..128-row projection tiles (gate/up unsplit with
    the SwiGLU epilogue, o split-K) with a ragged last row tile."""
    shape = {"mid": synth.MID, "narrow": NARROW, "narrow60": NARROW60}[shape_name]
    w = synth.make_weights(shape, seed=0)
    m = dory.Model(shape, w, kv_mode=mode, max_loops=2, max_seqs=n_seq, max_model_len=512, max_tokens=512)
    m.set_loops(2)
    lens = synth.batch_prompt_lengths(n_seq, min_len, max_len, seed=2)
    prompts = synth.batch_prompts(shape, lens, seed=1)
    say(f"[{shape_name} bf16] batched decode, {mode}, k=2, {n_seq} sequences, prompt lengths {list(lens)}")
    n_dec = 3
    o_all = [oracle_greedy(shape, w, mode, 2, p, n_dec) for p in prompts]
    first = []
    for s, p in enumerate(prompts):
        lg, ids = m.prefill(s, p, 1)
        first.append((lg[0].cpu().numpy(), int(ids[0].item())))
    g_lg = [[f[0]] for f in first]
    g_ids = [[f[1]] for f in first]
    for step in range(n_dec):
        toks = torch.tensor([int(o_all[s][0][step]) for s in range(n_seq)], dtype=torch.int32, device=m.device)
        lg, ids = m.decode(list(range(n_seq)), toks)
        lg = lg.cpu().numpy()
        ids = ids.cpu().numpy()
        for s in range(n_seq):
            g_lg[s].append(lg[s])
            g_ids[s].append(int(ids[s]))
    for s in range(n_seq):
        o_ids, o_lg, _ = o_all[s]
        err = float(np.max(np.abs(np.array(g_lg[s]) - o_lg)))
        agree = int(np.sum(np.array(g_ids[s]) == o_ids))
        say(f"  seq {s} (len {lens[s]}): logits max-abs {err:.2e}, ids {agree}/{len(o_ids)}")
        assert err <= 5e-2
        for i in range(len(o_ids)):
            if g_ids[s][i] != o_ids[i]:
                margin = o_lg[i][o_ids[i]] - o_lg[i][g_ids[s][i]]
                assert margin < 2 * np.max(np.abs(g_lg[s][i] - o_lg[i]))
    m.close()


def test_out_of_range_token_raises_device_flag(tiny):
    """A token id outside 0..V-1 is clamped by the embedding and reported through dory_device_flags."""
    _, m = tiny
    say("[tiny fp32] out-of-range token -> device flag bit 0")
    for s in range(4):
        if m.seq_len(s) >= 0:
            m.release(s)
    assert m.device_flags() == 0
    m.prefill(0, [3, synth.TINY.vocab + 5, 7], 1)
    assert m.device_flags() == 1
    assert m.device_flags() == 0      # the previous call reset it
    m.prefill(1, [3, 4, 5], 1)
    assert m.device_flags() == 0
    m.release(0)
    m.release(1)
