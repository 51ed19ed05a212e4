"""The bounds-checked debug build (libdory_checked.so).

On valid state its guards only read, so it computes bitwise what the default build computes and
raises no device flag: checked on the tiny fp32 model (row attention kernel, per-row RoPE/KV
write), and on a narrow bf16 model with three query heads per KV head (flash prefill, page-tiled
RoPE, bs1 split MFMA decode, a 5-row chunk on the multi-row decode kernel, a 20-row batched decode
on the fixed-offset VALU kernel). A page id one past the cache region, written into the device
page table from the host, is caught (flag bit 2) and clamped to page 0, so no access leaves the
pool; once the entry is restored and the affected step truncated away, the context decodes
exactly as the default build again."""
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
FLAG_PAGE_ID = 4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_single(shape, w, checked):
    m = dory.Model(shape, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=1400, max_tokens=1200,
                   checked=checked)
    m.set_loops(2)
    out = []
    lg, tok = m.prefill(0, synth.prompt_tokens(shape, 300), 1)
    out.append(lg.cpu().numpy())
    for _ in range(3):
        lg, tok = m.decode([0], tok)
        out.append(lg.cpu().numpy())
    lg, _ = m.prefill(0, synth.prompt_tokens(shape, 5, seed=9), 5)
    out.append(lg.cpu().numpy())
    flags = m.device_flags()
    m.close()
    return out, flags


def run_batched(shape, w, checked):
    n = 20
    lens = synth.batch_prompt_lengths(n, 40, 600, seed=3)
    prompts = synth.batch_prompts(shape, lens, seed=4)
    m = dory.Model(shape, w, kv_mode="per_loop", max_loops=2, max_seqs=n, max_model_len=700, max_tokens=600,
                   checked=checked)
    m.set_loops(2)
    tok = torch.cat([m.prefill(s, p, 1)[1] for s, p in enumerate(prompts)])
    out = []
    for _ in range(2):
        lg, tok = m.decode(list(range(n)), tok)
        out.append(lg.cpu().numpy())
    flags = m.device_flags()
    m.close()
    return out, flags


@pytest.mark.parametrize("which", ["tiny_fp32", "narrow3_bf16"])
def test_checked_build_equals_default_on_valid_state(which):
    shape = synth.TINY if which == "tiny_fp32" else NARROW3
    w = synth.make_weights(shape, seed=0)
    say(f"[checked] {which}: single-sequence prefill / decode / chunk, default then checked build")
    a, fa = run_single(shape, w, False)
    b, fb = run_single(shape, w, True)
    same = all(np.array_equal(x, y) for x, y in zip(a, b))
    say(f"[checked] {which}: bitwise equal {same}, flags {fa} / {fb}")
    assert same and fa == 0 and fb == 0
    if which == "narrow3_bf16":
        say("[checked] narrow3: 20-row batched decode, default then checked build")
        a, fa = run_batched(shape, w, False)
        b, fb = run_batched(shape, w, True)
        same = all(np.array_equal(x, y) for x, y in zip(a, b))
        say(f"[checked] narrow3 batched: bitwise equal {same}, flags {fa} / {fb}")
        assert same and fa == 0 and fb == 0


def test_checked_build_catches_a_page_id_outside_the_pool():
    w = synth.make_weights(NARROW3, seed=0)
    prompt = synth.prompt_tokens(NARROW3, 40)          # pages 0..2 of 16 tokens
    ref = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=256, max_tokens=64)
    m = dory.Model(NARROW3, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=256, max_tokens=64,
                   checked=True)
    for x in (ref, m):
        x.set_loops(2)
    _, tok_ref = ref.prefill(0, prompt, 1)
    _, tok = m.prefill(0, prompt, 1)
    assert m.device_flags() == 0
    bad = m.stats()["pages_total"]                       # one past the last page of each slot's region
    say(f"[checked] injecting page id {bad} at page index 1 of sequence 0")
    old = m.debug_set_page(0, 1, bad)
    assert 0 <= old < bad
    m.decode([0], tok)
    flags = m.device_flags()
    say(f"[checked] flags after the decode step: {flags}")
    assert flags == FLAG_PAGE_ID
    assert m.debug_set_page(0, 1, old) == bad
    m.truncate(0, 40)                                    # drop the step that read the clamped page
    lg_ref, _ = ref.decode([0], tok_ref)
    lg, _ = m.decode([0], tok)
    assert m.device_flags() == 0
    assert np.array_equal(lg.cpu().numpy(), lg_ref.cpu().numpy())
    ref.close()
    m.close()
