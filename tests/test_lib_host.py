"""Host-side checks of libdory.so that need no GPU.

The library is loaded and every symbol its header declares is looked up; the
scheduler and KV manager run in dry-run contexts (no HIP call is made) so the
layer-application counts, cache-slot counts, page accounting and every error
path of the boundary can be forced on the CPU.
"""
import os
import re

import pytest

from looped_ngpt_language_amd import dory, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STACKS = synth.ModelShape(d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, d_ff=256, vocab=512,
                          n_in=8, n_rec=20, n_out=8, window=16, dtype=synth.BF16)


def header_functions():
    text = open(os.path.join(ROOT, "include", "dory.h")).read()
    return sorted(set(re.findall(r"\b(dory_[a-z_0-9]+)\s*\(", text)))


@pytest.mark.parametrize("checked", [False, True])
def test_library_exports_every_declared_function(checked):
    lib = dory.lib(checked)
    names = header_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    assert set(dory.EXPORTS) == set(names)
    assert lib.dory_checked_build() == (1 if checked else 0)


@pytest.mark.parametrize("checked", [False, True])
def test_debug_page_poke_refused_outside_a_checked_gpu_context(checked):
    # the default build never writes the device page table on request; a dry-run context has none
    m = dry(checked=checked)
    with pytest.raises(dory.DoryError) as e:
        m.debug_set_page(0, 0, 1)
    assert e.value.status == dory.DORY_E_STATE
    m.close()


def dry(shape=synth.TINY, mode="per_loop", **kw):
    kw.setdefault("max_model_len", 256)
    kw.setdefault("max_seqs", 4)
    return dory.Model(shape, kv_mode=mode, dry_run=True, **kw)


@pytest.mark.parametrize("k,blocks,full,swa", [(1, 36, 9, 27), (2, 56, 14, 42), (4, 96, 24, 72)])
def test_scheduler_application_counts(k, blocks, full, swa):
    m = dry(STACKS)
    m.set_loops(k)
    m.prefill(0, [1, 2, 3], 1)
    st = m.stats()
    assert st["block_apps"] == blocks
    assert st["sublayer_apps"] == 2 * blocks
    assert (st["full_apps"], st["swa_apps"]) == (full, swa)
    m.decode([0], [4])
    assert m.stats()["block_apps"] == 2 * blocks


@pytest.mark.parametrize("mode,max_loops,slots", [("per_loop", 1, 36), ("per_loop", 2, 56), ("per_loop", 4, 96),
                                                  ("last_loop", 1, 36), ("last_loop", 4, 36)])
def test_slot_counts_and_kv_bytes(mode, max_loops, slots):
    m = dry(STACKS, mode, max_loops=max_loops)
    assert m.stats()["n_slots"] == slots
    m.set_loops(max_loops)
    m.prefill(0, list(range(40)), 1)          # 40 tokens -> 3 pages
    st = m.stats()
    assert st["pages_in_use"] == 3
    page_slot_bytes = 2 * STACKS.n_kv_heads * 16 * STACKS.head_dim * 2
    assert m.kv_bytes_in_use() == 3 * slots * page_slot_bytes


def test_last_loop_kv_is_k_independent_and_per_loop_grows():
    sizes = {}
    for mode in ("per_loop", "last_loop"):
        for k in (1, 2, 4):
            m = dry(STACKS, mode, max_loops=k)
            m.set_loops(k)
            m.prefill(0, list(range(100)), 1)
            sizes[mode, k] = m.kv_bytes_in_use()
    assert sizes["last_loop", 1] == sizes["last_loop", 2] == sizes["last_loop", 4] == sizes["per_loop", 1]
    assert sizes["per_loop", 2] * 36 == sizes["last_loop", 2] * 56
    assert sizes["per_loop", 4] * 36 == sizes["last_loop", 4] * 96


def test_pages_follow_length_truncate_release():
    m = dry(max_model_len=200, max_seqs=3)
    m.prefill(1, list(range(17)), 1)
    assert m.stats()["pages_in_use"] == 2
    for t in range(15):
        m.decode([1], [t])
    assert m.seq_len(1) == 32 and m.stats()["pages_in_use"] == 2
    m.decode([1], [0])
    assert m.stats()["pages_in_use"] == 3
    m.truncate(1, 16)
    assert m.seq_len(1) == 16 and m.stats()["pages_in_use"] == 1
    m.truncate(1, 0)
    assert m.stats()["pages_in_use"] == 0 and m.seq_len(1) == 0
    m.release(1)
    assert m.seq_len(1) == -1 and m.stats()["live_seqs"] == 0


def status_of(fn, *a):
    with pytest.raises(dory.DoryError) as e:
        fn(*a)
    return e.value.status


def test_error_paths():
    m = dry(max_model_len=64, max_seqs=2, max_tokens=40)
    assert status_of(m.set_loops, 0) == dory.DORY_E_INVALID
    assert status_of(m.set_loops, 5) == dory.DORY_E_INVALID
    assert status_of(m.prefill, 2, [1], 1) == dory.DORY_E_INVALID            # seq id out of range
    assert status_of(m.prefill, 0, [1] * 41, 1) == dory.DORY_E_INVALID       # chunk > max_tokens
    assert status_of(m.prefill, 0, [1, 2], 3) == dory.DORY_E_INVALID         # logits_rows > n
    assert status_of(m.decode, [0], [1]) == dory.DORY_E_INVALID              # not live
    m.set_loops(2)
    m.prefill(0, [1] * 40, 1)
    assert status_of(m.prefill, 0, [1] * 25, 1) == dory.DORY_E_INVALID       # 65 > max_model_len
    assert status_of(m.set_kv_mode, "last_loop") == dory.DORY_E_STATE       # live sequence
    m.set_loops(4)
    assert status_of(m.decode, [0], [1]) == dory.DORY_E_STATE                # per-loop cache holds 2 loops
    m.set_loops(1)
    m.decode([0], [1])
    m.set_loops(2)
    assert status_of(m.decode, [0], [1]) == dory.DORY_E_STATE                # newest position has 1 loop
    m.truncate(0, 40)
    m.decode([0], [1])                                                        # truncation restored 2 loops
    m.prefill(1, [1], 1)
    assert status_of(m.decode, [0, 0], [1, 1]) == dory.DORY_E_INVALID        # listed twice
    assert status_of(m.truncate, 0, 100) == dory.DORY_E_INVALID
    assert status_of(m.release, 3) == dory.DORY_E_INVALID
    m.release(0)
    m.release(1)
    m.set_kv_mode("last_loop")
    m.set_loops(4)
    m.prefill(0, [1] * 10, 1)
    m.set_loops(1)
    m.decode([0], [2])
    m.set_loops(4)
    m.decode([0], [2])                                                        # last-loop: any loop count


def test_pool_exhaustion_is_detected_before_any_state_change():
    m = dry(max_model_len=256, max_seqs=4, kv_tokens=64)                      # 4 pages
    m.prefill(0, [1] * 48, 1)
    assert status_of(m.prefill, 1, [1] * 20, 1) == dory.DORY_E_NOMEM
    assert m.seq_len(1) == -1 and m.stats()["pages_in_use"] == 3
    m.prefill(1, [1] * 16, 1)
    assert status_of(m.decode, [0, 1], [1, 1]) == dory.DORY_E_NOMEM
    assert m.seq_len(0) == 48 and m.seq_len(1) == 16


def test_config_validation():
    bad = [synth.TINY.replace(head_dim=48), synth.TINY.replace(n_kv_heads=3),
           synth.TINY.replace(page_size=32), STACKS.replace(d_model=100)]
    for shape in bad:
        cfg = dory.make_config(shape, dry_run=True)
        with pytest.raises(dory.DoryError):
            dory.query_sizes(cfg, "per_loop", 64)
    cfg = dory.make_config(synth.TINY, max_loops=5, dry_run=True)
    with pytest.raises(dory.DoryError):
        dory.query_sizes(cfg, "per_loop", 64)


def test_mxfp8_flag_sizes_and_validation():
    """The MXFP8 flag adds ~1.03 bytes per weight to the workspace and is refused for fp32
    models and for widths the weight-streaming GEMV does not cover."""
    base = dory.make_config(synth.MID, dry_run=True)
    mx = dory.make_config(synth.MID, dry_run=True, gemv_weights="mxfp8")
    _, ws0 = dory.query_sizes(base, "per_loop", 4096)
    _, ws1 = dory.query_sizes(mx, "per_loop", 4096)
    s = synth.MID
    params = s.n_blocks * ((s.n_heads + 2 * s.n_kv_heads) * s.head_dim * s.d_model + s.d_model * s.n_heads * s.head_dim
                           + 3 * s.d_ff * s.d_model) + s.vocab * s.d_model
    assert params * 33 // 32 <= ws1 - ws0 <= params * 33 // 32 + (1 << 20)
    with pytest.raises(dory.DoryError):
        dory.query_sizes(dory.make_config(synth.TINY, dry_run=True, gemv_weights="mxfp8"), "per_loop", 64)
    with pytest.raises(dory.DoryError):
        dory.query_sizes(dory.make_config(STACKS, dry_run=True, gemv_weights="mxfp8"), "per_loop", 64)


def test_mxfp4_flag_sizes_and_validation():
    """The MXFP4 flag adds ~0.53 bytes per weight (two codes per byte plus a scale per 32) and
    cannot be combined with the MXFP8 flag."""
    base = dory.make_config(synth.MID, dry_run=True)
    mx4 = dory.make_config(synth.MID, dry_run=True, gemv_weights="mxfp4")
    _, ws0 = dory.query_sizes(base, "per_loop", 4096)
    _, ws1 = dory.query_sizes(mx4, "per_loop", 4096)
    s = synth.MID
    params = s.n_blocks * ((s.n_heads + 2 * s.n_kv_heads) * s.head_dim * s.d_model + s.d_model * s.n_heads * s.head_dim
                           + 3 * s.d_ff * s.d_model) + s.vocab * s.d_model
    assert params * 17 // 32 <= ws1 - ws0 <= params * 17 // 32 + (1 << 20)
    both = dory.make_config(synth.MID, dry_run=True, gemv_weights="mxfp4")
    both.flags |= dory.FLAG_MXFP8_GEMV
    with pytest.raises(dory.DoryError):
        dory.query_sizes(both, "per_loop", 64)
    with pytest.raises(dory.DoryError):
        dory.query_sizes(dory.make_config(synth.TINY, dry_run=True, gemv_weights="mxfp4"), "per_loop", 64)


def test_quantize_mxfp4_argument_errors():
    lib = dory.lib()
    assert lib.dory_quantize_mxfp4(None, 4, 30, None, None, None) == dory.DORY_E_INVALID   # cols % 32
    assert lib.dory_quantize_mxfp4(None, -1, 32, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_quantize_mxfp4(None, 4, 32, None, None, None) == dory.DORY_E_INVALID    # NULL buffers
    assert lib.dory_quantize_mxfp4(None, 0, 32, None, None, None) == dory.DORY_OK          # nothing to do


def test_quantize_mxfp8_argument_errors():
    lib = dory.lib()
    assert lib.dory_quantize_mxfp8(None, 4, 30, None, None, None) == dory.DORY_E_INVALID   # cols % 32
    assert lib.dory_quantize_mxfp8(None, -1, 32, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_quantize_mxfp8(None, 4, 32, None, None, None) == dory.DORY_E_INVALID    # NULL buffers
    assert lib.dory_quantize_mxfp8(None, 0, 32, None, None, None) == dory.DORY_OK          # nothing to do


def test_sample_argument_errors():
    lib = dory.lib()
    nan = float("nan")
    assert lib.dory_sample(None, -1, 100, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_sample(None, 1, 0, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID          # vocab < 1
    assert lib.dory_sample(None, 1, (1 << 23) + 1, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_sample(None, 2, 100, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID         # NULL buffers
    assert lib.dory_sample(None, 0, 100, nan, 0.95, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_sample(None, 0, 100, 1.0, nan, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_sample(None, 0, 100, 1.0, 0.95, None, None, None) == dory.DORY_OK               # nothing to do
    inf = float("inf")
    assert lib.dory_sample(None, 0, 100, inf, 0.95, None, None, None) == dory.DORY_E_INVALID
    assert lib.dory_sample(None, 0, 100, -inf, 0.95, None, None, None) == dory.DORY_E_INVALID
    for fn in (lib.dory_sample_static,):
        assert fn(None, -1, 100, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID
        assert fn(None, 2, 100, 1.0, 0.95, None, None, None) == dory.DORY_E_INVALID      # NULL buffers
        assert fn(None, 0, 100, inf, 0.95, None, None, None) == dory.DORY_E_INVALID
        assert fn(None, 0, 100, 1.0, nan, None, None, None) == dory.DORY_E_INVALID
        assert fn(None, 0, 100, 1.0, 0.95, None, None, None) == dory.DORY_OK


def test_sample_scratch_sizes():
    """Scratch per call: about 8.3 KB per row plus the chunk partials; every call of at most 256
    rows fits the static 4 MiB array, and a larger one that does not is refused before any GPU work
    (the NULL buffers would otherwise be the error)."""
    lib = dory.lib()
    assert lib.dory_sample_scratch_bytes(0, 100) == 0
    assert lib.dory_sample_scratch_bytes(1, 0) == 0
    one = lib.dory_sample_scratch_bytes(1, 131072)
    assert 8256 <= one <= 16384
    for rows in (1, 7, 128, 256):
        for v in (1, 1000, 131072, 1 << 23):
            assert lib.dory_sample_scratch_bytes(rows, v) <= 4 << 20
    big = 1024
    assert lib.dory_sample_scratch_bytes(big, 131072) > 4 << 20
    dummy = 256   # non-NULL pointers: the size check must refuse before anything is launched
    assert lib.dory_sample_static(dummy, big, 131072, 1.0, 0.95, dummy, dummy, None) == dory.DORY_E_INVALID


def test_swa_recycling_pool_size_4b_long_context():
    # 131072 + 512 tokens, last-loop KV: the 9 full-attention slots keep every page, the 27
    # sliding-window slots only what one sequence's window, reserve and chunk reach
    s = synth.DORY4B
    kw = dict(max_seqs=1, max_model_len=131072 + 512 + 16, max_tokens=4096, dry_run=True)
    tokens = 131072 + 512
    b0, _ = dory.query_sizes(dory.make_config(s, **kw), "last_loop", tokens)
    b1, _ = dory.query_sizes(dory.make_config(s, swa_recycle=True, **kw), "last_loop", tokens)
    pb = 2 * s.n_kv_heads * 16 * s.head_dim * 2
    pages = -(-tokens // 16)
    assert b0 == pages * 36 * pb                                     # ~19.4 GB
    assert b1 == (pages * 9 + ((4096 + 64 + 4096) // 16 + 3) * 27) * pb
    # the pool also holds one 4096-token chunk of window pages: ~5.8 GB allocated, ~5.3 GB in use
    # while decoding (full pages + window and reserve)
    assert 19.0e9 < b0 < 19.6e9 and 5.5e9 < b1 < 5.9e9


def test_swa_recycling_page_accounting():
    s = synth.TINY                      # window 16; blocks 3 and 7 full: last-loop 2 full + 6 window slots
    m = dry(s, mode="last_loop", max_model_len=1024, max_tokens=32, max_seqs=2, swa_recycle=True)
    pb = 2 * s.n_kv_heads * 16 * s.head_dim * 4
    m.prefill(0, list(range(32)), 1)
    before = 32
    for _ in range(300):
        m.decode([0], [1])
        before += 1
    length = before
    st = m.stats()
    assert st["pages_in_use"] == -(-length // 16)
    # held window pages: logical pages from (len_before_last_call - 16 + 1 - 64) // 16 to the end
    lo = max(0, (length - 1) - 16 + 1 - 64) // 16
    assert st["swa_pages_in_use"] == -(-length // 16) - lo
    assert m.kv_bytes_in_use() == (st["pages_in_use"] * 2 + st["swa_pages_in_use"] * 6) * pb
    m.truncate(0, length - 10)                       # inside the reserve
    with pytest.raises(dory.DoryError) as e:
        m.truncate(0, length - 200)                  # its window pages are gone
    assert e.value.status == dory.DORY_E_STATE
    assert m.seq_len(0) == length - 10
    # a second sequence reuses recycled window pages
    m.prefill(1, list(range(32)), 1)
    st2 = m.stats()
    assert st2["swa_pages_in_use"] == (-(-(length - 10) // 16) - lo) + 2   # truncated seq 0, plus 2 pages of seq 1
    m.release(0)
    m.release(1)
    st3 = m.stats()
    assert st3["pages_in_use"] == 0 and st3["swa_pages_in_use"] == 0


def test_swa_recycling_off_keeps_every_slot_page():
    s = synth.TINY
    m = dry(s, mode="last_loop", max_model_len=1024, max_tokens=32, max_seqs=2)
    m.prefill(0, list(range(32)), 1)
    for _ in range(300):
        m.decode([0], [1])
    st = m.stats()
    assert st["swa_pages_total"] == 0 and st["swa_pages_in_use"] == 0
    assert m.kv_bytes_in_use() == st["pages_in_use"] * 8 * (2 * s.n_kv_heads * 16 * s.head_dim * 4)


def test_batched_decode_upload_fits():
    """One decode call for 128 sequences uploads their (seq, pos) rows, the page-table updates of
    both tables (every sequence at a page boundary, sliding-window recycling on) and the rows'
    longest-first order: all of it fits the upload area sized at create."""
    s = synth.TINY
    n = 128
    m = dry(s, mode="last_loop", max_model_len=256, max_tokens=n, max_seqs=n, swa_recycle=True)
    for q in range(n):
        m.prefill(q, list(range(16 * (1 + q % 5))), 1)     # whole pages: the decode opens a new one
    m.decode(list(range(n)), [1] * n)
    assert all(m.seq_len(q) == 16 * (1 + q % 5) + 1 for q in range(n))
    assert m.stats()["pages_in_use"] == sum(1 + q % 5 + 1 for q in range(n))


def test_decode_step_launch_count_at_4b_shapes():
    """Launches of one batch-1 decode step at the ~4B shapes (2560-token context, 21 key splits),
    counted by the library in a dry run: six per block application (qkv GEMV with the pending
    residual step in its prologue, attention, split merge, o GEMV, gate/up GEMV with the
    residual prologue, down GEMV), so each recurrent loop adds 20 x 6 block launches plus one
    loop-boundary launch; the rest of the step (embedding, entering the core, final step, LM head,
    argmax) is the same at every k."""
    counts = {}
    for k in (1, 2, 4):
        m = dory.Model(synth.DORY4B, kv_mode="last_loop", dry_run=True, max_model_len=2700, max_seqs=1,
                       max_tokens=2560, max_loops=4)
        m.set_loops(k)
        m.prefill(0, list(range(2560)), 1)
        before = m.stats()["kernel_launches"]
        m.decode([0], [5])
        st = m.stats()
        counts[k] = st["kernel_launches"] - before
        assert st["max_attn_splits"] == 21
        m.close()
    assert counts[2] - counts[1] == 20 * 6 + 1
    assert counts[4] - counts[2] == 2 * (20 * 6 + 1)
    assert counts[1] == 16 * 6 + 20 * 6 + 4
