"""GPU parity of the temperature / top-p sampler (dory_sample) against the oracle's sampler on
the same fp32 logits and uniforms: ids equal, except where a near-tie makes both answers
correct (then the device id must be the oracle's for u or top_p moved by 1e-6)."""
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
from oracle.sampling import sample_row  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def near_tie_ok(l, t, p, u, gid):
    for dp in (-1e-6, 0.0, 1e-6):
        for du in (-1e-6, 0.0, 1e-6):
            if sample_row(l, t, min(max(p + dp, 0.0), 1.0), min(max(u + du, 0.0), 1 - 1e-12)) == gid:
                return True
    return False


def logits_of(kind, rows, v, rng):
    if kind == "normal":
        return rng.standard_normal((rows, v)).astype(np.float32)
    if kind == "peaked":
        return (rng.standard_normal((rows, v)) * 8).astype(np.float32)
    if kind == "zipf":
        out = np.empty((rows, v), np.float32)
        for r in range(rows):
            out[r] = -1.2 * np.log(rng.permutation(v) + 1.0)
        return out
    if kind == "ties":
        return rng.integers(-3, 4, (rows, v)).astype(np.float32)
    if kind == "masked":
        x = rng.standard_normal((rows, v)).astype(np.float32)
        x[rng.random((rows, v)) < 0.3] = -np.inf
        return x
    if kind == "equal":
        return np.full((rows, v), 0.5, np.float32)
    raise ValueError(kind)


def run(logits, us, t, p):
    g = dory.sample(torch.from_numpy(logits).to("cuda:0"), torch.from_numpy(us.astype(np.float32)).to("cuda:0"),
                    temperature=t, top_p=p)
    torch.cuda.synchronize()
    return g.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("v", [1024, 32768, 131072])
@pytest.mark.parametrize("kind", ["normal", "peaked", "zipf", "ties", "masked", "equal"])
def test_sampler_matches_oracle(v, kind):
    rng = np.random.default_rng(v + 7 * ["normal", "peaked", "zipf", "ties", "masked", "equal"].index(kind))
    rows = 4
    l = logits_of(kind, rows, v, rng)
    settings = [(1.0, 0.95), (0.7, 0.5), (1.3, 1.0), (1.0, 0.0), (0.0, 0.95)]
    exact = near = 0
    for t, p in settings:
        us = rng.random(rows).astype(np.float32)
        gid = run(l, us, t, p)
        for r in range(rows):
            oid = sample_row(l[r].astype(np.float64), t, p, float(us[r]))
            if gid[r] == oid:
                exact += 1
            else:
                assert near_tie_ok(l[r].astype(np.float64), t, p, float(us[r]), gid[r]), (t, p, r, gid[r], oid)
                near += 1
    say(f"[sample] V={v} {kind}: {exact} equal, {near} near-tie of {exact + near}")
    assert near <= 1


def test_stratified_draws_follow_the_nucleus():
    # one row of logits repeated with u_k = (k + 1/2) / n: the device ids reproduce the oracle's draw
    # for every k, so their counts are the renormalised nucleus masses within one draw
    rng = np.random.default_rng(5)
    v, n = 48, 4096
    row = (rng.standard_normal(v) * 1.5).astype(np.float32)
    l = np.repeat(row[None, :], n, axis=0)
    us = ((np.arange(n) + 0.5) / n).astype(np.float32)
    for t, p in [(1.0, 0.95), (0.8, 0.6)]:
        gid = run(l, us, t, p)
        oid = np.array([sample_row(row.astype(np.float64), t, p, float(u)) for u in us])
        mism = np.nonzero(gid != oid)[0]
        for k in mism:
            assert near_tie_ok(row.astype(np.float64), t, p, float(us[k]), gid[k])
        say(f"[sample] stratified T={t} p={p}: {len(mism)} near-tie of {n}")
        assert len(mism) <= 2


def test_sampled_decode_on_device_logits():
    """Draws from a mid model's decode logits: the device sampler on the logits the decode wrote,
    against the oracle sampler on a copy of the same logits; temperature 0 equals the decode's
    own greedy ids."""
    w = synth.make_weights(synth.MID, seed=0)
    m = dory.Model(synth.MID, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=256, max_tokens=128)
    m.set_loops(2)
    prompt = synth.prompt_tokens(synth.MID, 64)
    lg, gid = m.prefill(0, prompt, 1)
    rng = np.random.default_rng(11)
    tok = int(gid[0].item())
    near = 0
    for step in range(8):
        lg, greedy = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        lg = lg.contiguous()
        u = rng.random(1).astype(np.float32)
        sid = dory.sample(lg, torch.from_numpy(u).to(m.device), temperature=1.0, top_p=0.95)
        g0 = dory.sample(lg, torch.from_numpy(u).to(m.device), temperature=0.0, top_p=0.95)
        torch.cuda.synchronize()
        host = lg[0].double().cpu().numpy()
        oid = sample_row(host, 1.0, 0.95, float(u[0]))
        s = int(sid[0].item())
        if s != oid:
            assert near_tie_ok(host, 1.0, 0.95, float(u[0]), s)
            near += 1
        assert int(g0[0].item()) == int(greedy[0].item())
        tok = s
    say(f"[sample] mid decode, 8 sampled steps: {near} near-tie")
    assert near <= 1


def test_tiny_temperature_draws_among_the_tied_maxima():
    """T = 1e-40 (1/T overflows fp32): only the largest logit and its ties keep mass, shared
    evenly; the device draws among them by u exactly as the oracle does."""
    rng = np.random.default_rng(23)
    v, rows = 32768, 64
    l = rng.integers(-3, 4, (rows, v)).astype(np.float32)     # many ties at the maximum 3
    us = rng.random(rows).astype(np.float32)
    for p in (0.95, 1.0):
        gid = run(l, us, 1e-40, p)
        for r in range(rows):
            assert gid[r] == sample_row(l[r].astype(np.float64), 1e-40, p, float(us[r])), (r, p)
    say(f"[sample] T=1e-40: {rows} rows equal the oracle")


def test_sampler_wide_batch_and_single_row():
    """The chunked sampler at the row counts serving uses (1, 3, 128 rows) over the ~4B vocabulary,
    against the oracle on every row."""
    rng = np.random.default_rng(31)
    v = 131072
    for rows in (1, 3, 128):
        l = (rng.standard_normal((rows, v)) * 2).astype(np.float32)
        us = rng.random(rows).astype(np.float32)
        gid = run(l, us, 1.0, 0.95)
        near = 0
        for r in range(rows):
            oid = sample_row(l[r].astype(np.float64), 1.0, 0.95, float(us[r]))
            if gid[r] != oid:
                assert near_tie_ok(l[r].astype(np.float64), 1.0, 0.95, float(us[r]), gid[r])
                near += 1
        say(f"[sample] {rows} rows x {v}: {near} near-tie")
        assert near <= 1
