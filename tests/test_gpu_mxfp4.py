"""GPU parity of the MXFP4 weight path (OCP Microscaling Formats v1.0: FP4 E2M1 elements, two per
byte, E8M0 scale per 32 elements): the device quantiser against the oracle's byte for byte, and
decode calls that stream the MXFP4 copies against the oracle computing with the same dequantised
weights (bf16 bars: logits 5e-2, hidden states 3e-2; ids equal except near-ties)."""
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
from oracle.mx import quantize_mxfp4  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_device(a):
    bits = synth.to_bf16_bits(np.asarray(a, dtype=np.float32)).view(np.int16)
    return torch.from_numpy(bits).to("cuda:0").view(torch.bfloat16), synth.from_bf16_bits(synth.to_bf16_bits(a))


def test_quantizer_byte_exact_against_oracle():
    rng = np.random.default_rng(8)
    rows = [rng.standard_normal((64, 3072)) / np.sqrt(3072),
            rng.standard_normal((32, 3072)) * np.exp(rng.uniform(-30, 30, (32, 1)))]
    z = np.zeros((4, 3072))
    z[1, 5] = -0.0
    z[2, ::32] = 7.5                                          # 7.5 / 2^(2-2) saturates to 6
    ties = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4)     # block max 4 -> X = 1: exact ties
    z[3, :] = np.tile(ties, 96)
    rows.append(z)
    w = np.concatenate(rows).astype(np.float32)
    dev, w_bf16 = bf16_device(w)
    codes, scales = dory.quantize_mxfp4(dev)
    torch.cuda.synchronize()
    oc, osc = quantize_mxfp4(w_bf16)
    packed = codes.cpu().numpy()
    g_codes = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    g_codes[:, 0::2] = packed & 0xF            # element 2i: low nibble
    g_codes[:, 1::2] = packed >> 4
    g_scales = scales.cpu().numpy()
    say(f"[mxfp4] {w.shape[0]} rows x {w.shape[1]}: codes equal {np.mean(g_codes == oc):.6f}, "
        f"scales equal {np.mean(g_scales == osc):.6f}")
    np.testing.assert_array_equal(g_scales, osc)
    np.testing.assert_array_equal(g_codes, oc)


def decode_vs_oracle(tag, shape, w, m, mode, k, prompt_len, n_dec):
    m.set_kv_mode(mode)
    m.set_loops(k)
    prompt = synth.prompt_tokens(shape, prompt_len)
    om = OracleModel(shape, w, mode, k, gemv_weights="mxfp4")
    _, oid = om.prefill(0, prompt, 1)
    m.prefill(0, prompt, 1)
    tok = int(oid[0])
    g_lg, o_lg, g_h, o_h, g_ids, o_ids = [], [], [], [], [], []
    for _ in range(n_dec):
        l1, i1 = m.decode([0], torch.tensor([tok], dtype=torch.int32, device=m.device))
        ol, oi = om.decode([0], [tok])
        g_lg.append(l1[0].cpu().numpy())
        o_lg.append(ol[0])
        g_h.append(m.last_hidden(1)[0].cpu().numpy())
        o_h.append(om.last_hidden[0])
        g_ids.append(int(i1[0].item()))
        o_ids.append(int(oi[0]))
        tok = int(oi[0])
    g_lg, o_lg = np.array(g_lg), np.array(o_lg)
    err_l = float(np.max(np.abs(g_lg - o_lg)))
    err_h = float(np.max(np.abs(np.array(g_h) - np.array(o_h))))
    say(f"  {tag}: logits max-abs {err_l:.3e}, hidden max-abs {err_h:.3e}, "
        f"ids {sum(a == b for a, b in zip(g_ids, o_ids))}/{n_dec}")
    assert err_l <= 5e-2 and err_h <= 3e-2
    for i in range(n_dec):
        if g_ids[i] != o_ids[i]:
            assert o_lg[i][o_ids[i]] - o_lg[i][g_ids[i]] < 2 * np.max(np.abs(g_lg[i] - o_lg[i]))
    m.release(0)


@pytest.mark.parametrize("mode,k", [("per_loop", 1), ("last_loop", 2)])
def test_mid_mxfp4_decode_vs_oracle(mode, k):
    w = synth.make_weights(synth.MID, seed=0)
    m = dory.Model(synth.MID, w, kv_mode=mode, max_loops=2, max_seqs=2, max_model_len=512, max_tokens=300,
                   gemv_weights="mxfp4")
    say(f"[mid mxfp4] mode={mode} k={k} prompt=300 decode=4 (teacher-forced)")
    decode_vs_oracle(f"mid k={k} {mode}", synth.MID, w, m, mode, k, 300, 4)
    m.close()


def test_4b_width_mxfp4_decode_vs_oracle():
    """The MXFP4 GEMV instances the ~4B decode streams (K = 3072 with and without the residual
    prologue, K = 8192 for down) on a 3-block model of the ~4B widths."""
    shape = synth.ModelShape(d_model=3072, n_heads=24, n_kv_heads=8, head_dim=128, d_ff=8192, vocab=4096,
                             n_in=1, n_rec=1, n_out=1, window=4096, dtype=synth.BF16)
    w = synth.make_weights(shape, seed=4)
    m = dory.Model(shape, w, kv_mode="last_loop", max_loops=2, max_seqs=1, max_model_len=128, max_tokens=64,
                   gemv_weights="mxfp4")
    say("[4B width mxfp4] 64-token prompt + 3 decode steps, k=2, last-loop")
    decode_vs_oracle("4B width k=2", shape, w, m, "last_loop", 2, 64, 3)
    m.close()
