"""Pins of the oracle's MXFP8 quantiser (oracle/mx.py) against the OCP Microscaling (MX)
Formats Specification v1.0: the FP8 E4M3 element format (bias 7, 3 mantissa bits, largest
normal 448, smallest normal 2^-6, smallest subnormal 2^-9, S.1111.111 = NaN), the E8M0 shared
scale 2^(code - 127), and the conversion rule X = 2^(floor(log2 max|V|) - 8) with round to
nearest even and saturation. CPU only."""
import numpy as np

from looped_ngpt_language_amd import synth
from oracle import OracleModel
from oracle.mx import E4M3_TABLE, dequantize_mxfp8, e8m0_value, quantize_mxfp8, round_e4m3


def test_e4m3_table_closed_forms():
    t = E4M3_TABLE
    assert t[0] == 0.0 and t[1] == 2.0 ** -9 and t[7] == 7 * 2.0 ** -9       # subnormals m * 2^-9
    assert t[8] == 2.0 ** -6                                                  # smallest normal
    assert t[56] == 1.0 and t[57] == 1.125 and t[63] == 1.875                 # 2^0 * (1 + m/8)
    assert t[120] == 256.0 and t[126] == 448.0                                # 2^8, largest normal 1.75 * 2^8
    assert np.isnan(t[127]) and np.isnan(t[255])                              # S.1111.111
    assert t[128] == 0.0 and np.signbit(t[128])                               # negative zero
    assert np.all(t[128:255] == -t[:127])                                     # sign bit mirrors
    assert np.all(np.diff(t[:127]) > 0)                                       # codes 0..126 increase


def test_e4m3_round_trip_midpoints_and_saturation():
    codes = np.arange(127)
    np.testing.assert_array_equal(round_e4m3(E4M3_TABLE[:127]), codes)       # exact values round-trip
    mid = 0.5 * (E4M3_TABLE[:126] + E4M3_TABLE[1:127])                         # ties between codes c, c+1
    want = np.where(codes[:126] % 2 == 0, codes[:126], codes[:126] + 1)       # the even code wins
    np.testing.assert_array_equal(round_e4m3(mid), want)
    np.testing.assert_array_equal(round_e4m3(-mid), want | 0x80)
    assert round_e4m3([447.9])[0] == 126 and round_e4m3([460.0])[0] == 126 and round_e4m3([1e6])[0] == 126
    assert round_e4m3([1.0 + 1e-9])[0] == 56 and round_e4m3([1.0625 + 1e-9])[0] == 57


def test_mx_scale_rule_hand_values():
    rows = np.zeros((5, 32))
    rows[0, :] = 1.0                  # max 1     -> X = 2^(0 - 8),  code 119; element 256 -> code 120
    rows[1, 3] = 300.0                # max 300   -> X = 2^(8 - 8),  code 127; 300 -> nearest 288 (code 121)
    rows[2, 0] = -0.75                # max 0.75  -> X = 2^(-1 - 8), code 118; -0.75 / X = -384 -> code 0x80|124
    rows[3, 0] = 1.9                  # 1.9 / 2^-8 = 486.4 saturates to 448 -> 1.75
    codes, sc = quantize_mxfp8(rows)  # row 4: all zero -> scale code 0, zero elements
    np.testing.assert_array_equal(sc[:, 0], [119, 127, 118, 119, 0])
    assert codes[0, 0] == 120 and codes[1, 3] == 121 and codes[2, 0] == (0x80 | 124) and codes[3, 0] == 126
    assert np.all(codes[4] == 0) and np.all(codes[1, :3] == 0)
    deq = dequantize_mxfp8(codes, sc)
    assert deq[0, 0] == 1.0 and deq[1, 3] == 288.0 and deq[2, 0] == -0.75 and deq[3, 0] == 1.75
    assert e8m0_value(127) == 1.0 and e8m0_value(0) == 2.0 ** -127


def test_mx_error_bound_and_idempotence():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-8, 3, (16, 1)))
    codes, sc = quantize_mxfp8(w)
    deq = dequantize_mxfp8(codes, sc)
    X = np.repeat(e8m0_value(sc), 32, axis=1)
    q = np.abs(w / X)
    normal = (q >= 2.0 ** -6) & (q <= 448.0)
    rel = np.abs(deq - w)[normal] / np.abs(w)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-15          # half a unit in the last place of a 3-bit mantissa
    assert np.all(np.abs(deq[q > 448.0]) == 448.0 * X[q > 448.0])
    c2, s2 = quantize_mxfp8(deq)                   # already representable: unchanged values
    np.testing.assert_array_equal(dequantize_mxfp8(c2, s2), deq)


def test_oracle_model_uses_mx_weights_only_for_calls_of_at_most_two_rows():
    w = synth.make_weights(synth.TINY, seed=0)
    base = OracleModel(synth.TINY, w, "per_loop", 2)
    mx = OracleModel(synth.TINY, w, "per_loop", 2, gemv_weights="mxfp8")
    prompt = synth.prompt_tokens(synth.TINY, 12)
    l0, _ = base.prefill(0, prompt, 3)
    l1, _ = mx.prefill(0, prompt, 3)
    np.testing.assert_array_equal(l0, l1)           # 12 rows: as-given weights
    d0, _ = base.decode([0], [5])
    d1, _ = mx.decode([0], [5])
    assert 0 < np.max(np.abs(d0 - d1)) < 0.5        # one row: quantised weights, close but different
    np.testing.assert_array_equal(mx.blocks_mx[0]["alpha_attn"], base.blocks[0]["alpha_attn"])


# ---------------------------------------------------------------- MXFP4 (FP4 E2M1 elements)

from oracle.mx import E2M1_TABLE, dequantize_mxfp4, quantize_mxfp4, round_e2m1  # noqa: E402


def test_e2m1_table_closed_forms():
    """FP4 E2M1 (OCP MX v1.0): bias 1, one mantissa bit; the eight magnitudes are
    0, 0.5 (the subnormal), 1, 1.5, 2, 3, 4, 6; the sign bit mirrors them."""
    np.testing.assert_array_equal(E2M1_TABLE[:8], [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    assert E2M1_TABLE[8] == 0.0 and np.signbit(E2M1_TABLE[8])
    np.testing.assert_array_equal(E2M1_TABLE[8:], -E2M1_TABLE[:8])


def test_e2m1_rounding_ties_and_saturation():
    np.testing.assert_array_equal(round_e2m1(E2M1_TABLE[:8]), np.arange(8))
    # midpoints, hand-derived: the even code (mantissa bit 0) wins
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    want = [0, 2, 2, 4, 4, 6, 6]     # 0, 1, 1, 2, 2, 4, 4
    np.testing.assert_array_equal(round_e2m1(mids), want)
    np.testing.assert_array_equal(round_e2m1([-m for m in mids]), [w | 0x8 for w in want])
    np.testing.assert_array_equal(round_e2m1([0.26, 0.74, 2.51, 5.01]), [1, 1, 5, 7])
    np.testing.assert_array_equal(round_e2m1([6.0, 7.0, 100.0, -1e9]), [7, 7, 7, 15])   # saturate at 6


def test_mxfp4_scale_rule_hand_values():
    rows = np.zeros((4, 32))
    rows[0, :] = 1.0                  # max 1   -> X = 2^(0 - 2),  code 125; element 4 -> code 6
    rows[1, 5] = 6.0                  # max 6   -> X = 2^(2 - 2),  code 127; element 6 -> code 7
    rows[1, 6] = 0.2                  #             0.2 -> nearest of 0 / 0.5 is 0 -> code 0
    rows[2, 0] = -0.3                 # max 0.3 -> X = 2^(-2 - 2), code 123; -0.3 / X = -4.8 -> -4 (code 0xE)
    codes, sc = quantize_mxfp4(rows)  # row 3: all zero -> code 0, zero elements
    np.testing.assert_array_equal(sc[:, 0], [125, 127, 123, 0])
    assert np.all(codes[0] == 6)
    assert codes[1, 5] == 7 and codes[1, 6] == 0 and codes[1, 0] == 0
    assert codes[2, 0] == 0xE and codes[2, 1] == 0
    assert np.all(codes[3] == 0)
    deq = dequantize_mxfp4(codes, sc)
    assert deq[0, 0] == 1.0 and deq[1, 5] == 6.0 and deq[2, 0] == -0.25


def test_mxfp4_error_bound_and_idempotence():
    """|v - dq(q(v))| <= half an E2M1 step at v's magnitude times X, except above the largest
    element value 6, where the spec saturates (the block maximum over X lies in [4, 8), so the
    top elements may lose up to 2 X): there the error is exactly (|v| / X - 6) X. Re-quantising
    the dequantised values changes nothing."""
    rng = np.random.default_rng(3)
    w = rng.standard_normal((16, 256)) * np.exp(rng.uniform(-6, 6, (16, 1)))
    codes, sc = quantize_mxfp4(w)
    deq = dequantize_mxfp4(codes, sc)
    X = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    q = np.abs(w) / X
    step = np.select([q < 2, q < 4], [0.5, 1.0], 2.0)    # spacing of E2M1 values around q
    inside = q <= 6.0
    assert np.all(np.abs(w - deq)[inside] <= (0.5 * step * X)[inside] + 1e-300)
    np.testing.assert_allclose(np.abs(w - deq)[~inside], ((q - 6.0) * X)[~inside], rtol=1e-12)
    assert np.any(~inside)
    c2, s2 = quantize_mxfp4(deq)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, sc)


def test_oracle_model_uses_mxfp4_weights_only_for_calls_of_at_most_two_rows():
    """As for MXFP8: 12-row calls use the weights as given; one-row calls the MXFP4 copies, whose
    logits differ more than MXFP8's (4-bit elements) but stay close."""
    w = synth.make_weights(synth.TINY, seed=0)
    base = OracleModel(synth.TINY, w, "per_loop", 2)
    m8 = OracleModel(synth.TINY, w, "per_loop", 2, gemv_weights="mxfp8")
    m4 = OracleModel(synth.TINY, w, "per_loop", 2, gemv_weights="mxfp4")
    prompt = synth.prompt_tokens(synth.TINY, 12)
    l0, _ = base.prefill(0, prompt, 3)
    m8.prefill(0, prompt, 3)
    l4, _ = m4.prefill(0, prompt, 3)
    np.testing.assert_array_equal(l0, l4)
    d0, _ = base.decode([0], [5])
    d8, _ = m8.decode([0], [5])
    d4, _ = m4.decode([0], [5])
    e8, e4 = np.max(np.abs(d0 - d8)), np.max(np.abs(d0 - d4))
    assert 0 < e8 < e4 < 0.5
    q, sc = quantize_mxfp4(w.blocks[0]["wq"])
    np.testing.assert_array_equal(m4.blocks_mx[0]["wq"], dequantize_mxfp4(q, sc))
