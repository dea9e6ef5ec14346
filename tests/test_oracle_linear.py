"""Pins for the oracle's INT4 linear layer (both modes) and the activation
quantizer, against exact arithmetic and brute force -- never against the
oracle's own formulas retyped."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import qspec_oracle as O
from quantized_speculative_decoding_int4_amd import workloads as W


def _brute_w4a16(x, q, s):
    """Pure-Python triple loop with exact rationals: y[m][n] = sum_k x*q*scale."""
    m_, k_ = x.shape
    n_ = q.shape[0]
    out = [[Fraction(0)] * n_ for _ in range(m_)]
    for m in range(m_):
        for n in range(n_):
            acc = Fraction(0)
            for k in range(k_):
                acc += Fraction(float(x[m, k])) * int(q[n, k]) * Fraction(float(s[n, k // 128]))
            out[m][n] = acc
    return out


def test_w4a16_exact_integer_case_brute_force():
    rng = W.rng_for(11)
    q, s = W.integer_case_weights(rng, 5, 384, exponents=(-3, -4, -5, -6, -7))
    x = W.integer_activations(rng, 3, 384)
    y = O.linear_w4a16(x, q, s)
    ref = _brute_w4a16(x, q, s)
    for m in range(3):
        for n in range(5):
            assert Fraction(y[m, n]) == ref[m][n]


def test_w4a16_group_index_matters():
    # scales differ per group, so a wrong group mapping changes the result
    rng = W.rng_for(12)
    q, s = W.integer_case_weights(rng, 4, 256, exponents=(-2, -8))
    x = W.integer_activations(rng, 2, 256)
    y = O.linear_w4a16(x, q, s)
    s_swapped = s[:, ::-1].copy()
    if not np.array_equal(s, s_swapped):
        assert not np.array_equal(y, O.linear_w4a16(x, q, s_swapped))


def test_w4a16_random_against_brute_force():
    rng = W.rng_for(13)
    q, s = W.int4_weights(rng, 3, 256)
    x, _ = W.activations(rng, 2, 256, n_outliers=2)
    y = O.linear_w4a16(x, q, s)
    ref = _brute_w4a16(x, q, s)
    for m in range(2):
        for n in range(3):
            assert abs(y[m, n] - float(ref[m][n])) <= 1e-12 * max(1.0, abs(float(ref[m][n])))


def _round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _all_finite_fp16():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("amax", [7.0, 1.0, 3.3, 0.0625, 1000.0, 20.5])
def test_act_quant_brute_force_all_fp16(amax):
    """Every finite fp16 value v with |v| <= amax, quantized in a row whose
    maximum is amax, against exact rational round-half-even."""
    a16 = np.float16(amax)
    vals = _all_finite_fp16()
    vals = vals[np.abs(vals.astype(np.float64)) <= float(a16)]
    x = np.stack([np.full(vals.shape, a16), vals], axis=1).astype(np.float16)
    xq, sx = O.quantize_activations(x)
    s = sx[0]
    assert np.all(sx == s)
    s_fr = Fraction(float(s))
    ref = np.array([max(-8, min(7, _round_half_even(Fraction(float(v)) / s_fr))) for v in vals])
    assert np.array_equal(xq[:, 1].astype(np.int64), ref)
    # ties must actually be exercised for the rounding rule to be pinned
    ties = [v for v in vals if (Fraction(float(v)) / s_fr).denominator == 2]
    if amax in (7.0, 1000.0, 20.5):
        assert len(ties) > 0


def test_act_quant_scale_values():
    # s = fp16(fp32(amax) / 7): exact cases and a zero row
    x = np.array([[7.0, -1.0], [-3.5, 0.25], [0.0, 0.0], [14.0, 2.0]], dtype=np.float16)
    xq, sx = O.quantize_activations(x)
    assert sx.tolist() == [1.0, 0.5, 0.0, 2.0]
    assert xq.tolist() == [[7, -1], [-7, 0], [0, 0], [7, 1]]


def test_act_quant_scale_rounding_one_over_seven():
    # fp32(1/7) = 0x3E124925 -> fp16 RNE: 0.142822265625 (0x3092)
    x = np.array([[1.0]], dtype=np.float16)
    _, sx = O.quantize_activations(x)
    assert sx.view(np.uint16)[0] == 0x3092
    assert np.float32(1.0) / np.float32(7.0) == np.frombuffer(np.uint32(0x3E124925).tobytes(), np.float32)[0]


def test_act_quant_multiples_of_scale():
    # x = j * s exactly  ->  xq = j
    s = np.float16(0.25)
    row = np.array([7 * s] + [j * s for j in range(-7, 8)], dtype=np.float16)
    xq, sx = O.quantize_activations(row[None, :])
    assert sx[0] == s
    assert xq[0, 1:].tolist() == list(range(-7, 8))


def test_act_quant_invariants_random_rows():
    rng = W.rng_for(14)
    x, _ = W.activations(rng, 64, 4096)
    xq, sx = O.quantize_activations(x)
    s64 = sx.astype(np.float64)[:, None]
    assert np.all(np.abs(xq).max(axis=1) == 7)
    err = np.abs(x.astype(np.float64) - xq * s64)
    assert np.all(err <= s64 / 2 + 1e-300)


def test_w4a4_accumulators_brute_force():
    rng = W.rng_for(15)
    q, s = W.int4_weights(rng, 4, 384)
    x, _ = W.activations(rng, 3, 384, n_outliers=1)
    r = O.linear_w4a4(x, q, s)
    xq = r["xq"]
    for m in range(3):
        for n in range(4):
            for g in range(3):
                ref = sum(int(xq[m, k]) * int(q[n, k]) for k in range(128 * g, 128 * g + 128))
                assert r["acc"][m, n, g] == ref
    # y from exact rationals
    for m in range(3):
        for n in range(4):
            tot = Fraction(0)
            for g in range(3):
                tot += Fraction(float(s[n, g])) * int(r["acc"][m, n, g])
            tot *= Fraction(float(r["sx"][m]))
            assert abs(r["y"][m, n] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))


def test_w4a4_zero_row_and_bound():
    rng = W.rng_for(16)
    q, s = W.int4_weights(rng, 8, 256)
    x = np.zeros((2, 256), dtype=np.float16)
    x[1] = W.activations(rng, 1, 256)[0][0]
    r = O.linear_w4a4(x, q, s)
    assert np.all(r["xq"][0] == 0) and r["sx"][0] == 0 and np.all(r["y"][0] == 0)
    assert np.abs(r["acc"]).max() <= 128 * 8 * 8


def test_w4a4_approximates_w4a16():
    # W4A4 is W4A16 with the activations replaced by their quantized values
    rng = W.rng_for(17)
    q, s = W.int4_weights(rng, 16, 512)
    x, _ = W.activations(rng, 2, 512)
    r = O.linear_w4a4(x, q, s)
    xdq = (r["xq"].astype(np.float64) * r["sx"].astype(np.float64)[:, None])
    y_ref = xdq @ O.dequantize_weights(q, s).T
    assert np.allclose(r["y"], y_ref, rtol=1e-12, atol=1e-12)


def test_lm_head_chunking_matches_full():
    rng = W.rng_for(18)
    q, s = W.int4_weights(rng, 300, 256)
    x, _ = W.activations(rng, 3, 256)
    for mode, full in (("w4a16", O.linear_w4a16(x, q, s)), ("w4a4", O.linear_w4a4(x, q, s)["y"])):
        assert np.array_equal(O.lm_head(mode, x, q, s, chunk=64), full)


def _balanced_chain_case(rng):
    """Stage 1 maps a one-hot input row to outputs of exactly +-2^-6 with equal
    counts, so standardisation gives exactly +-1 and stage 2 is exact integer
    arithmetic."""
    k1, n1 = 128, 256
    q1 = np.zeros((n1, k1), np.int8)
    half = np.array([1, -1] * 64, np.int8)        # balanced within the 128 columns read
    signs = np.concatenate([rng.permutation(half), rng.permutation(half)])
    q1[:, 0] = signs
    q1[:, 1:] = rng.integers(-8, 8, size=(n1, k1 - 1), dtype=np.int8)
    s1 = np.full((n1, 1), 2.0 ** -6, np.float16)
    x = np.zeros((2, k1), np.float16)
    x[:, 0] = 1.0
    q2, s2 = W.integer_case_weights(rng, 8, 128, exponents=(-5,))
    return x, [(q1, s1), (q2, s2)], signs


def test_chain_exact_balanced_case():
    rng = W.rng_for(19)
    x, layers, signs = _balanced_chain_case(rng)
    y = O.chain_forward("w4a16", x, layers)
    mid = np.tile(signs[:128].astype(np.float16), (2, 1))     # standardised stage-1 output
    ref = _brute_w4a16(mid, *layers[1])
    for m in range(2):
        for n in range(8):
            assert Fraction(y[m, n]) == ref[m][n]


def test_standardize_rows_properties():
    rng = W.rng_for(21)
    y = rng.standard_normal((3, 1000)) * 5 + 3
    z = O.standardize_rows(y).astype(np.float64)
    assert np.allclose(z.mean(axis=1), 0, atol=2e-3) and np.allclose(z.std(axis=1), 1, atol=2e-3)
    assert np.all(O.standardize_rows(np.full((1, 8), 2.5)) == 0)          # zero spread -> zeros
    assert np.array_equal(O.standardize_rows(np.array([[1.0, -1.0, 1.0, -1.0]])),
                          np.array([[1, -1, 1, -1]], np.float16))


def test_chain_single_stage_is_the_linear():
    rng = W.rng_for(20)
    q, s = W.int4_weights(rng, 64, 256)
    x, _ = W.activations(rng, 3, 256)
    assert np.array_equal(O.chain_forward("w4a16", x, [(q, s)]), O.linear_w4a16(x, q, s))
    assert np.array_equal(O.chain_forward("w4a4", x, [(q, s)]), O.linear_w4a4(x, q, s)["y"])


# ---------------------------------------------------------------- W4A8 (8-bit activations)

@pytest.mark.parametrize("amax", [127.0, 1.0, 3.3, 0.0625, 1000.0, 20.5])
def test_act_quant_int8_brute_force_all_fp16(amax):
    """Every finite fp16 value v with |v| <= amax, quantized in a row whose
    maximum is amax, against exact rational round-half-even and the int8 clamp."""
    a16 = np.float16(amax)
    vals = _all_finite_fp16()
    vals = vals[np.abs(vals.astype(np.float64)) <= float(a16)]
    x = np.stack([np.full(vals.shape, a16), vals], axis=1).astype(np.float16)
    xq, sx = O.quantize_activations_int8(x)
    s = sx[0]
    assert np.all(sx == s)
    s_fr = Fraction(float(s))
    ref = np.array([max(-128, min(127, _round_half_even(Fraction(float(v)) / s_fr))) for v in vals])
    assert np.array_equal(xq[:, 1].astype(np.int64), ref)
    ties = [v for v in vals if (Fraction(float(v)) / s_fr).denominator == 2]
    if amax in (127.0, 1.0, 20.5):
        assert len(ties) > 0


def test_act_quant_int8_scale_values():
    # s = fp16(fp32(amax) / 127): exact cases, a zero row, and 1/127 rounded twice
    x = np.array([[127.0, -1.0], [-63.5, 0.25], [0.0, 0.0], [254.0, 3.0]], dtype=np.float16)
    xq, sx = O.quantize_activations_int8(x)
    assert sx.tolist() == [1.0, 0.5, 0.0, 2.0]
    assert xq.tolist() == [[127, -1], [-127, 0], [0, 0], [127, 2]]  # 3 / 2 = 1.5 -> 2 (half to even)
    _, s1 = O.quantize_activations_int8(np.array([[1.0]], dtype=np.float16))
    f32 = np.float32(1.0) / np.float32(127.0)
    assert s1[0] == np.float16(f32) and abs(float(s1[0]) - 1.0 / 127.0) <= 2.0 ** -17


def test_act_quant_int8_multiples_of_scale_and_invariants():
    s = np.float16(0.125)
    row = np.array([127 * s] + [j * s for j in range(-127, 128)], dtype=np.float16)
    xq, sx = O.quantize_activations_int8(row[None, :])
    assert sx[0] == s and xq[0, 1:].tolist() == list(range(-127, 128))
    rng = W.rng_for(18)
    x, _ = W.activations(rng, 32, 1024)
    xq, sx = O.quantize_activations_int8(x)
    s64 = sx.astype(np.float64)[:, None]
    assert np.all(np.abs(xq).max(axis=1) >= 126)
    assert np.all(np.abs(x.astype(np.float64) - xq * s64) <= s64 / 2 + 1e-300)


def test_w4a8_accumulators_and_output_brute_force():
    rng = W.rng_for(19)
    q, s = W.int4_weights(rng, 3, 256)
    x, _ = W.activations(rng, 2, 256, n_outliers=1)
    r = O.linear_w4a8(x, q, s)
    xq = r["xq"]
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for g in range(2):
                ref = sum(int(xq[m, k]) * int(q[n, k]) for k in range(128 * g, 128 * g + 128))
                assert r["acc"][m, n, g] == ref
                tot += Fraction(float(s[n, g])) * ref
            tot *= Fraction(float(r["sx"][m]))
            assert abs(r["y"][m, n] - float(tot)) <= 1e-12 * max(1.0, abs(float(tot)))
    assert np.abs(r["acc"]).max() <= 128 * 128 * 8


def test_w4a8_is_closer_to_w4a16_than_w4a4():
    # 8-bit activations: quantization error ~ s/2 with s = max|x| / 127 instead of / 7
    rng = W.rng_for(20)
    q, s = W.int4_weights(rng, 64, 1024)
    x, _ = W.activations(rng, 4, 1024)
    ref = O.linear_w4a16(x, q, s)
    e8 = np.linalg.norm(O.linear_w4a8(x, q, s)["y"] - ref)
    e4 = np.linalg.norm(O.linear_w4a4(x, q, s)["y"] - ref)
    assert e8 < e4 / 8


def test_integer_output_equals_the_group_sum_form_exactly():
    """The oracle's W4A4 / W4A8 output (one product with the dequantized weights) equals the
    per-group form s_m * sum_g s[n, g] * acc[m, n, g] summed with exact rationals, bit for bit: the
    float64 evaluation is exact for these magnitudes, so any summation order gives it."""
    rng = W.rng_for(22)
    q, s = W.int4_weights(rng, 6, 1024)
    x, _ = W.activations(rng, 3, 1024)
    for r in (O.linear_w4a4(x, q, s), O.linear_w4a8(x, q, s)):
        for m in range(3):
            for n in range(6):
                tot = sum(Fraction(float(s[n, g])) * int(r["acc"][m, n, g]) for g in range(8))
                assert Fraction(float(r["y"][m, n])) == tot * Fraction(float(r["sx"][m]))


def test_dequantized_weights_group_mapping():
    q = np.arange(-8, 8, dtype=np.int8).repeat(32).reshape(2, 256)
    s = np.array([[1.0, 2.0], [4.0, 0.5]], np.float16)
    w = O.dequantize_weights(q, s)
    assert w[0, 5] == q[0, 5] * 1.0 and w[0, 130] == q[0, 130] * 2.0
    assert w[1, 0] == q[1, 0] * 4.0 and w[1, 255] == q[1, 255] * 0.5
