"""Pins for the oracle's chain (the stack of linears of one draft / verify pass) and for the bound
the GPU chain tests use: exact special cases, the fp16 rounding step, and the chain's own
sensitivity to rounding-sized perturbations (tests/chain_sensitivity.py), recomputed here and
compared with the recorded values in tests/golden/chain_sensitivity.json."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import qspec_oracle as O
from quantized_speculative_decoding_int4_amd import workloads as W
from tests import chain_sensitivity as CS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "chain_sensitivity.json")


def test_fp16_rounding_is_correct_from_float64():
    """The chain rounds float64 values to fp16 directly (NumPy's conversion): just above and below
    every midpoint between neighbouring finite fp16 values the nearest neighbour wins, exactly at the
    midpoint the even one.  Rounding through fp32 first gets thousands of these wrong (double
    rounding), which is why a kernel must not do that."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    a, b = h[:-1].astype(np.float64), h[1:].astype(np.float64)
    mid = (a + b) / 2                                           # exact in float64
    up, dn = np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)
    assert np.all(up.astype(np.float16).astype(np.float64) == b)
    assert np.all(dn.astype(np.float16).astype(np.float64) == a)
    even = np.where((h[:-1].view(np.uint16) & 1) == 0, a, b)
    assert np.all(mid.astype(np.float16).astype(np.float64) == even)
    assert np.all((-up).astype(np.float16).astype(np.float64) == -b)
    twice = up.astype(np.float32).astype(np.float16).astype(np.float64)
    assert np.count_nonzero(twice != b) > 1000


def test_chain_w4a16_standardisation_with_a_mean_exact():
    """Stage 1 outputs exactly 2^-6 (3 +- 1) with equal counts: mean 3 * 2^-6, std 2^-6, so the
    standardised row is exactly +-1 and the W4A16 stage 2 is exact; brute force with rationals.  A
    dropped mean (or a wrong std) changes every value."""
    rng = W.rng_for(23)
    k1, n1 = 128, 256
    q1 = np.zeros((n1, k1), np.int8)
    half = np.array([1, -1] * 64, np.int8)
    signs = np.concatenate([rng.permutation(half), rng.permutation(half)])
    q1[:, 0] = signs
    q1[:, 1] = 3
    q1[:, 2:] = rng.integers(-8, 8, size=(n1, k1 - 2), dtype=np.int8)
    s1 = np.full((n1, 1), 2.0 ** -6, np.float16)
    x = np.zeros((2, k1), np.float16)
    x[:, 0] = 1.0
    x[:, 1] = 1.0
    q2, s2 = W.integer_case_weights(rng, 8, 128, exponents=(-5,))
    y = O.chain_forward("w4a16", x, [(q1, s1), (q2, s2)])
    z = signs[:128]
    for m in range(2):
        for n in range(8):
            ref = sum(Fraction(int(z[k])) * int(q2[n, k]) * Fraction(float(s2[n, 0])) for k in range(128))
            assert Fraction(y[m, n]) == ref
    # the integer modes round the (exact) +-1 to fp16 and quantize it: codes +-7, scale 1/7 in fp16
    for mode in ("w4a4", "w4a8"):
        yi = O.chain_forward(mode, x, [(q1, s1), (q2, s2)])
        qmax = 7 if mode == "w4a4" else 127
        sx = np.float16(np.float32(1.0) / np.float32(qmax))
        codes = np.rint(z.astype(np.float64) / float(sx)).clip(-qmax - 1, qmax)
        for n in range(8):
            ref = sum(Fraction(int(codes[k])) * int(q2[n, k]) for k in range(128))
            assert Fraction(yi[0, n]) == ref * Fraction(float(s2[n, 0])) * Fraction(float(sx))


def test_unperturbed_pair_is_the_oracle_chain():
    rng = W.rng_for(24)
    layers = [W.int4_weights(rng, n, k) for n, k in [(384, 256), (256, 384), (300, 256)]]
    x, _ = W.activations(rng, 3, 256)
    for mode in ("w4a16", "w4a4", "w4a8"):
        y_ref, y_same = CS.chain_pair(mode, x, lambda i: layers[i], 3, seed=0, eps_y=0.0, eps_n=0.0)
        assert np.array_equal(y_ref, O.chain_forward(mode, x, layers))
        assert np.array_equal(y_same, y_ref)


@pytest.mark.parametrize("key,m", [("long75_m4", 4), ("small_llama_m4", 4), ("long75_m12", 12)])
def test_recorded_sensitivity_is_reproduced(key, m):
    """The recorded spreads are the oracle's: rerunning the recording's configuration gives the same
    numbers (the GPU bound rests on them)."""
    from tests.golden.make_chain_sensitivity import measure, small_llama_like, small_long_chain
    with open(GOLDEN) as f:
        rec = json.load(f)["configs"][key]
    make = small_long_chain if key.startswith("long75") else small_llama_like
    got = measure(key, make, m, seeds=tuple(r["seed"] for r in rec["runs"]))
    assert got["rel_fro"] == pytest.approx(rec["rel_fro"], rel=1e-9)
    assert got["max_abs_over_rms"] == pytest.approx(rec["max_abs_over_rms"], rel=1e-9)


def test_recorded_bounds_shape():
    """What the recording says about chains: a 9-stage W4A16 chain stays inside the single-linear
    bar (rel-Frobenius 2e-3) under fp32-sized perturbations, while a 129-stage one does not -- so the
    full stack needs the chain bound and cannot be held to the single-linear bar end to end -- and
    the drift grows with depth."""
    with open(GOLDEN) as f:
        cfg = json.load(f)["configs"]
    assert all(cfg[k]["rel_fro"] < 1e-3 for k in cfg if k.startswith("small_llama"))
    assert cfg["llama_full_m4"]["rel_fro"] > 2e-3 and cfg["llama_full_m128"]["rel_fro"] > 2e-3
    assert cfg["llama_full_m4"]["rel_fro"] > cfg["long75_m4"]["rel_fro"] > cfg["small_llama_m4"]["rel_fro"]
    assert cfg["llama_full_m4"]["rel_fro"] < 1e-2


def test_integer_chains_need_exact_standardisation():
    """Why the integer modes' kernels standardise and scale in fp64 and round once: in W4A8 an
    fp32-sized error in the standardised values alone (nothing else perturbed) already flips codes
    that then cascade -- over 9 stages at 256 rows the output moves by far more than the 1e-2
    bar -- whereas the unperturbed chain is reproduced exactly."""
    rng = W.rng_for(801)
    h, inter = 512, 1024
    shapes = [(h + 256, h), (h, h), (2 * inter, h), (h, inter)] * 2 + [(3000, h)]
    layers = [W.int4_weights(rng, n, k) for n, k in shapes]
    x, _ = W.activations(rng, 256, h)
    y_ref, y_per = CS.chain_pair("w4a8", x, lambda i: layers[i], len(layers), seed=1, eps_y=0.0,
                                 eps_n=CS.EPS_NORM)
    assert np.abs(y_per - y_ref).max() > 1e-2
    y_ref2, y_same = CS.chain_pair("w4a8", x, lambda i: layers[i], len(layers), seed=1, eps_y=0.0, eps_n=0.0)
    assert np.array_equal(y_same, y_ref2) and np.array_equal(y_ref2, y_ref)
