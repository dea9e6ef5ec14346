"""Host-side planner (speed-up model and draft-length choice): CPU only.

Pins: the worked value and the alpha = 1 case of kasblo.com "Speculative
Decodingとは？" section "1回のtarget検証で何token進むか" (tests/golden/
expected_tokens.json), the oracle's term-by-term sum, a Monte Carlo estimate of
the committed length, and brute force over a small table of times."""

import json
import os

import numpy as np
import pytest

from oracle import qspec_oracle as O
from quantized_speculative_decoding_int4_amd import planner as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "expected_tokens.json")


def test_expected_tokens_matches_the_pages_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert P.expected_tokens(c["alpha"], c["gamma"]) == pytest.approx(c["expected_tokens"], abs=1e-12)


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.8, 0.96, 0.999, 1.0])
@pytest.mark.parametrize("gamma", [0, 1, 3, 5, 7])
def test_expected_tokens_closed_form_equals_the_oracle_sum(alpha, gamma):
    assert P.expected_tokens(alpha, gamma) == pytest.approx(O.expected_tokens(alpha, gamma), rel=1e-12)


def test_expected_tokens_monte_carlo():
    """Commit = accepted prefix + 1, each candidate accepted with probability alpha."""
    rng = np.random.default_rng(5)
    alpha, gamma, n = 0.96, 3, 400_000
    acc = rng.random((n, gamma)) < alpha
    prefix = np.where(acc.all(axis=1), gamma, np.argmin(acc, axis=1))
    committed = prefix + 1
    se = committed.std() / np.sqrt(n)
    assert abs(committed.mean() - P.expected_tokens(alpha, gamma)) <= 4 * se


def test_speedup_matches_the_oracle_model():
    et = O.expected_tokens(0.96, 3)
    ref = O.speedup_model(et, 1.3, 1.28, 3, 1.32, 0.04)
    assert P.modelled_speedup(0.96, 3, 1.3, 1.28, 1.32, 0.04) == pytest.approx(ref, rel=1e-12)
    # a draft as costly as the target loses even at high acceptance (shared weights, same bytes)
    assert P.modelled_speedup(0.96, 3, 1.0, 1.0, 1.0) < 1.0
    # a free draft and a verify costing one target pass give exactly E[T]
    assert P.modelled_speedup(0.8, 4, 1.0, 0.0, 1.0) == pytest.approx(3.3616, abs=1e-12)


def test_inter_token_latency():
    assert P.inter_token_latency(0.8, 4, 3.3616) == pytest.approx(1.0, abs=1e-12)


def test_choose_gamma_brute_force():
    rng = np.random.default_rng(9)
    for _ in range(200):
        alpha = float(rng.uniform(0.2, 1.0))
        batch = int(rng.integers(1, 17))
        t_draft = float(rng.uniform(0.1, 2.0))
        tv = {g: float(rng.uniform(0.5, 5.0)) for g in (1, 3, 5, 7)}
        over = float(rng.uniform(0.0, 0.2))
        got = P.choose_gamma(alpha, batch, t_draft, tv, over)
        rates = {g: batch * O.expected_tokens(alpha, g) / (g * t_draft + tv[g] + over) for g in tv}
        best = max(rates.values())
        assert rates[got["best_gamma"]] == pytest.approx(best, rel=1e-12)
        for g in tv:
            assert got["table"][g]["tokens_per_time"] == pytest.approx(rates[g], rel=1e-12)


def test_choose_gamma_prefers_short_lookahead_when_acceptance_is_low():
    tv = {1: 1.0, 3: 1.0, 7: 1.0}
    assert P.choose_gamma(0.1, 1, 0.5, tv)["best_gamma"] == 1
    assert P.choose_gamma(0.99, 1, 0.01, tv)["best_gamma"] == 7


def test_planner_rejects_bad_arguments():
    with pytest.raises(ValueError):
        P.expected_tokens(1.5, 3)
    with pytest.raises(ValueError):
        P.expected_tokens(0.5, -1)
    with pytest.raises(ValueError):
        P.choose_gamma(0.5, 0, 1.0, {3: 1.0})
