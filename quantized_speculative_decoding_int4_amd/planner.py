"""Host-side planning of a speculative iteration from measured pass times.

The timing model of kasblo.com, "Speculative Decodingとは？LLM生成を速くする方法":
* section "1回のtarget検証で何token進むか": with draft length gamma and a constant
  per-candidate acceptance rate alpha, one verify commits on average
  E[T] = (1 - alpha^(gamma+1)) / (1 - alpha) tokens (gamma + 1 at alpha = 1);
* section "3.36 token進んでも3.36倍速いとは限らない": one iteration costs about
  gamma * t_draft + t_verify + t_overhead, so the speed-up over plain decoding
  (one target pass of t_target per token) is about E[T] * t_target / that sum;
* section "draft modelとlookahead長の選び方": a longer lookahead is not always
  better, and the number of candidates may be adjusted at run time.  The
  choice below takes, for a batch of B sequences, the gamma that maximises
  committed tokens per second, B * E[T] / iteration time, over the gammas for
  which a verify time was measured.

Only arithmetic on times measured elsewhere; no device work.
"""

from __future__ import annotations


def expected_tokens(alpha: float, gamma: int) -> float:
    """Mean tokens committed per verify, E[T], closed form."""
    if gamma < 0:
        raise ValueError("gamma must be >= 0")
    if not 0.0 <= alpha <= 1.0:
        raise ValueError("alpha must lie in [0, 1]")
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def iteration_time(gamma: int, t_draft: float, t_verify: float, t_overhead: float = 0.0) -> float:
    """gamma sequential draft steps, one verify of gamma + 1 positions, control work."""
    return gamma * t_draft + t_verify + t_overhead


def modelled_speedup(alpha: float, gamma: int, t_target: float, t_draft: float, t_verify: float,
                     t_overhead: float = 0.0) -> float:
    """E[T] * t_target / (gamma * t_draft + t_verify + t_overhead)."""
    return expected_tokens(alpha, gamma) * t_target / iteration_time(gamma, t_draft, t_verify, t_overhead)


def inter_token_latency(alpha: float, gamma: int, t_iteration: float) -> float:
    """Mean time between committed tokens of one sequence: iteration time / E[T]."""
    return t_iteration / expected_tokens(alpha, gamma)


def choose_gamma(alpha: float, batch: int, t_draft: float, t_verify_by_gamma: dict,
                 t_overhead: float = 0.0) -> dict:
    """Pick the draft length for a batch of `batch` sequences.

    t_draft: one draft step at `batch` rows; t_verify_by_gamma: {gamma: verify
    time at batch * (gamma + 1) rows}.  Times in any one unit (rates are per
    that unit).  Returns the per-gamma table (iteration time, E[T], committed
    tokens per unit time) and the best gamma (the smaller one on a tie).
    """
    if batch < 1 or not t_verify_by_gamma:
        raise ValueError("need batch >= 1 and at least one measured verify time")
    table = {}
    for g in sorted(t_verify_by_gamma):
        it = iteration_time(g, t_draft, t_verify_by_gamma[g], t_overhead)
        et = expected_tokens(alpha, g)
        table[g] = {"iteration": it, "expected_tokens": et, "tokens_per_time": batch * et / it}
    best = max(sorted(table), key=lambda g: (table[g]["tokens_per_time"], -g))
    return {"best_gamma": best, "table": table}
