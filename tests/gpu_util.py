"""Helpers for GPU parity tests: moving seeded numpy inputs to the device and
the tolerance checks the parity bar fixes."""

import json
import os

import numpy as np
import torch

# Floating-point parity bar for the linear / LM-head fp32 outputs (W4A16; the integer modes are held
# bit-exact, see assert_exact).
REL_FRO = 2e-3
MAX_ABS = 1e-2
# Absolute bar for accept probabilities and the final (residual) distribution.
PROB_ABS = 1e-5
# End-to-end bound of a W4A16 chain.  Its intermediate activations are fp16 on both sides, so two
# correct implementations whose fp32 arithmetic differs round some stage values to neighbouring
# fp16 values, and those differences travel down the chain.  How far that moves the output is a
# property of the chain, measured on the oracle alone (tests/chain_sensitivity.py, recorded by
# tests/golden/make_chain_sensitivity.py and checked again on the CPU): the GPU chain is held to
# twice the largest spread recorded for its configuration, and never to less than the
# single-linear bar.
_SENSITIVITY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "chain_sensitivity.json")


def chain_bound(key: str):
    """(rel-Frobenius bound, max-abs bound in units of the reference's rms) for chain config `key`, or
    for the family of configs whose names start with `key` (the largest spread among them)."""
    with open(_SENSITIVITY) as f:
        cfg = json.load(f)["configs"]
    recs = [cfg[key]] if key in cfg else [v for k, v in cfg.items() if k.startswith(key)]
    assert recs, f"no recorded chain sensitivity for {key}"
    rel = max(r["rel_fro"] for r in recs)
    mx = max(r["max_abs_over_rms"] for r in recs)
    return max(REL_FRO, 2.0 * rel), 2.0 * mx


def assert_chain_close(y: np.ndarray, ref: np.ndarray, key: str, what: str = ""):
    rel, mx = linear_errors(y, ref)
    rb, ab = chain_bound(key)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = max(MAX_ABS, ab * rms)
    print(f"  {what}: rel_fro={rel:.3e} max_abs={mx:.3e} (bound {rb:.3e} / {bound:.3e}, {key})", flush=True)
    assert rel <= rb and mx <= bound, f"{what}: rel_fro={rel:.3e} max_abs={mx:.3e} over the {key} bound"
    return rel, mx


def assert_exact(y: np.ndarray, ref: np.ndarray, what: str = ""):
    """Integer modes: the GPU's fp32 output is the oracle's exact float64 value rounded once."""
    y = np.asarray(y)
    r32 = np.asarray(ref, dtype=np.float64).astype(np.float32)
    bad = int(np.count_nonzero(y != r32))
    assert bad == 0, (f"{what}: {bad} of {y.size} values differ from the oracle's rounded value "
                      f"(max abs {np.abs(y.astype(np.float64) - ref).max():.3e})")


# A sampling decision is tie-ambiguous when the uniform lies this close to the
# threshold the oracle computed in float64: the accept decision compares the uniform
# with the kernel's fp32 acceptance probability (errors ~1e-6), so TIE_TAU; the final
# draw runs in fp64 and misplaces only slots whose p and q agree to fp32 rounding,
# so its CDF boundaries are held to the tighter DRAW_TAU.
TIE_TAU = 1e-5
DRAW_TAU = 1e-6


def max_ambiguous(decisions: int) -> int:
    """Largest number of tie-ambiguous decisions a parity test accepts among `decisions`: a uniform
    falls within TIE_TAU of a threshold with probability about 2e-5 per decision, so more than a
    couple (plus one per thousand decisions) means a systematic difference, not ties."""
    return 2 + decisions // 1000


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def linear_errors(y: np.ndarray, ref: np.ndarray):
    err = y.astype(np.float64) - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.abs(err).max(initial=0.0))


def assert_linear_close(y: np.ndarray, ref: np.ndarray, what: str = ""):
    rel, mx = linear_errors(y, ref)
    assert rel <= REL_FRO and mx <= MAX_ABS, f"{what}: rel_fro={rel:.3e} max_abs={mx:.3e}"
    return rel, mx


def oracle_workers() -> int:
    """Threads for the oracle's chunked evaluation: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_chain(mode_name: str, x: np.ndarray, layers) -> np.ndarray:
    """The oracle's chain_forward, its stages evaluated in column chunks on oracle_workers() threads
    (one BLAS thread each): same values, a fraction of the wall time for full-size stacks."""
    from threadpoolctl import threadpool_limits

    from oracle import qspec_oracle as O
    with threadpool_limits(limits=1, user_api="blas"):
        return O.chain_forward(mode_name, x, layers, workers=oracle_workers())
