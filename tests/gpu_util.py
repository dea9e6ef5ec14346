"""Helpers for GPU parity tests: moving seeded numpy inputs to the device and
the tolerance checks the parity bar fixes."""

import numpy as np
import torch

# Floating-point parity bar for the linear / LM-head fp32 outputs.
REL_FRO = 2e-3
MAX_ABS = 1e-2
# Absolute bar for accept probabilities and the final (residual) distribution.
PROB_ABS = 1e-5
# A chain of n linears keeps its intermediate activations in fp16 (unit roundoff
# u = 2^-11) on both sides.  Once the two sides differ by any rounding, a value near
# an fp16 rounding boundary lands one ulp (2u) apart; such flips enter every stage
# and add up like a random walk, so the end-to-end relative error of a chain grows
# as about 2u * sqrt(n).  The oracle always runs the whole chain from the shared
# inputs; no GPU output is fed back into it.
FP16_U = 2.0 ** -11


def chain_rel_tolerance(n_stages: int) -> float:
    return max(REL_FRO, 2.0 * FP16_U * float(np.sqrt(n_stages)))


# A sampling decision is tie-ambiguous when the uniform lies this close to the
# threshold the oracle computed in float64 (fp32 errors of the kernel are ~1e-6).
TIE_TAU = 1e-5


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
