"""Sensitivity of the oracle's chain to rounding-sized perturbations.

A chain of linears keeps its intermediate activations in fp16 (the stage
outputs, and in the integer modes the standardised rows that are quantized).
Two correct implementations that differ only in how they round or order fp32
arithmetic produce stage values a few fp32 ulps apart; wherever such a value
sits near an fp16 rounding boundary the two round it to neighbouring fp16
values, and from there the difference travels down the chain.

`perturbed_chain` runs the oracle's own chain steps (oracle.chain_forward's
reading, step for step) but multiplies every value a stage rounds -- the
stage's output before its fp16 rounding, and the standardised input of the
next stage -- by (1 + eps * u), u uniform on [-1, 1).  With eps at the size of
an fp32 accumulation error this measures how far the chain's output can move
for reasons that have nothing to do with a wrong kernel.  The result pins the
end-to-end bound the GPU chain tests use; it is computed from the oracle only.
"""

from __future__ import annotations

import numpy as np

from oracle import qspec_oracle as O

# Perturbation sizes: a stage output carries the error of an fp32 dot product of a few thousand
# terms (about 2^-18 relative, generous); a standardised value that of a few fp32 operations.
EPS_Y = 2.0 ** -18
EPS_NORM = 2.0 ** -22


def _stage(mode, i, v, q, s, rng, eps_y, eps_n):
    """One stage of the chain on the fp16 input v, perturbed (eps > 0) or not."""
    if mode == "w4a16":
        z = v.astype(np.float64) if i == 0 else O.standardize_rows_exact(v)
        if i > 0 and eps_n > 0:
            z = z * (1.0 + eps_n * rng.uniform(-1.0, 1.0, z.shape))
        y = z @ O.dequantize_weights(q, s).T
    else:
        if i == 0:
            z16 = v
        else:
            z = O.standardize_rows_exact(v)
            if eps_n > 0:
                z = z * (1.0 + eps_n * rng.uniform(-1.0, 1.0, z.shape))
            z16 = z.astype(np.float16)
        y = (O.linear_w4a4 if mode == "w4a4" else O.linear_w4a8)(z16, q, s)["y"]
    if eps_y > 0:
        y = y * (1.0 + eps_y * rng.uniform(-1.0, 1.0, y.shape))
    return y


def chain_pair(mode, x, layer_fn, n_layers, seed, eps_y=EPS_Y, eps_n=EPS_NORM):
    """Runs the unperturbed chain and the perturbed one side by side; layer_fn(i) returns stage i's
    (q, s) (generated on demand, so a full-size stack never has to be held).  Returns (reference
    output, perturbed output)."""
    rng = np.random.default_rng(seed)
    ref, per = x, x
    y_ref = y_per = None
    for i in range(n_layers):
        q, s = layer_fn(i)
        k = q.shape[1]
        y_ref = _stage(mode, i, np.ascontiguousarray(ref[:, :k]), q, s, rng, 0.0, 0.0)
        y_per = _stage(mode, i, np.ascontiguousarray(per[:, :k]), q, s, rng, eps_y, eps_n)
        if i + 1 < n_layers:
            ref, per = y_ref.astype(np.float16), y_per.astype(np.float16)
    return y_ref, y_per


def spread(y_ref, y_per):
    """(relative Frobenius distance, max-abs distance / rms of the reference)."""
    err = y_per - y_ref
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    return float(np.linalg.norm(err) / np.linalg.norm(y_ref)), float(np.abs(err).max()) / rms
