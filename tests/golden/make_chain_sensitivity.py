"""Writes tests/golden/chain_sensitivity.json: how far the oracle's W4A16 chain
output moves when every value a stage rounds carries an fp32-sized relative
perturbation (tests/chain_sensitivity.py), for the chains the GPU tests run end
to end.  Calls only the oracle and the seeded input generators.

    python tests/golden/make_chain_sensitivity.py

The GPU chain tests hold the kernels to twice the largest spread recorded here
(rel-Frobenius, and max-abs in units of the reference's rms).  Takes about 20
minutes on 8 cores (the full Llama-3-8B-shaped stack in float64).
"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from quantized_speculative_decoding_int4_amd import workloads as W  # noqa: E402
from tests import chain_sensitivity as CS  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "chain_sensitivity.json")


def llama_stack(seed, head_rows=3000):
    """Layer generator for the 32-layer stack + LM-head restricted to head_rows sampled vocabulary rows."""
    shapes = W.stack_shapes()
    rng = W.rng_for(seed)
    cols = np.sort(rng.choice(W.VOCAB, size=head_rows, replace=False))

    def layer(i):
        name, n, k = shapes[i]
        lr = W.rng_for(seed * 1000 + i)
        if name == "lm_head":
            return W.int4_weights(lr, head_rows, k)  # the head's rows are independent of each other
        return W.int4_weights(lr, n, k)

    return layer, len(shapes)


def small_long_chain(seed):
    shapes = [(384, 256), (256, 384)] * 37 + [(1000, 256)]
    rng = W.rng_for(seed)
    layers = [W.int4_weights(rng, n, k) for n, k in shapes]
    return (lambda i: layers[i]), len(layers), 256


def small_llama_like(seed):
    h, inter = 512, 1024
    shapes = [(h + 256, h), (h, h), (2 * inter, h), (h, inter)] * 2 + [(3000, h)]
    rng = W.rng_for(seed)
    layers = [W.int4_weights(rng, n, k) for n, k in shapes]
    return (lambda i: layers[i]), len(layers), h


def measure(name, make, rows, seeds, mode="w4a16"):
    worst = [0.0, 0.0]
    runs = []
    for sd in seeds:
        t0 = time.time()
        fn, n, k0 = make(sd)
        x, _ = W.activations(W.rng_for(10_000 + sd), rows, k0)
        y_ref, y_per = CS.chain_pair(mode, x, fn, n, seed=sd)
        rel, mx = CS.spread(y_ref, y_per)
        runs.append({"seed": sd, "rel_fro": rel, "max_abs_over_rms": mx})
        worst = [max(worst[0], rel), max(worst[1], mx)]
        print(f"{name} seed {sd}: rel {rel:.3e} max/rms {mx:.3e} ({time.time() - t0:.0f} s)", flush=True)
    return {"mode": mode, "rows": rows, "stages": n, "eps_y": CS.EPS_Y, "eps_norm": CS.EPS_NORM,
            "rel_fro": worst[0], "max_abs_over_rms": worst[1], "runs": runs}


def main():
    res = {}
    for m in (1, 2, 4, 12, 16):
        res[f"long75_m{m}"] = measure(f"long75_m{m}", small_long_chain, m, seeds=(1, 2, 3))
    for m in (4, 12, 20, 70, 256):
        res[f"small_llama_m{m}"] = measure(f"small_llama_m{m}", small_llama_like, m, seeds=(1, 2, 3))
    for m in (4, 128):
        res[f"llama_full_m{m}"] = measure(f"llama_full_m{m}", lambda sd: (*llama_stack(sd), W.HIDDEN), m,
                                          seeds=(1, 2))
    with open(OUT, "w") as f:
        json.dump({"what": "spread of the oracle's W4A16 chain under fp32-sized perturbations of every rounded "
                           "value; max over seeds",
                   "script": "tests/golden/make_chain_sensitivity.py", "configs": res}, f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
