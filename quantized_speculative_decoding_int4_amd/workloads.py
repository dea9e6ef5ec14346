"""Seeded synthetic input generators.

This module only draws random inputs of the right shapes and distributions;
it contains none of the method's arithmetic (no quantization, no softmax, no
argmax, no acceptance rule).  Both the GPU path and the CPU oracle are fed the
identical bytes it produces.

Recipe (Llama-3-8B-shaped synthetic stand-in for the pages' GSM8K runs with a
trained checkpoint, neither of which is available):
  * weight codes  q ~ uniform integers in [-8, 7]           (int8 [N, K])
  * group scales  s ~ U(0.005, 0.02) rounded to fp16        (fp16 [N, K/128])
  * activations   x ~ N(0, 1) in fp32, 8 outlier channels (drawn without
    replacement, the same for every row) multiplied by 20, then rounded to fp16
  * target logits ~ N(0, sigma) fp32; draft logits = target logits +
    N(0, 0.3) noise (standard deviation 0.3)
  * uniforms      ~ U[0, 1) drawn directly in fp32 (never rounds up to 1.0)
All generators take a numpy Generator (PCG64) so each config is reproducible
from its seed.
"""

from __future__ import annotations

import numpy as np

GROUP = 128

# One Llama-3-8B-shaped decoder layer: (name, N = out features, K = in features)
LAYER_LINEARS = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)
N_LAYERS = 32
HIDDEN = 4096
VOCAB = 128256


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def int4_weights(rng: np.random.Generator, n: int, k: int,
                 s_lo: float = 0.005, s_hi: float = 0.02):
    """Logical INT4 weights: codes int8 [n, k] in [-8, 7], fp16 scales [n, k/128]."""
    assert k % GROUP == 0
    q = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    s = rng.uniform(s_lo, s_hi, size=(n, k // GROUP)).astype(np.float16)
    return q, s


def activations(rng: np.random.Generator, m: int, k: int, n_outliers: int = 8,
                outlier_scale: float = 20.0, outlier_cols=None):
    """fp16 [m, k]: N(0,1) with `n_outliers` channels scaled by `outlier_scale`
    (in fp32, before the fp16 rounding).  Returns (x, outlier column indices)."""
    x = rng.standard_normal((m, k), dtype=np.float32)
    if outlier_cols is None:
        outlier_cols = rng.choice(k, size=min(n_outliers, k), replace=False)
    x[:, outlier_cols] *= np.float32(outlier_scale)
    return x.astype(np.float16), np.asarray(outlier_cols)


def integer_case_weights(rng: np.random.Generator, n: int, k: int,
                         exponents=(-6,)):
    """Codes uniform in [-8, 7]; every scale a power of two chosen from
    `exponents` (per group).  With small-integer activations every product and
    partial sum is then exactly representable in fp32."""
    q = rng.integers(-8, 8, size=(n, k), dtype=np.int8)
    e = rng.choice(np.asarray(exponents), size=(n, k // GROUP))
    s = np.ldexp(np.ones((n, k // GROUP)), e).astype(np.float16)
    return q, s


def integer_activations(rng: np.random.Generator, m: int, k: int, lo: int = -4, hi: int = 4):
    """fp16 [m, k] holding small integers in [lo, hi]."""
    return rng.integers(lo, hi + 1, size=(m, k)).astype(np.float16)


def logits(rng: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """fp32 logits ~ N(0, sigma)."""
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def perturb(rng: np.random.Generator, base: np.ndarray, sigma: float = 0.3) -> np.ndarray:
    """base + N(0, sigma) noise in fp32 (draft logits near the target's)."""
    noise = rng.standard_normal(base.shape, dtype=np.float32) * np.float32(sigma)
    return (base.astype(np.float32) + noise).astype(np.float32)


def uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms in [0, 1)."""
    return rng.random(shape, dtype=np.float32)


def agreeing_ids(rng: np.random.Generator, reference_ids: np.ndarray, vocab: int,
                 agree_p: float = 0.96) -> np.ndarray:
    """For each position keep reference_ids[i] with probability agree_p, else
    draw uniformly from the other vocab-1 ids.  The reference ids (e.g. the
    target's Top-1 tokens) are an input; nothing is computed from logits here."""
    ref = np.asarray(reference_ids, dtype=np.int64)
    keep = rng.random(ref.shape) < agree_p
    other = rng.integers(0, vocab - 1, size=ref.shape)
    other = other + (other >= ref)          # skip the reference id
    return np.where(keep, ref, other).astype(np.int32)


def int4_weights_device(gen, n: int, k: int, device="cuda", s_lo: float = 0.005, s_hi: float = 0.02):
    """Same distribution as int4_weights, drawn on the GPU with a seeded
    torch.Generator (for the multi-GB stacks where host generation is slow)."""
    import torch
    assert k % GROUP == 0
    q = torch.randint(-8, 8, (n, k), dtype=torch.int8, device=device, generator=gen)
    s = (torch.rand((n, k // GROUP), device=device, generator=gen) * (s_hi - s_lo) + s_lo).to(torch.float16)
    return q, s


# The verify/draft pass of the Llama-3-8B-shaped stack as a chain of linears:
# per layer the fused q|k|v (N = 4096 + 1024 + 1024), o, fused gate|up
# (N = 2 * 14336) and down, then the LM-head.  Fusing q|k|v and gate|up into one
# matrix each streams exactly the same weight bytes as the separate linears.
def stack_shapes(n_layers: int = N_LAYERS):
    per_layer = [("qkv", 4096 + 1024 + 1024, HIDDEN), ("o", HIDDEN, HIDDEN),
                 ("gateup", 2 * 14336, HIDDEN), ("down", HIDDEN, 14336)]
    shapes = []
    for layer in range(n_layers):
        for name, n, k in per_layer:
            shapes.append((f"L{layer}.{name}", n, k))
    shapes.append(("lm_head", VOCAB, HIDDEN))
    return shapes
