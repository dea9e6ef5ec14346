"""Plain CPU oracle for the INT4 dual-mode linear, the LM-head and the
speculative verify/accept step of QSpec-style quantized speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
module imports nothing from the product path.

Everything here works on *logical* tensors and is written to be checked by
eye, not to be fast:
  * weight codes   q  int8  [N, K], values in [-8, 7]
  * weight scales  s  fp16  [N, K/128], one per group of 128 consecutive k
  * activations    x  fp16  [M, K]
  * logits            fp32  [rows, V]  (exactly the buffer the GPU reads)
Real arithmetic is float64, integer sums are int64.  No blocking, fusion or
reordering beyond what each definition states.

Sources (pages; each function names the section it follows):
  [P1] qiita.com, "QSpec実行時の2つの量子化による推論の一致率を調べる"
       (measuring Top-1 agreement of QSpec's two quantized modes)
  [P2] aibr.jp, summary of a paper on combining speculative decoding with
       low-bit quantization
  [P3] kasblo.com, "Speculative Decodingとは？LLM生成を速くする方法"
       (tutorial on speculative decoding)
Where the pages leave a detail open (grouping, rounding, tie rules), the
reading taken is stated at the function.
"""

from __future__ import annotations

import numpy as np

GROUP = 128  # k-elements per weight scale group (reading: symmetric INT4, group 128 along K)


# --------------------------------------------------------------------------
# Quantized linear layer, one shared INT4 weight set, two execution modes.
# [P1] sections "W4A16: 重みのみを 4-bit に量子化", "W4A4 : 重みと活性値の両方を
# 4-bit に量子化" and the mode tree in "QSpec の W4A4 モードと W4A16 モード":
# one 4-bit weight set is run either with 16-bit activations or with
# activations quantized to 4 bits at compute time.
# --------------------------------------------------------------------------

def _check_weights(q: np.ndarray, s: np.ndarray) -> tuple[int, int, int]:
    assert q.dtype == np.int8 and q.ndim == 2
    n, k = q.shape
    assert k % GROUP == 0, "K must be a multiple of the group size"
    assert s.dtype == np.float16 and s.shape == (n, k // GROUP)
    assert q.min(initial=0) >= -8 and q.max(initial=0) <= 7
    return n, k, k // GROUP


def dequantize_weights(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W[n, k] = q[n, k] * s[n, floor(k / 128)] in float64.

    Symmetric (no zero point); the scale of element (n, k) is the one of the
    128-wide group that k falls in, within the same output row n.
    """
    n, k, g = _check_weights(q, s)
    w = q.astype(np.float64).reshape(n, g, GROUP) * s.astype(np.float64)[:, :, None]
    return w.reshape(n, k)


def linear_w4a16(x: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W4A16 mode: y[m, n] = sum_k x[m, k] * W[n, k], float64.

    [P1] "W4A16" section: weights stay 4-bit in memory and are turned into
    16-bit values during the matrix product with 16-bit activations.  The
    oracle is the plain matrix product with the exact fp16 activation values.
    """
    assert x.dtype == np.float16 and x.ndim == 2
    w = dequantize_weights(q, s)
    assert x.shape[1] == w.shape[1]
    return x.astype(np.float64) @ w.T


def quantize_activations(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-token symmetric INT4 activation quantization.

    [P1] "W4A4" section says only that activations are quantized to 4 bits at
    compute time.  Reading taken (per token m):
      amax_m = max_k |x[m, k]|
      s_m    = fp16( fp32(amax_m) / 7 )   -- correctly rounded fp32 quotient,
                                             then round-to-nearest-even to fp16
      xq     = clamp(rint(x / s_m), -8, 7)   with rint = round half to even of
                                             the exact quotient
      s_m == 0 (all-zero row)  ->  xq = 0
    Exactness of the quotient: x and s_m are fp16, so an exact tie x/s = j+1/2
    is exactly representable in float64 and the float64 quotient equals it;
    away from ties the exact quotient lies at least 2**-15 from any j+1/2,
    far more than float64 rounding can move it.  So rint of the float64
    quotient is rint of the exact quotient.
    Returns xq int8 [M, K] and s fp16 [M].
    """
    assert x.dtype == np.float16 and x.ndim == 2
    amax = np.abs(x.astype(np.float32)).max(axis=1)              # exact (fp16 -> fp32)
    s32 = amax.astype(np.float32) / np.float32(7.0)              # one fp32 rounding
    s16 = s32.astype(np.float16)                                 # one fp16 rounding (RNE)
    s64 = s16.astype(np.float64)
    xq = np.zeros(x.shape, dtype=np.int8)
    nz = s64 > 0
    if nz.any():
        quot = x[nz].astype(np.float64) / s64[nz, None]
        xq[nz] = np.clip(np.rint(quot), -8, 7).astype(np.int8)
    return xq, s16


def group_accumulators(xq: np.ndarray, q: np.ndarray) -> np.ndarray:
    """acc[m, n, g] = sum_{k in group g} xq[m, k] * q[n, k], exact int64.

    The integer dot products that an int8 matrix engine accumulates in i32.
    Reading: the sums are per 128-wide group, because each group carries its
    own weight scale; a whole-K integer sum would mix scales.
    The products are formed in float64 and summed by the matrix routine: every
    product (|xq * q| <= 128 * 8) and every partial sum (|.| <= 128 * 1024 <
    2**53) is an integer that float64 holds exactly, so the result is the exact
    integer sum whatever order the routine adds in.
    """
    m, k = xq.shape
    n, k2 = q.shape
    assert k == k2 and k % GROUP == 0
    assert np.abs(xq.astype(np.int64)).max(initial=0) <= 128
    g = k // GROUP
    xg = xq.astype(np.float64).reshape(m, g, GROUP)
    qg = q.astype(np.float64).reshape(n, g, GROUP)
    acc = np.empty((m, n, g), dtype=np.int64)
    for gi in range(g):
        acc[:, :, gi] = (xg[:, gi, :] @ qg[:, gi, :].T).astype(np.int64)
    return acc


def integer_output(xq: np.ndarray, sx: np.ndarray, q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """y[m, n] = s_m * sum_g s[n, g] * acc[m, n, g] = s_m * sum_k xq[m, k] * q[n, k] * s[n, k/128],
    float64.  Written as the second form (one matrix product with the dequantized weights).  Every
    term xq * q * s is exact in float64 (at most 8 + 4 + 11 significant bits); every partial sum,
    and the product with s_m (11 bits), stays below 2**53 units of the smallest term's last bit
    while log2(K / 128) + (binades spanned by the row's scales) <= 13 -- K <= 16384 with scales in
    [0.005, 0.02] (2 binades) is well inside -- so the result is the exact value of either form,
    whatever order the matrix routine adds in."""
    return sx.astype(np.float64)[:, None] * (xq.astype(np.float64) @ dequantize_weights(q, s).T)


def linear_w4a4(x: np.ndarray, q: np.ndarray, s: np.ndarray) -> dict:
    """W4A4 mode: quantize activations per token, integer group sums, rescale.

      y[m, n] = s_m * sum_g s[n, g] * acc[m, n, g]     (float64, exact: integer_output)

    Returns dict(xq, sx, acc, y).  [P1] "W4A4" section: both weights and the
    activations are 4-bit, so a dedicated integer kernel can be used.
    """
    _check_weights(q, s)
    xq, sx = quantize_activations(x)
    acc = group_accumulators(xq, q)
    return {"xq": xq, "sx": sx, "acc": acc, "y": integer_output(xq, sx, q, s)}


# --------------------------------------------------------------------------
# W4A8: the same INT4 weights with 8-bit activations.  [P2] aibr.jp summary of
# a paper on combining speculative decoding with quantization, section
# "3.中核となる技術的要素": W4A16 and W4A8 are the weight/activation bit widths
# whose memory-traffic/compute balance the work evaluates.  The page gives no
# quantizer; the reading mirrors the W4A4 one with the int8 range.
# --------------------------------------------------------------------------

def quantize_activations_int8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-token symmetric INT8 activation quantization (reading, per token m):
      s_m = fp16( fp32(max_k |x[m, k]|) / 127 )     (fp32 quotient, then RNE to fp16)
      xq  = clamp(rint(x / s_m), -128, 127)         (round half to even of the exact quotient)
      s_m == 0  ->  xq = 0
    The float64 quotient of two fp16 values rounds to the same integer as the
    exact quotient (same argument as for the 4-bit quantizer: a non-tie lies
    at least 2**-12 from any j + 1/2 here).  Returns xq int8 [M, K], s fp16 [M].
    """
    assert x.dtype == np.float16 and x.ndim == 2
    amax = np.abs(x.astype(np.float32)).max(axis=1)
    s16 = (amax.astype(np.float32) / np.float32(127.0)).astype(np.float16)
    s64 = s16.astype(np.float64)
    xq = np.zeros(x.shape, dtype=np.int8)
    nz = s64 > 0
    if nz.any():
        quot = x[nz].astype(np.float64) / s64[nz, None]
        xq[nz] = np.clip(np.rint(quot), -128, 127).astype(np.int8)
    return xq, s16


def linear_w4a8(x: np.ndarray, q: np.ndarray, s: np.ndarray) -> dict:
    """W4A8 mode: 8-bit per-token activations, exact integer group sums, rescale
      y[m, n] = s_m * sum_g s[n, g] * acc[m, n, g]     (float64)
    Returns dict(xq, sx, acc, y)."""
    _check_weights(q, s)
    xq, sx = quantize_activations_int8(x)
    acc = group_accumulators(xq, q)
    return {"xq": xq, "sx": sx, "acc": acc, "y": integer_output(xq, sx, q, s)}


def lm_head(mode: str, x: np.ndarray, q: np.ndarray, s: np.ndarray,
            chunk: int = 8192) -> np.ndarray:
    """LM-head logits: the same linear (mode 'w4a16', 'w4a4' or 'w4a8') with N = vocab.

    Processed in chunks of output rows only to bound memory; each chunk is the
    same definition as the full linear.  Returns float64 [M, V].
    """
    n = q.shape[0]
    out = np.empty((x.shape[0], n), dtype=np.float64)
    if mode in ("w4a4", "w4a8"):
        # one activation quantization for the whole row, shared by all chunks
        xq, sx = quantize_activations(x) if mode == "w4a4" else quantize_activations_int8(x)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        if mode == "w4a16":
            out[:, lo:hi] = linear_w4a16(x, q[lo:hi], s[lo:hi])
        elif mode in ("w4a4", "w4a8"):
            out[:, lo:hi] = integer_output(xq, sx, q[lo:hi], s[lo:hi])
        else:
            raise ValueError(mode)
    return out


def standardize_rows_exact(v: np.ndarray) -> np.ndarray:
    """Row-wise (v - mean) / std over the columns given (population std), in
    float64 and NOT rounded; a row with zero spread maps to zeros.

    Reading (the pages give no layer internals): this stands in for the
    normalisation between the linears of the synthetic stack, like a layer norm
    without learned affine parameters.  It keeps activations well scaled over
    many stages for weight codes uniform on [-8, 7], whose mean of -0.5 would
    otherwise amplify the all-ones direction stage after stage."""
    v64 = np.asarray(v, dtype=np.float64)
    mu = v64.mean(axis=1, keepdims=True)
    sd = np.sqrt(((v64 - mu) ** 2).mean(axis=1, keepdims=True))
    out = np.zeros_like(v64)
    ok = sd[:, 0] > 0
    out[ok] = (v64[ok] - mu[ok]) / sd[ok]
    return out


def standardize_rows(v: np.ndarray) -> np.ndarray:
    """standardize_rows_exact, then rounded to fp16 (round to nearest even,
    directly from float64): the 16-bit input that the integer modes quantize."""
    return standardize_rows_exact(v).astype(np.float16)


def _by_column_chunks(fn, n: int, workers: int, chunk: int = 2048) -> np.ndarray:
    """[M, n] result of fn(lo, hi) (the output columns lo..hi-1) evaluated chunk by chunk, `workers`
    chunks at a time on threads.  Each output column is computed by the same definition whatever
    the chunk, so the chunking only bounds memory and time."""
    spans = [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]
    if workers <= 1 or len(spans) == 1:
        return np.concatenate([fn(lo, hi) for lo, hi in spans], axis=1)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return np.concatenate(list(ex.map(lambda sp: fn(*sp), spans)), axis=1)


def chain_forward(mode: str, x: np.ndarray, layers, workers: int = 1) -> np.ndarray:
    """One forward pass of a stack of quantized linears in one mode.

    Reading for the synthetic stack (the pages give no layer internals):
    stage 0 reads x; stage i > 0 reads v = the first K_i columns of the
    previous stage's output, kept as fp16 (rounded to nearest even from the
    float64 value), and standardises each row of v; the last stage's output is
    returned unrounded (float64).  layers: sequence of (q, s).
      * W4A16 (verify): the 16-bit activations entering the product are the
        fp16 stage outputs v themselves; the row standardisation is an affine
        map of each row, applied exactly (standardize_rows_exact, no rounding):
            y[m, n] = sum_k ((v[m, k] - mu_m) / sd_m) * W[n, k]
      * W4A4 / W4A8 (draft): the standardised row is rounded to fp16
        (standardize_rows) and that 16-bit row is quantized per token as in
        the single linear of the mode.
    [P3] "draft modelとtarget modelの処理フロー": a pass scores all of its rows
    (candidate positions) at once.  workers > 1 evaluates each stage's output
    columns in chunks on that many threads (same values, see _by_column_chunks).
    """
    cur = x
    n_layers = len(layers)
    y = None
    for i, layer in enumerate(layers):
        q, s = layer[0], layer[1]
        k = q.shape[1]
        v = np.ascontiguousarray(cur[:, :k])
        if mode == "w4a16":
            z = v.astype(np.float64) if i == 0 else standardize_rows_exact(v)
            y = _by_column_chunks(lambda lo, hi: z @ dequantize_weights(q[lo:hi], s[lo:hi]).T, q.shape[0], workers)
        elif mode in ("w4a4", "w4a8"):
            z16 = v if i == 0 else standardize_rows(v)
            xq, sx = (quantize_activations if mode == "w4a4" else quantize_activations_int8)(z16)
            y = _by_column_chunks(lambda lo, hi: integer_output(xq, sx, q[lo:hi], s[lo:hi]), q.shape[0], workers)
        else:
            raise ValueError(mode)
        if i + 1 < n_layers:
            cur = y.astype(np.float16)
    return y


# --------------------------------------------------------------------------
# Next-token distributions and Top-1.
# [P3] "通常のLLM生成はなぜ逐次処理になるのか": the model gives a distribution
# over the next token; [P1] "結果": each mode's Top-1 token and the probability
# it assigns to it.
# --------------------------------------------------------------------------

def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """p[r, j] = exp(l[r, j] - max_r) / sum_j exp(l[r, j] - max_r), float64.

    Temperature 1, no top-k/top-p (the pages give no sampling knobs)."""
    l64 = np.asarray(logits, dtype=np.float64)
    mx = l64.max(axis=-1, keepdims=True)
    e = np.exp(l64 - mx)
    return e / e.sum(axis=-1, keepdims=True)


def top1(logits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Top-1 token per row (lowest index among equal maxima, as np.argmax)
    and its probability 1 / sum_j exp(l_j - l_max)."""
    l64 = np.asarray(logits, dtype=np.float64)
    t = np.argmax(l64, axis=-1).astype(np.int64)
    mx = l64.max(axis=-1, keepdims=True)
    prob = 1.0 / np.exp(l64 - mx).sum(axis=-1)
    return t, prob


# --------------------------------------------------------------------------
# Verification.  [P3] "draft modelとtarget modelの処理フロー": the target scores
# the gamma draft positions plus the next one; candidates are checked left to
# right, the first mismatch/rejection stops the scan, later candidates are
# dropped, and the new prefix starts the next iteration.
# --------------------------------------------------------------------------

def verify_greedy(tgt_logits: np.ndarray, draft_ids: np.ndarray) -> dict:
    """Greedy prefix-match acceptance.

    [P3] "greedy decodingでは一致するprefixを採用する": accept draft tokens while
    they equal the target's argmax; at the first mismatch take the target's
    token; if all gamma match, the extra position adds a bonus token, so
    1..gamma+1 tokens are committed per verify.  [P1] "Speculative Decoding":
    a rejected draft token is replaced by the target's own prediction.

    tgt_logits fp32 [B, gamma+1, V]; draft_ids int [B, gamma].  Draft ids
    outside [0, V) never equal an argmax, so they count as mismatches.
    Returns dict(t [B, gamma+1], top1_prob [B, gamma+1], n_accept [B],
    out_tokens [B, gamma+1] padded with -1).
    """
    b, gp1, v = tgt_logits.shape
    t, prob = top1(tgt_logits.reshape(b * gp1, v))
    t = t.reshape(b, gp1)
    prob = prob.reshape(b, gp1)
    acc = greedy_accept(t, draft_ids)
    return {"t": t, "top1_prob": prob, "n_accept": acc["n_accept"], "out_tokens": acc["out_tokens"]}


def greedy_accept(t: np.ndarray, draft_ids: np.ndarray) -> dict:
    """The prefix rule of greedy verification on the target's Top-1 ids t [B, gamma+1]
    ([P3] "greedy decodingでは一致するprefixを採用する"): draft token i is accepted while it and
    every draft token before it equal the target's Top-1 at their positions; the first mismatch
    (or the position after the last draft token) contributes the target's own Top-1.  A negative
    t (no Top-1) equals no draft token.  Returns dict(n_accept [B], out_tokens [B, gamma+1]
    padded with -1)."""
    t = np.asarray(t, dtype=np.int64)
    b, gp1 = t.shape
    gamma = gp1 - 1
    d = np.asarray(draft_ids, dtype=np.int64).reshape(b, gamma)
    n_accept = np.zeros(b, dtype=np.int64)
    out = np.full((b, gp1), -1, dtype=np.int64)
    for bi in range(b):
        n = 0
        while n < gamma and t[bi, n] >= 0 and d[bi, n] == t[bi, n]:
            n += 1
        out[bi, :n] = d[bi, :n]
        out[bi, n] = t[bi, n]
        n_accept[bi] = n
    return {"n_accept": n_accept, "out_tokens": out}


def acceptance_probability(p_x: float, q_x: float) -> float:
    """a(x) = min(1, p(x) / q(x))  ([P3] "samplingでもtargetの確率分布を保つ",
    acceptance equation).  Edge readings: p(x) = 0 -> 0; q(x) = 0 < p(x) -> 1."""
    if p_x <= 0.0:
        return 0.0
    if q_x <= 0.0:
        return 1.0
    return min(1.0, p_x / q_x)


def residual_distribution(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """p'(x) = max(0, p(x) - q(x)) / sum_y max(0, p(y) - q(y))
    ([P3] same section, residual-distribution equation).  If the sum is 0
    (impossible after a rejection in exact arithmetic) fall back to p."""
    r = np.maximum(0.0, p - q)
    z = r.sum()
    if z > 0.0:
        return r / z
    return p.copy()


def sample_inverse_cdf(f: np.ndarray, u: float) -> int:
    """Smallest j with sum_{k<=j} f_k > u (u in [0, 1)).  If rounding leaves
    no such j, the last j with f_j > 0.  (Reading: inverse-CDF sampling with a
    uniform passed in.)"""
    cdf = np.cumsum(f)
    hit = np.nonzero(cdf > u)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(f > 0)[0][-1])


def verify_sample(tgt_logits: np.ndarray, drf_logits: np.ndarray,
                  draft_ids: np.ndarray, u_acc: np.ndarray,
                  u_fin: np.ndarray) -> dict:
    """Sampling acceptance with residual resampling.

    [P3] "samplingでもtargetの確率分布を保つ" and its 3-token worked example:
      p_i = softmax(target logits row i), i = 0..gamma
      q_i = softmax(draft logits row i),  i = 0..gamma-1
      a_i = min(1, p_i(d_i) / q_i(d_i)) for every i < gamma
      n   = first i with u_acc[i] >= a_i (accept iff u < a), else gamma
      f   = normalised max(0, p_n - q_n) if n < gamma, else p_gamma
      final token = inverse CDF of f at u_fin
      out = d_0 .. d_{n-1}, final token, then -1 padding
    Draft ids outside [0, V) get a = 0.  Returns dict(accept_prob [B, gamma],
    n_accept [B], out_tokens [B, gamma+1], final_dist [B, V], cdf [B, V]).
    """
    b, gp1, v = tgt_logits.shape
    gamma = gp1 - 1
    d = np.asarray(draft_ids, dtype=np.int64).reshape(b, gamma)
    u_acc = np.asarray(u_acc, dtype=np.float64).reshape(b, gamma)
    u_fin = np.asarray(u_fin, dtype=np.float64).reshape(b)
    p = softmax_rows(tgt_logits)                       # [B, gamma+1, V]
    q = softmax_rows(drf_logits) if gamma > 0 else np.zeros((b, 0, v))
    accept_prob = np.zeros((b, gamma), dtype=np.float64)
    n_accept = np.zeros(b, dtype=np.int64)
    out = np.full((b, gp1), -1, dtype=np.int64)
    final = np.zeros((b, v), dtype=np.float64)
    for bi in range(b):
        for i in range(gamma):
            di = d[bi, i]
            if 0 <= di < v:
                accept_prob[bi, i] = acceptance_probability(p[bi, i, di], q[bi, i, di])
        n = 0
        while n < gamma and u_acc[bi, n] < accept_prob[bi, n]:
            n += 1
        if n < gamma:
            f = residual_distribution(p[bi, n], q[bi, n])
        else:
            f = p[bi, gamma]
        out[bi, :n] = d[bi, :n]
        out[bi, n] = sample_inverse_cdf(f, u_fin[bi])
        n_accept[bi] = n
        final[bi] = f
    return {"accept_prob": accept_prob, "n_accept": n_accept,
            "out_tokens": out, "final_dist": final,
            "cdf": np.cumsum(final, axis=1)}


# --------------------------------------------------------------------------
# Tree-shaped greedy verification.  [P2] aibr.jp summary, section
# "3.中核となる技術的要素": verification can expand into a tree of candidates
# (several branches scored in one target pass).  The page gives no rule; the
# reading is the greedy prefix rule of [P3] "greedy decodingでは一致するprefixを
# 採用する" applied along every root-to-node path.
# --------------------------------------------------------------------------

def verify_tree_greedy(tgt_logits: np.ndarray, tokens: np.ndarray, parent: np.ndarray) -> dict:
    """Greedy acceptance over a tree of draft tokens per sequence.

    tgt_logits fp32 [B, T, V]: row t is the target's next-token scores after
    node t; node 0 is the root (the last committed token).  tokens [B, T]: the
    draft token of node t >= 1 (tokens[:, 0] unused).  parent [B, T]: the
    parent of node t >= 1, valid only in [0, t) (parent[:, 0] unused).
    Node t >= 1 is accepted iff its parent is valid and accepted and tokens[t]
    equals the target's Top-1 (first maximal index) of row parent[t]; the root
    is accepted.  The deepest accepted node wins, the lowest index on equal
    depth.  Committed: the tokens along the root-to-winner path, then the
    target's Top-1 at the winner.
    Returns dict(t [B, T], n_accept [B], out_tokens [B, T], out_nodes [B, T]),
    out_* padded with -1; out_nodes lists the accepted path's nodes (root
    excluded).
    """
    b_, t_, v_ = tgt_logits.shape
    top = np.empty((b_, t_), dtype=np.int64)
    for b in range(b_):
        top[b], _ = top1(tgt_logits[b])
    n_acc = np.zeros(b_, dtype=np.int64)
    out = np.full((b_, t_), -1, dtype=np.int64)
    nodes = np.full((b_, t_), -1, dtype=np.int64)
    for b in range(b_):
        acc = [True] + [False] * (t_ - 1)
        depth = [0] * t_
        for t in range(1, t_):
            p = int(parent[b, t])
            if 0 <= p < t and acc[p] and int(tokens[b, t]) == int(top[b, p]):
                acc[t] = True
                depth[t] = depth[p] + 1
        win = 0
        for t in range(1, t_):
            if acc[t] and depth[t] > depth[win]:
                win = t
        path = []
        node = win
        while node != 0:
            path.append(node)
            node = int(parent[b, node])
        path.reverse()
        n_acc[b] = len(path)
        for i, node in enumerate(path):
            out[b, i] = tokens[b, node]
            nodes[b, i] = node
        out[b, len(path)] = top[b, win]
    return {"t": top, "n_accept": n_acc, "out_tokens": out, "out_nodes": nodes}


# --------------------------------------------------------------------------
# Closed forms used as pins ([P3] "1回のtarget検証で何token進むか").
# --------------------------------------------------------------------------

def expected_tokens(alpha: float, gamma: int) -> float:
    """E[T] = 1 + alpha + ... + alpha**gamma, tokens committed per verify when
    each candidate is accepted independently with probability alpha."""
    return float(sum(alpha ** i for i in range(gamma + 1)))


def overlap_mass(p: np.ndarray, q: np.ndarray) -> float:
    """beta = sum_x min(p(x), q(x)): probability that a draft x ~ q is accepted
    under a(x) = min(1, p/q)."""
    return float(np.minimum(p, q).sum())


def accept_length_distribution(betas: list[float]) -> np.ndarray:
    """P(n = k), k = 0..gamma, for independent per-position acceptance
    probabilities beta_0..beta_{gamma-1}: prod_{i<k} beta_i * (1 - beta_k) for
    k < gamma, and prod_{i<gamma} beta_i for k = gamma."""
    gamma = len(betas)
    out = np.zeros(gamma + 1)
    run = 1.0
    for k in range(gamma):
        out[k] = run * (1.0 - betas[k])
        run *= betas[k]
    out[gamma] = run
    return out


def speedup_model(e_t: float, t_target: float, t_draft: float, gamma: int,
                  t_verify: float, t_overhead: float = 0.0) -> float:
    """Rough speedup of one iteration over plain decoding ([P3] "3.36 token進んでも
    3.36倍速いとは限らない"): E[T] * t_target / (gamma*t_draft + t_verify + t_overhead)."""
    return e_t * t_target / (gamma * t_draft + t_verify + t_overhead)
