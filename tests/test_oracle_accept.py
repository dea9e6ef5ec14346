"""Pins for the oracle's softmax/Top-1, greedy and sampling acceptance against
what the pages print (worked examples under tests/golden/), closed forms,
brute-force enumeration and Monte Carlo."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import qspec_oracle as O
from quantized_speculative_decoding_int4_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _log_fp32(p):
    """fp32 logits whose softmax is p (the buffer a verify kernel would read)."""
    return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


# ---------------------------------------------------------------- softmax / Top-1

def test_top1_equal_logits_uniform_lowest_index():
    lg = np.zeros((2, 7), dtype=np.float32)
    t, prob = O.top1(lg)
    assert t.tolist() == [0, 0]
    assert np.allclose(prob, 1 / 7, rtol=0, atol=1e-15)
    assert np.allclose(O.softmax_rows(lg), 1 / 7, rtol=0, atol=1e-15)


def test_top1_ties_lowest_index_and_known_probs():
    p = np.array([0.1, 0.35, 0.2, 0.35])
    t, prob = O.top1(_log_fp32(p)[None])
    assert t[0] == 1
    assert abs(prob[0] - 0.35) < 1e-7
    assert np.allclose(O.softmax_rows(_log_fp32(p)), p, atol=1e-7)


def test_softmax_shift_invariance():
    rng = W.rng_for(21)
    lg = W.logits(rng, (3, 50), sigma=4.0)
    assert np.allclose(O.softmax_rows(lg), O.softmax_rows(lg + np.float32(100.0)), atol=1e-12)


# ---------------------------------------------------------------- greedy

def _onehot_logits(t_ids, v):
    lg = np.zeros((len(t_ids), v), dtype=np.float32)
    for i, t in enumerate(t_ids):
        lg[i, t] = 1.0
    return lg


def test_greedy_worked_examples():
    for case in _golden("greedy_examples.json")["cases"]:
        vocab = case["vocab"]
        ids = {w: i for i, w in enumerate(vocab)}
        d = np.array([[ids[w] for w in case["draft"]]])
        tg = _onehot_logits([ids[w] for w in case["target_argmax"]], len(vocab))[None]
        r = O.verify_greedy(tg, d)
        assert r["n_accept"][0] == case["n_accept"]
        committed = [vocab[i] for i in r["out_tokens"][0] if i >= 0]
        assert committed == case["committed"]
        assert all(i == -1 for i in r["out_tokens"][0][len(committed):])


def test_greedy_brute_force_v3():
    """All (draft, target-argmax) pairs over a 3-token vocab, gamma <= 3."""
    v = 3
    for gamma in range(0, 4):
        for t_ids in itertools.product(range(v), repeat=gamma + 1):
            lg = _onehot_logits(t_ids, v)[None]
            drafts = list(itertools.product(range(v), repeat=gamma))
            for d_ids in drafts:
                r = O.verify_greedy(lg, np.array([d_ids], dtype=np.int64).reshape(1, gamma))
                # independent statement: length of the common prefix
                n = 0
                for a, b in zip(d_ids, t_ids):
                    if a != b:
                        break
                    n += 1
                assert r["n_accept"][0] == n
                expect = list(d_ids[:n]) + [t_ids[n]] + [-1] * (gamma - n)
                assert r["out_tokens"][0].tolist() == expect


def test_greedy_accept_from_top1_ids_brute_force():
    """The prefix rule on Top-1 ids (the fused path), over all ids in {-1, 0, 1} for gamma <= 3: the
    common prefix of draft and target ids, where a missing target id (-1) matches nothing, not even
    a -1 draft id."""
    ids = (-1, 0, 1)
    for gamma in range(0, 4):
        for t_ids in itertools.product(ids, repeat=gamma + 1):
            for d_ids in itertools.product(ids, repeat=gamma):
                r = O.greedy_accept(np.array([t_ids]), np.array([d_ids], dtype=np.int64).reshape(1, gamma))
                n = next((i for i in range(gamma) if t_ids[i] < 0 or d_ids[i] != t_ids[i]), gamma)
                assert r["n_accept"][0] == n
                assert r["out_tokens"][0].tolist() == list(d_ids[:n]) + [t_ids[n]] + [-1] * (gamma - n)


def test_greedy_out_of_range_draft_ids_mismatch():
    lg = _onehot_logits([2, 0, 1], 4)[None]
    r = O.verify_greedy(lg, np.array([[-1, 0]]))
    assert r["n_accept"][0] == 0 and r["out_tokens"][0].tolist() == [2, -1, -1]
    r = O.verify_greedy(lg, np.array([[2, 4]]))
    assert r["n_accept"][0] == 1 and r["out_tokens"][0].tolist() == [2, 0, -1]


def test_greedy_monte_carlo_expected_tokens():
    """Bernoulli(alpha) agreement per position -> mean committed = E[T]."""
    g = _golden("expected_tokens.json")["cases"][0]
    gamma, alpha = g["gamma"], g["alpha"]
    rng = W.rng_for(22)
    b, v = 200000, 5
    t_ids = rng.integers(0, v, size=(b, gamma + 1))
    lg = np.full((b, gamma + 1, v), -1.0, dtype=np.float32)
    np.put_along_axis(lg, t_ids[..., None], 1.0, axis=2)
    d = W.agreeing_ids(rng, t_ids[:, :gamma], v, agree_p=alpha)
    r = O.verify_greedy(lg, d)
    mean_t = (r["n_accept"] + 1).mean()
    sd = np.sqrt(((r["n_accept"] + 1) - mean_t).var())
    assert abs(mean_t - g["expected_tokens"]) <= 4 * sd / np.sqrt(b)


# ---------------------------------------------------------------- E[T] closed form

def test_expected_tokens_closed_form():
    for c in _golden("expected_tokens.json")["cases"]:
        assert abs(O.expected_tokens(c["alpha"], c["gamma"]) - c["expected_tokens"]) < 1e-12
    for alpha in (0.3, 0.8, 0.96):
        for gamma in (1, 3, 7):
            geo = (1 - alpha ** (gamma + 1)) / (1 - alpha)
            assert abs(O.expected_tokens(alpha, gamma) - geo) < 1e-12


def test_speedup_model_reduces_to_expected_tokens():
    assert abs(O.speedup_model(3.3616, 1.0, 0.0, 4, 1.0) - 3.3616) < 1e-12


# ---------------------------------------------------------------- sampling: A/B/C example

def test_abc_accept_probability_and_residual():
    g = _golden("abc_example.json")
    lp = _log_fp32(g["p_target"])
    lq = _log_fp32(g["q_draft"])
    tg = np.stack([lp, lp])[None]          # gamma = 1: rows p_0 (checked) and p_1 (bonus)
    dr = lq[None, None]
    a_idx = g["tokens"].index(g["proposed"])
    # accepted (u < 0.75)
    r = O.verify_sample(tg, dr, np.array([[a_idx]]), np.array([[0.5]]), np.array([0.1]))
    assert abs(r["accept_prob"][0, 0] - g["accept_probability"]) < 1e-6
    assert r["n_accept"][0] == 1 and r["out_tokens"][0, 0] == a_idx
    assert abs(g["q_draft"][a_idx] * r["accept_prob"][0, 0] - g["proposed_and_accepted"]) < 1e-6
    # rejected (u >= 0.75): residual (0, 0.1, 0) normalised -> B for every u_fin
    res_tok = g["tokens"].index(g["residual_token"])
    expect_res = np.array(g["residual_unnormalised"]) / sum(g["residual_unnormalised"])
    for u_fin in (0.0, 0.3, 0.999):
        r = O.verify_sample(tg, dr, np.array([[a_idx]]), np.array([[0.9]]), np.array([u_fin]))
        assert r["n_accept"][0] == 0
        assert r["out_tokens"][0].tolist() == [res_tok, -1]
        assert np.allclose(r["final_dist"][0], expect_res, atol=1e-6)


def _first_token_distribution(lp, lq, grid):
    """Enumerate draft d ~ q (weight q(d)) and (u_acc, u_fin) on a midpoint
    grid; return the distribution of the first committed token (gamma = 1)."""
    v = lp.shape[0]
    q = O.softmax_rows(lq)
    us = (np.arange(grid) + 0.5) / grid
    dist = np.zeros(v)
    tg = np.stack([lp, lp])[None]
    dr = lq[None, None]
    for d in range(v):
        for ua in us:
            for uf in us:
                r = O.verify_sample(tg, dr, np.array([[d]]), np.array([[ua]]), np.array([uf]))
                dist[r["out_tokens"][0, 0]] += q[d] / grid ** 2
    return dist


def test_abc_final_distribution_by_enumeration():
    g = _golden("abc_example.json")
    dist = _first_token_distribution(_log_fp32(g["p_target"]), _log_fp32(g["q_draft"]), grid=40)
    assert np.allclose(dist, g["final_distribution"], atol=2 / 40)


def test_distribution_preserved_random_pairs():
    rng = W.rng_for(23)
    for _ in range(2):
        lp = W.logits(rng, (3,), sigma=1.5)
        lq = W.logits(rng, (3,), sigma=1.5)
        dist = _first_token_distribution(lp, lq, grid=40)
        assert np.allclose(dist, O.softmax_rows(lp), atol=2 / 40)


def test_accept_length_distribution_gamma2_enumeration():
    """P(n = k) for gamma = 2 against prod beta_i (1 - beta_k), by enumeration of
    draft ids (weight q) and u_acc on a midpoint grid; the token committed after
    an accepted d_0 follows p_1."""
    rng = W.rng_for(24)
    v, gamma, grid = 3, 2, 24
    lp = W.logits(rng, (gamma + 1, v), sigma=1.2)
    lq = W.logits(rng, (gamma, v), sigma=1.2)
    p = O.softmax_rows(lp)
    q = O.softmax_rows(lq)
    betas = [O.overlap_mass(p[i], q[i]) for i in range(gamma)]
    us = (np.arange(grid) + 0.5) / grid
    pn = np.zeros(gamma + 1)
    second = np.zeros(v)
    second_mass = 0.0
    for d0 in range(v):
        for d1 in range(v):
            w = q[0, d0] * q[1, d1]
            for u0 in us:
                for u1 in us:
                    for uf in us:
                        r = O.verify_sample(lp[None], lq[None], np.array([[d0, d1]]),
                                            np.array([[u0, u1]]), np.array([uf]))
                        wt = w / grid ** 3
                        n = r["n_accept"][0]
                        pn[n] += wt
                        if n >= 1:
                            second[r["out_tokens"][0, 1]] += wt
                            second_mass += wt
    assert np.allclose(pn, O.accept_length_distribution(betas), atol=3 * gamma / grid)
    assert np.allclose(second / second_mass, p[1], atol=4 / grid)


def test_pointwise_identity_and_residual_support():
    rng = W.rng_for(25)
    for _ in range(5):
        p = O.softmax_rows(W.logits(rng, (50,), sigma=2.0))
        q = O.softmax_rows(W.logits(rng, (50,), sigma=2.0))
        beta = O.overlap_mass(p, q)
        a = np.array([O.acceptance_probability(p[x], q[x]) for x in range(50)])
        f = O.residual_distribution(p, q)
        assert np.allclose(q * a + (1 - beta) * f, p, atol=1e-12)
        assert abs(f.sum() - 1) < 1e-12
        assert np.all(f[p <= q] == 0)


def test_acceptance_probability_edges():
    assert O.acceptance_probability(0.0, 0.3) == 0.0
    assert O.acceptance_probability(0.2, 0.0) == 1.0
    assert O.acceptance_probability(0.6, 0.3) == 1.0
    assert O.acceptance_probability(0.3, 0.6) == 0.5


def test_sampling_gamma0_is_plain_inverse_cdf():
    p = np.array([0.25, 0.5, 0.25])
    lp = _log_fp32(p)[None, None]
    for u, tok in ((0.1, 0), (0.3, 1), (0.74, 1), (0.76, 2)):
        r = O.verify_sample(lp, np.zeros((1, 0, 3), np.float32), np.zeros((1, 0), np.int64),
                            np.zeros((1, 0)), np.array([u]))
        assert r["out_tokens"][0].tolist() == [tok] and r["n_accept"][0] == 0


def test_sampling_out_of_range_draft_rejected():
    p = np.array([0.2, 0.5, 0.3])
    lp = np.stack([_log_fp32(p)] * 2)[None]
    lq = _log_fp32([0.3, 0.3, 0.4])[None, None]
    r = O.verify_sample(lp, lq, np.array([[5]]), np.array([[0.0]]), np.array([0.5]))
    assert r["accept_prob"][0, 0] == 0 and r["n_accept"][0] == 0


@pytest.mark.slow
def test_sampling_monte_carlo_expected_tokens():
    """gamma = 4, p = (0.2, 0.6, 0.2), q = (0.4, 0.4, 0.2): beta = 0.8 at every
    position, drafts drawn from q -> mean committed tokens = E[T] = 3.3616."""
    g = _golden("expected_tokens.json")["cases"][0]
    gamma = g["gamma"]
    p = np.array([0.2, 0.6, 0.2])
    q = np.array([0.4, 0.4, 0.2])
    assert abs(O.overlap_mass(p, q) - g["alpha"]) < 1e-12
    rng = W.rng_for(26)
    b = 300000
    lp = np.broadcast_to(_log_fp32(p), (b, gamma + 1, 3)).copy()
    lq = np.broadcast_to(_log_fp32(q), (b, gamma, 3)).copy()
    # drafts ~ q by inverse CDF on separate uniforms
    ud = rng.random((b, gamma))
    d = np.searchsorted(np.cumsum(q), ud, side="right")
    r = O.verify_sample(lp, lq, d, W.uniforms(rng, (b, gamma)), W.uniforms(rng, (b,)))
    t = r["n_accept"] + 1
    se = t.std() / np.sqrt(b)
    assert abs(t.mean() - g["expected_tokens"]) <= 4 * se


def test_bonus_token_follows_last_target_row():
    """All gamma candidates accepted -> the extra token is drawn from p_gamma
    (the target's extra position), not from an earlier row."""
    p_rows = np.array([[0.2, 0.6, 0.2], [0.5, 0.3, 0.2], [0.7, 0.1, 0.2]])
    lp = _log_fp32(p_rows)[None]
    lq = _log_fp32(p_rows[:2])[None]        # q = p: every draft is accepted (a = 1)
    grid = 200
    dist = np.zeros(3)
    for uf in (np.arange(grid) + 0.5) / grid:
        r = O.verify_sample(lp, lq, np.array([[1, 0]]), np.array([[0.99, 0.99]]), np.array([uf]))
        assert r["n_accept"][0] == 2
        dist[r["out_tokens"][0, 2]] += 1 / grid
    assert np.allclose(dist, p_rows[2], atol=2 / grid)
    # greedy: bonus is the argmax of the last row
    r = O.verify_greedy(lp, np.array([[1, 0]]))
    assert r["out_tokens"][0].tolist() == [1, 0, 0]


# ---------------------------------------------------------------- tree-shaped greedy verification

def _tree_brute(top, tokens, parent):
    """Independent statement: a node is committed-reachable iff every edge on
    its explicit root path matches; winner = deepest such node, lowest index."""
    t_ = len(top)
    best, best_path = 0, []
    for t in range(1, t_):
        path, node, ok = [], t, True
        seen = set()
        while node != 0:
            p = int(parent[node])
            if not (0 <= p < node) or node in seen:
                ok = False
                break
            seen.add(node)
            if int(tokens[node]) != int(top[p]):
                ok = False
            path.append(node)
            node = p
        if ok and len(path) > len(best_path):
            best, best_path = t, path[::-1]
    return best, best_path


def _random_tree(rng, t_):
    parent = np.zeros(t_, dtype=np.int64)
    parent[0] = -1
    for t in range(1, t_):
        parent[t] = rng.integers(0, t)
    return parent


def test_tree_greedy_brute_force_small_trees():
    rng = np.random.default_rng(31)
    v = 3
    for _ in range(3000):
        t_ = int(rng.integers(1, 8))
        parent = _random_tree(rng, t_)
        top = rng.integers(0, v, size=t_)
        tokens = rng.integers(0, v, size=t_)
        if rng.random() < 0.1 and t_ > 1:
            parent[rng.integers(1, t_)] = rng.choice([-1, t_ + 3])    # invalid parents never accept
        lg = _onehot_logits(top, v)[None]
        r = O.verify_tree_greedy(lg, tokens[None], parent[None])
        win, path = _tree_brute(top, tokens, parent)
        assert r["n_accept"][0] == len(path)
        assert r["out_nodes"][0].tolist() == path + [-1] * (t_ - len(path))
        assert r["out_tokens"][0].tolist() == [int(tokens[n]) for n in path] + [int(top[win])] + [-1] * (t_ - len(path) - 1)


def test_tree_greedy_chain_is_the_prefix_rule():
    """A chain (parent[t] = t - 1) is the plain greedy verify over gamma = T - 1."""
    rng = np.random.default_rng(32)
    for _ in range(200):
        t_ = int(rng.integers(1, 9))
        lg = rng.normal(size=(2, t_, 7)).astype(np.float32)
        tok = rng.integers(-1, 8, size=(2, t_))
        par = np.tile(np.arange(-1, t_ - 1), (2, 1))
        tree = O.verify_tree_greedy(lg, tok, par)
        flat = O.verify_greedy(lg, tok[:, 1:])
        assert np.array_equal(tree["n_accept"], flat["n_accept"])
        assert np.array_equal(tree["out_tokens"], flat["out_tokens"])


def test_tree_greedy_hand_example():
    """Root's Top-1 is 2; branches 2->1 (matches the Top-1 of node 1, which is
    1) and 2->3 (no match), plus a sibling 0 under the root: the path
    root -> node 1 (2) -> node 3 (1) is accepted, and node 3's Top-1 (0) is
    the bonus token."""
    top = [2, 1, 0, 0, 3]
    tokens = [9, 2, 0, 1, 3]
    parent = [-1, 0, 0, 1, 1]
    lg = _onehot_logits(top, 4)[None]
    r = O.verify_tree_greedy(lg, np.array([tokens]) % 4, np.array([parent]))
    assert r["n_accept"][0] == 2
    assert r["out_nodes"][0].tolist() == [1, 3, -1, -1, -1]
    assert r["out_tokens"][0].tolist() == [2, 1, 0, -1, -1]
