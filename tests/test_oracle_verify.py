"""Pins of the oracle's verified-tree walks (CPU only).

Greedy ("Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1 step 5):
  * topk_cap=1 reduces to linear DFlash's accept rule -- accept the depth-d
    draft token iff the target argmax at the previous position equals it
    ("Implementing Temperature-Aware Tree Sampling for DDTree", "The Context:
    What Led to This Message"), written here as a plain loop over the chain;
  * brute force over all nodes: the walk ends at the unique deepest node
    whose every edge satisfies argmax[parent] == token;
  * greedy-chain containment: accept(tree) >= min(accept(rank-0 chain), depth);
  * planted targets (ragged workload recipe): the expected accept length is
    recomputed from the plant records alone.

Sampled (Section 3; "Path B: CPU-Side Tree Rejection Sampling"):
  * chi-square: the first emitted token follows the target law w/R at the
    root, and the token after an accepted child c follows the law at c
    (this is what makes speculative sampling exact);
  * small temperature: when every non-maximal weight is 0, sampling equals
    the greedy walk for any uniforms;
  * uniform extremes u = 0 and u = 2^64 - 1, and a bonus draw at a chosen
    cumulative-weight boundary, worked out from the weights directly.
"""
import numpy as np
import pytest
from scipy.stats import chisquare

import workloads
from oracle import (attach_draft_topk, build_tree, verify_greedy, verify_sample, vocab_reduce,
                    weight_constants, weights)


def _rand_tree(rng, B, D, K, budget, V=40):
    lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
    tok = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(D)])
                    for _ in range(B)]).astype(np.int32)
    return build_tree(lp, tok, rng.integers(0, V, B).astype(np.int32), np.zeros(B, np.int32),
                      budget), tok


def _matching_argmax(rng, t, tok, p_match=0.7, V=40):
    """argmax that equals some child's token with probability p_match."""
    B, N = t["token"].shape
    am = rng.integers(0, V, size=(B, N)).astype(np.int32)
    for b in range(B):
        for n in range(int(t["num_nodes"][b])):
            d = int(t["depth"][b, n])
            if d < tok.shape[1] and rng.random() < p_match:
                am[b, n] = tok[b, d, rng.integers(0, tok.shape[2])]
    return am


def test_topk1_equals_linear_dflash_rule():
    rng = np.random.default_rng(1)
    D = 7
    for trial in range(200):
        t, tok = _rand_tree(rng, 1, D, 1, D, V=6)
        am = rng.integers(0, 6, size=(1, D + 1)).astype(np.int32)
        draft = [int(x) for x in tok[0, :, 0]]
        a = 0
        while a < D and am[0, a] == draft[a]:      # position a predicts draft token a+1
            a += 1
        r = verify_greedy(t, am, D)
        assert int(r["accept_len"][0]) == a
        assert int(r["bonus"][0]) == int(am[0, a])
        assert list(r["out_tokens"][0, :a + 1]) == draft[:a] + [int(am[0, a])]


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_deepest_matching_node(seed):
    rng = np.random.default_rng(seed)
    B, D, K, budget = 6, 5, 3, 30
    t, tok = _rand_tree(rng, B, D, K, budget)
    am = _matching_argmax(rng, t, tok)
    r = verify_greedy(t, am, D)
    for b in range(B):
        n = int(t["num_nodes"][b])
        good = []
        for i in range(n):
            ok, j = True, i
            while j > 0:
                p = int(t["parent"][b, j])
                ok &= int(am[b, p]) == int(t["token"][b, j])
                j = p
            if ok:
                good.append(i)
        deepest = max(good, key=lambda i: int(t["depth"][b, i]))
        assert sum(int(t["depth"][b, i]) == int(t["depth"][b, deepest]) for i in good) == 1
        assert int(r["accept_len"][b]) == int(t["depth"][b, deepest])
        assert int(r["path_nodes"][b, r["accept_len"][b]]) == deepest
        assert int(r["bonus"][b]) == int(am[b, deepest])


@pytest.mark.parametrize("seed", range(4))
def test_tree_accepts_at_least_the_greedy_chain(seed):
    rng = np.random.default_rng(50 + seed)
    B, D, K, budget = 8, 8, 4, 32
    t, tok = _rand_tree(rng, B, D, K, budget)
    am = _matching_argmax(rng, t, tok, p_match=0.9)
    r = verify_greedy(t, am, D)
    for b in range(B):
        chain, cur, depth = 0, 0, 0
        while True:                                        # linear rule on the rank-0 chain
            c = int(t["first_child"][b, cur])
            if c == -1:
                break
            depth += 1
            if chain == depth - 1 and int(am[b, cur]) == int(t["token"][b, c]):
                chain += 1
            cur = c
        assert int(r["accept_len"][b]) >= min(chain, depth)


def test_planted_targets_give_expected_accept_length():
    cfg = workloads.config("ragged", B=6, ctx=(4, 9), V=512, Hq=1, Hkv=1, Dh=8)
    inp = attach_draft_topk(workloads.make_inputs(cfg), cfg.D, cfg.K)
    t = build_tree(inp["draft_lp"], inp["draft_tok"], inp["root_tok"], inp["prefix_len"], cfg.budget)
    logits, planted = workloads.make_target_logits(cfg, inp, t["depth"], t["num_nodes"])
    am = vocab_reduce(logits, t["num_nodes"], 0.0, dtype="bf16")["argmax"]
    r = verify_greedy(t, am, cfg.D)
    for b in range(cfg.B):
        cur, a = 0, 0
        while True:                                          # follow plant records only
            kids = [c for c in range(int(t["num_nodes"][b])) if t["parent"][b, c] == cur
                    and int(t["token"][b, c]) == int(planted[b, cur])]
            if not kids:
                break
            cur, a = kids[0], a + 1
        assert int(r["accept_len"][b]) == a
        assert int(r["bonus"][b]) == int(planted[b, cur])


# --- sampled walk -------------------------------------------------------------------------

def _small_tree():
    # D=3, K=2, budget 5, V=16 with fixed draft proposals
    lp = np.array([[[-0.3, -1.2], [-0.4, -1.5], [-0.2, -2.0]]], dtype=np.float32)
    tok = np.array([[[3, 7], [5, 1], [9, 2]]], dtype=np.int32)
    return build_tree(lp, tok, np.array([0]), np.array([0]), 5)


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_chi_square_first_and_second_token(T):
    rng = np.random.default_rng(int(T * 100))
    t = _small_tree()
    V, N = 16, 6
    logits = rng.standard_normal((1, N, V)).astype(np.float32)
    vr = vocab_reduce(logits, t["num_nodes"], T)
    c, a = weight_constants(T)
    law = [weights(logits[0, n], vr["maxv"][0, n], c, a).astype(np.float64) / float(vr["R"][0, n])
           for n in range(N)]
    trials = 60000
    u = rng.integers(0, 2 ** 64, size=(trials, N, 2), dtype=np.uint64)
    first = np.zeros(V, np.int64)
    second = {}
    for k in range(trials):
        r = verify_sample(t, logits, vr["maxv"], vr["R"], T, u[k:k + 1], 3)
        first[r["out_tokens"][0, 0]] += 1
        if r["accept_len"][0] >= 1:
            node = int(r["path_nodes"][0, 1])
            second.setdefault(node, np.zeros(V, np.int64))[r["out_tokens"][0, 1]] += 1
    p = chisquare(first, law[0] * trials).pvalue
    assert p > 1e-4, p
    for node, counts in second.items():
        if counts.sum() < 5000:
            continue
        exp = law[node] * counts.sum()
        keep = exp > 5
        obs, ex = counts[keep], exp[keep]
        if (~keep).any() and exp[~keep].sum() > 0:          # lump the rare cells together
            obs = np.append(obs, counts[~keep].sum())
            ex = np.append(ex, exp[~keep].sum())
        assert chisquare(obs, ex * obs.sum() / ex.sum()).pvalue > 1e-4


def test_small_temperature_equals_greedy():
    rng = np.random.default_rng(3)
    for seed in range(20):
        t, tok = _rand_tree(rng, 3, 5, 3, 20)
        B, N = t["token"].shape
        V = 40
        logits = (rng.integers(0, 40, size=(B, N, V)) * 0.25).astype(np.float32)
        am = _matching_argmax(rng, t, tok)
        for b in range(B):                      # make the argmax a strict max by 1.0
            for n in range(N):
                logits[b, n, am[b, n]] = logits[b, n].max() + 1.0
        T = 0.01                                # every non-max weight is 2^(-144) -> 0
        vr = vocab_reduce(logits, t["num_nodes"], T)
        assert np.all(vr["R"][:, :1] == 2 ** 32)
        g = verify_greedy(t, vr["argmax"], 5)
        s = verify_sample(t, logits, vr["maxv"], vr["R"], T,
                          rng.integers(0, 2 ** 64, size=(B, N, 2), dtype=np.uint64), 5)
        for k in ("accept_len", "bonus", "out_tokens", "path_nodes"):
            assert np.array_equal(g[k], s[k]), k


def test_uniform_extremes_and_bonus_boundary():
    t = _small_tree()
    V, N = 16, 6
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((1, N, V)).astype(np.float32)
    T = 1.0
    vr = vocab_reduce(logits, t["num_nodes"], T)
    c, a = weight_constants(T)
    w0 = weights(logits[0, 0], vr["maxv"][0, 0], c, a)
    R0 = int(vr["R"][0, 0])
    # hand trace of the build: n1=(d1,r0) n2=(d2,r0 of n1) n3=(d3,r0 of n2) n4=(d1,r1) n5
    kids = [1, 4]                                     # root's children, in rank order
    assert int(t["first_child"][0, 0]) == 1 and int(t["next_sibling"][0, 1]) == 4
    assert int(t["next_sibling"][0, 4]) == -1
    # u = 0 everywhere: t = 0 < w(first child) -> always accepted until a leaf
    u = np.zeros((1, N, 2), np.uint64)
    r = verify_sample(t, logits, vr["maxv"], vr["R"], T, u, 3)
    assert int(r["path_nodes"][0, 1]) == 1
    # u = 2^64-1 for both children: t = R_res - 1, accepted only if w(c) == R_res -> rejected.
    # Then the bonus at the root with u_bonus chosen so that t hits the start of token x.
    tok1, tok3 = int(t["token"][0, 1]), int(t["token"][0, 4])
    res = w0.copy()
    res[[tok1, tok3]] = 0
    R_res = R0 - int(w0[tok1]) - int(w0[tok3])
    assert R_res == int(res.sum())
    csum = np.cumsum(res.astype(object))
    for x in [v for v in range(V) if res[v] > 0][:5]:
        start = int(csum[x] - res[x])               # t == start selects x
        ub = -(-(start << 64) // R_res)             # smallest u with floor(u R / 2^64) >= start
        assert (ub * R_res) >> 64 == start
        u = np.zeros((1, N, 2), np.uint64)
        u[0, 1, 0] = u[0, 4, 0] = np.uint64(2 ** 64 - 1)
        u[0, 0, 1] = np.uint64(ub)
        r = verify_sample(t, logits, vr["maxv"], vr["R"], T, u, 3)
        assert int(r["accept_len"][0]) == 0 and int(r["bonus"][0]) == x
