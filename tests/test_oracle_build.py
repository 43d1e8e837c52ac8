"""Pins of the oracle's best-first tree build (CPU only).

What fixes the build independently of the oracle's heap code:
  * brute force: on tie-free inputs the best-first order over rank sequences
    is exactly "all sequences sorted by cumulative score", truncated at budget;
  * the closed form 1 + min(budget, sum_d K^d) for the node count;
  * the single-chain case topk_cap=1 ("The Tree That Couldn't Branch",
    "The Experiment: budget=7, topk_cap=1"), which must be the draft's greedy
    chain and a lower-triangular visibility;
  * the greedy-chain containment ("Context: The Road to DDTree": the tree
    should contain the greedy chain) in its exact form: the tree's maximum
    depth equals the length of the rank-0 chain it contains;
  * two trees worked out by hand from the definition (exact binary-fraction
    log-probs), one of them exercising the parent-index tie-break.
"""
import itertools

import numpy as np
import pytest

from oracle import build_tree


def _sorted_lp(rng, B, D, K, scale=2.0):
    lp = -np.abs(rng.standard_normal((B, D, K))).astype(np.float32) * np.float32(scale)
    return -np.sort(-lp, axis=-1)          # non-increasing along K


def _tokens(rng, B, D, K, V=1000):
    return np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(D)])
                     for _ in range(B)]).astype(np.int32)


def _rank_seq(tree, b, i):
    seq = []
    while i > 0:
        seq.append(int(tree["rank"][b, i]))
        i = int(tree["parent"][b, i])
    return tuple(reversed(seq))


def _brute(lp, D, K):
    """Every rank sequence of length 1..D with its fp32 cumulative score."""
    out = {}
    for d in range(1, D + 1):
        for seq in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for depth, r in enumerate(seq):
                s = np.float32(s + lp[depth, r])
            out[seq] = float(s)
    return out


@pytest.mark.parametrize("D,K", [(1, 1), (1, 3), (2, 2), (3, 2), (3, 3), (4, 2), (4, 3), (2, 1)])
def test_brute_force_top_budget(D, K):
    rng = np.random.default_rng(100 * D + K)
    total = sum(K ** d for d in range(1, D + 1))
    checked = 0
    for trial in range(6):
        lp = _sorted_lp(rng, 1, D, K)
        scores = _brute(lp[0], D, K)
        vals = sorted(scores.values())
        if len(set(vals)) != len(vals):
            continue                                   # pin only tie-free inputs
        order = sorted(scores, key=lambda s: -scores[s])
        for budget in range(1, total + 3):
            t = build_tree(lp, _tokens(rng, 1, D, K), np.array([7]), np.array([10]), budget)
            n = int(t["num_nodes"][0])
            assert n == 1 + min(budget, total)
            got = [_rank_seq(t, 0, i) for i in range(1, n)]
            assert got == order[: n - 1]
            for i in range(1, n):
                assert float(t["score"][0, i]) == scores[got[i - 1]]
        checked += 1
    assert checked >= 3


@pytest.mark.parametrize("seed", range(5))
def test_structure_invariants(seed):
    rng = np.random.default_rng(seed)
    B, D, K, budget = 3, 6, 4, 40
    lp = _sorted_lp(rng, B, D, K)
    tok = _tokens(rng, B, D, K)
    t = build_tree(lp, tok, np.arange(B), np.array([5, 0, 99]), budget)
    for b in range(B):
        n = int(t["num_nodes"][b])
        assert n == 1 + min(budget, sum(K ** d for d in range(1, D + 1)))
        sc = t["score"][b, :n]
        assert np.all(np.diff(sc.astype(np.float64)) <= 0)            # popped best-first
        for i in range(1, n):
            p, r, d = int(t["parent"][b, i]), int(t["rank"][b, i]), int(t["depth"][b, i])
            assert 0 <= p < i                                        # prefix-closed
            assert d == int(t["depth"][b, p]) + 1
            assert t["token"][b, i] == tok[b, d - 1, r]
            assert t["position"][b, i] == [5, 0, 99][b] + d
            if r > 0:                                                 # sibling-closed
                sib = [j for j in range(1, i) if t["parent"][b, j] == p and t["rank"][b, j] == r - 1]
                assert len(sib) == 1 and t["next_sibling"][b, sib[0]] == i
            else:
                assert t["first_child"][b, p] == i
            # ancestor-or-self visibility from parent pointers
            anc, j = {i}, i
            while j > 0:
                j = int(t["parent"][b, j])
                anc.add(j)
            bits = {k for k in range(n) if (int(t["vis"][b, i, k // 64]) >> (k % 64)) & 1}
            assert bits == anc
        # linked lists reproduce exactly the children in rank order
        for p in range(n):
            kids = [i for i in range(1, n) if t["parent"][b, i] == p]
            walk, c = [], int(t["first_child"][b, p])
            while c != -1:
                walk.append(c)
                c = int(t["next_sibling"][b, c])
            assert walk == sorted(kids, key=lambda i: int(t["rank"][b, i]))
        assert np.all(t["token"][b, n:] == -1) and np.all(t["vis"][b, n:] == 0)


def test_chain_topk1_is_greedy_chain():
    rng = np.random.default_rng(3)
    D = 8
    lp = _sorted_lp(rng, 1, D, 1)
    tok = _tokens(rng, 1, D, 1)
    for budget in (1, 3, 7, 8, 12):
        t = build_tree(lp, tok, np.array([42]), np.array([100]), budget)
        n = int(t["num_nodes"][0])
        assert n == 1 + min(budget, D)
        assert int(t["max_depth"][0]) == min(budget, D)
        assert list(t["parent"][0, :n]) == [-1] + list(range(n - 1))
        assert list(t["token"][0, 1:n]) == list(tok[0, : n - 1, 0])
        for i in range(n):
            assert int(t["vis"][0, i, 0]) == (1 << (i + 1)) - 1          # lower-triangular


@pytest.mark.parametrize("seed", range(8))
def test_greedy_chain_depth_equals_tree_depth(seed):
    rng = np.random.default_rng(1000 + seed)
    B, D, K = 4, 8, 8
    lp = _sorted_lp(rng, B, D, K, scale=3.0)
    for budget in (8, 32, 64):
        t = build_tree(lp, _tokens(rng, B, D, K), np.zeros(B, np.int32), np.zeros(B, np.int32),
                       budget)
        for b in range(B):
            n = int(t["num_nodes"][b])
            chain, c = 0, int(t["first_child"][b, 0])
            while c != -1:
                chain += 1
                c = int(t["first_child"][b, c])
            assert chain == int(t["depth"][b, :n].max()) == int(t["max_depth"][b])


def test_hand_example_distinct_scores():
    # D=2, K=2.  depth-1 log-probs (-1/4, -1), depth-2 (-1/2, -2), budget 4.
    # Frontier trace: take (d1,r0,-0.25) -> node1; offer child -0.75 and sibling -1.
    # take -0.75 -> node2 (depth 2, no child); offer its sibling -0.25-2 = -2.25.
    # take -1 -> node3 (d1 r1); offer child -1.5.  take -1.5 -> node4.  Budget reached.
    lp = np.array([[[-0.25, -1.0], [-0.5, -2.0]]], dtype=np.float32)
    tok = np.array([[[11, 12], [21, 22]]], dtype=np.int32)
    t = build_tree(lp, tok, np.array([5]), np.array([3]), 4)
    assert int(t["num_nodes"][0]) == 5
    assert list(t["parent"][0]) == [-1, 0, 1, 0, 3]
    assert list(t["depth"][0]) == [0, 1, 2, 1, 2]
    assert list(t["rank"][0]) == [-1, 0, 0, 1, 0]
    assert list(t["token"][0]) == [5, 11, 21, 12, 21]
    assert list(t["score"][0]) == [0.0, -0.25, -0.75, -1.0, -1.5]
    assert list(t["first_child"][0]) == [1, 2, -1, 4, -1]
    assert list(t["next_sibling"][0]) == [-1, 3, -1, -1, -1]
    assert list(t["position"][0]) == [3, 4, 5, 4, 5]
    assert int(t["max_depth"][0]) == 2
    assert [int(v) for v in t["vis"][0, :, 0]] == [0b1, 0b11, 0b111, 0b1001, 0b11001]


def test_hand_example_parent_tie_break():
    # All log-probs -1: equal scores are taken by smaller parent index first.
    # Trace: n1=(p0,r0); n2=(p0,r1); then the two depth-2 candidates of n1 and n2
    # tie at -2 and n1's children come first: n3=(p1,r0), n4=(p1,r1), n5=(p2,r0), n6=(p2,r1).
    lp = np.full((1, 2, 2), -1.0, dtype=np.float32)
    tok = np.array([[[1, 2], [3, 4]]], dtype=np.int32)
    t = build_tree(lp, tok, np.array([0]), np.array([0]), 6)
    assert list(t["parent"][0]) == [-1, 0, 0, 1, 1, 2, 2]
    assert list(t["rank"][0]) == [-1, 0, 1, 0, 1, 0, 1]
    assert list(t["score"][0]) == [0.0, -1.0, -1.0, -2.0, -2.0, -2.0, -2.0]


def test_wide_tree_two_vis_words():
    rng = np.random.default_rng(9)
    D, K, budget = 16, 4, 64
    lp = _sorted_lp(rng, 1, D, K)
    t = build_tree(lp, _tokens(rng, 1, D, K), np.array([1]), np.array([0]), budget)
    assert t["vis"].shape == (1, 65, 2)
    assert int(t["num_nodes"][0]) == 65
    assert (int(t["vis"][0, 64, 1]) & 1) == 1            # node 64 sees itself in word 1


def test_hand_example_minus_inf_logprobs():
    # A real log-prob may be -inf (a masked token).  D=2, K=2, depth-1 (-1, -inf),
    # depth-2 (-1/2, -inf), budget 6 (every rank sequence fits: 2 + 4 nodes).
    # Trace: n1=(p0,r0,-1); n2=(p1,r0,-1.5), which offers only its sibling (depth 2 = D);
    # then four entries at -inf, taken by parent index, then rank: n3=(p0,r1),
    # n4=(p1,r1), n5=(p3,r0), n6=(p3,r1).  No entry below depth D or past rank K-1
    # is ever offered, so none can take a slot even though it would tie at -inf.
    lp = np.array([[[-1.0, -np.inf], [-0.5, -np.inf]]], dtype=np.float32)
    tok = np.array([[[1, 2], [3, 4]]], dtype=np.int32)
    t = build_tree(lp, tok, np.array([9]), np.array([0]), 6)
    assert int(t["num_nodes"][0]) == 7
    assert list(t["parent"][0]) == [-1, 0, 1, 0, 1, 3, 3]
    assert list(t["rank"][0]) == [-1, 0, 0, 1, 1, 0, 1]
    assert list(t["depth"][0]) == [0, 1, 2, 1, 2, 2, 2]
    assert list(t["token"][0]) == [9, 1, 3, 2, 4, 3, 4]
    assert list(t["score"][0][:3]) == [0.0, -1.0, -1.5]
    assert np.all(np.isneginf(t["score"][0][3:]))


def test_flat_logprobs_exhaust_budget_at_depth_one():
    # "Hypothesis 1: Best-First Search Exhaustion": with every log-prob equal
    # (-1) a depth-d node scores exactly -d, so best-first takes all K^d nodes
    # of depth d before any of depth d + 1: max_depth is 1 for budget <= K,
    # 2 for K < budget <= K + K^2, 3 just past that.
    D, K = 8, 4
    lp = np.full((2, D, K), -1.0, dtype=np.float32)
    tok = np.tile(np.arange(K, dtype=np.int32), (2, D, 1))
    for budget, want in ((1, 1), (K, 1), (K + 1, 2), (K + K * K, 2), (K + K * K + 1, 3)):
        t = build_tree(lp, tok, np.zeros(2, np.int32), np.zeros(2, np.int32), budget)
        assert list(t["max_depth"]) == [want, want], budget
