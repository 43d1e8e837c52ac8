"""Pins of the oracle's top-p (nucleus) truncation and of the walk on it (CPU only).

"Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 3 (top_p
threaded through to the verify walk).  What fixes them independently of the
oracle's sort:
  * brute force over every subset of tiny rows (ties included): the nucleus
    has the fewest tokens of any subset reaching p of the mass, the largest
    sum among subsets of that size, and, among those, the smallest ids;
  * closed forms of the fixed-point p (p = 1, 1/2, tiny, out of range);
  * p = 1 keeps every token of positive weight: the walk equals the plain
    sampled walk on the same uniforms;
  * a tiny p keeps only the most probable token (the lowest id among equal
    maxima): the walk equals the greedy walk for any uniforms;
  * chi-square: the first emitted token follows the truncated law w_p / R_p;
  * the per-block kept sums add up to R_p, and equal the vocabulary oracle's
    block sums at p = 1.
Planted mistakes (ties by larger id, a strict reach test, a mask ignoring or
shifting the id cut, an off-by-one block) each fail one of these.
"""
import itertools

import numpy as np
import pytest
from scipy.stats import chisquare

from oracle import (build_tree, keep_mask, nucleus_row, top_p_fixed, verify_greedy,
                    verify_sample, vocab_reduce, vocab_top_p, weight_constants, weights)


def test_fixed_point_p():
    assert top_p_fixed(1.0) == 1 << 32
    assert top_p_fixed(0.5) == 1 << 31
    assert top_p_fixed(1e-30) == 1
    assert top_p_fixed(0.25) == 1 << 30
    for bad in (0.0, -0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            top_p_fixed(bad)


@pytest.mark.parametrize("seed", range(6))
def test_nucleus_brute_force(seed):
    rng = np.random.default_rng(seed)
    for _ in range(60):
        V = int(rng.integers(1, 8))
        w = [int(x) for x in rng.integers(0, 6, size=V)]
        if sum(w) == 0:
            w[int(rng.integers(0, V))] = 3
        P = int(rng.integers(1, (1 << 32) + 1))
        R = sum(w)
        reach = [s for k in range(1, V + 1) for s in itertools.combinations(range(V), k)
                 if (sum(w[y] for y in s) << 32) >= P * R]
        k = min(len(s) for s in reach)
        best = max(sum(w[y] for y in s) for s in reach if len(s) == k)
        want = min(s for s in reach if len(s) == k and sum(w[y] for y in s) == best)
        tw, tid, rp = nucleus_row(w, P)
        got = tuple(int(y) for y in np.flatnonzero(keep_mask(w, tw, tid)))
        assert got == want, (w, P, got, want)
        assert rp == best


def _small_tree():
    lp = np.array([[[-0.3, -1.2], [-0.4, -1.5], [-0.2, -2.0]]], dtype=np.float32)
    tok = np.array([[[3, 7], [5, 1], [9, 2]]], dtype=np.int32)
    return build_tree(lp, tok, np.array([0]), np.array([0]), 5)


def _rand_tree(rng, B, D, K, budget, V):
    lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
    tok = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(D)])
                    for _ in range(B)]).astype(np.int32)
    return build_tree(lp, tok, rng.integers(0, V, B).astype(np.int32), np.zeros(B, np.int32),
                      budget), tok


def test_p_one_is_the_plain_walk():
    rng = np.random.default_rng(11)
    V, T = 50, 0.8
    for _ in range(10):
        t, tok = _rand_tree(rng, 2, 4, 3, 12, V)
        B, N = t["token"].shape
        logits = rng.standard_normal((B, N, V)).astype(np.float32) * 2
        vr = vocab_reduce(logits, t["num_nodes"], T)
        tp = vocab_top_p(logits, vr["maxv"], t["num_nodes"], T, 1.0)
        nn = t["num_nodes"]
        for b in range(B):
            assert np.array_equal(tp["Rp"][b, :nn[b]], vr["R"][b, :nn[b]])
        u = rng.integers(0, 2 ** 64, size=(B, N, 2), dtype=np.uint64)
        plain = verify_sample(t, logits, vr["maxv"], vr["R"], T, u, 4)
        nuc = verify_sample(t, logits, vr["maxv"], tp["Rp"], T, u, 4,
                            nucleus=(tp["thr_w"], tp["thr_id"]))
        for k in plain:
            assert np.array_equal(plain[k], nuc[k]), k


def test_tiny_p_is_the_greedy_walk():
    rng = np.random.default_rng(12)
    V, T = 30, 1.0
    for _ in range(15):
        t, tok = _rand_tree(rng, 3, 5, 3, 20, V)
        B, N = t["token"].shape
        # coarse logits: ties at the maximum are common
        logits = (rng.integers(0, 12, size=(B, N, V)) * 0.5).astype(np.float32)
        for b in range(B):                          # let the argmax follow children often
            for n in range(int(t["num_nodes"][b])):
                kids = [c for c in range(N) if int(t["parent"][b, c]) == n]
                if kids and rng.random() < 0.7:
                    logits[b, n, t["token"][b, kids[0]]] = logits[b, n].max()
        vr = vocab_reduce(logits, t["num_nodes"], T)
        tp = vocab_top_p(logits, vr["maxv"], t["num_nodes"], T, 1e-9)
        for b in range(B):
            for n in range(int(t["num_nodes"][b])):
                assert int(tp["thr_id"][b, n]) == int(vr["argmax"][b, n])
                assert int(tp["Rp"][b, n]) == 1 << 32
        u = rng.integers(0, 2 ** 64, size=(B, N, 2), dtype=np.uint64)
        s = verify_sample(t, logits, vr["maxv"], tp["Rp"], T, u, 5,
                          nucleus=(tp["thr_w"], tp["thr_id"]))
        g = verify_greedy(t, vr["argmax"], 5)
        for k in g:
            assert np.array_equal(g[k], s[k]), k


def test_chi_square_first_token_follows_the_truncated_law():
    rng = np.random.default_rng(13)
    t = _small_tree()
    V, N, T, p = 16, 6, 1.0, 0.7
    logits = (rng.standard_normal((1, N, V)) * 1.5).astype(np.float32)
    vr = vocab_reduce(logits, t["num_nodes"], T)
    tp = vocab_top_p(logits, vr["maxv"], t["num_nodes"], T, p)
    c, a = weight_constants(T)
    w0 = weights(logits[0, 0], vr["maxv"][0, 0], c, a)
    kept = np.where(keep_mask(w0, int(tp["thr_w"][0, 0]), int(tp["thr_id"][0, 0])), w0, 0)
    assert 1 < np.count_nonzero(kept) < V
    law = kept.astype(np.float64) / float(tp["Rp"][0, 0])
    trials = 40000
    u = rng.integers(0, 2 ** 64, size=(trials, N, 2), dtype=np.uint64)
    first = np.zeros(V, np.int64)
    for k in range(trials):
        r = verify_sample(t, logits, vr["maxv"], tp["Rp"], T, u[k:k + 1], 3,
                          nucleus=(tp["thr_w"], tp["thr_id"]))
        first[r["out_tokens"][0, 0]] += 1
    assert first[law == 0].sum() == 0                  # nothing outside the nucleus
    sel = law > 0
    assert chisquare(first[sel], law[sel] * trials).pvalue > 1e-4


def test_block_sums_partition_the_kept_mass():
    """Rp_blocks sums to Rp for any p; at p = 1 it is the vocabulary oracle's R_blocks."""
    rng = np.random.default_rng(14)
    t = _small_tree()
    V, N, T = 70000, 6, 1.0
    logits = (rng.standard_normal((1, N, V)) * 3).astype(np.float32)
    logits[0, :, 0] = logits[0].max(axis=-1) + 0.5          # token 0 is in every nucleus
    vr = vocab_reduce(logits, t["num_nodes"], T)
    for p in (1.0, 0.9, 0.3):
        tp = vocab_top_p(logits, vr["maxv"], t["num_nodes"], T, p)
        assert np.array_equal(tp["Rp_blocks"].sum(axis=-1, dtype=np.uint64), tp["Rp"])
        if p == 1.0:
            assert np.array_equal(tp["Rp_blocks"], vr["R_blocks"])
