"""Pins of the oracle's tree attention (CPU only).

What fixes it independently of the oracle's own formula code:
  * every tree node's output equals ordinary causal attention (torch's
    scaled_dot_product_attention on the CPU, float64) of that node over the
    request's context followed by the root-to-node path, the path taken from
    parent pointers rather than from the visibility bits -- this is what the
    mask is for ("Dissecting DDTree's Tree-Parallel Evaluation Strategy",
    Section 1 step 3; "The Tree That Couldn't Branch", "Hypothesis 3");
  * a single chain (topk_cap=1) is textbook causal attention over
    [context; chain], bottom-right aligned;
  * with an empty context the root sees only itself: o_root = v_root exactly;
  * invariance under any permutation of the context keys (the context is a
    set shared by every node, loaded once: Section 2);
  * a three-node tree whose two siblings would contaminate each other's
    output if the mask leaked;
  * lse against scipy's logsumexp of the explicit scores.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import build_tree, tree_attention


def _tree(rng, B, D, K, budget):
    lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
    tok = rng.integers(0, 50, size=(B, D, K)).astype(np.int32)
    return build_tree(lp, tok, np.zeros(B, np.int32), np.zeros(B, np.int32), budget)


def _sdpa_last(qv, keys, vals, scale):
    """Causal attention of the last position over `keys` (torch, float64)."""
    q = torch.from_numpy(qv[None, None, None, :])
    k = torch.from_numpy(keys[None, None])
    v = torch.from_numpy(vals[None, None])
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 2), (3, 1)])
def test_each_node_is_causal_attention_over_its_path(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    B, D, K, budget, Dh = 2, 4, 3, 12, 16
    t = _tree(rng, B, D, K, budget)
    N = budget + 1
    lens = np.array([7, 0])
    offs = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((B, N, hq, Dh)).astype(np.float32)
    kc = rng.standard_normal((offs[-1], hkv, Dh)).astype(np.float32)
    vc = rng.standard_normal((offs[-1], hkv, Dh)).astype(np.float32)
    kt = rng.standard_normal((B, N, hkv, Dh)).astype(np.float32)
    vt = rng.standard_normal((B, N, hkv, Dh)).astype(np.float32)
    scale = 0.37
    o, lse = tree_attention(q, kc, vc, offs, kt, vt, t["vis"], t["num_nodes"], scale)
    g = hq // hkv
    for b in range(B):
        for i in range(int(t["num_nodes"][b])):
            path, j = [], i
            while j >= 0:
                path.append(j)
                j = int(t["parent"][b, j])
            path = path[::-1]
            for h in range(hq):
                keys = np.concatenate([kc[offs[b]:offs[b + 1], h // g], kt[b, path, h // g]]).astype(np.float64)
                vals = np.concatenate([vc[offs[b]:offs[b + 1], h // g], vt[b, path, h // g]]).astype(np.float64)
                ref = _sdpa_last(q[b, i, h].astype(np.float64), keys, vals, scale)
                np.testing.assert_allclose(o[b, i, h], ref, rtol=1e-12, atol=1e-12)
                s = keys @ q[b, i, h].astype(np.float64) * scale
                assert abs(lse[b, i, h] - logsumexp(s)) < 1e-12


def test_chain_equals_bottom_right_causal():
    rng = np.random.default_rng(5)
    D, Dh, L = 6, 8, 9
    t = _tree(rng, 1, D, 1, D)
    N = D + 1
    q = rng.standard_normal((1, N, 1, Dh))
    kc = rng.standard_normal((L, 1, Dh))
    vc = rng.standard_normal((L, 1, Dh))
    kt = rng.standard_normal((1, N, 1, Dh))
    vt = rng.standard_normal((1, N, 1, Dh))
    o, _ = tree_attention(q, kc, vc, np.array([0, L]), kt, vt, t["vis"], t["num_nodes"], 0.5)
    # textbook: query r (0..N-1) sees keys [0, L + r] of the concatenation
    K_all = torch.from_numpy(np.concatenate([kc[:, 0], kt[0, :, 0]]))
    V_all = torch.from_numpy(np.concatenate([vc[:, 0], vt[0, :, 0]]))
    mask = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0, :, 0])[None], K_all[None], V_all[None], attn_mask=mask[None],
        scale=0.5)[0].numpy()
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_empty_context_root_is_its_own_value():
    rng = np.random.default_rng(6)
    t = _tree(rng, 1, 3, 2, 5)
    q = rng.standard_normal((1, 6, 2, 4))
    kt = rng.standard_normal((1, 6, 2, 4))
    vt = rng.standard_normal((1, 6, 2, 4))
    empty = np.zeros((0, 2, 4))
    o, lse = tree_attention(q, empty, empty, np.array([0, 0]), kt, vt, t["vis"], t["num_nodes"])
    assert np.array_equal(o[0, 0], vt[0, 0])
    np.testing.assert_allclose(lse[0, 0], (q[0, 0] * kt[0, 0]).sum(-1) / 2.0, rtol=0, atol=1e-15)


def test_context_permutation_invariance():
    rng = np.random.default_rng(7)
    t = _tree(rng, 1, 4, 2, 9)
    L, Dh = 40, 8
    q = rng.standard_normal((1, 10, 2, Dh))
    kc = rng.standard_normal((L, 2, Dh))
    vc = rng.standard_normal((L, 2, Dh))
    kt = rng.standard_normal((1, 10, 2, Dh))
    vt = rng.standard_normal((1, 10, 2, Dh))
    o1, l1 = tree_attention(q, kc, vc, np.array([0, L]), kt, vt, t["vis"], t["num_nodes"])
    p = rng.permutation(L)
    o2, l2 = tree_attention(q, kc[p], vc[p], np.array([0, L]), kt, vt, t["vis"], t["num_nodes"])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-13)


def test_siblings_do_not_see_each_other():
    # root with two children (D=1, K=2).  Give the second child's key a huge
    # score for every query: if the first child leaked it, its output would be v[2].
    lp = np.array([[[-0.5, -1.0]]], dtype=np.float32)
    t = build_tree(lp, np.array([[[3, 4]]], np.int32), np.array([0]), np.array([0]), 2)
    assert list(t["parent"][0]) == [-1, 0, 0]
    Dh = 4
    q = np.ones((1, 3, 1, Dh))
    kt = np.zeros((1, 3, 1, Dh))
    kt[0, 2, 0] = 50.0
    vt = np.arange(3 * Dh, dtype=np.float64).reshape(1, 3, 1, Dh)
    empty = np.zeros((0, 1, Dh))
    o, _ = tree_attention(q, empty, empty, np.array([0, 0]), kt, vt, t["vis"], t["num_nodes"], 1.0)
    np.testing.assert_allclose(o[0, 1, 0], (vt[0, 0, 0] + vt[0, 1, 0]) / 2, rtol=1e-14)
    np.testing.assert_allclose(o[0, 2, 0], vt[0, 2, 0], rtol=1e-14)    # sees itself (huge score)


def test_padding_nodes_are_zero():
    rng = np.random.default_rng(8)
    t = _tree(rng, 1, 2, 1, 6)          # only 3 nodes exist
    assert int(t["num_nodes"][0]) == 3
    q = rng.standard_normal((1, 7, 1, 4))
    kt = rng.standard_normal((1, 7, 1, 4))
    vt = rng.standard_normal((1, 7, 1, 4))
    kc = rng.standard_normal((5, 1, 4))
    o, lse = tree_attention(q, kc, kc, np.array([0, 5]), kt, vt, t["vis"], t["num_nodes"])
    assert np.all(o[0, 3:] == 0) and np.all(np.isneginf(lse[0, 3:]))
