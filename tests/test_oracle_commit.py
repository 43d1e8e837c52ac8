"""Pins of the oracle's path commit (CPU only).

What fixes it independently of the oracle's own copy loop:
  * attention equivalence: after the commit, ordinary causal attention (torch's
    scaled_dot_product_attention on the CPU, float64) of every accepted node
    over the request's cache rows up to that node's position equals the tree
    attention the verify pass computed for it -- committing the path must
    leave the cache holding exactly what those nodes attended to, in position
    order ("Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
    step 5 and Section 2).  Dropping the root, swapping K and V, reversing the
    path or writing at the wrong positions each change some node's output;
  * a single chain (topk_cap = 1) numbers its nodes by depth, so the committed
    rows are the first accept_len + 1 tree rows, in order;
  * only accept_len + 1 rows of each request change, every other byte of the
    cache is untouched;
  * closed forms: next prefix = prefix_len + accept_len + 1, next root = bonus;
    positions at or past the capacity are not written.
"""
import numpy as np
import pytest
import torch

from oracle import build_tree, commit_path, tree_attention, verify_greedy


def _case(rng, B, D, K, budget, lens, Hkv=2, Hq=4, Dh=8, V=30, p_follow=0.8):
    lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
    tok = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(D)])
                    for _ in range(B)]).astype(np.int32)
    t = build_tree(lp, tok, rng.integers(0, V, B).astype(np.int32), np.asarray(lens, np.int32),
                   budget)
    N = budget + 1
    # target argmax: usually the token of one of the node's children, so paths get long
    am = rng.integers(0, V, size=(B, N)).astype(np.int32)
    for b in range(B):
        nn = int(t["num_nodes"][b])
        for n in range(nn):
            kids = [c for c in range(nn) if int(t["parent"][b, c]) == n]
            if kids and rng.random() < p_follow:
                am[b, n] = t["token"][b, kids[rng.integers(0, len(kids))]]
    w = verify_greedy(t, am, D)
    q = rng.standard_normal((B, N, Hq, Dh))
    kt = rng.standard_normal((B, N, Hkv, Dh))
    vt = rng.standard_normal((B, N, Hkv, Dh))
    return t, w, q, kt, vt


def _slab(rng, lens, cap, Hkv, Dh):
    """Per-request slabs of `cap` rows; context rows random, the rest a sentinel."""
    B = len(lens)
    kc = np.full((B * cap, Hkv, Dh), 1234.5)
    vc = np.full((B * cap, Hkv, Dh), -987.25)
    for b, L in enumerate(lens):
        kc[b * cap:b * cap + L] = rng.standard_normal((L, Hkv, Dh))
        vc[b * cap:b * cap + L] = rng.standard_normal((L, Hkv, Dh))
    return kc, vc, np.arange(B, dtype=np.int64) * cap


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cache_after_commit_reproduces_path_attention(seed):
    rng = np.random.default_rng(seed)
    B, D, K, budget, cap, Hkv, Hq, Dh = 3, 5, 3, 14, 40, 2, 4, 8
    lens = [9, 0, 17]
    t, w, q, kt, vt = _case(rng, B, D, K, budget, lens, Hkv, Hq, Dh, p_follow=1.0)
    kc, vc, base = _slab(rng, lens, cap, Hkv, Dh)
    # the verify pass: tree attention over the packed contexts
    offs = np.concatenate([[0], np.cumsum(lens)])
    kp = np.concatenate([kc[base[b]:base[b] + lens[b]] for b in range(B)])
    vp = np.concatenate([vc[base[b]:base[b] + lens[b]] for b in range(B)])
    o, _ = tree_attention(q, kp, vp, offs, kt, vt, t["vis"], t["num_nodes"], 0.3)
    c = commit_path(t, w["accept_len"], w["path_nodes"], w["bonus"], kt, vt, kc, vc, base, cap)
    assert max(int(a) for a in w["accept_len"]) >= 2     # the check covers real paths
    g = Hq // Hkv
    for b in range(B):
        for j in range(int(w["accept_len"][b]) + 1):
            n = int(w["path_nodes"][b, j])
            last = base[b] + lens[b] + j                  # this node's own row
            for h in range(Hq):
                keys = torch.from_numpy(c["k_cache"][base[b]:last + 1, h // g])
                vals = torch.from_numpy(c["v_cache"][base[b]:last + 1, h // g])
                qq = torch.from_numpy(q[b, n, h])
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq[None, None, None], keys[None, None], vals[None, None], scale=0.3)[0, 0, 0]
                np.testing.assert_allclose(o[b, n, h], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_chain_commits_a_prefix_of_the_tree_rows():
    rng = np.random.default_rng(4)
    B, D, cap, Hkv, Dh = 2, 6, 20, 1, 4
    lens = [3, 5]
    t, w, q, kt, vt = _case(rng, B, D, 1, D, lens, Hkv, 1, Dh, p_follow=0.9)
    kc, vc, base = _slab(rng, lens, cap, Hkv, Dh)
    c = commit_path(t, w["accept_len"], w["path_nodes"], w["bonus"], kt, vt, kc, vc, base, cap)
    for b in range(B):
        a = int(w["accept_len"][b])
        r0 = base[b] + lens[b]
        assert np.array_equal(c["k_cache"][r0:r0 + a + 1], kt[b, :a + 1])
        assert np.array_equal(c["v_cache"][r0:r0 + a + 1], vt[b, :a + 1])


@pytest.mark.parametrize("seed", [5, 6])
def test_only_the_path_rows_change_and_closed_forms(seed):
    rng = np.random.default_rng(seed)
    B, D, K, budget, cap, Hkv, Dh = 4, 4, 2, 10, 24, 2, 4
    lens = [0, 6, 11, 2]
    t, w, q, kt, vt = _case(rng, B, D, K, budget, lens, Hkv, 2, Dh)
    kc, vc, base = _slab(rng, lens, cap, Hkv, Dh)
    c = commit_path(t, w["accept_len"], w["path_nodes"], w["bonus"], kt, vt, kc, vc, base, cap)
    changed = np.flatnonzero((c["k_cache"] != kc).any(axis=(1, 2)))
    expect = sorted(base[b] + lens[b] + j for b in range(B) for j in range(int(w["accept_len"][b]) + 1))
    assert changed.tolist() == expect
    assert np.array_equal(np.flatnonzero((c["v_cache"] != vc).any(axis=(1, 2))), changed)
    assert np.array_equal(c["next_prefix_len"], np.asarray(lens) + w["accept_len"] + 1)
    assert np.array_equal(c["next_root"], w["bonus"])
    # the inputs are not modified
    assert (kc[base[0]:base[0] + cap] == 1234.5).all() or lens[0] > 0


def test_positions_past_capacity_are_not_written():
    rng = np.random.default_rng(8)
    B, D, K, budget, cap, Hkv, Dh = 2, 6, 1, 6, 10, 1, 4
    lens = [7, 2]
    t, w, q, kt, vt = _case(rng, B, D, K, budget, lens, Hkv, 1, Dh, p_follow=1.0)
    assert int(w["accept_len"][0]) == D              # a full chain: positions 7..13
    kc, vc, base = _slab(rng, lens, cap, Hkv, Dh)
    c = commit_path(t, w["accept_len"], w["path_nodes"], w["bonus"], kt, vt, kc, vc, base, cap)
    assert np.array_equal(c["k_cache"][7:10], kt[0, :3])   # positions 7, 8, 9 fit
    # request 0's positions 10.. would land on request 1's slab: its context stays,
    # and its own path follows it
    assert np.array_equal(c["k_cache"][10:12], kc[10:12])
    a1 = int(w["accept_len"][1])
    assert np.array_equal(c["k_cache"][12:13 + a1], kt[1, w["path_nodes"][1, :a1 + 1]])
    assert np.array_equal(c["k_cache"][13 + a1:], kc[13 + a1:])
    assert int(c["next_prefix_len"][0]) == 7 + D + 1
