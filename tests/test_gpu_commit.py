"""GPU parity of ddtree_commit against the oracle's commit_path (bit-exact).

The tree comes from the GPU build (its parity with the oracle is pinned in
test_gpu_parity), the walk from the GPU greedy walk on a target argmax that
follows a child with high probability (so accept lengths vary up to the full
depth); the oracle replays the same walk from its own tree.  Every byte of the
cache, the next prefix lengths and the next roots must match.  Cases: the small
variants and the full-size workloads, per-request slabs and a compact layout
with negative bases, a capacity that cuts paths, an accept length out of
range, and a two-step loop in which the second step's tree attention reads the
cache the first step committed.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import DEV, assert_attention_close, attn_to_f64, dev_tensor, say
from tests.test_gpu_parity import case

pytestmark = pytest.mark.gpu

NAMES = ["tiny", "bf16_gqa", "bf16_dh64", "f32_dh128", "chain_topk1", "max_nodes", "single",
         "batched", "long", "ragged"]


def _follow_argmax(tree, V, seed, p_follow=0.85):
    """Target argmax: with probability p_follow the token of one of the node's children."""
    rng = np.random.default_rng(seed)
    B, N = tree["token"].shape
    am = rng.integers(0, V, size=(B, N)).astype(np.int32)
    for b in range(B):
        nn = int(tree["num_nodes"][b])
        kids = [[] for _ in range(nn)]
        for c in range(1, nn):
            kids[int(tree["parent"][b, c])].append(c)
        for n in range(nn):
            if kids[n] and rng.random() < p_follow:
                am[b, n] = tree["token"][b, kids[n][rng.integers(0, len(kids[n]))]]
    return am


def _cache(rng, rows, Hkv, Dh, dtype):
    """Random cache contents as storage arrays (uint16 bf16 bits or float32)."""
    if dtype == "bf16":
        return rng.integers(0, 1 << 16, size=(rows, Hkv, Dh), dtype=np.uint16)
    return rng.standard_normal((rows, Hkv, Dh)).astype(np.float32)


def _bits(t, dtype):
    a = t.cpu()
    return a.view(torch.int16).numpy() if dtype == "bf16" else a.view(torch.int32).numpy()


def _run(c, am, base, rows, capacity, seed, invalid=None):
    """invalid: a request whose accept length is set past D before the commit
    (the library then writes nothing for it and returns next prefix -1)."""
    import tree_verification_build_amd as lib
    cfg, i = c.cfg, c.inp
    rng = np.random.default_rng(seed)
    kc0 = _cache(rng, rows, cfg.Hkv, cfg.Dh, cfg.dtype)
    vc0 = _cache(rng, rows, cfg.Hkv, cfg.Dh, cfg.dtype)
    ref_w = oracle.verify_greedy(c.tree, am, cfg.D)
    t = c.gpu_tree()
    w = lib.ddtree_verify_greedy(t, dev_tensor(am, None))
    acc = ref_w["accept_len"].copy()
    if invalid is not None:
        w["accept_len"][invalid] = cfg.D + 1
        acc[invalid] = -1                 # the oracle then commits no row for it
    kc, vc = dev_tensor(kc0, cfg.dtype), dev_tensor(vc0, cfg.dtype)
    nxt, root = lib.ddtree_commit(t, w, c.d("k_tree"), c.d("v_tree"), kc, vc,
                                  torch.from_numpy(base).to(DEV), capacity)
    torch.cuda.synchronize()
    ref = oracle.commit_path(c.tree, acc, ref_w["path_nodes"], ref_w["bonus"],
                             i["k_tree"], i["v_tree"], kc0, vc0, base, capacity)
    if invalid is not None:
        ref["next_prefix_len"][invalid] = -1
    st = "bf16" if cfg.dtype == "bf16" else "f32"
    ref_k = ref["k_cache"].view(np.int16) if st == "bf16" else ref["k_cache"].view(np.int32)
    ref_v = ref["v_cache"].view(np.int16) if st == "bf16" else ref["v_cache"].view(np.int32)
    assert np.array_equal(_bits(kc, st), ref_k), "k_cache"
    assert np.array_equal(_bits(vc, st), ref_v), "v_cache"
    assert np.array_equal(nxt.cpu().numpy(), ref["next_prefix_len"]), "next_prefix_len"
    assert np.array_equal(root.cpu().numpy(), ref["next_root"]), "next_root"
    return ref_w, ref


@pytest.mark.parametrize("name", NAMES)
def test_commit_slabs(name):
    c = case(name)
    cfg = c.cfg
    say("commit slabs", name)
    am = _follow_argmax(c.tree, cfg.V, 100 + len(name))
    lens = c.inp["ctx_lens"].astype(np.int64)
    if cfg.B * (int(lens.max()) + cfg.D + 2) * cfg.Hkv * cfg.Dh > 64 << 20:
        # full-size batches: a compact cache holding only the committed region of
        # each request (base + position starts at row b * (D + 1))
        base = np.arange(cfg.B, dtype=np.int64) * (cfg.D + 1) - lens
        rows = cfg.B * (cfg.D + 1)
    else:
        cap = int(lens.max()) + cfg.D + 2
        base = np.arange(cfg.B, dtype=np.int64) * cap
        rows = cfg.B * cap
    ref_w, _ = _run(c, am, base, rows, 1 << 30, seed=7)
    assert ref_w["accept_len"].max() >= min(cfg.D, 2)


@pytest.mark.parametrize("name", ["bf16_gqa", "max_nodes"])
def test_commit_capacity_and_bad_accept_len(name):
    c = case(name)
    cfg = c.cfg
    say("commit capacity", name)
    am = _follow_argmax(c.tree, cfg.V, 5, p_follow=1.0)
    lens = c.inp["ctx_lens"].astype(np.int64)
    cap = int(lens.min()) + 3          # the shortest request keeps 3 path rows, longer ones none
    base = np.arange(cfg.B, dtype=np.int64) * (int(lens.max()) + cfg.D + 2)
    rows = int(base[-1]) + int(lens.max()) + cfg.D + 2
    _run(c, am, base, rows, cap, seed=8)
    # an accept length outside [0, D]: nothing written, next prefix -1
    _run(c, am, base, rows, 1 << 30, seed=9, invalid=0)


def test_commit_then_next_step_attention():
    """Step 1 commits into the context buffer; step 2's tree attention reads it."""
    import tree_verification_build_amd as lib
    cfg = workloads.config("single", ctx=700, V=4096, seed_index=31)
    c = case_cfg(cfg)
    say("commit two-step")
    i = c.inp
    L = int(i["ctx_lens"][0])
    cap = L + 2 * (cfg.D + 1)
    kc0 = np.zeros((cap, cfg.Hkv, cfg.Dh), np.uint16)
    vc0 = np.zeros((cap, cfg.Hkv, cfg.Dh), np.uint16)
    kc0[:L], vc0[:L] = i["k_ctx"], i["v_ctx"]
    am = _follow_argmax(c.tree, cfg.V, 11, p_follow=1.0)
    ref_w = oracle.verify_greedy(c.tree, am, cfg.D)
    ref = oracle.commit_path(c.tree, ref_w["accept_len"], ref_w["path_nodes"], ref_w["bonus"],
                             i["k_tree"], i["v_tree"], kc0, vc0, np.zeros(1, np.int64), cap)
    t = c.gpu_tree()
    w = lib.ddtree_verify_greedy(t, dev_tensor(am, None))
    kc, vc = dev_tensor(kc0, "bf16"), dev_tensor(vc0, "bf16")
    prefix, root = lib.ddtree_commit(t, w, c.d("k_tree"), c.d("v_tree"), kc, vc,
                                     torch.zeros(1, dtype=torch.int64, device=DEV), cap)
    # step 2: a new tree at the committed prefix, new queries and tree K/V
    L2 = int(ref["next_prefix_len"][0])
    assert L2 == L + int(ref_w["accept_len"][0]) + 1 and L2 > L + 1
    rng = np.random.default_rng(12)
    q2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["q"].shape).astype(np.float32))
    kt2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["k_tree"].shape).astype(np.float32))
    vt2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["v_tree"].shape).astype(np.float32))
    tree2 = oracle.build_tree(i["draft_lp"], i["draft_tok"], ref["next_root"],
                              ref["next_prefix_len"], cfg.budget)
    t2 = lib.ddtree_build(c.d("draft_lp"), c.d("draft_tok"), root, prefix, cfg.budget)
    offs2 = np.array([0, L2], np.int32)
    o2, _ = lib.ddtree_tree_attention(dev_tensor(q2, "bf16"), kc, vc, dev_tensor(offs2, None),
                                      offs2, dev_tensor(kt2, "bf16"), dev_tensor(vt2, "bf16"), t2)
    torch.cuda.synchronize()
    assert np.array_equal(t2.position.cpu().numpy(), tree2["position"])
    o_ref, _ = oracle.tree_attention(q2, ref["k_cache"][:L2], ref["v_cache"][:L2], offs2, kt2, vt2,
                                     tree2["vis"], tree2["num_nodes"], dtype="bf16")
    assert_attention_close(attn_to_f64(o2), o_ref, "bf16")


_cfg_cache = {}


def case_cfg(cfg):
    from tests.gpu_cases import Case
    key = repr(cfg)
    if key not in _cfg_cache:
        _cfg_cache[key] = Case(cfg)
    return _cfg_cache[key]
