"""A chained decode loop on the GPU against the oracle's own chain.

Every step runs the whole verify step on the state that the previous step
left: the best-first build from the previous bonus token (the root) and prefix
length; the tree attention of every node over its request's cache slab
(ddtree_tree_attention_ranges, its split plan made anew from the grown
lengths) and over its ancestors; the vocabulary pass; the walk (greedy, or
rejection sampling at temperature T); and ddtree_commit, which appends the
accepted path's K/V to the slabs and gives the next (prefix length, root).
The oracle runs the same chain from its own outputs: build_tree, tree_attention
over the packed copy of its slabs, vocab_reduce, verify_greedy / verify_sample,
commit_path.  Per step the trees, the walks and the next (prefix length, root)
agree bit for bit and the attention within its tolerance; at the end every
byte of the slabs does.

Per-step inputs come from the seeded generators (a seed per step): draft
logits and their top-K (the oracle's draft_topk, fed to both sides), the
nodes' q / k / v, target logits planted on the step's tree shape (which
depends only on the draft log-probs), the uniforms.  Slab rows outside a
request's committed range hold NaN, so a read outside the range poisons the
output.  Cases: bf16 with grouped heads and sampling, bf16 greedy, fp32
greedy at head_dim 64, and a batch of 66 requests (past 64 the splits are
looked up on the device) — with empty contexts at the start in the ragged ones.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import DEV, assert_attention_close, assert_tree_equal, attn_to_f64, \
    dev_tensor, say

pytestmark = pytest.mark.gpu

CASES = {
    "sample_bf16_gqa": (workloads.config("ragged", B=4, ctx=(0, 700), Hq=8, Hkv=2, Dh=128,
                                         V=2048, temperature=1.0, plant=True, seed_index=61),
                        10),
    "greedy_bf16": (workloads.config("batched", B=3, ctx=300, Hq=4, Hkv=4, Dh=128, V=2048,
                                     temperature=0.0, plant=True, seed_index=62), 8),
    "greedy_f32_dh64": (workloads.config("tiny", B=2, ctx=(0, 200), Hq=4, Hkv=2, Dh=64,
                                         V=1024, D=6, budget=20, K=3, temperature=0.0,
                                         plant=True, seed_index=63), 8),
    "sample_b66_bf16": (workloads.config("ragged", B=66, ctx=(0, 200), Hq=2, Hkv=2, Dh=128,
                                         V=512, D=4, budget=12, K=3, temperature=0.7,
                                         plant=True, seed_index=64), 8),
}


def _fill(rows, Hkv, Dh, dtype):
    if dtype == "bf16":
        return np.full((rows, Hkv, Dh), 0x7FC0, dtype=np.uint16)
    return np.full((rows, Hkv, Dh), np.nan, dtype=np.float32)


def _bits(t, dtype):
    a = t.cpu()
    return a.view(torch.int16).numpy() if dtype == "bf16" else a.view(torch.int32).numpy()


def _step_inputs(cfg, s):
    """The seeded inputs of step s (a seed of their own per step)."""
    c = dataclasses.replace(cfg, seed_index=cfg.seed_index * 100 + s)
    return oracle.attach_draft_topk(workloads.make_inputs(c), c.D, c.K), c


@pytest.mark.parametrize("name", list(CASES))
def test_decode_loop_matches_oracle_chain(name):
    import tree_verification_build_amd as lib
    cfg, steps = CASES[name]
    B, D, T, dt = cfg.B, cfg.D, cfg.temperature, cfg.dtype
    inp0 = workloads.make_inputs(cfg)
    lens = inp0["ctx_lens"].astype(np.int64)
    cap = int(lens.max()) + steps * (D + 1) + 1
    base = np.arange(B, dtype=np.int64) * cap
    k_ref = _fill(B * cap, cfg.Hkv, cfg.Dh, dt)
    v_ref = _fill(B * cap, cfg.Hkv, cfg.Dh, dt)
    offs = inp0["ctx_offsets"]
    for b in range(B):
        k_ref[base[b]:base[b] + lens[b]] = inp0["k_ctx"][offs[b]:offs[b + 1]]
        v_ref[base[b]:base[b] + lens[b]] = inp0["v_ctx"][offs[b]:offs[b + 1]]
    prefix_ref = inp0["prefix_len"].astype(np.int32)
    root_ref = inp0["root_tok"].astype(np.int32)
    # the GPU chain's state: its own slabs, prefix lengths and roots
    kc, vc = dev_tensor(k_ref, dt), dev_tensor(v_ref, dt)
    base_d = torch.from_numpy(base).to(DEV)
    start_h = base.astype(np.int32)
    start_d = torch.from_numpy(start_h).to(DEV)
    prefix_d = torch.from_numpy(prefix_ref.copy()).to(DEV)
    root_d = torch.from_numpy(root_ref.copy()).to(DEV)
    accepted = 0
    for s in range(steps):
        say("decode loop", name, "step", s, "prefix", prefix_ref[:4].tolist())
        i, cs = _step_inputs(cfg, s)
        # oracle step
        tree = oracle.build_tree(i["draft_lp"], i["draft_tok"], root_ref, prefix_ref, cfg.budget)
        logits, _ = workloads.make_target_logits(cs, i, tree["depth"], tree["num_nodes"])
        pk = np.concatenate([k_ref[base[b]:base[b] + prefix_ref[b]] for b in range(B)])
        pv = np.concatenate([v_ref[base[b]:base[b] + prefix_ref[b]] for b in range(B)])
        poffs = np.concatenate([[0], np.cumsum(prefix_ref)]).astype(np.int32)
        o_ref, _ = oracle.tree_attention(i["q"], pk, pv, poffs, i["k_tree"], i["v_tree"],
                                         tree["vis"], tree["num_nodes"], dtype=dt)
        vr = oracle.vocab_reduce(logits, tree["num_nodes"], T, dtype=dt)
        if T > 0:
            w_ref = oracle.verify_sample(tree, logits, vr["maxv"], vr["R"], T, i["uniforms"], D,
                                         dtype=dt)
        else:
            w_ref = oracle.verify_greedy(tree, vr["argmax"], D)
        cm = oracle.commit_path(tree, w_ref["accept_len"], w_ref["path_nodes"], w_ref["bonus"],
                                i["k_tree"], i["v_tree"], k_ref, v_ref, base, cap)
        # GPU step on the GPU chain's own state; the host copy of the lengths is
        # the GPU's (read back after the previous step, as a serving loop does)
        prefix_h = prefix_d.cpu().numpy()
        t = lib.ddtree_build(dev_tensor(i["draft_lp"], None), dev_tensor(i["draft_tok"], None),
                             root_d, prefix_d, cfg.budget)
        kt, vt = dev_tensor(i["k_tree"], dt), dev_tensor(i["v_tree"], dt)
        o, _ = lib.ddtree_tree_attention_ranges(dev_tensor(i["q"], dt), kc, vc, start_d, prefix_d,
                                                start_h, prefix_h, kt, vt, t)
        lg = dev_tensor(logits, dt)
        v = lib.ddtree_vocab_reduce(lg, t.num_nodes, T)
        if T > 0:
            w = lib.ddtree_verify_sample(t, lg, v["maxv"], v["R"], v["R_blocks"], T,
                                         dev_tensor(i["uniforms"], None))
        else:
            w = lib.ddtree_verify_greedy(t, v["argmax"])
        prefix_d, root_d = lib.ddtree_commit(t, w, kt, vt, kc, vc, base_d, cap)
        torch.cuda.synchronize()
        assert_tree_equal(t.to_numpy(), tree)
        assert_attention_close(attn_to_f64(o), o_ref, dt)
        for k in w_ref:
            assert np.array_equal(w[k].cpu().numpy(), w_ref[k]), (s, k)
        assert np.array_equal(prefix_d.cpu().numpy(), cm["next_prefix_len"]), s
        assert np.array_equal(root_d.cpu().numpy(), cm["next_root"]), s
        k_ref, v_ref = cm["k_cache"], cm["v_cache"]
        prefix_ref, root_ref = cm["next_prefix_len"], cm["next_root"]
        accepted += int(w_ref["accept_len"].sum())
    assert accepted > 0
    assert np.array_equal(_bits(kc, dt), k_ref.view(np.int16 if dt == "bf16" else np.int32))
    assert np.array_equal(_bits(vc, dt), v_ref.view(np.int16 if dt == "bf16" else np.int32))


@pytest.mark.parametrize("name", ["sample_bf16_gqa", "greedy_bf16", "greedy_f32_dh64"])
def test_decode_loop_graph_matches_oracle_chain(name):
    """The same chain with each GPU step a replayed HIP graph, captured once
    per step parity before the loop: the attention is
    ddtree_tree_attention_ranges_capped (the lengths read on the device, the
    slab capacities as bounds), the walk writes accept_len and bonus to pinned
    host memory and ddtree_commit reads them there, and the (prefix length,
    root) and walk buffers alternate between steps.  Each step's inputs are
    copied into the captured buffers before its replay; nothing is planned or
    read back on the host."""
    import tree_verification_build_amd as lib
    cfg, steps = CASES[name]
    B, D, T, dt = cfg.B, cfg.D, cfg.temperature, cfg.dtype
    inp0 = workloads.make_inputs(cfg)
    lens = inp0["ctx_lens"].astype(np.int64)
    cap = int(lens.max()) + steps * (D + 1) + 1
    base = np.arange(B, dtype=np.int64) * cap
    k_ref = _fill(B * cap, cfg.Hkv, cfg.Dh, dt)
    v_ref = _fill(B * cap, cfg.Hkv, cfg.Dh, dt)
    offs = inp0["ctx_offsets"]
    for b in range(B):
        k_ref[base[b]:base[b] + lens[b]] = inp0["k_ctx"][offs[b]:offs[b + 1]]
        v_ref[base[b]:base[b] + lens[b]] = inp0["v_ctx"][offs[b]:offs[b + 1]]
    prefix_ref = inp0["prefix_len"].astype(np.int32)
    root_ref = inp0["root_tok"].astype(np.int32)
    kc, vc = dev_tensor(k_ref, dt), dev_tensor(v_ref, dt)
    base_d = torch.from_numpy(base).to(DEV)
    start_h = base.astype(np.int32)
    caps_h = np.full(B, cap, dtype=np.int32)
    start_d = torch.from_numpy(start_h).to(DEV)
    prefix_d = [torch.from_numpy(prefix_ref.copy()).to(DEV), torch.zeros(B, dtype=torch.int32,
                                                                          device=DEV)]
    root_d = [torch.from_numpy(root_ref.copy()).to(DEV), torch.zeros(B, dtype=torch.int32,
                                                                      device=DEV)]
    # the captured input buffers, filled before every replay
    i0, c0 = _step_inputs(cfg, 0)
    tree0 = oracle.build_tree(i0["draft_lp"], i0["draft_tok"], root_ref, prefix_ref, cfg.budget)
    logits0, _ = workloads.make_target_logits(c0, i0, tree0["depth"], tree0["num_nodes"])
    buf = {"draft_lp": dev_tensor(i0["draft_lp"], None), "draft_tok": dev_tensor(i0["draft_tok"], None),
           "q": dev_tensor(i0["q"], dt), "k_tree": dev_tensor(i0["k_tree"], dt),
           "v_tree": dev_tensor(i0["v_tree"], dt), "logits": dev_tensor(logits0, dt),
           "uniforms": dev_tensor(i0["uniforms"], None)}
    t = lib.alloc_tree(B, cfg.budget, D, cfg.K, DEV)
    attn = torch.empty_like(buf["q"])
    ws_a = torch.empty(max(16, lib.ddtree_tree_attention_ranges_workspace_size(
        B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, caps_h)), dtype=torch.uint8, device=DEV)
    ws_v = torch.empty(max(16, lib.ddtree_vocab_reduce_workspace_size(B, cfg.N, cfg.V)),
                       dtype=torch.uint8, device=DEV)
    walks = [{"accept_len": torch.empty((B,), dtype=torch.int32, pin_memory=True),
              "bonus": torch.empty((B,), dtype=torch.int32, pin_memory=True),
              "path_nodes": torch.empty((B, D + 1), dtype=torch.int32, device=DEV),
              "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=DEV)}
             for _ in range(2)]
    keep = []

    def step(p):
        lib.ddtree_build(buf["draft_lp"], buf["draft_tok"], root_d[p], prefix_d[p], cfg.budget,
                         tree=t)
        lib.ddtree_tree_attention_ranges_capped(buf["q"], kc, vc, start_d, prefix_d[p], start_h,
                                                caps_h, buf["k_tree"], buf["v_tree"], t,
                                                out=attn, workspace=ws_a)
        v = lib.ddtree_vocab_reduce(buf["logits"], t.num_nodes, T, workspace=ws_v)
        keep.append(v)
        if T > 0:
            lib.ddtree_verify_sample(t, buf["logits"], v["maxv"], v["R"], v["R_blocks"], T,
                                     buf["uniforms"], outputs=walks[p])
        else:
            lib.ddtree_verify_greedy(t, v["argmax"], outputs=walks[p])
        lib.ddtree_commit(t, walks[p], buf["k_tree"], buf["v_tree"], kc, vc, base_d, cap,
                          next_prefix_len=prefix_d[1 - p], next_root=root_d[1 - p])

    graphs = []
    for p in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(p)
        graphs.append(g)
    torch.cuda.synchronize()
    accepted = 0
    for s in range(steps):
        say("decode loop graph", name, "step", s, "prefix", prefix_ref[:4].tolist())
        i, cs = _step_inputs(cfg, s)
        tree = oracle.build_tree(i["draft_lp"], i["draft_tok"], root_ref, prefix_ref, cfg.budget)
        logits, _ = workloads.make_target_logits(cs, i, tree["depth"], tree["num_nodes"])
        pk = np.concatenate([k_ref[base[b]:base[b] + prefix_ref[b]] for b in range(B)])
        pv = np.concatenate([v_ref[base[b]:base[b] + prefix_ref[b]] for b in range(B)])
        poffs = np.concatenate([[0], np.cumsum(prefix_ref)]).astype(np.int32)
        o_ref, _ = oracle.tree_attention(i["q"], pk, pv, poffs, i["k_tree"], i["v_tree"],
                                         tree["vis"], tree["num_nodes"], dtype=dt)
        vr = oracle.vocab_reduce(logits, tree["num_nodes"], T, dtype=dt)
        if T > 0:
            w_ref = oracle.verify_sample(tree, logits, vr["maxv"], vr["R"], T, i["uniforms"], D,
                                         dtype=dt)
        else:
            w_ref = oracle.verify_greedy(tree, vr["argmax"], D)
        cm = oracle.commit_path(tree, w_ref["accept_len"], w_ref["path_nodes"], w_ref["bonus"],
                                i["k_tree"], i["v_tree"], k_ref, v_ref, base, cap)
        for k, a in (("draft_lp", i["draft_lp"]), ("draft_tok", i["draft_tok"]),
                     ("uniforms", i["uniforms"])):
            buf[k].copy_(dev_tensor(a, None))
        for k, a in (("q", i["q"]), ("k_tree", i["k_tree"]), ("v_tree", i["v_tree"]),
                     ("logits", logits)):
            buf[k].copy_(dev_tensor(a, dt))
        p = s % 2
        graphs[p].replay()
        torch.cuda.synchronize()
        assert_tree_equal(t.to_numpy(), tree)
        assert_attention_close(attn_to_f64(attn), o_ref, dt)
        for k in w_ref:
            assert np.array_equal(walks[p][k].cpu().numpy(), w_ref[k]), (s, k)
        assert np.array_equal(prefix_d[1 - p].cpu().numpy(), cm["next_prefix_len"]), s
        assert np.array_equal(root_d[1 - p].cpu().numpy(), cm["next_root"]), s
        k_ref, v_ref = cm["k_cache"], cm["v_cache"]
        prefix_ref, root_ref = cm["next_prefix_len"], cm["next_root"]
        accepted += int(w_ref["accept_len"].sum())
    assert accepted > 0
    assert np.array_equal(_bits(kc, dt), k_ref.view(np.int16 if dt == "bf16" else np.int32))
    assert np.array_equal(_bits(vc, dt), v_ref.view(np.int16 if dt == "bf16" else np.int32))
