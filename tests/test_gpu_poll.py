"""GPU: every walk stores accept_len last, after its other outputs and a
system-scope release, so a host polling accept_len in pinned memory can read
the rest as soon as it changes, without a stream synchronisation.

Each case puts all of a walk's outputs in pinned host memory, computes the
reference outputs with a synchronised call (checked against the oracle by
the parity tests), then repeats: fill the outputs with sentinels (accept_len
-1, the others -7), launch the walk (a replayed HIP graph of the step, or the
walk call itself), spin on accept_len until every entry is >= 0, and read the
other outputs at once, before any synchronisation.  Every read must equal the
reference: a walk that stored accept_len before the rest would show the
sentinels.
"""
import time

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_cases import DEV, Case, say

pytestmark = pytest.mark.gpu

ROUNDS = 40


def _pinned_outputs(B, D, with_path=True):
    out = {"accept_len": torch.empty((B,), dtype=torch.int32, pin_memory=True),
           "bonus": torch.empty((B,), dtype=torch.int32, pin_memory=True),
           "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, pin_memory=True)}
    if with_path:
        out["path_nodes"] = torch.empty((B, D + 1), dtype=torch.int32, pin_memory=True)
    return out


def _poll_rounds(launch, out, ref, what):
    views = {k: v.numpy() for k, v in out.items()}
    acc = views["accept_len"]
    for r in range(ROUNDS):
        for k, v in views.items():
            v.fill(-1 if k == "accept_len" else -7)
        launch()
        t0 = time.perf_counter()
        while (acc < 0).any():
            assert time.perf_counter() - t0 < 5.0, f"{what}: no accept lengths after 5 s"
        got = {k: v.copy() for k, v in views.items()}      # before any synchronisation
        torch.cuda.synchronize()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (what, r, k, got[k], ref[k])


def _greedy_case():
    return Case(workloads.config("single", ctx=900, V=40960, seed_index=71))


def _sampling_case():
    return Case(workloads.config("batched", B=3, ctx=(700, 1300), V=40960, seed_index=72))


@pytest.mark.parametrize("mode", ["fused", "calls"])
def test_poll_greedy_step_graph(mode):
    """The greedy step captured as one graph (build, attention, vocabulary, walk)."""
    import tree_verification_build_amd as lib
    c = _greedy_case()
    cfg = c.cfg
    say("poll greedy", mode, cfg)
    t = lib.alloc_tree(cfg.B, cfg.budget, cfg.D, cfg.K, DEV)
    attn = torch.empty_like(c.d("q"))
    ws_a = torch.empty(max(16, lib.ddtree_tree_attention_workspace_size(
        cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, c.inp["ctx_offsets"])), dtype=torch.uint8,
        device=DEV)
    ws_v = torch.empty(max(16, lib.ddtree_vocab_reduce_workspace_size(cfg.B, cfg.N, cfg.V)),
                       dtype=torch.uint8, device=DEV)
    am = torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=DEV)
    mx = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=DEV)
    out = _pinned_outputs(cfg.B, cfg.D)
    keep = {}

    def step():
        lib.ddtree_build(c.d("draft_lp"), c.d("draft_tok"), c.d("root_tok"), c.d("prefix_len"),
                         cfg.budget, tree=t)
        lib.ddtree_tree_attention(c.d("q"), c.d("k_ctx"), c.d("v_ctx"), c.d("ctx_offsets"),
                                  c.inp["ctx_offsets"], c.d("k_tree"), c.d("v_tree"), t,
                                  out=attn, workspace=ws_a)
        if mode == "fused":
            lib.ddtree_vocab_verify_greedy(c.d("logits"), t, workspace=ws_v, outputs=out,
                                           argmax=am, maxv=mx)
        else:
            keep["v"] = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, 0.0, workspace=ws_v)
            lib.ddtree_verify_greedy(t, keep["v"]["argmax"], outputs=out)

    step()
    torch.cuda.synchronize()
    ref = {k: v.numpy().copy() for k, v in out.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    _poll_rounds(g.replay, out, ref, f"greedy {mode}")
    say("poll greedy", mode, "accept", ref["accept_len"].tolist(), "ok")


@pytest.mark.parametrize("walk", ["sample", "lazy", "top_p"])
def test_poll_sampled_walks(walk):
    """The sampled walks, launched eagerly after a synchronised vocabulary pass."""
    import tree_verification_build_amd as lib
    c = _sampling_case()
    cfg = c.cfg
    T = cfg.temperature
    say("poll sampled", walk, cfg)
    t = c.gpu_tree()
    lg = c.d("logits")
    v = lib.ddtree_vocab_reduce(lg, t.num_nodes, T)
    nuc = lib.ddtree_vocab_top_p(lg, t.num_nodes, v["maxv"], v["R"], T, 0.9) if walk == "top_p" \
        else None
    torch.cuda.synchronize()
    out = _pinned_outputs(cfg.B, cfg.D)

    def launch():
        if walk == "sample":
            lib.ddtree_verify_sample(t, lg, v["maxv"], v["R"], v["R_blocks"], T, c.d("uniforms"),
                                     outputs=out)
        elif walk == "lazy":
            lib.ddtree_verify_sample_lazy(t, lg, T, c.d("uniforms"), outputs=out)
        else:
            lib.ddtree_verify_sample_top_p(t, lg, v["maxv"], nuc, T, c.d("uniforms"), outputs=out)

    launch()
    torch.cuda.synchronize()
    ref = {k: x.numpy().copy() for k, x in out.items()}
    _poll_rounds(launch, out, ref, walk)
    say("poll sampled", walk, "accept", ref["accept_len"].tolist(), "ok")


def test_poll_linear_sample():
    import tree_verification_build_amd as lib
    B, D, V, T = 4, 6, 9000, 0.8
    rng = np.random.default_rng(73)
    dl = rng.normal(0, 3, (B, D + 1, V)).astype(np.float32)
    tl = (dl + rng.normal(0, 0.5, dl.shape)).astype(np.float32)
    x = rng.integers(0, V, size=(B, D)).astype(np.int32)
    u = rng.integers(0, 2 ** 62, size=(B, D + 1, 2), dtype=np.int64)
    tg, dg = torch.from_numpy(tl).to(DEV), torch.from_numpy(dl[:, :D].copy()).to(DEV)
    xg, ug = torch.from_numpy(x).to(DEV), torch.from_numpy(u).to(DEV)
    out = _pinned_outputs(B, D, with_path=False)

    def launch():
        lib.ddtree_verify_linear_sample(tg, dg, xg, T, ug, outputs=out)

    launch()
    torch.cuda.synchronize()
    ref = {k: v.numpy().copy() for k, v in out.items()}
    _poll_rounds(launch, out, ref, "linear")
    say("poll linear", "accept", ref["accept_len"].tolist(), "ok")
