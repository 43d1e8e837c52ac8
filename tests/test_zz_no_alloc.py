"""ddtree_tree_attention_noalloc (split partials in the library's device array,
for callers that cannot allocate) against ddtree_tree_attention with a caller
workspace: same kernels and plan, so outputs and lse must match bit for bit;
two calls in a row, the second on a smaller input, then a third on the first
input again (the array keeps the last call's contents, which no call reads)."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_cases import Case, say

pytestmark = pytest.mark.gpu

CASES = [
    ("single", workloads.config("single")),
    ("small_gqa", workloads.config("ragged", B=3, ctx=(300, 900), Hq=8, Hkv=2, Dh=128, V=1024,
                                   plant=True, seed_index=61)),
    ("small_f32", workloads.config("tiny", B=2, ctx=(100, 700), Hq=2, Hkv=2, Dh=64,
                                   seed_index=62)),
]


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def _both(c):
    import tree_verification_build_amd as lib
    t = c.gpu_tree()
    ref, ref_lse = c.gpu_attention(t, want_lse=True)
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    ws_need = lib.ddtree_tree_attention_workspace_size(c.cfg.B, c.cfg.N, c.cfg.Hq, c.cfg.Hkv,
                                                       c.cfg.Dh, c.inp["ctx_offsets"])
    say("noalloc attention", c.cfg.name, "B", c.cfg.B, "partials bytes", ws_need)
    lib.ddtree_tree_attention_noalloc(c.d("q"), c.d("k_ctx"), c.d("v_ctx"), c.d("ctx_offsets"),
                                      c.inp["ctx_offsets"], c.d("k_tree"), c.d("v_tree"), t,
                                      out=out, lse=lse)
    torch.cuda.synchronize()
    return ref, ref_lse, out, lse, ws_need


def test_noalloc_matches_workspace_form_two_calls_then_smaller():
    cases = [Case(cfg) for _, cfg in CASES]
    needs = []
    for c in cases + cases[:1]:
        ref, ref_lse, out, lse, need = _both(c)
        needs.append(need)
        assert torch.equal(_bits(out), _bits(ref)), c.cfg.name
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), c.cfg.name
    # the sequence ran a multi-split plan, then smaller ones (the second call's input is smaller)
    assert needs[0] > needs[1] > 0


def test_noalloc_in_a_graph_replayed():
    """Captured once into a HIP graph and replayed with other inputs copied into
    the captured buffers between replays: every replay equals the eager call."""
    import tree_verification_build_amd as lib
    cfg = workloads.config("ragged", B=4, ctx=(500, 2500), Hq=8, Hkv=8, Dh=128, V=1024,
                           seed_index=63)
    c = Case(cfg)
    t = c.gpu_tree()
    q = c.d("q").clone()
    out = torch.empty_like(q)
    args = (c.d("k_ctx"), c.d("v_ctx"), c.d("ctx_offsets"), c.inp["ctx_offsets"], c.d("k_tree"),
            c.d("v_tree"), t)
    lib.ddtree_tree_attention_noalloc(q, *args, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.ddtree_tree_attention_noalloc(q, *args, out=out)
    gen = torch.Generator(device="cpu").manual_seed(5)
    for rep in range(3):
        q.copy_(torch.randn(q.shape, generator=gen).to(q.dtype))
        say("noalloc graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        ref, _ = lib.ddtree_tree_attention(q, *args)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(ref)), rep
