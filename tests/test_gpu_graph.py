"""GPU: the verify step as bench.py times it -- captured once as a HIP graph
and replayed -- gives the eager step's outputs on every replay.

The step (build, tree attention, vocabulary reduction, walk) writes into
buffers allocated before capture, as in bench.py; walk results go to pinned
host memory.  Each case replays the graph several times, with eager work (a
second input set's step) and synchronisations between the replays, and checks
every replay bit for bit against the eager step on the same inputs: tree,
attention output, argmax / max (and R, R_blocks when sampling) and the walk's
outputs.  The eager step itself is checked against the oracle by the parity
tests.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import Case, say

pytestmark = pytest.mark.gpu

CASES = {
    # bf16 greedy, several attention splits per request, sliced vocabulary pass
    "greedy": workloads.config("single", ctx=900, V=40960, seed_index=61),
    # bf16 sampling at T 0.7 over three requests (greedy pass + streamed weights)
    "sampling": workloads.config("batched", B=3, ctx=(700, 1300), V=40960, seed_index=62),
    # the headline workload at full size, in the bench's launch configuration
    "single": workloads.config("single"),
}
REPLAYS = 4


class Step:
    """Persistent buffers and the step of one case (two input sets: the
    case's own and a perturbed copy that the eager work in between uses)."""

    def __init__(self, c, mode):
        import tree_verification_build_amd as lib
        self.lib, self.c, self.mode = lib, c, mode
        cfg = c.cfg
        dev = "cuda:0"
        self.T = cfg.temperature
        self.tree = lib.alloc_tree(cfg.B, cfg.budget, cfg.D, cfg.K, dev)
        self.attn = torch.empty_like(c.d("q"))
        self.ws_a = torch.empty(max(16, lib.ddtree_tree_attention_workspace_size(
            cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, c.inp["ctx_offsets"])), dtype=torch.uint8,
            device=dev)
        self.ws_v = torch.empty(max(16, lib.ddtree_vocab_reduce_workspace_size(
            cfg.B, cfg.N, cfg.V)), dtype=torch.uint8, device=dev)
        res = torch.empty((2, cfg.B), dtype=torch.int32, pin_memory=True)
        self.out = {"accept_len": res[0], "bonus": res[1],
                    "path_nodes": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32, device=dev),
                    "out_tokens": torch.empty((cfg.B, cfg.D + 1), dtype=torch.int32, device=dev)}
        self.am = torch.empty((cfg.B, cfg.N), dtype=torch.int32, device=dev)
        self.mx = torch.empty((cfg.B, cfg.N), dtype=torch.float32, device=dev)
        self.logits = [c.d("logits"), c.d("logits").flip(-1).contiguous()]

    def run(self, which):
        lib, c, t = self.lib, self.c, self.tree
        lib.ddtree_build(c.d("draft_lp"), c.d("draft_tok"), c.d("root_tok"), c.d("prefix_len"),
                         c.cfg.budget, tree=t)
        lib.ddtree_tree_attention(c.d("q"), c.d("k_ctx"), c.d("v_ctx"), c.d("ctx_offsets"),
                                  c.inp["ctx_offsets"], c.d("k_tree"), c.d("v_tree"), t,
                                  out=self.attn, workspace=self.ws_a)
        logits = self.logits[which]
        if self.mode == "fused":
            lib.ddtree_vocab_verify_greedy(logits, t, workspace=self.ws_v, outputs=self.out,
                                           argmax=self.am, maxv=self.mx)
            return {"argmax": self.am, "maxv": self.mx}
        # the vocabulary outputs are allocated by the call (inside a capture,
        # from the graph's own pool): the caller keeps the returned tensors
        v = lib.ddtree_vocab_reduce(logits, t.num_nodes, self.T, workspace=self.ws_v)
        if self.T > 0:
            lib.ddtree_verify_sample(t, logits, v["maxv"], v["R"], v["R_blocks"], self.T,
                                     c.d("uniforms"), outputs=self.out)
        else:
            lib.ddtree_verify_greedy(t, v["argmax"], outputs=self.out)
        return v

    def snapshot(self, v):
        got = {k: np.array(a, copy=True) for k, a in self.tree.to_numpy().items()}
        got["attn"] = self.attn.float().cpu().numpy().copy()
        for k, a in v.items():
            if a is not None:
                got["v_" + k] = a.cpu().numpy().copy()
        for k, v in self.out.items():
            got["o_" + k] = v.cpu().numpy().copy()
        return got


def _equal(a, b, what):
    assert a.keys() == b.keys(), what
    for k in a:
        x, y = np.asarray(a[k]), np.asarray(b[k])
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), (what, k)


@pytest.mark.parametrize("name,mode", [("greedy", "calls"), ("greedy", "fused"),
                                       ("sampling", "calls"), ("single", "calls"),
                                       ("single", "fused")])
def test_step_graph_replays(name, mode):
    c = Case(CASES[name])
    say("graph replay", name, mode, c.cfg)
    st = Step(c, mode)
    v0 = st.run(0)
    torch.cuda.synchronize()
    eager = st.snapshot(v0)
    # the eager step agrees with the oracle on the walk (the parity tests check the rest)
    ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], c.cfg.temperature,
                                dtype=c.cfg.dtype)
    if c.cfg.temperature > 0:
        ref = oracle.verify_sample(c.tree, c.logits, ref_v["maxv"], ref_v["R"],
                                   c.cfg.temperature, c.inp["uniforms"], c.cfg.D,
                                   dtype=c.cfg.dtype)
    else:
        ref = oracle.verify_greedy(c.tree, ref_v["argmax"], c.cfg.D)
    for k in ref:
        assert np.array_equal(eager["o_" + k], ref[k]), k
    v1 = st.run(1)              # the other input set, eagerly
    torch.cuda.synchronize()
    other = st.snapshot(v1)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vg = st.run(0)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        _equal(st.snapshot(vg), eager, f"replay {r}")
        v1 = st.run(1)          # eager work between replays, into the same buffers
        torch.cuda.synchronize()
        _equal(st.snapshot(v1), other, f"eager after replay {r}")
    say("graph replay", name, mode, "ok")
