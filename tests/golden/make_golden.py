"""Writes tests/golden/tiny_oracle.json from the CPU oracle alone (regression fixture).

The pages print no numeric worked example, so the stored values here are the
oracle's own outputs on the seeded tiny workload (batch 1, context 256, 4 heads
of dim 64 in fp32, depth 8, budget 8, top-k cap 2, vocabulary 1024), plus a
sampled walk at T = 0.8.  They guard the oracle against accidental change;
they are not an independent pin.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def compute():
    cfg = workloads.config("tiny")
    inp = oracle.attach_draft_topk(workloads.make_inputs(cfg), cfg.D, cfg.K)
    t = oracle.build_tree(inp["draft_lp"], inp["draft_tok"], inp["root_tok"], inp["prefix_len"],
                          cfg.budget)
    logits, _ = workloads.make_target_logits(cfg, inp, t["depth"], t["num_nodes"])
    o, lse = oracle.tree_attention(inp["q"], inp["k_ctx"], inp["v_ctx"], inp["ctx_offsets"],
                                   inp["k_tree"], inp["v_tree"], t["vis"], t["num_nodes"],
                                   dtype="f32")
    vr = oracle.vocab_reduce(logits, t["num_nodes"], 0.8)
    g = oracle.verify_greedy(t, vr["argmax"], cfg.D)
    s = oracle.verify_sample(t, logits, vr["maxv"], vr["R"], 0.8, inp["uniforms"], cfg.D)
    out = {k: t[k].tolist() for k in ("token", "parent", "depth", "rank", "position",
                                      "first_child", "next_sibling", "num_nodes", "max_depth")}
    out["score_hex"] = [[float(x).hex() for x in row] for row in t["score"]]
    out["vis"] = [[[int(w) for w in n] for n in row] for row in t["vis"]]
    out["argmax"] = vr["argmax"].tolist()
    out["maxv_hex"] = [[float(x).hex() for x in row] for row in vr["maxv"]]
    out["R_T0.8"] = [[int(x) for x in row] for row in vr["R"]]
    out["attn_o_first4_hex"] = [[[[float(x).hex() for x in o[0, n, h, :4]] for h in range(4)]
                                 for n in range(cfg.N)]]
    out["greedy"] = {k: g[k].tolist() for k in g}
    out["sample_T0.8"] = {k: s[k].tolist() for k in s}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(compute(), f, indent=0)
    print("wrote", path)
