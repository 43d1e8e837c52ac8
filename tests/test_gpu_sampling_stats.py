"""Sampled verification on the GPU reproduces the target softmax (chi-square).

A tiny fixed tree (depth 3, top-k cap 2, budget 5) over a 16-token vocabulary
is replicated across 40000 requests that differ only in their uniforms, so
one call of each kernel draws 40000 independent samples.  The first emitted
token must follow the target law w/R at the root, and the token after an
accepted child c the law at c ("Dissecting DDTree's Tree-Parallel Evaluation
Strategy", Section 3: tree rejection sampling keeps the target distribution).
"""
import numpy as np
import pytest
import torch
from scipy.stats import chisquare

import oracle
from tests.gpu_cases import dev_tensor, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [0.7, 1.0])
def test_gpu_sampling_chi_square(T):
    import tree_verification_build_amd as lib
    B, V, N = 40000, 16, 6
    lp = np.array([[-0.3, -1.2], [-0.4, -1.5], [-0.2, -2.0]], dtype=np.float32)
    tok = np.array([[3, 7], [5, 1], [9, 2]], dtype=np.int32)
    rng = np.random.default_rng(int(T * 1000))
    row_logits = rng.standard_normal((N, V)).astype(np.float32)
    say("chi-square", T, B)
    t = lib.ddtree_build(dev_tensor(np.broadcast_to(lp, (B, 3, 2)).copy(), None),
                         dev_tensor(np.broadcast_to(tok, (B, 3, 2)).copy(), None),
                         dev_tensor(np.zeros(B, np.int32), None),
                         dev_tensor(np.zeros(B, np.int32), None), 5)
    logits = dev_tensor(np.broadcast_to(row_logits, (B, N, V)).copy(), None)
    u = rng.integers(0, 2 ** 64, size=(B, N, 2), dtype=np.uint64)
    v = lib.ddtree_vocab_reduce(logits, t.num_nodes, T)
    o = lib.ddtree_verify_sample(t, logits, v["maxv"], v["R"], v["R_blocks"], T,
                                 dev_tensor(u, None))
    torch.cuda.synchronize()
    tree1 = oracle.build_tree(lp[None], tok[None], np.array([0]), np.array([0]), 5)
    vr = oracle.vocab_reduce(row_logits[None], tree1["num_nodes"], T)
    c, a = oracle.weight_constants(T)
    law = [oracle.weights(row_logits[n], vr["maxv"][0, n], c, a).astype(np.float64) /
           float(vr["R"][0, n]) for n in range(N)]
    toks = o["out_tokens"].cpu().numpy()
    acc = o["accept_len"].cpu().numpy()
    path = o["path_nodes"].cpu().numpy()
    first = np.bincount(toks[:, 0], minlength=V)
    assert chisquare(first, law[0] * B).pvalue > 1e-4
    for node in np.unique(path[acc >= 1, 1]):
        sel = (acc >= 1) & (path[:, 1] == node)
        if sel.sum() < 5000:
            continue
        counts = np.bincount(toks[sel, 1], minlength=V)
        exp = law[node] * sel.sum()
        keep = exp > 5
        obs, ex = counts[keep], exp[keep]
        if (~keep).any() and exp[~keep].sum() > 0:          # lump the rare cells together
            obs = np.append(obs, counts[~keep].sum())
            ex = np.append(ex, exp[~keep].sum())
        assert chisquare(obs, ex * obs.sum() / ex.sum()).pvalue > 1e-4
