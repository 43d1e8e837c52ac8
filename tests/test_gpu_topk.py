"""GPU parity of ddtree_draft_topk against the oracle (oracle/topk.py).

Tokens are compared exactly (they come from comparisons of the given logits
only).  Log-probs: the kernel forms logit - log-sum-exp in fp32; the oracle
rounds the exact (float64) value once.  The difference is the fp32 error of
the log-sum-exp (a sum of V exponentials, each within a few ulp, accumulated
over <= 32 terms per thread and then pairwise across threads and slices:
relative error of the sum well below 1e-5 for V = 163840, so an absolute
error below 1e-5 in its logarithm) plus one rounding of the difference
(|lp| < 64: half an ulp is < 4e-6).  The bound used is 2e-5.

Cases: the draft rows of the workloads (fp32 draft logits, K = 2, 4, 8, 4;
every row of the small ones, a seeded sample of rows of the large ones), the
same rows in bf16, heavy ties (quantised logits: the many-candidate path),
a few-way tie at the top (the ranking path with equal values), constant rows,
tiny and odd vocabularies, K = 1 and K = 64.  Then the build fed by the GPU
top-K gives the oracle's tree for those same log-probs, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import assert_tree_equal, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LP_TOL = 2e-5


def _gpu_topk(x, K, bf16=False):
    import tree_verification_build_amd as lib
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    if bf16:
        t = t.to(torch.bfloat16)
    tok, lp = lib.ddtree_draft_topk(t, K)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lp.cpu().numpy(), t


def _check(x, K, rows=None, bf16=False):
    tok, lp, t = _gpu_topk(x, K, bf16)
    xv = t.float().cpu().numpy().reshape(-1, x.shape[-1])
    tok = tok.reshape(-1, K)
    lp = lp.reshape(-1, K)
    sel = range(xv.shape[0]) if rows is None else rows
    err = 0.0
    for r in sel:
        rt, rl = oracle.draft_topk(xv[r][None], K)
        assert np.array_equal(tok[r], rt[0]), (r, tok[r], rt[0])
        e = np.abs(lp[r].astype(np.float64) - rl[0]).max()
        err = max(err, e)
    assert err <= LP_TOL, err
    return err


@pytest.mark.parametrize("name", ["tiny", "single", "batched", "long", "ragged"])
@pytest.mark.parametrize("bf16", [False, True])
def test_draft_topk_workloads(name, bf16):
    cfg = workloads.config(name)
    if name == "ragged":
        cfg = workloads.config(name, B=16)      # 16 x 9 rows of 163840
    inp = workloads.make_inputs(cfg, with_kv=False)
    dl = inp["draft_logits"]                    # [B, D+1, V] fp32
    nrows = dl.shape[0] * dl.shape[1]
    rows = None if nrows <= 20 else np.random.default_rng(7).choice(nrows, 20, replace=False)
    err = _check(dl, cfg.K, rows, bf16)
    say("draft topk", name, "bf16" if bf16 else "f32", "rows", nrows, "max lp err", err)


def test_draft_topk_ties():
    rng = np.random.default_rng(11)
    V = 163840
    x = np.empty((6, V), dtype=np.float32)
    x[0] = rng.integers(-3, 4, V)                       # heavy ties everywhere
    x[1] = 1.25                                         # constant row
    x[2] = rng.normal(0, 3, V)
    x[2, rng.choice(V, 40, replace=False)] = x[2].max() + 1.0   # 40-way tie at the top
    x[3] = rng.normal(0, 3, V)
    x[3, rng.choice(V, 300, replace=False)] = 20.0      # 300-way tie at the top
    x[4] = -0.0                                          # zeros of both signs
    x[4, ::2] = 0.0
    x[5] = rng.normal(0, 1e3, V)                        # large magnitudes
    for K in (1, 4, 8, 64):
        err = _check(x, K)
        say("draft topk ties K", K, "max lp err", err)


@pytest.mark.parametrize("V,K", [(1, 1), (5, 5), (64, 64), (1001, 7), (2049, 3), (70000, 16)])
def test_draft_topk_shapes(V, K):
    rng = np.random.default_rng(V)
    x = rng.normal(0, 3, (3, 2, V)).astype(np.float32)
    _check(x, K)
    _check(x, K, bf16=True)


def test_build_from_gpu_topk_matches_oracle_build():
    """Draft logits -> GPU top-K -> GPU build, against the oracle build of the
    GPU's own top-K (the log-probs feed the build's comparisons bit for bit)."""
    import tree_verification_build_amd as lib
    for name in ("tiny", "batched", "long"):
        cfg = workloads.config(name)
        inp = workloads.make_inputs(cfg, with_kv=False)
        dl = torch.from_numpy(inp["draft_logits"][:, :cfg.D].copy()).to(DEV)
        tok, lp = lib.ddtree_draft_topk(dl, cfg.K)
        root = torch.from_numpy(inp["root_tok"]).to(DEV)
        pre = torch.from_numpy(inp["prefix_len"]).to(DEV)
        tree = lib.ddtree_build(lp, tok, root, pre, cfg.budget)
        torch.cuda.synchronize()
        ref = oracle.build_tree(lp.cpu().numpy(), tok.cpu().numpy(), inp["root_tok"],
                                inp["prefix_len"], cfg.budget)
        got = tree.to_numpy()
        assert_tree_equal(got, ref)
        say("topk -> build", name, "nodes", int(got["num_nodes"].sum()))
