"""GPU parity of ddtree_verify_linear_sample against the oracle
(oracle/linear.py): accept length, emitted tokens and bonus bit for bit.

Inputs: seeded target and draft logits (the target = the draft plus noise, so
acceptances and rejections both occur), drafted tokens drawn from the draft's
exact law w/R (through the oracle's weights), raw 64-bit uniforms.  Cases:
fp32 and bf16, odd and full-size vocabularies, chains of 1 to 8 tokens, equal
draft and target (every token accepted: the bonus path), a target that gives
the drafted token no mass (always rejected), and the uniform extremes.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _law(row, T):
    c, a = oracle.weight_constants(T)
    w = oracle.weights(row, row.max() + np.float32(0.0), c, a).astype(np.float64)
    return w / w.sum()


def _inputs(B, D, V, T, seed, noise=1.0, same=False):
    rng = np.random.default_rng(seed)
    dl = rng.normal(0, 3, (B, D + 1, V)).astype(np.float32)
    tl = dl if same else (dl + rng.normal(0, noise, dl.shape)).astype(np.float32)
    draft = dl[:, :D].copy()
    x = np.stack([[rng.choice(V, p=_law(draft[b, k], T)) for k in range(D)] for b in range(B)])
    u = rng.integers(0, 2 ** 63, size=(B, D + 1, 2), dtype=np.int64).astype(np.uint64) * np.uint64(2)
    return tl, draft, x.astype(np.int32), u


def _run(tl, dl, x, u, T, dtype):
    import tree_verification_build_amd as lib
    if dtype == "bf16":
        tb, db = workloads.f32_to_bf16_bits(tl), workloads.f32_to_bf16_bits(dl)
        tg = torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).to(DEV)
        dg = torch.from_numpy(db.view(np.int16)).view(torch.bfloat16).to(DEV)
        tref, dref = tb, db
    else:
        tg, dg = torch.from_numpy(tl).to(DEV), torch.from_numpy(dl).to(DEV)
        tref, dref = tl, dl
    o = lib.ddtree_verify_linear_sample(tg, dg, torch.from_numpy(x).to(DEV), T,
                                        torch.from_numpy(u.view(np.int64)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.verify_linear_sample(tref, dref, x, T, u, dtype=dtype)
    for k in ref:
        assert np.array_equal(o[k].cpu().numpy(), ref[k]), (k, o[k].cpu().numpy(), ref[k])
    return ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,D,V,T", [(5, 1, 1001, 1.0), (5, 3, 4096, 0.7), (3, 8, 9000, 1.0),
                                     (2, 8, 40000, 0.5)])
def test_linear_sample_parity(dtype, B, D, V, T):
    tl, dl, x, u = _inputs(B, D, V, T, seed=V + D)
    ref = _run(tl, dl, x, u, T, dtype)
    say("linear sample", dtype, B, D, V, T, "accept", ref["accept_len"].tolist())


@pytest.mark.parametrize("noise", [0.05, 1.5])
def test_linear_sample_full_vocab(noise):
    """Full vocabulary: near-equal laws (long acceptances, the bonus path) and
    the workloads' target noise (rejections, residuals over 163840 tokens)."""
    B, D, V, T = 4, 8, 163840, 0.7
    tl, dl, x, u = _inputs(B, D, V, T, seed=3, noise=noise)
    ref = _run(tl, dl, x, u, T, "bf16")
    say("linear sample full vocab, noise", noise, "accept", ref["accept_len"].tolist())


def test_linear_sample_equal_laws_and_zero_mass():
    B, D, V, T = 6, 4, 2048, 1.0
    tl, dl, x, u = _inputs(B, D, V, T, seed=9, same=True)
    ref = _run(tl, dl, x, u, T, "f32")
    assert np.all(ref["accept_len"] == D)
    tl2 = tl.copy()
    for b in range(B):
        tl2[b, 0, x[b, 0]] = -1e4          # the first drafted token has no target mass
    ref = _run(tl2, dl, x, u, T, "f32")
    assert np.all(ref["accept_len"] == 0)


def test_linear_sample_uniform_extremes():
    B, D, V, T = 4, 2, 512, 1.0
    tl, dl, x, u = _inputs(B, D, V, T, seed=4)
    for fill in (0, 2 ** 64 - 1):
        u2 = u.copy()
        u2[:, :, :] = np.uint64(fill)
        _run(tl, dl, x, u2, T, "f32")
