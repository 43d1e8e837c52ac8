"""GPU parity of ddtree_vocab_top_p and ddtree_verify_sample_top_p (bit-exact).

The nucleus thresholds (weight, id), kept totals and block sums of every row
(sampled rows at the full workload sizes) and the walk's accept length, path,
tokens and bonus must equal the oracle's, for p in {1e-6, 0.5, 0.9, 1}, on the
small variants and the full workloads, bf16 and fp32.  The oracle walk takes
its rows' nuclei lazily, so only the rows it visits are computed at full size.
Flat rows (every weight equal) make the kernel's candidate set exceed its LDS
capacity and exercise the row-pass search.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import dev_tensor, say
from tests.test_gpu_parity import case

pytestmark = pytest.mark.gpu

SMALL = ["tiny", "bf16_gqa", "bf16_dh64", "f32_dh128", "chain_topk1", "max_nodes", "odd_vocab"]
PS = [1e-6, 0.5, 0.9, 1.0]


def _temp(c):
    return c.cfg.temperature if c.cfg.temperature > 0 else 0.8


class _LazyNucleus:
    """Oracle nucleus per (b, n), computed when the walk first reads it."""

    def __init__(self, c, ref_v, T, p):
        self.c, self.ref_v, self.T, self.p = c, ref_v, T, p
        self.cache = {}

    def get(self, b, n):
        if (b, n) not in self.cache:
            r = oracle.vocab_top_p(self.c.logits, self.ref_v["maxv"], self.c.tree["num_nodes"],
                                   self.T, self.p, dtype=self.c.cfg.dtype, rows=[(b, n)])
            self.cache[(b, n)] = (int(r["thr_w"][b, n]), int(r["thr_id"][b, n]), int(r["Rp"][b, n]),
                                  r["Rp_blocks"][b, n].copy())
        return self.cache[(b, n)]

    def view(self, k):
        outer = self

        class _V:
            def __getitem__(self, key):
                return outer.get(*key)[k]
        return _V()


def _gpu(c, T, p):
    import tree_verification_build_amd as lib
    t = c.gpu_tree()
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, T)
    tp = lib.ddtree_vocab_top_p(c.d("logits"), t.num_nodes, v["maxv"], v["R"], T, p)
    w = lib.ddtree_verify_sample_top_p(t, c.d("logits"), v["maxv"], tp, T, c.d("uniforms"))
    torch.cuda.synchronize()
    return ({k: x.cpu().numpy() for k, x in tp.items()}, {k: x.cpu().numpy() for k, x in w.items()})


def _check(name, p, rows=None):
    c = case(name)
    T = _temp(c)
    say("top_p", name, p)
    tp, w = _gpu(c, T, p)
    ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], T, dtype=c.cfg.dtype)
    lazy = _LazyNucleus(c, ref_v, T, p)
    B, N = c.tree["token"].shape
    nn = c.tree["num_nodes"]
    todo = rows if rows is not None else [(b, n) for b in range(B) for n in range(N)]
    for b, n in todo:
        if n >= nn[b]:
            assert tp["thr_id"][b, n] == -1 and tp["Rp"][b, n] == 0
            continue
        ref = lazy.get(b, n)
        got = (int(tp["thr_w"][b, n]), int(tp["thr_id"][b, n]), int(tp["Rp"][b, n]))
        assert got == ref[:3], (b, n, got, ref[:3])
        assert np.array_equal(tp["Rp_blocks"][b, n].view(np.uint64), ref[3]), (b, n)
    rw = oracle.verify_sample(c.tree, c.logits, ref_v["maxv"], lazy.view(2), T,
                              c.inp["uniforms"], c.cfg.D, dtype=c.cfg.dtype,
                              nucleus=(lazy.view(0), lazy.view(1)))
    for k in rw:
        assert np.array_equal(w[k], rw[k]), k
    return rw


@pytest.mark.parametrize("p", PS)
@pytest.mark.parametrize("name", SMALL)
def test_top_p_small(name, p):
    _check(name, p)


@pytest.mark.parametrize("name,p", [("single", 0.5), ("single", 0.9), ("batched", 0.5),
                                    ("batched", 0.9), ("ragged", 0.9)])
def test_top_p_full(name, p):
    c = case(name)
    rng = np.random.default_rng(len(name))
    B, N = c.tree["token"].shape
    rows = {(int(rng.integers(0, B)), int(rng.integers(0, N))) for _ in range(10)} | {(0, 0)}
    _check(name, p, rows=sorted(rows))


def test_top_p_one_equals_plain_walk():
    import tree_verification_build_amd as lib
    c = case("bf16_gqa")
    T = _temp(c)
    _, w = _gpu(c, T, 1.0)
    t = c.gpu_tree()
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, T)
    plain = lib.ddtree_verify_sample(t, c.d("logits"), v["maxv"], v["R"], v["R_blocks"], T,
                                     c.d("uniforms"))
    torch.cuda.synchronize()
    for k in plain:
        assert np.array_equal(plain[k].cpu().numpy(), w[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_flat_rows_take_the_row_pass_search(dtype):
    """Every weight equal (constant rows of 40000 tokens): the candidates exceed the
    LDS capacity; the nucleus is the lowest-id tokens, ceil(P / 2^32 * V) of them."""
    import tree_verification_build_amd as lib
    B, N, V, T = 2, 3, 40000, 1.0
    base = np.zeros((B, N, V), np.float32)
    base[1, 1, 17] = 0.25                       # one row with a single larger logit
    logits = base if dtype == "f32" else (base.view(np.uint32) >> 16).astype(np.uint16)
    nn = np.array([N, 2], np.int32)                # row (1, 2) is padding
    x = dev_tensor(logits, dtype)
    nd = torch.from_numpy(nn).cuda()
    v = lib.ddtree_vocab_reduce(x, nd, T)
    ref_v = oracle.vocab_reduce(logits, nn, T, dtype=dtype)
    for p in (0.3, 0.77, 1.0):
        say("top_p flat", dtype, p)
        tp = lib.ddtree_vocab_top_p(x, nd, v["maxv"], v["R"], T, p)
        torch.cuda.synchronize()
        ref = oracle.vocab_top_p(logits, ref_v["maxv"], nn, T, p, dtype=dtype)
        for k in ("thr_w", "thr_id", "Rp", "Rp_blocks"):
            got = tp[k].cpu().numpy()
            assert np.array_equal(got.view(ref[k].dtype) if got.dtype != ref[k].dtype else got,
                                  ref[k]), (k, p)
        P = oracle.top_p_fixed(p)
        assert int(ref["thr_id"][0, 0]) == -(-P * V // (1 << 32)) - 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_candidate_list_sizes(dtype):
    """Rows with k head tokens at five logit levels (many equal weights) and a tail
    that weighs 0: the first candidate pass takes exactly the k head tokens, so k
    walks the candidate list across the sizes the kernel treats differently (one,
    two, four and eight slots per thread of the sorted cut, more than
    the LDS holds)."""
    import tree_verification_build_amd as lib
    ks = [1, 2, 64, 300, 511, 512, 513, 1000, 1024, 1025, 2500, 4096, 4097]
    V, T = 40000, 1.0
    rng = np.random.default_rng(4242)
    base = np.full((1, len(ks), V), -57.0, np.float32)
    for n, k in enumerate(ks):
        ids = rng.choice(V, size=k, replace=False)
        base[0, n, ids] = 3.0 - 0.5 * rng.integers(0, 5, size=k)
    logits = base if dtype == "f32" else (base.view(np.uint32) >> 16).astype(np.uint16)
    nn = np.array([len(ks)], np.int32)
    x = dev_tensor(logits, dtype)
    nd = torch.from_numpy(nn).cuda()
    v = lib.ddtree_vocab_reduce(x, nd, T)
    ref_v = oracle.vocab_reduce(logits, nn, T, dtype=dtype)
    for p in (1e-6, 0.5, 0.9):
        say("top_p candidate sizes", dtype, p)
        tp = lib.ddtree_vocab_top_p(x, nd, v["maxv"], v["R"], T, p)
        torch.cuda.synchronize()
        ref = oracle.vocab_top_p(logits, ref_v["maxv"], nn, T, p, dtype=dtype)
        for key in ("thr_w", "thr_id", "Rp", "Rp_blocks"):
            got = tp[key].cpu().numpy()
            assert np.array_equal(got.view(ref[key].dtype) if got.dtype != ref[key].dtype else got,
                                  ref[key]), (key, p)
