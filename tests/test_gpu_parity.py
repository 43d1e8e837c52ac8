"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bit-exact: tree structure and scores, argmax, maxv, R, accept length, path,
tokens and bonus.  Tolerance (tree attention): max-abs 2e-2 for bf16 and
1e-4 for fp32, also relative to max|o|.  Small cases cover every output; the
full-size workloads (single request 8192 ctx, batch of 16 x 4096, 65536 ctx,
ragged batch of 64) cover all of the tree, vocabulary and walk outputs and
spot-check attention on a sample of (request, head) pairs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import Case, assert_attention_close, assert_tree_equal, attn_to_f64, \
    dev_tensor, say

pytestmark = pytest.mark.gpu

# small variants: span several tiles, a ragged tail, empty contexts, GQA, both head dims
SMALL = {
    "tiny": workloads.config("tiny"),
    "bf16_gqa": workloads.config("ragged", B=3, ctx=(0, 300), Hq=8, Hkv=2, Dh=128, V=4096,
                                 plant=True, seed_index=21),
    "bf16_dh64": workloads.config("batched", B=2, ctx=200, Hq=4, Hkv=4, Dh=64, V=2048,
                                  seed_index=22),
    "f32_dh128": workloads.config("tiny", ctx=130, Hq=2, Hkv=2, Dh=128, seed_index=23),
    "short_tree": workloads.config("tiny", D=2, K=2, budget=10, ctx=70, seed_index=24),
    "chain_topk1": workloads.config("single", ctx=500, budget=7, K=1, D=8, V=4096,
                                    seed_index=25),
    "max_nodes": workloads.config("long", B=2, ctx=(64, 400), D=16, K=8, budget=127, Hq=2,
                                  Hkv=2, V=2048, seed_index=26),
    "odd_vocab": workloads.config("batched", B=2, ctx=100, V=1001, Hq=2, Hkv=2,
                                  seed_index=27),
}
_cache = {}


def case(name):
    if name not in _cache:
        cfg = SMALL.get(name) or workloads.config(name)
        _cache[name] = Case(cfg)
    return _cache[name]


ALL = list(SMALL) + ["single", "batched", "long", "ragged"]


@pytest.mark.parametrize("name", ALL)
def test_build(name):
    c = case(name)
    say("build", name, c.cfg)
    t = c.gpu_tree()
    torch.cuda.synchronize()
    assert_tree_equal(t.to_numpy(), c.tree)


@pytest.mark.parametrize("D,K,budget", [(4, 3, 120), (3, 4, 84), (2, 8, 72)])
def test_build_small_table_two_slot_sets(D, K, budget):
    """D * K <= 64 (one register of log-probs per lane) with more than 65 nodes
    (the frontier's second slot set)."""
    import tree_verification_build_amd as lib
    rng = np.random.default_rng(D * 100 + K)
    B = 2
    lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
    tok = np.stack([np.stack([rng.choice(5000, K, replace=False) for _ in range(D)])
                    for _ in range(B)]).astype(np.int32)
    root = rng.integers(0, 5000, size=B).astype(np.int32)
    prefix = rng.integers(0, 100, size=B).astype(np.int32)
    say("build small table, two slot sets", D, K, budget)
    ref = oracle.build_tree(lp, tok, root, prefix, budget)
    t = lib.ddtree_build(*(torch.from_numpy(x).to("cuda:0") for x in (lp, tok, root, prefix)),
                         budget)
    torch.cuda.synchronize()
    assert_tree_equal(t.to_numpy(), ref)


def test_build_random_small_tables():
    """Trees of at most 65 nodes with a draft table of at most 64 entries (one
    frontier slot set): random depths, top-k caps and budgets, including
    budgets the tree cannot fill, 64 and 65 nodes, and log-probs drawn from a
    few values so that scores tie and the parent, then rank, decide; bit for
    bit with the oracle."""
    import tree_verification_build_amd as lib
    rng = np.random.default_rng(515)
    cases = [(1, 1, 1), (1, 4, 4), (2, 2, 6), (2, 2, 10), (8, 4, 63), (8, 4, 64), (16, 4, 64),
             (8, 8, 64), (4, 8, 40), (32, 2, 64), (64, 1, 64), (3, 5, 30)]
    for _ in range(20):
        D = int(rng.integers(1, 17))
        K = int(rng.integers(1, min(8, 64 // D) + 1))
        cases.append((D, K, int(rng.integers(1, 65))))
    for ci, (D, K, budget) in enumerate(cases):
        B = 4
        if ci % 2:
            vals = np.array([-0.25, -0.5, -1.0, -2.0], np.float32)   # ties
            lp = -np.sort(-rng.choice(vals, size=(B, D, K)), axis=-1).astype(np.float32)
        else:
            lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
        tok = np.stack([np.stack([rng.choice(5000, K, replace=False) for _ in range(D)])
                        for _ in range(B)]).astype(np.int32)
        root = rng.integers(0, 5000, size=B).astype(np.int32)
        prefix = rng.integers(0, 100, size=B).astype(np.int32)
        say("build random small table", D, K, budget)
        ref = oracle.build_tree(lp, tok, root, prefix, budget)
        t = lib.ddtree_build(*(torch.from_numpy(x).to("cuda:0") for x in (lp, tok, root, prefix)),
                             budget)
        torch.cuda.synchronize()
        assert_tree_equal(t.to_numpy(), ref)


def test_build_minus_inf_logprobs():
    """Draft log-probs of -inf (masked tokens) in the top-k: real offers that
    score -inf tie one another and are taken by parent, then rank, exactly as
    the oracle takes them; entries below depth D or past rank K - 1, which do
    not exist, are never taken."""
    import tree_verification_build_amd as lib
    for seed, (D, K, budget) in enumerate([(2, 2, 6), (4, 3, 120), (3, 4, 84), (8, 4, 32),
                                           (16, 8, 127)]):
        rng = np.random.default_rng(300 + seed)
        B = 3
        lp = -np.sort(np.abs(rng.standard_normal((B, D, K))), axis=-1).astype(np.float32)
        # trailing ranks of some depths masked (-inf keeps them non-increasing)
        for b in range(B):
            for d in range(D):
                r = int(rng.integers(0, K + 1))
                if r < K and (b + d) % 2 == 0:
                    lp[b, d, max(r, 1 if d == 0 and b == 0 else 0):] = -np.inf
        tok = np.stack([np.stack([rng.choice(5000, K, replace=False) for _ in range(D)])
                        for _ in range(B)]).astype(np.int32)
        root = rng.integers(0, 5000, size=B).astype(np.int32)
        prefix = rng.integers(0, 100, size=B).astype(np.int32)
        say("build -inf log-probs", D, K, budget)
        ref = oracle.build_tree(lp, tok, root, prefix, budget)
        t = lib.ddtree_build(*(torch.from_numpy(x).to("cuda:0") for x in (lp, tok, root, prefix)),
                             budget)
        torch.cuda.synchronize()
        assert_tree_equal(t.to_numpy(), ref)
        if budget == sum(K ** d for d in range(1, D + 1)):
            # every rank sequence fits the budget: the -inf ones are in the tree
            assert np.isneginf(ref["score"][ref["depth"] > 0]).any()


def _temps(c):
    return sorted({0.0, c.cfg.temperature, 0.8 if c.cfg.V <= 4096 else c.cfg.temperature})


@pytest.mark.parametrize("name", ALL)
def test_vocab_reduce(name):
    import tree_verification_build_amd as lib
    c = case(name)
    nn = c.tree["num_nodes"]
    for T in _temps(c):
        say("vocab", name, "T", T)
        r = lib.ddtree_vocab_reduce(c.d("logits"), torch.from_numpy(nn).to("cuda:0"), T,
                                    want_lse=True)
        torch.cuda.synchronize()
        ref = oracle.vocab_reduce(c.logits, nn, T, dtype=c.cfg.dtype)
        assert np.array_equal(r["argmax"].cpu().numpy(), ref["argmax"])
        assert np.array_equal(r["maxv"].cpu().numpy().view(np.uint32), ref["maxv"].view(np.uint32))
        lse = r["lse"].cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref["lse"])
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.abs(lse[fin] - ref["lse"][fin]).max() <= 1e-4
        if T > 0:
            assert np.array_equal(r["R"].cpu().numpy().view(np.uint64), ref["R"])
            assert np.array_equal(r["R_blocks"].cpu().numpy().view(np.uint64), ref["R_blocks"])
            # without the log-sum-exp, bf16 rows take their weights from a table
            r2 = lib.ddtree_vocab_reduce(c.d("logits"), torch.from_numpy(nn).to("cuda:0"), T)
            torch.cuda.synchronize()
            assert np.array_equal(r2["argmax"].cpu().numpy(), ref["argmax"])
            assert np.array_equal(r2["maxv"].cpu().numpy().view(np.uint32),
                                  ref["maxv"].view(np.uint32))
            assert np.array_equal(r2["R"].cpu().numpy().view(np.uint64), ref["R"])
            assert np.array_equal(r2["R_blocks"].cpu().numpy().view(np.uint64), ref["R_blocks"])


def _awkward_bf16_rows(V, seed):
    """bf16 logit rows whose weights fall outside a per-row table of the
    larger magnitudes: tiny, zero, negative-zero and subnormal values, values
    spread over many binades, a row max of 0, a large row max, a negative
    row max, equal values, and the most negative finite bf16 value."""
    rng = np.random.default_rng(seed)
    rows = []
    mag = np.exp2(rng.uniform(-140, 6, size=V)).astype(np.float32)   # 2^-140 .. 2^6
    rows.append(mag * rng.choice([-1.0, 1.0], size=V).astype(np.float32))
    r = rng.normal(0, 3, size=V).astype(np.float32)
    r[rng.integers(0, V, size=V // 8)] = 0.0
    r[rng.integers(0, V, size=V // 8)] = -0.0
    r[rng.integers(0, V, size=V // 16)] = np.float32(1e-40)          # subnormal
    rows.append(r)
    r = -np.abs(rng.normal(0, 1e-3, size=V)).astype(np.float32)
    r[rng.integers(0, V)] = 0.0                                       # max 0
    rows.append(r)
    rows.append((rng.normal(0, 3, size=V) + 3.0e4).astype(np.float32))  # large max
    rows.append((rng.normal(0, 50, size=V) - 400.0).astype(np.float32))  # negative max, wide
    rows.append(np.full(V, 1.5, dtype=np.float32))                   # all equal
    r = rng.normal(0, 3, size=V).astype(np.float32)
    r[rng.integers(0, V, size=V // 4)] = np.float32(-3.3895314e38)  # bf16 0xFF7F
    rows.append(r)
    x = np.stack(rows)[None]                                          # [1, 7, V]
    return workloads.f32_to_bf16_bits(x)


@pytest.mark.parametrize("V", [40960 + 8 * 7, 163840])
@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 25.0])
def test_vocab_sampling_awkward_rows(T, V):
    """R and its block sums on rows built to miss the weight table (bit-exact):
    a row length that ends inside a thread's vectors, and the full vocabulary
    (every thread's 20 vectors whole)."""
    import tree_verification_build_amd as lib
    bits = _awkward_bf16_rows(V, 51)
    nn = np.array([bits.shape[1]], dtype=np.int32)
    say("vocab awkward rows", "T", T, "V", V)
    logits = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    r = lib.ddtree_vocab_reduce(logits, torch.from_numpy(nn).to("cuda:0"), T)
    torch.cuda.synchronize()
    ref = oracle.vocab_reduce(bits, nn, T, dtype="bf16")
    assert np.array_equal(r["argmax"].cpu().numpy(), ref["argmax"])
    assert np.array_equal(r["maxv"].cpu().numpy().view(np.uint32), ref["maxv"].view(np.uint32))
    assert np.array_equal(r["R"].cpu().numpy().view(np.uint64), ref["R"])
    assert np.array_equal(r["R_blocks"].cpu().numpy().view(np.uint64), ref["R_blocks"])


def _sign_rows(V, seed):
    """bf16 rows whose maximum lies on the negative side or is a signed zero:
    log-softmax values (every logit negative), negatives with a -0 before a
    +0 (equal as floats: the -0's index is the argmax), negatives with -0 as
    their only zeros, and a positive maximum repeated at scattered indices."""
    rng = np.random.default_rng(seed)
    rows = []
    x = rng.normal(0, 3, size=V)
    top = x.max()
    rows.append((x - top - np.log(np.exp(x - top).sum())).astype(np.float32))
    r = (-np.abs(rng.normal(0, 2, size=V)) - 0.01).astype(np.float32)
    lo, hi = sorted(int(i) for i in rng.choice(V, size=2, replace=False))
    r[lo], r[hi] = -0.0, 0.0
    rows.append(r)
    r = (-np.abs(rng.normal(0, 2, size=V)) - 0.01).astype(np.float32)
    r[rng.choice(V, size=5, replace=False)] = -0.0
    rows.append(r)
    r = rng.normal(0, 3, size=V).astype(np.float32)
    r[rng.choice(V, size=7, replace=False)] = 40.0
    rows.append(r)
    return workloads.f32_to_bf16_bits(np.stack(rows)[None])


@pytest.mark.parametrize("V", [40960 + 8 * 7, 163840])
@pytest.mark.parametrize("T", [0.0, 0.7])
def test_vocab_sign_rows(T, V):
    """Row maxima that are negative or a signed zero, and repeated maxima:
    argmax, max, R and R_blocks bit for bit with the oracle."""
    import tree_verification_build_amd as lib
    bits = _sign_rows(V, 52)
    nn = np.array([bits.shape[1]], dtype=np.int32)
    say("vocab sign rows", "T", T, "V", V)
    logits = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    r = lib.ddtree_vocab_reduce(logits, torch.from_numpy(nn).to("cuda:0"), T)
    torch.cuda.synchronize()
    ref = oracle.vocab_reduce(bits, nn, T, dtype="bf16")
    assert np.array_equal(r["argmax"].cpu().numpy(), ref["argmax"])
    assert np.array_equal(r["maxv"].cpu().numpy().view(np.uint32), ref["maxv"].view(np.uint32))
    if T > 0:
        assert np.array_equal(r["R"].cpu().numpy().view(np.uint64), ref["R"])
        assert np.array_equal(r["R_blocks"].cpu().numpy().view(np.uint64), ref["R_blocks"])


@pytest.mark.parametrize("B,N,V", [(4, 69, 163840), (4, 69, 40960 + 8 * 7), (8, 76, 163840)])
def test_vocab_sampling_uneven_rounds(B, N, V):
    """Sampling rows that leave the last round of the persistent workgroups
    partly filled (the CU count plus 20 rows, twice it plus 96): the
    workgroups with one row fewer start late, which changes only the timing.
    argmax, max, R and R_blocks bit for bit with the oracle, padding rows
    included."""
    import tree_verification_build_amd as lib
    rng = np.random.default_rng(B * 1000 + N + V)
    x = rng.normal(0, 3, size=(B, N, V)).astype(np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    nn = rng.integers(1, N + 1, size=B).astype(np.int32)
    nn[0] = N
    say("vocab uneven rounds", B, N, V, "cus",
        torch.cuda.get_device_properties(0).multi_processor_count)
    logits = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    r = lib.ddtree_vocab_reduce(logits, torch.from_numpy(nn).to("cuda:0"), 0.7)
    torch.cuda.synchronize()
    ref = oracle.vocab_reduce(bits, nn, 0.7, dtype="bf16")
    assert np.array_equal(r["argmax"].cpu().numpy(), ref["argmax"])
    assert np.array_equal(r["maxv"].cpu().numpy().view(np.uint32), ref["maxv"].view(np.uint32))
    assert np.array_equal(r["R"].cpu().numpy().view(np.uint64), ref["R"])
    assert np.array_equal(r["R_blocks"].cpu().numpy().view(np.uint64), ref["R_blocks"])


@pytest.mark.parametrize("name", ["bf16_gqa", "batched"])
def test_vocab_sampling_without_workspace(name):
    """Called with no workspace (a sampling reduce needs none), through the C
    ABI directly: the same outputs as the oracle, bit for bit."""
    from tree_verification_build_amd import _lib as L
    c = case(name)
    T = c.cfg.temperature if c.cfg.temperature > 0 else 0.8
    nn = c.tree["num_nodes"]
    logits = c.d("logits")
    B, N, V = logits.shape
    dev = logits.device
    am = torch.empty((B, N), dtype=torch.int32, device=dev)
    mx = torch.empty((B, N), dtype=torch.float32, device=dev)
    R = torch.empty((B, N), dtype=torch.int64, device=dev)
    nb = (V + L.R_BLOCK - 1) // L.R_BLOCK
    Rb = torch.empty((B, N, nb), dtype=torch.int64, device=dev)
    nn_d = torch.from_numpy(nn).to(dev)
    say("vocab without workspace", name, "T", T)
    L._check(L.lib.ddtree_vocab_reduce(L._ptr(logits), L._dtype_code(logits), B, N, V,
                                       L._ptr(nn_d), float(T), L._ptr(am), L._ptr(mx), L._ptr(R),
                                       L._ptr(Rb), None, None, 0, L._stream(None)))
    torch.cuda.synchronize()
    # every valid row at small size; a sample (with padding rows) at full size
    rng = np.random.default_rng(11)
    todo = [(b, n) for b in range(B) for n in range(N)]
    if len(todo) > 64:
        todo = [todo[i] for i in sorted(rng.choice(len(todo), size=48, replace=False))]
    ref = oracle.vocab_reduce(c.logits, nn, T, dtype=c.cfg.dtype,
                              rows=[(b, n) for b, n in todo if n < nn[b]])
    bi = np.array([b for b, _ in todo]), np.array([n for _, n in todo])
    assert np.array_equal(am.cpu().numpy()[bi], ref["argmax"][bi])
    assert np.array_equal(mx.cpu().numpy().view(np.uint32)[bi], ref["maxv"].view(np.uint32)[bi])
    assert np.array_equal(R.cpu().numpy().view(np.uint64)[bi], ref["R"][bi])
    assert np.array_equal(Rb.cpu().numpy().view(np.uint64)[bi], ref["R_blocks"][bi])


@pytest.mark.parametrize("name", ALL)
def test_verify_greedy(name):
    import tree_verification_build_amd as lib
    c = case(name)
    say("verify_greedy", name)
    t = c.gpu_tree()
    ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], 0.0, dtype=c.cfg.dtype)
    # the walk consumes the GPU's own argmax, whose parity is pinned above
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, 0.0)
    o = lib.ddtree_verify_greedy(t, v["argmax"])
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(c.tree, ref_v["argmax"], c.cfg.D)
    for k in ref:
        assert np.array_equal(o[k].cpu().numpy(), ref[k]), k
    if c.cfg.plant:
        assert ref["accept_len"].max() > 0


@pytest.mark.parametrize("name", ALL)
def test_vocab_verify_greedy(name):
    """The fused call equals ddtree_vocab_reduce + ddtree_verify_greedy (and the
    oracle) bit for bit, at every workload's vocabulary and tree shape."""
    import tree_verification_build_amd as lib
    c = case(name)
    t = c.gpu_tree()
    say("vocab_verify_greedy", name)
    f = lib.ddtree_vocab_verify_greedy(c.d("logits"), t)
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, 0.0)
    g = lib.ddtree_verify_greedy(t, v["argmax"])
    torch.cuda.synchronize()
    assert np.array_equal(f["argmax"].cpu().numpy(), v["argmax"].cpu().numpy())
    assert np.array_equal(f["maxv"].cpu().numpy().view(np.uint32),
                          v["maxv"].cpu().numpy().view(np.uint32))
    for k in g:
        assert np.array_equal(f[k].cpu().numpy(), g[k].cpu().numpy()), k
    ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], 0.0, dtype=c.cfg.dtype)
    ref = oracle.verify_greedy(c.tree, ref_v["argmax"], c.cfg.D)
    assert np.array_equal(f["argmax"].cpu().numpy(), ref_v["argmax"])
    for k in ref:
        assert np.array_equal(f[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("name", ALL)
def test_verify_sample(name):
    import tree_verification_build_amd as lib
    c = case(name)
    T = c.cfg.temperature if c.cfg.temperature > 0 else 0.8
    say("verify_sample", name, "T", T)
    t = c.gpu_tree()
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, T)
    o = lib.ddtree_verify_sample(t, c.d("logits"), v["maxv"], v["R"], v["R_blocks"], T,
                                 c.d("uniforms"))
    torch.cuda.synchronize()
    ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], T, dtype=c.cfg.dtype)
    ref = oracle.verify_sample(c.tree, c.logits, ref_v["maxv"], ref_v["R"], T,
                               c.inp["uniforms"], c.cfg.D, dtype=c.cfg.dtype)
    for k in ref:
        assert np.array_equal(o[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("name", ALL)
def test_verify_sample_lazy(name):
    """The lazy walk reduces only the rows it visits; its outputs are the
    oracle's (vocab pass + walk) bit for bit, at two temperatures, also when a
    tiny temperature makes it follow the greedy path far into the tree."""
    import tree_verification_build_amd as lib
    c = case(name)
    temps = sorted({c.cfg.temperature if c.cfg.temperature > 0 else 0.8, 0.05})
    t = c.gpu_tree()
    for T in temps:
        say("verify_sample_lazy", name, "T", T)
        o = lib.ddtree_verify_sample_lazy(t, c.d("logits"), T, c.d("uniforms"))
        torch.cuda.synchronize()
        ref_v = oracle.vocab_reduce(c.logits, c.tree["num_nodes"], T, dtype=c.cfg.dtype)
        ref = oracle.verify_sample(c.tree, c.logits, ref_v["maxv"], ref_v["R"], T,
                                   c.inp["uniforms"], c.cfg.D, dtype=c.cfg.dtype)
        for k in ref:
            assert np.array_equal(o[k].cpu().numpy(), ref[k]), (T, k)


def _attn_sample(c):
    """Oracle calls as (requests, heads) pairs: everything when small; at full
    size every request on one head (head b % Hq for request b) and so, with
    B >= Hq, every head on several requests; a single request on all heads."""
    cfg = c.cfg
    if name_is_full(cfg):
        return [([b for b in range(cfg.B) if b % cfg.Hq == h] or [0], [h])
                for h in range(cfg.Hq)]
    return [(None, None)]


def name_is_full(cfg):
    return cfg.name in ("single", "batched", "long", "ragged") and cfg == workloads.config(cfg.name)


@pytest.mark.parametrize("name", ALL)
def test_tree_attention(name):
    c = case(name)
    say("attention", name, c.cfg)
    t = c.gpu_tree()
    out, lse = c.gpu_attention(t)
    torch.cuda.synchronize()
    o_ref = lse_ref = None
    for reqs, heads in _attn_sample(c):
        say("attention oracle", name, "requests", reqs, "heads", heads)
        o1, l1 = c.oracle_attention(reqs, heads)
        if o_ref is None:
            o_ref, lse_ref = o1, l1
        else:
            m = ~np.isnan(o1)
            o_ref[m] = o1[m]
            ml = ~np.isnan(l1)
            lse_ref[ml] = l1[ml]
    checked = ~np.isnan(o_ref[..., 0])
    say("attention", name, "checked (request, node, head) rows", int(checked.sum()), "of",
        checked.size)
    o = attn_to_f64(out)
    err, scale = assert_attention_close(o, o_ref, c.cfg.dtype)
    say("attention", name, "max abs err", err, "max |o|", scale)
    l = lse.cpu().numpy().astype(np.float64)
    sel = ~np.isnan(lse_ref) & np.isfinite(lse_ref)
    assert np.abs(l[sel] - lse_ref[sel]).max() < 1e-3
    assert np.all(np.isneginf(l[np.isneginf(lse_ref)]))
    if name_is_full(c.cfg):
        # every request and every head were compared
        assert checked.any(axis=(1, 2)).all() and checked.any(axis=(0, 1)).all()


# bf16 head dim 128 runs the DMA kernel in one variant per count of 16-row query
# blocks (1-4: four waves, reads issued ahead of use; 5-8: eight waves); the
# workloads above reach 1, 3, 5 and 8 blocks.  Contexts of 300-1500 tokens give
# both single-split and multi-split requests.
QUERY_BLOCKS = {
    2: dict(budget=19, Hq=2, Hkv=2, D=8, K=4),     # M = 20
    4: dict(budget=27, Hq=4, Hkv=2, D=8, K=4),     # M = 56
    6: dict(budget=47, Hq=4, Hkv=2, D=8, K=4),     # M = 96
    7: dict(budget=111, Hq=2, Hkv=2, D=16, K=8),   # M = 112
}


@pytest.mark.parametrize("qb", sorted(QUERY_BLOCKS))
def test_attention_query_blocks(qb):
    cfg = workloads.config("ragged", B=3, ctx=(300, 1500), Dh=128, V=1024, temperature=0.0,
                           seed_index=40 + qb, **QUERY_BLOCKS[qb])
    c = Case(cfg)
    M = (cfg.budget + 1) * cfg.Hq // cfg.Hkv
    assert (M + 15) // 16 == qb
    say("attention query blocks", qb, cfg)
    t = c.gpu_tree()
    out, lse = c.gpu_attention(t)
    torch.cuda.synchronize()
    o_ref, lse_ref = c.oracle_attention()
    err, scale = assert_attention_close(attn_to_f64(out), o_ref, "bf16")
    say("attention query blocks", qb, "max abs err", err, "max |o|", scale)
    l = lse.cpu().numpy().astype(np.float64)
    sel = np.isfinite(lse_ref)
    assert np.abs(l[sel] - lse_ref[sel]).max() < 1e-3


@pytest.mark.parametrize("name", ["bf16_gqa", "single", "ragged"])
def test_attention_deterministic(name):
    c = case(name)
    say("attention determinism", name)
    t = c.gpu_tree()
    a, _ = c.gpu_attention(t, want_lse=False)
    b, _ = c.gpu_attention(t, want_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_attention_split_size_invariance():
    """Other context split sizes and LDS ring depths (ddtree_tree_attention_tuned)
    change only rounding, within tolerance."""
    import tree_verification_build_amd as lib
    c = case("single")
    t = c.gpu_tree()
    base, _ = c.gpu_attention(t, want_lse=False)
    for tu in ({"split_keys": 64}, {"split_keys": 1024}, {"split_keys": 8192},
               {"stages": 3}, {"stages": 4}, {"split_keys": 256, "stages": 4}):
        say("attention tuning", tu)
        o, _ = lib.ddtree_tree_attention_tuned(
            c.d("q"), c.d("k_ctx"), c.d("v_ctx"), c.d("ctx_offsets"), c.inp["ctx_offsets"],
            c.d("k_tree"), c.d("v_tree"), t, tuning=tu)
        torch.cuda.synchronize()
        d = (o.float() - base.float()).abs().max().item()
        assert d <= 2e-2 * base.float().abs().max().item(), (tu, d)


@pytest.mark.parametrize("name", ["bf16_gqa", "batched"])
def test_walk_outputs_in_pinned_host_memory(name):
    """The walks' outputs may live in pinned host memory (what a serving loop
    reads each step): same results as device outputs, visible after a sync."""
    import tree_verification_build_amd as lib
    c = case(name)
    say("pinned walk outputs", name)
    t = c.gpu_tree()
    T = c.cfg.temperature
    v = lib.ddtree_vocab_reduce(c.d("logits"), t.num_nodes, T)

    def outputs(pinned):
        kw = dict(dtype=torch.int32, pin_memory=True) if pinned else \
            dict(dtype=torch.int32, device="cuda:0")
        B, D = c.cfg.B, c.cfg.D
        return {"accept_len": torch.full((B,), -7, **kw), "bonus": torch.full((B,), -7, **kw),
                "path_nodes": torch.full((B, D + 1), -7, **kw),
                "out_tokens": torch.full((B, D + 1), -7, **kw)}
    res = []
    for pinned in (False, True):
        o = outputs(pinned)
        if T > 0:
            lib.ddtree_verify_sample(t, c.d("logits"), v["maxv"], v["R"], v["R_blocks"], T,
                                     c.d("uniforms"), outputs=o)
        else:
            lib.ddtree_verify_greedy(t, v["argmax"], outputs=o)
        torch.cuda.synchronize()
        res.append({k: x.cpu().numpy().copy() for k, x in o.items()})
    for k in res[0]:
        assert np.array_equal(res[0][k], res[1][k]), k


# More than 128 query rows per KV head are cut into 128-row slices along the
# grid's z axis, each streaming the context once: up to the limit of 1024 rows
# (128 nodes x 8 grouped heads), for the bf16 DMA kernel and the fp32 one.
ROW_SLICES = {
    "bf16_m1024": dict(dtype="bf16", budget=127, Hq=8, Hkv=1, D=16, K=8, V=1024),
    "f32_m256": dict(dtype="f32", budget=63, Hq=8, Hkv=2, D=8, K=8, V=1024),
}


@pytest.mark.parametrize("name", sorted(ROW_SLICES))
def test_attention_row_slices(name):
    cfg = workloads.config("ragged", B=2, ctx=(100, 700), Dh=128, temperature=0.0,
                           seed_index=60 + len(name), **ROW_SLICES[name])
    c = Case(cfg)
    M = (cfg.budget + 1) * cfg.Hq // cfg.Hkv
    say("attention row slices", name, "M", M, "slices", (M + 127) // 128)
    t = c.gpu_tree()
    out, lse = c.gpu_attention(t)
    torch.cuda.synchronize()
    o_ref, lse_ref = c.oracle_attention()
    assert_attention_close(attn_to_f64(out), o_ref, cfg.dtype)
    l = lse.cpu().numpy().astype(np.float64)
    sel = np.isfinite(lse_ref)
    assert np.abs(l[sel] - lse_ref[sel]).max() < 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 3, 8, 9, 100])
def test_vocab_tiny_rows(V, dtype):
    """Vocabularies shorter than one 16-byte vector per thread (and a single
    token): argmax / max / lse greedy, R and R_blocks sampling, bit for bit."""
    import tree_verification_build_amd as lib
    rng = np.random.default_rng(1000 + V)
    B, N = 3, 5
    x = rng.normal(0, 2, size=(B, N, V)).astype(np.float32)
    x[0, 1, :] = 0.5                                   # ties: the lowest index wins
    nn = np.array([5, 3, 1], dtype=np.int32)
    bits = workloads.f32_to_bf16_bits(x) if dtype == "bf16" else x
    dev = dev_tensor(bits, dtype)
    nd = torch.from_numpy(nn).to("cuda:0")
    say("vocab tiny rows", dtype, "V", V)
    g = lib.ddtree_vocab_reduce(dev, nd, 0.0, want_lse=True)
    s = lib.ddtree_vocab_reduce(dev, nd, 0.9)
    torch.cuda.synchronize()
    ref_g = oracle.vocab_reduce(bits, nn, 0.0, dtype=dtype)
    ref_s = oracle.vocab_reduce(bits, nn, 0.9, dtype=dtype)
    assert np.array_equal(g["argmax"].cpu().numpy(), ref_g["argmax"])
    assert np.array_equal(g["maxv"].cpu().numpy().view(np.uint32), ref_g["maxv"].view(np.uint32))
    lse, lse_ref = g["lse"].cpu().numpy().astype(np.float64), ref_g["lse"]
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lse_ref[fin]).max() < 1e-5
    assert np.array_equal(s["R"].cpu().numpy().view(np.uint64), ref_s["R"])
    assert np.array_equal(s["R_blocks"].cpu().numpy().view(np.uint64), ref_s["R_blocks"])


def test_deep_chain_full_accept():
    """A 64-deep chain (top-k 1, budget 64, the depth limit) whose target
    argmax follows it to the end: the build's visibility rows over 64
    ancestors, and the greedy walks (separate and fused) and the sampled walk
    at T 0.05 accepting all 64 tokens, bit for bit with the oracle."""
    import tree_verification_build_amd as lib
    cfg = workloads.config("single", B=2, ctx=96, D=64, K=1, budget=64, V=512, Hq=2, Hkv=2,
                           temperature=0.0, seed_index=71)
    c = Case(cfg)
    tree = c.tree
    assert int(tree["max_depth"].min()) == 64
    rng = np.random.default_rng(72)
    x = rng.normal(0, 1, size=(cfg.B, cfg.N, cfg.V)).astype(np.float32)
    for b in range(cfg.B):
        for i in range(cfg.N - 1):
            x[b, i, tree["token"][b, i + 1]] = 12.0
    bits = workloads.f32_to_bf16_bits(x)
    lg = dev_tensor(bits, "bf16")
    t = c.gpu_tree()
    assert_tree_equal(t.to_numpy(), tree)
    v = lib.ddtree_vocab_reduce(lg, t.num_nodes, 0.0)
    g = lib.ddtree_verify_greedy(t, v["argmax"])
    f = lib.ddtree_vocab_verify_greedy(lg, t)
    T = 0.05
    vs = lib.ddtree_vocab_reduce(lg, t.num_nodes, T)
    u = dev_tensor(c.inp["uniforms"], None)
    s = lib.ddtree_verify_sample(t, lg, vs["maxv"], vs["R"], vs["R_blocks"], T, u)
    torch.cuda.synchronize()
    ref_v = oracle.vocab_reduce(bits, tree["num_nodes"], 0.0, dtype="bf16")
    ref_g = oracle.verify_greedy(tree, ref_v["argmax"], cfg.D)
    ref_vs = oracle.vocab_reduce(bits, tree["num_nodes"], T, dtype="bf16")
    ref_s = oracle.verify_sample(tree, bits, ref_vs["maxv"], ref_vs["R"], T, c.inp["uniforms"],
                                 cfg.D, dtype="bf16")
    assert list(ref_g["accept_len"]) == [64] * cfg.B
    for k in ref_g:
        assert np.array_equal(g[k].cpu().numpy(), ref_g[k]), ("greedy", k)
        assert np.array_equal(f[k].cpu().numpy(), ref_g[k]), ("fused", k)
    for k in ref_s:
        assert np.array_equal(s[k].cpu().numpy(), ref_s[k]), ("sample", k)
    say("deep chain", "greedy accept", ref_g["accept_len"].tolist(), "sampled accept",
        ref_s["accept_len"].tolist())
