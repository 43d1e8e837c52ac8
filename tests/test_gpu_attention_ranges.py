"""GPU parity of ddtree_tree_attention_ranges (context as per-request row ranges).

The contexts of a workload are scattered into a larger buffer in a shuffled
order with gaps filled with NaN (a read outside a request's range would poison
its output).  The range form must give bit-for-bit the output of the packed
form on the packed copy (same split plan, same kernels) and match the oracle
within the attention tolerance; batches above and below the size at which the
split plan is passed in the kernel arguments (64 requests) are covered, and a
batched two-step loop runs the range form over per-request slabs after
ddtree_commit has appended each request's accepted path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_cases import (DEV, Case, assert_attention_close, attn_to_f64, dev_tensor, say)

pytestmark = pytest.mark.gpu

CFGS = {
    "ranges_b3_bf16": workloads.config("ragged", B=3, ctx=(0, 700), Hq=8, Hkv=2, Dh=128,
                                       V=2048, seed_index=41),
    "ranges_b20_bf16": workloads.config("ragged", B=20, ctx=(0, 400), Hq=4, Hkv=4, Dh=128,
                                        V=2048, seed_index=42),
    "ranges_b5_dh64": workloads.config("batched", B=5, ctx=300, Hq=4, Hkv=4, Dh=64, V=2048,
                                       seed_index=43),
    "ranges_b18_f32": workloads.config("tiny", B=18, ctx=(0, 600), Hq=2, Hkv=2, Dh=128,
                                       seed_index=44),
    # past 64 requests the splits are looked up on the device
    "ranges_b70_bf16": workloads.config("ragged", B=70, ctx=(0, 400), Hq=2, Hkv=2, Dh=128,
                                        V=1024, seed_index=45),
    "ranges_b66_f32": workloads.config("tiny", B=66, ctx=(0, 300), Hq=2, Hkv=2, Dh=64,
                                       seed_index=46),
}
_cases = {}


def _case(name):
    if name not in _cases:
        _cases[name] = Case(CFGS[name])
    return _cases[name]


def _nan_rows(rows, Hkv, Dh, dtype):
    if dtype == "bf16":
        return np.full((rows, Hkv, Dh), 0x7FC0, dtype=np.uint16)
    return np.full((rows, Hkv, Dh), np.nan, dtype=np.float32)


def _scatter(c, seed):
    """Request contexts at shuffled, gapped row ranges of a NaN-filled buffer."""
    i, cfg = c.inp, c.cfg
    rng = np.random.default_rng(seed)
    lens = i["ctx_lens"].astype(np.int64)
    order = rng.permutation(cfg.B)
    gaps = rng.integers(0, 40, size=cfg.B)
    start = np.zeros(cfg.B, np.int64)
    row = int(rng.integers(0, 9))
    for b in order:
        row += int(gaps[b])
        start[b] = row
        row += int(lens[b])
    rows = row + 7
    kc = _nan_rows(rows, cfg.Hkv, cfg.Dh, cfg.dtype)
    vc = _nan_rows(rows, cfg.Hkv, cfg.Dh, cfg.dtype)
    offs = i["ctx_offsets"]
    for b in range(cfg.B):
        kc[start[b]:start[b] + lens[b]] = i["k_ctx"][offs[b]:offs[b + 1]]
        vc[start[b]:start[b] + lens[b]] = i["v_ctx"][offs[b]:offs[b + 1]]
    return kc, vc, start.astype(np.int32), lens.astype(np.int32)


@pytest.mark.parametrize("name", list(CFGS))
def test_ranges_equal_packed_and_oracle(name):
    import tree_verification_build_amd as lib
    c = _case(name)
    cfg = c.cfg
    say("attention ranges", name)
    kc, vc, start, lens = _scatter(c, 3)
    t = c.gpu_tree()
    o_pack, l_pack = c.gpu_attention(t)
    o_rng, l_rng = lib.ddtree_tree_attention_ranges(
        c.d("q"), dev_tensor(kc, cfg.dtype), dev_tensor(vc, cfg.dtype), dev_tensor(start, None),
        dev_tensor(lens, None), start, lens, c.d("k_tree"), c.d("v_tree"), t, want_lse=True)
    torch.cuda.synchronize()
    a, b = o_pack.cpu(), o_rng.cpu()
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
    assert torch.equal(a.view(bits), b.view(bits)), "range form differs from the packed form"
    assert torch.equal(l_pack.cpu().view(torch.int32), l_rng.cpu().view(torch.int32))
    ref, ref_lse = c.oracle_attention()
    assert_attention_close(attn_to_f64(o_rng), ref, cfg.dtype)


def test_ranges_validation():
    import tree_verification_build_amd as lib
    from tree_verification_build_amd import DdtreeError
    c = _case("ranges_b3_bf16")
    cfg = c.cfg
    t = c.gpu_tree()
    kc, vc, start, lens = _scatter(c, 4)
    bad = lens.copy()
    bad[1] = -1
    with pytest.raises(DdtreeError):
        lib.ddtree_tree_attention_ranges(
            c.d("q"), dev_tensor(kc, cfg.dtype), dev_tensor(vc, cfg.dtype),
            dev_tensor(start, None), dev_tensor(bad, None), start, bad, c.d("k_tree"),
            c.d("v_tree"), t)


def test_batched_commit_then_ranges_attention():
    """Two steps over per-request slabs: step 1 attends over the initial contexts,
    commits the accepted paths into the slabs; step 2's range-form attention reads
    ctx_len = the committed prefix lengths."""
    import tree_verification_build_amd as lib
    from tests.test_gpu_commit import _follow_argmax
    c = _case("ranges_b3_bf16")
    cfg, i = c.cfg, c.inp
    say("batched commit + ranges")
    lens = i["ctx_lens"].astype(np.int64)
    cap = int(lens.max()) + 2 * (cfg.D + 1)
    base = np.arange(cfg.B, dtype=np.int64) * cap
    kc0 = _nan_rows(cfg.B * cap, cfg.Hkv, cfg.Dh, "bf16")
    vc0 = _nan_rows(cfg.B * cap, cfg.Hkv, cfg.Dh, "bf16")
    offs = i["ctx_offsets"]
    for b in range(cfg.B):
        kc0[base[b]:base[b] + lens[b]] = i["k_ctx"][offs[b]:offs[b + 1]]
        vc0[base[b]:base[b] + lens[b]] = i["v_ctx"][offs[b]:offs[b + 1]]
    am = _follow_argmax(c.tree, cfg.V, 21, p_follow=1.0)
    ref_w = oracle.verify_greedy(c.tree, am, cfg.D)
    ref = oracle.commit_path(c.tree, ref_w["accept_len"], ref_w["path_nodes"], ref_w["bonus"],
                             i["k_tree"], i["v_tree"], kc0, vc0, base, cap)
    t = c.gpu_tree()
    w = lib.ddtree_verify_greedy(t, dev_tensor(am, None))
    kc, vc = dev_tensor(kc0, "bf16"), dev_tensor(vc0, "bf16")
    cb = torch.from_numpy(base).to(DEV)
    prefix, root = lib.ddtree_commit(t, w, c.d("k_tree"), c.d("v_tree"), kc, vc, cb, cap)
    # step 2
    plen = ref["next_prefix_len"]
    assert (plen > lens + 1).any()
    rng = np.random.default_rng(22)
    q2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["q"].shape).astype(np.float32))
    kt2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["k_tree"].shape).astype(np.float32))
    vt2 = workloads.f32_to_bf16_bits(rng.standard_normal(i["v_tree"].shape).astype(np.float32))
    tree2 = oracle.build_tree(i["draft_lp"], i["draft_tok"], ref["next_root"], plen, cfg.budget)
    t2 = lib.ddtree_build(c.d("draft_lp"), c.d("draft_tok"), root, prefix, cfg.budget)
    st = base.astype(np.int32)
    o2, _ = lib.ddtree_tree_attention_ranges(
        dev_tensor(q2, "bf16"), kc, vc, dev_tensor(st, None), prefix, st, plen,
        dev_tensor(kt2, "bf16"), dev_tensor(vt2, "bf16"), t2)
    torch.cuda.synchronize()
    assert np.array_equal(prefix.cpu().numpy(), plen)
    packed_k = np.concatenate([ref["k_cache"][base[b]:base[b] + plen[b]] for b in range(cfg.B)])
    packed_v = np.concatenate([ref["v_cache"][base[b]:base[b] + plen[b]] for b in range(cfg.B)])
    offs2 = np.concatenate([[0], np.cumsum(plen)]).astype(np.int32)
    o_ref, _ = oracle.tree_attention(q2, packed_k, packed_v, offs2, kt2, vt2, tree2["vis"],
                                     tree2["num_nodes"], dtype="bf16")
    assert_attention_close(attn_to_f64(o2), o_ref, "bf16")


@pytest.mark.parametrize("direction", ["shorter", "longer"])
def test_device_lengths_disagreeing_with_host_copy(direction):
    """Past 64 requests the kernels read the device context offsets while the
    grid and the workspace follow the host copy.  When the two disagree (a
    broken precondition) the output is undefined, but no access may leave the
    planned splits' workspace: the call completes, and a following call with
    agreeing copies is exact again.  Device ranges stay inside the K/V buffer."""
    import tree_verification_build_amd as lib
    c = _case("ranges_b70_bf16")
    cfg, i = c.cfg, c.inp
    t = c.gpu_tree()
    lens = i["ctx_lens"].astype(np.int64)
    rng = np.random.default_rng(5)
    if direction == "shorter":
        bad = np.maximum(lens - rng.integers(0, 300, size=cfg.B), 0)
    else:
        bad = lens + rng.integers(0, 900, size=cfg.B)
    bad_offs = np.concatenate([[0], np.cumsum(bad)]).astype(np.int32)
    rows = max(int(bad_offs[-1]), int(i["ctx_offsets"][-1]))
    kc = np.zeros((rows, cfg.Hkv, cfg.Dh), np.uint16)
    vc = np.zeros((rows, cfg.Hkv, cfg.Dh), np.uint16)
    kc[:i["k_ctx"].shape[0]] = i["k_ctx"]
    vc[:i["v_ctx"].shape[0]] = i["v_ctx"]
    kd, vd = dev_tensor(kc, "bf16"), dev_tensor(vc, "bf16")
    say("attention, device offsets", direction, "than the host copy", "B", cfg.B)
    lib.ddtree_tree_attention(c.d("q"), kd, vd, dev_tensor(bad_offs, None), i["ctx_offsets"],
                              c.d("k_tree"), c.d("v_tree"), t)
    torch.cuda.synchronize()
    out, _ = lib.ddtree_tree_attention(c.d("q"), kd, vd, c.d("ctx_offsets"), i["ctx_offsets"],
                                       c.d("k_tree"), c.d("v_tree"), t)
    torch.cuda.synchronize()
    ref, _ = c.oracle_attention()
    assert_attention_close(attn_to_f64(out), ref, "bf16")


def _slabs(c, caps, seed):
    """Request b's context at the start of a slab of caps[b] rows (the rest NaN)."""
    i, cfg = c.inp, c.cfg
    lens = i["ctx_lens"].astype(np.int64)
    rng = np.random.default_rng(seed)
    gaps = rng.integers(0, 40, size=cfg.B)
    start = np.zeros(cfg.B, np.int64)
    row = 3
    for b in range(cfg.B):
        row += int(gaps[b])
        start[b] = row
        row += int(caps[b])
    kc = _nan_rows(row + 5, cfg.Hkv, cfg.Dh, cfg.dtype)
    vc = _nan_rows(row + 5, cfg.Hkv, cfg.Dh, cfg.dtype)
    offs = i["ctx_offsets"]
    for b in range(cfg.B):
        kc[start[b]:start[b] + lens[b]] = i["k_ctx"][offs[b]:offs[b + 1]]
        vc[start[b]:start[b] + lens[b]] = i["v_ctx"][offs[b]:offs[b + 1]]
    return kc, vc, start.astype(np.int32)


def _oracle_over(c, kc, vc, start, lens, tree):
    cfg = c.cfg
    pk = np.concatenate([kc[start[b]:start[b] + lens[b]] for b in range(cfg.B)])
    pv = np.concatenate([vc[start[b]:start[b] + lens[b]] for b in range(cfg.B)])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, _ = oracle.tree_attention(c.inp["q"], pk, pv, offs, c.inp["k_tree"], c.inp["v_tree"],
                                 tree["vis"], tree["num_nodes"], dtype=cfg.dtype)
    return o


CAPPED = ["ranges_b3_bf16", "ranges_b20_bf16", "ranges_b5_dh64", "ranges_b18_f32"]


@pytest.mark.parametrize("name", CAPPED)
def test_capped_ranges(name):
    """Bounds above the lengths: the oracle's output over the device lengths;
    bounds equal to the lengths: bit for bit the exact-length range form."""
    import tree_verification_build_amd as lib
    c = _case(name)
    cfg = c.cfg
    lens = c.inp["ctx_lens"].astype(np.int32)
    rng = np.random.default_rng(31)
    caps = (lens + rng.integers(0, 700, size=cfg.B)).astype(np.int32)
    say("attention ranges capped", name, "caps", caps.tolist()[:6])
    kc, vc, start = _slabs(c, caps, 7)
    kd, vd = dev_tensor(kc, cfg.dtype), dev_tensor(vc, cfg.dtype)
    sd, ld = dev_tensor(start, None), dev_tensor(lens, None)
    t = c.gpu_tree()
    o_cap, _ = lib.ddtree_tree_attention_ranges_capped(c.d("q"), kd, vd, sd, ld, start, caps,
                                                       c.d("k_tree"), c.d("v_tree"), t)
    o_eq, _ = lib.ddtree_tree_attention_ranges_capped(c.d("q"), kd, vd, sd, ld, start, lens,
                                                      c.d("k_tree"), c.d("v_tree"), t)
    o_rng, _ = lib.ddtree_tree_attention_ranges(c.d("q"), kd, vd, sd, ld, start, lens,
                                                c.d("k_tree"), c.d("v_tree"), t)
    torch.cuda.synchronize()
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
    assert torch.equal(o_eq.cpu().view(bits), o_rng.cpu().view(bits))
    assert_attention_close(attn_to_f64(o_cap), _oracle_over(c, kc, vc, start, lens, c.tree),
                           cfg.dtype)


def test_capped_graph_replays_as_contexts_grow():
    """One captured call, replayed while the device lengths grow (and one
    request's shrinks to 0) and new context rows are written: every replay
    matches the oracle over the lengths of that moment."""
    import tree_verification_build_amd as lib
    c = _case("ranges_b20_bf16")
    cfg = c.cfg
    lens = c.inp["ctx_lens"].astype(np.int32)
    grow = 3 * 200
    caps = (lens + grow).astype(np.int32)
    kc, vc, start = _slabs(c, caps, 8)
    kd, vd = dev_tensor(kc, cfg.dtype), dev_tensor(vc, cfg.dtype)
    sd, ld = dev_tensor(start, None), dev_tensor(lens, None)
    t = c.gpu_tree()
    out = torch.empty_like(c.d("q"))
    ws = torch.empty(max(16, lib.ddtree_tree_attention_ranges_workspace_size(
        cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh, caps)), dtype=torch.uint8, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.ddtree_tree_attention_ranges_capped(c.d("q"), kd, vd, sd, ld, start, caps,
                                                c.d("k_tree"), c.d("v_tree"), t, out=out,
                                                workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    cur = lens.copy()
    for step in range(4):
        if step > 0:
            add = rng.integers(0, 201, size=cfg.B).astype(np.int32)
            new = np.minimum(cur + add, caps)
            if step == 2:
                new[0] = 0
            for b in range(cfg.B):
                if new[b] > cur[b]:
                    rows = rng.standard_normal((new[b] - cur[b], cfg.Hkv, cfg.Dh)).astype(np.float32)
                    kc[start[b] + cur[b]:start[b] + new[b]] = workloads.f32_to_bf16_bits(rows)
                    vc[start[b] + cur[b]:start[b] + new[b]] = workloads.f32_to_bf16_bits(rows[::-1])
            kd.copy_(dev_tensor(kc, cfg.dtype))
            vd.copy_(dev_tensor(vc, cfg.dtype))
            ld.copy_(torch.from_numpy(new))
            cur = new
        g.replay()
        torch.cuda.synchronize()
        say("capped graph replay", step, "total context", int(cur.sum()))
        assert_attention_close(attn_to_f64(out), _oracle_over(c, kc, vc, start, cur, c.tree),
                               cfg.dtype)


def test_capped_lengths_outside_the_bounds():
    """Device lengths above their bounds are read as the bounds, negative ones as
    0: the same output, bit for bit, as lengths already clamped."""
    import tree_verification_build_amd as lib
    c = _case("ranges_b3_bf16")
    cfg = c.cfg
    lens = c.inp["ctx_lens"].astype(np.int32)
    caps = lens.copy()
    kc, vc, start = _slabs(c, caps + 200, 12)
    kd, vd = dev_tensor(kc, cfg.dtype), dev_tensor(vc, cfg.dtype)
    sd = dev_tensor(start, None)
    wild = (lens + 150).astype(np.int32)
    wild[1] = -7
    clamped = np.minimum(np.maximum(wild, 0), caps).astype(np.int32)
    t = c.gpu_tree()
    say("attention ranges capped, lengths outside the bounds", wild.tolist(), caps.tolist())
    o_w, _ = lib.ddtree_tree_attention_ranges_capped(c.d("q"), kd, vd, sd, dev_tensor(wild, None),
                                                     start, caps, c.d("k_tree"), c.d("v_tree"), t)
    o_c, _ = lib.ddtree_tree_attention_ranges_capped(c.d("q"), kd, vd, sd,
                                                     dev_tensor(clamped, None), start, caps,
                                                     c.d("k_tree"), c.d("v_tree"), t)
    torch.cuda.synchronize()
    assert torch.equal(o_w.cpu().view(torch.int16), o_c.cpu().view(torch.int16))
    assert_attention_close(attn_to_f64(o_c), _oracle_over(c, kc, vc, start, clamped, c.tree),
                           cfg.dtype)
