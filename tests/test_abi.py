"""The C-ABI library: loads, exports every declared symbol, validates arguments on the host.

No kernel is launched here (these run without a GPU): every call below is
rejected by host-side validation before anything is enqueued, or is a
host-only helper.
"""
import ctypes
import decimal
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddtree.h")
LIB = os.path.join(ROOT, "tree_verification_build_amd", "libddtree.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libddtree.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtree_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    names = _declared()
    assert {"ddtree_build", "ddtree_tree_attention", "ddtree_vocab_reduce",
            "ddtree_verify_greedy", "ddtree_verify_sample"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_error_string():
    import tree_verification_build_amd as t
    assert "gfx950" in t.ddtree_version()
    assert isinstance(t.ddtree_last_error(), str)


def test_sampling_constants_match_oracle_and_exact_values():
    import tree_verification_build_amd as t
    from oracle import weight_constants
    decimal.getcontext().prec = 50
    ln2 = decimal.Decimal(2).ln()
    for T in (0.3, 0.7, 1.0, 1.7, 2.0):
        c, a = t.ddtree_sampling_constants(T)
        oc, oa = weight_constants(T)
        assert c == oc
        assert np.array_equal(a, oa)
        for n in range(7):
            exact = ln2 ** n / math.factorial(n)
            err = abs(decimal.Decimal(float(a[n])) - exact)
            ulp = decimal.Decimal(float(np.spacing(a[n])))
            assert err <= ulp / 2
    with pytest.raises(t.DdtreeError):
        t.ddtree_sampling_constants(0.0)


def _fake_tree(B=1, N=9, D=8, K=2, W=1):
    from tree_verification_build_amd._lib import _CTree
    return _CTree(*([16] * 10), B, N, D, K, W)


def test_host_validation_rejects_bad_arguments():
    from tree_verification_build_amd._lib import lib
    fake = ctypes.c_void_p(16)
    t = _fake_tree()
    # draft top-k
    assert lib.ddtree_draft_topk(None, 0, 9, 1024, 2, fake, fake, None, 0, None) == 1
    assert lib.ddtree_draft_topk(fake, 0, 9, 1024, 0, fake, fake, None, 0, None) == 1   # K < 1
    assert lib.ddtree_draft_topk(fake, 0, 9, 1024, 65, fake, fake, None, 0, None) == 1  # K > 64
    assert lib.ddtree_draft_topk(fake, 0, 9, 3, 4, fake, fake, None, 0, None) == 1      # K > V
    assert lib.ddtree_draft_topk(fake, 5, 9, 1024, 2, fake, fake, None, 0, None) == 1   # dtype
    assert lib.ddtree_draft_topk(fake, 0, 0, 1024, 2, fake, fake, None, 0, None) == 1   # rows
    assert lib.ddtree_draft_topk(fake, 0, 70000, 1024, 2, fake, fake, None, 0, None) == 2
    # split rows need their workspace
    assert lib.ddtree_draft_topk(fake, 0, 9, 163840, 4, fake, fake, None, 0, None) == 1
    # ddtree_build
    assert lib.ddtree_build(None, fake, fake, fake, 1, 8, 2, 8, ctypes.byref(t), None) == 1
    assert lib.ddtree_build(fake, fake, fake, fake, 1, 8, 2, 200, ctypes.byref(t), None) == 1
    assert lib.ddtree_build(fake, fake, fake, fake, 1, 8, 2, 7, ctypes.byref(t), None) == 1
    bad = _fake_tree(W=2)
    assert lib.ddtree_build(fake, fake, fake, fake, 1, 8, 2, 8, ctypes.byref(bad), None) == 1
    assert lib.ddtree_build(fake, fake, fake, fake, 1, 8, 2, 8, None, None) == 1
    # vocab
    assert lib.ddtree_vocab_reduce(fake, 1, 1, 9, 0, fake, 0.0, fake, fake, None, None, None,
                                   None, 0, None) == 1
    assert lib.ddtree_vocab_reduce(fake, 1, 1, 9, 100, fake, -1.0, fake, fake, None, None, None,
                                   None, 0, None) == 1
    assert lib.ddtree_vocab_reduce(fake, 1, 1, 9, 100, fake, 0.5, fake, fake, None, None, None,
                                   None, 0, None) == 1               # R missing with T > 0
    assert lib.ddtree_vocab_reduce(fake, 1, 1, 9, 64 * 32768 + 1, fake, 0.5, fake, fake, fake,
                                   fake, None, None, 0, None) == 2   # sampling row too long
    assert lib.ddtree_vocab_reduce(fake, 7, 1, 9, 100, fake, 0.0, fake, fake, None, None, None,
                                   None, 0, None) == 1               # unknown dtype
    # greedy split pass needs its workspace at this size
    assert lib.ddtree_vocab_reduce(fake, 1, 1, 9, 163840, fake, 0.0, fake, fake, None, None,
                                   None, None, 0, None) == 1
    # walks
    assert lib.ddtree_verify_greedy(ctypes.byref(t), None, fake, fake, fake, fake, None) == 1
    # vocabulary reduction + greedy walk in one call
    vvg = lib.ddtree_vocab_verify_greedy
    assert vvg(None, 1, 100, ctypes.byref(t), fake, fake, fake, fake, fake, fake, fake, 1 << 20,
               None) == 1                                                      # null logits
    assert vvg(fake, 1, 0, ctypes.byref(t), fake, fake, fake, fake, fake, fake, fake, 1 << 20,
               None) == 1                                                      # V < 1
    assert vvg(fake, 7, 100, ctypes.byref(t), fake, fake, fake, fake, fake, fake, fake, 1 << 20,
               None) == 1                                                      # dtype
    assert vvg(fake, 1, 163840, ctypes.byref(t), fake, fake, fake, fake, fake, fake, None, 0,
               None) == 1                                                      # split rows, no workspace
    assert vvg(fake, 1, 100, ctypes.byref(t), fake, fake, None, fake, fake, fake, fake, 1 << 20,
               None) == 1                                                      # null accept_len
    bad = _fake_tree(N=200)
    assert vvg(fake, 1, 100, ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, 1 << 20,
               None) == 1                                                      # N > 128
    assert lib.ddtree_verify_sample(ctypes.byref(t), fake, 1, 100, fake, fake, fake, 0.0, fake,
                                    fake, fake, fake, fake, None) == 1      # T <= 0
    assert lib.ddtree_verify_sample(ctypes.byref(t), fake, 1, 100, fake, fake, None, 0.7, fake,
                                    fake, fake, fake, fake, None) == 1      # R_blocks missing
    assert lib.ddtree_verify_sample(ctypes.byref(t), fake, 1, 64 * 32768 + 1, fake, fake, fake,
                                    0.7, fake, fake, fake, fake, fake, None) == 2
    assert lib.ddtree_verify_sample_lazy(ctypes.byref(t), fake, 1, 100, 0.0, fake, fake, fake,
                                         fake, fake, None) == 1               # T <= 0
    assert lib.ddtree_verify_sample_lazy(ctypes.byref(t), None, 1, 100, 0.7, fake, fake, fake,
                                         fake, fake, None) == 1               # null logits
    assert lib.ddtree_verify_sample_lazy(ctypes.byref(t), fake, 1, 64 * 32768 + 1, 0.7, fake,
                                         fake, fake, fake, fake, None) == 2
    # commit (tree, accept_len, path_nodes, bonus, k/v tree, Hkv, Dh, dtype, k/v cache,
    # cache_base, cache_rows, capacity, next_prefix_len, next_root, stream)
    cm = [ctypes.byref(t), fake, fake, fake, fake, fake]
    tail = [fake, fake, fake, 100, 50, fake, fake, None]
    assert lib.ddtree_commit(ctypes.byref(t), None, *cm[2:], 8, 128, 1, *tail) == 1
    assert lib.ddtree_commit(*cm, 0, 128, 1, *tail) == 1                 # Hkv < 1
    assert lib.ddtree_commit(*cm, 8, 128, 4, *tail) == 1                 # dtype
    assert lib.ddtree_commit(*cm, 1, 4, 1, *tail) == 2                   # 8-byte rows
    assert lib.ddtree_commit(*cm, 8, 128, 1, fake, fake, fake, -1, 50, fake, fake, None) == 1
    assert lib.ddtree_commit(*cm, 8, 128, 1, fake, fake, fake, 100, -1, fake, fake, None) == 1
    assert lib.ddtree_commit(*cm, 8, 128, 1, fake, fake, fake, 100, 50, None, fake, None) == 1
    assert lib.ddtree_commit(*cm, 8, 128, 1, ctypes.c_void_p(24), fake, fake, 100, 50, fake,
                             fake, None) == 1                            # misaligned cache
    # top-p
    tp = [fake, 1, 1, 9, 100, fake, fake, fake]
    outs = [fake, fake, fake, fake, None]
    assert lib.ddtree_vocab_top_p(*tp, 0.8, 0.0, *outs) == 1            # top_p <= 0
    assert lib.ddtree_vocab_top_p(*tp, 0.8, 1.5, *outs) == 1            # top_p > 1
    assert lib.ddtree_vocab_top_p(*tp, 0.0, 0.9, *outs) == 1            # T <= 0
    assert lib.ddtree_vocab_top_p(fake, 1, 1, 9, 64 * 32768 + 1, fake, fake, fake, 0.8, 0.9,
                                  *outs) == 2
    assert lib.ddtree_vocab_top_p(None, *tp[1:], 0.8, 0.9, *outs) == 1
    sv = [ctypes.byref(t), fake, 1, 100, fake, fake, fake, fake, fake]
    wo = [fake, fake, fake, fake, fake, None]
    assert lib.ddtree_verify_sample_top_p(*sv, 0.0, *wo) == 1            # T <= 0
    assert lib.ddtree_verify_sample_top_p(*sv[:7], None, fake, 0.8, *wo) == 1   # thr_w missing
    # attention, range form
    st1, ln1, lnbad = (ctypes.c_int32 * 1)(0), (ctypes.c_int32 * 1)(64), (ctypes.c_int32 * 1)(-1)
    rg = [fake, fake, fake, fake, fake]
    assert lib.ddtree_tree_attention_ranges(*rg, st1, lnbad, fake, fake, ctypes.byref(t), 4, 4, 64,
                                            1, 0.125, fake, None, None, 0, None) == 1
    assert lib.ddtree_tree_attention_ranges(*rg, None, ln1, fake, fake, ctypes.byref(t), 4, 4, 64,
                                            1, 0.125, fake, None, None, 0, None) == 1
    assert lib.ddtree_tree_attention_ranges(*rg, st1, ln1, fake, fake, ctypes.byref(t), 4, 4, 96,
                                            1, 0.125, fake, None, None, 0, None) == 2
    # capped range form: the same checks on the bounds, and at most 64 requests
    cap = lib.ddtree_tree_attention_ranges_capped
    assert cap(*rg, st1, lnbad, fake, fake, ctypes.byref(t), 4, 4, 64, 1, 0.125, fake, None,
               None, 0, None) == 1
    assert cap(*rg, st1, None, fake, fake, ctypes.byref(t), 4, 4, 64, 1, 0.125, fake, None,
               None, 0, None) == 1
    assert cap(*rg, st1, ln1, fake, fake, ctypes.byref(t), 4, 4, 96, 1, 0.125, fake, None,
               None, 0, None) == 2
    t65 = _fake_tree(65, 33, 8, 4, 1)
    st65, ln65 = (ctypes.c_int32 * 65)(*range(0, 65 * 64, 64)), (ctypes.c_int32 * 65)(*[64] * 65)
    assert cap(*rg, st65, ln65, fake, fake, ctypes.byref(t65), 4, 4, 64, 1, 0.125, fake, None,
               fake, 1 << 30, None) == 2
    assert b"requests" in lib.ddtree_last_error()
    # attention
    offs = (ctypes.c_int32 * 2)(0, 64)
    args = [fake, fake, fake, fake, offs, fake, fake, ctypes.byref(t)]
    assert lib.ddtree_tree_attention(*args, 4, 3, 64, 1, 0.125, fake, None, None, 0, None) == 1
    assert lib.ddtree_tree_attention(*args, 4, 4, 96, 1, 0.125, fake, None, None, 0, None) == 2
    assert lib.ddtree_tree_attention(*args, 128, 1, 64, 1, 0.125, fake, None, None, 0, None) == 2
    assert lib.ddtree_tree_attention(*args, 4, 4, 64, 1, -1.0, fake, None, None, 0, None) == 1
    assert lib.ddtree_tree_attention(*args, 4, 4, 64, 5, 0.125, fake, None, None, 0, None) == 1
    assert lib.ddtree_tree_attention(*args, 4, 4, 64, 1, float("nan"), fake, None, None, 0,
                                     None) == 1
    mis = ctypes.c_void_p(24)
    assert lib.ddtree_tree_attention(mis, *args[1:], 4, 4, 64, 1, 0.125, fake, None, None, 0,
                                     None) == 1
    lib.ddtree_last_error.restype = ctypes.c_char_p
    assert b"aligned" in lib.ddtree_last_error()
    # tuned form: bad tuning values are rejected before any launch
    from tree_verification_build_amd._lib import _CTuning
    for sk, ns in ((-1, 0), (0, 1), (0, 5), (64, -2)):
        tu = _CTuning(sk, ns)
        assert lib.ddtree_tree_attention_tuned(*args, 4, 4, 64, 1, 0.0, fake, None, None, 0,
                                               ctypes.byref(tu), None) == 1, (sk, ns)
    assert lib.ddtree_tree_attention_tuned(*args, 4, 4, 96, 1, 0.0, fake, None, None, 0, None,
                                           None) == 2


def test_noalloc_attention_rejects_partials_beyond_its_scratch():
    """ddtree_tree_attention_noalloc checks the plan against its fixed device
    array on the host, before anything is launched (no GPU needed here)."""
    from tree_verification_build_amd._lib import lib, NOALLOC_SCRATCH_BYTES
    import tree_verification_build_amd as t
    fake = ctypes.c_void_p(16)
    tree = _fake_tree(B=64, N=33, D=8, K=4, W=1)
    big = np.arange(65, dtype=np.int64) * 65536          # 64 requests x 65536 keys
    offs = (ctypes.c_int32 * 65)(*[int(x) for x in big])
    need = t.ddtree_tree_attention_workspace_size(64, 33, 8, 8, 128, big.astype(np.int32))
    assert need > NOALLOC_SCRATCH_BYTES
    assert lib.ddtree_tree_attention_noalloc(fake, fake, fake, fake, offs, fake, fake,
                                             ctypes.byref(tree), 8, 8, 128, 1, 0.0, fake, None,
                                             None) == 2
    lib.ddtree_last_error.restype = ctypes.c_char_p
    assert b"scratch" in lib.ddtree_last_error()
    assert lib.ddtree_tree_attention_noalloc(fake, fake, fake, fake, offs, fake, fake,
                                             ctypes.byref(tree), 8, 8, 96, 1, 0.0, fake, None,
                                             None) == 2                     # head_dim 96
    # the five workloads' partials fit
    import workloads
    for name in ("tiny", "single", "batched", "long", "ragged"):
        cfg = workloads.config(name)
        o = np.concatenate([[0], np.cumsum(workloads.ctx_lengths(cfg))]).astype(np.int32)
        assert t.ddtree_tree_attention_workspace_size(cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.Dh,
                                                      o) <= NOALLOC_SCRATCH_BYTES, name


def test_workspace_sizes_are_host_only_and_sane():
    import tree_verification_build_amd as t
    offs = np.array([0, 8192], np.int32)
    ws = t.ddtree_tree_attention_workspace_size(1, 33, 8, 8, 128, offs)
    assert ws > 0 and ws % 4 == 0
    assert t.ddtree_tree_attention_workspace_size(1, 9, 4, 4, 96, offs) == 0
    # the range form sizes its workspace from the lengths alone
    lens = np.array([300, 0, 5000, 64], np.int32)
    packed = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert t.ddtree_tree_attention_ranges_workspace_size(4, 33, 8, 2, 128, lens) == \
        t.ddtree_tree_attention_workspace_size(4, 33, 8, 2, 128, packed) > 0
    # a tuned split size sizes its own workspace: smaller splits, more partials
    assert t.ddtree_tree_attention_tuned_workspace_size(1, 33, 8, 8, 128, offs) == ws
    assert t.ddtree_tree_attention_tuned_workspace_size(1, 33, 8, 8, 128, offs,
                                                        split_keys=64) > ws
    assert t.ddtree_tree_attention_tuned_workspace_size(1, 33, 8, 8, 128, offs,
                                                        split_keys=8192) == 0
    assert t.ddtree_vocab_reduce_workspace_size(1, 33, 163840) > 0
    assert t.ddtree_vocab_reduce_workspace_size(64, 33, 163840) == 0
    # draft top-k: slices of 1024..8192 elements, K keys and one (max, sum) pair each
    assert t.ddtree_draft_topk_workspace_size(9, 163840, 4) > 0
    assert t.ddtree_draft_topk_workspace_size(9, 1024, 2) == 0
    assert t.ddtree_draft_topk_workspace_size(9, 1024, 65) == 0
