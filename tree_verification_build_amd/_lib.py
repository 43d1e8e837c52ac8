"""ctypes binding of libddtree.so (argument marshalling only)."""
import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DDTREE_LIBRARY: another build of the same library (the host-sanitizer build)
library_path = os.environ.get("DDTREE_LIBRARY") or os.path.join(_HERE, "libddtree.so")

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is missing: build it first (__graft_entry__.build() or "
                      "python tree_verification_build_amd/_build.py)")
lib = ctypes.CDLL(library_path)

DDTREE_OK, DDTREE_EINVAL, DDTREE_EUNSUPPORTED, DDTREE_EDEVICE = 0, 1, 2, 3
DDTREE_F32, DDTREE_BF16 = 0, 1
R_BLOCK = 32768   # DDTREE_R_BLOCK: tokens per block of the sampling weight sums
_STATUS = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "EDEVICE"}


class DdtreeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _CTree(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("token", "parent", "depth", "rank", "position",
                                               "first_child", "next_sibling", "score", "vis",
                                               "num_nodes")] + \
               [(n, ctypes.c_int32) for n in ("B", "N", "D", "K", "W")] + \
               [("max_depth", ctypes.c_void_p)]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_tp = ctypes.POINTER(_CTree)
lib.ddtree_draft_topk_workspace_size.argtypes = [_i32, _i32, _i32]
lib.ddtree_draft_topk_workspace_size.restype = _sz
lib.ddtree_draft_topk.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
lib.ddtree_build.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _tp, _vp]
lib.ddtree_tree_attention_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp]
lib.ddtree_tree_attention_workspace_size.restype = _sz
lib.ddtree_tree_attention.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _tp, _i32, _i32, _i32,
                                      ctypes.c_int, _f32, _vp, _vp, _vp, _sz, _vp]
lib.ddtree_tree_attention_tuned_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp, _vp]
lib.ddtree_tree_attention_tuned_workspace_size.restype = _sz
lib.ddtree_tree_attention_tuned.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _tp, _i32, _i32,
                                            _i32, ctypes.c_int, _f32, _vp, _vp, _vp, _sz, _vp, _vp]
lib.ddtree_tree_attention_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _tp, _i32, _i32,
                                              _i32, ctypes.c_int, _f32, _vp, _vp, _vp]
lib.ddtree_tree_attention_ranges_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _vp]
lib.ddtree_tree_attention_ranges_workspace_size.restype = _sz
lib.ddtree_tree_attention_ranges.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _tp, _i32,
                                             _i32, _i32, ctypes.c_int, _f32, _vp, _vp, _vp, _sz,
                                             _vp]
lib.ddtree_tree_attention_ranges_capped.argtypes = lib.ddtree_tree_attention_ranges.argtypes
lib.ddtree_vocab_reduce_workspace_size.argtypes = [_i32, _i32, _i32]
lib.ddtree_vocab_reduce_workspace_size.restype = _sz
lib.ddtree_vocab_reduce.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _f32, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _sz, _vp]
lib.ddtree_verify_greedy.argtypes = [_tp, _vp, _vp, _vp, _vp, _vp, _vp]
lib.ddtree_vocab_verify_greedy.argtypes = [_vp, ctypes.c_int, _i32, _tp, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _sz, _vp]
lib.ddtree_verify_sample.argtypes = [_tp, _vp, ctypes.c_int, _i32, _vp, _vp, _vp, _f32, _vp, _vp, _vp,
                                     _vp, _vp, _vp]
lib.ddtree_verify_sample_lazy.argtypes = [_tp, _vp, ctypes.c_int, _i32, _f32, _vp, _vp, _vp, _vp,
                                          _vp, _vp]
lib.ddtree_verify_linear_sample.argtypes = [_vp, _vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _f32, _vp, _vp, _vp, _vp, _vp]
lib.ddtree_vocab_top_p.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp, _f32, _f32,
                                   _vp, _vp, _vp, _vp, _vp]
lib.ddtree_verify_sample_top_p.argtypes = [_tp, _vp, ctypes.c_int, _i32, _vp, _vp, _vp, _vp, _vp,
                                           _f32, _vp, _vp, _vp, _vp, _vp, _vp]
lib.ddtree_commit.argtypes = [_tp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, ctypes.c_int, _vp, _vp, _vp,
                              ctypes.c_int64, _i32, _vp, _vp, _vp]
lib.ddtree_sampling_constants.argtypes = [_f32, ctypes.POINTER(_f32), ctypes.POINTER(_f32)]
for _f in ("ddtree_draft_topk", "ddtree_build", "ddtree_tree_attention",
           "ddtree_tree_attention_tuned", "ddtree_tree_attention_noalloc",
           "ddtree_tree_attention_ranges", "ddtree_tree_attention_ranges_capped",
           "ddtree_vocab_reduce",
           "ddtree_verify_greedy", "ddtree_vocab_verify_greedy", "ddtree_verify_sample",
           "ddtree_verify_sample_lazy",
           "ddtree_verify_linear_sample", "ddtree_commit", "ddtree_vocab_top_p",
           "ddtree_verify_sample_top_p", "ddtree_sampling_constants"):
    getattr(lib, _f).restype = ctypes.c_int
lib.ddtree_last_error.restype = ctypes.c_char_p
lib.ddtree_version.restype = ctypes.c_char_p


def ddtree_last_error() -> str:
    return lib.ddtree_last_error().decode()


def ddtree_version() -> str:
    return lib.ddtree_version().decode()


def _check(st):
    if st != DDTREE_OK:
        raise DdtreeError(st, ddtree_last_error())


def _stream(stream):
    # the current device's index given explicitly: torch's own lookup of the
    # default device goes through an availability check on every call
    s = torch.cuda.current_stream(torch.cuda.current_device()) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _scratch(workspace, need, device, stream):
    """The caller's workspace if it is large enough, else a new one.  A new one
    is tied to `stream` when one is given, so that the caching allocator does
    not hand its memory out again while the call's kernels may still use it."""
    if workspace is not None and workspace.numel() >= need:
        return workspace
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _dev(t, name, dtype=None, shape=None, pinned_ok=False):
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or (pinned_ok and t.is_pinned())):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor"
                        + (" or pinned host memory" if pinned_ok else ""))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DDTREE_BF16
    if t.dtype == torch.float32:
        return DDTREE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


class Tree:
    """Device arrays of a token tree ([B, N] each; vis [B, N, W]; num_nodes and
    max_depth [B])."""

    FIELDS = ("token", "parent", "depth", "rank", "position", "first_child", "next_sibling")

    def __init__(self, B, N, D, K, device):
        self.B, self.N, self.D, self.K, self.W = B, N, D, K, (N + 63) // 64
        for f in self.FIELDS:
            setattr(self, f, torch.empty((B, N), dtype=torch.int32, device=device))
        self.score = torch.empty((B, N), dtype=torch.float32, device=device)
        self.vis = torch.empty((B, N, self.W), dtype=torch.int64, device=device)
        self.num_nodes = torch.empty((B,), dtype=torch.int32, device=device)
        self.max_depth = torch.empty((B,), dtype=torch.int32, device=device)
        self._c = _CTree(*[t.data_ptr() for t in (*[getattr(self, f) for f in self.FIELDS],
                                                   self.score, self.vis, self.num_nodes)],
                         B, N, D, K, self.W, self.max_depth.data_ptr())

    @property
    def cstruct(self):
        return ctypes.byref(self._c)

    def to_numpy(self) -> dict:
        out = {f: getattr(self, f).cpu().numpy() for f in self.FIELDS}
        out["score"] = self.score.cpu().numpy()
        out["vis"] = self.vis.cpu().numpy().view(np.uint64)
        out["num_nodes"] = self.num_nodes.cpu().numpy()
        out["max_depth"] = self.max_depth.cpu().numpy()
        return out


def alloc_tree(B, budget, D, K, device="cuda") -> Tree:
    return Tree(B, budget + 1, D, K, device)


def ddtree_draft_topk_workspace_size(rows, V, K) -> int:
    return int(lib.ddtree_draft_topk_workspace_size(rows, V, K))


def ddtree_draft_topk(logits, K, tokens=None, logprobs=None, workspace=None, stream=None):
    """Per-row top-K of draft logits [..., V] (bf16 or fp32): returns (tokens
    [..., K] int32, log-probs [..., K] fp32)."""
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    lead, V = tuple(logits.shape[:-1]), int(logits.shape[-1])
    rows = int(np.prod(lead)) if lead else 1
    dev = logits.device
    if tokens is None:
        tokens = torch.empty((*lead, K), dtype=torch.int32, device=dev)
    if logprobs is None:
        logprobs = torch.empty((*lead, K), dtype=torch.float32, device=dev)
    _dev(tokens, "tokens", torch.int32, (*lead, K))
    _dev(logprobs, "logprobs", torch.float32, (*lead, K))
    need = int(lib.ddtree_draft_topk_workspace_size(rows, V, K))
    workspace = _scratch(workspace, need, dev, stream)
    _check(lib.ddtree_draft_topk(_ptr(logits), _dtype_code(logits), rows, V, K, _ptr(tokens),
                                 _ptr(logprobs), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return tokens, logprobs


def ddtree_build(draft_lp, draft_tok, root_tok, prefix_len, budget, tree=None, stream=None):
    """Best-first tree from draft_lp/draft_tok [B, D, K]; returns a Tree."""
    B, D, K = draft_lp.shape
    _dev(draft_lp, "draft_lp", torch.float32)
    _dev(draft_tok, "draft_tok", torch.int32, (B, D, K))
    _dev(root_tok, "root_tok", torch.int32, (B,))
    _dev(prefix_len, "prefix_len", torch.int32, (B,))
    if tree is None:
        tree = alloc_tree(B, budget, D, K, draft_lp.device)
    _check(lib.ddtree_build(_ptr(draft_lp), _ptr(draft_tok), _ptr(root_tok), _ptr(prefix_len),
                            B, D, K, budget, tree.cstruct, _stream(stream)))
    return tree


def _host_offsets(ctx_offsets_host):
    a = np.ascontiguousarray(np.asarray(ctx_offsets_host, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def ddtree_tree_attention_workspace_size(B, N, Hq, Hkv, Dh, ctx_offsets_host) -> int:
    a, p = _host_offsets(ctx_offsets_host)
    return int(lib.ddtree_tree_attention_workspace_size(B, N, Hq, Hkv, Dh, p))


class _CTuning(ctypes.Structure):
    _fields_ = [("split_keys", ctypes.c_int32), ("stages", ctypes.c_int32)]


def ddtree_tree_attention_tuned_workspace_size(B, N, Hq, Hkv, Dh, ctx_offsets_host, split_keys=0,
                                               stages=0) -> int:
    a, p = _host_offsets(ctx_offsets_host)
    tu = _CTuning(split_keys, stages)
    return int(lib.ddtree_tree_attention_tuned_workspace_size(B, N, Hq, Hkv, Dh, p,
                                                              ctypes.byref(tu)))


def ddtree_tree_attention(q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree, v_tree, tree,
                          scale=None, out=None, want_lse=False, workspace=None, stream=None):
    """Returns (out [B, N, Hq, Dh], lse [B, N, Hq] or None).  scale None: the
    library's default, 1/sqrt(Dh)."""
    return ddtree_tree_attention_tuned(q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree,
                                       v_tree, tree, scale=scale, out=out, want_lse=want_lse,
                                       workspace=workspace, stream=stream, tuning=None)


def ddtree_tree_attention_tuned(q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree, v_tree,
                                tree, scale=None, out=None, want_lse=False, workspace=None,
                                stream=None, tuning=None):
    """ddtree_tree_attention with a caller-chosen work split: tuning = dict(split_keys=...,
    stages=...) (missing entries: 0, the planned choice), or None for the planned call."""
    B, N, Hq, Dh = q.shape
    Hkv = k_tree.shape[2]
    _dev(q, "q", (torch.bfloat16, torch.float32))
    _dev(k_tree, "k_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(v_tree, "v_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(k_ctx, "k_ctx", q.dtype)
    _dev(v_ctx, "v_ctx", q.dtype, tuple(k_ctx.shape))
    _dev(ctx_offsets, "ctx_offsets", torch.int32, (B + 1,))
    hoff, hptr = _host_offsets(ctx_offsets_host)
    if hoff.shape != (B + 1,) or int(hoff[0]) != 0:
        raise ValueError(f"ctx_offsets_host must hold B + 1 = {B + 1} offsets starting at 0")
    if k_ctx.shape[0] < int(hoff[-1]) or tuple(k_ctx.shape[1:]) != (Hkv, Dh):
        raise ValueError("k_ctx must be [ctx_offsets[B], Hkv, Dh]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, tuple(q.shape))
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    tu = None if tuning is None else _CTuning(int(tuning.get("split_keys", 0)),
                                              int(tuning.get("stages", 0)))
    tup = None if tu is None else ctypes.byref(tu)
    need = int(lib.ddtree_tree_attention_tuned_workspace_size(B, N, Hq, Hkv, Dh, hptr, tup))
    workspace = _scratch(workspace, need, q.device, stream)
    _check(lib.ddtree_tree_attention_tuned(
        _ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_offsets), hptr, _ptr(k_tree), _ptr(v_tree),
        tree.cstruct, Hq, Hkv, Dh, _dtype_code(q), 0.0 if scale is None else float(scale),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), tup, _stream(stream)))
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20   # DDTREE_NOALLOC_SCRATCH_BYTES


def ddtree_tree_attention_noalloc(q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree, v_tree,
                                  tree, out, lse=None, scale=None, stream=None):
    """ddtree_tree_attention with the split partials in the library's device
    array: the C call allocates nothing, so `out` (and `lse`, if wanted) must be
    given.  Returns (out, lse)."""
    B, N, Hq, Dh = q.shape
    Hkv = k_tree.shape[2]
    _dev(q, "q", (torch.bfloat16, torch.float32))
    _dev(k_tree, "k_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(v_tree, "v_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(k_ctx, "k_ctx", q.dtype)
    _dev(v_ctx, "v_ctx", q.dtype, tuple(k_ctx.shape))
    _dev(ctx_offsets, "ctx_offsets", torch.int32, (B + 1,))
    _dev(out, "out", q.dtype, tuple(q.shape))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, N, Hq))
    hoff, hptr = _host_offsets(ctx_offsets_host)
    if hoff.shape != (B + 1,) or int(hoff[0]) != 0:
        raise ValueError(f"ctx_offsets_host must hold B + 1 = {B + 1} offsets starting at 0")
    if k_ctx.shape[0] < int(hoff[-1]) or tuple(k_ctx.shape[1:]) != (Hkv, Dh):
        raise ValueError("k_ctx must be [ctx_offsets[B], Hkv, Dh]")
    _check(lib.ddtree_tree_attention_noalloc(
        _ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_offsets), hptr, _ptr(k_tree), _ptr(v_tree),
        tree.cstruct, Hq, Hkv, Dh, _dtype_code(q), 0.0 if scale is None else float(scale),
        _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def ddtree_tree_attention_ranges_workspace_size(B, N, Hq, Hkv, Dh, ctx_len_host) -> int:
    a, p = _host_offsets(ctx_len_host)
    return int(lib.ddtree_tree_attention_ranges_workspace_size(B, N, Hq, Hkv, Dh, p))


def ddtree_tree_attention_ranges(q, k_ctx, v_ctx, ctx_start, ctx_len, ctx_start_host,
                                 ctx_len_host, k_tree, v_tree, tree, scale=None, out=None,
                                 want_lse=False, workspace=None, stream=None):
    """Tree attention with request b's context = rows [ctx_start[b], ctx_start[b] +
    ctx_len[b]) of k_ctx / v_ctx.  Returns (out [B, N, Hq, Dh], lse or None)."""
    return _ranges(lib.ddtree_tree_attention_ranges, q, k_ctx, v_ctx, ctx_start, ctx_len,
                   ctx_start_host, ctx_len_host, k_tree, v_tree, tree, scale, out, want_lse,
                   workspace, stream)


def ddtree_tree_attention_ranges_capped(q, k_ctx, v_ctx, ctx_start, ctx_len, ctx_start_host,
                                        ctx_cap_host, k_tree, v_tree, tree, scale=None, out=None,
                                        want_lse=False, workspace=None, stream=None):
    """ddtree_tree_attention_ranges with the lengths read from ctx_len on the device when
    the kernels run; ctx_cap_host (host) bounds them and fixes the plan, so a captured
    call stays valid while ctx_len grows up to the bounds.  Returns (out, lse or None)."""
    return _ranges(lib.ddtree_tree_attention_ranges_capped, q, k_ctx, v_ctx, ctx_start, ctx_len,
                   ctx_start_host, ctx_cap_host, k_tree, v_tree, tree, scale, out, want_lse,
                   workspace, stream)


def _ranges(fn, q, k_ctx, v_ctx, ctx_start, ctx_len, ctx_start_host, ctx_len_host, k_tree,
            v_tree, tree, scale, out, want_lse, workspace, stream):
    B, N, Hq, Dh = q.shape
    Hkv = k_tree.shape[2]
    _dev(q, "q", (torch.bfloat16, torch.float32))
    _dev(k_tree, "k_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(v_tree, "v_tree", q.dtype, (B, N, Hkv, Dh))
    _dev(k_ctx, "k_ctx", q.dtype)
    _dev(v_ctx, "v_ctx", q.dtype, tuple(k_ctx.shape))
    _dev(ctx_start, "ctx_start", torch.int32, (B,))
    _dev(ctx_len, "ctx_len", torch.int32, (B,))
    hs, hsp = _host_offsets(ctx_start_host)
    hl, hlp = _host_offsets(ctx_len_host)
    if hs.shape != (B,) or hl.shape != (B,):
        raise ValueError("ctx_start_host / ctx_len_host must hold B values")
    end = int((hs.astype(np.int64) + hl).max()) if B else 0
    if k_ctx.shape[0] < end or tuple(k_ctx.shape[1:]) != (Hkv, Dh):
        raise ValueError(f"k_ctx must be [>= {end}, {Hkv}, {Dh}]")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype, tuple(q.shape))
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    need = int(lib.ddtree_tree_attention_ranges_workspace_size(B, N, Hq, Hkv, Dh, hlp))
    workspace = _scratch(workspace, need, q.device, stream)
    _check(fn(
        _ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(ctx_start), _ptr(ctx_len), hsp, hlp,
        _ptr(k_tree), _ptr(v_tree), tree.cstruct, Hq, Hkv, Dh, _dtype_code(q),
        0.0 if scale is None else float(scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def ddtree_vocab_reduce_workspace_size(B, N, V) -> int:
    return int(lib.ddtree_vocab_reduce_workspace_size(B, N, V))


def ddtree_vocab_reduce(logits, num_nodes, temperature=0.0, want_lse=False, workspace=None,
                        stream=None):
    """Returns dict(argmax [B,N] i32, maxv [B,N] f32, R [B,N] and R_blocks
    [B,N,ceil(V/R_BLOCK)] int64 bits of uint64 (or None when greedy), lse [B,N] f32 or None)."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(num_nodes, "num_nodes", torch.int32, (B,))
    dev = logits.device
    argmax = torch.empty((B, N), dtype=torch.int32, device=dev)
    maxv = torch.empty((B, N), dtype=torch.float32, device=dev)
    R = torch.empty((B, N), dtype=torch.int64, device=dev) if temperature > 0 else None
    nb = (V + R_BLOCK - 1) // R_BLOCK
    Rb = torch.empty((B, N, nb), dtype=torch.int64, device=dev) if temperature > 0 else None
    lse = torch.empty((B, N), dtype=torch.float32, device=dev) if want_lse else None
    need = int(lib.ddtree_vocab_reduce_workspace_size(B, N, V))
    workspace = _scratch(workspace, need, dev, stream)
    _check(lib.ddtree_vocab_reduce(_ptr(logits), _dtype_code(logits), B, N, V, _ptr(num_nodes),
                                   float(temperature), _ptr(argmax), _ptr(maxv), _ptr(R),
                                   _ptr(Rb), _ptr(lse), _ptr(workspace), workspace.numel(),
                                   _stream(stream)))
    return {"argmax": argmax, "maxv": maxv, "R": R, "R_blocks": Rb, "lse": lse}


def _walk_outputs(tree):
    dev = tree.token.device
    return {"accept_len": torch.empty((tree.B,), dtype=torch.int32, device=dev),
            "path_nodes": torch.empty((tree.B, tree.D + 1), dtype=torch.int32, device=dev),
            "out_tokens": torch.empty((tree.B, tree.D + 1), dtype=torch.int32, device=dev),
            "bonus": torch.empty((tree.B,), dtype=torch.int32, device=dev)}


def ddtree_verify_greedy(tree, argmax, outputs=None, stream=None):
    _dev(argmax, "argmax", torch.int32, (tree.B, tree.N))
    o = outputs or _walk_outputs(tree)
    _check(lib.ddtree_verify_greedy(tree.cstruct, _ptr(argmax), _ptr(o["accept_len"]),
                                    _ptr(o["path_nodes"]), _ptr(o["out_tokens"]),
                                    _ptr(o["bonus"]), _stream(stream)))
    return o



def ddtree_vocab_verify_greedy(logits, tree, workspace=None, outputs=None, argmax=None, maxv=None,
                               stream=None):
    """ddtree_vocab_reduce (greedy) + ddtree_verify_greedy in one call: returns the
    walk's outputs plus "argmax" and "maxv"."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    if (B, N) != (tree.B, tree.N):
        raise ValueError(f"logits rows {(B, N)} do not match the tree {(tree.B, tree.N)}")
    dev = logits.device
    argmax = argmax if argmax is not None else torch.empty((B, N), dtype=torch.int32, device=dev)
    maxv = maxv if maxv is not None else torch.empty((B, N), dtype=torch.float32, device=dev)
    _dev(argmax, "argmax", torch.int32, (B, N))
    _dev(maxv, "maxv", torch.float32, (B, N))
    need = int(lib.ddtree_vocab_reduce_workspace_size(B, N, V))
    workspace = _scratch(workspace, need, dev, stream)
    o = outputs or _walk_outputs(tree)
    _check(lib.ddtree_vocab_verify_greedy(_ptr(logits), _dtype_code(logits), V, tree.cstruct,
                                          _ptr(argmax), _ptr(maxv), _ptr(o["accept_len"]),
                                          _ptr(o["path_nodes"]), _ptr(o["out_tokens"]),
                                          _ptr(o["bonus"]), _ptr(workspace), workspace.numel(),
                                          _stream(stream)))
    return dict(o, argmax=argmax, maxv=maxv)


def ddtree_verify_sample(tree, logits, maxv, R, R_blocks, temperature, uniforms, outputs=None,
                         stream=None):
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(maxv, "maxv", torch.float32, (B, N))
    _dev(R, "R", torch.int64, (B, N))
    _dev(R_blocks, "R_blocks", torch.int64, (B, N, (V + R_BLOCK - 1) // R_BLOCK))
    _dev(uniforms, "uniforms", torch.int64, (B, N, 2))
    o = outputs or _walk_outputs(tree)
    _check(lib.ddtree_verify_sample(tree.cstruct, _ptr(logits), _dtype_code(logits), V,
                                    _ptr(maxv), _ptr(R), _ptr(R_blocks), float(temperature),
                                    _ptr(uniforms),
                                    _ptr(o["accept_len"]), _ptr(o["path_nodes"]),
                                    _ptr(o["out_tokens"]), _ptr(o["bonus"]), _stream(stream)))
    return o


def ddtree_verify_sample_lazy(tree, logits, temperature, uniforms, outputs=None, stream=None):
    """The sampled walk reducing only the visited target rows (no vocab pass needed)."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(uniforms, "uniforms", torch.int64, (B, N, 2))
    o = outputs or _walk_outputs(tree)
    _check(lib.ddtree_verify_sample_lazy(tree.cstruct, _ptr(logits), _dtype_code(logits), V,
                                         float(temperature), _ptr(uniforms),
                                         _ptr(o["accept_len"]), _ptr(o["path_nodes"]),
                                         _ptr(o["out_tokens"]), _ptr(o["bonus"]),
                                         _stream(stream)))
    return o


def ddtree_verify_linear_sample(target_logits, draft_logits, draft_tokens, temperature, uniforms,
                                target_stats=None, draft_stats=None, outputs=None, stream=None):
    """Linear speculative sampling over a chain of D drafted tokens.  target_logits
    [B, D+1, V], draft_logits [B, D, V], draft_tokens [B, D] int32, uniforms [B, D+1, 2]
    int64 bits.  target_stats / draft_stats: ddtree_vocab_reduce results of the two
    tensors at this temperature (computed here when omitted).  Returns dict(accept_len
    [B], out_tokens [B, D+1], bonus [B])."""
    B, D1, V = target_logits.shape
    D = D1 - 1
    _dev(target_logits, "target_logits", (torch.bfloat16, torch.float32))
    _dev(draft_logits, "draft_logits", target_logits.dtype, (B, D, V))
    _dev(draft_tokens, "draft_tokens", torch.int32, (B, D))
    _dev(uniforms, "uniforms", torch.int64, (B, D + 1, 2))
    dev = target_logits.device
    if target_stats is None:
        target_stats = ddtree_vocab_reduce(
            target_logits, torch.full((B,), D + 1, dtype=torch.int32, device=dev), temperature)
    if draft_stats is None:
        draft_stats = ddtree_vocab_reduce(
            draft_logits, torch.full((B,), D, dtype=torch.int32, device=dev), temperature)
    o = outputs or {"accept_len": torch.empty((B,), dtype=torch.int32, device=dev),
                    "out_tokens": torch.empty((B, D + 1), dtype=torch.int32, device=dev),
                    "bonus": torch.empty((B,), dtype=torch.int32, device=dev)}
    _check(lib.ddtree_verify_linear_sample(
        _ptr(target_logits), _ptr(draft_logits), _dtype_code(target_logits), B, D, V,
        _ptr(draft_tokens), _ptr(target_stats["maxv"]), _ptr(target_stats["R"]),
        _ptr(target_stats["R_blocks"]), _ptr(draft_stats["maxv"]), _ptr(draft_stats["R"]),
        float(temperature), _ptr(uniforms), _ptr(o["accept_len"]), _ptr(o["out_tokens"]),
        _ptr(o["bonus"]), _stream(stream)))
    return o


def ddtree_vocab_top_p(logits, num_nodes, maxv, R, temperature, top_p, outputs=None,
                       stream=None):
    """Per node row: the top-p nucleus (thr_w, thr_id) and its totals (Rp, Rp_blocks)."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(num_nodes, "num_nodes", torch.int32, (B,))
    _dev(maxv, "maxv", torch.float32, (B, N))
    _dev(R, "R", torch.int64, (B, N))
    dev = logits.device
    nb = (V + R_BLOCK - 1) // R_BLOCK
    o = outputs or {"thr_w": torch.empty((B, N), dtype=torch.int64, device=dev),
                    "thr_id": torch.empty((B, N), dtype=torch.int32, device=dev),
                    "Rp": torch.empty((B, N), dtype=torch.int64, device=dev),
                    "Rp_blocks": torch.empty((B, N, nb), dtype=torch.int64, device=dev)}
    _check(lib.ddtree_vocab_top_p(_ptr(logits), _dtype_code(logits), B, N, V, _ptr(num_nodes),
                                  _ptr(maxv), _ptr(R), float(temperature), float(top_p),
                                  _ptr(o["thr_w"]), _ptr(o["thr_id"]), _ptr(o["Rp"]),
                                  _ptr(o["Rp_blocks"]), _stream(stream)))
    return o


def ddtree_verify_sample_top_p(tree, logits, maxv, nucleus, temperature, uniforms, outputs=None,
                               stream=None):
    """The sampled walk on the nuclei of ddtree_vocab_top_p (`nucleus`: its outputs)."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(maxv, "maxv", torch.float32, (B, N))
    _dev(nucleus["Rp"], "Rp", torch.int64, (B, N))
    _dev(nucleus["Rp_blocks"], "Rp_blocks", torch.int64, (B, N, (V + R_BLOCK - 1) // R_BLOCK))
    _dev(nucleus["thr_w"], "thr_w", torch.int64, (B, N))
    _dev(nucleus["thr_id"], "thr_id", torch.int32, (B, N))
    _dev(uniforms, "uniforms", torch.int64, (B, N, 2))
    o = outputs or _walk_outputs(tree)
    _check(lib.ddtree_verify_sample_top_p(
        tree.cstruct, _ptr(logits), _dtype_code(logits), V, _ptr(maxv), _ptr(nucleus["Rp"]),
        _ptr(nucleus["Rp_blocks"]), _ptr(nucleus["thr_w"]), _ptr(nucleus["thr_id"]),
        float(temperature), _ptr(uniforms), _ptr(o["accept_len"]), _ptr(o["path_nodes"]),
        _ptr(o["out_tokens"]), _ptr(o["bonus"]), _stream(stream)))
    return o


def ddtree_commit(tree, walk, k_tree, v_tree, k_cache, v_cache, cache_base, capacity,
                  next_prefix_len=None, next_root=None, stream=None):
    """Write the accepted path's K/V rows into the cache (in place).

    walk: a verify walk's outputs (accept_len, path_nodes, bonus); k_tree, v_tree
    [B, N, Hkv, Dh]; k_cache, v_cache [rows, Hkv, Dh] of the same dtype;
    cache_base int64 [B] (row of position 0 of each request).  Returns
    (next_prefix_len, next_root), int32 [B]."""
    B, N = tree.B, tree.N
    _dev(k_tree, "k_tree", (torch.bfloat16, torch.float32))
    if k_tree.dim() != 4 or tuple(k_tree.shape[:2]) != (B, N):
        raise ValueError(f"k_tree has shape {tuple(k_tree.shape)}, expected ({B}, {N}, Hkv, Dh)")
    Hkv, Dh = int(k_tree.shape[2]), int(k_tree.shape[3])
    _dev(v_tree, "v_tree", k_tree.dtype, tuple(k_tree.shape))
    _dev(k_cache, "k_cache", k_tree.dtype)
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (Hkv, Dh):
        raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, expected (rows, {Hkv}, {Dh})")
    _dev(v_cache, "v_cache", k_tree.dtype, tuple(k_cache.shape))
    _dev(cache_base, "cache_base", torch.int64, (B,))
    # a walk's outputs may sit in pinned host memory (read by the kernel over the bus)
    _dev(walk["accept_len"], "accept_len", torch.int32, (B,), pinned_ok=True)
    _dev(walk["path_nodes"], "path_nodes", torch.int32, (B, tree.D + 1), pinned_ok=True)
    _dev(walk["bonus"], "bonus", torch.int32, (B,), pinned_ok=True)
    dev = k_tree.device
    if next_prefix_len is None:
        next_prefix_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if next_root is None:
        next_root = torch.empty((B,), dtype=torch.int32, device=dev)
    _check(lib.ddtree_commit(tree.cstruct, _ptr(walk["accept_len"]), _ptr(walk["path_nodes"]),
                             _ptr(walk["bonus"]), _ptr(k_tree), _ptr(v_tree), Hkv, Dh,
                             _dtype_code(k_tree), _ptr(k_cache), _ptr(v_cache), _ptr(cache_base),
                             int(k_cache.shape[0]), int(capacity), _ptr(next_prefix_len),
                             _ptr(next_root), _stream(stream)))
    return next_prefix_len, next_root


def ddtree_sampling_constants(temperature):
    """(c, a[7]) the library uses for the integer softmax weights at this temperature."""
    c = ctypes.c_float()
    a = (ctypes.c_float * 7)()
    _check(lib.ddtree_sampling_constants(float(temperature), ctypes.byref(c), a))
    return np.float32(c.value), np.array(list(a), dtype=np.float32)
