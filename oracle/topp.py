"""Top-p (nucleus) truncation of the target law for the sampled walk (oracle;
test infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 3: temperature and top_p are threaded through to
the verify step, whose sampling walk then runs on the truncated, renormalised
target distribution.

Readings where the pages are silent:
  * top-p keeps the smallest set of most probable tokens whose probability
    reaches p (nucleus sampling); "most probable" orders tokens by their
    integer softmax weight w (the vocabulary oracle's), larger first, and equal
    weights by token id, smaller first;
  * "reaches p" is decided exactly: with P = rint(p * 2^32) (p taken as fp32,
    P clamped to [1, 2^32]) and R the row's weight total, the kept prefix is
    the shortest whose weight sum S satisfies 2^32 * S >= P * R;
  * the kept set is then {w > w*} plus the tokens of weight w* up to id*, where
    w* and id* are the weight and id of the prefix's last token; the walk runs
    unchanged on w_p = w inside the set and 0 outside, with total R_p = S.
"""
import numpy as np

from .vocab import R_BLOCK, weight_constants, weights


def top_p_fixed(top_p) -> int:
    """P = rint(p * 2^32) for p as fp32, clamped to [1, 2^32]."""
    p = float(np.float32(top_p))
    if not (p > 0.0 and p <= 1.0):
        raise ValueError("top_p must be in (0, 1]")
    return int(min(max(int(np.rint(p * 2.0 ** 32)), 1), 1 << 32))


def nucleus_row(w, P: int):
    """w: integer weights of one row (any int sequence).  Returns (w*, id*, R_p)."""
    w = [int(x) for x in w]
    R = sum(w)
    order = sorted(range(len(w)), key=lambda y: (-w[y], y))
    acc = 0
    for y in order:
        acc += w[y]
        if (acc << 32) >= P * R:
            return w[y], y, acc
    raise AssertionError("the whole row must reach any p <= 1")


def keep_mask(w, thr_w: int, thr_id: int) -> np.ndarray:
    w = np.asarray(w, dtype=np.uint64)
    ids = np.arange(w.shape[0])
    return (w > np.uint64(thr_w)) | ((w == np.uint64(thr_w)) & (ids <= thr_id))


def _row(logits, b, n, dtype):
    r = np.asarray(logits[b, n])
    if dtype == "bf16":
        return (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return r.astype(np.float32)


def vocab_top_p(logits, maxv, num_nodes, temperature: float, top_p, dtype: str = "f32",
                rows=None) -> dict:
    """Per node row: thr_w u64 [B, N], thr_id i32 [B, N], Rp u64 [B, N] and
    Rp_blocks u64 [B, N, ceil(V / R_BLOCK)] (the kept weights per token block).
    Padding rows: thr_w 0, thr_id -1, Rp 0, Rp_blocks 0.  `rows` optionally
    restricts the work to a list of (b, n)."""
    c, a = weight_constants(temperature)
    P = top_p_fixed(top_p)
    x = np.asarray(logits)
    B, N, V = x.shape
    nb = (V + R_BLOCK - 1) // R_BLOCK
    out = {"thr_w": np.zeros((B, N), np.uint64), "thr_id": np.full((B, N), -1, np.int32),
           "Rp": np.zeros((B, N), np.uint64), "Rp_blocks": np.zeros((B, N, nb), np.uint64)}
    todo = rows if rows is not None else [(b, n) for b in range(B) for n in range(int(num_nodes[b]))]
    for b, n in todo:
        w = weights(_row(x, b, n, dtype), maxv[b, n], c, a)
        tw, tid, rp = nucleus_row(w, P)
        kept = np.where(keep_mask(w, tw, tid), w, np.uint64(0))
        out["thr_w"][b, n] = tw
        out["thr_id"][b, n] = tid
        out["Rp"][b, n] = rp
        for k in range(nb):
            out["Rp_blocks"][b, n, k] = int(kept[k * R_BLOCK:(k + 1) * R_BLOCK].sum(dtype=np.uint64))
    return out
