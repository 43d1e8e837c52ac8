"""Verified-tree walks (oracle; test infrastructure only).

Greedy: "The Architecture of Speculative Decoding: Dissecting DDTree's
Tree-Parallel Evaluation Strategy", Section 1 step 5 -- from the root, move to
the child whose draft token equals the target argmax at the current node, stop
when no child matches; the result is the accepted chain plus one bonus token
(the argmax at the last node).

Sampled: same page, Section 3 ("Tree DDTree temperature"), and
"Implementing Temperature-Aware Tree Sampling for DDTree", "Path B: CPU-Side
Tree Rejection Sampling" -- at each node test the children in order, accept a
child with probability min(1, q/p), on rejection renormalise the target
distribution without the rejected token; if every child is rejected (or the
node is a leaf) draw the bonus token from the residual and stop.

Readings where the pages are silent:
  * the children are the deterministic best-first top-k, so each child's
    proposal is a point mass (p = 1) and the acceptance probability is the
    residual target probability q_res(token);
  * children are tried in rank order; a leaf draws its bonus from its full
    distribution;
  * the target law is the integer-weight softmax of the vocabulary step
    (weights w, row total R); a draw t = floor(u * R_res / 2^64) from a 64-bit
    uniform u accepts child c iff t < w(c), and the residual draw picks the
    smallest token x whose running sum of residual weights exceeds t.
    Uniform slot 0 of a node is its accept test, slot 1 its bonus draw.
"""
import numpy as np

from .vocab import weight_constants, weights


def _children(tree, b, n):
    out = []
    c = int(tree["first_child"][b, n])
    while c != -1:
        out.append(c)
        c = int(tree["next_sibling"][b, c])
    return out


def _outputs(B, D):
    return {"accept_len": np.zeros(B, dtype=np.int32),
            "path_nodes": np.full((B, D + 1), -1, dtype=np.int32),
            "out_tokens": np.full((B, D + 1), -1, dtype=np.int32),
            "bonus": np.zeros(B, dtype=np.int32)}


def verify_greedy(tree: dict, argmax, D: int) -> dict:
    """Greedy walk.  tree: build outputs; argmax [B, N]; D = draft depth.

    Returns accept_len [B], path_nodes [B, D+1] (root .. last accepted node, then -1),
    out_tokens [B, D+1] (accepted draft tokens, then the bonus, then -1), bonus [B]."""
    B = tree["token"].shape[0]
    res = _outputs(B, D)
    for b in range(B):
        cur, a = 0, 0
        res["path_nodes"][b, 0] = 0
        while True:
            target = int(argmax[b, cur])
            nxt = [c for c in _children(tree, b, cur) if int(tree["token"][b, c]) == target]
            if not nxt:
                break
            cur = nxt[0]
            a += 1
            res["path_nodes"][b, a] = cur
            res["out_tokens"][b, a - 1] = tree["token"][b, cur]
        res["accept_len"][b] = a
        res["bonus"][b] = argmax[b, cur]
        res["out_tokens"][b, a] = argmax[b, cur]
    return res


def _row_f32(logits, b, n, dtype):
    r = np.asarray(logits[b, n])
    if dtype == "bf16":
        return (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return r.astype(np.float32)


def verify_sample(tree: dict, logits, maxv, R, temperature: float, uniforms, D: int,
                  dtype: str = "f32", nucleus=None) -> dict:
    """Tree rejection sampling.  logits [B, N, V]; maxv, R from the vocabulary step;
    uniforms u64 [B, N, 2].  Same outputs as verify_greedy.

    nucleus: optional (thr_w, thr_id) [B, N] from the top-p oracle; a token then
    weighs w inside its row's kept set and 0 outside, and R must be the kept
    totals R_p ("Dissecting DDTree's Tree-Parallel Evaluation Strategy",
    Section 3: top_p threaded through to the verify walk)."""
    if not temperature > 0:
        raise ValueError("verify_sample needs temperature > 0")
    c, a = weight_constants(temperature)

    def wsel(row, ids, b, n):
        w = weights(row[ids], maxv[b, n], c, a)
        if nucleus is None:
            return w
        tw, ti = np.uint64(nucleus[0][b, n]), int(nucleus[1][b, n])
        keep = (w > tw) | ((w == tw) & (np.asarray(ids) <= ti))
        return np.where(keep, w, np.uint64(0))

    B = tree["token"].shape[0]
    res = _outputs(B, D)
    for b in range(B):
        cur, acc = 0, 0
        res["path_nodes"][b, 0] = 0
        while True:
            row = _row_f32(logits, b, cur, dtype)
            r_res = int(R[b, cur])
            rejected = []
            moved = False
            for ch in _children(tree, b, cur):
                tok = int(tree["token"][b, ch])
                wc = int(wsel(row, np.array([tok]), b, cur)[0])
                t = (int(uniforms[b, ch, 0]) * r_res) >> 64
                if t < wc:
                    cur = ch
                    acc += 1
                    res["path_nodes"][b, acc] = ch
                    res["out_tokens"][b, acc - 1] = tok
                    moved = True
                    break
                r_res -= wc
                rejected.append(tok)
            if moved:
                continue
            w = wsel(row, np.arange(row.shape[0]), b, cur)
            w[rejected] = 0
            assert int(w.sum(dtype=np.uint64)) == r_res
            t = (int(uniforms[b, cur, 1]) * r_res) >> 64
            csum = np.cumsum(w, dtype=np.uint64)
            x = int(np.searchsorted(csum, np.uint64(t), side="right"))
            res["bonus"][b] = x
            res["out_tokens"][b, acc] = x
            break
        res["accept_len"][b] = acc
    return res
