"""Linear (chain) speculative sampling with the draft's own probabilities
(oracle; test infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 3, linear DFlash at temperature T: per position,
accept the drafted token t with probability min(1, p_target(t) / p_draft(t)),
otherwise draw from the residual and stop; "Mistakes and Incorrect
Assumptions": this needs the draft's full probability of the sampled token,
not only its top-k log-probs.

Readings where the pages are silent:
  * the drafted tokens were sampled by the draft from its full softmax at the
    same temperature T; the draft probabilities are that softmax (the draft
    logits are an input);
  * the residual is the standard one, proportional to max(0, q - p);
  * both distributions are represented exactly by the integer weights of the
    vocabulary oracle (w / R, each row with its own maximum), so every test is
    exact integer arithmetic: the draft token x at position i is accepted iff
        floor(u0 * wp(x) * Rq / 2^64) < wq(x) * Rp
    (u0 the position's first 64-bit uniform: probability min(1, q(x)/p(x))),
    and a rejection draws t = floor(u1 * Rr / 2^64) from the residual weights
    r(y) = max(0, wq(y) * Rp - wp(y) * Rq), Rr = sum r, taking the smallest y
    whose running sum exceeds t (u1 the position's second uniform).  If Rr is
    0 (q and p proportional; a rejection then needs wq(x) = wp(x) = 0) the
    draw is from q itself;
  * after D accepted tokens the bonus is drawn from the target row D with the
    second uniform of position D.
"""
import numpy as np

from .vocab import weight_constants, weights


def _row(x, b, i, dtype):
    r = np.asarray(x[b, i])
    if dtype == "bf16":
        return (r.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return r.astype(np.float32)


def _weights_int(row, c, a):
    m = row.max() + np.float32(0.0)
    w = weights(row, m, c, a)
    return [int(v) for v in w], int(w.sum(dtype=np.uint64))


def _draw(vals, total, u):
    """Smallest index whose running sum of `vals` exceeds floor(u * total / 2^64)."""
    t = (int(u) * total) >> 64
    acc = 0
    for y, v in enumerate(vals):
        acc += v
        if acc > t:
            return y
    raise AssertionError("draw past the end of the row")


def verify_linear_sample(target_logits, draft_logits, draft_tokens, temperature: float,
                         uniforms, dtype: str = "f32") -> dict:
    """target_logits [B, D+1, V] (row i: the target's distribution for position
    i + 1), draft_logits [B, D, V] (row i: the draft distribution the token of
    position i + 1 was drawn from), draft_tokens [B, D], uniforms u64 [B, D+1, 2].

    Returns accept_len [B], out_tokens [B, D+1] (the accepted draft tokens, then
    the residual or bonus token, then -1) and bonus [B] (that last token)."""
    if not temperature > 0:
        raise ValueError("linear sampling needs temperature > 0")
    c, a = weight_constants(temperature)
    tl = np.asarray(target_logits)
    draft_logits = np.asarray(draft_logits)
    draft_tokens = np.asarray(draft_tokens)
    uniforms = np.asarray(uniforms, dtype=np.uint64)
    B, D1, V = tl.shape
    D = D1 - 1
    acc_len = np.zeros(B, dtype=np.int32)
    out = np.full((B, D + 1), -1, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        k = 0
        while k < D:
            wq, Rq = _weights_int(_row(tl, b, k, dtype), c, a)
            wp, Rp = _weights_int(_row(draft_logits, b, k, dtype), c, a)
            x = int(draft_tokens[b, k])
            if (int(uniforms[b, k, 0]) * wp[x] * Rq) >> 64 < wq[x] * Rp:
                out[b, k] = x
                k += 1
                continue
            r = [max(0, wq[y] * Rp - wp[y] * Rq) for y in range(V)]
            Rr = sum(r)
            tok = _draw(r, Rr, uniforms[b, k, 1]) if Rr > 0 else _draw(wq, Rq, uniforms[b, k, 1])
            break
        else:
            wq, Rq = _weights_int(_row(tl, b, D, dtype), c, a)
            tok = _draw(wq, Rq, uniforms[b, D, 1])
        acc_len[b] = k
        out[b, k] = tok
        bonus[b] = tok
    return {"accept_len": acc_len, "out_tokens": out, "bonus": bonus}
