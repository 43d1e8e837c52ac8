"""Per-depth top-K of the draft head (oracle; test infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 1 step 1: from the hidden state of every depth
position, the draft's vocabulary head yields the top-k candidate tokens and
their log-probs, which step 2 turns into cumulative scores; Section 3 notes
that the draft probabilities come from these top-k log-probs.

Readings where the pages are silent:
  * the log-prob is the full-vocabulary log-softmax of the row at temperature
    1 (not renormalised over the top-K), computed in float64 and rounded once
    to fp32;
  * candidates are ordered by logit, descending, ties to the lower token id.
"""
import math

import numpy as np


def log_sum_exp(row) -> float:
    """Natural-log log-sum-exp of one row, in float64: m + log(sum(exp(x - m)))."""
    x = np.asarray(row, dtype=np.float64)
    m = float(x.max())
    return m + math.log(float(np.exp(x - m).sum()))


def topk_row(row, K: int):
    """(tokens [K] i32, log-probs [K] f32) of one row of logits."""
    x = np.asarray(row, dtype=np.float64)
    V = x.shape[0]
    if not 1 <= K <= V:
        raise ValueError(f"K={K} must be in [1, V={V}]")
    # order by (value desc, id asc): lexsort's last key is the primary one
    order = np.lexsort((np.arange(V), -x))[:K]
    lse = log_sum_exp(x)
    return order.astype(np.int32), (x[order] - lse).astype(np.float32)


def draft_topk(draft_logits, K: int):
    """Top-K tokens and full-vocabulary log-probs of every row.

    draft_logits: [..., V] (float32, or bf16 values already widened to float32).
    Returns (tokens [..., K] int32, log-probs [..., K] float32)."""
    x = np.asarray(draft_logits, dtype=np.float32)
    lead, V = x.shape[:-1], x.shape[-1]
    flat = x.reshape(-1, V)
    tok = np.empty((flat.shape[0], K), dtype=np.int32)
    lp = np.empty((flat.shape[0], K), dtype=np.float32)
    for r in range(flat.shape[0]):
        tok[r], lp[r] = topk_row(flat[r], K)
    return tok.reshape(*lead, K), lp.reshape(*lead, K)


def attach_draft_topk(inputs: dict, D: int, K: int) -> dict:
    """Adds the oracle's draft top-K of inputs["draft_logits"] [B, D+1, V]:
    draft_tok_all [B, D+1, K] (every row; the target-logit planting reads its
    ranking) and the tree build's inputs draft_tok, draft_lp [B, D, K] (rows
    0..D-1).  Returns the same dict."""
    tok, lp = draft_topk(inputs["draft_logits"], K)
    inputs["draft_tok_all"] = tok
    inputs["draft_tok"] = np.ascontiguousarray(tok[:, :D])
    inputs["draft_lp"] = np.ascontiguousarray(lp[:, :D])
    return inputs
