"""Per-node reduction over the target vocabulary (oracle; test infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 1 step 4: the target gives an argmax prediction
at every tree node in the one verify pass; Section 3: sampling needs the target
softmax at temperature T over the verify logits.

Readings where the pages are silent:
  * argmax ties go to the lowest token id; maxv is the logit at that id, with
    -0.0 written as +0.0.
  * the softmax used for sampling is represented exactly by integer weights
    w(l) ~ 2^32 * 2^((l - m) * log2(e) / T), m the row maximum, computed by
    the fixed fp32 recipe in `weights`; R = sum of w over the row (exact
    integer).  The sampled law is then w/R, within ~1e-6 relative of
    softmax(l / T), and identical on any machine that follows the recipe.
  * lse (informational) is the natural-log log-sum-exp of the raw logits.
"""
import math

import numpy as np

# 1/ln(2) as the nearest double (C's M_LOG2E)
LOG2E = float.fromhex("0x1.71547652b82fep+0")
# tokens per block of the per-block weight sums (a layout choice of the
# interface, not of the pages: any partition of the row sums to R)
R_BLOCK = 32768


def weight_constants(temperature: float):
    """(c, a): c = fp32(LOG2E / T) with T taken as fp32; a[n] = fp32((ln 2)^n / n!)
    for n = 0..6 (Taylor coefficients of 2^f)."""
    t32 = float(np.float32(temperature))
    c = np.float32(LOG2E / t32)
    a = np.array([math.log(2.0) ** n / math.factorial(n) for n in range(7)], dtype=np.float32)
    return c, a


def weights(l, m, c, a) -> np.ndarray:
    """Integer weights of logits l (float32) against row max m, following the recipe:

      y = (l - m) * c                       (two fp32 roundings, no fused multiply-add)
      y < -32  ->  w = 0
      k = round-half-even(y);  f = y - k    (f in [-1/2, 1/2])
      p = a6; p = p*f + a5; ...; p = p*f + a0   (each * and + rounded to fp32 separately)
      w = floor(p * 2^(32 + k))             (exact; w <= 2^33)
    """
    l = np.asarray(l, dtype=np.float32)
    y = (l - np.float32(m)) * np.float32(c)
    k = np.rint(y)
    f = y - k
    p = np.full_like(f, a[6])
    for n in range(5, -1, -1):
        p = p * f
        p = p + a[n]
    e = np.where(y < np.float32(-32.0), 0, 32 + k).astype(np.int64)
    w = np.floor(np.ldexp(p.astype(np.float64), e)).astype(np.uint64)
    w[y < np.float32(-32.0)] = 0
    return w


def vocab_reduce(logits, num_nodes, temperature: float = 0.0, dtype: str = "f32",
                 rows=None) -> dict:
    """logits [B, N, V] (bf16 bits as uint16, or float32); num_nodes [B].

    Returns argmax i32 [B, N], maxv f32 [B, N], lse f64 [B, N] and, if T > 0,
    R u64 [B, N] and R_blocks u64 [B, N, ceil(V / R_BLOCK)]: the same weights
    summed over each run of R_BLOCK consecutive tokens (a partition of R, used
    to locate a residual draw).  Padding rows (n >= num_nodes[b]): argmax -1,
    maxv -inf, lse -inf, R 0, R_blocks 0.  `rows` optionally restricts the work
    to a list of (b, n)."""
    x = np.asarray(logits)
    B, N, V = x.shape
    argmax = np.full((B, N), -1, dtype=np.int32)
    maxv = np.full((B, N), -np.inf, dtype=np.float32)
    lse = np.full((B, N), -np.inf, dtype=np.float64)
    R = np.zeros((B, N), dtype=np.uint64)
    nb = -(-V // R_BLOCK)
    R_blocks = np.zeros((B, N, nb), dtype=np.uint64)
    if temperature > 0:
        c, a = weight_constants(temperature)
    todo = [(b, n) for b in range(B) for n in range(int(num_nodes[b]))] if rows is None else rows
    for b, n in todo:
        if dtype == "bf16":
            row = (x[b, n].astype(np.uint32) << np.uint32(16)).view(np.float32)
        else:
            row = x[b, n].astype(np.float32)
        i = int(np.argmax(row))
        argmax[b, n] = i
        maxv[b, n] = row[i] + np.float32(0.0)
        r64 = row.astype(np.float64)
        lse[b, n] = np.logaddexp.reduce(r64)
        if temperature > 0:
            w = weights(row, maxv[b, n], c, a)
            R[b, n] = int(w.sum(dtype=np.uint64))
            for k in range(nb):
                R_blocks[b, n, k] = int(w[k * R_BLOCK:(k + 1) * R_BLOCK].sum(dtype=np.uint64))
    return {"argmax": argmax, "maxv": maxv, "lse": lse, "R": R, "R_blocks": R_blocks}
