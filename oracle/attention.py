"""Tree attention with the context loaded once (oracle; test infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 1 step 4 and Section 2: all budget+1 tree
tokens of a request are queries of one batched pass; every one of them sees
the request's whole cached context, and among the tree tokens only its own
ancestors (plus itself, the causal reading).  Written as the textbook formula

    o_i = sum_j softmax_j(scale * q_i . k_j) v_j,
    j in context[0, L_b)  union  {tree nodes j visible from i},

evaluated directly in float64 for every (request, query head, node).
Grouped heads: query head h reads KV head h // (Hq / Hkv).
Reading: scale = 1/sqrt(Dh) unless the caller passes another value (the pages
do not state it).  Nodes past num_nodes[b] are padding: output 0, lse -inf.
"""
import numpy as np


def to_f64(x, dtype: str) -> np.ndarray:
    """Exact upcast of stored values: bf16 bit patterns (uint16) or float32."""
    x = np.asarray(x)
    if dtype == "bf16":
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _visible(vis_row: np.ndarray, N: int) -> np.ndarray:
    return np.array([(int(vis_row[j // 64]) >> (j % 64)) & 1 for j in range(N)], dtype=bool)


def tree_attention(q, k_ctx, v_ctx, ctx_offsets, k_tree, v_tree, vis, num_nodes, scale=None,
                   dtype="f32", requests=None, heads=None):
    """q [B, N, Hq, Dh]; k_ctx, v_ctx [sum L, Hkv, Dh]; k_tree, v_tree [B, N, Hkv, Dh];
    ctx_offsets [B+1]; vis u64 [B, N, W]; num_nodes [B].

    Returns (o, lse): o float64 [B, N, Hq, Dh], lse float64 [B, N, Hq] (natural log of
    the softmax denominator of the scaled scores).  `requests` / `heads` restrict
    the work to a subset (other entries stay NaN) for spot checks at full size."""
    q = to_f64(q, dtype)
    B, N, Hq, Dh = q.shape
    Hkv = k_tree.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(Dh)
    o = np.full((B, N, Hq, Dh), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    req = range(B) if requests is None else requests
    hs = range(Hq) if heads is None else heads
    for b in req:
        L0, L1 = int(ctx_offsets[b]), int(ctx_offsets[b + 1])
        nn = int(num_nodes[b])
        o[b, nn:] = 0.0
        lse[b, nn:] = -np.inf
        for h in hs:
            kvh = h // g
            kc = to_f64(k_ctx[L0:L1, kvh], dtype)       # [L, Dh]
            vc = to_f64(v_ctx[L0:L1, kvh], dtype)
            kt = to_f64(k_tree[b, :, kvh], dtype)       # [N, Dh]
            vt = to_f64(v_tree[b, :, kvh], dtype)
            for i in range(nn):
                sel = _visible(vis[b, i], N)
                keys = np.concatenate([kc, kt[sel]], axis=0)
                vals = np.concatenate([vc, vt[sel]], axis=0)
                s = keys @ q[b, i, h] * scale
                m = s.max()
                p = np.exp(s - m)
                den = p.sum()
                o[b, i, h] = (p @ vals) / den
                lse[b, i, h] = m + np.log(den)
    return o, lse
