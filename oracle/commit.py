"""Commit of the accepted path into the context KV cache (oracle; test
infrastructure only).

"The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
Evaluation Strategy", Section 1 step 5 and its summary: after the walk the
single longest verified path is committed; Section 2: the context is a cache
that later steps read once and that grows by the committed tokens.

Readings where the pages are silent:
  * what is committed are the keys and values the verify pass computed for the
    root (the token anchored at position prefix_len, whose KV was not cached
    yet) and for the accepted nodes -- the walk's path_nodes[0 .. accept_len];
    the bonus token is not committed: it has no K/V yet and becomes the next
    step's root;
  * node n of the tree is stored at its tree position (prefix_len + depth), so
    the path lands on positions prefix_len .. prefix_len + accept_len;
  * the cache holds, per request b, the rows of positions 0, 1, ... starting at
    row cache_base[b] of a [rows, Hkv, Dh] array (the layout of the attention's
    packed context); a position >= capacity is not written (the request's
    cache is full) while the returned length still advances;
  * the next step's prefix length is prefix_len + accept_len + 1 and its root
    token is the bonus.
"""
import numpy as np


def commit_path(tree: dict, accept_len, path_nodes, bonus, k_tree, v_tree, k_cache, v_cache,
                cache_base, capacity: int) -> dict:
    """tree: the build's outputs (position [B, N] is used); accept_len [B];
    path_nodes [B, D+1]; bonus [B]; k_tree, v_tree [B, N, Hkv, Dh];
    k_cache, v_cache [rows, Hkv, Dh] (not modified: copies are returned);
    cache_base [B] row of position 0 of each request.

    Returns {"k_cache", "v_cache", "next_prefix_len" [B], "next_root" [B]}."""
    position = np.asarray(tree["position"])
    accept_len = np.asarray(accept_len)
    path_nodes = np.asarray(path_nodes)
    bonus = np.asarray(bonus)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    B = position.shape[0]
    nxt = np.zeros(B, dtype=np.int32)
    root = np.zeros(B, dtype=np.int32)
    for b in range(B):
        a = int(accept_len[b])
        for j in range(a + 1):
            n = int(path_nodes[b, j])
            pos = int(position[b, n])
            if pos < capacity:
                row = int(cache_base[b]) + pos
                k_out[row] = k_tree[b, n]
                v_out[row] = v_tree[b, n]
        nxt[b] = int(position[b, 0]) + a + 1
        root[b] = int(bonus[b])
    return {"k_cache": k_out, "v_cache": v_out, "next_prefix_len": nxt, "next_root": root}
