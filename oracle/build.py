"""Best-first token-tree build (oracle; test infrastructure only).

Follows "The Architecture of Speculative Decoding: Dissecting DDTree's
Tree-Parallel Evaluation Strategy", Section 1, steps 2 and 3: a heap keyed by
cumulative draft log-prob; repeatedly take the best entry, add it to the tree,
then offer its best child and its next sibling, until `budget` nodes besides
the root are chosen.  The visibility of a node is its ancestors (step 3) plus
itself; the position of a node at depth d is prefix_len + d ("The Tree That
Couldn't Branch", "Hypothesis 3: Position Encoding Bugs").  The candidates of
every depth-d node are that depth's top-K, independent of the path
("Hypothesis 4: The Block-Diffusion Fundamental Limitation").

Readings where the pages are silent:
  * score(child) = fp32(score(parent) + draft_lp[depth(child)-1, rank(child)]),
    one round-to-nearest-even fp32 add; the root scores +0.0.
  * frontier order: larger score first; ties by smaller parent index, then by
    smaller rank (a total order, since (parent, rank) is unique).
  * nodes are numbered in the order they are taken, root = 0.
  * a node sees itself as well as its ancestors.
"""
import heapq

import numpy as np

PAD = -1


def N_WORDS(N: int) -> int:
    return (N + 63) // 64


def build_tree(draft_lp, draft_tok, root_tok, prefix_len, budget: int) -> dict:
    """draft_lp f32 [B, D, K], draft_tok i32 [B, D, K], root_tok [B], prefix_len [B].

    Returns [B, N] arrays (N = budget + 1): token, parent, depth, rank, position,
    first_child, next_sibling (i32), score (f32), vis (u64 [B, N, W]),
    num_nodes (i32 [B]) and max_depth (i32 [B], the depth of the deepest node
    taken: the statistic of "Hypothesis 1: Best-First Search Exhaustion").
    Entries past num_nodes[b] hold -1 (score -inf, vis 0)."""
    lp = np.asarray(draft_lp, dtype=np.float32)
    tok = np.asarray(draft_tok, dtype=np.int32)
    B, D, K = lp.shape
    N = budget + 1
    W = N_WORDS(N)
    out = {name: np.full((B, N), PAD, dtype=np.int32)
           for name in ("token", "parent", "depth", "rank", "position", "first_child",
                        "next_sibling")}
    out["score"] = np.full((B, N), -np.inf, dtype=np.float32)
    out["vis"] = np.zeros((B, N, W), dtype=np.uint64)
    out["num_nodes"] = np.zeros(B, dtype=np.int32)
    out["max_depth"] = np.zeros(B, dtype=np.int32)

    for b in range(B):
        score = out["score"][b]
        vis = out["vis"][b]
        # root
        out["token"][b, 0] = root_tok[b]
        out["depth"][b, 0] = 0
        out["position"][b, 0] = prefix_len[b]
        score[0] = np.float32(0.0)
        vis[0, 0] = np.uint64(1)
        count = 1
        heap = []

        def offer(s, parent, rank, depth, pusher):
            s = np.float32(s) + np.float32(0.0)       # -0.0 -> +0.0
            heapq.heappush(heap, (-float(s), parent, rank, depth, pusher))

        if D >= 1 and K >= 1 and budget >= 1:
            offer(score[0] + lp[b, 0, 0], 0, 0, 1, 0)
        while heap and count < N:
            negs, parent, rank, depth, pusher = heapq.heappop(heap)
            i = count
            count += 1
            out["token"][b, i] = tok[b, depth - 1, rank]
            out["parent"][b, i] = parent
            out["depth"][b, i] = depth
            out["max_depth"][b] = max(out["max_depth"][b], depth)
            out["rank"][b, i] = rank
            out["position"][b, i] = prefix_len[b] + depth
            score[i] = np.float32(-negs)
            vis[i] = vis[parent]
            vis[i, i // 64] |= np.uint64(1) << np.uint64(i % 64)
            if rank == 0:
                out["first_child"][b, parent] = i
            else:
                out["next_sibling"][b, pusher] = i
            if depth < D:                              # best child of the new node
                offer(score[i] + lp[b, depth, 0], i, 0, depth + 1, i)
            if rank + 1 < K:                           # next sibling of the new node
                offer(score[parent] + lp[b, depth - 1, rank + 1], parent, rank + 1, depth, i)
        out["num_nodes"][b] = count
    return out
