"""Oracle for greedy token-tree verification (SpecInfer style), one tree at a time.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Source: the SpecInfer article (abeam.tech, arXiv:2305.09781), sections
"基本アイデア" (basic idea) and "推論方法" (inference): the large model scores
every node of the token tree in one pass, giving for each node the token that
should follow the sequence ending at that node; verification then starts at the
root, follows the branch whose tokens agree with those outputs, and appends the
run of agreeing tokens.  Greedy outputs are the argmax of each node's logits.

Readings of points the page leaves open:

* Logit row u scores the children of node u; node 0 is the root, whose token is
  already committed and is not emitted.
* The tree is a parent-index array with parents[0] = -1 and
  0 <= parents[i] < i for every other node (parents precede children).
* argmax ties resolve to the lowest token id; -0.0 equals +0.0; NaN is never
  the maximum (a row holding NaN sets ROW_NONFINITE; a row of only NaN yields 0).
* Among children with the wanted token the one with the lowest node id is
  taken (siblings carry distinct tokens when candidates are merged by common
  prefix, so this choice only matters for malformed input).
* After the accepted run, the argmax of the last accepted node is appended as
  the bonus token (as in the greedy worked example of the ai-compass page,
  where the target's own token replaces the first mismatching candidate).
* A malformed tree or a node token outside [0, V) sets its status bit and the
  tree takes the fallback result: nothing accepted, the root's argmax emitted.
"""

import numpy as np

from .chain import ROW_BAD_TREE, ROW_NONFINITE, ROW_TOKEN_RANGE


def argmax_first(z):
    """(lowest index x with z[x] == max z over non-NaN entries, whether z held NaN)."""
    z = np.asarray(z, dtype=np.float64)
    ok = ~np.isnan(z)
    if not ok.any():
        return 0, True
    m = np.max(z[ok])
    return int(np.flatnonzero(ok & (z == m))[0]), bool((~ok).any())


def tree_is_valid(parents):
    n = len(parents)
    if n < 1 or parents[0] != -1:
        return False
    return all(0 <= parents[i] < i for i in range(1, n))


def verify_tree_one(logits, parents, node_tokens):
    """Verify one tree.

    logits: [n_nodes, V] fp64; parents, node_tokens: [n_nodes] ints.
    Returns a dict: path (node ids from the root to the last accepted node),
    tokens (accepted tokens then the bonus argmax), k (nodes accepted),
    g (argmax of every node) and status bits.
    """
    logits = np.asarray(logits, dtype=np.float64)
    n, V = logits.shape
    parents = [int(x) for x in parents]
    node_tokens = [int(x) for x in node_tokens]
    status = 0
    g = []
    for u in range(n):
        gu, had_nan = argmax_first(logits[u])
        g.append(gu)
        if had_nan:
            status |= ROW_NONFINITE
    if not tree_is_valid(parents):
        status |= ROW_BAD_TREE
    if any(not (0 <= node_tokens[i] < V) for i in range(1, n)):
        status |= ROW_TOKEN_RANGE
    if status & (ROW_BAD_TREE | ROW_TOKEN_RANGE):
        return {"path": [0], "tokens": [g[0]], "k": 0, "g": g, "status": status}

    path = [0]
    u = 0
    while True:
        nxt = None
        for c in range(1, n):
            if parents[c] == u and node_tokens[c] == g[u]:
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        u = nxt
    tokens = [node_tokens[c] for c in path[1:]] + [g[u]]
    return {"path": path, "tokens": tokens, "k": len(path) - 1, "g": g, "status": status}


def verify_tree_batch(logits, dtype, parents, node_tokens, trees=None):
    """Run verify_tree_one over the trees of a batch (all, or the listed ones)."""
    from .chain import widen
    n_trees = logits.shape[0]
    trees = range(n_trees) if trees is None else trees
    return [verify_tree_one(widen(logits[t], dtype), parents[t], node_tokens[t]) for t in trees]
