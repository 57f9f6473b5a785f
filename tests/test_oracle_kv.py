"""Pins of the KV compaction oracle against facts that do not come from it.

* Composition with the token-tree oracle (pinned by brute-force path enumeration): when every
  KV row encodes its node's token, the compacted rows read back as the root's token followed by
  the accepted tokens of the verification, and rows of rejected nodes never appear.
* The ai-compass worked example: the root and the two accepted candidates land in order.
* A chain equals a tree whose path is 0, 1, .., k; bytes outside the destination range and
  other sequences' caches are untouched; bad indices copy nothing.
"""

import json
import os

import numpy as np

from oracle import kv as OK
from oracle import tree as OT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def token_rows(tokens, W, seq):
    """KV rows whose bytes encode (sequence, node token): row u = pattern of tokens[u]."""
    rows = np.zeros((len(tokens), W), dtype=np.uint8)
    for u, t in enumerate(tokens):
        rows[u] = (np.arange(W) * 7 + int(t) * 31 + seq * 13) % 251
    return rows


def decode_rows(rows, vocab, seq):
    out = []
    for r in rows:
        hits = [t for t in range(vocab) if np.array_equal(r, token_rows([t], len(r), seq)[0])]
        out.append(hits[0] if len(hits) == 1 else None)
    return out


def test_compaction_after_tree_walk_yields_accepted_tokens():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n, V, W = int(rng.integers(2, 14)), 5, 48
        parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n)]
        tokens = [int(rng.integers(0, V)) for _ in range(n)]
        logits = rng.integers(-2, 3, size=(n, V)).astype(np.float64)
        for u in range(n):
            kids = [c for c in range(1, n) if parents[c] == u]
            if kids and rng.random() < 0.8:
                logits[u, tokens[kids[0]]] = 9.0
        r = OT.verify_tree_one(logits, parents, tokens)
        src = token_rows(tokens, W, trial)
        dst = np.full((20, W), 255, dtype=np.uint8)
        st = OK.compact_one(src, dst, r["path"] + [-1] * (n - len(r["path"])), r["k"], 3)
        assert st == 0
        got = decode_rows(dst[3:3 + r["k"] + 1], V, trial)
        assert got == [tokens[0]] + r["tokens"][:-1]           # root, then the accepted run
        assert np.all(dst[:3] == 255) and np.all(dst[4 + r["k"]:] == 255)


def test_golden_greedy_example():
    g = json.load(open(os.path.join(GOLDEN, "p2_greedy_example.json")))
    t = g["tree"]
    W = 16
    src = token_rows(t["node_tokens"], W, 0)
    dst = np.zeros((8, W), dtype=np.uint8)
    path = g["expected"]["path"] + [-1, -1]
    assert OK.compact_one(src, dst, path, g["expected"]["num_accepted"], 2) == 0
    # The root (the context's last token) and the two accepted candidates, in order.
    assert decode_rows(dst[2:5], len(g["vocab"]), 0) == [0, 1, 2]
    assert not dst[5:].any() and not dst[:2].any()


def test_chain_equals_identity_path_and_bad_indices():
    rng = np.random.default_rng(12)
    src = rng.integers(0, 256, size=(3, 6, 10), dtype=np.uint8)
    dst1 = np.zeros((3, 10, 10), dtype=np.uint8)
    dst2 = np.zeros((3, 10, 10), dtype=np.uint8)
    k = np.array([0, 3, 5])
    start = np.array([0, 2, 4])
    s1 = OK.compact_batch(src, dst1, None, k, start)
    s2 = OK.compact_batch(src, dst2, np.tile(np.arange(6), (3, 1)), k, start)
    assert not s1.any() and not s2.any() and np.array_equal(dst1, dst2)
    assert np.array_equal(dst1[2, 4:10], src[2, :6]) and np.array_equal(dst1[0, :1], src[0, :1])
    assert np.array_equal(dst1[1, 2:6], src[1, :4]) and not dst1[1, 6:].any()
    dst = np.zeros((1, 4, 10), dtype=np.uint8)
    assert OK.compact_one(src[0], dst[0], [0, 7, -1], 1, 0) == OK.ROW_BAD_INDEX
    assert OK.compact_one(src[0], dst[0], None, 6, 0) == OK.ROW_BAD_INDEX
    assert OK.compact_one(src[0], dst[0], None, 2, 2) == OK.ROW_BAD_INDEX
    assert not dst.any()
