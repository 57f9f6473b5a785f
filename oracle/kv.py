"""Oracle for accepted-path KV compaction, one sequence (or tree) at a time.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Sources: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
(0h-n0.github.io explainer of arXiv:2302.01318), implementation notes (実装上の注意点), KV cache
management (KVキャッシュ管理): the cache entries of rejected tokens must be removed (rolled back);
SpecInfer article (abeam.tech, arXiv:2305.09781), inference (推論方法): the verified run of
matching tokens is appended to the sequence.

Reading: the verification pass computed one KV row per speculated position, including the
position that feeds the first draft (the chain's last committed token, the tree's root); row u
of a sequence's block belongs to node u (chain position u).  After verification the rows of the
accepted path -- the root and the k accepted nodes -- become the next k + 1 rows of the
sequence's cache, in path order; rejected rows are not copied.  Rows are opaque byte strings.
A path entry outside the block, k outside [0, path length - 1], or a destination range past the
cache's end sets ROW_BAD_INDEX and the sequence copies nothing.
"""

import numpy as np

ROW_BAD_INDEX = 64


def compact_one(src_block, dst_cache, path, k, dst_start):
    """Copy rows path[0..k] of src_block [src_rows, W] to dst_cache rows dst_start..dst_start+k.

    path: node ids (None for a chain: 0, 1, .., k).  Modifies dst_cache [dst_rows, W] in place;
    returns status bits.
    """
    src_rows = src_block.shape[0]
    dst_rows = dst_cache.shape[0]
    plen = src_rows if path is None else len(path)
    if not (0 <= k <= plen - 1) or dst_start < 0 or dst_start + k + 1 > dst_rows:
        return ROW_BAD_INDEX
    rows = list(range(k + 1)) if path is None else [int(path[j]) for j in range(k + 1)]
    if any(not (0 <= r < src_rows) for r in rows):
        return ROW_BAD_INDEX
    for j, r in enumerate(rows):
        dst_cache[dst_start + j, :] = src_block[r, :]
    return 0


def compact_batch(src, dst, paths, num_accepted, dst_start):
    """compact_one over every sequence: src [n, src_rows, W] bytes, dst [n, dst_rows, W] bytes
    (modified in place), paths [n, path_len] ints or None, num_accepted [n], dst_start [n].
    Returns the status bits per sequence."""
    st = []
    for b in range(src.shape[0]):
        st.append(compact_one(src[b], dst[b], None if paths is None else paths[b],
                              int(num_accepted[b]), int(dst_start[b])))
    return np.array(st, dtype=np.int64)
