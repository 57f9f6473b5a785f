"""Oracle for greedy chain verification (zero-temperature speculative decoding), one sequence
at a time, fp64.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Source: "投機的デコーディングとは？LLMの回答を高速化する仕組み" (ai-compass.weeybrid.co.jp),
section 候補の採用と棄却を具体例で見る (the worked example of accepting and rejecting
candidates): the target model checks the draft's candidates in order, keeps each candidate
that equals the token it would itself choose, and at the first candidate that differs discards
that candidate and everything after it and substitutes its own choice.  Under greedy decoding
the target's choice at a position is the argmax of its logits there.  The accept test of the
Speculative Sampling explainer (Step 3, ステップ3) reduces to the same rule when the
temperature goes to zero (p and q become one-hot), which the tests use as an independent pin.

Readings of points the page leaves open:

* Target row i scores draft token i; row gamma is the position after the last draft token, and
  its argmax is appended when every draft token is accepted (as the stochastic verify appends
  a bonus token).
* argmax ties resolve to the lowest token id; -0.0 equals +0.0; NaN is never the maximum (a row
  holding NaN sets ROW_NONFINITE; a row of only NaN yields 0).
* A draft token outside [0, V) sets ROW_TOKEN_RANGE and the sequence takes the fallback result:
  nothing accepted, the argmax of row 0 emitted.
"""

import numpy as np

from .chain import ROW_NONFINITE, ROW_TOKEN_RANGE, widen
from .tree import argmax_first


def verify_chain_greedy_seq(target, draft_tokens):
    """Verify one sequence greedily.

    target: [gamma+1, V] fp64 target logits; draft_tokens: [gamma] ints.
    Returns a dict: k (drafts accepted), tokens (the k accepted drafts then the target's choice
    at position k), g (argmax of every target row) and status bits.
    """
    target = np.asarray(target, dtype=np.float64)
    rows, V = target.shape
    gamma = rows - 1
    toks = [int(x) for x in draft_tokens]
    assert len(toks) == gamma
    status = 0
    g = []
    for i in range(rows):
        gi, had_nan = argmax_first(target[i])
        g.append(gi)
        if had_nan:
            status |= ROW_NONFINITE
    if any(not (0 <= x < V) for x in toks):
        status |= ROW_TOKEN_RANGE
        return {"k": 0, "tokens": [g[0]], "g": g, "status": status}
    k = 0
    while k < gamma and toks[k] == g[k]:
        k += 1
    return {"k": k, "tokens": toks[:k] + [g[k]], "g": g, "status": status}


def verify_chain_greedy_batch(target, dtype, draft_tokens, seqs=None):
    """Run verify_chain_greedy_seq over the sequences of a batch (all, or the listed ones).

    target [B, gamma+1, V] holds stored logits of the given dtype ("f32" or "bf16" bit
    patterns).
    """
    B = target.shape[0]
    seqs = range(B) if seqs is None else seqs
    return [verify_chain_greedy_seq(widen(target[b], dtype), draft_tokens[b]) for b in seqs]
