"""Oracle for chain verification (speculative sampling), fp64, one sequence at a time.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Each step follows the explainer of arXiv:2302.01318, "論文解説: Speculative
Sampling — ドラフトモデルによるLLMデコード高速化" (0h-n0.github.io), in its own
order:

1. Step 2 (ステップ2, 一括検証): the target gives gamma+1 distributions p_0..p_gamma
   from one pass; the draft gave q_0..q_{gamma-1}.  Both are temperature
   softmaxes of logits (the code sketch divides logits by the temperature
   before the softmax, for the draft and the target alike).
2. Step 3 (ステップ3, 受理/棄却判定): draft token i is accepted with probability
   min(1, p_i(x_i) / q_i(x_i)), tested in order i = 0, 1, ...; everything after
   the first rejection is discarded.
3. Modified rejection sampling (修正付き棄却サンプリング): on a rejection at
   position k, the replacement token is drawn from norm(max(0, p_k - q_k)).
4. When every draft token is accepted, one more token is drawn from the
   target's last distribution p_gamma (the expected-speedup section counts up
   to gamma+1 tokens per round, so a round that accepts all gamma drafts yields
   a (gamma+1)-th token).

Readings of points the page leaves open:

* Random numbers are inputs: uniforms[0:gamma] drive the accept tests and
  uniforms[gamma] drives the single draw (residual or bonus) by inverse CDF in
  token-id order, y = min{x : sum_{t<=x} w(t) > u * sum_t w(t)}.
* The accept test is the strict comparison u < min(1, p/q) of the page's code
  sketch.  q(x) = 0 < p(x) counts as ratio +inf (accept); p(x) = q(x) = 0
  rejects.  No epsilon is added to any denominator.
* Target row i scores draft token i; row gamma is the bonus position.
* If the residual mass is zero (possible only through rounding or degenerate
  inputs), the draw falls back to p_k and ROW_RESIDUAL_ZERO is set.
* Invalid data (a draft token outside [0, V), a NaN or +inf logit, a row of all
  -inf, a temperature that is not finite and positive, a uniform outside
  [0, 1)) sets its status bit and the sequence takes the fallback result
  (0 accepted, emitted token 0).
"""

import numpy as np

ROW_TOKEN_RANGE = 1
ROW_NONFINITE = 2
ROW_RESIDUAL_ZERO = 4
ROW_BAD_TREE = 8
ROW_BAD_TEMPERATURE = 16
ROW_BAD_UNIFORM = 32
FALLBACK_BITS = ROW_TOKEN_RANGE | ROW_NONFINITE | ROW_BAD_TEMPERATURE | ROW_BAD_UNIFORM

# Half-width of the bands inside which fp32-level rounding may legitimately flip
# an integer decision: |u - min(1, p/q)| for an accept test, and the distance of
# u*W to the nearer bucket edge of the inverse CDF, relative to W.
BAND = 1e-6


def widen(a, dtype):
    """Stored logits widened exactly to fp64.

    fp32 values convert exactly.  bf16 values are stored as their 16-bit
    patterns (uint16); a bf16 number is the fp32 number whose upper 16 bits are
    that pattern and whose lower 16 bits are zero.
    """
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown logit dtype {dtype!r}")


def row_is_valid(z):
    """A logit row defines a softmax iff it has no NaN, no +inf, and not only -inf."""
    return not (np.isnan(z).any() or np.isposinf(z).any() or np.isneginf(z).all())


def softmax_fp64(z, temperature):
    """Temperature softmax p(x) = exp((z(x) - max z) / T) / sum_x' exp((z(x') - max z) / T).

    Step 2 (ステップ2) and the code sketch of the Speculative Sampling explainer:
    both models' logits are divided by the temperature and passed through a
    softmax.  Subtracting the maximum does not change the result.
    """
    m = np.max(z)
    e = np.exp((z - m) / temperature)
    return e / np.sum(e)


def accept_threshold(p_x, q_x):
    """min(1, p(x)/q(x)) for the drafted token x, or None when both are zero.

    Step 3 (ステップ3) accept equation of the Speculative Sampling explainer.
    q(x) = 0 < p(x) is the ratio +inf, whose minimum with 1 is 1.
    """
    if q_x > 0.0:
        return min(1.0, p_x / q_x)
    if p_x > 0.0:
        return 1.0
    return None


def residual_weights(p, q):
    """Unnormalised residual max(0, p(x) - q(x)).

    Modified rejection sampling (修正付き棄却サンプリング) equation of the
    Speculative Sampling explainer; normalisation is left to the draw.
    """
    return np.maximum(0.0, p - q)


def inverse_cdf(w, u):
    """Draw by inverse CDF in token-id order: y = min{x : C(x) > u * W}.

    C is the running sum of the non-negative weights w in token-id order and W
    its total, so a token with zero weight is never chosen.  Also returns the
    distance of u*W to the nearer edge of bucket y, divided by W.  Bucket y is
    [C(y-1), C(y)) with C(-1) = 0: the lower distance is u*W - C(y-1), the upper
    one C(y) - u*W.
    """
    c = np.cumsum(w)
    total = c[-1]
    tau = u * total
    above = c > tau
    y = int(np.argmax(above))
    lower = c[y - 1] if y > 0 else 0.0
    edge = min(tau - lower, c[y] - tau) / total
    return y, float(edge)


def draw_band(w, u):
    """Tokens an inverse-CDF draw may return when its running sums and u * W carry an error
    below BAND * W (the parity band of the draw).

    Token x of positive weight is drawn exactly when u * W falls in its bucket
    [C(x-1), C(x)); an error of less than BAND * W can move u * W only into a bucket that
    intersects [u*W - BAND*W, u*W + BAND*W].  So the set holds the exact draw y, the token
    across each edge of bucket y that lies within the band (the nearest positive-weight
    neighbour on that side), and further tokens only when a neighbour's whole bucket is
    narrower than the band.  Zero-weight tokens have empty buckets and never appear.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    total = c[-1]
    tau = u * total
    b = BAND * total
    lo = np.concatenate(([0.0], c[:-1]))
    near = (w > 0.0) & (lo <= tau + b) & (c > tau - b)
    return {int(x) for x in np.flatnonzero(near)}


def _fallback(gamma, status):
    return {
        "k": 0, "tokens": [0], "p_at": np.full(gamma, np.nan), "q_at": np.full(gamma, np.nan),
        "status": status, "flag_accept": [], "edge": 1.0, "draw": None, "weights": None,
    }


def verify_chain_seq(target, draft, draft_tokens, uniforms, temperature, force=None):
    """Verify one sequence.

    target: [gamma+1, V] fp64 target logits (row i scores draft token i, row
    gamma is the bonus position); draft: [gamma, V] fp64 draft logits;
    draft_tokens: [gamma] ints; uniforms: [gamma+1]; temperature: scalar.
    force: optional {position: bool} that overrides the accept decision at a
    position (used to replay the other outcome of a test inside the band).

    Returns a dict: k (drafts accepted), tokens (the k accepted drafts then the
    drawn token), p_at / q_at (p_i(x_i), q_i(x_i) for every i < gamma), status
    bits, flag_accept (positions whose test fell inside the band), edge (the
    relative edge distance of the draw), draw ("residual", "residual_zero" or
    "bonus") and weights (the unnormalised weights the draw used).
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    gamma, V = draft.shape
    assert target.shape == (gamma + 1, V)
    toks = np.asarray(draft_tokens, dtype=np.int64)
    u = np.asarray(uniforms, dtype=np.float64)
    T = float(temperature)

    status = 0
    if not (np.isfinite(T) and T > 0.0):
        status |= ROW_BAD_TEMPERATURE
    if not np.all((u >= 0.0) & (u < 1.0)):
        status |= ROW_BAD_UNIFORM
    if np.any((toks < 0) | (toks >= V)):
        status |= ROW_TOKEN_RANGE
    if not all(row_is_valid(z) for z in list(target) + list(draft)):
        status |= ROW_NONFINITE
    if status & FALLBACK_BITS:
        return _fallback(gamma, status)

    p = [softmax_fp64(target[i], T) for i in range(gamma + 1)]
    q = [softmax_fp64(draft[i], T) for i in range(gamma)]
    p_at = np.array([p[i][toks[i]] for i in range(gamma)])
    q_at = np.array([q[i][toks[i]] for i in range(gamma)])

    k = gamma
    flag_accept = []
    for i in range(gamma):
        thr = accept_threshold(p_at[i], q_at[i])
        accept = thr is not None and u[i] < thr
        if thr is not None and abs(u[i] - thr) < BAND:
            flag_accept.append(i)
        if force is not None and i in force:
            accept = bool(force[i])
        if not accept:
            k = i
            break

    if k < gamma:
        w = residual_weights(p[k], q[k])
        draw = "residual"
        if not np.sum(w) > 0.0:
            w = p[k]
            status |= ROW_RESIDUAL_ZERO
            draw = "residual_zero"
    else:
        w = p[gamma]
        draw = "bonus"
    y, edge = inverse_cdf(w, u[gamma])
    tokens = [int(t) for t in toks[:k]] + [y]
    return {
        "k": k, "tokens": tokens, "p_at": p_at, "q_at": q_at, "status": status,
        "flag_accept": flag_accept, "edge": edge, "draw": draw, "weights": w,
    }


def verify_chain_batch(target, draft, dtype, draft_tokens, uniforms, temperature, seqs=None):
    """Run verify_chain_seq over the sequences of a batch (all, or the listed ones).

    target [B, gamma+1, V] and draft [B, gamma, V] hold stored logits of the
    given dtype ("f32" or "bf16" bit patterns).  Returns the per-sequence dicts
    in the order of seqs.
    """
    B = target.shape[0]
    seqs = range(B) if seqs is None else seqs
    out = []
    for b in seqs:
        out.append(verify_chain_seq(
            widen(target[b], dtype), widen(draft[b], dtype), draft_tokens[b],
            uniforms[b], temperature[b]))
    return out
