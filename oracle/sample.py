"""Oracle for the draft-side sampler: one token per logit row from the temperature softmax, fp64.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Source: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
(0h-n0.github.io explainer of arXiv:2302.01318), Step 1 (ステップ1) and the code sketch's draft
loop: the draft model proposes each token by sampling from the softmax of its logits divided by
the temperature.

Readings (shared with the chain oracle's draws):
* The random number is an input: y = min{x : sum_{t<=x} p(t) > u * sum_t p(t)}, inverse CDF in
  token-id order with u in [0, 1), so a token of probability zero is never drawn.
* A row that defines no softmax (NaN, +inf, only -inf) sets ROW_NONFINITE, a temperature that
  is not finite and positive ROW_BAD_TEMPERATURE, a uniform outside [0, 1) ROW_BAD_UNIFORM; such
  a row takes the fallback token 0.
* p(y) is returned with the token (the draft keeps q(y) for its own bookkeeping).
"""

import numpy as np

from .chain import (ROW_BAD_TEMPERATURE, ROW_BAD_UNIFORM, ROW_NONFINITE, inverse_cdf,
                    row_is_valid, softmax_fp64, widen)


def sample_row(z, temperature, u):
    """Draw one token from softmax(z / T) with the uniform u.

    Returns a dict: token, prob (p(token)), status bits, edge (relative distance of u * W to
    the nearer bucket edge, as in the chain oracle's draws) and weights (p).
    """
    z = np.asarray(z, dtype=np.float64)
    T = float(temperature)
    u = float(u)
    status = 0
    if not (np.isfinite(T) and T > 0.0):
        status |= ROW_BAD_TEMPERATURE
    if not (0.0 <= u < 1.0):
        status |= ROW_BAD_UNIFORM
    if not row_is_valid(z):
        status |= ROW_NONFINITE
    if status:
        return {"token": 0, "prob": np.nan, "status": status, "edge": 1.0, "weights": None}
    p = softmax_fp64(z, T)
    y, edge = inverse_cdf(p, u)
    return {"token": y, "prob": float(p[y]), "status": status, "edge": edge, "weights": p}


def sample_batch(logits, dtype, temperature, uniforms, rows=None):
    """sample_row over the rows of a batch of stored logits [R, V] (all, or the listed ones)."""
    rows = range(logits.shape[0]) if rows is None else rows
    return [sample_row(widen(logits[r], dtype), temperature[r], uniforms[r]) for r in rows]
