"""Oracle for per-position acceptance rates of chain speculative sampling, fp64, one sequence at a
time.

Test infrastructure only: imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.

Source: "論文解説: Speculative Sampling — ドラフトモデルによるLLMデコード高速化"
(0h-n0.github.io explainer of arXiv:2302.01318).  Step 3 (ステップ3) gives the probability of
accepting a drafted token x, min(1, p(x)/q(x)); the expected-speedup section (期待される高速化)
names alpha, the draft model's average acceptance rate, as the quantity the speedup depends on,
and the deployment section's monitoring list (監視・アラート) watches alpha continuously.

Reading: the acceptance rate of position i is the accept probability of Step 3 averaged over the
token the draft proposes there, x ~ q_i:
    alpha_i = sum_x q_i(x) * min(1, p_i(x) / q_i(x)),
which the mathematics reduces to sum_x min(p_i(x), q_i(x)) (the tests check both forms).  p_i and
q_i are the temperature softmaxes of target row i and draft row i, as in the chain verify.  A
row that defines no softmax (NaN, +inf, only -inf) gives NaN and ROW_NONFINITE; a temperature
that is not finite and positive is replaced by 1 and sets ROW_BAD_TEMPERATURE.
"""

import numpy as np

from .chain import ROW_BAD_TEMPERATURE, ROW_NONFINITE, row_is_valid, softmax_fp64, widen


def acceptance_rate(p, q):
    """Expected Step-3 accept probability of a token drawn from q: sum_x q(x) min(1, p(x)/q(x)),
    over the tokens with q(x) > 0 (the others are never drafted)."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    drafted = q > 0.0
    return float(np.sum(q[drafted] * np.minimum(1.0, p[drafted] / q[drafted])))


def acceptance_rates_seq(target, draft, temperature):
    """alpha_i for i < gamma of one sequence, with per-position status bits.

    target: [gamma+1, V] or [gamma, V] fp64 logits (a row gamma is not used); draft [gamma, V];
    temperature: scalar.  Returns (alpha [gamma] fp64, status [gamma] ints).
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    gamma = draft.shape[0]
    T = float(temperature)
    base = 0
    if not (np.isfinite(T) and T > 0.0):
        base |= ROW_BAD_TEMPERATURE
        T = 1.0
    alpha = np.empty(gamma)
    status = np.zeros(gamma, dtype=np.int64)
    for i in range(gamma):
        status[i] = base
        if not (row_is_valid(target[i]) and row_is_valid(draft[i])):
            status[i] |= ROW_NONFINITE
            alpha[i] = np.nan
            continue
        alpha[i] = acceptance_rate(softmax_fp64(target[i], T), softmax_fp64(draft[i], T))
    return alpha, status


def acceptance_rates_batch(target, draft, dtype, temperature, seqs=None):
    """acceptance_rates_seq over the sequences of a batch of stored logits (all, or listed)."""
    B = draft.shape[0]
    seqs = range(B) if seqs is None else seqs
    return [acceptance_rates_seq(widen(target[b], dtype), widen(draft[b], dtype), temperature[b])
            for b in seqs]
