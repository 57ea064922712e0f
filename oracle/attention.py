"""fp64 softmax attention of one query over a token set (oracle).

Test infrastructure only (see ``oracle/__init__.py``).

Definition (unite.ai axis-selection guide, values section): the attention
output is the sum of the value vectors over the tokens, weighted by the
softmax of the query-key scores.  Here the score of token t is
``alpha * sum_d q[d] * K[t, d]``.  Everything is computed in fp64 on inputs
that are exactly representable in fp64 (fp16 values and exactly dequantized
codes), so the only error is fp64 rounding.
"""

import numpy as np


def attention(q, k, v, alpha):
    """q [D], k [T, D], v [T, D] -> fp64 [D]; an empty token set gives 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[0], dtype=np.float64)
    scores = float(alpha) * (k @ q)
    p = np.exp(scores - scores.max())
    return (p @ v) / p.sum()


def partial(q, k, v, alpha):
    """Attention state of one token subset: (max score m, sum of
    exp(s - m), unnormalised sum of exp(s - m) * v).  Empty -> (-inf, 0, 0)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(q.shape[0], dtype=np.float64)
    scores = float(alpha) * (k @ q)
    m = scores.max()
    p = np.exp(scores - m)
    return m, p.sum(), p @ v


def merge(parts):
    """Combine subset states of disjoint token subsets into the output
    (log-sum-exp rescaling by exp(m_j - max_j m_j))."""
    parts = [p for p in parts if p[1] > 0]
    if not parts:
        return None
    top = max(p[0] for p in parts)
    den = sum(np.exp(m - top) * l for m, l, _ in parts)
    num = sum(np.exp(m - top) * acc for m, _, acc in parts)
    return num / den
