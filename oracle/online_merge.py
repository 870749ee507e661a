"""TEST INFRASTRUCTURE -- the online-softmax merge, restated in fp64 numpy.

Used only by the tests, to pin the two-pass oracle and the blockwise
recurrence against each other: splitting a score row into blocks, summarising
each block, and merging the summaries in any order must give the same output
and log-sum-exp as the two-pass softmax of the whole row.

Merge rule ("Self-Attention Kernel & Inference Engine from Scratch", section
"Online Softmax Formulation"): for two blocks with maxima m1, m2, normalisers
l1, l2 and normalised partial outputs O1, O2,

    m  = max(m1, m2)
    l  = exp(m1 - m) l1 + exp(m2 - m) l2
    O  = (exp(m1 - m) l1 / l) O1 + (exp(m2 - m) / l) (l2 O2)

where l2 O2 is the block's unnormalised sum of exp(x - m2) V, the second term
of the page's output update.  An empty block is (-inf, 0, 0) and merges as the
identity.
"""
from __future__ import annotations

import numpy as np


def block_summary(scores: np.ndarray, values: np.ndarray):
    """(m, l, O) of one block: its max, exp-sum and normalised weighted V sum."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scores.size == 0:
        return -np.inf, 0.0, np.zeros(values.shape[-1])
    m = scores.max()
    e = np.exp(scores - m)
    l = e.sum()
    return m, l, (e @ values) / l


def merge(a, b):
    m1, l1, o1 = a
    m2, l2, o2 = b
    if l1 == 0.0:
        return b
    if l2 == 0.0:
        return a
    m = max(m1, m2)
    w1 = np.exp(m1 - m)
    w2 = np.exp(m2 - m)
    l = w1 * l1 + w2 * l2
    return m, l, (w1 * l1 / l) * o1 + (w2 / l) * (l2 * o2)


def lse(summary) -> float:
    m, l, _ = summary
    return -np.inf if l == 0.0 else m + np.log(l)
