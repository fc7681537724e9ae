"""The online-softmax state as a monoid: TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

"Não escreva kernels, derive-os", section "Aprofundamento" (first paragraph),
and "Tang Project Derives GPU Kernels via IR ...", section "Details" (first
bullet), name the streaming softmax as a monoid reduction; neither page writes
the rule out, so it is written here from the definition of softmax.

For one query row, a set of keys J is summarised by
    m = max_{j in J} s_j,   l = sum_{j in J} exp(s_j - m),   acc = sum_{j in J} exp(s_j - m) v_j
with the empty set mapped to the identity (-inf, 0, 0).  Two disjoint sets
combine by rescaling both to the larger maximum.  The fold over any grouping of
the keys gives the same (m, l, acc) up to rounding, and
    O = acc / l,   LSE = m + ln l
is softmax attention.  Everything here is fp64 numpy.
"""
from __future__ import annotations

import math

import numpy as np


def identity(d: int):
    return (-math.inf, 0.0, np.zeros(d, np.float64))


def leaf(s_j: float, v_j) -> tuple:
    """The state of a single key with (already scaled) score s_j and value row v_j."""
    return (float(s_j), 1.0, np.asarray(v_j, np.float64).copy())


def combine(a, b):
    """(m1,l1,a1) (+) (m2,l2,a2).  A side whose maximum is -inf contributes nothing."""
    m1, l1, a1 = a
    m2, l2, a2 = b
    m = max(m1, m2)
    if m == -math.inf:
        return (-math.inf, 0.0, np.zeros_like(a1))
    f1 = 0.0 if m1 == -math.inf else math.exp(m1 - m)
    f2 = 0.0 if m2 == -math.inf else math.exp(m2 - m)
    return (m, l1 * f1 + l2 * f2, a1 * f1 + a2 * f2)


def fold(states, d: int):
    out = identity(d)
    for s in states:
        out = combine(out, s)
    return out


def finalize(state):
    """(O row, LSE) of a state; the identity gives O = 0, LSE = -inf."""
    m, l, acc = state
    if l == 0.0:
        return np.zeros_like(acc), -math.inf
    return acc / l, m + math.log(l)
