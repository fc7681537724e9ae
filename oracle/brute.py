"""50-digit brute force of softmax attention: TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

An evaluation path independent of attn_oracle.c, for tiny shapes only:
  * exp(s_ij) / sum_j exp(s_ij) taken literally, with no max subtraction
    (mpmath's exponent range makes that safe);
  * gradients by central finite differences of L = sum(dO * O) with h = 1e-20
    at 50 significant digits, which needs no analytic derivative at all.

The shared readings (bottom-right causal alignment, kv(h) = h / (Hq/Hkv), an
empty row giving O = 0 and LSE = -inf) are restated here, not imported.
"""
from __future__ import annotations

import mpmath
import numpy as np

DPS = 50


def _mp(a):
    return [[[[mpmath.mpf(float(x)) for x in row] for row in head] for head in bat] for bat in np.asarray(a)]


def _fwd_mp(Q, K, V, scale, causal):
    B, Hq, Nq, d = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    Hkv, Nk = len(K[0]), len(K[0][0])
    g = Hq // Hkv
    O = [[[[mpmath.mpf(0)] * d for _ in range(Nq)] for _ in range(Hq)] for _ in range(B)]
    LSE = [[[None] * Nq for _ in range(Hq)] for _ in range(B)]
    sc = mpmath.mpf(scale)
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            for i in range(Nq):
                js = [j for j in range(Nk) if (not causal) or j <= i + (Nk - Nq)]
                if not js:
                    LSE[b][h][i] = mpmath.mpf("-inf")
                    continue
                e = {}
                for j in js:
                    s = sc * mpmath.fsum(Q[b][h][i][c] * K[b][kv][j][c] for c in range(d))
                    e[j] = mpmath.exp(s)
                z = mpmath.fsum(e.values())
                for c in range(d):
                    O[b][h][i][c] = mpmath.fsum(e[j] * V[b][kv][j][c] for j in js) / z
                LSE[b][h][i] = mpmath.log(z)
    return O, LSE


def brute_fwd(q, k, v, scale: float, causal: bool):
    """(O, LSE) as float64 arrays, evaluated at 50 digits."""
    with mpmath.workdps(DPS):
        O, LSE = _fwd_mp(_mp(q), _mp(k), _mp(v), scale, causal)
        o = np.array([[[[float(x) for x in r] for r in h] for h in b] for b in O], np.float64)
        lse = np.array([[[float(x) for x in h] for h in b] for b in LSE], np.float64)
    return o, lse


def _loss(Q, K, V, dO, scale, causal):
    O, _ = _fwd_mp(Q, K, V, scale, causal)
    tot = mpmath.mpf(0)
    for b in range(len(O)):
        for h in range(len(O[0])):
            for i in range(len(O[0][0])):
                for c in range(len(O[0][0][0])):
                    tot += dO[b][h][i][c] * O[b][h][i][c]
    return tot


def fd_grads(q, k, v, dout, scale: float, causal: bool, h: str = "1e-20"):
    """Central finite differences of sum(dout * O) w.r.t. q, k and v (float64 arrays)."""
    with mpmath.workdps(DPS):
        Q, K, V, dO = _mp(q), _mp(k), _mp(v), _mp(dout)
        step = mpmath.mpf(h)
        grads = []
        for T, shape in ((Q, np.shape(q)), (K, np.shape(k)), (V, np.shape(v))):
            g = np.zeros(shape, np.float64)
            for idx in np.ndindex(*shape):
                b, hh, n, c = idx
                x0 = T[b][hh][n][c]
                T[b][hh][n][c] = x0 + step
                lp = _loss(Q, K, V, dO, scale, causal)
                T[b][hh][n][c] = x0 - step
                lm = _loss(Q, K, V, dO, scale, causal)
                T[b][hh][n][c] = x0
                g[idx] = float((lp - lm) / (2 * step))
            grads.append(g)
    return tuple(grads)
