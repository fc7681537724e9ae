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


def brute_fwd_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """Packed variable-length batch at 50 digits, read straight off the packed
    rows: query row i of sequence s (cu_q[s] <= i < cu_q[s+1]) sees key row j
    iff cu_k[s] <= j < cu_k[s+1] and, when causal,
    j - cu_k[s] <= (i - cu_q[s]) + (len_k(s) - len_q(s)).
    q [Hq, total_q, d], k, v [Hkv, total_k, d]; returns float64 (O, LSE)."""
    q, k, v = np.asarray(q, np.float64), np.asarray(k, np.float64), np.asarray(v, np.float64)
    Hq, tq, d = q.shape
    Hkv, tk = k.shape[0], k.shape[1]
    g = Hq // Hkv
    o = np.zeros((Hq, tq, d))
    lse = np.full((Hq, tq), -np.inf)
    with mpmath.workdps(DPS):
        sc = mpmath.mpf(scale)
        for h in range(Hq):
            kv = h // g
            for i in range(tq):
                s = max(t for t in range(len(cu_q) - 1) if cu_q[t] <= i)
                lq, lk = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
                js = [j for j in range(tk) if cu_k[s] <= j < cu_k[s + 1]
                      and (not causal or j - cu_k[s] <= (i - cu_q[s]) + (lk - lq))]
                if not js:
                    continue
                e = {j: mpmath.exp(sc * mpmath.fsum(mpmath.mpf(float(q[h, i, c])) * mpmath.mpf(float(k[kv, j, c]))
                                                    for c in range(d))) for j in js}
                z = mpmath.fsum(e.values())
                for c in range(d):
                    o[h, i, c] = float(mpmath.fsum(e[j] * mpmath.mpf(float(v[kv, j, c])) for j in js) / z)
                lse[h, i] = float(mpmath.log(z))
    return o, lse
