"""CPU oracle for fused softmax attention: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never imports, links or calls it, and
this package imports nothing from the GPU library: the two share no code.

Contents
  attn_oracle.c  plain fp64 three-pass forward and analytic backward (C, OpenMP)
  __init__.py    wrappers; fwd_varlen / fwd_varlen_rows compose the dense
                 forward per sequence of a packed variable-length batch
  monoid.py      the online-softmax state (m, l, acc) and its combine rule
  brute.py       50-digit mpmath evaluation of the definition (no max shift)

The C library is compiled with the host gcc into ``liboracle.so`` next to this
file.  ``build()`` compiles it unconditionally; ``lib()`` compiles it only if no
build exists yet (or the source is newer than the build).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile attn_oracle.c with gcc -O2 -fopenmp into liboracle.so."""
    tmp = _LIB + ".tmp"
    subprocess.run(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"],
        check=True,
    )
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    L = ctypes.CDLL(_LIB)
    i64, f64, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
    L.oracle_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f64, ci]
    L.oracle_fwd_rows.argtypes = [vp, vp, vp, vp, i64, vp, vp, i64, i64, i64, i64, i64, i64, f64, ci]
    L.oracle_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f64, ci]
    L.oracle_bwd_rowdot.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f64, ci]
    for f in (L.oracle_fwd, L.oracle_fwd_rows, L.oracle_bwd, L.oracle_bwd_rowdot, L.oracle_num_threads):
        f.restype = ci
    _lib = L
    return L


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Nq, Nk, d


def fwd(q, k, v, scale: float, causal: bool):
    """Three-pass softmax attention.  Returns (O [B,Hq,Nq,d], LSE [B,Hq,Nq]) in fp64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    o = np.empty((B, Hq, Nq, d), np.float64)
    lse = np.empty((B, Hq, Nq), np.float64)
    rc = lib().oracle_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), B, Hq, Hkv, Nq, Nk, d, float(scale), int(causal))
    if rc:
        raise ValueError(f"oracle_fwd rejected its arguments ({rc})")
    return o, lse


def fwd_rows(q, k, v, rows, scale: float, causal: bool):
    """Forward on selected rows.  rows: int array [n, 3] of (b, h, i).  Returns (O [n,d], LSE [n])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib().oracle_fwd_rows(_p(q), _p(k), _p(v), _p(rows), n, _p(o), _p(lse), B, Hq, Hkv, Nq, Nk, d,
                               float(scale), int(causal))
    if rc:
        raise ValueError(f"oracle_fwd_rows rejected its arguments ({rc})")
    return o, lse


def bwd(q, k, v, dout, scale: float, causal: bool):
    """Analytic gradient of sum(dout * O).  Returns (dQ, dK, dV) in fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    dq = np.empty((B, Hq, Nq, d), np.float64)
    dk = np.empty((B, Hkv, Nk, d), np.float64)
    dv = np.empty((B, Hkv, Nk, d), np.float64)
    rc = lib().oracle_bwd(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv), B, Hq, Hkv, Nq, Nk, d,
                          float(scale), int(causal))
    if rc:
        raise ValueError(f"oracle_bwd rejected its arguments ({rc})")
    return dq, dk, dv


def rowdot(q, k, v, dout, scale: float, causal: bool):
    """D_i = sum_j P_ij (dO_i . V_j), from the definition.  Returns [B,Hq,Nq] fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, Hq, Hkv, Nq, Nk, d = _dims(q, k, v)
    out = np.empty((B, Hq, Nq), np.float64)
    rc = lib().oracle_bwd_rowdot(_p(q), _p(k), _p(v), _p(dout), _p(out), B, Hq, Hkv, Nq, Nk, d, float(scale),
                                 int(causal))
    if rc:
        raise ValueError(f"oracle_bwd_rowdot rejected its arguments ({rc})")
    return out


def fwd_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """Packed variable-length batch: sequence s is the dense problem on query
    rows [cu_q[s], cu_q[s+1]) and key rows [cu_k[s], cu_k[s+1]) of every head
    (its own keys only; causal alignment per sequence), solved by fwd above.
    q [Hq, total_q, d], k, v [Hkv, total_k, d].  Returns (O [Hq, total_q, d],
    LSE [Hq, total_q]) in fp64.  Rows outside every sequence stay NaN."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    Hq, tq, d = q.shape
    o = np.full((Hq, tq, d), np.nan)
    lse = np.full((Hq, tq), np.nan)
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        c, e = int(cu_k[s]), int(cu_k[s + 1])
        if b == a:
            continue
        os_, ls_ = fwd(q[None, :, a:b], k[None, :, c:e], v[None, :, c:e], scale, causal)
        o[:, a:b] = os_[0]
        lse[:, a:b] = ls_[0]
    return o, lse


def fwd_varlen_rows(q, k, v, cu_q, cu_k, rows, scale: float, causal: bool):
    """Like fwd_varlen on selected rows only.  rows: int array [n, 2] of (h, i)
    with i a packed query row.  Returns (O [n, d], LSE [n])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    rows = np.asarray(rows, np.int64).reshape(-1, 2)
    cu_q = np.asarray(cu_q, np.int64)
    seq = np.searchsorted(cu_q, rows[:, 1], side="right") - 1
    o = np.empty((rows.shape[0], q.shape[2]))
    lse = np.empty(rows.shape[0])
    for s in np.unique(seq):
        sel = np.nonzero(seq == s)[0]
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        c, e = int(cu_k[s]), int(cu_k[s + 1])
        local = np.stack([np.zeros(len(sel), np.int64), rows[sel, 0], rows[sel, 1] - a], axis=1)
        os_, ls_ = fwd_rows(q[None, :, a:b], k[None, :, c:e], v[None, :, c:e], local, scale, causal)
        o[sel] = os_
        lse[sel] = ls_
    return o, lse


def e4m3_value(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> fp64 values, from the format's
    definition: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
    exponent 0 encodes (m / 8) 2^-6, otherwise (1 + m / 8) 2^(e - 7); the
    all-ones exponent and mantissa (0x7F, 0xFF) is NaN; no infinities."""
    c = np.asarray(codes, np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    return np.where((c & 0x7F) == 0x7F, np.nan, sign * mag)


def decode_fp8(q, k8, v8, k_scale, v_scale, scale: float):
    """One decode query per stream against an FP8 cache: the keys and values
    are k_scale[h] * E4M3(code) and v_scale[h] * E4M3(code) for kv head h,
    every key visible.  Solved per kv head with fwd above on the exact code
    values (fp32-exact) and the scales applied in fp64: the scores take
    scale * k_scale[h] as their scale and O is multiplied by v_scale[h] (the
    softmax weights do not depend on v).  Returns (O [B,Hq,1,d], LSE [B,Hq,1])."""
    q = _f32(q)
    B, Hq, Nq, d = q.shape
    Hkv = np.asarray(k8).shape[1]
    g = Hq // Hkv
    o = np.empty((B, Hq, Nq, d))
    lse = np.empty((B, Hq, Nq))
    for h in range(Hkv):
        k = e4m3_value(np.asarray(k8)[:, h:h + 1]).astype(np.float32)
        v = e4m3_value(np.asarray(v8)[:, h:h + 1]).astype(np.float32)
        oh, lh = fwd(q[:, h * g:(h + 1) * g], k, v, float(scale) * float(k_scale[h]), False)
        o[:, h * g:(h + 1) * g] = oh * float(v_scale[h])
        lse[:, h * g:(h + 1) * g] = lh
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, seq_lens, scale: float):
    """One decode query per stream against a paged cache: stream b's keys are
    j = 0 .. seq_lens[b] - 1, key j in slot j % P of page block_table[b, j // P]
    (P the page size), cache layout [num_pages, Hkv, P, d]; every key visible.
    The stream's keys are gathered into a dense [1, Hkv, L, d] history and
    solved with fwd above; a stream with no keys gets O = 0, LSE = -inf.
    Returns (O [B,Hq,1,d], LSE [B,Hq,1])."""
    q = _f32(q)
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    bt, sl = np.asarray(block_table), np.asarray(seq_lens)
    B, Hq, Nq, d = q.shape
    P = kc.shape[2]
    o = np.zeros((B, Hq, Nq, d))
    lse = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        L = int(sl[b])
        if L <= 0:
            continue
        j = np.arange(L)
        pages, slots = bt[b, j // P], j % P
        k = np.ascontiguousarray(kc[pages, :, slots, :].transpose(1, 0, 2)[None])  # [1, Hkv, L, d]
        v = np.ascontiguousarray(vc[pages, :, slots, :].transpose(1, 0, 2)[None])
        o[b:b + 1], lse[b:b + 1] = fwd(q[b:b + 1], k, v, scale, False)
    return o, lse


def fwd_varlen_paged(q, k_cache, v_cache, block_table, cu_q, lens_k, scale: float, causal: bool):
    """Packed variable-length forward with the keys of sequence s in pages:
    key j in slot j % P of page block_table[s, j // P] of a [num_pages, Hkv,
    P, d] cache.  Each sequence's keys are gathered into a packed [Hkv,
    sum(lens_k), d] history and fwd_varlen above solves the batch.  Returns
    (O [Hq, total_q, d], LSE [Hq, total_q])."""
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    bt = np.asarray(block_table)
    P = kc.shape[2]
    ks, vs = [], []
    for s_, L in enumerate(np.asarray(lens_k)):
        j = np.arange(max(int(L), 0))
        ks.append(kc[bt[s_, j // P], :, j % P, :].transpose(1, 0, 2))  # [Hkv, L, d]
        vs.append(vc[bt[s_, j // P], :, j % P, :].transpose(1, 0, 2))
    k = np.ascontiguousarray(np.concatenate(ks, axis=1))
    v = np.ascontiguousarray(np.concatenate(vs, axis=1))
    cu_k = np.concatenate([[0], np.cumsum(np.maximum(np.asarray(lens_k, np.int64), 0))]).astype(np.int32)
    return fwd_varlen(q, k, v, cu_q, cu_k, scale, causal)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel regions use."""
    return int(lib().oracle_num_threads())
