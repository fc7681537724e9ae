"""Pins of the CPU oracle against facts fixed by mathematics, not by the oracle itself.

Every test here runs on the CPU.  A plausible slip in the oracle (a dropped
scale, a wrong sign, a transposed operand, a wrong head map or causal offset,
a missing max shift, a wrong gradient term) fails at least one of them:

  brute force      50-digit mpmath evaluation of the definition, no max shift
  finite diffs     gradients of sum(dO*O) by 50-digit central differences
  closed forms     Q = 0 (mean of visible values), V = 1, Nk = 1, causal row 0
  invariants       rows of P sum to 1; shift of keys; permutations; linearity
  reductions       grouped-query heads = repeated kv heads; decode = Nq = 1 row
  monoid           any partition / merge tree of the keys gives the same result
"""
import math

import numpy as np
import pytest

import synth
from oracle import brute, monoid


def rel_close(a, b, rtol, atol=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


TINY = [
    # B, Hq, Hkv, Nq, Nk, d, causal
    (1, 1, 1, 4, 4, 3, False),
    (1, 1, 1, 5, 5, 2, True),
    (2, 2, 1, 3, 5, 3, True),    # GQA g=2, Nq < Nk: bottom-right causal
    (1, 2, 2, 6, 4, 2, True),    # Nq > Nk: the first rows see no key
    (1, 4, 2, 3, 6, 4, False),
    (1, 1, 1, 1, 6, 3, True),    # decode-shaped row: sees every key
]


@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("peak", [1.0, 6.0])
def test_fwd_matches_brute_force(oracle_mod, shape, peak):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v = synth.attn_inputs(11 + Nq * 7 + Nk, B, Hq, Hkv, Nq, Nk, d, bf16=False, scale=peak)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle_mod.fwd(q, k, v, scale, causal)
    ob, lseb = brute.brute_fwd(q, k, v, scale, causal)
    rel_close(o, ob, rtol=1e-12, atol=1e-13)
    fin = np.isfinite(lseb)
    assert np.array_equal(fin, np.isfinite(lse))
    rel_close(lse[fin], lseb[fin], rtol=1e-12, atol=1e-13)
    assert np.all(lse[~fin] == -np.inf)


def test_empty_rows_are_zero_and_minus_inf(oracle_mod):
    # causal with Nq > Nk: row i sees keys j <= i - (Nq - Nk); rows i < Nq - Nk see none
    q, k, v = synth.attn_inputs(5, 1, 1, 1, 7, 3, 4, bf16=False)
    o, lse = oracle_mod.fwd(q, k, v, 0.5, True)
    assert np.all(o[0, 0, :4] == 0.0) and np.all(lse[0, 0, :4] == -np.inf)
    assert np.all(np.isfinite(lse[0, 0, 4:]))
    do = synth.normal(6, [(1, 1, 7, 4)], bf16=False)[0]
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, 0.5, True)
    assert np.all(dq[0, 0, :4] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(oracle_mod, causal):
    # with V = identity (d = Nk) each output row is the probability row P_i
    Nq = Nk = 9
    q, k = synth.normal(21, [(1, 2, Nq, 5), (1, 2, Nk, 5)], bf16=False)
    kd = np.zeros((1, 2, Nk, Nk), np.float32)
    kd[..., :5] = k
    qd = np.zeros((1, 2, Nq, Nk), np.float32)
    qd[..., :5] = q
    v = np.broadcast_to(np.eye(Nk, dtype=np.float32), (1, 2, Nk, Nk)).copy()
    p, _ = oracle_mod.fwd(qd, kd, v, 0.7, causal)
    rel_close(p.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert np.all(p >= 0)
    if causal:
        assert np.all(np.triu(p[0, 0], 1) == 0.0)
        assert np.all(p[0, 0][np.tril_indices(Nq)] > 0.0)


@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_visible_values(oracle_mod, causal):
    B, H, Nq, Nk, d = 2, 3, 11, 11, 8
    _, k, v = synth.attn_inputs(31, B, H, H, Nq, Nk, d, bf16=True)
    q = np.zeros((B, H, Nq, d), np.float32)
    o, lse = oracle_mod.fwd(q, k, v, 0.125, causal)
    v64 = v.astype(np.float64)
    if causal:
        cnt = np.arange(1, Nk + 1, dtype=np.float64)
        expect = np.cumsum(v64, axis=2) / cnt[None, None, :, None]
        rel_close(lse, np.broadcast_to(np.log(cnt), lse.shape), rtol=1e-15, atol=1e-15)
    else:
        expect = np.broadcast_to(v64.mean(axis=2, keepdims=True), o.shape)
        rel_close(lse, math.log(Nk), rtol=1e-15, atol=1e-15)
    rel_close(o, expect, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_v_one_gives_one(oracle_mod, causal):
    q, k, _ = synth.attn_inputs(41, 1, 2, 1, 13, 17, 6, bf16=False, scale=3.0)
    v = np.ones((1, 1, 17, 6), np.float32)
    o, _ = oracle_mod.fwd(q, k, v, 0.4, causal)
    rel_close(o, 1.0, rtol=0, atol=1e-14)


def test_causal_row_zero_is_first_value(oracle_mod):
    q, k, v = synth.attn_inputs(51, 1, 2, 2, 8, 8, 4, bf16=True)
    scale = 0.5
    o, lse = oracle_mod.fwd(q, k, v, scale, True)
    assert np.array_equal(o[:, :, 0, :], v[:, :, 0, :].astype(np.float64))
    s00 = scale * np.einsum("bhd,bhd->bh", q[:, :, 0].astype(np.float64), k[:, :, 0].astype(np.float64))
    rel_close(lse[:, :, 0], s00, rtol=1e-15, atol=1e-15)


def test_single_key(oracle_mod):
    q, k, v = synth.attn_inputs(61, 2, 2, 1, 5, 1, 4, bf16=False)
    o, lse = oracle_mod.fwd(q, k, v, 0.3, False)
    rel_close(o, np.broadcast_to(v.astype(np.float64), o.shape), rtol=1e-15, atol=0)
    s = 0.3 * np.einsum("bhid,bd->bhi", q.astype(np.float64), k[:, 0, 0].astype(np.float64))
    rel_close(lse, s, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance_exercises_max_subtraction(oracle_mod, causal):
    # adding u to every key row adds scale*q_i.u to every score of row i:
    # O is unchanged and LSE moves by scale*q_i.u.  |u| is large enough that the
    # scores are ~1e3, where exp() without the max shift would overflow.
    B, H, Nq, Nk, d = 1, 2, 7, 7, 4
    q, k, v = synth.attn_inputs(71, B, H, H, Nq, Nk, d, bf16=False)
    k = (np.round(k * 1024.0) / 1024.0).astype(np.float32)  # so that k + u is exact in fp32
    u = np.array([400.0, -300.0, 250.0, 500.0], np.float32)
    k2 = (k + u).astype(np.float32)
    u_eff = k2.astype(np.float64) - k.astype(np.float64)
    assert np.all(u_eff == u.astype(np.float64))
    o1, l1 = oracle_mod.fwd(q, k, v, 1.0, causal)
    o2, l2 = oracle_mod.fwd(q, k2, v, 1.0, causal)
    shift = np.einsum("bhid,bhd->bhi", q.astype(np.float64), u_eff[:, :, 0, :])
    assert np.max(np.abs(shift)) > 300
    rel_close(o2, o1, rtol=1e-9, atol=1e-9)
    rel_close(l2, l1 + shift, rtol=1e-12, atol=1e-9)


def test_permutations(oracle_mod):
    B, H, Nq, Nk, d = 1, 2, 6, 9, 5
    q, k, v = synth.attn_inputs(81, B, H, H, Nq, Nk, d, bf16=False)
    o, lse = oracle_mod.fwd(q, k, v, 0.45, False)
    pk = np.random.default_rng(0).permutation(Nk)
    o2, lse2 = oracle_mod.fwd(q, k[:, :, pk], v[:, :, pk], 0.45, False)
    rel_close(o2, o, rtol=1e-13, atol=1e-14)
    rel_close(lse2, lse, rtol=1e-14, atol=0)
    pq = np.random.default_rng(1).permutation(Nq)
    o3, lse3 = oracle_mod.fwd(q[:, :, pq], k, v, 0.45, False)
    rel_close(o3, o[:, :, pq], rtol=1e-15, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_kv_heads(oracle_mod, causal):
    B, Hq, Hkv, Nq, Nk, d = 2, 6, 2, 5, 8, 4
    q, k, v = synth.attn_inputs(91, B, Hq, Hkv, Nq, Nk, d, bf16=True)
    o, lse = oracle_mod.fwd(q, k, v, 0.5, causal)
    g = Hq // Hkv
    kr = np.repeat(k, g, axis=1)  # heads 0..g-1 use kv head 0, and so on
    vr = np.repeat(v, g, axis=1)
    o2, lse2 = oracle_mod.fwd(q, kr, vr, 0.5, causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # a different head map would be caught: kv head 1 differs from kv head 0
    o_wrong, _ = oracle_mod.fwd(q, np.tile(k, (1, g, 1, 1)), np.tile(v, (1, g, 1, 1)), 0.5, causal)
    assert not np.allclose(o_wrong, o)


def test_linear_in_v(oracle_mod):
    q, k, v1 = synth.attn_inputs(101, 1, 2, 2, 6, 6, 4, bf16=False)
    v2 = synth.normal(102, [v1.shape], bf16=False)[0]
    a, b = 0.75, -2.5
    o1, _ = oracle_mod.fwd(q, k, v1, 0.5, True)
    o2, _ = oracle_mod.fwd(q, k, v2, 0.5, True)
    o3, _ = oracle_mod.fwd(q, k, (a * v1.astype(np.float64) + b * v2).astype(np.float32), 0.5, True)
    v3 = (a * v1.astype(np.float64) + b * v2).astype(np.float32).astype(np.float64)
    # the combined V was rounded to fp32; compare against O of the rounded values
    o3b, _ = oracle_mod.fwd(q, k, v3.astype(np.float32), 0.5, True)
    rel_close(o3, o3b, rtol=0, atol=0)
    rel_close(o3, a * o1 + b * o2, rtol=1e-6, atol=1e-6)


def test_peaked_row_selects_one_value(oracle_mod):
    # make key 3 align with query 0 so its score exceeds every other by > 60
    Nk, d = 8, 4
    q, k, v = synth.attn_inputs(111, 1, 1, 1, 1, Nk, d, bf16=False)
    k = k.copy()
    k[0, 0, 3] = q[0, 0, 0] * 200.0
    s = q[0, 0, 0].astype(np.float64) @ k[0, 0].astype(np.float64).T
    assert np.sort(s)[-1] - np.sort(s)[-2] > 60
    o, _ = oracle_mod.fwd(q, k, v, 1.0, False)
    rel_close(o[0, 0, 0], v[0, 0, 3], rtol=1e-20, atol=1e-20)


def test_decode_row_equals_last_row_of_prefill(oracle_mod):
    # with bottom-right alignment, a single query against Nk keys sees all of
    # them, and equals the last row of an Nk x Nk causal prefill
    Nk, d = 10, 4
    q, k, v = synth.attn_inputs(121, 1, 2, 1, Nk, Nk, d, bf16=True)
    o, lse = oracle_mod.fwd(q, k, v, 0.5, True)
    od, lsed = oracle_mod.fwd(q[:, :, -1:], k, v, 0.5, True)
    on, lsen = oracle_mod.fwd(q[:, :, -1:], k, v, 0.5, False)
    assert np.array_equal(od, on) and np.array_equal(lsed, lsen)
    rel_close(od[:, :, 0], o[:, :, -1], rtol=1e-15, atol=0)
    rel_close(lsed[:, :, 0], lse[:, :, -1], rtol=1e-15, atol=0)


def test_fwd_rows_equals_full(oracle_mod):
    q, k, v = synth.attn_inputs(131, 2, 4, 2, 9, 12, 8, bf16=True)
    o, lse = oracle_mod.fwd(q, k, v, 0.35, True)
    rows = synth.sample_rows(7, 10, 2, 4, 9, forced_i=(0, 8))
    orow, lrow = oracle_mod.fwd_rows(q, k, v, rows, 0.35, True)
    for t, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[t], o[b, h, i])
        assert lrow[t] == lse[b, h, i]


# ---------------------------------------------------------------- monoid


def _scores(q_row, kh, scale):
    return scale * (kh.astype(np.float64) @ q_row.astype(np.float64))


@pytest.mark.parametrize("seed", range(6))
def test_monoid_any_grouping_equals_three_pass(oracle_mod, seed):
    rng = np.random.default_rng(1000 + seed)
    Nk, d = int(rng.integers(1, 40)), 6
    q, k, v = synth.attn_inputs(140 + seed, 1, 1, 1, 1, Nk, d, bf16=False, scale=float(rng.uniform(0.5, 4)))
    scale = 0.6
    s = _scores(q[0, 0, 0], k[0, 0], scale)
    leaves = [monoid.leaf(s[j], v[0, 0, j]) for j in range(Nk)]
    # random partition into contiguous-or-not chunks, each folded left to right
    perm = rng.permutation(Nk)
    cuts = np.sort(rng.choice(np.arange(1, Nk), size=min(Nk - 1, int(rng.integers(0, 6))), replace=False)) if Nk > 1 else []
    chunks = np.split(perm, cuts)
    parts = [monoid.fold([leaves[j] for j in c], d) for c in chunks]
    parts += [monoid.identity(d) for _ in range(int(rng.integers(0, 3)))]  # identities anywhere
    rng.shuffle(parts)
    # random merge tree
    while len(parts) > 1:
        i = int(rng.integers(len(parts) - 1))
        parts[i:i + 2] = [monoid.combine(parts[i], parts[i + 1])]
    o_m, lse_m = monoid.finalize(parts[0])
    o, lse = oracle_mod.fwd(q, k, v, scale, False)
    rel_close(o_m, o[0, 0, 0], rtol=1e-12, atol=1e-13)
    rel_close(lse_m, lse[0, 0, 0], rtol=1e-13, atol=1e-13)


def test_monoid_identity_and_empty():
    d = 3
    e = monoid.identity(d)
    x = monoid.leaf(2.0, [1.0, 2.0, 3.0])
    for a, b in ((e, x), (x, e)):
        m, l, acc = monoid.combine(a, b)
        assert m == 2.0 and l == 1.0 and np.array_equal(acc, [1.0, 2.0, 3.0])
    o, lse = monoid.finalize(monoid.combine(e, e))
    assert np.all(o == 0) and lse == -math.inf


# ---------------------------------------------------------------- backward


BWD_TINY = [
    (1, 1, 1, 4, 4, 3, False),
    (1, 1, 1, 4, 4, 3, True),
    (1, 2, 1, 3, 5, 2, True),    # GQA g = 2, Nq < Nk
    (1, 2, 2, 5, 3, 2, True),    # Nq > Nk: empty rows
]


@pytest.mark.parametrize("shape", BWD_TINY)
def test_bwd_matches_finite_differences(oracle_mod, shape):
    B, Hq, Hkv, Nq, Nk, d, causal = shape
    q, k, v, do = synth.attn_inputs(150 + Nq + 10 * Nk, B, Hq, Hkv, Nq, Nk, d, bf16=False, with_dout=True)
    scale = 0.8
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, scale, causal)
    fq, fk, fv = brute.fd_grads(q, k, v, do, scale, causal)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        rel_close(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_invariants(oracle_mod, causal):
    B, Hq, Hkv, N, d = 2, 4, 2, 12, 8
    q, k, v, do = synth.attn_inputs(170, B, Hq, Hkv, N, N, d, bf16=True, with_dout=True)
    scale = 1 / math.sqrt(d)
    o, _ = oracle_mod.fwd(q, k, v, scale, causal)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, scale, causal)
    D = oracle_mod.rowdot(q, k, v, do, scale, causal)
    rel_close(D, np.sum(do.astype(np.float64) * o, -1), rtol=1e-12, atol=1e-12)
    g = Hq // Hkv
    # each row of P sums to 1, so sum_j dV_j = sum over the group's rows of dO_i
    sdo = do.astype(np.float64).reshape(B, Hkv, g, N, d).sum(axis=(2, 3))
    rel_close(dv.sum(axis=2), sdo, rtol=1e-12, atol=1e-12)
    # sum_j dS_ij = D_i - D_i = 0, so sum_j dK_j = 0
    rel_close(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)


def test_bwd_closed_forms(oracle_mod):
    B, H, N, d = 1, 2, 7, 4
    q, k, v, do = synth.attn_inputs(180, B, H, H, N, N, d, bf16=False, with_dout=True)
    # dO = 0: every gradient is 0
    z = np.zeros_like(do)
    for g in oracle_mod.bwd(q, k, v, z, 0.5, True):
        assert np.all(g == 0)
    # V = 0: dP = 0 so dQ = dK = 0, and dV = P^T dO
    dq, dk, dv = oracle_mod.bwd(q, k, np.zeros_like(v), do, 0.5, False)
    assert np.all(dq == 0) and np.all(dk == 0)
    eye = np.broadcast_to(np.eye(N, dtype=np.float32), (B, H, N, N)).copy()
    qp = np.zeros((B, H, N, N), np.float32)
    qp[..., :d] = q
    kp = np.zeros((B, H, N, N), np.float32)
    kp[..., :d] = k
    P, _ = oracle_mod.fwd(qp, kp, eye, 0.5, False)
    rel_close(dv, np.einsum("bhij,bhic->bhjc", P, do.astype(np.float64)), rtol=1e-12, atol=1e-13)
    # Q = 0, non-causal: P = 1/N, so dK = 0 and dV_j = mean over i of dO_i
    dq, dk, dv = oracle_mod.bwd(np.zeros_like(q), k, v, do, 0.5, False)
    rel_close(dk, 0.0, rtol=0, atol=1e-14)
    rel_close(dv, np.broadcast_to(do.astype(np.float64).mean(axis=2, keepdims=True), dv.shape), rtol=1e-13,
              atol=1e-14)
    # causal: the last key is seen only by the last row, dV_{N-1} = P_{N-1,N-1} dO_{N-1}
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, 0.5, True)
    o, lse = oracle_mod.fwd(q, k, v, 0.5, True)
    s_last = 0.5 * np.sum(q[:, :, -1].astype(np.float64) * k[:, :, -1].astype(np.float64), -1)
    p_last = np.exp(s_last - lse[:, :, -1])
    rel_close(dv[:, :, -1], p_last[..., None] * do[:, :, -1].astype(np.float64), rtol=1e-12, atol=1e-14)
    # causal row 0 sees only key 0 (P_00 = 1, dS_00 = 0): dQ_0 = 0
    rel_close(dq[:, :, 0], 0.0, rtol=0, atol=1e-15)
