"""Backward on the GPU against the analytic fp64 CPU oracle.  The GPU backward
takes the GPU forward's O and LSE (as a caller would); the oracle recomputes
everything from Q, K, V and dO alone."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_attn_amd as am
import synth
from gpu_helpers import TOL_GRAD, assert_close, dev, host

pytestmark = pytest.mark.gpu


def gpu_grads(q, k, v, do, causal, scale):
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


def run_case(oracle_mod, seed, B, Hq, Hkv, Nq, Nk, d, causal, peak=1.0, rel=None):
    print(f"bwd case seed={seed} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = synth.attn_inputs(seed, B, Hq, Hkv, Nq, Nk, d, bf16=True, with_dout=True, qk_scale=peak)
    gq, gk, gv = gpu_grads(q, k, v, do, causal, scale)
    eq, ek, ev = oracle_mod.bwd(q, k, v, do, scale, causal)
    errs = []
    for name, g, e in (("dQ", gq, eq), ("dK", gk, ek), ("dV", gv, ev)):
        tol = TOL_GRAD if rel is None else rel * float(np.abs(e).max())
        errs.append(assert_close(name, g, e, tol))
    print("  max-abs dQ {:.3e} dK {:.3e} dV {:.3e}".format(*errs), flush=True)


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 1, 1, 17, 17, 128),
    (2, 2, 2, 64, 64, 64),
    (1, 4, 2, 129, 129, 128),
    (1, 4, 1, 300, 300, 64),
    (1, 2, 2, 100, 260, 128),   # Nq < Nk
    (1, 2, 1, 260, 100, 128),   # Nq > Nk: rows with no visible key (causal)
    (2, 8, 2, 512, 512, 128),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_shapes(oracle_mod, shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    run_case(oracle_mod, 5000 + Nq + 3 * Nk + d, B, Hq, Hkv, Nq, Nk, d, causal)


def test_bwd_peaked(oracle_mod):
    # Q and K scaled by 2: gradients grow ~3x over the N(0,1) case, and the
    # bf16 operands (P, dS) bound the error relative to that magnitude.  At
    # N(0,1) the 5e-2 tolerance is ~2% of max|gradient|; the same 2% is held here.
    run_case(oracle_mod, 5100, 1, 2, 1, 200, 200, 128, True, peak=2.0, rel=0.02)


def test_bwd_zero_dout_gives_zero():
    q, k, v, _ = synth.attn_inputs(5200, 1, 4, 2, 100, 100, 128, bf16=True, with_dout=True)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=True)
    dq, dk, dv = am.attn_bwd(qd, kd, vd, o, torch.zeros_like(o), lse, causal=True)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.all(g == 0)


def test_bwd_repeatable_bitwise():
    q, k, v, do = synth.attn_inputs(5300, 1, 4, 2, 300, 300, 128, bf16=True, with_dout=True)
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=True)
    a = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    b = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- full size: B=4, H=16, N=2048, d=128, causal


@pytest.fixture(scope="module")
def c5_case(oracle_mod):
    """The full-size backward's inputs and the oracle's gradients of every
    (batch, head) problem, computed once for the tests that use them."""
    B, H, N, d = 4, 16, 2048, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = synth.attn_inputs(5, B, H, H, N, N, d, bf16=True, with_dout=True)
    print("C5 bwd: oracle over all 64 heads", flush=True)
    exp = oracle_mod.bwd(q, k, v, do, scale, True)
    return (q, k, v, do), exp, scale


def test_c5_full_size_all_heads(c5_case):
    # every one of the 64 (b, h) problems, element by element
    (q, k, v, do), (eq, ek, ev), scale = c5_case
    print("C5 bwd: launching", flush=True)
    gq, gk, gv = gpu_grads(q, k, v, do, True, scale)
    assert gq.shape == eq.shape and gk.shape == ek.shape and gv.shape == ev.shape
    errs = [assert_close(name, g, e, TOL_GRAD) for name, g, e in (("dQ", gq, eq), ("dK", gk, ek), ("dV", gv, ev))]
    print("  all heads: max-abs dQ {:.3e} dK {:.3e} dV {:.3e}".format(*errs), flush=True)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_xcd_local_order_all_heads(oracle_mod, causal):
    # B * Hkv = 16 (b, kv head) pairs split evenly over the 8 XCDs, so every
    # kernel takes its XCD-local work order; four query heads per kv head and
    # a ragged last tile; all 64 (b, h) problems compared in full
    run_case(oracle_mod, 5800 + int(causal), 2, 32, 8, 520, 520, 128, causal)


@pytest.mark.parametrize("grad_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 4, 2, 200, 333, 128), (2, 6, 3, 333, 200, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_guard_bands(oracle_mod, shape, causal, grad_dtype):
    # dq, dk and dv written into buffers with guard bands on both sides
    # (ragged grouped-query shapes, Nq != Nk): no store lands outside a
    # gradient, and the values inside still match the oracle
    from gpu_helpers import guarded_empty, guards_intact

    B, Hq, Hkv, Nq, Nk, d = shape
    print(f"bwd guard bands {shape} causal={causal} {grad_dtype}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = synth.attn_inputs(5900 + Nq + Nk + d, B, Hq, Hkv, Nq, Nk, d, bf16=True, with_dout=True)
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, fq = guarded_empty(q.shape, grad_dtype)
    dk, fk = guarded_empty(k.shape, grad_dtype)
    dv, fv = guarded_empty(v.shape, grad_dtype)
    am.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    for full, t in ((fq, dq), (fk, dk), (fv, dv)):
        assert guards_intact(full, t.numel())
    eq, ek, ev = oracle_mod.bwd(q, k, v, do, scale, causal)
    for name, g, e in (("dQ", dq, eq), ("dK", dk, ek), ("dV", dv, ev)):
        assert_close(name, host(g), e, TOL_GRAD)


# ---------------------------------------------------------------- bf16 gradients (attn_bwd_bf16_grads)


@pytest.mark.parametrize("shape", [(1, 1, 1, 17, 17, 128), (1, 4, 2, 129, 129, 128), (1, 4, 1, 300, 300, 64),
                                   (1, 2, 1, 260, 100, 128), (2, 8, 2, 512, 512, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_grads_are_the_fp32_grads_rounded(shape, causal):
    # the same kernels with bf16 final stores: every element equals the fp32
    # path's value rounded to nearest even
    B, Hq, Hkv, Nq, Nk, d = shape
    print(f"bf16 grads case {shape} causal={causal}", flush=True)
    q, k, v, do = synth.attn_inputs(5600 + Nq + Nk + d, B, Hq, Hkv, Nq, Nk, d, bf16=True, with_dout=True)
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=causal)
    g32 = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal)
    g16 = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), g32, g16):
        assert b.dtype == torch.bfloat16
        assert torch.equal(a.to(torch.bfloat16).view(torch.int16), b.view(torch.int16)), name


def test_bf16_grads_c5_tolerance_study(c5_case):
    # B=4 H=16 N=2048 d=128 causal, every head against the fp64 oracle:
    # rounding the output adds at most half a bf16 ulp, 2^-9 |g|, to the fp32
    # path's error; the bar stays the gradient tolerance
    (q, k, v, do), exp, scale = c5_case
    print("C5 bwd, bf16 gradients: launching", flush=True)
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=True, scale=scale)
    g16 = [host(g) for g in am.attn_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=scale, grad_dtype=torch.bfloat16)]
    g32 = [host(g) for g in am.attn_bwd(qd, kd, vd, o, dod, lse, causal=True, scale=scale)]
    torch.cuda.synchronize()
    for name, a16, a32, e in zip(("dQ", "dK", "dV"), g16, g32, exp):
        gmax = float(np.abs(e).max())
        e32 = assert_close(name + " fp32", a32, e, TOL_GRAD)
        e16 = assert_close(name + " bf16", a16, e, TOL_GRAD)
        # the rounding adds no more than half an ulp at the largest magnitude
        assert e16 <= e32 + 2.0 ** -9 * gmax * 1.0001
        print(f"  {name}: max|g| {gmax:.3f}  err fp32 {e32:.3e}  err bf16 {e16:.3e}", flush=True)


@pytest.mark.parametrize("causal,d", [(True, 128), (False, 128), (True, 64)])
def test_eight_wave_dq_ragged_gqa(oracle_mod, causal, d):
    # 2 x 32 query heads over 8 kv heads at 2100 rows: 576 query tiles of 256
    # rows, so dQ runs as eight-wave workgroups (the two-group kernel), with a
    # ragged last tile and four query heads accumulated into each kv head's
    # dK and dV; every head compared in full
    B, Hq, Hkv, N = 2, 32, 8, 2100
    assert B * Hq * ((N + 255) // 256) >= 512
    run_case(oracle_mod, 5700 + d + int(causal), B, Hq, Hkv, N, N, d, causal)
