"""Split-KV decode on the GPU against the fp64 CPU oracle (a single query row per stream)."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_attn_amd as am
import synth
from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, guarded_empty, guards_intact, host

pytestmark = pytest.mark.gpu


def inputs(seed, B, Hq, Hkv, L, d, peak=1.0):
    q, k, v = synth.attn_inputs(seed, B, Hq, Hkv, 1, L, d, bf16=True, qk_scale=peak)
    return q, k, v


def check(oracle_mod, q, k, v, num_splits=0, tol_o=TOL_O_BF16):
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d)
    o, lse = am.attn_decode_splitkv(dev(q, True), dev(k, True), dev(v, True), scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    eo, el = oracle_mod.fwd(q, k, v, scale, False)
    assert_close("O", host(o), eo, tol_o)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)
    return o, lse


# Qwen3-8B-shaped grouped-query decode: 32 query heads / 8 kv heads, d = 128
@pytest.mark.parametrize("streams", [1, 16, 48])
@pytest.mark.parametrize("L", [512, 1024, 2048, 4096])
def test_c3_grid(oracle_mod, streams, L):
    print(f"decode streams={streams} L={L} splits={am.decode_num_splits(streams, 32, 8, L, 128)}", flush=True)
    q, k, v = inputs(3000 + 100 * streams + int(math.log2(L // 512)), streams, 32, 8, L, 128)
    check(oracle_mod, q, k, v)


@pytest.mark.parametrize("num_splits", [1, 2, 3, 7, 0, 128])
def test_any_split_count_gives_the_same_result(oracle_mod, num_splits):
    q, k, v = inputs(3500, 2, 32, 8, 4096, 128)
    o, lse = check(oracle_mod, q, k, v, num_splits=num_splits)
    ref_o, ref_l = am.attn_decode_splitkv(dev(q, True), dev(k, True), dev(v, True), num_splits=1)
    torch.cuda.synchronize()
    # the monoid fold in any grouping: LSE agrees across split counts to fp32 rounding
    assert float((lse - ref_l).abs().max()) <= 1e-5


RAGGED = [
    # B, Hq, Hkv, L, d
    (1, 4, 1, 1, 128),
    (2, 8, 2, 31, 128),
    (1, 4, 4, 33, 64),
    (3, 16, 2, 1000, 64),
    (1, 32, 8, 4095, 128),
    (2, 16, 1, 777, 128),   # g = 16
    (1, 2, 2, 5000, 64),    # g = 1
]


@pytest.mark.parametrize("shape", RAGGED)
def test_ragged_shapes(oracle_mod, shape):
    B, Hq, Hkv, L, d = shape
    q, k, v = inputs(3600 + L, B, Hq, Hkv, L, d)
    check(oracle_mod, q, k, v)
    check(oracle_mod, q, k, v, num_splits=3)


# grids of more than 256 workgroups run the two-wave kernel (two workgroups per
# CU); ragged key counts and chunk ends, d = 64 and 128, g = 4 and 8
TWO_WAVE = [
    # B, Hq, Hkv, L, d, num_splits
    (40, 32, 8, 1000, 128, 0),     # 320 workgroups, one chunk each
    (48, 32, 8, 999, 64, 0),
    (12, 64, 8, 1500, 128, 3),     # 288 workgroups of three chunks per stream
]


@pytest.mark.parametrize("shape", TWO_WAVE)
def test_two_wave_grids(oracle_mod, shape):
    B, Hq, Hkv, L, d, S = shape
    plan = am.decode_num_splits(B, Hq, Hkv, L, d) if S == 0 else S
    assert B * Hkv * plan > 256
    print(f"two-wave decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} splits={plan}", flush=True)
    q, k, v = inputs(3700 + L + d, B, Hq, Hkv, L, d)
    check(oracle_mod, q, k, v, num_splits=S)


def test_peaked(oracle_mod):
    q, k, v = inputs(3700, 4, 32, 8, 2048, 128, peak=6.0)
    check(oracle_mod, q, k, v)


def test_empty_history():
    q = torch.ones(2, 8, 1, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(2, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = am.attn_decode_splitkv(q, kv, kv)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(lse == -math.inf)


def test_decode_equals_forward_last_row(oracle_mod):
    # one query at the end of a causal prefill sees every key: decode == fwd row
    B, Hq, Hkv, L, d = 2, 8, 2, 700, 128
    q, k, v = synth.attn_inputs(3800, B, Hq, Hkv, L, L, d, bf16=True)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    of, lf = am.attn_fwd(qd, kd, vd, causal=True)
    od, ld = am.attn_decode_splitkv(qd[:, :, -1:].contiguous(), kd, vd, num_splits=5)
    torch.cuda.synchronize()
    assert_close("O decode vs fwd", host(od)[:, :, 0], host(of)[:, :, -1], 2 * TOL_O_BF16)
    assert_close("LSE decode vs fwd", host(ld)[:, :, 0], host(lf)[:, :, -1], 2e-5)


def test_repeatable_bitwise():
    q, k, v = inputs(3900, 16, 32, 8, 2048, 128)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    o1, l1 = am.attn_decode_splitkv(qd, kd, vd)
    o2, l2 = am.attn_decode_splitkv(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_writes_outside_outputs():
    q, k, v = inputs(3901, 3, 32, 8, 1500, 128)
    o, ofull = guarded_empty(q.shape, torch.bfloat16)
    lse, lfull = guarded_empty(q.shape[:3], torch.float32)
    am.attn_decode_splitkv(dev(q, True), dev(k, True), dev(v, True), num_splits=4, out=o, lse=lse)
    torch.cuda.synchronize()
    assert guards_intact(ofull, o.numel()) and guards_intact(lfull, lse.numel())
