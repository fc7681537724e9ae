"""Every entry point on shapes drawn from a seeded generator (ragged sizes,
grouped-query ratios 1-8, d = 64 and 128, causal and not, empty and one-key
cases, explicit and automatic split counts) against the fp64 oracle at the
same tolerances as the fixed cases; the dense forward also on grids large
enough for the two-group kernel, checked on sampled rows.  Each case draws
its own shape from random.Random(seed of the case), so a failure names a
case that reruns alone."""
import math
import random

import numpy as np
import pytest
import torch

import attention_online_softmax_attn_amd as am
import oracle
import synth
from gpu_helpers import TOL_GRAD, TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu

N_CASES = 8


def _heads(r):
    hkv = r.choice([1, 2, 4, 8])
    return hkv * r.choice([1, 2, 4, 8]), hkv


def _check_o_lse(o, lse, eo, el):
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_forward(oracle_mod, case):
    r = random.Random(10_000 + case)
    B = r.choice([1, 2, 3])
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    causal = r.random() < 0.6
    Nq = r.choice([1, 2, 31, 64, 65, 127, 255, 256, 257, 500, 777, 1100])
    Nk = r.choice([Nq, Nq, r.randint(1, 1500)])
    while B * Hq * Nq * Nk * d > 3e8:
        Nq, Nk = max(1, Nq // 2), max(1, Nk // 2)
    print(f"fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
    q, k, v = synth.attn_inputs(10_000 + case, B, Hq, Hkv, Nq, Nk, d, bf16=True)
    o, lse = am.attn_fwd(dev(q, True), dev(k, True), dev(v, True), causal=causal)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, *oracle_mod.fwd(q, k, v, 1 / math.sqrt(d), causal))


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_forward_two_group_grids(oracle_mod, case):
    r = random.Random(11_000 + case)
    B = r.choice([1, 2])
    Hkv = r.choice([4, 8])
    Hq = Hkv * r.choice([2, 4])
    d = r.choice([64, 128])
    causal = r.random() < 0.6
    Nq = r.randint(2000, 9000)
    Nk = r.choice([Nq, r.randint(1000, 9000)])
    print(f"fwd two-group B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
    q, k, v = synth.attn_inputs(11_000 + case, B, Hq, Hkv, Nq, Nk, d, bf16=True)
    o, lse = am.attn_fwd(dev(q, True), dev(k, True), dev(v, True), causal=causal)
    torch.cuda.synchronize()
    rows = synth.sample_rows(11_000 + case, 300, B, Hq, Nq, forced_i=(0, Nq - 1, 255, 256))
    eo, el = oracle_mod.fwd_rows(q, k, v, rows, 1 / math.sqrt(d), causal)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    assert_close("O", host(o)[b, h, i], eo, TOL_O_BF16)
    assert_close("LSE", host(lse)[b, h, i], el, TOL_LSE_BF16)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_entry_points(oracle_mod, case):
    r = random.Random(12_000 + case)
    B = r.choice([1, 2, 5, 16, 33])
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    L = r.choice([1, 7, 64, 65, 500, 1000, 2049, 4096, 5000])
    while B * Hq * L * d > 2e8:
        L = max(1, L // 2)
    splits = r.choice([0, 0, 1, 2, 3, 5, 16])
    print(f"decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} splits={splits}", flush=True)
    q, k, v = synth.attn_inputs(12_000 + case, B, Hq, Hkv, 1, L, d, bf16=True)
    eo, el = oracle_mod.fwd(q, k, v, 1 / math.sqrt(d), False)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    o, lse = am.attn_decode_splitkv(qd, kd, vd, num_splits=splits)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, eo, el)
    o2, l2 = am.attn_decode_splitkv_fused(qd, kd, vd, num_splits=splits)
    torch.cuda.synchronize()
    _check_o_lse(o2, l2, eo, el)
    if splits > 0:  # the same chunks: the same kernels and fold, the same bits
        assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    if am.decode_noalloc_scratch_bytes(B, Hq, Hkv, L, d, splits) <= am.DECODE_SCRATCH_BYTES:
        o3, l3 = torch.empty_like(o), torch.empty_like(lse)
        am.attn_decode_splitkv_noalloc(qd, kd, vd, o3, l3, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o3.view(torch.int16), o.view(torch.int16))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_backward(oracle_mod, case):
    r = random.Random(13_000 + case)
    B = r.choice([1, 2])
    Hkv = r.choice([1, 2, 4])
    Hq = Hkv * r.choice([1, 2, 4])
    d = r.choice([64, 128])
    causal = r.random() < 0.6
    Nq = r.choice([1, 17, 63, 64, 65, 129, 300, 513, 700])
    Nk = r.choice([Nq, r.randint(1, 900)])
    g16 = r.random() < 0.3
    print(f"bwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} causal={causal} bf16 grads={g16}", flush=True)
    q, k, v, do = synth.attn_inputs(13_000 + case, B, Hq, Hkv, Nq, Nk, d, bf16=True, with_dout=True)
    qd, kd, vd, dod = dev(q, True), dev(k, True), dev(v, True), dev(do, True)
    o, lse = am.attn_fwd(qd, kd, vd, causal=causal)
    grads = am.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, grad_dtype=torch.bfloat16 if g16 else None)
    torch.cuda.synchronize()
    expect = oracle_mod.bwd(q, k, v, do, 1 / math.sqrt(d), causal)
    for name, g, e in zip(("dQ", "dK", "dV"), grads, expect):
        assert_close(name, host(g), e, TOL_GRAD)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_packed_batch(oracle_mod, case):
    r = random.Random(14_000 + case)
    n = r.randint(1, 12)
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    causal = r.random() < 0.7
    lq = [r.choice([0, 1, 5, 63, 64, 65, 200, 256, 257, 600]) for _ in range(n)]
    lk = [max(0, a + r.choice([0, 0, 100, 700, -3])) for a in lq]
    print(f"varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} causal={causal}", flush=True)
    q, k, v, cu_q, cu_k = synth.varlen_inputs(14_000 + case, lq, lk, Hq, Hkv, d, bf16=True)
    o, lse = am.attn_fwd_varlen(dev(q, True), dev(k, True), dev(v, True), torch.from_numpy(cu_q).cuda(),
                                torch.from_numpy(cu_k).cuda(), max(lq), causal=causal)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, *oracle.fwd_varlen(q, k, v, cu_q, cu_k, 1 / math.sqrt(d), causal))


def _poisoned(kc, vc, used):
    kd, vd = dev(kc, True), dev(vc, True)
    mask = torch.from_numpy(~used).cuda()[:, None, :, None].expand(kd.shape)
    return kd.masked_fill(mask, float("nan")).contiguous(), vd.masked_fill(mask, float("nan")).contiguous()


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_paged_decode(oracle_mod, case):
    r = random.Random(15_000 + case)
    n = r.randint(1, 10)
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    page = r.choice([64, 128, 256])
    lens = [r.choice([0, 1, 63, 64, 65, 300, 1000, 2500]) for _ in range(n)]
    splits = r.choice([0, 1, 3])
    print(f"paged decode lens={lens} Hq={Hq} Hkv={Hkv} page={page} d={d} splits={splits}", flush=True)
    q, kc, vc, table, lens_a, used = synth.paged_kv_inputs(15_000 + case, lens, Hq, Hkv, page, d)
    kd, vd = _poisoned(kc, vc, used)
    o, lse = am.attn_decode_paged(dev(q, True), kd, vd, torch.from_numpy(table).cuda(), torch.from_numpy(lens_a).cuda(),
                                  int(lens_a.max()), num_splits=splits)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, *oracle.decode_paged(q, kc, vc, table, lens_a, 1 / math.sqrt(d)))


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_random_paged_packed_batch(oracle_mod, case):
    r = random.Random(16_000 + case)
    n = r.randint(1, 8)
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    page = r.choice([64, 128])
    causal = r.random() < 0.7
    lq = [r.choice([0, 1, 63, 64, 65, 300]) for _ in range(n)]
    lk = [a + r.choice([0, 64, 500]) for a in lq]
    print(f"paged varlen lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} page={page} d={d} causal={causal}", flush=True)
    q, kc, vc, table, cu_q, lens_k, used = synth.paged_varlen_inputs(16_000 + case, lq, lk, Hq, Hkv, page, d)
    kd, vd = _poisoned(kc, vc, used)
    o, lse = am.attn_fwd_varlen_paged(dev(q, True), kd, vd, torch.from_numpy(table).cuda(), torch.from_numpy(cu_q).cuda(),
                                      torch.from_numpy(lens_k).cuda(), max(lq), int(max(lk)), causal=causal)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, *oracle.fwd_varlen_paged(q, kc, vc, table, cu_q, lens_k, 1 / math.sqrt(d), causal))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_fp8_decode(oracle_mod, case):
    r = random.Random(17_000 + case)
    B = r.choice([1, 3, 16])
    Hq, Hkv = _heads(r)
    d = r.choice([64, 128])
    L = r.choice([1, 31, 64, 500, 1000, 4096])
    while B * Hq * L * d > 2e8:
        L = max(1, L // 2)
    splits = r.choice([0, 1, 2, 7])
    print(f"fp8 decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} splits={splits}", flush=True)
    q, k8, v8, ks, vs = synth.fp8_kv_inputs(17_000 + case, B, Hq, Hkv, L, d)
    o, lse = am.attn_decode_splitkv_fp8(dev(q, True), torch.from_numpy(k8).cuda(), torch.from_numpy(v8).cuda(),
                                        torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda(), num_splits=splits)
    torch.cuda.synchronize()
    _check_o_lse(o, lse, *oracle.decode_fp8(q, k8, v8, ks, vs, 1 / math.sqrt(d)))
