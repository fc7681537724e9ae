"""Split-KV decode in one launch: the last chunk of each (stream, kv head) to
finish folds every chunk's partial state, so no merge kernel runs.

The fold is the online-softmax monoid of "Não escreva kernels, derive-os"
(section "Aprofundamento"): any grouping of the chunks gives the same value up
to rounding, and the single-launch path folds them in index order whichever
finishes last, so it must give the two-launch path's bits.  "Tang Project
Derives GPU Kernels via IR ..." (section "Details") reports that the split
granularity changed the engine's accuracy at 48 streams; the split-count
sweep below checks that here it does not, beyond fp32 rounding.

GPU only (the CPU side of the entry point, argument checks and workspace
layout, is in test_abi_cpu.py).
"""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Hq, Hkv, L, d):
    return synth.attn_inputs(seed, B, Hq, Hkv, 1, L, d, bf16=True)


def _counts_zero(ws):
    return bool((ws[:65536] == 0).all())


@pytest.mark.parametrize("shape", [(1, 32, 8, 512, 128), (1, 32, 8, 4096, 128), (16, 32, 8, 4096, 128),
                                   (48, 32, 8, 2048, 128), (48, 32, 8, 4096, 128), (3, 16, 2, 1000, 64),
                                   (2, 16, 1, 777, 128), (1, 2, 2, 5000, 64)])
@pytest.mark.parametrize("splits", [0, 2, 3, 7, 128])
def test_fused_equals_two_launch(shape, splits):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    B, Hq, Hkv, L, d = shape
    print(f"fused decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d} splits={splits}", flush=True)
    q, k, v = _inputs(4000 + L + B, B, Hq, Hkv, L, d)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    if splits == 0:
        splits = am.decode_fused_num_splits(B, Hq, Hkv, L, d)  # the single-launch plan, for both
    o2, l2 = am.attn_decode_splitkv(qd, kd, vd, num_splits=splits)
    o1, l1 = am.attn_decode_splitkv_fused(qd, kd, vd, num_splits=splits)
    torch.cuda.synchronize()
    # the same partial states folded in the same order: identical bits
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("streams,L", [(1, 512), (1, 4096), (16, 1024), (48, 4096)])
def test_fused_matches_oracle(oracle_mod, streams, L):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    print(f"fused decode vs oracle streams={streams} L={L}", flush=True)
    q, k, v = _inputs(4100 + streams + L, streams, 32, 8, L, 128)
    o, lse = am.attn_decode_splitkv_fused(dev(q, True), dev(k, True), dev(v, True))
    torch.cuda.synchronize()
    eo, el = oracle_mod.fwd(q, k, v, 1.0 / math.sqrt(128), False)
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)


def test_fused_workspace_is_reused_across_calls():
    """One zeroed workspace serves calls of different sizes and split counts in
    a row; every call leaves its arrival counts at zero."""
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    big = (48, 32, 8, 4096, 128)
    plan = [(big, 0), ((4, 32, 8, 1500, 128), 7), (big, 3), ((1, 32, 8, 4096, 128), 0), (big, 0),
            ((2, 16, 1, 777, 128), 5), (big, 2)]
    need = max(am.decode_fused_workspace_bytes(*shape, s) for shape, s in plan)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, ((B, Hq, Hkv, L, d), splits) in enumerate(plan):
        print(f"reuse call {i}: B={B} L={L} splits={splits}", flush=True)
        splits = splits or am.decode_fused_num_splits(B, Hq, Hkv, L, d)
        q, k, v = _inputs(4200 + i, B, Hq, Hkv, L, d)
        qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
        o1, l1 = am.attn_decode_splitkv_fused(qd, kd, vd, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert _counts_zero(ws)
        o2, l2 = am.attn_decode_splitkv(qd, kd, vd, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fused_back_to_back_on_one_stream():
    """Calls queued without a host synchronisation between them: each starts
    after the previous one has returned its counts to zero (stream order)."""
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    B, Hq, Hkv, L, d, S = 16, 32, 8, 4096, 128, 4
    q, k, v = _inputs(4300, B, Hq, Hkv, L, d)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    ws = torch.zeros(am.decode_fused_workspace_bytes(B, Hq, Hkv, L, d, S), dtype=torch.uint8, device="cuda")
    ref_o, ref_l = am.attn_decode_splitkv(qd, kd, vd, num_splits=S)
    outs = [am.attn_decode_splitkv_fused(qd, kd, vd, num_splits=S, workspace=ws) for _ in range(8)]
    torch.cuda.synchronize()
    assert _counts_zero(ws)
    for o, lse in outs:
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


@pytest.mark.parametrize("streams", [1, 48])
def test_split_count_sweep_accuracy(oracle_mod, streams):
    """Error against the fp64 oracle at every split count from 1 to 64 keys
    chunks (and the automatic plan): all within the bf16 bar, LSE equal
    across split counts to fp32 rounding, and no trend with the count."""
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    L = 4096
    q, k, v = _inputs(4400 + streams, streams, 32, 8, L, 128)
    eo, el = oracle_mod.fwd(q, k, v, 1.0 / math.sqrt(128), False)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    errs, lses = {}, {}
    for s in [1, 2, 4, 8, 16, 32, 64, 0]:
        o, lse = am.attn_decode_splitkv_fused(qd, kd, vd, num_splits=s)
        torch.cuda.synchronize()
        oh, lh = host(o), host(lse)
        assert_close("O", oh, eo, TOL_O_BF16)
        assert_close("LSE", lh, el, TOL_LSE_BF16)
        errs[s] = (float(np.abs(oh - eo).max()), float(np.abs(lh - el).max()))
        lses[s] = lh
    print(f"streams={streams} (max |dO|, max |dLSE|) by split count: {errs}", flush=True)
    for s in lses:
        assert np.abs(lses[s] - lses[1]).max() <= 1e-5
    o_errs = [e[0] for e in errs.values()]
    assert max(o_errs) <= 1.5 * min(o_errs) + 1e-6
