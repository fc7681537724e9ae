"""The allocation-free decode (attn_decode_splitkv_noalloc): its partial
states live in the library's fixed device scratch.  Two calls in a row, the
second smaller, each compared bit for bit with attn_decode_splitkv at the same
split plan (the same kernels) and with the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_attn_amd as am
import synth
from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _case(oracle_mod, seed, B, Hq, Hkv, Nk, d, splits):
    print(f"noalloc decode seed={seed} B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} d={d} splits={splits}", flush=True)
    scale = 1.0 / math.sqrt(d)
    q, k, v = synth.attn_inputs(seed, B, Hq, Hkv, 1, Nk, d, bf16=True)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    assert am.decode_noalloc_scratch_bytes(B, Hq, Hkv, Nk, d, splits) > 0  # the plan splits: the scratch is used
    o1 = torch.empty_like(qd)
    l1 = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    am.attn_decode_splitkv_noalloc(qd, kd, vd, o1, l1, scale=scale, num_splits=splits)
    o2, l2 = am.attn_decode_splitkv(qd, kd, vd, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    eo, el = oracle_mod.fwd(q, k, v, scale, False)
    assert_close("O", host(o1), eo, TOL_O_BF16)
    assert_close("LSE", host(l1), el, TOL_LSE_BF16)


def test_noalloc_decode_two_calls_second_smaller(oracle_mod):
    _case(oracle_mod, 7100, 3, 32, 8, 3000, 128, 5)
    # the automatic plan splits one stream of 2000 keys (8 chunks)
    _case(oracle_mod, 7101, 1, 16, 4, 2000, 64, 0)


def test_noalloc_decode_rejects_plans_beyond_the_scratch():
    # 16 streams x 32 heads x 64 chunks of partial states need ~17 MB, more
    # than the 8 MiB scratch: refused on the host before any launch
    B, Hq, Hkv, Nk, d = 16, 32, 8, 4096, 128
    assert am.decode_noalloc_scratch_bytes(B, Hq, Hkv, Nk, d, 64) > am.DECODE_SCRATCH_BYTES
    q = torch.zeros(B, Hq, 1, d, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Hkv, Nk, d, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(am.AttnError) as e:
        am.attn_decode_splitkv_noalloc(q, k, k, torch.empty_like(q), num_splits=64)
    assert e.value.status == am.ATTN_ERR_SCRATCH
