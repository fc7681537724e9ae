"""Calls on several streams at once.

The library keeps no state between calls (workspaces belong to the caller),
so a forward, a decode and a backward issued on two side streams and running
concurrently give the same bits as the same calls issued one after another on
the default stream.  Streams keep the default priority.
"""
import pytest
import torch

import synth
from gpu_helpers import dev

pytestmark = pytest.mark.gpu


def test_concurrent_streams_match_serial_bits():
    import attention_online_softmax_attn_amd as am

    q, k, v = synth.attn_inputs(810, 2, 16, 4, 700, 900, 128, bf16=True)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    dq, dk, dv = synth.attn_inputs(811, 8, 32, 8, 1, 3000, 128, bf16=True)
    dqd, dkd, dvd = dev(dq, True), dev(dk, True), dev(dv, True)
    bq, bk, bv = synth.attn_inputs(812, 2, 8, 8, 500, 500, 64, bf16=True)
    bqd, bkd, bvd = dev(bq, True), dev(bk, True), dev(bv, True)
    bdo = dev(synth.attn_inputs(813, 2, 8, 8, 500, 500, 64, bf16=True)[0], True)
    bo, blse = am.attn_fwd(bqd, bkd, bvd, causal=True)

    def run():
        o, lse = am.attn_fwd(qd, kd, vd, causal=True)
        od, ld = am.attn_decode_splitkv(dqd, dkd, dvd, num_splits=3)
        g = am.attn_bwd(bqd, bkd, bvd, bo, bdo, blse, causal=True)
        return [o, lse, od, ld, *g]

    ref = run()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = run()
        with torch.cuda.stream(s2):
            b = run()
        outs += [a, b]
    s1.synchronize()
    s2.synchronize()
    for got in outs:
        for x, y in zip(got, ref):
            assert torch.equal(x, y)
