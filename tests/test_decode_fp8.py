"""Split-KV decode over an FP8 (OCP E4M3) KV cache with a scale per kv head.

FP8 KV caches are what the fastest engine the page "Tang Project Derives GPU
Kernels via IR ..." compares against serves (section "Details"); decoding
from such a cache reads half the bytes of bf16.

CPU: the oracle's E4M3 decoder against values the format definition fixes,
the test-input encoder against that decoder (round trip, ties to even,
saturation), and the FP8 oracle against a direct fp64 evaluation.
GPU: attn_decode_splitkv_fp8 against the oracle at the 32 / 8-head decode
shapes and a ragged d = 64 one, across split counts, and bit-for-bit against
the bf16 decode of the same dequantized cache when the scales are powers of
two (then every dequantized value is a bf16 value and the scales commute
with rounding).
"""
import math

import numpy as np
import pytest

import oracle
import synth

# ---------------------------------------------------------------- CPU pins


def test_e4m3_decoder_fixed_values():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9          # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert v(0x08) == 2.0 ** -6          # smallest normal
    assert v(0x38) == 1.0
    assert v(0x3C) == 1.5
    assert v(0x40) == 2.0
    assert v(0x7E) == 448.0              # largest finite
    assert v(0xB8) == -1.0 and v(0xFE) == -448.0
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    pos = oracle.e4m3_value(np.arange(127))
    assert np.all(np.diff(pos) > 0)      # codes 0..126 increase
    assert np.array_equal(oracle.e4m3_value(np.arange(127) | 0x80), -pos)


def test_e4m3_encoder_round_trip_ties_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0x80, 0xFF)], np.uint8)
    assert np.array_equal(synth.quantize_e4m3(oracle.e4m3_value(codes), 1.0), codes)
    q = lambda x: int(synth.quantize_e4m3(np.array([x]), 1.0)[0])
    assert q(1.0625) == 0x38             # halfway between 1 and 1.125: to the even code
    assert q(1.1875) == 0x3A             # halfway between 1.125 and 1.25: to the even code
    assert q(1000.0) == 0x7E and q(-1000.0) == 0xFE
    assert q(2.0 ** -10) == 0x00         # halfway between 0 and the smallest subnormal
    assert q(1.5 * 2.0 ** -10) == 0x01
    assert q(0.5) == 0x30 and q(-3.0) == 0xC4


def test_fp8_oracle_matches_direct_evaluation():
    q, k8, v8, ks, vs = synth.fp8_kv_inputs(21, 2, 8, 2, 40, 16)
    o, lse = oracle.decode_fp8(q, k8, v8, ks, vs, 0.25)
    k = oracle.e4m3_value(k8) * ks.astype(np.float64).reshape(1, -1, 1, 1)
    v = oracle.e4m3_value(v8) * vs.astype(np.float64).reshape(1, -1, 1, 1)
    kk, vv = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    s = 0.25 * np.einsum("bhqd,bhkd->bhqk", q.astype(np.float64), kk)
    m = s.max(-1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(-1, keepdims=True)
    assert np.max(np.abs(o - np.einsum("bhqk,bhkd->bhqd", p / z, vv))) < 1e-13
    assert np.max(np.abs(lse - (m + np.log(z))[..., 0])) < 1e-13


# ---------------------------------------------------------------- GPU parity

SHAPES = [(1, 32, 8, 512, 128), (16, 32, 8, 4096, 128), (48, 32, 8, 2048, 128), (3, 8, 2, 1000, 64)]


def _run(q, k8, v8, ks, vs, splits):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    d = q.shape[3]
    return am.attn_decode_splitkv_fp8(dev(q, True), torch.from_numpy(k8).cuda(), torch.from_numpy(v8).cuda(),
                                      torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda(),
                                      scale=1.0 / math.sqrt(d), num_splits=splits)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", SHAPES)
def test_fp8_decode_matches_oracle(oracle_mod, shape):
    import torch

    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, host

    B, Hq, Hkv, L, d = shape
    print(f"fp8 decode B={B} Hq={Hq} Hkv={Hkv} L={L} d={d}", flush=True)
    q, k8, v8, ks, vs = synth.fp8_kv_inputs(700 + L, B, Hq, Hkv, L, d)
    o_ref, lse_ref = oracle.decode_fp8(q, k8, v8, ks, vs, 1.0 / math.sqrt(d))
    o, lse = _run(q, k8, v8, ks, vs, 0)
    torch.cuda.synchronize()
    assert_close("O", host(o), o_ref, TOL_O_BF16)
    assert_close("LSE", host(lse), lse_ref, TOL_LSE_BF16)


@pytest.mark.gpu
@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_fp8_decode_split_counts(oracle_mod, splits):
    import torch

    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, host

    B, Hq, Hkv, L, d = 4, 32, 8, 1500, 128
    print(f"fp8 decode splits={splits}", flush=True)
    q, k8, v8, ks, vs = synth.fp8_kv_inputs(800, B, Hq, Hkv, L, d)
    o_ref, lse_ref = oracle.decode_fp8(q, k8, v8, ks, vs, 1.0 / math.sqrt(d))
    o, lse = _run(q, k8, v8, ks, vs, splits)
    torch.cuda.synchronize()
    assert_close("O", host(o), o_ref, TOL_O_BF16)
    assert_close("LSE", host(lse), lse_ref, TOL_LSE_BF16)


@pytest.mark.gpu
@pytest.mark.parametrize("splits", [1, 2])
def test_fp8_decode_equals_bf16_decode_of_dequantized_cache(splits):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    B, Hq, Hkv, L, d = 6, 32, 8, 700, 128
    print(f"fp8 vs bf16 decode splits={splits}", flush=True)
    q, k8, v8, _, _ = synth.fp8_kv_inputs(900, B, Hq, Hkv, L, d)
    ks = np.array([2.0 ** -(7 + h % 3) for h in range(Hkv)], np.float32)
    vs = np.array([2.0 ** -(6 + h % 2) for h in range(Hkv)], np.float32)
    k = (oracle.e4m3_value(k8) * ks.reshape(1, -1, 1, 1)).astype(np.float32)
    v = (oracle.e4m3_value(v8) * vs.reshape(1, -1, 1, 1)).astype(np.float32)
    o8, l8 = _run(q, k8, v8, ks, vs, splits)
    ob, lb = am.attn_decode_splitkv(dev(q, True), dev(k, True), dev(v, True), scale=1.0 / math.sqrt(d),
                                    num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o8, ob)
    assert torch.equal(l8, lb)
