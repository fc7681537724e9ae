"""Variable-length (packed) forward and chunked prefill against a KV history.

Each sequence of a packed batch is its own softmax-attention problem over its
own keys, with the causal rule applied per sequence (bottom-right: a sequence
with Lk > Lq attends to Lk - Lq cached keys before its new tokens).  The
engine setting is the one the page "Tang Project Derives GPU Kernels via IR
..." describes in its "Details" section (a long prefill, many concurrent
streams of unequal length).

CPU: the oracle's packed-batch composition is pinned to a 50-digit brute
force that reads sequence membership straight off the packed rows.
GPU: attn_fwd_varlen against that oracle on every row of small batches
(ragged lengths across tile boundaries, empty sequences, Lq < Lk and
Lq > Lk, grouped-query heads, d = 64 and 128; two of them large enough in
tiles for the two-group kernel), against the dense entry point
when every sequence has the same length, and on sampled rows of a large
chunked-prefill batch.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import brute

# ---------------------------------------------------------------- CPU pins


@pytest.mark.parametrize("causal", [True, False])
def test_oracle_varlen_matches_brute_force(causal):
    # lengths: a short sequence, an empty one, Lq > Lk (causal rows with no
    # visible key), Lq < Lk (a history before the new tokens)
    lens_q, lens_k = [2, 0, 3, 2], [3, 1, 1, 5]
    q, k, v, cu_q, cu_k = synth.varlen_inputs(11, lens_q, lens_k, 4, 2, 3, bf16=False)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, 0.7, causal)
    ob, lb = brute.brute_fwd_varlen(q, k, v, cu_q, cu_k, 0.7, causal)
    assert np.array_equal(np.isfinite(lse), np.isfinite(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin])) < 1e-12
    assert np.max(np.abs(o - ob)) < 1e-12
    if causal:
        # sequence 2 has Lq = 3, Lk = 1: its first two rows see no key
        r = int(cu_q[2])
        assert np.all(np.isneginf(lse[:, r:r + 2])) and np.all(o[:, r:r + 2] == 0.0)


def test_oracle_varlen_rows_match_full():
    lens_q, lens_k = [5, 9, 1], [7, 9, 4]
    q, k, v, cu_q, cu_k = synth.varlen_inputs(12, lens_q, lens_k, 4, 1, 8, bf16=True)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, 0.35, True)
    rows = np.array([(h, i) for h in range(4) for i in range(int(cu_q[-1]))], np.int64)
    orr, lr = oracle.fwd_varlen_rows(q, k, v, cu_q, cu_k, rows, 0.35, True)
    assert np.max(np.abs(orr - o[rows[:, 0], rows[:, 1]])) == 0.0
    fin = np.isfinite(lr)
    assert np.array_equal(lr[fin], lse[rows[:, 0], rows[:, 1]][fin])


def test_chunked_prefill_lengths_recipe():
    lq, lk = synth.chunked_prefill_lengths(3, 16, (512, 2048), (0, 4096))
    assert len(lq) == len(lk) == 16
    assert all(512 <= a <= 2048 and a <= b <= a + 4096 for a, b in zip(lq, lk))
    cu = synth.offsets(lq)
    assert cu.dtype == np.int32 and cu[0] == 0 and cu[-1] == sum(lq)


# ---------------------------------------------------------------- GPU parity

SMALL = [
    # (lens_q, lens_k, Hq, Hkv, d)
    ([1, 63, 64, 65, 130, 257, 0, 5], [1, 63, 64, 65, 130, 257, 0, 5], 4, 2, 128),
    ([100, 37, 256, 3], [300, 37, 1000, 3], 4, 4, 64),       # chunked prefill: history before the new rows
    ([40, 200, 17], [20, 60, 0], 2, 1, 128),                 # Lq > Lk and a sequence with no keys
    ([300, 1, 129], [700, 513, 129], 8, 2, 64),
]

# 300 short sequences: past the 256 whose sizes the item placement keeps in
# registers, so the rest are read again from the offsets; 300 x 8 heads reach
# the two-group kernel
_r300 = np.random.default_rng(300)
LQ300 = [int(x) for x in _r300.integers(0, 41, size=300)]
LK300 = [lq + int(h) for lq, h in zip(LQ300, _r300.integers(0, 61, size=300))]
SMALL.append((LQ300, LK300, 8, 2, 64))


# Packed batches of at least 2048 tiles of 256 rows (every sequence counted at
# the longest one's length) take the two-group 8-wave kernel: here one
# 1100-row sequence gives 16 x 32 x 5 = 2560 such tiles, and the other
# sequences are short, ragged, empty or without keys, so that every row can
# be checked against the oracle.
TWO_GROUP_LQ = [1100, 37, 300, 5, 256, 257, 0, 64, 129, 700, 1, 90, 255, 513, 31, 200]
TWO_GROUP_LK = [1300, 37, 400, 5, 256, 900, 0, 64, 129, 700, 300, 90, 255, 513, 31, 0]
SMALL += [(TWO_GROUP_LQ, TWO_GROUP_LK, 32, 8, 128), (TWO_GROUP_LQ, TWO_GROUP_LK, 32, 8, 64)]


def test_two_group_cases_reach_the_packed_threshold():
    for lens_q, _, Hq, _, _ in SMALL[-2:]:
        assert len(lens_q) * Hq * -(-max(lens_q) // 256) >= 2048


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(SMALL)))
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_all_rows(oracle_mod, case, causal):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    lens_q, lens_k, Hq, Hkv, d = SMALL[case]
    print(f"varlen case {case} causal={causal} lens_q={lens_q} lens_k={lens_k} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
    q, k, v, cu_q, cu_k = synth.varlen_inputs(500 + case, lens_q, lens_k, Hq, Hkv, d, bf16=True)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale, causal)
    cq = torch.from_numpy(cu_q).cuda()
    ck = torch.from_numpy(cu_k).cuda()
    o, lse = am.attn_fwd_varlen(dev(q, True), dev(k, True), dev(v, True), cq, ck, max(lens_q), causal=causal)
    torch.cuda.synchronize()
    assert_close("O", host(o), o_ref, TOL_O_BF16)
    assert_close("LSE", host(lse), lse_ref, TOL_LSE_BF16)


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_equal_lengths_match_dense(causal):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    B, Hq, Hkv, N, d = 3, 4, 2, 300, 128
    print(f"varlen vs dense B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal}", flush=True)
    q, k, v = synth.attn_inputs(77, B, Hq, Hkv, N, N, d, bf16=True)
    qd, kd, vd = dev(q, True), dev(k, True), dev(v, True)
    o_dense, lse_dense = am.attn_fwd(qd, kd, vd, causal=causal)
    # [B, H, N, d] -> packed [H, B * N, d]
    pack = lambda t: t.permute(1, 0, 2, 3).reshape(t.shape[1], B * N, d).contiguous()
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o, lse = am.attn_fwd_varlen(pack(qd), pack(kd), pack(vd), cu, cu, N, causal=causal)
    torch.cuda.synchronize()
    # the same kernel on the same tiles: identical bits
    assert torch.equal(o, pack(o_dense))
    assert torch.equal(lse, lse_dense.permute(1, 0, 2).reshape(Hq, B * N))


@pytest.mark.gpu
def test_varlen_large_chunked_prefill_sampled_rows(oracle_mod):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    lens_q, lens_k = synth.chunked_prefill_lengths(8, 16, (512, 2048), (0, 4096))
    Hq, Hkv, d = 32, 8, 128
    print(f"varlen large: {len(lens_q)} sequences, total_q={sum(lens_q)} total_k={sum(lens_k)}", flush=True)
    q, k, v, cu_q, cu_k = synth.varlen_inputs(9, lens_q, lens_k, Hq, Hkv, d, bf16=True)
    cq = torch.from_numpy(cu_q).cuda()
    ck = torch.from_numpy(cu_k).cuda()
    o, lse = am.attn_fwd_varlen(dev(q, True), dev(k, True), dev(v, True), cq, ck, max(lens_q), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = np.stack([rng.integers(0, Hq, 256), rng.integers(0, int(cu_q[-1]), 256)], axis=1)
    # every sequence's first and last rows too
    extra = [(int(rng.integers(Hq)), int(i)) for s in range(len(lens_q)) for i in (cu_q[s], cu_q[s + 1] - 1)]
    rows = np.concatenate([rows, np.array(extra, np.int64)])
    o_ref, lse_ref = oracle.fwd_varlen_rows(q, k, v, cu_q, cu_k, rows, 1.0 / math.sqrt(d), True)
    og, lg = host(o), host(lse)
    assert_close("O", og[rows[:, 0], rows[:, 1]], o_ref, TOL_O_BF16)
    assert_close("LSE", lg[rows[:, 0], rows[:, 1]], lse_ref, TOL_LSE_BF16)
