"""Packed variable-length forward over a paged K/V cache.

A chunked prefill whose new tokens' K and V have been appended to a paged
cache: each sequence's queries attend (bottom-right causal, or fully) to its
keys, key j of sequence s in slot j % P of page block_table[s, j // P].  The
engine setting is the one "Tang Project Derives GPU Kernels via IR ..."
describes in its "Details" section (long prefill, many concurrent streams of
unequal length).

CPU: the oracle's gather against an independent scatter of packed histories
(the paged oracle is then the packed oracle on the same keys, bit for bit).
GPU: attn_fwd_varlen_paged against that oracle with every unused slot and
page set to NaN, over empty sequences, Lq < Lk and Lq > Lk, pages of 64 to
256 keys, grouped heads and d = 64 and 128; bit for bit against
attn_fwd_varlen when the pages hold the packed keys in order; and sampled
rows of a large chunked-prefill batch.
"""
import math

import numpy as np
import pytest

import oracle
import synth

# ---------------------------------------------------------------- CPU pins


@pytest.mark.parametrize("causal", [True, False])
def test_paged_varlen_oracle_equals_packed_oracle(causal):
    lens_q, lens_k = [3, 0, 5, 2], [7, 0, 5, 1]
    Hq, Hkv, d, P = 4, 2, 8, 4
    q, k, v, cu_q, cu_k = synth.varlen_inputs(41, lens_q, lens_k, Hq, Hkv, d, bf16=True)
    rng = np.random.default_rng(9)
    n_pages = sum((n + P - 1) // P for n in lens_k) + 2
    kc = np.full((n_pages, Hkv, P, d), np.nan, np.float32)
    vc = np.full((n_pages, Hkv, P, d), np.nan, np.float32)
    table = np.full((len(lens_k), 2), -1, np.int32)
    free = list(rng.permutation(n_pages))
    for s, n in enumerate(lens_k):
        for j in range(n):                       # scatter key by key
            if j % P == 0:
                table[s, j // P] = free.pop()
            kc[table[s, j // P], :, j % P] = k[:, cu_k[s] + j]
            vc[table[s, j // P], :, j % P] = v[:, cu_k[s] + j]
    o, lse = oracle.fwd_varlen_paged(q, kc, vc, table, cu_q, np.array(lens_k, np.int32), 0.3, causal)
    eo, el = oracle.fwd_varlen(q, k, v, cu_q, cu_k, 0.3, causal)
    assert np.array_equal(o, eo) and np.array_equal(lse, el)


# ---------------------------------------------------------------- GPU parity

CASES = [
    # lens_q, lens_k, Hq, Hkv, page, d
    ([100, 37, 256, 3], [300, 37, 1000, 3], 4, 4, 64, 64),
    ([40, 200, 17, 0], [20, 60, 0, 5], 2, 1, 128, 128),          # Lq > Lk, a sequence with no keys
    ([300, 1, 129], [700, 513, 129], 8, 2, 256, 128),
    ([65, 64, 63], [65, 64, 63], 4, 2, 64, 128),                  # prefill from an empty cache
    # 16 x 32 x 5 tiles of 256 rows: the two-group 8-wave kernel; the longest
    # history spans more than 64 pages of 64 keys (the page-table path past
    # the per-lane copy)
    ([1100, 37, 300, 5, 256, 257, 0, 64, 129, 700, 1, 90, 255, 513, 31, 200],
     [4300, 37, 400, 5, 256, 900, 0, 64, 129, 700, 300, 90, 255, 513, 31, 0], 32, 8, 64, 128),
]


# 300 short sequences (past the 256 whose sizes the item placement keeps in
# registers; 300 x 4 heads take the 4-wave kernel)
_r300 = np.random.default_rng(301)
_lq300 = [int(x) for x in _r300.integers(0, 41, size=300)]
CASES.append((_lq300, [lq + int(h) for lq, h in zip(_lq300, _r300.integers(0, 100, size=300))], 4, 2, 64, 64))

def _dev_cache(kc, vc, used):
    import torch

    from gpu_helpers import dev

    kd, vd = dev(kc, True), dev(vc, True)
    mask = torch.from_numpy(~used).cuda()[:, None, :, None].expand(kd.shape)
    return kd.masked_fill(mask, float("nan")).contiguous(), vd.masked_fill(mask, float("nan")).contiguous()


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("causal", [True, False])
def test_paged_varlen_matches_oracle(oracle_mod, case, causal):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    lens_q, lens_k, Hq, Hkv, page, d = CASES[case]
    print(f"paged varlen case {case} causal={causal} lens_q={lens_q} lens_k={lens_k} page={page} d={d}", flush=True)
    q, kc, vc, table, cu_q, lens, used = synth.paged_varlen_inputs(600 + case, lens_q, lens_k, Hq, Hkv, page, d)
    kd, vd = _dev_cache(kc, vc, used)
    o, lse = am.attn_fwd_varlen_paged(dev(q, True), kd, vd, torch.from_numpy(table).cuda(),
                                      torch.from_numpy(cu_q).cuda(), torch.from_numpy(lens).cuda(), max(lens_q),
                                      max(lens_k), causal=causal)
    torch.cuda.synchronize()
    eo, el = oracle.fwd_varlen_paged(q, kc, vc, table, cu_q, lens, 1.0 / math.sqrt(d), causal)
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [True, False])
def test_paged_varlen_in_order_equals_packed(causal):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    lens_q, lens_k, Hq, Hkv, d, P = [200, 64, 130], [512, 128, 256], 8, 2, 128, 128
    q, k, v, cu_q, cu_k = synth.varlen_inputs(620, lens_q, lens_k, Hq, Hkv, d, bf16=True)
    # the packed keys of each sequence cut into pages, in order
    pages_k, pages_v, table = [], [], np.zeros((3, 4), np.int32)
    for s, n in enumerate(lens_k):
        for pi in range(n // P):
            table[s, pi] = len(pages_k)
            a0 = cu_k[s] + pi * P
            pages_k.append(k[:, a0:a0 + P])
            pages_v.append(v[:, a0:a0 + P])
    kc, vc = np.stack(pages_k), np.stack(pages_v)  # [num_pages, Hkv, P, d]
    lens = np.array(lens_k, np.int32)
    cq = torch.from_numpy(cu_q).cuda()
    o_p, l_p = am.attn_fwd_varlen_paged(dev(q, True), dev(kc, True), dev(vc, True), torch.from_numpy(table).cuda(),
                                        cq, torch.from_numpy(lens).cuda(), max(lens_q), max(lens_k), causal=causal)
    o_d, l_d = am.attn_fwd_varlen(dev(q, True), dev(k, True), dev(v, True), cq, torch.from_numpy(cu_k).cuda(),
                                  max(lens_q), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_d)
    assert torch.equal(l_p, l_d)


@pytest.mark.gpu
def test_paged_varlen_large_chunked_prefill_sampled_rows(oracle_mod):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, dev, host

    lens_q, lens_k = synth.chunked_prefill_lengths(8, 16, (512, 2048), (0, 4096))
    Hq, Hkv, d, page = 32, 8, 128, 64
    print(f"paged varlen large: total_q={sum(lens_q)} total_k={sum(lens_k)}", flush=True)
    q, kc, vc, table, cu_q, lens, used = synth.paged_varlen_inputs(630, lens_q, lens_k, Hq, Hkv, page, d)
    kd, vd = _dev_cache(kc, vc, used)
    o, lse = am.attn_fwd_varlen_paged(dev(q, True), kd, vd, torch.from_numpy(table).cuda(),
                                      torch.from_numpy(cu_q).cuda(), torch.from_numpy(lens).cuda(), max(lens_q),
                                      max(lens_k), causal=True)
    torch.cuda.synchronize()
    # the packed histories the pages hold, for the oracle's row sampler
    j_all = [np.arange(n) for n in lens_k]
    k = np.concatenate([kc[table[s, j // page], :, j % page, :].transpose(1, 0, 2) for s, j in enumerate(j_all)], 1)
    v = np.concatenate([vc[table[s, j // page], :, j % page, :].transpose(1, 0, 2) for s, j in enumerate(j_all)], 1)
    cu_k = synth.offsets(lens_k)
    rng = np.random.default_rng(631)
    rows = np.stack([rng.integers(0, Hq, 256), rng.integers(0, int(cu_q[-1]), 256)], axis=1)
    o_ref, lse_ref = oracle.fwd_varlen_rows(q, np.ascontiguousarray(k), np.ascontiguousarray(v), cu_q, cu_k, rows,
                                            1.0 / math.sqrt(d), True)
    og, lg = host(o), host(lse)
    assert_close("O", og[rows[:, 0], rows[:, 1]], o_ref, TOL_O_BF16)
    assert_close("LSE", lg[rows[:, 0], rows[:, 1]], lse_ref, TOL_LSE_BF16)
