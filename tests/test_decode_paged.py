"""Split-KV decode over a paged KV cache with a length per stream.

Serving engines keep the cache in pages and decode many streams of unequal
length at once; "Tang Project Derives GPU Kernels via IR ..." (section
"Details") measures decode at 16-48 concurrent streams.  Key j of stream b
is slot j % P of page block_table[b, j // P] of a [num_pages, Hkv, P, d]
cache.

CPU: the oracle's gather against an independent scatter of dense histories
(so the paged oracle is the dense oracle on the same keys), and the input
recipe.  GPU: attn_decode_paged against that oracle with every slot and page
that no stream uses set to NaN (a read of one would show), lengths of 0, 1,
below, at and above page and tile boundaries, page sizes 32 to 256, grouped
and ungrouped heads, d = 64 and 128 and several split counts; and bit for
bit against the dense decode when the table maps the pages in order.
"""
import math

import numpy as np
import pytest

import oracle
import synth

# ---------------------------------------------------------------- CPU pins


def test_paged_oracle_equals_dense_oracle_on_scattered_histories():
    B, Hq, Hkv, d, P = 3, 4, 2, 16, 8
    lens = [13, 0, 24]
    q, k, v = synth.attn_inputs(31, B, Hq, Hkv, 1, max(lens), d, bf16=True)
    rng = np.random.default_rng(5)
    n_pages = sum((n + P - 1) // P for n in lens) + 2
    kc = np.full((n_pages, Hkv, P, d), np.nan, np.float32)
    vc = np.full((n_pages, Hkv, P, d), np.nan, np.float32)
    table = np.full((B, 3), -1, np.int32)
    free = list(rng.permutation(n_pages))
    for b, n in enumerate(lens):
        for j in range(n):               # scatter key by key
            if j % P == 0:
                table[b, j // P] = free.pop()
            kc[table[b, j // P], :, j % P] = k[b, :, j]
            vc[table[b, j // P], :, j % P] = v[b, :, j]
    o, lse = oracle.decode_paged(q, kc, vc, table, np.array(lens, np.int32), 0.25)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b]))
            continue
        eo, el = oracle.fwd(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.25, False)
        assert np.array_equal(o[b:b + 1], eo) and np.array_equal(lse[b:b + 1], el)


def test_paged_inputs_recipe():
    q, kc, vc, table, lens, used = synth.paged_kv_inputs(3, [0, 1, 64, 65, 200], 8, 2, 64, 32)
    assert kc.shape == vc.shape == (int(((lens + 63) // 64).sum()) + 3, 2, 64, 32)
    ids = table[table >= 0]
    assert len(set(ids.tolist())) == len(ids)                 # no page shared
    assert list((table >= 0).sum(1)) == [0, 1, 1, 2, 4]
    assert used.sum() == sum(lens)


# ---------------------------------------------------------------- GPU parity

CASES = [
    # lens, Hq, Hkv, page, d
    ([0, 1, 31, 32, 33, 700], 8, 2, 32, 128),
    ([300, 0, 129, 64], 4, 4, 64, 64),
    ([256, 255, 1000], 16, 2, 256, 128),
    ([5000, 17], 2, 1, 128, 64),
    # 300 streams: past the 256 whose lengths the longest-first placement
    # keeps in registers, the rest read again from seq_lens
    ([int(x) for x in np.random.default_rng(302).integers(0, 200, size=300)], 8, 2, 32, 64),
]


def _run(q, kc, vc, table, lens, used, splits, poison=True):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    kd, vd = dev(kc, True), dev(vc, True)
    if poison:
        mask = torch.from_numpy(~used).cuda()[:, None, :, None].expand(kd.shape)
        kd = kd.masked_fill(mask, float("nan")).contiguous()
        vd = vd.masked_fill(mask, float("nan")).contiguous()
    return am.attn_decode_paged(dev(q, True), kd, vd, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                                int(lens.max()) if len(lens) else 0, num_splits=splits)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_paged_matches_oracle(oracle_mod, case, splits):
    import torch

    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, host

    lens, Hq, Hkv, page, d = CASES[case]
    print(f"paged decode lens={lens} Hq={Hq} Hkv={Hkv} page={page} d={d} splits={splits}", flush=True)
    q, kc, vc, table, lens_a, used = synth.paged_kv_inputs(900 + case, lens, Hq, Hkv, page, d)
    o, lse = _run(q, kc, vc, table, lens_a, used, splits)
    torch.cuda.synchronize()
    eo, el = oracle.decode_paged(q, kc, vc, table, lens_a, 1.0 / math.sqrt(d))
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)


@pytest.mark.gpu
def test_paged_48_streams_unequal_lengths(oracle_mod):
    import torch

    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, host

    rng = np.random.default_rng(48)
    lens = [int(x) for x in rng.integers(512, 4097, size=48)]
    print(f"paged decode 48 streams, {sum(lens)} keys", flush=True)
    q, kc, vc, table, lens_a, used = synth.paged_kv_inputs(948, lens, 32, 8, 64, 128)
    o, lse = _run(q, kc, vc, table, lens_a, used, 0)
    torch.cuda.synchronize()
    eo, el = oracle.decode_paged(q, kc, vc, table, lens_a, 1.0 / math.sqrt(128))
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)


@pytest.mark.gpu
@pytest.mark.parametrize("splits", [1, 2, 5])
def test_paged_in_order_equals_dense_decode(splits):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    B, Hq, Hkv, L, d, P = 4, 32, 8, 1024, 128, 64
    q, k, v = synth.attn_inputs(950, B, Hq, Hkv, 1, L, d, bf16=True)
    # page p of stream b holds its keys p*P .. p*P + P - 1: [B, Hkv, L, d] -> [B * L/P, Hkv, P, d]
    to_pages = lambda x: np.ascontiguousarray(x.reshape(B, Hkv, L // P, P, d).transpose(0, 2, 1, 3, 4)
                                              .reshape(B * L // P, Hkv, P, d))
    table = np.arange(B * L // P, dtype=np.int32).reshape(B, L // P)
    lens = np.full(B, L, np.int32)
    o_p, l_p = am.attn_decode_paged(dev(q, True), dev(to_pages(k), True), dev(to_pages(v), True),
                                    torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), L,
                                    num_splits=splits)
    o_d, l_d = am.attn_decode_splitkv(dev(q, True), dev(k, True), dev(v, True), num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_d)
    assert torch.equal(l_p, l_d)


# ---------------------------------------------------------------- single launch

def _run_fused(q, kc, vc, table, lens, used, splits, workspace=None):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import dev

    kd, vd = dev(kc, True), dev(vc, True)
    mask = torch.from_numpy(~used).cuda()[:, None, :, None].expand(kd.shape)
    kd = kd.masked_fill(mask, float("nan")).contiguous()
    vd = vd.masked_fill(mask, float("nan")).contiguous()
    return am.attn_decode_paged_fused(dev(q, True), kd, vd, torch.from_numpy(table).cuda(),
                                      torch.from_numpy(lens).cuda(), int(lens.max()) if len(lens) else 0,
                                      num_splits=splits, workspace=workspace)


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("splits", [1, 3])
def test_paged_fused_equals_two_launch_bits(case, splits):
    import torch

    lens, Hq, Hkv, page, d = CASES[case]
    print(f"paged decode, one launch vs two: lens[:8]={lens[:8]} Hq={Hq} Hkv={Hkv} page={page} d={d} splits={splits}",
          flush=True)
    q, kc, vc, table, lens_a, used = synth.paged_kv_inputs(900 + case, lens, Hq, Hkv, page, d)
    o1, l1 = _run(q, kc, vc, table, lens_a, used, splits)
    o2, l2 = _run_fused(q, kc, vc, table, lens_a, used, splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


@pytest.mark.gpu
def test_paged_fused_auto_plan_and_workspace_reuse(oracle_mod):
    import torch

    import attention_online_softmax_attn_amd as am
    from gpu_helpers import TOL_LSE_BF16, TOL_O_BF16, assert_close, host

    # 16 streams of unequal length: the plan splits (fewer (stream, kv head)
    # pairs than CUs), so the last chunk of each pair merges
    rng = np.random.default_rng(16)
    lens = [int(x) for x in rng.integers(512, 4097, size=16)]
    assert am.decode_paged_fused_workspace_bytes(16, 32, 8, max(lens), 128) > 65536
    q, kc, vc, table, lens_a, used = synth.paged_kv_inputs(960, lens, 32, 8, 64, 128)
    ws = torch.zeros(am.decode_paged_fused_workspace_bytes(16, 32, 8, max(lens), 128), dtype=torch.uint8,
                     device="cuda")
    print(f"paged decode in one launch, 16 streams, {sum(lens)} keys, workspace {ws.numel()} bytes", flush=True)
    o, lse = _run_fused(q, kc, vc, table, lens_a, used, 0, workspace=ws)
    torch.cuda.synchronize()
    eo, el = oracle.decode_paged(q, kc, vc, table, lens_a, 1.0 / math.sqrt(128))
    assert_close("O", host(o), eo, TOL_O_BF16)
    assert_close("LSE", host(lse), el, TOL_LSE_BF16)
    assert int(ws[:65536].count_nonzero()) == 0      # every arrival count back at zero
    # the same workspace serves a smaller call
    q2, kc2, vc2, table2, lens2, used2 = synth.paged_kv_inputs(961, lens[:5], 32, 8, 64, 128)
    o2, l2 = _run_fused(q2, kc2, vc2, table2, lens2, used2, 0, workspace=ws)
    torch.cuda.synchronize()
    e2, f2 = oracle.decode_paged(q2, kc2, vc2, table2, lens2, 1.0 / math.sqrt(128))
    assert_close("O", host(o2), e2, TOL_O_BF16)
    assert_close("LSE", host(l2), f2, TOL_LSE_BF16)
    assert int(ws[:65536].count_nonzero()) == 0
