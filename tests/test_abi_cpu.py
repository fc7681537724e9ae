"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments on the host before any HIP call.  No compute runs."""
import ctypes
import os
import re

import pytest

import attention_online_softmax_attn_amd as am

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(attn_[a-z0-9_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("attn_fwd", "attn_fwd_varlen", "attn_decode_splitkv", "attn_decode_splitkv_fp8", "attn_bwd",
              "attn_decode_splitkv_fused", "attn_decode_fused_workspace_bytes", "attn_decode_workspace_bytes",
              "attn_decode_paged", "attn_fwd_varlen_paged", "attn_decode_paged_fused",
              "attn_decode_paged_fused_workspace_bytes",
              "attn_bwd_workspace_bytes", "attn_decode_num_splits", "attn_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = am.lib()
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in include/attn.h but not exported"
    out = os.popen(f"nm -D --defined-only {am.LIB_PATH}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, re.M), f"{n} is not a defined dynamic symbol"


def test_library_targets_gfx950():
    data = open(am.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_strerror():
    assert am.strerror(am.ATTN_OK) == "ok"
    assert "workspace" in am.strerror(am.ATTN_ERR_WORKSPACE)
    assert am.strerror(99) == "unknown status"


# Fake device pointers are only used for calls that must be rejected on the
# host.  They are never passed where a GPU is visible.
no_gpu = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0, reason="host-only rejection tests use fake pointers"
)
P = ctypes.c_void_p(0x100000)
NUL = None


def fwd(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=2, Hkv=1, Nq=8, Nk=8, d=64, scale=0.125, causal=0, dt=am.ATTN_BF16):
    return am.lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dt, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(o=NUL), am.ATTN_ERR_INVALID),
        (dict(k=NUL), am.ATTN_ERR_INVALID),
        (dict(B=-1), am.ATTN_ERR_INVALID),
        (dict(Hq=3, Hkv=2), am.ATTN_ERR_INVALID),
        (dict(Hkv=0), am.ATTN_ERR_INVALID),
        (dict(Nq=-2), am.ATTN_ERR_INVALID),
        (dict(scale=0.0), am.ATTN_ERR_INVALID),
        (dict(scale=-1.0), am.ATTN_ERR_INVALID),
        (dict(scale=float("nan")), am.ATTN_ERR_INVALID),
        (dict(scale=float("inf")), am.ATTN_ERR_INVALID),
        (dict(dt=7), am.ATTN_ERR_INVALID),
        (dict(d=96), am.ATTN_ERR_UNSUPPORTED),
        (dict(d=256), am.ATTN_ERR_UNSUPPORTED),
        (dict(Nk=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(B=1 << 11, Hq=1 << 10, Hkv=1 << 10), am.ATTN_ERR_UNSUPPORTED),          # B * Hq above 2^20
        (dict(B=1 << 10, Hq=1 << 10, Hkv=1, Nq=1 << 22), am.ATTN_ERR_UNSUPPORTED),  # a query grid of 2^37 workgroups
    ],
)
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


@no_gpu
def test_empty_outputs_launch_nothing():
    # B = 0 or Nq = 0: nothing to write, accepted even with null pointers
    assert fwd(q=NUL, k=NUL, v=NUL, o=NUL, lse=NUL, B=0) == am.ATTN_OK
    assert fwd(q=NUL, k=NUL, v=NUL, o=NUL, lse=NUL, Nq=0) == am.ATTN_OK


def fwd_varlen(q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, n=3, tq=300, tk=500, maxq=128, Hq=4, Hkv=2, d=128,
               scale=0.088, causal=1, dt=am.ATTN_BF16):
    return am.lib().attn_fwd_varlen(q, k, v, o, lse, cq, ck, n, tq, tk, maxq, Hq, Hkv, d, scale, causal, dt, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(o=NUL), am.ATTN_ERR_INVALID),
        (dict(cq=NUL), am.ATTN_ERR_INVALID),
        (dict(ck=NUL), am.ATTN_ERR_INVALID),
        (dict(k=NUL), am.ATTN_ERR_INVALID),
        (dict(n=-1), am.ATTN_ERR_INVALID),
        (dict(tq=-1), am.ATTN_ERR_INVALID),
        (dict(tk=-5), am.ATTN_ERR_INVALID),
        (dict(maxq=-1), am.ATTN_ERR_INVALID),
        (dict(Hq=3), am.ATTN_ERR_INVALID),
        (dict(scale=0.0), am.ATTN_ERR_INVALID),
        (dict(dt=9), am.ATTN_ERR_INVALID),
        (dict(dt=am.ATTN_F32), am.ATTN_ERR_UNSUPPORTED),
        (dict(d=96), am.ATTN_ERR_UNSUPPORTED),
        (dict(tq=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(tk=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(maxq=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_fwd_varlen_rejects(kw, code):
    assert fwd_varlen(**kw) == code


@no_gpu
def test_fwd_varlen_empty_launches_nothing():
    for kw in (dict(n=0), dict(tq=0), dict(maxq=0)):
        assert fwd_varlen(q=NUL, k=NUL, v=NUL, o=NUL, lse=NUL, cq=NUL, ck=NUL, **kw) == am.ATTN_OK


def dec(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=32, Hkv=8, Nq=1, Nk=4096, d=128, scale=0.088, splits=0, ws=P,
        ws_bytes=1 << 30, dt=am.ATTN_BF16):
    return am.lib().attn_decode_splitkv(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 0, splits, ws, ws_bytes, dt,
                                        None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(Nq=2), am.ATTN_ERR_INVALID),
        (dict(splits=-1), am.ATTN_ERR_INVALID),
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(dt=am.ATTN_F32), am.ATTN_ERR_UNSUPPORTED),
        (dict(Hq=64, Hkv=1), am.ATTN_ERR_UNSUPPORTED),
        (dict(ws=NUL), am.ATTN_ERR_WORKSPACE),
        (dict(ws_bytes=16), am.ATTN_ERR_WORKSPACE),
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_decode_rejects(kw, code):
    assert dec(**kw) == code


def decf(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=32, Hkv=8, Nq=1, Nk=4096, d=128, scale=0.088, splits=0, ws=P,
         ws_bytes=1 << 30, dt=am.ATTN_BF16):
    return am.lib().attn_decode_splitkv_fused(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 0, splits, ws, ws_bytes,
                                              dt, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(Nq=2), am.ATTN_ERR_INVALID),
        (dict(splits=-1), am.ATTN_ERR_INVALID),
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(dt=am.ATTN_F32), am.ATTN_ERR_UNSUPPORTED),
        (dict(ws=NUL), am.ATTN_ERR_WORKSPACE),
        (dict(ws=ctypes.c_void_p(0x100002)), am.ATTN_ERR_INVALID),   # counts need 4-byte alignment
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
        (dict(B=4097, Nk=512, splits=2), am.ATTN_ERR_UNSUPPORTED),      # more pairs than counts
    ],
)
def test_decode_fused_rejects(kw, code):
    assert decf(**kw) == code


@no_gpu
def test_decode_fused_workspace_must_hold_the_counts():
    # exactly the two-launch workspace is too small: the counts come first
    B, Hq, Hkv, L, d, S = 2, 32, 8, 4096, 128, 8
    need2 = am.decode_workspace_bytes(B, Hq, Hkv, L, d, S)
    assert decf(ws_bytes=need2, splits=S) == am.ATTN_ERR_WORKSPACE
    assert decf(ws_bytes=am.decode_fused_workspace_bytes(B, Hq, Hkv, L, d, S) - 1, splits=S) == am.ATTN_ERR_WORKSPACE
    assert decf(ws_bytes=am.decode_fused_workspace_bytes(B, Hq, Hkv, L, d, 0) - 1) == am.ATTN_ERR_WORKSPACE


def test_decode_fused_workspace_layout():
    for B, L, s in [(1, 512, 4), (48, 4096, 2), (16, 4096, 3), (2, 4096, 1), (48, 4096, 128), (48, 4096, 0),
                    (1, 4096, 0)]:
        if s == 0:
            s = am.decode_fused_num_splits(B, 32, 8, L, 128)   # the automatic plans of the two may differ
            assert am.decode_fused_workspace_bytes(B, 32, 8, L, 128, 0) == am.decode_fused_workspace_bytes(
                B, 32, 8, L, 128, s)
        two = am.decode_workspace_bytes(B, 32, 8, L, 128, s)
        one = am.decode_fused_workspace_bytes(B, 32, 8, L, 128, s)
        if two == 0:
            assert one == 0                       # one chunk: no partials, no counts
        else:
            assert one == two + 65536                # a fixed region of arrival counts first


def fvp(q=P, k=P, v=P, bt=P, o=P, lse=P, cq=P, lk=P, n=4, tq=1000, maxq=400, maxk=2000, Hq=32, Hkv=8, d=128,
        pages=200, page=64, maxp=40, scale=0.088, causal=1):
    return am.lib().attn_fwd_varlen_paged(q, k, v, bt, o, lse, cq, lk, n, tq, maxq, maxk, Hq, Hkv, d, pages, page,
                                          maxp, scale, causal, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(page=32), am.ATTN_ERR_UNSUPPORTED),                   # not a multiple of 64
        (dict(page=0), am.ATTN_ERR_UNSUPPORTED),
        (dict(maxp=(1 << 22) // 64 + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(maxk=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(tq=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(n=-1), am.ATTN_ERR_INVALID),
        (dict(cq=NUL), am.ATTN_ERR_INVALID),
        (dict(lk=NUL), am.ATTN_ERR_INVALID),
        (dict(bt=NUL), am.ATTN_ERR_INVALID),
        (dict(k=NUL), am.ATTN_ERR_INVALID),
        (dict(pages=0), am.ATTN_ERR_INVALID),
        (dict(Hq=30), am.ATTN_ERR_INVALID),
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
        (dict(scale=float("nan")), am.ATTN_ERR_INVALID),
    ],
)
def test_fwd_varlen_paged_rejects(kw, code):
    assert fvp(**kw) == code


@no_gpu
def test_fwd_varlen_paged_empty_launches_nothing():
    assert fvp(q=NUL, k=NUL, v=NUL, bt=NUL, o=NUL, lse=NUL, cq=NUL, lk=NUL, n=0) == am.ATTN_OK
    assert fvp(q=NUL, k=NUL, v=NUL, bt=NUL, o=NUL, lse=NUL, cq=NUL, lk=NUL, tq=0) == am.ATTN_OK


def decp(q=P, k=P, v=P, bt=P, sl=P, o=P, lse=P, B=4, Hq=32, Hkv=8, d=128, pages=100, page=64, maxp=20,
         maxl=1280, scale=0.088, splits=0, ws=P, ws_bytes=1 << 30, fn="attn_decode_paged"):
    return getattr(am.lib(), fn)(q, k, v, bt, sl, o, lse, B, Hq, Hkv, d, pages, page, maxp, maxl, scale, splits,
                                 ws, ws_bytes, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(page=48), am.ATTN_ERR_UNSUPPORTED),                 # not a multiple of 32
        (dict(page=0), am.ATTN_ERR_UNSUPPORTED),
        (dict(page=-32), am.ATTN_ERR_INVALID),
        (dict(maxp=(1 << 22) // 64 + 1), am.ATTN_ERR_UNSUPPORTED),  # reach above the longest sequence
        (dict(maxl=(1 << 22) + 1), am.ATTN_ERR_UNSUPPORTED),
        (dict(sl=NUL), am.ATTN_ERR_INVALID),
        (dict(bt=NUL), am.ATTN_ERR_INVALID),
        (dict(k=NUL), am.ATTN_ERR_INVALID),
        (dict(pages=0), am.ATTN_ERR_INVALID),
        (dict(maxp=0), am.ATTN_ERR_INVALID),
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(Hq=30), am.ATTN_ERR_INVALID),
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
        (dict(splits=-1), am.ATTN_ERR_INVALID),
        (dict(splits=4, ws=NUL), am.ATTN_ERR_WORKSPACE),
        (dict(splits=4, ws_bytes=16), am.ATTN_ERR_WORKSPACE),
    ],
)
def test_decode_paged_rejects(kw, code):
    assert decp(**kw) == code
    assert decp(fn="attn_decode_paged_fused", **kw) == code


@no_gpu
def test_decode_paged_fused_workspace_rules():
    B, Hq, Hkv, L, d = 4, 32, 8, 1280, 128
    need = am.decode_paged_fused_workspace_bytes(B, Hq, Hkv, L, d, 4)
    # the arrival counts (64 KiB) come first, then four chunks' partial states
    assert need == 65536 + am.decode_workspace_bytes(B, Hq, Hkv, L, d, 4)
    f = dict(fn="attn_decode_paged_fused", splits=4)
    assert decp(ws_bytes=need - 1, **f) == am.ATTN_ERR_WORKSPACE
    assert decp(ws=ctypes.c_void_p(0x1002), ws_bytes=need, **f) == am.ATTN_ERR_INVALID   # not 4-byte aligned
    assert decp(B=2049, Hkv=8, Hq=8, maxl=L, ws_bytes=1 << 40, **f) == am.ATTN_ERR_UNSUPPORTED  # > 16384 counts
    assert am.decode_paged_fused_workspace_bytes(B, Hq, Hkv, L, d, 1) == 0
    assert am.decode_paged_fused_workspace_bytes(48, Hq, Hkv, 4096, d, 0) == 0   # one chunk at 48 streams


@no_gpu
def test_decode_paged_empty_batch_launches_nothing():
    assert decp(q=NUL, k=NUL, v=NUL, bt=NUL, sl=NUL, o=NUL, lse=NUL, B=0) == am.ATTN_OK


def dec8(q=P, k=P, v=P, ks=P, vs=P, o=P, lse=P, B=2, Hq=32, Hkv=8, Nq=1, Nk=4096, d=128, scale=0.088, splits=0,
         ws=P, ws_bytes=1 << 30):
    return am.lib().attn_decode_splitkv_fp8(q, k, v, ks, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, splits, ws,
                                            ws_bytes, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(Nq=2), am.ATTN_ERR_INVALID),
        (dict(splits=-1), am.ATTN_ERR_INVALID),
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(k=NUL), am.ATTN_ERR_INVALID),
        (dict(ks=NUL), am.ATTN_ERR_INVALID),
        (dict(vs=NUL), am.ATTN_ERR_INVALID),
        (dict(scale=0.0), am.ATTN_ERR_INVALID),
        (dict(Hq=30), am.ATTN_ERR_INVALID),
        (dict(Hq=64, Hkv=1), am.ATTN_ERR_UNSUPPORTED),
        (dict(ws=NUL), am.ATTN_ERR_WORKSPACE),
        (dict(ws_bytes=16), am.ATTN_ERR_WORKSPACE),
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
    ],
)
def test_decode_fp8_rejects(kw, code):
    assert dec8(**kw) == code


@no_gpu
def test_decode_fp8_empty_launches_nothing():
    assert dec8(q=NUL, k=NUL, v=NUL, ks=NUL, vs=NUL, o=NUL, lse=NUL, B=0) == am.ATTN_OK
    assert dec8(q=NUL, k=NUL, v=NUL, ks=NUL, vs=NUL, o=NUL, lse=NUL, Nq=0) == am.ATTN_OK


def test_split_plan_and_workspace():
    n = am.decode_num_splits
    # grouped-query decode at 32 q / 8 kv heads, d = 128
    for B, L in [(1, 512), (1, 4096), (16, 4096), (48, 2048), (48, 4096)]:
        s = n(B, 32, 8, L, 128)
        assert 1 <= s <= max(1, L // 32)
        ws = am.decode_workspace_bytes(B, 32, 8, L, 128, 0)
        # enough for this plan (and the FP8 entry point's, which may split more)
        assert ws >= (0 if s == 1 else B * 32 * s * (128 + 2) * 4)
        assert am.decode_workspace_bytes(B, 32, 8, L, 128, 1) == 0
    # the cost model: from 20 streams x 8 kv heads up the cache is streamed by
    # enough workgroups without splitting, 16 streams of 4096 keys take two
    # chunks; one stream splits into 8..32 chunks of its 4096 keys; plans are
    # powers of two; the single-launch path, with no merge launch to pay for,
    # splits at least as much
    assert n(48, 32, 8, 4096, 128) == 1 and n(20, 32, 8, 4096, 128) == 1 and n(48, 32, 8, 512, 128) == 1
    assert n(16, 32, 8, 4096, 128) == 2
    assert 8 <= n(1, 32, 8, 4096, 128) <= 32
    for B in (1, 2, 4, 8, 16, 48):
        for L in (1, 100, 512, 1024, 2048, 4096, 32768):
            s, f = n(B, 32, 8, L, 128), am.decode_fused_num_splits(B, 32, 8, L, 128)
            assert s & (s - 1) == 0 and f & (f - 1) == 0 and 1 <= s <= f <= 64
    # explicit split counts are honoured up to one split per 32-key tile
    assert am.decode_workspace_bytes(1, 4, 1, 100, 64, 7) == am.decode_workspace_bytes(1, 4, 1, 100, 64, 4)
    assert am.decode_workspace_bytes(1, 4, 1, 0, 64, 0) == 0
    assert am.bwd_workspace_bytes(4, 16, 2048, 128) >= 4 * 16 * 2048 * 4


def bwd(ws=P, ws_bytes=1 << 30, dt=am.ATTN_BF16, d=128, lse=P, Hq=4, Hkv=2, dq=P, fn="attn_bwd"):
    return getattr(am.lib(), fn)(P, P, P, P, P, lse, dq, P, P, 1, Hq, Hkv, 64, 64, d, 0.1, 1, ws, ws_bytes, dt, None)


@no_gpu
@pytest.mark.parametrize("fn", ["attn_bwd", "attn_bwd_bf16_grads"])
def test_bwd_rejects(fn):
    assert bwd(ws=NUL, fn=fn) == am.ATTN_ERR_WORKSPACE
    assert bwd(ws_bytes=4, fn=fn) == am.ATTN_ERR_WORKSPACE
    assert bwd(dt=am.ATTN_F32, fn=fn) == am.ATTN_ERR_UNSUPPORTED
    assert bwd(d=32, fn=fn) == am.ATTN_ERR_UNSUPPORTED
    assert bwd(lse=NUL, fn=fn) == am.ATTN_ERR_INVALID
    assert bwd(dq=NUL, fn=fn) == am.ATTN_ERR_INVALID
    assert bwd(Hq=3, fn=fn) == am.ATTN_ERR_INVALID
    # a key grid of 2^37 dK/dV workgroups (B * Hkv * Nk / 32), a query grid the common check accepts
    big = getattr(am.lib(), fn)(P, P, P, P, P, P, P, P, P, 1 << 10, 1 << 10, 1 << 10, 1, 1 << 22, 128, 0.1, 1, P,
                                1 << 40, am.ATTN_BF16, None)
    assert big == am.ATTN_ERR_UNSUPPORTED


def test_bwd_binding_refuses_other_gradient_dtypes():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="grad_dtype"):
        am.attn_bwd(q, q, q, q, q, torch.zeros(1, 1, 4), grad_dtype=torch.float16)


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        am.attn_fwd(q, q, q)


def test_binding_rejects_mis_sized_caller_buffers():
    # caller-supplied outputs and inputs must match the shape and dtype the
    # call uses: a wrong one is refused before any address reaches the library
    import torch

    am._want(None, (2, 3), torch.float32, "x")
    am._want(torch.empty(2, 3), (2, 3), torch.float32, "x")
    with pytest.raises(ValueError):
        am._want(torch.empty(2, 4), (2, 3), torch.float32, "x")
    with pytest.raises(TypeError):
        am._want(torch.empty(2, 3, dtype=torch.bfloat16), (2, 3), torch.float32, "x")


def decn(q=P, k=P, v=P, o=P, lse=P, B=2, Hq=32, Hkv=8, Nq=1, Nk=4096, d=128, scale=0.088, splits=0,
         dt=am.ATTN_BF16):
    return am.lib().attn_decode_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, 0, splits, dt, None)


@no_gpu
@pytest.mark.parametrize(
    "kw,code",
    [
        (dict(Nq=2), am.ATTN_ERR_INVALID),
        (dict(splits=-1), am.ATTN_ERR_INVALID),
        (dict(q=NUL), am.ATTN_ERR_INVALID),
        (dict(dt=am.ATTN_F32), am.ATTN_ERR_UNSUPPORTED),
        (dict(d=80), am.ATTN_ERR_UNSUPPORTED),
        # 16 x 32 rows x 64 chunks of partial states (~17 MB) exceed the fixed scratch
        (dict(B=16, splits=64), am.ATTN_ERR_SCRATCH),
    ],
)
def test_decode_noalloc_rejects(kw, code):
    assert decn(**kw) == code


def test_decode_noalloc_scratch_sizes():
    # the scratch holds what the two-launch decode's workspace would, and the
    # size check matches the header's bound
    for args in ((1, 32, 8, 4096, 128, 0), (3, 32, 8, 3000, 128, 5), (16, 32, 8, 4096, 128, 64)):
        assert am.decode_noalloc_scratch_bytes(*args) <= am.decode_workspace_bytes(*args)
    assert am.decode_noalloc_scratch_bytes(16, 32, 8, 4096, 128, 64) > am.DECODE_SCRATCH_BYTES
    assert am.decode_noalloc_scratch_bytes(48, 32, 8, 4096, 128, 0) == 0  # one chunk: no scratch read
    assert "scratch" in am.strerror(am.ATTN_ERR_SCRATCH)
