"""Shared helpers of the GPU parity tests: host<->device transfer of the seeded
inputs (identical bits on both sides) and the max-abs comparison."""
from __future__ import annotations

import numpy as np
import torch

import synth

# Tolerances (max-abs, against the fp64 oracle)
TOL_O_F32 = 1e-4
TOL_LSE_F32 = 1e-4
TOL_O_BF16 = 2e-2
TOL_LSE_BF16 = 1e-3
TOL_GRAD = 5e-2


def dev(x: np.ndarray, bf16: bool) -> torch.Tensor:
    """Host fp32 array (holding exact bf16 values when bf16) -> contiguous GPU tensor."""
    if bf16:
        bits = synth.round_bf16_bits(x)
        assert np.array_equal(synth.bf16_bits_to_f32(bits).reshape(x.shape), x), "input is not bf16-exact"
        return torch.from_numpy(bits.view(np.int16).reshape(x.shape)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(got, expect) -> float:
    got = np.asarray(got, np.float64)
    expect = np.asarray(expect, np.float64)
    fin = np.isfinite(expect)
    assert np.array_equal(fin, np.isfinite(got)), "non-finite values differ from the oracle"
    if not fin.all():
        assert np.array_equal(got[~fin], expect[~fin]), "infinite values differ from the oracle"
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(got[fin] - expect[fin])))


def assert_close(name: str, got, expect, tol: float):
    err = max_abs(got, expect)
    assert err <= tol, f"{name}: max-abs error {err:.3e} > {tol:.1e}"
    return err


def guarded_empty(shape, dtype, sentinel=12345.0, pad=4096):
    """A buffer with guard bands: returns (view, full) where view is the
    contiguous output region inside `full`, which is filled with a sentinel."""
    n = int(np.prod(shape))
    full = torch.full((n + 2 * pad,), sentinel, dtype=dtype, device="cuda")
    return full[pad:pad + n].view(*shape), full


def guards_intact(full, n, sentinel=12345.0, pad=4096) -> bool:
    head = full[:pad]
    tail = full[pad + n:]
    return bool(torch.all(head == sentinel).item() and torch.all(tail == sentinel).item())
