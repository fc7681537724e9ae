"""Seeded synthetic inputs shared by the GPU library's tests/benchmark and the oracle.

This module holds no attention arithmetic: it draws i.i.d. standard normal
tensors from a seeded numpy generator, rounds them to bfloat16 when asked, and
picks sampled row indices.  Both sides of every comparison receive the same
bits from here.

Recipe:
  * ``numpy.random.default_rng(seed).standard_normal(shape, float32)``, drawn
    in the order the caller lists the tensors (Q, K, V, dO by convention);
  * bf16 inputs are those fp32 draws rounded to nearest-even bfloat16; the
    fp32 arrays returned then hold exactly the bf16 values.
"""
from __future__ import annotations

import numpy as np


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.  Inputs must be finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exact fp32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(seed: int, shapes, bf16: bool, scale: float = 1.0):
    """Draw tensors of the given shapes, in order, from one generator.

    Returns a list of fp32 arrays.  With ``bf16`` the values are rounded to
    bfloat16 (so each fp32 array holds exact bf16 values).  ``scale``
    multiplies the draws before rounding (used for peaked inputs).
    """
    rng = np.random.default_rng(seed)
    out = []
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if scale != 1.0:
            x = (x * np.float32(scale)).astype(np.float32)
        if bf16:
            x = bf16_bits_to_f32(round_bf16_bits(x)).reshape(shp)
        out.append(x)
    return out


def attn_inputs(seed: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, bf16: bool, with_dout: bool = False,
                scale: float = 1.0, qk_scale: float = 1.0):
    """Q [B,Hq,Nq,d], K, V [B,Hkv,Nk,d] (and dO [B,Hq,Nq,d]) drawn in that order.

    ``scale`` multiplies every tensor; ``qk_scale`` multiplies Q and K only
    (before rounding), which sharpens the softmax without enlarging V or dO.
    """
    shapes = [(B, Hq, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d)]
    if with_dout:
        shapes.append((B, Hq, Nq, d))
    out = normal(seed, shapes, False, scale)
    if qk_scale != 1.0:
        out[0] = (out[0] * np.float32(qk_scale)).astype(np.float32)
        out[1] = (out[1] * np.float32(qk_scale)).astype(np.float32)
    if bf16:
        out = [bf16_bits_to_f32(round_bf16_bits(x)).reshape(x.shape) for x in out]
    return out


def sample_rows(seed: int, n: int, B: int, Hq: int, Nq: int, forced_i=()) -> np.ndarray:
    """n distinct (b, h, i) triples from a generator separate from the data's.

    The positions in ``forced_i`` come first (each at a random b, h); the rest
    are uniform.  Returns int64 [n, 3].
    """
    rng = np.random.default_rng(seed)
    seen = set()
    rows = []
    for i in forced_i:
        if 0 <= i < Nq:
            t = (int(rng.integers(B)), int(rng.integers(Hq)), int(i))
            if t not in seen:
                seen.add(t)
                rows.append(t)
    while len(rows) < n:
        t = (int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Nq)))
        if t not in seen:
            seen.add(t)
            rows.append(t)
    return np.array(rows[:n], np.int64)


def offsets(lengths) -> np.ndarray:
    """Row offsets of a packed batch: int32 [n + 1], 0 then the running sums."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, np.int64))]).astype(np.int32)


def varlen_inputs(seed: int, lens_q, lens_k, Hq: int, Hkv: int, d: int, bf16: bool):
    """Packed variable-length batch: Q [Hq, sum(lens_q), d], K, V [Hkv, sum(lens_k), d]
    drawn in that order, and the int32 offsets cu_q, cu_k."""
    cu_q, cu_k = offsets(lens_q), offsets(lens_k)
    q, k, v = normal(seed, [(Hq, int(cu_q[-1]), d), (Hkv, int(cu_k[-1]), d), (Hkv, int(cu_k[-1]), d)], bf16)
    return q, k, v, cu_q, cu_k


def chunked_prefill_lengths(seed: int, n: int, lq_range, history_range):
    """Lengths of n sequences that append lq new tokens to a history of h
    cached ones: lens_q = lq, lens_k = h + lq, each uniform in its range
    (inclusive) from a generator separate from the data's."""
    rng = np.random.default_rng(seed)
    lq = rng.integers(lq_range[0], lq_range[1] + 1, size=n)
    h = rng.integers(history_range[0], history_range[1] + 1, size=n)
    return [int(x) for x in lq], [int(x + y) for x, y in zip(h, lq)]


def quantize_e4m3(x: np.ndarray, scale: float) -> np.ndarray:
    """x / scale to the nearest OCP FP8 E4M3 code (ties to the even code),
    saturating at +-448; uint8 codes of x's shape.  Test-input encoding only.
    E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    holds the subnormals m 2^-9.  Normal values round the fp32 significand to
    3 bits (round to nearest even on the bits dropped) and rebias the
    exponent; values below 2^-6 round to the nearest multiple of 2^-9."""
    x = np.asarray(x, np.float32)
    y = np.minimum(np.abs(x) * np.float32(1.0 / float(scale)), np.float32(448.0))
    bits = y.view(np.int32)
    r = (bits + 0x7FFFF + ((bits >> 20) & 1)) >> 20      # exponent and 3 rounded mantissa bits
    code = r - (120 << 3)                                  # fp32 bias 127 -> E4M3 bias 7
    small = y < np.float32(2.0 ** -6)
    code[small] = np.rint(y[small] * np.float32(512.0)).astype(np.int32)
    np.minimum(code, 0x7E, out=code)
    code[(x < 0) & (code > 0)] |= 0x80
    return code.astype(np.uint8)


def fp8_kv_inputs(seed: int, B: int, Hq: int, Hkv: int, Nk: int, d: int):
    """Decode inputs with an FP8 cache: q bf16-exact [B,Hq,1,d] (fp32 array),
    K, V codes uint8 [B,Hkv,Nk,d] and per-kv-head scales (max |x| / 448 over the
    head, as an fp32 value), drawn as attn_inputs(seed, ...) draws them."""
    q, k, v = attn_inputs(seed, B, Hq, Hkv, 1, Nk, d, bf16=False)
    q = bf16_bits_to_f32(round_bf16_bits(q)).reshape(q.shape)
    ks = np.array([max(float(np.abs(k[:, h]).max()), 1e-30) / 448.0 for h in range(Hkv)], np.float32)
    vs = np.array([max(float(np.abs(v[:, h]).max()), 1e-30) / 448.0 for h in range(Hkv)], np.float32)
    k8 = np.stack([quantize_e4m3(k[:, h], ks[h]) for h in range(Hkv)], axis=1)
    v8 = np.stack([quantize_e4m3(v[:, h], vs[h]) for h in range(Hkv)], axis=1)
    return q, k8, v8, ks, vs


def paged_kv_inputs(seed: int, lens, Hq: int, Hkv: int, page: int, d: int, spare_pages: int = 3):
    """Decode inputs over a paged cache: q bf16-exact [B,Hq,1,d] and a cache
    K, V [num_pages, Hkv, page, d] drawn as normal(seed, ...) draws them (q,
    K, V), a block table int32 [B, max_pages] that gives each stream
    ceil(len / page) distinct pages in a random order (from a generator
    separate from the data's; entries past a stream's pages are -1), the
    int32 lengths, and used [num_pages, page]: True where a slot holds one of
    some stream's keys (callers may poison the rest)."""
    lens = [int(x) for x in lens]
    need = [(n + page - 1) // page for n in lens]
    num_pages = sum(need) + spare_pages
    max_pages = max(1, max(need) if need else 1)
    q, kc, vc = normal(seed, [(len(lens), Hq, 1, d), (num_pages, Hkv, page, d), (num_pages, Hkv, page, d)], True)
    rng = np.random.default_rng(seed + 7919)
    perm = rng.permutation(num_pages)
    table = np.full((len(lens), max_pages), -1, np.int32)
    used = np.zeros((num_pages, page), bool)
    at = 0
    for b, (n, m) in enumerate(zip(lens, need)):
        table[b, :m] = perm[at:at + m]
        for j in range(m):
            used[perm[at + j], :min(page, n - j * page)] = True
        at += m
    return q, kc, vc, table, np.asarray(lens, np.int32), used


def paged_varlen_inputs(seed: int, lens_q, lens_k, Hq: int, Hkv: int, page: int, d: int, spare_pages: int = 3):
    """Packed queries q [Hq, sum(lens_q), d] (bf16-exact) with int32 offsets
    cu_q, and a paged cache as paged_kv_inputs gives it for lens_k (K, V
    [num_pages, Hkv, page, d], block table, int32 lengths, used slots)."""
    _, kc, vc, table, lens, used = paged_kv_inputs(seed, lens_k, Hq, Hkv, page, d, spare_pages)
    cu_q = offsets(lens_q)
    (q,) = normal(seed + 104729, [(Hq, int(cu_q[-1]), d)], True)
    return q, kc, vc, table, cu_q, lens, used
