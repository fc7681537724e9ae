"""Benchmark of the fused-attention hot path on one MI355X.

One step is one pass over every path of the hot path, each at the shape its
throughput target is stated for:
  prefill   causal forward, B=1, Hq=32, Hkv=8, N=44032, d=128 (bf16 in, fp32 accumulate)
  decode    split-KV decode, 48 streams, 32 q / 8 kv heads, d=128, 4096 keys each
  backward  causal backward from the saved LSE, B=4, H=16, N=2048, d=128 (fp32 grads)
Inputs are seeded synthetic N(0,1) tensors rounded to bf16 and are resident in
HBM before the timed region.  The backward's O and LSE come from a forward run
outside the timed region.

value    = algorithmic attention TFLOP/s of the whole step
           (fwd 4*B*Hq*Nq*Nk*d, bwd 10*B*Hq*Nq*Nk*d, both halved when causal;
            decode 4*B*Hq*Nk*d)
paths    = per-path time, TFLOP/s or GB/s, and fraction of the MI355X roofline
roofline = the prefill forward kernel (the step's dominant kernel) against the
           dense bf16 MFMA peak, timed with HIP events on its own stream
cpu_baseline = the CPU oracle on a bounded sample of the same step's work

Opt-in paths (not part of the default step): varlen = chunked prefill of a
packed batch of 16 sequences (attn_fwd_varlen); decode_fp8 = the decode shape
over an FP8 E4M3 KV cache (attn_decode_splitkv_fp8); decode_fused = the decode
shape in one launch (attn_decode_splitkv_fused, the last split merges);
decode_paged = 48 streams of 512..4096 keys each (seeded) in a paged cache of
64-key pages through a block table (attn_decode_paged); decode_paged_fused =
the same paged batch in one launch (attn_decode_paged_fused); varlen_paged = the
varlen batch with each sequence's keys in 64-key pages of a shuffled cache
(attn_fwd_varlen_paged).

--sweep times every point the targets are stated for instead (forward causal
N = 2048..44032 at 32 q / 8 kv heads and at B=4 H=16 N=2048, the backward, and
the backward also with bf16 gradients, and the decode at 1/16/48 streams x
512..4096 keys with both decode entry points),
one JSON line per point with median / p10 / p90 / min over >= 50 calls, inputs
rotating over copies of >= 512 MiB so that no call finds them in the MALL.

Usage: python bench.py [--steps K] [--warmup W] [--no-cpu]
                       [--paths fwd,decode,bwd[,varlen][,decode_fp8][,decode_fused][,decode_paged]
                                [,decode_paged_fused][,varlen_paged]]
       python bench.py --sweep
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
METRIC = "attention fwd/bwd TFLOP/s + decode KV GB/s, as % of MI355X MFMA/HBM peak"

PREFILL = dict(B=1, Hq=32, Hkv=8, N=44032, d=128, causal=True, seed=4)
DECODE = dict(B=48, Hq=32, Hkv=8, L=4096, d=128, seed=3000 + 100 * 48 + 3)
BACKWARD = dict(B=4, H=16, N=2048, d=128, causal=True, seed=5)
# opt-in path (--paths ...,varlen): chunked prefill of 16 sequences, each
# appending 512..2048 new tokens to a cached history of 0..4096 tokens
VARLEN = dict(n=16, lq=(512, 2048), hist=(0, 4096), Hq=32, Hkv=8, d=128, seed=6, len_seed=7)
# every path --paths may name, in the order a step runs them
PATH_NAMES = ("fwd", "decode", "bwd", "decode_fp8", "decode_fused", "decode_paged", "decode_paged_fused", "varlen",
              "varlen_paged")

# opt-in path (--paths ...,decode_paged): 48 streams of unequal length in 64-key pages
PAGED = dict(B=48, Hq=32, Hkv=8, lens=(512, 4096), page=64, d=128, seed=9, len_seed=10)


CSRC = os.path.join(ROOT, "attention_online_softmax_attn_amd", "csrc")
FWD_COUNTERS = os.path.join(ROOT, "profiles", "fwd_bf16_prefill_n44032_hbm_counters.md")


def source_digest(names, base=CSRC):
    """SHA-256 of the named kernel sources with comments and white space
    removed, so that a change of code, not of commentary, retires counters
    taken on the earlier code; None if a file is missing."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in names:
        try:
            text = open(os.path.join(base, name), encoding="utf-8").read()
        except OSError:
            return None
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update((" ".join(text.split()) + "\n").encode())
    return h.hexdigest()


def counted_traffic(summary_path):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel code has changed since the counters were taken."""
    try:
        text = open(summary_path).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip()
        for key in ("source_files:", "source_sha256:", "traffic_bytes_per_launch:"):
            if line.startswith(key):
                fields[key[:-1]] = line[len(key):].strip()
    if len(fields) != 3:
        return None
    if source_digest(fields["source_files"].split()) != fields["source_sha256"]:
        return None
    return int(fields["traffic_bytes_per_launch"])


def fwd_flops(B, Hq, Nq, Nk, d, causal):
    return 4.0 * B * Hq * Nq * Nk * d * (0.5 if causal else 1.0)


def bwd_flops(B, Hq, Nq, Nk, d, causal):
    return 10.0 * B * Hq * Nq * Nk * d * (0.5 if causal else 1.0)


def varlen_flops(lens_q, lens_k, Hq, d):
    """4 d flop per visible (query, key) pair, causal per sequence (bottom-right)."""
    pairs = 0
    for lq, lk in zip(lens_q, lens_k):
        off = lk - lq
        pairs += sum(max(0, min(lk, i + off + 1)) for i in range(lq))
    return 4.0 * Hq * d * pairs


def decode_bytes(B, Hq, Hkv, L, d, kv_bytes_per_elem=2):
    return 2.0 * B * Hkv * L * d * kv_bytes_per_elem + 2.0 * B * Hq * d * 2 + B * Hq * 4


def decode_flops(B, Hq, L, d):
    return 4.0 * B * Hq * L * d


def to_dev(x):
    import numpy as np
    import torch

    import synth

    bits = synth.round_bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16).reshape(x.shape)).view(torch.bfloat16).cuda()


def setup(paths):
    import synth

    st = {}
    if "fwd" in paths:
        c = PREFILL
        q, k, v = synth.attn_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["N"], c["d"], bf16=True)
        st["fwd_host"] = (q, k, v)
        st["fwd"] = (to_dev(q), to_dev(k), to_dev(v))
    if "decode" in paths:
        c = DECODE
        q, k, v = synth.attn_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], 1, c["L"], c["d"], bf16=True)
        st["decode_host"] = (q, k, v)
        st["decode"] = (to_dev(q), to_dev(k), to_dev(v))
    if "decode_fused" in paths:
        c = DECODE
        q, k, v = synth.attn_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], 1, c["L"], c["d"], bf16=True)
        st["decode_fused"] = (to_dev(q), to_dev(k), to_dev(v))
    if "bwd" in paths:
        c = BACKWARD
        q, k, v, do = synth.attn_inputs(c["seed"], c["B"], c["H"], c["H"], c["N"], c["N"], c["d"], bf16=True,
                                        with_dout=True)
        st["bwd_host"] = (q, k, v, do)
        st["bwd"] = (to_dev(q), to_dev(k), to_dev(v), to_dev(do))
    if "decode_fp8" in paths:
        import torch

        c = DECODE
        q, k8, v8, ks, vs = synth.fp8_kv_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["L"], c["d"])
        st["decode_fp8"] = (to_dev(q), torch.from_numpy(k8).cuda(), torch.from_numpy(v8).cuda(),
                            torch.from_numpy(ks).cuda(), torch.from_numpy(vs).cuda())
    if "decode_paged" in paths or "decode_paged_fused" in paths:
        import numpy as np
        import torch

        c = PAGED
        lens = np.random.default_rng(c["len_seed"]).integers(c["lens"][0], c["lens"][1] + 1, size=c["B"])
        q, kc, vc, table, lens_a, _ = synth.paged_kv_inputs(c["seed"], lens, c["Hq"], c["Hkv"], c["page"], c["d"])
        st["decode_paged"] = (to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(table).cuda(),
                              torch.from_numpy(lens_a).cuda(), int(lens_a.max()))
        st["decode_paged_lens"] = [int(x) for x in lens_a]
    if "varlen_paged" in paths:
        import torch

        c = VARLEN
        lens_q, lens_k = synth.chunked_prefill_lengths(c["len_seed"], c["n"], c["lq"], c["hist"])
        q, kc, vc, table, cu_q, lens, _ = synth.paged_varlen_inputs(c["seed"], lens_q, lens_k, c["Hq"], c["Hkv"],
                                                                    PAGED["page"], c["d"])
        st["varlen_paged_lens"] = (lens_q, lens_k)
        st["varlen_paged"] = (to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(table).cuda(),
                              torch.from_numpy(cu_q).cuda(), torch.from_numpy(lens).cuda(), max(lens_q), max(lens_k))
    if "varlen" in paths:
        import torch

        c = VARLEN
        lens_q, lens_k = synth.chunked_prefill_lengths(c["len_seed"], c["n"], c["lq"], c["hist"])
        q, k, v, cu_q, cu_k = synth.varlen_inputs(c["seed"], lens_q, lens_k, c["Hq"], c["Hkv"], c["d"], bf16=True)
        st["varlen_lens"] = (lens_q, lens_k)
        st["varlen"] = (to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(),
                        max(lens_q))
    return st


def _sysfs_card():
    """sysfs directory of the GPU torch uses (matched by PCI bus id), or None."""
    import glob

    import torch

    try:
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
    except Exception:
        bus = None
    cards = []
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        if not os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
            continue
        try:
            addr = os.path.basename(os.path.realpath(dev))  # e.g. 0000:05:00.0
            cards.append((int(addr.split(":")[1], 16), dev))
        except (ValueError, IndexError):
            cards.append((None, dev))
    if bus is not None:
        for b, dev in cards:
            if b == bus:
                return dev
    return cards[0][1] if len(cards) == 1 else None


class ClockSampler:
    """Samples the GPU's current shader clock (sysfs pp_dpm_sclk, the level
    marked '*') every few milliseconds while the timed steps run, so that the
    line can state the clock the kernels actually ran at."""

    def __init__(self, period_s=0.005):
        import threading

        self.dev = _sysfs_card()
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        try:
            for line in open(os.path.join(self.dev, "pp_dpm_sclk")):
                if "*" in line:
                    return float(line.split(":")[1].strip().lower().replace("*", "").replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        if self.dev is not None:
            self._t.start()
        return self

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self.dev is not None:
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return {"source": "sysfs pp_dpm_sclk, sampled every 5 ms over the timed steps", "samples": len(xs),
                "mhz_median": xs[len(xs) // 2], "mhz_min": xs[0], "mhz_max": xs[-1]}


def run_gpu(paths, steps, warmup):
    import torch

    import attention_online_softmax_attn_amd as am

    st = setup(paths)
    dev_out = {}
    # preallocated outputs and workspaces: the timed region only launches kernels
    if "fwd" in paths:
        q, k, v = st["fwd"]
        dev_out["fwd"] = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"))
    if "decode" in paths:
        q, k, v = st["decode"]
        c = DECODE
        ws = am.decode_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], 0)
        dev_out["decode"] = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"),
                             torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda"))
    if "bwd" in paths:
        q, k, v, do = st["bwd"]
        c = BACKWARD
        o, lse = am.attn_fwd(q, k, v, causal=True)
        ws = am.bwd_workspace_bytes(c["B"], c["H"], c["N"], c["d"])
        f32 = dict(dtype=torch.float32, device="cuda")
        dev_out["bwd"] = (o, lse, torch.empty(q.shape, **f32), torch.empty(k.shape, **f32), torch.empty(v.shape, **f32),
                          torch.empty(ws, dtype=torch.uint8, device="cuda"))
    if "decode_fp8" in paths:
        q = st["decode_fp8"][0]
        c = DECODE
        ws = am.decode_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], 0)
        dev_out["decode_fp8"] = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"),
                                 torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda"))
    if "decode_fused" in paths:
        q = st["decode_fused"][0]
        c = DECODE
        ws = am.decode_fused_workspace_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], 0)
        # the arrival counts start at zero; every call leaves them zero
        dev_out["decode_fused"] = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"),
                                   torch.zeros(max(ws, 1), dtype=torch.uint8, device="cuda"))
    if "decode_paged" in paths:
        q = st["decode_paged"][0]
        c = PAGED
        ws = am.decode_workspace_bytes(c["B"], c["Hq"], c["Hkv"], st["decode_paged"][5], c["d"], 0)
        dev_out["decode_paged"] = (torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"),
                                   torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda"))
    if "decode_paged_fused" in paths:
        q = st["decode_paged"][0]
        c = PAGED
        ws = am.decode_paged_fused_workspace_bytes(c["B"], c["Hq"], c["Hkv"], st["decode_paged"][5], c["d"], 0)
        # the arrival counts start at zero; every call leaves them zero
        dev_out["decode_paged_fused"] = (torch.empty_like(q),
                                         torch.empty(q.shape[:3], dtype=torch.float32, device="cuda"),
                                         torch.zeros(max(ws, 1), dtype=torch.uint8, device="cuda"))
    if "varlen" in paths:
        q = st["varlen"][0]
        dev_out["varlen"] = (torch.empty_like(q), torch.empty(q.shape[:2], dtype=torch.float32, device="cuda"))
    if "varlen_paged" in paths:
        q = st["varlen_paged"][0]
        dev_out["varlen_paged"] = (torch.empty_like(q), torch.empty(q.shape[:2], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()

    def run_path(name):
        if name == "fwd":
            q, k, v = st["fwd"]
            o, lse = dev_out["fwd"]
            am.attn_fwd(q, k, v, causal=True, out=o, lse=lse)
        elif name == "decode":
            q, k, v = st["decode"]
            o, lse, ws = dev_out["decode"]
            am.attn_decode_splitkv(q, k, v, workspace=ws, out=o, lse=lse)
        elif name == "decode_fp8":
            q, k8, v8, ks, vs = st["decode_fp8"]
            o, lse, ws = dev_out["decode_fp8"]
            am.attn_decode_splitkv_fp8(q, k8, v8, ks, vs, workspace=ws, out=o, lse=lse)
        elif name == "decode_fused":
            q, k, v = st["decode_fused"]
            o, lse, ws = dev_out["decode_fused"]
            am.attn_decode_splitkv_fused(q, k, v, workspace=ws, out=o, lse=lse)
        elif name == "decode_paged":
            q, kc, vc, bt, sl, ml = st["decode_paged"]
            o, lse, ws = dev_out["decode_paged"]
            am.attn_decode_paged(q, kc, vc, bt, sl, ml, workspace=ws, out=o, lse=lse)
        elif name == "decode_paged_fused":
            q, kc, vc, bt, sl, ml = st["decode_paged"]
            o, lse, ws = dev_out["decode_paged_fused"]
            am.attn_decode_paged_fused(q, kc, vc, bt, sl, ml, workspace=ws, out=o, lse=lse)
        elif name == "varlen":
            q, k, v, cq, ck, mq = st["varlen"]
            o, lse = dev_out["varlen"]
            am.attn_fwd_varlen(q, k, v, cq, ck, mq, causal=True, out=o, lse=lse)
        elif name == "varlen_paged":
            q, kc, vc, bt, cq, lk, mq, mk = st["varlen_paged"]
            o, lse = dev_out["varlen_paged"]
            am.attn_fwd_varlen_paged(q, kc, vc, bt, cq, lk, mq, mk, causal=True, out=o, lse=lse)
        else:
            q, k, v, do = st["bwd"]
            o, lse, dq, dk, dv, ws = dev_out["bwd"]
            am.attn_bwd(q, k, v, o, do, lse, causal=True, workspace=ws, dq=dq, dk=dk, dv=dv)

    order = [p for p in PATH_NAMES if p in paths]
    for _ in range(warmup):
        for p in order:
            run_path(p)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(order) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for s in range(steps):
            ev[s][0].record()
            for i, p in enumerate(order):
                run_path(p)
                ev[s][i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    st["sclk"] = clk.summary()
    per = {p: [] for p in order}
    for s in range(steps):
        for i, p in enumerate(order):
            per[p].append(ev[s][i].elapsed_time(ev[s][i + 1]))
    step_ms = [sum(per[p][s] for p in order) for s in range(steps)]
    return st, per, step_ms, wall


def cpu_baseline(st, paths, budget_s):
    """The oracle, as it stands, on a bounded sample of the step's work."""
    import numpy as np

    import oracle
    import synth

    flops = 0.0
    secs = 0.0
    parts = []
    fwd_rate = None
    # the oracle leg covers the default step's paths (not the opt-in varlen one)
    share = budget_s / max(1, len([p for p in paths if p in ("fwd", "decode", "bwd")]))
    if "fwd" in paths:
        c = PREFILL
        q, k, v = st["fwd_host"]
        rng_seed = 40004
        n, done_rows = 64, 0
        t_fwd = 0.0
        fwd_flops_done = 0.0
        while t_fwd < share:
            rows = synth.sample_rows(rng_seed + done_rows, n, c["B"], c["Hq"], c["N"])
            t = time.perf_counter()
            oracle.fwd_rows(q, k, v, rows, 1.0 / math.sqrt(c["d"]), True)
            t_fwd += time.perf_counter() - t
            f_rows = float(np.sum(4.0 * c["d"] * (rows[:, 2] + 1)))
            flops += f_rows
            fwd_flops_done += f_rows
            done_rows += n
            n *= 2
        secs += t_fwd
        parts.append(f"{done_rows} random query rows of the N=44032 causal prefill")
        fwd_rate = fwd_flops_done / t_fwd
    if "decode" in paths:
        c = DECODE
        q, k, v = st["decode_host"]
        t = time.perf_counter()
        oracle.fwd(q, k, v, 1.0 / math.sqrt(c["d"]), False)
        secs += time.perf_counter() - t
        flops += decode_flops(c["B"], c["Hq"], c["L"], c["d"])
        parts.append("the full 48x4096 decode")
    if "bwd" in paths:
        c = BACKWARD
        q, k, v, do = st["bwd_host"]
        nth = oracle.num_threads()
        heads = 0
        t_bwd = 0.0
        while t_bwd < share and heads < c["B"] * c["H"]:
            n = min(nth, c["B"] * c["H"] - heads)
            sel = [(h // c["H"], h % c["H"]) for h in range(heads, heads + n)]
            bs, hs = [x[0] for x in sel], [x[1] for x in sel]
            sl = lambda x: np.ascontiguousarray(x[bs, hs][:, None])
            t = time.perf_counter()
            oracle.bwd(sl(q), sl(k), sl(v), sl(do), 1.0 / math.sqrt(c["d"]), True)
            t_bwd += time.perf_counter() - t
            flops += n * bwd_flops(1, 1, c["N"], c["N"], c["d"], True)
            heads += n
        secs += t_bwd
        parts.append(f"the backward of {heads} of the 64 (batch, head) problems at N=2048")
    out = {
        "value": round(flops / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "; ".join(parts) + f" ({secs:.1f} s of fp64 CPU work)",
        "cpu_model": cpu_model(),
    }
    if fwd_rate:
        c = PREFILL
        full = fwd_flops(c["B"], c["Hq"], c["N"], c["N"], c["d"], True)
        out["prefill_full_size_s_extrapolated"] = round(full / fwd_rate, 1)
    one = single_thread_run(st, paths)
    if one is not None:
        out["single_thread"] = one
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def single_thread_run(st, paths):
    """The oracle at one OpenMP thread on the whole decode of the step (48
    streams x 4096 keys), for reference beside the all-cores figure."""
    import ctypes

    import oracle

    if "decode" not in paths:
        return None
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    c = DECODE
    q, k, v = st["decode_host"]
    nb = c["B"]
    n_all = oracle.num_threads()
    gomp.omp_set_num_threads(1)
    try:
        t = time.perf_counter()
        oracle.fwd(q[:nb], k[:nb], v[:nb], 1.0 / math.sqrt(c["d"]), False)
        secs = time.perf_counter() - t
    finally:
        gomp.omp_set_num_threads(n_all)
    f = decode_flops(nb, c["Hq"], c["L"], c["d"])
    return {"value": round(f / secs / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "sample": f"the full {nb}x{c['L']} decode at one thread ({secs:.1f} s)"}


def copy_probe(mib):
    """A plain device copy of known size: the HBM byte counters of this one
    dispatch (read and written bytes = mib MiB each) calibrate the counters
    taken on the attention kernels."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copy_probe_kib": n * 4 // 1024}), flush=True)


# --sweep: every point the throughput targets are stated for, each timed on
# its own with percentiles (fwd and bwd >= 50 % of bf16 MFMA at N >= 2048,
# decode >= 70 % of HBM where its KV cache is >= 256 MiB)
SWEEP_FWD = [(1, 32, 8, n) for n in (2048, 4096, 8192, 16384, 44032)] + [(4, 16, 16, 2048)]
# the transformer-block forward (B=4, H=8, N=512, d=64), causal and not: reported, no target
SWEEP_SMALL = [(4, 8, 8, 512, 64, True), (4, 8, 8, 512, 64, False)]
SWEEP_DECODE = [(b, n) for b in (1, 16, 48) for n in (512, 1024, 2048, 4096)]
POOL_BYTES = 512 << 20  # inputs rotate over copies of at least this size (twice the 256 MB MALL)


def time_calls(fn, n_inputs, warm=10, min_reps=50, min_ms=100.0):
    """Per-call HIP-event times of fn(i) (i selects the input copy), after warm
    untimed calls: at least min_reps calls and min_ms of GPU time.  Also the
    wall clock over the timed loop with one synchronisation."""
    import torch

    for i in range(warm):
        fn(i % n_inputs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn(0)
    e1.record()
    torch.cuda.synchronize()
    reps = max(min_reps, int(min_ms / max(e0.elapsed_time(e1), 1e-3)) + 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(reps):
        ev[r][0].record()
        fn(r % n_inputs)
        ev[r][1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / reps
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    pick = lambda f: ms[min(len(ms) - 1, int(f * len(ms)))]
    mean = sum(ms) / len(ms)
    return {"reps": reps, "ms_median": round(pick(0.5), 5), "ms_p10": round(pick(0.1), 5),
            "ms_p90": round(pick(0.9), 5), "ms_min": round(ms[0], 5), "wall_ms": round(wall, 5),
            "timers_agree": abs(wall - mean) <= 0.1 * mean + 0.01}


def sweep():
    import torch

    import attention_online_softmax_attn_amd as am

    gen = torch.Generator(device="cuda").manual_seed(8)
    rnd = lambda *shape: torch.randn(*shape, device="cuda", generator=gen).to(torch.bfloat16)
    lines = []

    def emit(d):
        lines.append(d)
        print(json.dumps(d), flush=True)

    for B, Hq, Hkv, N in SWEEP_FWD:
        d = 128
        per_copy = 2 * B * (Hq + 2 * Hkv) * N * d
        n = max(1, -(-POOL_BYTES // per_copy))
        qs = [(rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d)) for _ in range(n)]
        o = torch.empty_like(qs[0][0])
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda")
        t = time_calls(lambda i: am.attn_fwd(*qs[i], causal=True, out=o, lse=lse), n)
        f = fwd_flops(B, Hq, N, N, d, True)
        tf = f / t["ms_median"] / 1e9
        emit({"path": "fwd", "shape": f"B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal", "copies": n, **t,
              "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "target": 0.5,
              "meets": tf / PEAK_BF16_TFLOPS >= 0.5})
        del qs, o, lse
    for B, Hq, Hkv, N, d, causal in SWEEP_SMALL:
        per_copy = 2 * B * (Hq + 2 * Hkv) * N * d
        n = max(1, -(-POOL_BYTES // per_copy))
        qs = [(rnd(B, Hq, N, d), rnd(B, Hkv, N, d), rnd(B, Hkv, N, d)) for _ in range(n)]
        o = torch.empty_like(qs[0][0])
        lse = torch.empty(B, Hq, N, dtype=torch.float32, device="cuda")
        t = time_calls(lambda i: am.attn_fwd(*qs[i], causal=causal, out=o, lse=lse), n)
        f = fwd_flops(B, Hq, N, N, d, causal)
        tf = f / t["ms_median"] / 1e9
        emit({"path": "fwd", "shape": f"B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} " + ("causal" if causal else "non-causal"),
              "copies": n, **t, "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4),
              "target": None, "meets": None})
        del qs, o, lse
    # backward at B=4 H=16 N=2048 (O and LSE from the forward, outside the timing)
    c = BACKWARD
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    n = max(1, -(-POOL_BYTES // (2 * 5 * B * H * N * d)))
    sets = []
    for _ in range(n):
        q, k, v, do = rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d), rnd(B, H, N, d)
        o, lse = am.attn_fwd(q, k, v, causal=True)
        sets.append((q, k, v, o, do, lse))
    f32 = dict(dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty(B, H, N, d, **f32), torch.empty(B, H, N, d, **f32), torch.empty(B, H, N, d, **f32)
    ws = torch.empty(am.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
    t = time_calls(lambda i: am.attn_bwd(*sets[i], causal=True, workspace=ws, dq=dq, dk=dk, dv=dv), n)
    f = bwd_flops(B, H, N, N, d, True)
    tf = f / t["ms_median"] / 1e9
    emit({"path": "bwd", "shape": f"B={B} H={H} N={N} d={d} causal", "copies": n, **t, "tflops": round(tf, 1),
          "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "target": 0.5, "meets": tf / PEAK_BF16_TFLOPS >= 0.5})
    # the same backward writing bf16 gradients (attn_bwd_bf16_grads)
    g16 = dict(dtype=torch.bfloat16, device="cuda")
    dq, dk, dv = torch.empty(B, H, N, d, **g16), torch.empty(B, H, N, d, **g16), torch.empty(B, H, N, d, **g16)
    t = time_calls(lambda i: am.attn_bwd(*sets[i], causal=True, workspace=ws, dq=dq, dk=dk, dv=dv,
                                         grad_dtype=torch.bfloat16), n)
    tf = f / t["ms_median"] / 1e9
    emit({"path": "bwd_bf16_grads", "shape": f"B={B} H={H} N={N} d={d} causal", "copies": n, **t,
          "tflops": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4), "meets": None})
    del sets, dq, dk, dv
    # decode, two launches and one
    for B, L in SWEEP_DECODE:
        Hq, Hkv, d = 32, 8, 128
        kv = 2 * B * Hkv * L * d * 2
        n = max(1, -(-POOL_BYTES // kv))
        q = rnd(B, Hq, 1, d)
        kvs = [(rnd(B, Hkv, L, d), rnd(B, Hkv, L, d)) for _ in range(n)]
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, 1, dtype=torch.float32, device="cuda")
        ws2 = torch.empty(max(1, am.decode_workspace_bytes(B, Hq, Hkv, L, d, 0)), dtype=torch.uint8, device="cuda")
        ws1 = torch.zeros(max(1, am.decode_fused_workspace_bytes(B, Hq, Hkv, L, d, 0)), dtype=torch.uint8,
                          device="cuda")
        b = decode_bytes(B, Hq, Hkv, L, d)
        for name, fn in (("decode", lambda i: am.attn_decode_splitkv(q, *kvs[i], workspace=ws2, out=o, lse=lse)),
                         ("decode_fused",
                          lambda i: am.attn_decode_splitkv_fused(q, *kvs[i], workspace=ws1, out=o, lse=lse))):
            t = time_calls(fn, n)
            gbs = b / t["ms_median"] / 1e6
            bound = kv >= (256 << 20)
            emit({"path": name, "shape": f"{B} streams x {L} keys, Hq={Hq} Hkv={Hkv} d={d}",
                  "splits": am.decode_num_splits(B, Hq, Hkv, L, d), "copies": n, **t, "gbs": round(gbs, 1),
                  "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "target": 0.7 if bound else None,
                  "meets": (gbs / PEAK_HBM_GBS >= 0.7) if bound else None})
        del kvs
    met = [x["meets"] for x in lines if x["meets"] is not None]
    print(json.dumps({"sweep_points": len(lines), "targets": len(met), "targets_met": sum(met),
                      "timers_agree": all(x["timers_agree"] for x in lines)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--paths", default="fwd,decode,bwd")
    ap.add_argument("--sweep", action="store_true",
                    help="time every target point (fwd N sweep, bwd, all decode points), one JSON line each")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    paths = [p for p in args.paths.split(",") if p]
    unknown = [p for p in paths if p not in PATH_NAMES]
    if unknown:
        print(f"bench.py: unknown path(s) {', '.join(unknown)}; known: {', '.join(PATH_NAMES)}", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return
    if args.sweep:
        sweep()
        return
    st, per, step_ms, wall = run_gpu(paths, args.steps, args.warmup)

    med = lambda xs: sorted(xs)[len(xs) // 2]
    out_paths = {}
    total_flops = 0.0
    if "fwd" in paths:
        c = PREFILL
        f = fwd_flops(c["B"], c["Hq"], c["N"], c["N"], c["d"], True)
        t = sum(per["fwd"]) / len(per["fwd"])
        out_paths["prefill_fwd"] = {"ms": round(t, 4), "ms_median": round(med(per["fwd"]), 4),
                                    "tflops": round(f / t / 1e9, 2), "frac_mfma": round(f / t / 1e9 / PEAK_BF16_TFLOPS, 4),
                                    "shape": "B=1 Hq=32 Hkv=8 N=44032 d=128 causal"}
        total_flops += f
    if "decode" in paths:
        c = DECODE
        b = decode_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"])
        t = sum(per["decode"]) / len(per["decode"])
        out_paths["decode"] = {"ms": round(t, 4), "ms_median": round(med(per["decode"]), 4),
                               "gbs": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / PEAK_HBM_GBS, 4),
                               "shape": "48 streams, Hq=32 Hkv=8 d=128, 4096 keys"}
        total_flops += decode_flops(c["B"], c["Hq"], c["L"], c["d"])
    if "bwd" in paths:
        c = BACKWARD
        f = bwd_flops(c["B"], c["H"], c["N"], c["N"], c["d"], True)
        t = sum(per["bwd"]) / len(per["bwd"])
        out_paths["backward"] = {"ms": round(t, 4), "ms_median": round(med(per["bwd"]), 4),
                                 "tflops": round(f / t / 1e9, 2), "frac_mfma": round(f / t / 1e9 / PEAK_BF16_TFLOPS, 4),
                                 "shape": "B=4 H=16 N=2048 d=128 causal"}
        total_flops += f
    if "decode_fp8" in paths:
        c = DECODE
        b = decode_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"], kv_bytes_per_elem=1)
        t = sum(per["decode_fp8"]) / len(per["decode_fp8"])
        out_paths["decode_fp8"] = {"ms": round(t, 4), "ms_median": round(med(per["decode_fp8"]), 4),
                                   "gbs": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / PEAK_HBM_GBS, 4),
                                   "shape": "48 streams, Hq=32 Hkv=8 d=128, 4096 keys, FP8 E4M3 KV cache"}
        total_flops += decode_flops(c["B"], c["Hq"], c["L"], c["d"])
    if "decode_fused" in paths:
        c = DECODE
        b = decode_bytes(c["B"], c["Hq"], c["Hkv"], c["L"], c["d"])
        t = sum(per["decode_fused"]) / len(per["decode_fused"])
        out_paths["decode_fused"] = {"ms": round(t, 4), "ms_median": round(med(per["decode_fused"]), 4),
                                     "gbs": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / PEAK_HBM_GBS, 4),
                                     "shape": "48 streams, Hq=32 Hkv=8 d=128, 4096 keys, one launch"}
        total_flops += decode_flops(c["B"], c["Hq"], c["L"], c["d"])
    for name, how in (("decode_paged", ""), ("decode_paged_fused", ", one launch")):
        if name not in paths:
            continue
        c = PAGED
        lens = st["decode_paged_lens"]
        b = sum(2.0 * c["Hkv"] * n * c["d"] * 2 for n in lens) + 2.0 * c["B"] * c["Hq"] * c["d"] * 2 + c["B"] * c["Hq"] * 4
        t = sum(per[name]) / len(per[name])
        out_paths[name] = {"ms": round(t, 4), "ms_median": round(med(per[name]), 4),
                           "gbs": round(b / t / 1e6, 1), "frac_hbm": round(b / t / 1e6 / PEAK_HBM_GBS, 4),
                           "shape": f"48 streams of 512..4096 keys ({sum(lens)} in all), 64-key pages, "
                                    f"Hq=32 Hkv=8 d=128{how}"}
        total_flops += sum(decode_flops(1, c["Hq"], n, c["d"]) for n in lens)
    if "varlen" in paths:
        c = VARLEN
        lens_q, lens_k = st["varlen_lens"]
        f = varlen_flops(lens_q, lens_k, c["Hq"], c["d"])
        t = sum(per["varlen"]) / len(per["varlen"])
        out_paths["varlen_chunked_prefill"] = {
            "ms": round(t, 4), "ms_median": round(med(per["varlen"]), 4), "tflops": round(f / t / 1e9, 2),
            "frac_mfma": round(f / t / 1e9 / PEAK_BF16_TFLOPS, 4),
            "shape": f"{c['n']} sequences, new tokens {sum(lens_q)}, keys {sum(lens_k)}, Hq=32 Hkv=8 d=128, "
                     "causal per sequence"}
        total_flops += f
    if "varlen_paged" in paths:
        c = VARLEN
        lens_q, lens_k = st["varlen_paged_lens"]
        f = varlen_flops(lens_q, lens_k, c["Hq"], c["d"])
        t = sum(per["varlen_paged"]) / len(per["varlen_paged"])
        out_paths["varlen_paged_chunked_prefill"] = {
            "ms": round(t, 4), "ms_median": round(med(per["varlen_paged"]), 4), "tflops": round(f / t / 1e9, 2),
            "frac_mfma": round(f / t / 1e9 / PEAK_BF16_TFLOPS, 4),
            "shape": f"{c['n']} sequences, new tokens {sum(lens_q)}, keys {sum(lens_k)} in 64-key pages, "
                     "Hq=32 Hkv=8 d=128, causal per sequence"}
        total_flops += f
    ms_step = sum(step_ms) / len(step_ms)
    value = total_flops / ms_step / 1e9

    roofline = None
    if "fwd" in paths:
        c = PREFILL
        f = fwd_flops(c["B"], c["Hq"], c["N"], c["N"], c["d"], True)
        t = sum(per["fwd"]) / len(per["fwd"])
        ach = f / t / 1e9
        # the launcher picks the 8-wave (256-row) configuration at this size:
        # 32 heads x 172 query tiles = 5504 workgroups of 512 threads
        roofline = {"kernel": "fwd_pp_kernel<128, true, false, false> (5504 x 512)", "bound": "mfma", "achieved": round(ach, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": counted_traffic(FWD_COUNTERS)}
    sane = all(v.get("frac_mfma", 0) <= 1.0 and v.get("frac_hbm", 0) <= 1.0 for v in out_paths.values())
    wall_ms = wall * 1e3 / args.steps
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused attention hot path: causal prefill fwd N=44032 (32q/8kv) + split-KV decode "
                               "48x4096 (32q/8kv) + causal bwd B=4 H=16 N=2048", "d": 128,
                   "paths": ",".join(paths)},
        "paths": out_paths,
        "roofline": roofline,
        "timer_check": {"event_ms_per_step": round(ms_step, 4), "wall_ms_per_step": round(wall_ms, 4),
                        "agree": abs(wall_ms - ms_step) <= 0.1 * ms_step + 0.05},
        "sane": sane,
        "sclk": st.get("sclk"),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(st, paths, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
