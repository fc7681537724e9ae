"""bench.py's contract and accounting, on the host: the one-GPU guard, the
metric's work formulas at the configured shapes, and the rule that a
committed HBM-counter summary is used only while the kernel sources still
hash to the value it records."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_an_unknown_path_name_is_refused_with_the_known_ones():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--paths", "fwd,decode_pagd"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "decode_pagd" in r.stderr and "decode_paged_fused" in r.stderr


def test_work_formulas_at_the_configured_shapes():
    # causal prefill at 44032 tokens, 32 query heads, d = 128: 15.88 TFLOP
    assert bench.fwd_flops(1, 32, 44032, 44032, 128, True) == pytest.approx(15.88e12, rel=1e-3)
    # causal backward at B=4 H=16 N=2048 d=128: 171.8 GFLOP (2.5x the forward's 68.7)
    assert bench.bwd_flops(4, 16, 2048, 2048, 128, True) == pytest.approx(171.8e9, rel=1e-3)
    assert bench.fwd_flops(4, 16, 2048, 2048, 128, True) == pytest.approx(68.7e9, rel=1e-3)
    # decode at 48 streams x 4096 keys, 32 q / 8 kv heads: K and V once, q, o and LSE
    assert bench.decode_bytes(48, 32, 8, 4096, 128) == 2 * 48 * 8 * 4096 * 128 * 2 + 2 * 48 * 32 * 128 * 2 + 48 * 32 * 4
    assert bench.decode_bytes(48, 32, 8, 4096, 128) == pytest.approx(805.8e6, rel=1e-3)
    # the FP8 cache moves one byte per element
    assert bench.decode_bytes(48, 32, 8, 4096, 128, kv_bytes_per_elem=1) < 0.51 * bench.decode_bytes(48, 32, 8, 4096, 128)


def _summary(path, files, digest, traffic=123456789):
    with open(path, "w") as f:
        f.write("summary\n\n    source_files: " + " ".join(files) + "\n")
        f.write(f"    source_sha256: {digest}\n    traffic_bytes_per_launch: {traffic}\n")


def test_source_digest_follows_code_not_comments(tmp_path):
    src = "// header comment\n__global__ void k(int* p) {  /* block\ncomment */\n  p[0] = 1;  // store\n}\n"
    (tmp_path / "a.hip").write_text(src)
    d0 = bench.source_digest(["a.hip"], base=str(tmp_path))
    (tmp_path / "a.hip").write_text("// another comment\n" + src.replace("  p[0]", "\n\n    p[0]"))
    assert bench.source_digest(["a.hip"], base=str(tmp_path)) == d0
    (tmp_path / "a.hip").write_text(src.replace("p[0] = 1", "p[0] = 2"))
    assert bench.source_digest(["a.hip"], base=str(tmp_path)) != d0
    # the digest of the bare code text, written out independently
    code = "__global__ void k(int* p) { p[0] = 1; }"
    assert d0 == hashlib.sha256((code + "\n").encode()).hexdigest()
    assert bench.source_digest(["missing.hip"], base=str(tmp_path)) is None


def test_counter_summary_is_used_only_for_the_sources_it_was_taken_on(tmp_path):
    files = ["fwd_kernels.hip", "device_common.hpp", "kernels.h"]
    good = tmp_path / "good.md"
    _summary(good, files, bench.source_digest(files))
    assert bench.counted_traffic(str(good)) == 123456789
    stale = tmp_path / "stale.md"
    _summary(stale, files, "0" * 64)
    assert bench.counted_traffic(str(stale)) is None
    missing = tmp_path / "missing.md"
    _summary(missing, files + ["no_such_file.hip"], bench.source_digest(files))
    assert bench.counted_traffic(str(missing)) is None
    assert bench.counted_traffic(str(tmp_path / "absent.md")) is None
