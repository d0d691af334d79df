"""bench.py's host-side contract (no GPU needed): one GPU only, and the
algorithmic work it prices the roofline with."""

from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "single GPU" in r.stderr or "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""                   # no JSON line


def test_decode_work_matches_the_mxfp4_byte_count():
    # GPT-OSS-20B-shaped decode with every expert touched: each expert's W13
    # is 2F rows of D/2 code bytes plus D/32 scale bytes, and x is 2 T D bytes
    # of bf16: 32 * 5760 * 1530 + 2 * 32 * 2880 = 282,193,920 bytes
    from synth import moe_inputs as MI
    b = _bench_module()
    cfg = MI.CONFIGS["gptoss20b_decode"]
    w = b.algorithmic_work(cfg, np.full(cfg.E, 4))
    assert w["touched"] == 32
    assert w["gateup_bytes"] == 282_193_920
    # one untouched expert removes exactly its W13 bytes
    counts = np.full(cfg.E, 4)
    counts[7] = 0
    assert b.algorithmic_work(cfg, counts)["gateup_bytes"] == 282_193_920 - 5760 * 1530
    # flops of the prefill shape: 4 D F per pair for gate/up, 6 D F per pair in all
    p = MI.CONFIGS["gptoss20b_prefill"]
    wp = b.algorithmic_work(p, np.full(p.E, 1024))
    assert wp["gateup_flops"] == 4 * 2880 * 2880 * 8192 * 4
    assert wp["step_flops"] == 6 * 2880 * 2880 * 8192 * 4


def test_traffic_summaries_are_used_only_on_the_sources_they_were_taken_on(tmp_path):
    # read_traffic accepts a committed counter summary only while its digest
    # covers the current kernel file and every device header: a change to a
    # shared header (where the kernel bodies live) makes it report null.
    import shutil
    b = _bench_module()
    root = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "mxfp4_quantized_mixture_amd", "csrc"),
                    root / "mxfp4_quantized_mixture_amd" / "csrc")
    (root / "profiles").mkdir()
    b.ROOT = str(root)
    digest = b.kernel_source_digest("expert_mlp.hip")
    (root / "profiles" / "gateup.w.traffic.txt").write_text(
        "# test summary\nkernel: k\nworkload: w\nweight_layout: packed\n"
        "kernel_source_sha256: %s\nhbm_bytes_per_dispatch: 1234\n" % digest)
    assert b.read_traffic("gateup", "w", "expert_mlp.hip", "packed") == 1234.0
    assert b.read_traffic("gateup", "w", "expert_mlp.hip", "row-major") is None
    hdr = root / "mxfp4_quantized_mixture_amd" / "csrc" / "stream_device.h"
    hdr.write_text(hdr.read_text() + "\n// changed\n")
    assert b.kernel_source_digest("expert_mlp.hip") != digest
    assert b.read_traffic("gateup", "w", "expert_mlp.hip", "packed") is None
