"""Host logic of bench.py: the per-step byte model and the oracle CPU
baseline in every storage format (tiny sizes; no GPU)."""
import numpy as np
import pytest

import bench
import synth


def test_step_bytes_entry_sizes():
    w = synth.WORKLOADS["decode_64k_b32"]
    # a gathered entry: 288 code bytes + 9 fp32 scales (group 64) ...
    a = bench.step_bytes(w, 32768.0)
    assert a["gather"] == 1 * 32 * 512 * (288 + 36)
    # ... or 36 E8M0 bytes (16 channels), with value planes 256 + 32 more
    m = bench.step_bytes(synth.scaled(w, k_group=16, v_group=16), 32768.0, mx16=True)
    assert m["gather"] == 1 * 32 * 512 * (288 + 36 + 256 + 32)
    # indexer keys: 256 B bf16, 64 + 8 B in FP4; window rows 1152 B bf16, 576 B FP8
    f = bench.step_bytes(w, 32768.0, idx_fp4=True, swa_fp8=True)
    assert a["indexer_keys"] == 32 * 32768 * 256 and f["indexer_keys"] == 32 * 32768 * 72
    assert a["window"] == 2 * f["window"] == 32 * 128 * 1152
    assert a["total"] == sum(v for k, v in a.items() if k != "total")


def test_scans_per_step_with_pool():
    w = synth.WORKLOADS["group_128k_b64"]
    assert bench.scans_per_step(w, None) == (2, 0)
    assert bench.scans_per_step(w, (2048, 8)) == (1, 1)


@pytest.mark.parametrize("fmt", [(0, 0, 0), (1, 1, 1)])
def test_cpu_baseline_runs_every_format(fmt):
    idx_format, swa_format, k_format = fmt
    w = synth.scaled(synth.WORKLOADS["decode_64k_b32"], batch=2, entries=700,
                     k_group=16 if k_format else 64)
    r = bench.cpu_baseline(synth, w, 0, 0.01, None, idx_format, swa_format, k_format)
    assert r["kind"] == "oracle" and r["unit"] == "steps/s" and np.isfinite(r["value"]) and r["value"] > 0
    assert r["cores"] >= 1


def test_cpu_baseline_prefill_workload():
    """The tiny workload's cache is built from prefill tokens through the
    compressor on the oracle side too (an odd count leaves one pending)."""
    w = synth.scaled(synth.WORKLOADS["tiny_t4096"], prefill_tokens=301, entries=151)
    r = bench.cpu_baseline(synth, w, 0, 0.01)
    assert r["kind"] == "oracle" and np.isfinite(r["value"]) and r["value"] > 0


def test_more_than_one_gpu_is_refused():
    import subprocess
    import sys
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=60)
    assert p.returncode == 2 and "one GPU" in p.stderr
