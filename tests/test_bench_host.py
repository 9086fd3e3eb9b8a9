"""Host-side checks of bench.py (CPU only): the multi-GPU refusal, the
algorithmic byte counts and the measured-traffic record's staleness rule."""

import json
import os
import subprocess
import sys

import bench
from rank_step_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_bytes_per_param():
    assert bench.bytes_per_param(WORKLOADS[4], True) == 42      # 8 bf16 slices + 12 + 12 + 2
    assert bench.bytes_per_param(WORKLOADS[2], False) == 40     # 4 fp32 slices + 12 + 12
    assert bench.bytes_per_param(WORKLOADS[5], True) == 30      # 1 fp32 slice + 12 + 12 + 2


def test_infinity_cache_rotation_rule():
    # the headline and 70B shards stream tens of GB per step and step one copy
    # of the state; the Llama block and the 128 MiB unit fit within a few
    # Infinity Caches and rotate through enough copies that at least
    # ROTATE_BYTES of other traffic passes between two steps on one copy
    local = {4: 842_301_952, 5: 2_204_803_328, 3: 25_297_920, 2: 8_388_608}
    for cfg, rotated in ((4, False), (5, False), (3, True), (2, True)):
        w = WORKLOADS[cfg]
        step_bytes = bench.bytes_per_param(w, w.bf16_out) * local[cfg]
        assert (step_bytes < bench.ROTATE_BYTES) == rotated, cfg
        if rotated:
            n = -(-bench.ROTATE_BYTES // step_bytes) + 1
            assert n <= bench.MAX_COPIES and (n - 1) * step_bytes >= bench.ROTATE_BYTES
    assert bench.ROTATE_BYTES >= 4 * bench.INFINITY_CACHE_BYTES


def test_traffic_record_is_tied_to_the_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_hash": bench.kernel_source_hash(), "total_numel": 123,
           "bytes_per_launch": 4567}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [os.path.join(ROOT, s) for s in bench.KERNEL_SOURCES])
    assert bench.measured_traffic("x", 123) == 4567
    assert bench.measured_traffic("x", 124) is None              # another workload size
    rec["kernel_source_hash"] = "0" * 16                        # taken on another kernel
    (tmp_path / "profiles" / "traffic_x.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("x", 123) is None
    assert bench.measured_traffic("missing", 123) is None


def test_committed_traffic_record_matches_the_current_kernels():
    """The counters in profiles/ were taken on the kernels as they stand: a
    kernel change without a new counter run would leave the bench's
    roofline traffic empty."""
    rec = bench.measured_traffic("llama7b_full_n8", 842_301_952)
    assert rec is not None, "profiles/traffic_llama7b_full_n8.json is stale: re-run the counters"
    assert 1.0 <= rec / (42 * 842_301_952) < 1.05     # FETCH+WRITE within 5 % of the algorithmic bytes
