"""Host-side checks of bench.py: the one-GPU rule, the committed traffic records, and
the algorithmic byte and flop counts the roofline figures divide by."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import moe_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("workload", sorted(bench.TRAFFIC_WORKLOADS))
def test_traffic_records_are_valid_for_the_current_kernel_sources(workload):
    """The committed record of the dominant kernel matches the kernel that the plan runs
    on that workload and the current sources (else the bench reports traffic null):
    re-record after changing any of them."""
    rec = json.load(open(bench.traffic_path(workload)))
    kind = bench.TRAFFIC_WORKLOADS[workload][2]
    assert rec["kernel"] == bench.GATEUP_KERNELS[kind][1]
    assert rec["source_sha256"] == bench.kernel_sha(workload)
    n = bench.traffic_record(workload)
    assert isinstance(n, int) and n > 0
    # the copy-probe calibration (stored rounded to 4 decimals) and the per-launch sums agree
    # with the stored total
    cp = rec["copy_probe"]
    fs, ws = cp["bytes_read"] / (cp["fetch_size_kib"] * 1024), cp["bytes_written"] / (cp["write_size_kib"] * 1024)
    assert abs(fs - cp["fetch_scale"]) < 1e-4 and abs(ws - cp["write_scale"]) < 1e-4
    total = rec["fetch_size_kib_per_launch"] * 1024 * fs + rec["write_size_kib_per_launch"] * 1024 * ws
    assert abs(n - total) <= 1e-6 * total


def test_algorithmic_work_of_a_small_layer():
    """Bytes and flops of one forward counted by hand for a 3-token bf16 layer with a
    shared expert and one dropped pair."""
    sp = S.SPECS["olmoe"].replace(d=64, E=8, k=2, ffn=32, n_shared=1, ffn_shared=16)
    idx = torch.tensor([[0, 3], [3, 5], [1, 0]], dtype=torch.int32)
    drop = torch.tensor([[0, 0], [0, 1], [0, 0]], dtype=torch.uint8)  # expert 5's pair dropped
    w = bench.alg_work(sp, 3, idx, drop)
    assert w["touched"] == 3 and w["kept"] == 5  # experts 0, 1, 3
    per_expert = 3 * 64 * 32 * 2
    shared = 3 * 64 * 16 * 2
    assert w["bytes"] == 3 * per_expert + shared + 8 * 64 * 2 + 2 * 3 * 64 * 2
    gateup = 4 * 64 * 32 * 5 + 4 * 64 * 16 * 1 * 3
    assert w["gateup_flops"] == gateup
    assert w["flops"] == 1.5 * gateup + 2 * 3 * 64 * 8
    # gate/up launch bytes: touched gate + up weights, the shared expert's, x once, h written
    assert bench.gateup_alg_bytes(sp, 3, w) == (3 * 2 * 64 * 32 + 2 * 64 * 16) * 2 + 3 * 64 * 2 + (5 * 32 + 3 * 16) * 2


def test_expert_bytes_per_weight_type():
    base = S.SPECS["olmoe"].replace(d=256, ffn=128)
    n = 3 * 256 * 128
    assert bench.expert_bytes(base) == 2 * n
    assert bench.expert_bytes(base.replace(expert="int4")) == n // 2 + (n // 128) * 2
    assert bench.expert_bytes(base.replace(expert="fp8")) == n + (2 * 128 + 256) * 4
    assert np.isclose(bench.expert_bytes(base.replace(expert="f32")), 4 * n)
