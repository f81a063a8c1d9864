"""bench.py's host-side contract (CPU): it refuses more than one GPU before
touching a device, and its algorithmic byte / flop accounting matches the
figures computed by hand for the tiny workload."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and res.stdout == ""


def test_accounting_of_the_tiny_workload():
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    g, _ = workloads.make_config("c1", device="cpu")
    acc = bench.workload_accounting(g)
    # seq_lens 37 and 100: 137 cache tokens of 576 bf16 values
    assert acc["kv_bytes"] == 137 * 576 * 2 == 157_824
    assert acc["q_bytes"] == 2 * 16 * 576 * 2
    assert acc["out_bytes"] == 2 * 16 * (512 * 4 + 4)
    assert acc["bt_bytes"] == (1 + 2) * 4 + 2 * 4        # live pages (1 and 2) + seq_lens
    assert acc["flops"] == 137 * 16 * 2 * (576 + 512)     # every token visible to every head (q_len 1)
    assert acc["rows"] == 32 and acc["tokens"] == 137


def test_roofline_bound_and_causal_accounting():
    """The long-context workload's accounting (q_len 2, causal: token t sees
    n - (1 - t) tokens) and the binding roof the bench reports for it (MFMA:
    484 FLOP per KV byte against a bf16 ridge of 312), against hand arithmetic."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    inp = workloads.make_decode_inputs(4, 2, 128, [131072] * 4, "bf16", seed=5, device="cpu", poison=False,
                                       extra_pages=0)
    acc = bench.workload_accounting(inp)
    assert acc["kv_bytes"] == 4 * 131072 * 1152 == 603_979_776
    assert acc["flops"] == 4 * (2 * 131072 - 1) * 128 * 2176
    roof = bench.decode_roofline(acc, "bf16", kern_ms=0.2)
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert abs(roof["achieved"] - acc["flops"] / 0.2e-3 / 1e12) < 0.1
    g, _ = workloads.make_config("c1", device="cpu")
    small = bench.decode_roofline(bench.workload_accounting(g), "bf16", kern_ms=0.01)
    assert small["bound"] == "hbm" and small["unit"] == "GB/s"
    assert bench.median([3.0, 1.0, 2.0]) == 2.0 and bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5
