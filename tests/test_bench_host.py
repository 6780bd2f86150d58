"""Host-side checks of bench.py (no GPU): the refusal of more than one GPU, the algorithmic byte
model against the formulas written out independently, and the counter summary's calibration
arithmetic on a synthetic rocprofv3 counter file."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


@pytest.mark.parametrize("n,m,k,wb", [(2, 4, 6, 2), (1, 4, 4, 2), (2, 8, 28, 2), (4, 8, 70, 2), (2, 4, 6, 4)])
def test_byte_model(n, m, k, wb):
    """Per weight: the forward reads w and K/m logits and writes w_masked; the backward also reads
    the upstream gradient and writes K/m logit gradients; pack reads w and the logits and writes
    n/m values plus n fields of ceil(log2 m) bits per m weights; unpack reverses the last."""
    b = bench.bytes_per_weight(wb, n, m, k)
    bits = 2 if m == 4 else 3
    assert b["fwd"] == pytest.approx(wb + 4 * k / m + wb)
    assert b["bwd"] == pytest.approx(wb + wb + 4 * k / m + 4 * k / m)
    assert b["harden_pack"] == pytest.approx(wb + 4 * k / m + wb * n / m + n * bits / 8 / m)
    assert b["unpack"] == pytest.approx(wb * n / m + n * bits / 8 / m + wb)
    if (n, m, wb) == (2, 4, 2):  # the numbers quoted for the LLaMA-7B-shaped layer
        assert (b["fwd"], b["bwd"], b["harden_pack"], b["unpack"]) == (10, 16, 9.125, 3.125)


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, kib in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_counter_summary_divides_by_the_copy_calibration(tmp_path):
    gib_kib = (1 << 30) / 1024
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    bwd = "void nm::" + bench.KERNELS["bwd"] + "(nm::BwdArgs)"
    # the counter reads half of the copied bytes for fetches and all of them for writes
    _counter_csv(fetch, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib * 0.5)] * 4 +
                 [(bwd, 100.0), (bwd, 300.0), ("__amd_rocclr_copyBuffer", 1.0)])
    _counter_csv(write, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib)] * 4 + [(bwd, 50.0)])
    res = bench.summarize_pmc(str(fetch), str(write))
    assert res["bwd"]["FETCH_SIZE"]["copy_scale"] == 0.5
    assert res["bwd"]["FETCH_SIZE"]["bytes_per_dispatch"] == pytest.approx(200.0 * 1024 / 0.5)
    assert res["bwd"]["WRITE_SIZE"]["bytes_per_dispatch"] == pytest.approx(50.0 * 1024)
    assert set(res) == {"bwd"}


def test_stored_traffic_is_dropped_when_the_kernels_change(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "not-the-stored-hash")
    assert bench.stored_traffic("bwd") is None


def test_cpu_baseline_uses_every_available_core():
    """The oracle's CPU leg runs on all cores the process may use (affinity, capped by a cgroup
    quota when set) and reports what the host says next to it."""
    threads, host = bench.host_cores()
    assert threads >= 1
    assert host["os_cpu_count"] == os.cpu_count()
    assert threads <= host["affinity"] <= (os.cpu_count() or host["affinity"])
    if host["cgroup_cpu_quota"] is None:
        assert threads == host["affinity"]
