"""bench.py behaviour that needs no GPU: it refuses more than one GPU with a
JSON message, and the stored HBM traffic is only reported for the workload
and library build it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_stored_traffic_matches_workload_and_sources():
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    workload = stored["workload"]
    kernels = sorted(stored["kernels"])[:1]
    assert bench.measured_traffic(kernels, "some_other_workload") is None
    assert bench.measured_traffic(["fa::no_such_kernel<1>"], workload) is None
    got = bench.measured_traffic(kernels, workload)
    if stored.get("source_sha256") == bench.source_sha256():
        k = stored["kernels"][kernels[0]]
        assert got == pytest.approx(k["read_bytes"] + k["write_bytes"]) and got > 0
    else:
        assert got is None


def test_source_hash_ignores_the_checkout_path(tmp_path):
    """The traffic key hashes the kernel sources and flags, not the binary
    (whose bytes depend on where the library was built)."""
    import shutil
    sys.path.insert(0, ROOT)
    import bench
    for sub in ("exact_tiled_attention_27_amd/csrc", "include"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub)
    shutil.copy(os.path.join(ROOT, "exact_tiled_attention_27_amd", "build.py"),
                tmp_path / "exact_tiled_attention_27_amd" / "build.py")
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    code = "import bench; print(bench.source_sha256())"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True,
                       text=True, timeout=120, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == bench.source_sha256()


def test_roofline_kernels_are_in_the_stored_traffic():
    """The names bench.py looks up for each call of its step are the ones the
    profiler recorded (template arguments included), when the stored counters
    are for the bench's default workload."""
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    src = open(os.path.join(ROOT, "bench.py")).read()
    for pat in ('f"fa::bwd_dkdv_split_kernel<{d}, {cz}, 0, false>"',
                'f"fa::bwd_dkdv_split_kernel<{d}, {cz}, 1, false>"',
                'f"fa::bwd_dq_kernel<{d}, {cz}, false, false>"',
                'f"fa::fwd_kernel<{d}, {cz}, 0, false, false>"', 'f"fa::bwd_pre_kernel<{d}>"'):
        assert pat in src, pat
    if stored["workload"] != "fwdbwd_causal_n8192":
        pytest.skip("stored counters are for another workload")
    dkdv0 = "fa::bwd_dkdv_split_kernel<128, true, 0, false>"
    dkdv1 = "fa::bwd_dkdv_split_kernel<128, true, 1, false>"
    # The preprocess is stored per mode, under the kernel dispatched after it.
    for name in ("fa::fwd_kernel<128, true, 0, false, false>", dkdv0, dkdv1,
                 "fa::bwd_dq_kernel<128, true, false, false>",
                 f"fa::bwd_pre_kernel<128> (before {dkdv0})",
                 f"fa::bwd_pre_kernel<128> (before {dkdv1})"):
        assert name in stored["kernels"], name
    pre_det = stored["kernels"][f"fa::bwd_pre_kernel<128> (before {dkdv0})"]["write_bytes"]
    pre_atomic = stored["kernels"][f"fa::bwd_pre_kernel<128> (before {dkdv1})"]["write_bytes"]
    # Only the atomic modes' preprocess zeroes dQ (B2 Hq16 N8192 d128 fp32: 128 MiB).
    assert pre_atomic - pre_det > 120 * 2**20
