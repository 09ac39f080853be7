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


def test_stored_traffic_matches_workload_and_build():
    sys.path.insert(0, ROOT)
    import bench
    kernels = ["fa::fwd_kernel<128, false, 0, false, false>"]
    assert bench.measured_traffic(kernels, "some_other_workload") is None
    assert bench.measured_traffic(["fa::no_such_kernel<1>"], "fwd_n4096") is None
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    got = bench.measured_traffic(kernels, "fwd_n4096")
    if stored["library_sha256"] == bench.library_sha256():
        k = stored["kernels"][kernels[0]]
        assert got == pytest.approx(k["read_bytes"] + k["write_bytes"]) and got > 0
    else:
        assert got is None


def test_roofline_kernels_are_in_the_stored_traffic():
    """The names bench.py looks up for the dominant call are the ones the
    profiler recorded for the current build (template arguments included)."""
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    for name in ("fa::fwd_kernel<128, false, 0, false, false>", "fa::bwd_pre_kernel<128>",
                 "fa::bwd_dkdv_split_kernel<128, false, 0, false>",
                 "fa::bwd_dq_kernel<128, false, false>"):
        assert name in stored["kernels"], name
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'f"fa::bwd_dkdv_split_kernel<{d}, {cz}, 0, false>"' in src
    assert 'f"fa::bwd_dq_kernel<{d}, {cz}, false>"' in src
    assert 'f"fa::fwd_kernel<{d}, {cz}, 0, false, false>"' in src
