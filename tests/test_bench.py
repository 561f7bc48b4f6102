"""bench.py's command line and the JSON line it prints.

The CPU tests check the refusal of more than one GPU (bench.py decides it
before it imports torch); the GPU test runs the small two-worker workload for a
few steps and checks every field of the line.
"""

import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT, flush_print

BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None, timeout=60):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH] + args, capture_output=True, text=True, env=env,
                          timeout=timeout, cwd=ROOT)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    res = _run(args, env)
    assert res.returncode != 0
    assert "one GPU only" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_json_line(gpu):
    flush_print("running bench.py --config 1 --steps 3 --warmup 1 --cpu-budget 1")
    res = _run(["--config", "1", "--steps", "3", "--warmup", "1", "--cpu-budget", "1"], timeout=240)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout
    rec = json.loads(lines[0])
    flush_print(lines[0][:400])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["higher_is_better"] is True and rec["data"] == "synthetic"
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"] == "small_k2_f32" and rec["config"]["K"] == 2

    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-12 * roof["frac"]
    assert roof["kernel"] in ("gram", "tree", "exact", "wsum")

    cpu = rec["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and 1 <= cpu["cores"] <= 16 and cpu["value"] > 0
    assert cpu["one_core"]["value"] > 0 and cpu["one_core"]["unit"] == cpu["unit"]

    # the last timed step's result against the oracle on the sampled segments
    par = rec["parity"]
    assert par["segments"] >= 1 and par["tol_rel_l2"] == 1e-5 and par["tol_coeff"] == 1e-6
    assert par["rel_l2"] <= par["tol_rel_l2"] and par["max_coeff_err"] <= par["tol_coeff"] and par["pass"] is True

    # this small one-stage combine is two launches: gram, then the walk
    # (with any exact recomputation) and the weighted sum in one
    assert set(rec["kernels"]) == {"gram", "wsum"}
    launches = {k: v["launches"] for k, v in rec["kernels"].items()}
    assert launches == {"gram": 3, "wsum": 3}, launches
    for key in ("mean", "median", "min", "max"):
        assert rec["step_ms"][key] > 0 and rec["step_ms_with_launch_events"][key] > 0
    assert rec["step_ms"]["min"] <= rec["step_ms"]["median"] <= rec["step_ms"]["max"]
    # the same combines with no event inside the loop, and as graph replays
    assert rec["step_ms_without_events"] > 0 and rec["step_ms_graph_replay"] > 0
