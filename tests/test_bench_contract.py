"""bench.py's output contract.

CPU: a request for more than one GPU (the flag, or a multi-rank launch) exits
with status 2 and says why, before touching the GPU.  GPU: a short run on the
smallest decode workload prints one JSON line with every field of the
contract, typed and consistent (value against ms_per_step and the call's K/V
bytes, the roofline fraction against its achieved rate and peak)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env=None, timeout=60):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, BENCH] + args, cwd=ROOT, env=e, timeout=timeout,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8", "--steps", "1"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_carries_the_contract():
    print("bench: --config 1 --steps 3 --warmup 1", flush=True)
    r = _run(["--config", "1", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"], timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["cpu_baseline"] is None
    assert d["config"]["workload"] == "mha1x1-L4096-f32" and d["dtype"] == "f32"
    # value is the call's K/V bytes over the time per call
    kv = d["config"]["kv_bytes_per_call"]
    assert abs(d["value"] - kv / (d["ms_per_step"] * 1e-3) / 1e9) <= 1e-3 * d["value"] + 0.02
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert rl["achieved"] > 0 and abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    assert "traffic" in rl
    assert d["read_ceiling"] is None      # the vector kernel's loads are not the probe's pattern
    assert d["library_plan"]["ms_per_call"] > 0
