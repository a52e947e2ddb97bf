"""bench.py's command-line contract: one JSON line with the fields the
benchmark record needs (a GPU run), and the refusal of more than one GPU
(no GPU needed)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("args,bound", [
    (("--steps", "3", "--warmup", "1"), "mfma"),
    (("--workload", "decode_gqa_b16_hq32_hkv8_sq1_skv32768_d128_bf16", "--steps", "3",
      "--warmup", "1", "--no-cpu-baseline"), "hbm"),
    (("--workload", "2,8,2,300,700,64,1,f16", "--steps", "2", "--warmup", "1",
      "--no-cpu-baseline"), None),
])
def test_json_line(args, bound):
    r = _bench(*args)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["higher_is_better"] is True and d["unit"] == "TFLOP/s"
    assert d["steps"] == int(args[args.index("--steps") + 1])
    assert "workload" in d["config"]
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    if bound:
        assert roof["bound"] == bound
    if "--no-cpu-baseline" in args:
        assert d["cpu_baseline"] is None
    else:
        cpu = d["cpu_baseline"]
        assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
