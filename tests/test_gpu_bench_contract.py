"""bench.py's output contract, on the GPU: one JSON line with the metric, the
whole-job throughput and its unit, the step counts and time, the workload
config, the roofline object of the dominant kernel (algorithmic rate against
the MI355X peak, with HBM traffic from the committed counter summary or
null) and the measured streaming-copy bandwidth; run in-process with few
steps."""
import json

import pytest

import bench

pytestmark = pytest.mark.gpu


def _run(capsys, argv):
    rc = bench.main(argv)
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert rc == 0 and len(lines) == 1, lines
    return json.loads(lines[0])


def test_prefill_line(capsys):
    d = _run(capsys, ["--steps", "3", "--warmup", "1", "--no-cpu-baseline"])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernel_ms"):
        assert key in d, key
    assert d["unit"] == "tokens/s" and d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["data"] == "synthetic" and d["vs_baseline"] is None
    assert d["config"]["workload"] == "long_T8192_H32" and d["config"]["T"] == 8192 and d["config"]["H"] == 32
    # value is the whole job's tokens per second of the timed steps
    assert abs(d["value"] - 8192 / (d["ms_per_step"] / 1e3)) <= 1e-3 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["kernel"] in d["kernel_ms"] and 0 < r["frac"] <= 1 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # achieved = the path's algorithmic bytes (1282 B per token-head, plus the bf16 final state)
    # over the dominant kernel's time; never the library's own intermediates
    assert r["alg_bytes"] == 1282 * 8192 * 32 + 32 * 128 * 128 * 2
    assert abs(r["achieved"] - r["alg_bytes"] / (d["kernel_ms"][r["kernel"]] * 1e-3) / 1e9) <= 1e-3 * r["achieved"]
    assert r["frac_interface"] > r["frac"]
    assert r["traffic"] is None or r["traffic"] > 0
    assert r["copy_gbs"] > 1000 and set(r["kernels"]) == set(d["kernel_ms"])
    shares = sum(k["alg_share_bytes"] for k in r["kernels"].values())
    assert shares == r["alg_bytes"]  # the kernels' shares add up to the path's bytes
    assert d["dtype"] == "bf16" and "fp16" in d["mfma_operands"]


def test_decode_line(capsys):
    d = _run(capsys, ["--decode", "4", "--steps", "5", "--warmup", "1"])
    assert d["unit"] == "tokens/s" and d["config"]["N"] == 4 and d["roofline"]["kernel"] == "kda_decode_split4_kernel"
    assert abs(d["value"] - 4 / (d["ms_per_step"] / 1e3)) <= 1e-3 * d["value"]


def test_more_than_one_gpu_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
