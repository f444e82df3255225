"""The bench's one-line JSON contract.

CPU: the single-GPU guard and the defaults.  GPU: one short run of the
headline workload, whose line must carry the fields the contract names, the
roofline fraction as achieved over peak, and a dominant kernel measured live.
"""

import json
import math

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU only" in capsys.readouterr().err


def test_defaults_are_the_headline_workload():
    a = bench.parse_args([])
    assert (a.gpus, a.workload, a.steps, a.warmup) == (1, "long", 100, 5)
    assert not (a.noncausal or a.decay or a.gated or a.gla or a.backward)


@pytest.mark.gpu
def test_headline_line(lib, span):
    import torch
    from kernelized_linear_attention_elu_amd import synth
    args = bench.parse_args(["--steps", "3", "--warmup", "1", "--settle", "0.05", "--no-cpu-baseline"])
    res = bench.bench_prefill(args, torch, lib, synth)
    json.dumps(res)  # serialisable as one line
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "path_roofline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 3 and res["warmup"] == 1
    assert res["higher_is_better"] is True and res["dtype"] == "bf16" and res["data"] == "synthetic"
    w = synth.WORKLOADS["long"]
    assert math.isclose(res["value"], w.B * w.N / (res["ms_per_step"] * 1e-3), rel_tol=1e-6)
    assert "workload" in res["config"]
    roof = res["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1 and math.isclose(roof["frac"], roof["achieved"] / roof["peak"], rel_tol=1e-9)
    assert roof["traffic"] is None or roof["traffic"] > 0
    # the dominant kernel's live duration fits inside the step
    assert 0 < res["dominant_kernel_us_live"] < res["ms_per_step"] * 1e3
