"""The benchmark's JSON line on the GPU: one short run of each measuring
leg (F^H D with its other path choices and the CPU-oracle baseline; an
operator leg), checked for the fields the line promises and for parity."""
import json

import pytest
import torch

import bench
from non_cartesian_mri_fhd_amd import binding, build

pytestmark = pytest.mark.gpu

ROOFLINE_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    build.ensure_built()
    binding.load()
    return torch.device("cuda:0")


def run(capsys, argv):
    assert bench.main(argv) == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, lines
    return json.loads(lines[0])


def test_adjoint_line(dev, capsys):
    d = run(capsys, ["--workload", "random16", "--steps", "3", "--warmup", "2", "--cpu-seconds", "0.5"])
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["unit"] == "terms/s"
    assert d["higher_is_better"] is True and d["vs_baseline"] is None and d["data"] == "synthetic"
    assert d["config"]["workload"].startswith("random16")
    assert d["config"]["N"] == 16 ** 3 and d["config"]["M"] == 2048
    assert ROOFLINE_KEYS <= set(d["roofline"]) and 0 < d["roofline"]["frac"] < 1
    assert d["kernel_ms"]["count"] == 3
    base = d["cpu_baseline"]
    assert base["kind"] == "oracle" and base["value"] > 0 and base["cores"] >= 1 and base["sample"]
    assert d["parity"]["rel_l2"] < d["parity"]["tolerance"] == 5e-4
    assert set(d["other_paths"]) == {"vector", "bf16x3"}
    for p, o in d["other_paths"].items():
        assert o["parity"]["rel_l2"] < 5e-4, p
        assert o["kernel_ms"]["count"] == 5 and o["terms_per_s"] > 0, p


def test_operator_line(dev, capsys):
    d = run(capsys, ["--op", "normal", "--workload", "random16", "--steps", "2", "--warmup", "1",
                     "--no-cpu-baseline"])
    assert d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["op"] == "normal" and d["config"]["terms_per_step"] == 2 * 16 ** 3 * 2048
    assert ROOFLINE_KEYS <= set(d["roofline"])
    assert "cpu_baseline" not in d
