"""Host-side checks of bench.py: the one-GPU guard, the step-time spread and
the CPU-oracle baseline on a tiny workload (no GPU needed)."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_spread_is_nearest_rank():
    import bench
    v = [float(i) for i in range(1, 22)]   # 21 sorted values
    s = bench._spread(v)
    assert s == {"median": 11.0, "p10": 3.0, "p90": 19.0, "n": 21}
    assert bench._spread([2.5]) == {"median": 2.5, "p10": 2.5, "p90": 2.5, "n": 1}


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    import bench
    from sparse_mixture_experts_23_amd.workloads import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg, seed=0, device="cpu")
    out = bench.cpu_baseline(cfg, inp, 64)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["sample"].startswith("64-token routing group")
    assert set(out["phase_s"]) == {"route", "dispatch", "experts_and_combine"}
    assert all(v >= 0 for v in out["phase_s"].values())


def test_cpu_baseline_checks_a_run_against_the_oracle():
    """With the whole routing group as the sample, the baseline leg compares a
    run's outputs with the oracle's: a run that reproduces them is within
    tolerance, one with a perturbed element is reported outside it."""
    import types

    import numpy as np
    import torch

    import bench
    from oracle import moe_oracle as O
    from sparse_mixture_experts_23_amd.workloads import CONFIGS, make_inputs
    cfg = CONFIGS["tiny_fp32"]
    inp = make_inputs(cfg, seed=0, device="cpu")
    f = lambda t: t.numpy().astype(np.float64)  # noqa: E731
    ref = O.forward(f(inp.x), inp.w_r.numpy(), None, (f(inp.w_gate), f(inp.w_up), f(inp.w_down)), cfg.k,
                    cfg.gate_mode)
    run = types.SimpleNamespace(topk_ids=torch.from_numpy(ref.route.ids.astype(np.int32)),
                                y=torch.from_numpy(ref.y.astype(np.float32)),
                                slot=torch.from_numpy(ref.dispatch.slot.astype(np.int32)))
    p = bench.cpu_baseline(cfg, inp, cfg.T, run)["parity_vs_gpu"]
    assert p["within_tol"] and p["set_flips"] == 0 and p["slots_equal"] and p["elements"] == cfg.T * cfg.d
    run.y[5, 7] += 1.0
    p = bench.cpu_baseline(cfg, inp, cfg.T, run)["parity_vs_gpu"]
    assert not p["within_tol"] and p["max_rel_err"] > 0.1
    assert bench.cpu_baseline(cfg, inp, 64, run)["parity_vs_gpu"] is None   # a sample smaller than the group
