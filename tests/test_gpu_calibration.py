"""calibrate_schedule on the GPU library (LiteAttentionRunner): every output within its budget,
infinite budgets take the loosest candidate."""
import math

import pytest
import torch

from gpu_util import device, log, make_attention
import temporally_sparse_attention_amd as tsa
from workloads import Workload, derive, get_config

pytestmark = pytest.mark.gpu


def test_gpu_calibration_respects_budgets():
    dev = device()
    cfg = derive(get_config(3), name="calib_gpu", heads=[0, 7], grid=(3, 15, 40), steps=6)
    wl = Workload(cfg, dev)
    xs = [wl.inputs(t) for t in range(cfg.steps)]
    runner = tsa.LiteAttentionRunner(make_attention(cfg), dev)
    budgets = [0.02 + 0.06 * t / (cfg.steps - 1) for t in range(cfg.steps)]
    res = tsa.calibrate_schedule(runner, lambda t: xs[t], cfg.steps, budgets)
    log(f"  schedule {res.log_eps} errors {[round(e, 4) for e in res.errors]}")
    assert all(e <= b for e, b in zip(res.errors, budgets))
    assert any(x > -math.inf for x in res.log_eps)
    loose = tsa.calibrate_schedule(runner, lambda t: xs[t], cfg.steps, [math.inf] * cfg.steps,
                                   candidates=(-4.0, -8.0))
    assert loose.log_eps == (-4.0,) * cfg.steps


def test_gpu_calibration_agrees_with_the_oracle_calibration():
    """The same calibration driven by the GPU library and by the CPU oracle, on the same bf16
    inputs. GPU and oracle outputs may differ by the output tolerance, so each error the
    calibration measures may move by twice that; the test checks that the two calibrations
    differ by no more than that: each schedule, replayed on the other side, meets its budgets
    within the tolerance, and the errors each side reports for the GPU's schedule agree."""
    from gpu_util import OUT_MAX
    from test_calibration import OracleRunner
    dev = device()
    cfg = derive(get_config(3), name="calib_vs_oracle", heads=[0, 7], grid=(3, 15, 40), steps=6)
    wl = Workload(cfg, dev)
    xs = [wl.inputs(t) for t in range(cfg.steps)]
    xs_cpu = [tuple(a.cpu() for a in x) for x in xs]
    budgets = [0.02 + 0.06 * t / (cfg.steps - 1) for t in range(cfg.steps)]
    gpu_runner = tsa.LiteAttentionRunner(make_attention(cfg), dev)
    ref_runner = OracleRunner(cfg)
    gpu = tsa.calibrate_schedule(gpu_runner, lambda t: xs[t], cfg.steps, budgets)
    ref = tsa.calibrate_schedule(ref_runner, lambda t: xs_cpu[t], cfg.steps, budgets)
    log(f"  GPU    schedule {gpu.log_eps} errors {[round(e, 4) for e in gpu.errors]}")
    log(f"  oracle schedule {ref.log_eps} errors {[round(e, 4) for e in ref.errors]}")

    def replay(runner, x, schedule):
        mask, errs = runner.empty_mask(), []
        for t in range(cfg.steps):
            out, mask = runner.step(x[t], mask, schedule[t], t)
            errs.append(runner.error(out, runner.dense(x[t], t)))
        return errs

    tol = 2 * OUT_MAX
    ref_at_gpu = replay(ref_runner, xs_cpu, gpu.log_eps)    # the GPU's schedule on the oracle
    gpu_at_ref = replay(gpu_runner, xs, ref.log_eps)        # the oracle's schedule on the GPU
    log(f"  oracle errors under the GPU schedule {[round(e, 4) for e in ref_at_gpu]}")
    log(f"  GPU errors under the oracle schedule {[round(e, 4) for e in gpu_at_ref]}")
    agree = sum(a == b for a, b in zip(gpu.log_eps, ref.log_eps))
    log(f"  schedules agree on {agree} of {cfg.steps} steps")
    for t in range(cfg.steps):
        assert gpu.errors[t] <= budgets[t] and ref.errors[t] <= budgets[t], t
        assert abs(gpu.errors[t] - ref_at_gpu[t]) <= tol, (t, gpu.errors[t], ref_at_gpu[t])
        assert ref_at_gpu[t] <= budgets[t] + tol, (t, ref_at_gpu[t])
        assert gpu_at_ref[t] <= budgets[t] + tol, (t, gpu_at_ref[t])
        if gpu.log_eps[t] != ref.log_eps[t]:
            # a differing pick at step t shows in step t+1's error: it must be a tie within the
            # tolerance on both sides
            assert t + 1 < cfg.steps
            assert abs(ref_at_gpu[t + 1] - budgets[t + 1]) <= tol or \
                abs(gpu_at_ref[t + 1] - budgets[t + 1]) <= tol, t
