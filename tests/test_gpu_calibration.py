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
