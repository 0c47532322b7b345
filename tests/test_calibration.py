"""Calibration of the per-step budgets from accumulated output error (calibrate_schedule), driven
by the CPU oracle: the host logic of the calibration is checked against what it promises."""
import math

import numpy as np
import pytest
import torch

from oracle import empty_mask, lite_attn_step_ref, mask_to_bits
import temporally_sparse_attention_amd as tsa
from workloads import Workload, derive, get_config


class OracleRunner:
    def __init__(self, cfg):
        self.cfg = cfg

    def empty_mask(self):
        c = self.cfg
        return empty_mask(c.batch, c.heads, c.seq_len, c.tile_q, c.tile_k)

    def step(self, x, mask, log_eps, t):
        q, k, v = x
        c = self.cfg
        r = lite_attn_step_ref(q, k, v, mask, tile_q=c.tile_q, tile_k=c.tile_k,
                               softmax_scale=c.softmax_scale, log_eps=log_eps, step=t,
                               order=c.order, dense_prefix=c.dense_prefix)
        return r.out, r.mask_next

    def dense(self, x, t):
        return self.step(x, self.empty_mask(), -math.inf, t)[0]

    def error(self, out, ref):
        return float(np.abs(out - ref).max())


@pytest.fixture(scope="module")
def case():
    cfg = derive(get_config(5), name="calib", heads=[8, 9], grid=(2, 12, 16), steps=5)
    wl = Workload(cfg, "cpu")
    xs = [tuple(a.float() for a in wl.inputs(t)) for t in range(cfg.steps)]
    return cfg, (lambda t: xs[t])


def test_infinite_budgets_take_the_loosest_candidate(case):
    cfg, inputs = case
    cands = (-3.0, -9.0, -15.0)
    res = tsa.calibrate_schedule(OracleRunner(cfg), inputs, cfg.steps, [math.inf] * cfg.steps,
                                 candidates=cands)
    assert res.log_eps == (-3.0,) * cfg.steps
    assert res.errors[0] == 0.0


def test_zero_budgets_leave_every_output_exact(case):
    cfg, inputs = case
    res = tsa.calibrate_schedule(OracleRunner(cfg), inputs, cfg.steps, [0.0] * cfg.steps)
    assert all(e == 0.0 for e in res.errors)


@pytest.mark.parametrize("lo,hi", [(0.002, 0.02), (0.01, 0.2), (0.0, 0.05)])
def test_every_output_stays_within_its_budget_and_replays(case, lo, hi):
    cfg, inputs = case
    budgets = [lo + (hi - lo) * t / (cfg.steps - 1) for t in range(cfg.steps)]
    runner = OracleRunner(cfg)
    res = tsa.calibrate_schedule(runner, inputs, cfg.steps, budgets)
    assert all(e <= b for e, b in zip(res.errors, budgets)), (res.errors, budgets)
    # replaying the chosen schedule gives the same errors, and the mask only grows
    mask = runner.empty_mask()
    for t in range(cfg.steps):
        out, nxt = runner.step(inputs(t), mask, res.log_eps[t], t)
        assert runner.error(out, runner.dense(inputs(t), t)) == res.errors[t]
        assert np.array_equal(nxt | mask, nxt)
        mask = nxt
    looser = tsa.calibrate_schedule(runner, inputs, cfg.steps, [10 * b + 1.0 for b in budgets])
    assert sum(res.log_eps) <= sum(looser.log_eps)


def test_rejects_bad_arguments(case):
    cfg, inputs = case
    with pytest.raises(ValueError):
        tsa.calibrate_schedule(OracleRunner(cfg), inputs, cfg.steps, [0.1] * (cfg.steps - 1))
    with pytest.raises(ValueError):
        tsa.calibrate_schedule(OracleRunner(cfg), inputs, cfg.steps, [0.1] * cfg.steps,
                               candidates=(0.5,))
