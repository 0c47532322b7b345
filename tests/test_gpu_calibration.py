"""Calibration of the per-step budgets on the GPU: the library's error reduction
(lite_attn_output_max_abs_diff) against a host reduction, the library's calibration loop
(lite_attn_calibrate) against the Python driver and against the oracle's calibration, and the
Python driver on the library (LiteAttentionRunner): every output within its budget, infinite
budgets take the loosest candidate."""
import math

import numpy as np

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
    """The same calibration run inside the GPU library (lite_attn_calibrate) and driven over the
    CPU oracle, on the same bf16 inputs. GPU and oracle outputs may differ by the output tolerance, so each error the
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
    att = make_attention(cfg)
    gpu = att.calibrate([x[0] for x in xs], [x[1] for x in xs], [x[2] for x in xs], budgets)
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


def _host_max_abs_diff(a, b):
    x = a.detach().cpu().float().numpy()
    y = b.detach().cpu().float().numpy()
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - y)))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_output_max_abs_diff_matches_a_host_reduction(dtype):
    """Bit-exact against numpy on the same values (a maximum of float32 differences does not
    depend on the order of reduction), through contiguous and strided layouts; the memory
    between rows is never read (it holds NaN here); a NaN in a valid element gives NaN."""
    dev = device()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(11)
    B, H, N, D = 2, 3, 1000, 128
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype=dtype)
    a = torch.randn(B, H, N, D, generator=g).to(tdt).to(dev)
    b = (a.float().cpu() + 1e-2 * torch.randn(B, H, N, D, generator=g)).to(tdt).to(dev)
    b[1, 2, 999, 127] = a[1, 2, 999, 127] + 3.0          # the largest difference, last element
    got = att.max_abs_diff(a, b).item()
    want = _host_max_abs_diff(a, b)
    log(f"  {dtype} contiguous {got} host {want}")
    assert got == want and got >= 2.9
    a[0, 0, 0, 0] = float("nan")
    assert math.isnan(att.max_abs_diff(a, b).item())
    # packed [B][N][H][3D] layout (a fused projection), the unread columns filled with NaN
    strides = (N * H * 3 * D, 3 * D, H * 3 * D)
    sat = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype=dtype, strides=strides)
    base_a = torch.full((B, N, H, 3 * D), float("nan"), dtype=tdt, device=dev)
    base_b = torch.full((B, N, H, 3 * D), float("nan"), dtype=tdt, device=dev)
    va = base_a[..., D:2 * D].permute(0, 2, 1, 3)
    vb = base_b[..., D:2 * D].permute(0, 2, 1, 3)
    va.copy_(torch.randn(B, H, N, D, generator=g).to(tdt))
    vb.copy_(torch.randn(B, H, N, D, generator=g).to(tdt))
    got = sat.max_abs_diff(va, vb).item()
    want = _host_max_abs_diff(va, vb)
    log(f"  {dtype} strided {got} host {want}")
    assert got == want and not math.isnan(got)
    # an empty problem reports 0
    e = tsa.LiteAttention(1, 0, 100, 64, tile_q=64, dtype=dtype)
    z = torch.empty(1, 0, 100, 64, dtype=tdt, device=dev)
    r = torch.full((1,), 7.0, device=dev)
    assert e.max_abs_diff(z, z, r).item() == 0.0


def test_library_calibration_matches_the_python_driver():
    """lite_attn_calibrate and calibrate_schedule over LiteAttentionRunner run the same steps
    through the same kernels, so they pick the same budgets and measure the same errors, bit for
    bit; also with an alternating order, a dense prefix and a single step."""
    dev = device()
    cfg = derive(get_config(3), name="calib_c_vs_py", heads=[0, 7], grid=(3, 15, 40), steps=6)
    wl = Workload(cfg, dev)
    xs = [wl.inputs(t) for t in range(cfg.steps)]
    budgets = [float(np.float32(0.02 + 0.06 * t / (cfg.steps - 1))) for t in range(cfg.steps)]
    picks = []
    for over, n in (({}, cfg.steps), ({"dense_prefix": 300}, cfg.steps), ({}, 1)):
        att = make_attention(cfg, **over)
        py = tsa.calibrate_schedule(tsa.LiteAttentionRunner(att, dev), lambda t: xs[t], n,
                                    budgets[:n])
        lib = att.calibrate([x[0] for x in xs[:n]], [x[1] for x in xs[:n]],
                            [x[2] for x in xs[:n]], budgets[:n])
        log(f"  {over} steps={n}: library {lib.log_eps} {[round(e, 5) for e in lib.errors]}")
        assert lib.log_eps == py.log_eps
        assert lib.errors == py.errors
        picks.append(lib.log_eps)
    assert any(x > -math.inf for x in picks[0])      # the case does skip tiles
    assert picks[2] == (-math.inf,) and lib.errors == (0.0,)
