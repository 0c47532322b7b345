"""Per-step error budgets for the QK-Skip test.

LiteAttention, page 1 "Architecture Overview" (accumulated-error calibration): each denoising
step gets its own error budget, and early steps tolerate less error. A budget is the natural
log of the largest ratio, between a tile's local maximum attention weight and the running
maximum, that still lets the tile be skipped; -inf disables skipping for that step.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Sequence, Tuple


class ErrorBudgetSchedule:
    """Validated per-step budgets log_eps_t: each in [-inf, 0], never loosening then
    tightening (non-decreasing in t, so early steps are the strictest)."""

    def __init__(self, log_eps: Iterable[float]):
        vals = [float(x) for x in log_eps]
        for t, x in enumerate(vals):
            if math.isnan(x) or x > 0.0:
                raise ValueError(f"log_eps[{t}] = {x} is not in [-inf, 0]")
        for t in range(1, len(vals)):
            if vals[t] < vals[t - 1]:
                raise ValueError(f"budget tightens at step {t} ({vals[t - 1]} -> {vals[t]}); "
                                 "early steps must be the strictest")
        self.values: Tuple[float, ...] = tuple(vals)

    @classmethod
    def linear(cls, steps: int, start: float, end: float) -> "ErrorBudgetSchedule":
        if steps == 1:
            return cls([start])
        return cls([start + (end - start) * t / (steps - 1) for t in range(steps)])

    @classmethod
    def constant(cls, steps: int, value: float) -> "ErrorBudgetSchedule":
        return cls([value] * steps)

    def __len__(self) -> int:
        return len(self.values)

    def __getitem__(self, t: int) -> float:
        return self.values[t]

    def __iter__(self):
        return iter(self.values)


# ---------------------------------------------------------------------------------------------
# Calibration of the budgets from accumulated error
# ---------------------------------------------------------------------------------------------
DEFAULT_CANDIDATES = (-2.0, -4.0, -6.0, -8.0, -10.0, -12.0, -14.0, -16.0, -20.0, -24.0)


class CalibrationResult:
    """Per-step budgets chosen by calibrate_schedule, the output error each step reached against
    dense attention, and the error budget it had."""

    def __init__(self, log_eps, errors, budgets):
        self.log_eps: Tuple[float, ...] = tuple(log_eps)
        self.errors: Tuple[float, ...] = tuple(errors)
        self.budgets: Tuple[float, ...] = tuple(budgets)

    def as_dict(self):
        return {"log_eps": list(self.log_eps), "errors": list(self.errors),
                "budgets": list(self.budgets)}


def calibrate_schedule(runner, inputs, steps: int, error_budgets: Sequence[float],
                       candidates: Sequence[float] = DEFAULT_CANDIDATES) -> CalibrationResult:
    """Derive log_eps_t from per-step output-error budgets (LiteAttention, page 1 "Architecture
    Overview": accumulated-error calibration, early steps tolerate less error).

    The flags of step t first change the output of step t+1, so log_eps_t is the loosest
    candidate whose flags, added to the mask carried so far, keep the error of step t+1's output
    against dense attention within error_budgets[t+1]; -inf (flag nothing) when none does. The
    last step's flags change no output, so it keeps the previous step's budget. The error is the
    accumulated one: the mask holds every flag since the generation started.

    runner: empty_mask(); step(x, mask, log_eps, t) -> (out, new_mask) without changing `mask`;
            dense(x, t) -> out (no tile skipped); error(out, ref) -> float.
    inputs: inputs(t) -> the step's inputs x (passed through to the runner).
    error_budgets: one budget per step (step 0's output is exact: its mask is empty).
    """
    if len(error_budgets) != steps:
        raise ValueError("one error budget per step is needed")
    cands = sorted({float(c) for c in candidates}, reverse=True)   # loosest first
    for c in cands:
        if math.isnan(c) or c > 0.0:
            raise ValueError(f"candidate {c} is not in [-inf, 0]")
    mask = runner.empty_mask()
    chosen: List[float] = []
    errors: List[float] = []
    x_t = inputs(0)
    dense_t = runner.dense(x_t, 0)
    for t in range(steps):
        if t + 1 < steps:
            x_n = inputs(t + 1)
            dense_n = runner.dense(x_n, t + 1)
            pick = -math.inf
            for eps in cands:
                _, m_try = runner.step(x_t, mask, eps, t)
                out_n, _ = runner.step(x_n, m_try, -math.inf, t + 1)
                if runner.error(out_n, dense_n) <= error_budgets[t + 1]:
                    pick = eps
                    break
        else:
            x_n = dense_n = None
            pick = chosen[-1] if chosen else -math.inf
        out, mask = runner.step(x_t, mask, pick, t)
        errors.append(float(runner.error(out, dense_t)))
        chosen.append(pick)
        x_t, dense_t = x_n, dense_n
    return CalibrationResult(chosen, errors, error_budgets)


class LiteAttentionRunner:
    """calibrate_schedule runner on the GPU library: x = (q, k, v) device tensors; the error is
    max |out - ref| over the valid elements, reduced on the device by the library
    (lite_attn_output_max_abs_diff). LiteAttention.calibrate runs the same loop inside the
    library."""

    def __init__(self, attention, device):
        self.att = attention
        self.device = device
        self._result = None

    def empty_mask(self):
        return self.att.new_mask(self.device)

    def step(self, x, mask, log_eps: float, t: int):
        import torch
        q, k, v = x
        m = mask.clone()
        out = torch.empty_like(q)
        self.att.step(q, k, v, out, m, log_eps, t)
        return out, m

    def dense(self, x, t: int):
        return self.step(x, self.empty_mask(), -math.inf, t)[0]

    def error(self, out, ref) -> float:
        import torch
        if self._result is None:
            self._result = torch.empty(1, dtype=torch.float32, device=self.device)
        return float(self.att.max_abs_diff(out, ref, self._result).item())
