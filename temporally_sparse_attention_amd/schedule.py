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
