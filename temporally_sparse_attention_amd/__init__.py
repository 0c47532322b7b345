"""MI355X (gfx950) implementation of LiteAttention's hot path.

Tiled self-attention with an embedded QK-Skip test and a persistent skip bitmask carried
across denoising steps ("LiteAttention: Temporal Sparse Attention for Diffusion
Transformers", page 1 "Core Concept" and "Architecture Overview"). The computation runs in
liblite_attn.so (hand-written HIP kernels behind a C ABI, include/lite_attn.h); this package
is a thin binding with the same names plus a small convenience wrapper.
"""
from __future__ import annotations

from .binding import (  # noqa: F401
    ABI_VERSION,
    EXPORTS,
    OPT_IN_STEP_SKIP,
    LIB_PATH,
    Handle,
    LiteAttnError,
    lite_attn_calibrate,
    lite_attn_calibrate_workspace_bytes,
    lite_attn_create,
    lite_attn_destroy,
    lite_attn_last_error,
    lite_attn_last_launch,
    lite_attn_mask_bytes,
    lite_attn_mask_geometry,
    lite_attn_mask_popcount,
    lite_attn_output_max_abs_diff,
    lite_attn_reset_mask,
    lite_attn_status_string,
    lite_attn_step,
    lite_attn_step_refresh,
    lite_attn_step_scheduled,
    lite_attn_step_scheduled_static,
    lite_attn_workspace_bytes,
    make_config,
)
from .schedule import (  # noqa: F401
    DEFAULT_CANDIDATES,
    CalibrationResult,
    ErrorBudgetSchedule,
    LiteAttentionRunner,
    calibrate_schedule,
)


class LiteAttention:
    """One attention call site: a handle plus helpers to allocate and inspect its mask.

    att = LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1.0)
    mask = att.new_mask(device)            # zeroed skip mask (a fresh generation)
    for t, log_eps in enumerate(schedule):
        att.step(q_t, k_t, v, out, mask, log_eps, t)
    """

    def __init__(self, batch: int, heads: int, seq_len: int, head_dim: int, **kw):
        self.handle = lite_attn_create(batch, heads, seq_len, head_dim, **kw)

    @property
    def mask_shape(self):
        return self.handle.mask_shape

    @property
    def tiles(self):
        return self.handle.tiles_q, self.handle.tiles_k

    def new_mask(self, device, stream=None):
        import torch
        mask = torch.empty(self.mask_shape, dtype=torch.int32, device=device)
        if mask.numel():
            lite_attn_reset_mask(self.handle, mask, stream)
        return mask

    def reset_mask(self, mask, stream=None):
        lite_attn_reset_mask(self.handle, mask, stream)

    def new_workspace(self, device):
        """Device workspace for scheduled steps (query tiles ordered by visit count: heavy first,
        short last)."""
        import torch
        return torch.empty(max(1, lite_attn_workspace_bytes(self.handle)), dtype=torch.uint8,
                           device=device)

    def new_tile_stats(self, device):
        """References of the divergence refresh (float32 [B, H, Tq], NaN: none yet)."""
        import torch
        c = self.handle.cfg
        return torch.full((c.batch, c.heads, self.handle.tiles_q), float("nan"),
                          dtype=torch.float32, device=device)

    def step(self, q, k, v, out, mask, log_eps_t: float, step: int, stream=None, workspace=None,
             tile_stats=None, refresh_delta: float = float("inf")):
        """One denoising step. With a workspace the query tiles run heavy first and short last; with
        tile_stats the mask rows whose statistic moved by more than refresh_delta are cleared
        (divergence refresh). The two options are separate entry points and do not combine."""
        if tile_stats is not None:
            if workspace is not None:
                raise ValueError("workspace and tile_stats do not combine")
            lite_attn_step_refresh(self.handle, q, k, v, out, mask, tile_stats, refresh_delta,
                                   log_eps_t, step, stream)
        elif workspace is None:
            lite_attn_step(self.handle, q, k, v, out, mask, log_eps_t, step, stream)
        else:
            lite_attn_step_scheduled(self.handle, q, k, v, out, mask, log_eps_t, step, workspace,
                                     stream)

    def popcount(self, mask, counts=None, stream=None):
        """Per-head skipped-tile counts (device int32 [B*H]); asynchronous."""
        import torch
        c = self.handle.cfg
        if counts is None:
            counts = torch.empty(c.batch * c.heads, dtype=torch.int32, device=mask.device)
        lite_attn_mask_popcount(self.handle, mask, counts, stream)
        return counts

    def skipped_fraction(self, mask) -> float:
        """Skipped-tile fraction of a mask (synchronises with the host)."""
        c = self.handle.cfg
        total = c.batch * c.heads * self.handle.tiles_q * self.handle.tiles_k
        if total == 0:
            return 0.0
        return float(self.popcount(mask).to("cpu").long().sum().item()) / total

    def max_abs_diff(self, a, b, result=None, stream=None):
        """Device float32 [1] tensor holding max |a - b| over the valid elements; asynchronous."""
        import torch
        if result is None:
            result = torch.empty(1, dtype=torch.float32, device=a.device)
        lite_attn_output_max_abs_diff(self.handle, a, b, result, stream)
        return result

    def new_calibration_workspace(self, device):
        import torch
        return torch.empty(max(1, lite_attn_calibrate_workspace_bytes(self.handle)),
                           dtype=torch.uint8, device=device)

    def calibrate(self, qs, ks, vs, error_budgets, candidates=DEFAULT_CANDIDATES,
                  workspace=None, stream=None) -> CalibrationResult:
        """Per-step budgets log_eps_t from per-step output-error limits, chosen by the library
        (lite_attn_calibrate); qs, ks, vs hold one device tensor per step. Blocks until done."""
        if workspace is None and len(qs):
            workspace = self.new_calibration_workspace(qs[0].device)
        log_eps, errors = lite_attn_calibrate(self.handle, qs, ks, vs, error_budgets, candidates,
                                              workspace, stream)
        return CalibrationResult(log_eps, errors, [float(x) for x in error_budgets])
