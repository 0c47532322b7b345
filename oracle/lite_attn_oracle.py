"""CPU oracle for one LiteAttention denoising step (float64, numpy).

TEST INFRASTRUCTURE ONLY. This is the correctness reference for the HIP path. Only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and this module imports nothing from the product package.

What one step computes (LiteAttention: Temporal Sparse Attention for Diffusion Transformers;
page 1 "Core Concept" and "Architecture Overview", page 2 abstract):

Tiling. Queries and keys of each (batch, head) are cut into tiles of tile_q rows and tile_k
columns; the last tile of each may be ragged. Row tile i covers rows
[i*tile_q, min(N, (i+1)*tile_q)), column tile j covers [j*tile_k, min(N, (j+1)*tile_k)).

Skip-Mask (page 1 "Architecture Overview", the bitmask bullet). One bit per
(batch, head, query tile, key tile): mask[b, h, i, j // 32] bit (j % 32). A set bit means the
tile is skipped.

Output (page 1 "Core Concept": flagged tiles are not computed; page 1 "Architecture
Overview": the kernel is FlashAttention with the skip logic inside it). Given the mask at the
start of the step, the output is exact softmax attention restricted to the key tiles whose
bit is clear:
    O[r] = sum_{c in A(i)} softmax_{c in A(i)}(scale * q_r . k_c) v_c,
    A(i) = union of the columns of tiles j with mask[b,h,i,j] == 0.
This is a plain definition, so it is written out directly (one matmul for all scores, a
softmax over the allowed columns, one matmul with V). A row tile with no allowed tile gets a
zero output (reading: the pages never reach that case).

QK-Skip and propagation (page 1 "Core Concept": a tile whose local maximum QK score is far
below the cumulative maximum is flagged; "Architecture Overview": decisions carry forward;
page 2: skip decisions propagate across the denoising sequence). For each row tile, the key
tiles are visited in the traversal order of this step (ascending, or - in the alternating
order - descending on odd steps). Skipped tiles are not visited at all. For a visited tile j:
    mt[r]     = max over the tile's columns of the scaled score of row r
    margin(j) = max over the tile's rows of (mt[r] - m[r]) - log_eps
    m[r]      = max(m[r], mt[r])            (m starts at -inf: the cumulative maximum)
and tile j is flagged when margin(j) < 0, i.e. when every row's local maximum is more than
|log_eps| below that row's running maximum, unless the tile is exempt (its rows or columns
touch the dense prefix [0, dense_prefix)). A NaN margin never flags. Flags take effect from
the next step: mask_next = mask | flagged. Bits are never cleared here.

In-step skip (an option, off by default; page 1 "Architecture Overview": the skip logic sits
inside the softmax pipeline). A tile flagged while it is visited is also left out of this
step's own output. Flagging never changes the running maximum (a flagged tile's row maxima lie
below it), so the flags are the same as without the option, and the output is the plain
definition above taken over the mask *after* the step: A'(i) = tiles clear in mask_next.

Divergence-triggered refresh (an option; page 1 "Core Concept": the mask is updated only when
the attention pattern diverges significantly; "Architecture Overview": decisions carry forward
unless the attention distribution shifts significantly). The statistic of a row tile is the mean
over its valid rows of the running row maximum at the end of the step (the largest scaled score
over the key tiles it computed). A reference is taken on the first step that has none (stored as
NaN). When the statistic later moves by more than refresh_delta from the reference - or the
difference is NaN - the tile's mask row is cleared instead of updated (the next step computes
it densely and flags afresh) and the reference is dropped (NaN); otherwise the row is updated as
usual and the reference kept. A row maximum falls when the mass moves into skipped tiles, which
is exactly the divergence the skip mask cannot see.

Page 1's code sketch expresses the threshold as a ratio on scores; on exponentiated scores the
ratio test exp(mt) < ratio * exp(m) is exactly mt - m < ln(ratio), which is the log-domain
budget log_eps used here (page 1 "Architecture Overview", accumulated-error calibration,
gives one budget per step).

Inputs are widened to float64 exactly (bfloat16 and float32 values are representable).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional, Tuple

import numpy as np

__all__ = [
    "mask_geometry",
    "empty_mask",
    "mask_to_bits",
    "bits_to_mask",
    "StepResult",
    "lite_attn_step_ref",
    "run_chain_ref",
]


def mask_geometry(seq_len: int, tile_q: int, tile_k: int) -> Tuple[int, int, int]:
    """(Tq, Tk, W): query tiles, key tiles and 32-bit words per mask row."""
    tq = -(-seq_len // tile_q)
    tk = -(-seq_len // tile_k)
    w = -(-tk // 32)
    return tq, tk, w


def empty_mask(batch: int, heads: int, seq_len: int, tile_q: int, tile_k: int) -> np.ndarray:
    tq, _, w = mask_geometry(seq_len, tile_q, tile_k)
    return np.zeros((batch, heads, tq, w), dtype=np.uint32)


def mask_to_bits(mask: np.ndarray, tiles_k: int) -> np.ndarray:
    """uint32 [..., W] -> bool [..., Tk] (bit j % 32 of word j // 32)."""
    mask = np.asarray(mask, dtype=np.uint32)
    j = np.arange(tiles_k)
    return ((mask[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)


def bits_to_mask(bits: np.ndarray) -> np.ndarray:
    """bool [..., Tk] -> uint32 [..., ceil(Tk/32)]."""
    bits = np.asarray(bits, dtype=bool)
    tk = bits.shape[-1]
    w = -(-tk // 32)
    out = np.zeros(bits.shape[:-1] + (w,), dtype=np.uint32)
    for j in range(tk):
        out[..., j // 32] |= bits[..., j].astype(np.uint32) << np.uint32(j % 32)
    return out


@dataclasses.dataclass
class StepResult:
    out: np.ndarray        # [B, H, N, D] float64; NaN in rows that were not requested
    mask_next: np.ndarray  # [B, H, Tq, W] uint32
    margins: np.ndarray    # [B, H, Tq, Tk] float64; NaN where the tile was not visited
    computed_rows: np.ndarray  # [B, H, Tq] bool: which row tiles were evaluated
    stats: Optional[np.ndarray] = None        # [B, H, Tq] refresh statistic of this step
    stats_next: Optional[np.ndarray] = None   # [B, H, Tq] reference after the step (NaN: none)
    refreshed: Optional[np.ndarray] = None    # [B, H, Tq] bool: row cleared by the refresh


def _head(x, b: int, h: int) -> np.ndarray:
    """One head of a [B, H, N, D] array-like as float64 numpy (torch CPU tensors included)."""
    xh = x[b, h]
    if hasattr(xh, "detach"):  # torch tensor (possibly bfloat16): widen exactly via float64
        import torch
        return xh.detach().to("cpu", torch.float64).numpy()
    return np.asarray(xh, dtype=np.float64)


def _row_tile(qi: np.ndarray, kh: np.ndarray, vh: np.ndarray, skipped: np.ndarray, i: int, *,
              tile_q: int, tile_k: int, scale: float, log_eps: float, descending: bool,
              dense_prefix: int, in_step_skip: bool = False):
    """Output rows, flags and margins of row tile i of one head."""
    n = kh.shape[0]
    tk = skipped.shape[0]
    nr = qi.shape[0]
    dv = vh.shape[1]

    # Scaled scores of these rows against every key (float64).
    s = scale * (qi @ kh.T)                                   # [nr, N]

    # Per-row maximum of each key tile (padding columns of the ragged last tile are -inf).
    padded = np.full((nr, tk * tile_k), -np.inf)
    padded[:, :n] = s
    tile_max = padded.reshape(nr, tk, tile_k).max(axis=2)     # [nr, Tk]

    # QK-Skip over the visited tiles, in this step's traversal order.
    row_exempt = i * tile_q < dense_prefix
    order = range(tk - 1, -1, -1) if descending else range(tk)
    running = np.full(nr, -np.inf)
    flags = np.zeros(tk, dtype=bool)
    margins = np.full(tk, np.nan)
    for j in order:
        if skipped[j]:
            continue
        mt = tile_max[:, j]
        margin = np.max(mt - running) - log_eps   # running = -inf gives +inf; NaN propagates
        margins[j] = margin
        col_exempt = j * tile_k < dense_prefix
        if margin < 0 and not (row_exempt or col_exempt):
            flags[j] = True
        running = np.maximum(running, mt)

    # Output: softmax over the allowed columns only (with in-step skip, tiles flagged in this
    # step are not allowed either).
    stat = float(np.mean(running))   # refresh statistic: mean of the rows' running maxima
    out_skipped = (skipped | flags) if in_step_skip else skipped
    allowed_cols = np.repeat(~out_skipped, tile_k)[:n]
    if allowed_cols.any():
        sa = np.where(allowed_cols[None, :], s, -np.inf)
        row_max = sa.max(axis=1, keepdims=True)
        p = np.exp(sa - row_max)
        out = (p @ vh) / p.sum(axis=1, keepdims=True)
    else:
        out = np.zeros((nr, dv))
    return out, flags, margins, stat


def lite_attn_step_ref(q, k, v, mask, *, tile_q: int, tile_k: int, softmax_scale: float,
                       log_eps: float, step: int, order: str = "alt", dense_prefix: int = 0,
                       rows: Optional[Iterable[Tuple[int, int, int]]] = None,
                       in_step_skip: bool = False, tile_stats: Optional[np.ndarray] = None,
                       refresh_delta: float = math.inf) -> StepResult:
    """One denoising step of LiteAttention on [B, H, N, D] inputs.

    q, k, v: numpy arrays or torch CPU tensors [B, H, N, D] (any float dtype).
    mask:    uint32 [B, H, Tq, W], the skip mask at the start of the step.
    order:   "asc" (always ascending key tiles) or "alt" (ascending on even steps,
             descending on odd steps).
    rows:    optional (b, h, i) row tiles to evaluate; default every row tile. Rows of the
             output not evaluated are NaN; mask rows not evaluated are copied unchanged.
    in_step_skip: also leave the tiles flagged in this step out of this step's output.
    tile_stats: float [B, H, Tq] references of the divergence refresh (NaN: none yet), or None
             for no refresh; refresh_delta: the largest move of the statistic that keeps a row.
    """
    if order not in ("asc", "alt"):
        raise ValueError("order must be 'asc' or 'alt'")
    if not (log_eps <= 0.0):
        raise ValueError("log_eps must be <= 0 (or -inf)")
    bsz, nh, n, _ = (int(x) for x in q.shape)
    dv = int(v.shape[-1])
    tq, tk, w = mask_geometry(n, tile_q, tile_k)
    mask = np.asarray(mask, dtype=np.uint32)
    if mask.shape != (bsz, nh, tq, w):
        raise ValueError(f"mask shape {mask.shape} != {(bsz, nh, tq, w)}")
    descending = order == "alt" and step % 2 == 1

    refresh = tile_stats is not None
    if refresh:
        tile_stats = np.asarray(tile_stats, dtype=np.float64)
        if tile_stats.shape != (bsz, nh, tq):
            raise ValueError(f"tile_stats shape {tile_stats.shape} != {(bsz, nh, tq)}")
        if not (refresh_delta >= 0.0):
            raise ValueError("refresh_delta must be >= 0")
        stats = np.full((bsz, nh, tq), np.nan)
        stats_next = tile_stats.copy()
        refreshed = np.zeros((bsz, nh, tq), dtype=bool)
    out = np.full((bsz, nh, n, dv), np.nan)
    mask_next = mask.copy()
    margins = np.full((bsz, nh, tq, tk), np.nan)
    computed = np.zeros((bsz, nh, tq), dtype=bool)
    if rows is None:
        rows = [(b, h, i) for b in range(bsz) for h in range(nh) for i in range(tq)]
    by_head = {}
    for (b, h, i) in rows:
        by_head.setdefault((b, h), []).append(i)

    skipped_all = mask_to_bits(mask, tk)
    for (b, h), tiles in by_head.items():
        qh, kh, vh = _head(q, b, h), _head(k, b, h), _head(v, b, h)
        for i in tiles:
            r0, r1 = i * tile_q, min(n, (i + 1) * tile_q)
            o, flags, marg, stat = _row_tile(qh[r0:r1], kh, vh, skipped_all[b, h, i], i,
                                             tile_q=tile_q, tile_k=tile_k, scale=softmax_scale,
                                             log_eps=log_eps, descending=descending,
                                             dense_prefix=dense_prefix,
                                             in_step_skip=in_step_skip)
            out[b, h, r0:r1] = o
            margins[b, h, i] = marg
            computed[b, h, i] = True
            mask_next[b, h, i] = mask[b, h, i] | bits_to_mask(flags)
            if refresh:
                stats[b, h, i] = stat
                ref = tile_stats[b, h, i]
                if math.isnan(ref):
                    stats_next[b, h, i] = stat
                elif not (abs(stat - ref) <= refresh_delta):
                    mask_next[b, h, i] = 0          # valid bits cleared, reserved bits stay 0
                    stats_next[b, h, i] = np.nan
                    refreshed[b, h, i] = True
    if refresh:
        return StepResult(out=out, mask_next=mask_next, margins=margins, computed_rows=computed,
                          stats=stats, stats_next=stats_next, refreshed=refreshed)
    return StepResult(out=out, mask_next=mask_next, margins=margins, computed_rows=computed)


def run_chain_ref(inputs_for_step, steps: int, log_eps_schedule, *, batch: int, heads: int,
                  seq_len: int, tile_q: int, tile_k: int, softmax_scale: float,
                  order: str = "alt", dense_prefix: int = 0, rows=None,
                  in_step_skip: bool = False):
    """Run `steps` denoising steps from an empty mask. inputs_for_step(t) -> (q, k, v).
    Yields (t, mask_at_start, StepResult) per step."""
    mask = empty_mask(batch, heads, seq_len, tile_q, tile_k)
    for t in range(steps):
        q, k, v = inputs_for_step(t)
        res = lite_attn_step_ref(q, k, v, mask, tile_q=tile_q, tile_k=tile_k,
                                 softmax_scale=softmax_scale, log_eps=log_eps_schedule[t],
                                 step=t, order=order, dense_prefix=dense_prefix, rows=rows,
                                 in_step_skip=in_step_skip)
        yield t, mask, res
        mask = res.mask_next
