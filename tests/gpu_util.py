"""Helpers for the GPU parity tests: run the HIP path through the C ABI, run the oracle on the
same inputs (teacher-forced: both start each step from the oracle's mask), compare."""
import math
import sys

import numpy as np
import torch

import temporally_sparse_attention_amd as tsa
from oracle import lite_attn_step_ref, mask_to_bits

OUT_MAX = 2e-2       # max |GPU - oracle| over valid output elements
OUT_MEAN = 2e-3      # mean |GPU - oracle|
MARGIN_BAND = 1e-3   # tiles whose decision margin is this close to 0 may differ


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_mask_tensor(mask_np: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(mask_np, dtype=np.uint32).view(np.int32)).to(dev)


def from_mask_tensor(mask: torch.Tensor) -> np.ndarray:
    return mask.cpu().numpy().view(np.uint32).copy()


class Comparison:
    def __init__(self):
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.count = 0
        self.near = 0
        self.mismatch = 0
        self.tiles = 0
        self.flags = 0

    def add_out(self, gpu: np.ndarray, ref: np.ndarray):
        d = np.abs(gpu.astype(np.float64) - ref)
        assert np.all(np.isfinite(gpu)), "non-finite GPU output"
        if d.size:
            self.max_abs = max(self.max_abs, float(d.max()))
            self.sum_abs += float(d.sum())
            self.count += d.size

    def add_mask(self, gpu_bits: np.ndarray, ref_bits: np.ndarray, margins: np.ndarray,
                 start_bits: np.ndarray):
        """Adds one step's mask comparison; returns that step's (mismatches beyond the margin
        band, near-threshold tiles, near-threshold tiles that differ)."""
        near = np.abs(np.nan_to_num(margins, nan=np.inf)) <= MARGIN_BAND
        diff = gpu_bits != ref_bits
        step = (int((diff & ~near).sum()), int(near.sum()), int((diff & near).sum()))
        self.near += step[1]
        self.mismatch += step[0]
        self.tiles += gpu_bits.size
        self.flags += int((ref_bits & ~start_bits).sum())
        return step

    @property
    def mean_abs(self):
        return self.sum_abs / max(1, self.count)

    def check(self, label=""):
        log(f"[{label}] out max|d|={self.max_abs:.3e} mean|d|={self.mean_abs:.3e} "
            f"mask mismatches={self.mismatch} near-threshold={self.near} new flags={self.flags} "
            f"tiles={self.tiles}")
        assert self.mismatch == 0, f"{label}: {self.mismatch} mask bits differ beyond the margin band"
        assert self.max_abs <= OUT_MAX, f"{label}: max|d| {self.max_abs}"
        assert self.mean_abs <= OUT_MEAN, f"{label}: mean|d| {self.mean_abs}"


def make_attention(cfg, **over):
    kw = dict(tile_q=cfg.tile_q, tile_k=cfg.tile_k,
              dtype="bf16" if cfg.dtype == torch.bfloat16 else "fp32",
              softmax_scale=cfg.softmax_scale, order=cfg.order, dense_prefix=cfg.dense_prefix)
    kw.update(over)
    return tsa.LiteAttention(cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, **kw)


def teacher_forced_chain(cfg, workload, steps, *, rows=None, att=None, order=None,
                         scale=None, label="", log_eps=None, in_step_skip=False, workspace=None,
                         make_out=None):
    """Run `steps` steps. Before each step the GPU mask rows under test are overwritten with
    the oracle's mask; outputs and new mask rows are compared on `rows` (default: all). With a
    workspace the GPU runs the scheduled step (lite_attn_step_scheduled). make_out(q) allocates
    the output (default: a NaN-filled tensor like q)."""
    dev = workload.device
    order = order or cfg.order
    scale = cfg.softmax_scale if scale is None else scale
    att = att or make_attention(cfg, order=order, softmax_scale=scale, in_step_skip=in_step_skip)
    tq, tk = att.tiles
    B, H = cfg.batch, cfg.heads
    ref_mask = np.zeros(att.mask_shape, dtype=np.uint32)
    gpu_mask = att.new_mask(dev)
    cmp = Comparison()
    sel = None
    if rows is not None:
        sel = np.zeros((B, H, tq), dtype=bool)
        for (b, h, i) in rows:
            sel[b, h, i] = True
    for t in range(steps):
        le = cfg.log_eps[t] if log_eps is None else log_eps[t]
        q, k, v = workload.inputs(t)
        out = make_out(q) if make_out is not None else torch.full_like(q, float("nan"))
        if sel is None:
            gpu_mask.copy_(to_mask_tensor(ref_mask, dev))
        else:
            cur = from_mask_tensor(gpu_mask)
            cur[sel] = ref_mask[sel]
            gpu_mask.copy_(to_mask_tensor(cur, dev))
        att.step(q, k, v, out, gpu_mask, le, t, workspace=workspace)
        torch.cuda.synchronize()
        qc, kc, vc = (q.cpu(), k.cpu(), v.cpu()) if sel is None else (q, k, v)
        if sel is not None:
            # only the heads that hold sampled rows travel to the host
            heads = sorted({(b, h) for (b, h, _) in rows})
            ref = None
            ref_out = np.full(tuple(q.shape), np.nan)
            margins = np.full((B, H, tq, tk), np.nan)
            new_mask = ref_mask.copy()
            for (b, h) in heads:
                tiles = [i for (bb, hh, i) in rows if (bb, hh) == (b, h)]
                r = lite_attn_step_ref(q[b:b + 1, h:h + 1].cpu(), k[b:b + 1, h:h + 1].cpu(),
                                       v[b:b + 1, h:h + 1].cpu(), ref_mask[b:b + 1, h:h + 1],
                                       tile_q=att.handle.cfg.tile_q, tile_k=cfg.tile_k,
                                       softmax_scale=scale, log_eps=le, step=t, order=order,
                                       dense_prefix=cfg.dense_prefix,
                                       rows=[(0, 0, i) for i in tiles],
                                       in_step_skip=in_step_skip)
                for i in tiles:
                    r0, r1 = i * att.handle.cfg.tile_q, min(cfg.seq_len, (i + 1) * att.handle.cfg.tile_q)
                    ref_out[b, h, r0:r1] = r.out[0, 0, r0:r1]
                    margins[b, h, i] = r.margins[0, 0, i]
                    new_mask[b, h, i] = r.mask_next[0, 0, i]
            gout = out.double().cpu().numpy()
            for (b, h, i) in rows:
                r0, r1 = i * att.handle.cfg.tile_q, min(cfg.seq_len, (i + 1) * att.handle.cfg.tile_q)
                cmp.add_out(gout[b, h, r0:r1], ref_out[b, h, r0:r1])
            gbits = mask_to_bits(from_mask_tensor(gpu_mask), tk)[sel]
            per_step = cmp.add_mask(gbits, mask_to_bits(new_mask, tk)[sel], margins[sel],
                                    mask_to_bits(ref_mask, tk)[sel])
            ref_mask = new_mask
        else:
            ref = lite_attn_step_ref(qc, kc, vc, ref_mask, tile_q=att.handle.cfg.tile_q,
                                     tile_k=cfg.tile_k, softmax_scale=scale, log_eps=le, step=t,
                                     order=order, dense_prefix=cfg.dense_prefix,
                                     in_step_skip=in_step_skip)
            cmp.add_out(out.double().cpu().numpy(), ref.out)
            per_step = cmp.add_mask(mask_to_bits(from_mask_tensor(gpu_mask), tk),
                                    mask_to_bits(ref.mask_next, tk), ref.margins,
                                    mask_to_bits(ref_mask, tk))
            ref_mask = ref.mask_next
        sk = mask_to_bits(ref_mask, tk)
        sk = sk[sel].mean() if sel is not None else sk.mean()
        log(f"  [{label}] step {t}: log_eps={le:.4g} skipped(next, compared rows)={sk:.3f} "
            f"mismatches beyond band={per_step[0]} near-threshold={per_step[1]} "
            f"(differing {per_step[2]}) max|d| so far={cmp.max_abs:.2e}")
    cmp.check(label)
    return cmp, ref_mask
