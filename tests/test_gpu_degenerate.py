"""Degenerate budgets and inputs against the oracle, through the C ABI:
- the boundary budgets log_eps = 0 and -1e-6, where a tile is flagged as soon as every valid
  row's tile maximum lies below its running maximum;
- logits of several hundred that grow along the key axis, so that the exponent reference of the
  online softmax moves on most tiles of an ascending pass;
- many short heads: more query tiles than resident workgroups, N a multiple of neither tile;
- NaN in one query row and in one key row: the output is NaN exactly where the oracle's is, no
  tile with a NaN margin is flagged, and everything else follows the oracle."""
import math

import numpy as np
import pytest
import torch

from gpu_util import (MARGIN_BAND, OUT_MAX, OUT_MEAN, device, from_mask_tensor, log,
                      make_attention, teacher_forced_chain, to_mask_tensor)
from oracle import lite_attn_step_ref, mask_to_bits
from workloads import Workload, derive, get_config

pytestmark = pytest.mark.gpu


class FixedInputs:
    """Per-step (q, k, v) given up front, in the shape of a workload."""

    def __init__(self, dev, per_step):
        self.device = dev
        self._steps = per_step

    def inputs(self, t):
        return self._steps[t]


@pytest.mark.parametrize("d", [64, 128])
def test_boundary_budgets(d):
    dev = device()
    base = get_config(5) if d == 64 else get_config(2)
    cfg = derive(base, name="boundary", heads=[8, 9] if d == 64 else [0, 1], grid=(2, 12, 20),
                 steps=3)
    cmp, mask = teacher_forced_chain(cfg, Workload(cfg, dev), 3, log_eps=[0.0, -1e-6, 0.0],
                                     label=f"log_eps 0 / -1e-6 D{d}")
    assert cmp.flags > 0, "the boundary budget flagged nothing"


@pytest.mark.parametrize("d", [64, 128])
def test_large_growing_logits(d):
    """Scores reach several hundred and grow with the key index: ascending passes move the
    exponent reference again and again. No budget (-inf): outputs only, mask untouched."""
    dev = device()
    base = get_config(5) if d == 64 else get_config(2)
    cfg = derive(base, name="large_logits", heads=[0, 1], grid=(1, 20, 35), steps=2)
    n = cfg.seq_len
    g = torch.Generator().manual_seed(1234)
    ramp = (1.0 + 7.0 * torch.arange(n, dtype=torch.float32) / n)[:, None]
    steps = []
    for _ in range(2):
        q = 2.0 * torch.randn(cfg.batch, cfg.heads, n, d, generator=g)
        k = 2.0 * torch.randn(cfg.batch, cfg.heads, n, d, generator=g) * ramp
        v = torch.randn(cfg.batch, cfg.heads, n, d, generator=g)
        steps.append(tuple(x.to(torch.bfloat16).to(dev) for x in (q, k, v)))
    s_max = float((steps[0][0].float() @ steps[0][1].float().transpose(-1, -2).contiguous()).abs().max())
    log(f"  largest |score| {s_max:.0f}")
    assert s_max > 200.0
    cmp, mask = teacher_forced_chain(cfg, FixedInputs(dev, steps), 2,
                                     log_eps=[-math.inf, -math.inf], label=f"large logits D{d}")
    assert cmp.flags == 0 and not mask.any()


def test_many_short_heads():
    """384 (batch, head) pairs of 200 tokens: 768 query tiles of 2 x 4 tiles each, more than
    the workgroups resident at once, so the persistent launch takes several rounds."""
    dev = device()
    cfg = derive(get_config(5), name="many_heads", batch=4, heads=list(range(16)) * 6,
                 grid=(1, 10, 20), steps=2)
    assert cfg.batch * cfg.heads * cfg.tiles_q > 512
    teacher_forced_chain(cfg, Workload(cfg, dev), 2, log_eps=[-12.0, -6.0], label="many heads")


def test_nan_rows():
    dev = device()
    cfg = derive(get_config(2), name="nan", heads=[0, 1, 2], grid=(1, 10, 30), steps=2)
    wl = Workload(cfg, dev)
    att = make_attention(cfg)
    tq, tk = att.tiles
    ref_mask = np.zeros(att.mask_shape, dtype=np.uint32)
    gmask = att.new_mask(dev)
    for t, le in enumerate([-6.0, -4.0]):
        q, k, v = (x.clone() for x in wl.inputs(t))
        q[0, 0, 37, :] = float("nan")     # one query row of head 0
        k[0, 1, 150, :] = float("nan")    # one key row of head 1 (key tile 2)
        out = torch.zeros_like(q)
        gmask.copy_(to_mask_tensor(ref_mask, dev))
        att.step(q, k, v, out, gmask, le, t)
        torch.cuda.synchronize()
        ref = lite_attn_step_ref(q.cpu(), k.cpu(), v.cpu(), ref_mask, tile_q=cfg.tile_q,
                                 tile_k=cfg.tile_k, softmax_scale=cfg.softmax_scale, log_eps=le,
                                 step=t, order=cfg.order)
        gout = out.double().cpu().numpy()
        gnan, rnan = np.isnan(gout), np.isnan(ref.out)
        assert rnan[0, 0, 37].all() and rnan[0, 1].all(), "the oracle's NaN pattern is not the expected one"
        assert np.array_equal(gnan, rnan), (
            f"step {t}: NaN pattern differs at {np.argwhere(gnan != rnan)[:4].tolist()}")
        d = np.abs(gout[~rnan] - ref.out[~rnan])
        log(f"  [nan] step {t}: finite max|d|={d.max():.3e} mean|d|={d.mean():.3e}")
        assert d.max() <= OUT_MAX and d.mean() <= OUT_MEAN
        gbits = mask_to_bits(from_mask_tensor(gmask), tk)
        rbits = mask_to_bits(ref.mask_next, tk)
        start = mask_to_bits(ref_mask, tk)
        nan_margin = np.isnan(ref.margins) & ~start        # visited tiles with a NaN margin
        assert nan_margin[0, 0, 0].any() and nan_margin[0, 1].any()
        assert not (gbits & nan_margin).any(), "a tile with a NaN margin was flagged"
        near = np.abs(np.nan_to_num(ref.margins, nan=np.inf)) <= MARGIN_BAND
        bad = (gbits != rbits) & ~near
        assert not bad.any(), f"step {t}: {int(bad.sum())} mask bits differ"
        # head 2 has no NaN: it must still skip normally on the second step's budget
        ref_mask = ref.mask_next
    assert mask_to_bits(ref_mask, tk)[0, 2].any(), "the NaN-free head flagged nothing"
