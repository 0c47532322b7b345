"""Divergence-triggered refresh (lite_attn_step_refresh) against the oracle: teacher-forced per
step (mask rows and references copied from the oracle before each step). Outputs within the
usual tolerances; mask rows bit-exact except tiles whose QK-Skip margin, or whose refresh
decision (|statistic - reference| - delta), is within 1e-3 of its threshold; statistics within
1e-3 (relative) of the oracle's."""
import math

import numpy as np
import pytest
import torch

from gpu_util import (MARGIN_BAND, OUT_MAX, OUT_MEAN, device, from_mask_tensor, log,
                      make_attention, to_mask_tensor)
from test_gpu_parity import _sample_rows
from oracle import lite_attn_step_ref, mask_to_bits
from workloads import Workload, derive, get_config

pytestmark = pytest.mark.gpu


def refresh_chain(cfg, wl, steps, delta, *, log_eps=None, inputs=None, label=""):
    dev = wl.device
    att = make_attention(cfg)
    tq, tk = att.tiles
    B, H = cfg.batch, cfg.heads
    ref_mask = np.zeros(att.mask_shape, dtype=np.uint32)
    ref_stats = np.full((B, H, tq), np.nan)
    gmask = att.new_mask(dev)
    gstats = att.new_tile_stats(dev)
    worst_out, sum_out, cnt_out, refreshed_total = 0.0, 0.0, 0, 0
    for t in range(steps):
        le = cfg.log_eps[t] if log_eps is None else log_eps[t]
        q, k, v = wl.inputs(t) if inputs is None else inputs(t)
        out = torch.full_like(q, float("nan"))
        gmask.copy_(to_mask_tensor(ref_mask, dev))
        gstats.copy_(torch.from_numpy(ref_stats.astype(np.float32)).to(dev))
        att.step(q, k, v, out, gmask, le, t, tile_stats=gstats, refresh_delta=delta)
        torch.cuda.synchronize()
        ref = lite_attn_step_ref(q.cpu(), k.cpu(), v.cpu(), ref_mask, tile_q=cfg.tile_q,
                                 tile_k=cfg.tile_k, softmax_scale=cfg.softmax_scale, log_eps=le,
                                 step=t, order=cfg.order, dense_prefix=cfg.dense_prefix,
                                 tile_stats=ref_stats, refresh_delta=delta)
        d = np.abs(out.double().cpu().numpy() - ref.out)
        worst_out = max(worst_out, float(d.max()))
        sum_out += float(d.sum())
        cnt_out += d.size
        # refresh decisions near the threshold may differ (float32 vs float64 statistics)
        move = np.abs(ref.stats - ref_stats)
        near_refresh = np.abs(move - delta) <= 1e-3 * np.maximum(1.0, np.abs(ref.stats))
        gbits = mask_to_bits(from_mask_tensor(gmask), tk)
        rbits = mask_to_bits(ref.mask_next, tk)
        near_margin = np.abs(np.nan_to_num(ref.margins, nan=np.inf)) <= MARGIN_BAND
        bad = (gbits != rbits) & ~near_margin & ~near_refresh[..., None]
        assert not bad.any(), f"{label} step {t}: {int(bad.sum())} mask bits differ"
        gs = gstats.double().cpu().numpy()
        both_nan = np.isnan(gs) & np.isnan(ref.stats_next)
        close = np.abs(gs - ref.stats_next) <= 1e-3 * np.maximum(1.0, np.abs(ref.stats_next))
        ok = both_nan | close | near_refresh
        assert ok.all(), f"{label} step {t}: statistics differ at {np.argwhere(~ok)[:4].tolist()}"
        refreshed_total += int(ref.refreshed.sum())
        log(f"  [{label}] step {t}: refreshed {int(ref.refreshed.sum())} rows, "
            f"skipped(next) {rbits.mean():.3f}")
        ref_mask, ref_stats = ref.mask_next, ref.stats_next
    mean_out = sum_out / max(1, cnt_out)
    log(f"[{label}] out max|d|={worst_out:.3e} mean|d|={mean_out:.3e} refreshed={refreshed_total}")
    assert worst_out <= OUT_MAX and mean_out <= OUT_MEAN
    return refreshed_total


def test_refresh_with_infinite_delta_is_the_plain_chain():
    dev = device()
    cfg = derive(get_config(5), name="rf_inf", heads=[8, 9], grid=(2, 16, 32), steps=4)
    n = refresh_chain(cfg, Workload(cfg, dev), 4, math.inf, label="rf-inf")
    assert n == 0


@pytest.mark.parametrize("cid,kw,steps,delta", [
    (3, dict(heads=[0, 7], grid=(2, 15, 40)), 4, 0.5),
    (5, dict(heads=[8, 12], grid=(2, 16, 32)), 5, 0.3),
    (1, {}, 4, 0.2),
])
def test_refresh_parity(cid, kw, steps, delta):
    dev = device()
    cfg = derive(get_config(cid), name="rf", steps=steps, **kw) if kw else get_config(cid)
    refresh_chain(cfg, Workload(cfg, dev), steps, delta, label=f"rf-{cfg.name}-{delta}")


def test_refresh_clears_rows_when_attention_moves():
    """Keys rolled by half the sequence at step 2: every row's best keys land in tiles that the
    earlier steps flagged, the statistic falls, and rows are cleared."""
    dev = device()
    cfg = derive(get_config(5), name="rf_roll", heads=[8, 9], grid=(2, 16, 32), steps=4)
    wl = Workload(cfg, dev)

    def inputs(t):
        q, k, v = wl.inputs(t)
        if t >= 2:
            k = torch.roll(k, shifts=cfg.seq_len // 2, dims=2).contiguous()
        return q, k, v
    n = refresh_chain(cfg, wl, 4, 1.0, inputs=inputs, label="rf-roll")
    assert n > 0


def test_refresh_full_size_sampled_parity():
    """The 75600-token workload over its whole schedule at full size, teacher-forced on sampled
    query tiles: before each step the sampled tiles' mask rows and references are set to the
    oracle's (the others keep the GPU's own), and the sampled outputs, mask rows and statistics
    are compared as in the small cases."""
    dev = device()
    cfg = get_config(3)
    delta = 0.2
    att = make_attention(cfg)
    tq, tk = att.tiles
    B, H = cfg.batch, cfg.heads
    rows = _sample_rows(cfg, np.random.default_rng(77), n_heads=2, per_head=2)
    sel = np.zeros((B, H, tq), dtype=bool)
    for (b, h, i) in rows:
        sel[b, h, i] = True
    heads = sorted({(b, h) for (b, h, _) in rows})
    log(f"== refresh {cfg.name} full size, {len(rows)} sampled query tiles, delta {delta}")
    wl = Workload(cfg, dev)
    ref_mask = np.zeros(att.mask_shape, dtype=np.uint32)
    ref_stats = np.full((B, H, tq), np.nan)
    gmask = att.new_mask(dev)
    gstats = att.new_tile_stats(dev)
    worst, total, n_el, refreshed = 0.0, 0.0, 0, 0
    for t in range(cfg.steps):
        le = cfg.log_eps[t]
        q, k, v = wl.inputs(t)
        out = torch.full_like(q, float("nan"))
        cur = from_mask_tensor(gmask)
        cur[sel] = ref_mask[sel]
        gmask.copy_(to_mask_tensor(cur, dev))
        gs = gstats.cpu().numpy()
        gs[sel] = ref_stats[sel]
        gstats.copy_(torch.from_numpy(gs.astype(np.float32)).to(dev))
        att.step(q, k, v, out, gmask, le, t, tile_stats=gstats, refresh_delta=delta)
        torch.cuda.synchronize()
        gbits_all = mask_to_bits(from_mask_tensor(gmask), tk)
        gstats_all = gstats.double().cpu().numpy()
        gout = out
        for (b, h) in heads:
            tiles = [i for (bb, hh, i) in rows if (bb, hh) == (b, h)]
            r = lite_attn_step_ref(q[b:b + 1, h:h + 1].cpu(), k[b:b + 1, h:h + 1].cpu(),
                                   v[b:b + 1, h:h + 1].cpu(), ref_mask[b:b + 1, h:h + 1],
                                   tile_q=cfg.tile_q, tile_k=cfg.tile_k,
                                   softmax_scale=cfg.softmax_scale, log_eps=le, step=t,
                                   order=cfg.order, dense_prefix=cfg.dense_prefix,
                                   rows=[(0, 0, i) for i in tiles],
                                   tile_stats=ref_stats[b:b + 1, h:h + 1], refresh_delta=delta)
            for i in tiles:
                r0, r1 = i * cfg.tile_q, min(cfg.seq_len, (i + 1) * cfg.tile_q)
                d = np.abs(gout[b, h, r0:r1].double().cpu().numpy() - r.out[0, 0, r0:r1])
                worst = max(worst, float(d.max()))
                total += float(d.sum())
                n_el += d.size
                move = abs(r.stats[0, 0, i] - ref_stats[b, h, i])
                near_refresh = abs(move - delta) <= 1e-3 * max(1.0, abs(r.stats[0, 0, i]))
                near_margin = np.abs(np.nan_to_num(r.margins[0, 0, i], nan=np.inf)) <= MARGIN_BAND
                rbits = mask_to_bits(r.mask_next[0:1, 0:1, i:i + 1], tk)[0, 0, 0]
                bad = (gbits_all[b, h, i] != rbits) & ~near_margin & ~near_refresh
                assert not bad.any(), f"step {t} tile {(b, h, i)}: {int(bad.sum())} bits differ"
                want, got = r.stats_next[0, 0, i], gstats_all[b, h, i]
                ok = (np.isnan(want) and np.isnan(got)) or near_refresh or \
                    abs(got - want) <= 1e-3 * max(1.0, abs(want))
                assert ok, f"step {t} tile {(b, h, i)}: statistic {got} against {want}"
                ref_mask[b, h, i] = r.mask_next[0, 0, i]
                ref_stats[b, h, i] = r.stats_next[0, 0, i]
                refreshed += int(r.refreshed[0, 0, i])
        log(f"  [refresh-{cfg.name}] step {t}: skipped(next, sampled) "
            f"{mask_to_bits(ref_mask, tk)[sel].mean():.3f} refreshed so far {refreshed} "
            f"max|d| so far {worst:.2e}")
    mean = total / max(1, n_el)
    log(f"[refresh-{cfg.name}] out max|d|={worst:.3e} mean|d|={mean:.3e} refreshed={refreshed}")
    assert worst <= OUT_MAX and mean <= OUT_MEAN
    wl.drop_cache()
    torch.cuda.empty_cache()
