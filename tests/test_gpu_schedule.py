"""Scheduled steps (lite_attn_step_scheduled): the same results as lite_attn_step, bit for bit,
and the documented tile order (heavy query tiles first in natural order, then the middle tiles
head by head, heads by decreasing work, each head in the step's traversal direction, then the
short tiles in traversal order)."""
import numpy as np
import pytest
import torch

from gpu_util import device, from_mask_tensor, log, make_attention
from oracle import mask_to_bits
from workloads import Workload, derive, get_config

pytestmark = pytest.mark.gpu


def tail_max() -> int:
    """Short tiles the library puts last at most: eight per workgroup slot, two slots per CU."""
    return 16 * torch.cuda.get_device_properties(0).multi_processor_count


def expected_order(mask_np: np.ndarray, tiles_k: int, tiles_q: int, descending: bool,
                   tail: int) -> np.ndarray:
    """Reference tile order for a mask [B, H, Tq, W]:
    - heavy tiles (visiting at least half of all key tiles and at least four times the mean)
      first, in natural order;
    - short tiles last: the non-heavy tiles with a visit count below the largest cut c that
      leaves at most min(tail, non-heavy // 4) of them (counts of 2048 are never short), in the
      step's traversal order (natural order, reversed on descending steps);
    - between them the middle tiles, head by head, heads by decreasing middle work (sum of their
      visit counts; ties by index), each head's tiles in the direction of the step's key
      traversal (natural head order above 1024 heads)."""
    bits = mask_to_bits(mask_np, tiles_k).reshape(-1, tiles_k)
    count = (tiles_k - bits.sum(axis=1)).astype(np.int64)
    n = count.size
    heavy = (2 * count >= tiles_k) & (count * n >= 4 * count.sum())
    k = min(tail, (n - int(heavy.sum())) // 4)
    rest = count[~heavy]
    rest = rest[rest < 2048]
    cut = max(c for c in range(2049) if int((rest < c).sum()) <= k)
    short = ~heavy & (count < cut)
    middle = ~heavy & ~short
    order = list(np.nonzero(heavy)[0])
    heads = n // tiles_q
    if heads > 1024:
        order += list(np.nonzero(middle)[0])
    else:
        work = [int(count[h * tiles_q:(h + 1) * tiles_q][middle[h * tiles_q:(h + 1) * tiles_q]].sum())
                for h in range(heads)]
        for h in sorted(range(heads), key=lambda h: (-work[h], h)):
            rows = range(tiles_q - 1, -1, -1) if descending else range(tiles_q)
            order += [h * tiles_q + i for i in rows if middle[h * tiles_q + i]]
    tail_tiles = list(np.nonzero(short)[0])
    order += tail_tiles[::-1] if descending else tail_tiles
    return np.array(order)


CASES = [
    ("sched_stress", 5, dict(heads=[0, 9, 10], grid=(2, 16, 32)), 5),
    ("sched_hunyuan_prefix", 4, dict(heads=[0, 1], grid=(2, 9, 40), prefix=256, dense_prefix=256), 4),
    ("sched_tiny_fp32", 1, {}, 4),
]


@pytest.mark.parametrize("label,cid,kw,steps", CASES, ids=[c[0] for c in CASES])
def test_scheduled_step_matches_plain_step(label, cid, kw, steps):
    dev = device()
    cfg = derive(get_config(cid), name=label, steps=steps, **kw) if kw else get_config(cid)
    wl = Workload(cfg, dev)
    att = make_attention(cfg)
    tq, tk = att.tiles
    ws = att.new_workspace(dev)
    m_plain, m_sched = att.new_mask(dev), att.new_mask(dev)
    n = cfg.batch * cfg.heads * tq
    for t in range(steps):
        q, k, v = wl.inputs(t)
        o_plain, o_sched = torch.empty_like(q), torch.empty_like(q)
        start = from_mask_tensor(m_sched)
        att.step(q, k, v, o_plain, m_plain, cfg.log_eps[t], t)
        att.step(q, k, v, o_sched, m_sched, cfg.log_eps[t], t, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o_plain, o_sched), f"{label} step {t}: outputs differ"
        assert torch.equal(m_plain, m_sched), f"{label} step {t}: masks differ"
        perm = ws[:4 * n].view(torch.int32).cpu().numpy()
        desc = cfg.order == "alt" and t % 2 == 1
        assert np.array_equal(perm, expected_order(start, tk, tq, desc, tail_max())), \
            f"{label} step {t}: order"
        log(f"  [{label}] step {t}: first tiles {perm[:6].tolist()}")


def test_scheduled_full_size_order_and_result():
    """At the HunyuanVideo shape (dense prefix rows never skip), one sparse step: the prefix
    query tiles of every head come first, and the results equal the plain step."""
    dev = device()
    cfg = get_config(4)
    wl = Workload(cfg, dev)
    att = make_attention(cfg)
    tq, tk = att.tiles
    ws = att.new_workspace(dev)
    mask = att.new_mask(dev)
    for t in range(2):
        q, k, v = wl.inputs(t)
        out = torch.empty_like(q)
        att.step(q, k, v, out, mask, cfg.log_eps[t], t)
    q, k, v = wl.inputs(2)
    m1, m2 = mask.clone(), mask.clone()
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    start = from_mask_tensor(m2)
    att.step(q, k, v, o1, m1, cfg.log_eps[2], 2)
    att.step(q, k, v, o2, m2, cfg.log_eps[2], 2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2)
    n = cfg.batch * cfg.heads * tq
    perm = ws[:4 * n].view(torch.int32).cpu().numpy()
    assert np.array_equal(perm, expected_order(start, tk, tq, False, tail_max()))
    # the prefix query tiles (rows [0, 256) of every head) are never skipped, so in a sparse
    # step they are heavy and run first
    bits = mask_to_bits(start, tk).reshape(-1, tk)
    count = (tk - bits.sum(axis=1)).astype(np.int64)
    n_heavy = int(((2 * count >= tk) & (count * count.size >= 4 * count.sum())).sum())
    prefix_tiles = [h * tq + i for h in range(cfg.heads) for i in range(2)]
    log(f"  heavy tiles: {n_heavy}")
    assert set(prefix_tiles) <= set(perm[:n_heavy].tolist())
    wl.drop_cache()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("label,cid,kw,steps", CASES[:2], ids=[c[0] + "_in_step" for c in CASES[:2]])
def test_scheduled_in_step_matches_plain_in_step(label, cid, kw, steps):
    """The schedule composes with in-step skip: with the option on, the scheduled step equals the
    plain step bit for bit."""
    dev = device()
    cfg = derive(get_config(cid), name=label + "_ins", steps=steps, **kw)
    wl = Workload(cfg, dev)
    att = make_attention(cfg, in_step_skip=True)
    ws = att.new_workspace(dev)
    m_plain, m_sched = att.new_mask(dev), att.new_mask(dev)
    for t in range(steps):
        q, k, v = wl.inputs(t)
        o_plain, o_sched = torch.empty_like(q), torch.empty_like(q)
        att.step(q, k, v, o_plain, m_plain, cfg.log_eps[t], t)
        att.step(q, k, v, o_sched, m_sched, cfg.log_eps[t], t, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o_plain, o_sched), f"{label} step {t}: outputs differ"
        assert torch.equal(m_plain, m_sched), f"{label} step {t}: masks differ"
