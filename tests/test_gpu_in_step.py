"""GPU parity of the in-step-skip option (LITE_ATTN_OPT_IN_STEP_SKIP): a tile flagged while it is
visited is also left out of the step's own output. The oracle's in-step variant is the
reference (teacher-forced, same tolerances as the plain method); the flags, and so the masks,
must be the same as without the option."""
import numpy as np
import pytest
import torch

from gpu_util import device, from_mask_tensor, log, make_attention, teacher_forced_chain
from test_gpu_parity import _sample_rows
from workloads import Workload, derive, get_config

pytestmark = pytest.mark.gpu

SMALL = [
    ("ins_tiny_ref", 1, {}, 4),
    ("ins_wan14b_recipe_1200", 3, dict(heads=[0, 7], grid=(2, 15, 40)), 4),
    ("ins_hunyuan_recipe_976_prefix", 4, dict(heads=[0, 1], grid=(2, 9, 40), prefix=256,
                                              dense_prefix=256), 3),
    ("ins_stress_recipe_1000", 5, dict(heads=[9, 10], grid=(1, 25, 40)), 6),
]


@pytest.mark.parametrize("label,cid,kw,steps", SMALL, ids=[s[0] for s in SMALL])
def test_in_step_small_full_parity(label, cid, kw, steps):
    dev = device()
    cfg = derive(get_config(cid), name=label, steps=steps, **kw) if kw else get_config(cid)
    cmp, _ = teacher_forced_chain(cfg, Workload(cfg, dev), steps, label=label, in_step_skip=True)
    assert cmp.flags > 0, "the case must flag tiles to exercise the option"


@pytest.mark.parametrize("order", ["asc", "alt"])
@pytest.mark.parametrize("tile_q", [64, 128])
def test_in_step_orders_and_tile_q(order, tile_q):
    dev = device()
    cfg = derive(get_config(5), name="ins_orders", heads=[8, 12], grid=(2, 12, 20), steps=4,
                 tile_q=tile_q)
    teacher_forced_chain(cfg, Workload(cfg, dev), 4, order=order, label=f"ins-{order}-tq{tile_q}",
                         in_step_skip=True)


@pytest.mark.parametrize("dtype_name,d", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_in_step_dtype_headdim_variants(dtype_name, d):
    dev = device()
    base = get_config(2) if d == 128 else get_config(5)
    cfg = derive(base, name="ins_variant", batch=1, heads=[0, 1], grid=(2, 7, 33), steps=3,
                 dtype=torch.bfloat16 if dtype_name == "bf16" else torch.float32)
    teacher_forced_chain(cfg, Workload(cfg, dev), 3, label=f"ins-{dtype_name}-D{d}",
                         in_step_skip=True)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_in_step_full_size_sampled_parity(cid):
    """Every step of each bf16 workload's schedule at full size, on sampled query tiles (with
    the HunyuanVideo shape's dense-prefix tiles and the stress shape's D = 64)."""
    dev = device()
    cfg = get_config(cid)
    rows = _sample_rows(cfg, np.random.default_rng(33 + cid), n_heads=2, per_head=2)
    log(f"== in-step {cfg.name} full size, {len(rows)} sampled query tiles, {cfg.steps} steps")
    wl = Workload(cfg, dev)
    teacher_forced_chain(cfg, wl, cfg.steps, rows=rows, label="ins-" + cfg.name,
                         in_step_skip=True)
    wl.drop_cache()
    torch.cuda.empty_cache()


def test_in_step_free_chain_has_the_same_masks():
    """Free-running chains with and without the option produce identical masks (the flags do
    not depend on the option), and outputs that differ only where tiles were flagged."""
    dev = device()
    cfg = derive(get_config(5), name="ins_chain", heads=[0, 9], grid=(2, 16, 32), steps=5)
    wl = Workload(cfg, dev)
    plain = make_attention(cfg)
    ins = make_attention(cfg, in_step_skip=True)
    m0, m1 = plain.new_mask(dev), ins.new_mask(dev)
    for t in range(cfg.steps):
        q, k, v = wl.inputs(t)
        o0, o1 = torch.empty_like(q), torch.empty_like(q)
        before = from_mask_tensor(m0)
        plain.step(q, k, v, o0, m0, cfg.log_eps[t], t)
        ins.step(q, k, v, o1, m1, cfg.log_eps[t], t)
        torch.cuda.synchronize()
        assert torch.equal(m0, m1), f"step {t}: masks differ"
        new_flags = int(np.unpackbits((from_mask_tensor(m0) & ~before).view(np.uint8)).sum())
        d = (o0.float() - o1.float()).abs().max().item()
        log(f"  step {t}: new flags {new_flags}, max|plain - in-step| = {d:.3e}")
        if new_flags == 0:
            assert d < 1e-5
        assert d < 2e-2


def test_in_step_with_a_loose_budget_follows_the_in_step_definition():
    """A budget close to 0 flags tiles that still carry real softmax mass, so the in-step output
    differs from the plain one by far more than the tolerance; the GPU must follow the in-step
    definition (teacher-forced against the oracle's in-step variant)."""
    from oracle import empty_mask, lite_attn_step_ref
    dev = device()
    cfg = derive(get_config(5), name="ins_loose", heads=[8, 9, 10, 11], grid=(1, 16, 32), steps=3)
    wl = Workload(cfg, dev)
    gap = 0.0
    for t in range(cfg.steps):
        q, k, v = (x.cpu() for x in wl.inputs(t))
        kw = dict(tile_q=cfg.tile_q, tile_k=cfg.tile_k, softmax_scale=cfg.softmax_scale,
                  log_eps=-0.5, step=t, order=cfg.order)
        m = empty_mask(cfg.batch, cfg.heads, cfg.seq_len, cfg.tile_q, cfg.tile_k)
        plain = lite_attn_step_ref(q, k, v, m, **kw)
        ins = lite_attn_step_ref(q, k, v, m, in_step_skip=True, **kw)
        gap = max(gap, float(np.nanmax(np.abs(plain.out - ins.out))))
    log(f"  oracle plain vs in-step max|d| = {gap:.3f}")
    assert gap > 0.06, "the case must separate the two definitions"
    cmp, _ = teacher_forced_chain(cfg, wl, 3, label="ins-loose", in_step_skip=True,
                                  log_eps=[-0.5, -0.5, -0.5])
    assert cmp.flags > 0
