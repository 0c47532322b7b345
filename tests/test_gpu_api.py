"""GPU behaviour of the C ABI beyond parity chains: edge sizes, degenerate masks, reserved
bits, strided inputs, reset/popcount, determinism, -inf budgets, monotonicity."""
import math

import numpy as np
import pytest
import torch

import temporally_sparse_attention_amd as tsa
from gpu_util import Comparison, device, from_mask_tensor, log, make_attention, to_mask_tensor
from oracle import bits_to_mask, lite_attn_step_ref, mask_geometry, mask_to_bits

pytestmark = pytest.mark.gpu


def _rand_inputs(B, H, N, D, dtype, seed, spread=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda s: (torch.randn(B, H, N, D, generator=g) * s).to(dtype)
    return mk(spread), mk(spread), mk(1.0)


def _step_both(B, H, N, D, dtype, mask_np, log_eps, step, tile_q=128, order="alt", prefix=0,
               seed=0, spread=1.5, scale=1.0):
    dev = device()
    q, k, v = _rand_inputs(B, H, N, D, dtype, seed, spread)
    att = tsa.LiteAttention(B, H, N, D, tile_q=tile_q, dtype="bf16" if dtype == torch.bfloat16 else "fp32",
                            softmax_scale=scale, order=order, dense_prefix=prefix)
    out = torch.full((B, H, N, D), float("nan"), dtype=dtype, device=dev)
    mask = to_mask_tensor(mask_np, dev)
    att.step(q.to(dev), k.to(dev), v.to(dev), out, mask, log_eps, step)
    torch.cuda.synchronize()
    ref = lite_attn_step_ref(q, k, v, mask_np, tile_q=tile_q, tile_k=64, softmax_scale=scale,
                             log_eps=log_eps, step=step, order=order, dense_prefix=prefix)
    return out.double().cpu().numpy(), from_mask_tensor(mask), ref


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 129, 191, 300])
def test_edge_lengths(n):
    tq, tk, w = mask_geometry(n, 128, 64)
    out, m, ref = _step_both(1, 2, n, 128, torch.bfloat16, np.zeros((1, 2, tq, w), np.uint32),
                             -2.0, 0, seed=n)
    c = Comparison()
    c.add_out(out, ref.out)
    c.add_mask(mask_to_bits(m, tk), mask_to_bits(ref.mask_next, tk), ref.margins,
               np.zeros((1, 2, tq, tk), bool))
    c.check(f"N={n}")


def test_random_masks_all_skipped_rows_and_reserved_bits():
    n, D = 1000, 64
    tq, tk, w = mask_geometry(n, 128, 64)    # Tk = 16: bits 16..31 of the word are reserved
    rng = np.random.default_rng(5)
    bits = rng.random((2, 3, tq, tk)) < 0.5
    bits[0, 0, 3, :] = True                  # a query tile with nothing left to visit
    mask = bits_to_mask(bits)
    mask[1, 2, :, 0] |= np.uint32(0xFFFF0000)  # reserved bits set: must be left alone
    ref_in = bits_to_mask(bits)
    out, m, ref = _step_both(2, 3, n, D, torch.bfloat16, mask, -3.0, 1, seed=11)
    ref_reserved = lite_attn_step_ref(*_rand_inputs(2, 3, n, D, torch.bfloat16, 11, 1.5), ref_in,
                                      tile_q=128, tile_k=64, softmax_scale=1.0, log_eps=-3.0,
                                      step=1, order="alt")
    c = Comparison()
    c.add_out(out, ref_reserved.out)
    c.add_mask(mask_to_bits(m, tk), mask_to_bits(ref_reserved.mask_next, tk),
               ref_reserved.margins, bits)
    c.check("random masks")
    assert np.all(out[0, 0, 3 * 128:4 * 128] == 0.0)          # empty row tile -> zeros
    assert np.all((m[1, 2, :, 0] & np.uint32(0xFFFF0000)) == np.uint32(0xFFFF0000))
    assert not np.any(mask_to_bits(mask, tk) & ~mask_to_bits(m, tk))  # nothing cleared


def test_no_skip_budget_is_dense_attention_and_mask_untouched():
    n, D = 700, 128
    tq, tk, w = mask_geometry(n, 128, 64)
    out, m, ref = _step_both(1, 2, n, D, torch.bfloat16, np.zeros((1, 2, tq, w), np.uint32),
                             -math.inf, 0, seed=3, spread=2.0)
    assert not m.any()
    c = Comparison()
    c.add_out(out, ref.out)
    c.check("-inf budget")


def test_dense_prefix_exemption():
    n, D, P = 900, 128, 200
    tq, tk, w = mask_geometry(n, 128, 64)
    for step in (0, 1):
        out, m, ref = _step_both(1, 2, n, D, torch.bfloat16, np.zeros((1, 2, tq, w), np.uint32),
                                 -1.0, step, prefix=P, seed=21, spread=2.0)
        bits = mask_to_bits(m, tk)
        assert not bits[:, :, :2].any() and not bits[:, :, :, :4].any()
        c = Comparison()
        c.add_out(out, ref.out)
        c.add_mask(bits, mask_to_bits(ref.mask_next, tk), ref.margins, np.zeros_like(bits))
        c.check(f"prefix step {step}")


def test_strided_inputs_from_packed_qkv():
    """q, k, v as views of one [B, N, 3, H, D] tensor (stride_n = 3*H*D, stride_h = D)."""
    dev = device()
    B, H, N, D = 2, 3, 500, 128
    g = torch.Generator(device="cpu").manual_seed(9)
    qkv = (torch.randn(B, N, 3, H, D, generator=g) * 1.5).to(torch.bfloat16).to(dev)
    q, k, v = (qkv[:, :, c].permute(0, 2, 1, 3) for c in range(3))
    st = q.stride()
    out_full = torch.full((B, N, 3, H, D), float("nan"), dtype=torch.bfloat16, device=dev)
    out = out_full[:, :, 0].permute(0, 2, 1, 3)
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1.0,
                            strides=(st[0], st[1], st[2]))
    mask = att.new_mask(dev)
    att.step(q, k, v, out, mask, -2.0, 0)
    torch.cuda.synchronize()
    ref = lite_attn_step_ref(q.cpu(), k.cpu(), v.cpu(), np.zeros(att.mask_shape, np.uint32),
                             tile_q=128, tile_k=64, softmax_scale=1.0, log_eps=-2.0, step=0)
    c = Comparison()
    c.add_out(out.double().cpu().numpy(), ref.out)
    tk = att.tiles[1]
    c.add_mask(mask_to_bits(from_mask_tensor(mask), tk), mask_to_bits(ref.mask_next, tk),
               ref.margins, np.zeros((B, H, att.tiles[0], tk), bool))
    c.check("strided")
    assert torch.isnan(out_full[:, :, 1:].float()).all()  # nothing written outside out


def test_reset_and_popcount():
    dev = device()
    att = tsa.LiteAttention(2, 3, 5000, 64, tile_q=128, dtype="bf16")
    tq, tk = att.tiles
    rng = np.random.default_rng(1)
    bits = rng.random((2, 3, tq, tk)) < 0.3
    m = bits_to_mask(bits)
    m[..., -1] |= np.uint32(1 << 31) if tk % 32 else np.uint32(0)   # reserved bit, not counted
    mask = to_mask_tensor(m, dev)
    counts = att.popcount(mask)
    torch.cuda.synchronize()
    assert counts.cpu().numpy().tolist() == bits.reshape(6, -1).sum(1).tolist()
    assert abs(att.skipped_fraction(mask) - bits.mean()) < 1e-12
    att.reset_mask(mask)
    torch.cuda.synchronize()
    assert not mask.cpu().numpy().any()


def test_determinism_and_monotone_free_chain():
    dev = device()
    from workloads import Workload, derive, get_config
    cfg = derive(get_config(3), name="det", heads=[3, 4], grid=(3, 12, 30), steps=6)
    wl = Workload(cfg, dev)
    att = make_attention(cfg)
    masks, outs = [], []
    for rep in range(2):
        mask = att.new_mask(dev)
        prev = from_mask_tensor(mask)
        seq = []
        for t in range(cfg.steps):
            q, k, v = wl.inputs(t)
            out = torch.empty_like(q)
            att.step(q, k, v, out, mask, cfg.log_eps[t], t)
            cur = from_mask_tensor(mask)
            assert not np.any(prev & ~cur), "a bit was cleared"
            prev = cur
            seq.append(out.clone())
        masks.append(prev)
        outs.append(seq)
    assert np.array_equal(masks[0], masks[1])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    log(f"free chain skipped fraction {mask_to_bits(masks[0], att.tiles[1]).mean():.3f}")


def test_binding_rejects_bad_tensors():
    dev = device()
    att = tsa.LiteAttention(1, 2, 256, 64, tile_q=128, dtype="bf16")
    q = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16, device=dev)
    mask = att.new_mask(dev)
    with pytest.raises(TypeError):
        att.step(q.float(), q, q, torch.empty_like(q), mask, -1.0, 0)
    with pytest.raises(ValueError):
        att.step(q.cpu(), q, q, torch.empty_like(q), mask, -1.0, 0)
    with pytest.raises(ValueError):
        att.step(q[:, :, :128], q, q, torch.empty_like(q), mask, -1.0, 0)
    with pytest.raises(tsa.LiteAttnError):
        att.step(q, q, q, torch.empty_like(q), mask, 0.5, 0)
    with pytest.raises(tsa.LiteAttnError):
        att.step(q, q, q, q, mask, -1.0, 0)   # out aliases q


def test_largest_supported_length():
    """N = 131072 (2048 key tiles, the visiting-list capacity; 64 mask words per row), with a
    random mask that leaves about half the tiles; sampled query tiles against the oracle, and
    the whole output finite."""
    dev = device()
    n, D = 131072, 128
    tq, tk, w = mask_geometry(n, 128, 64)
    assert tk == 2048 and w == 64
    rng = np.random.default_rng(131072)
    bits = rng.random((1, 1, tq, tk)) < 0.5
    bits[0, 0, :, 0] = False
    mask_np = bits_to_mask(bits)
    q, k, v = _rand_inputs(1, 1, n, D, torch.bfloat16, 7, 1.0)
    att = tsa.LiteAttention(1, 1, n, D, tile_q=128, dtype="bf16", softmax_scale=1.0 / 11.3)
    out = torch.empty((1, 1, n, D), dtype=torch.bfloat16, device=dev)
    mask = to_mask_tensor(mask_np, dev)
    att.step(q.to(dev), k.to(dev), v.to(dev), out, mask, -0.3, 1)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    rows = [(0, 0, i) for i in (0, 1, 511, tq - 1)]
    ref = lite_attn_step_ref(q, k, v, mask_np, tile_q=128, tile_k=64, softmax_scale=1.0 / 11.3,
                             log_eps=-0.3, step=1, order="alt", rows=rows)
    got = out.double().cpu().numpy()
    gbits = mask_to_bits(from_mask_tensor(mask), tk)
    rbits = mask_to_bits(ref.mask_next, tk)
    c = Comparison()
    for (_, _, i) in rows:
        r0, r1 = i * 128, min(n, (i + 1) * 128)
        c.add_out(got[0, 0, r0:r1], ref.out[0, 0, r0:r1])
        c.add_mask(gbits[0, 0, i], rbits[0, 0, i], ref.margins[0, 0, i], bits[0, 0, i])
    c.check("N=131072")


@pytest.mark.parametrize("tile_q,D,P", [(64, 64, 200), (64, 128, 64), (128, 64, 1100), (128, 128, 2000)])
def test_dense_prefix_order_shapes(tile_q, D, P):
    """The persistent launch hands out the dense-prefix query tiles first (ceil(P / tile_q) per
    head, over all batches and heads), then the rest in traversal direction. Every tile must
    still be computed exactly once: a random prior mask, both traversal directions, B = 2,
    H = 3, and prefixes of under one tile, exactly one tile, several tiles and the whole
    sequence (P = N)."""
    n = 2000 if P <= 2000 else P
    B, H = 2, 3
    tq, tk, w = mask_geometry(n, tile_q, 64)
    rng = np.random.default_rng(tile_q * 1000 + D + P)
    bits = rng.random((B, H, tq, tk)) < 0.4
    for step in (0, 1):
        out, m, ref = _step_both(B, H, n, D, torch.bfloat16, bits_to_mask(bits), -2.0, step,
                                 tile_q=tile_q, prefix=P, seed=31 + step, spread=2.0)
        c = Comparison()
        c.add_out(out, ref.out)
        c.add_mask(mask_to_bits(m, tk), mask_to_bits(ref.mask_next, tk), ref.margins, bits)
        c.check(f"prefix order tq={tile_q} D={D} P={P} step {step}")
