"""Pins of the CPU oracle to facts that do not come from the oracle itself.

* hand-worked examples derived from the pages' definition (tests/golden/);
* the closed form: with log_eps = -inf nothing is ever flagged and the output is naive dense
  softmax attention; with any fixed mask the output is block-masked softmax attention;
* brute force on tiny inputs, recomputing every running maximum from scratch in pure Python;
* invariants: monotone masks, normalisation (V = 1 gives 1), the first visited tile is never
  flagged, flagged tiles carry little softmax mass, exemptions, head permutation, determinism.
"""
import json
import math
import os
import random

import numpy as np
import pytest

from oracle import bits_to_mask, empty_mask, lite_attn_step_ref, mask_geometry, mask_to_bits
import pyref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _one_head(x):
    return np.asarray(x, dtype=np.float64)[None, None]


# ------------------------------------------------------------------ golden, hand-worked
def test_golden_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "qk_skip_worked_example.json")))
    q = _one_head(g["q"])
    k = _one_head(g["k"])
    v = _one_head(np.ones((g["seq_len"], 1)))
    for case in g["cases"]:
        mask = np.asarray(case["mask_in"], dtype=np.uint32)[None, None]
        res = lite_attn_step_ref(q, k, v, mask, tile_q=g["tile_q"], tile_k=g["tile_k"],
                                 softmax_scale=case["scale"], log_eps=case.get("log_eps", g["log_eps"]),
                                 step=case["step"], order=case["order"],
                                 dense_prefix=case["dense_prefix"])
        got = res.mask_next[0, 0]
        assert got.tolist() == case["mask_out"], case["name"]
        new = mask_to_bits(res.mask_next, 5) & ~mask_to_bits(mask, 5)
        for i, fl in enumerate(case["flags"]):
            assert sorted(np.nonzero(new[0, 0, i])[0].tolist()) == fl, (case["name"], i)
        if "margins_row0" in case:
            m = res.margins[0, 0, 0]
            exp = case["margins_row0"]
            assert math.isinf(m[0]) and m[0] > 0
            np.testing.assert_allclose(m[1:], exp[1:], rtol=0, atol=1e-12)


def test_golden_bit_layout():
    g = json.load(open(os.path.join(GOLDEN, "mask_bit_layout.json")))
    n = g["seq_len"]
    kv = np.full((n, 1), g["k_default"])
    for c, val in g["k_special"].items():
        kv[int(c), 0] = val
    q = _one_head(np.ones((n, 1)))
    k = _one_head(kv)
    v = _one_head(np.zeros((n, 1)))
    res = lite_attn_step_ref(q, k, v, empty_mask(1, 1, n, g["tile_q"], g["tile_k"]),
                             tile_q=g["tile_q"], tile_k=g["tile_k"], softmax_scale=1.0,
                             log_eps=g["log_eps"], step=0, order="asc")
    assert res.mask_next[0, 0, 0].tolist() == g["mask_out"]


# ------------------------------------------------------------------ closed forms
def _rand(rng, n, d, spread=1.0):
    return (rng.standard_normal((n, d)) * spread).tolist()


@pytest.mark.parametrize("n,d,tq,tk", [(13, 3, 4, 3), (16, 2, 8, 8), (7, 5, 3, 2), (1, 1, 1, 1)])
def test_no_skip_equals_naive_dense_attention(n, d, tq, tk):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, d)
    scale = 0.7
    res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), empty_mask(1, 1, n, tq, tk),
                             tile_q=tq, tile_k=tk, softmax_scale=scale, log_eps=-math.inf,
                             step=1, order="alt")
    want = pyref.masked_attention(q, k, v, [[True] * n for _ in range(n)], scale)
    np.testing.assert_allclose(res.out[0, 0], np.array(want), rtol=1e-12, atol=1e-12)
    assert not res.mask_next.any()


@pytest.mark.parametrize("seed", range(6))
def test_fixed_mask_equals_block_masked_attention(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(5, 30))
    d = int(rng.integers(1, 5))
    tq = int(rng.integers(1, 9))
    tk = int(rng.integers(1, 9))
    q, k, v = _rand(rng, n, d, 1.5), _rand(rng, n, d, 1.5), _rand(rng, n, 3)
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    bits = rng.random((tqn, tkn)) < 0.4
    mask = bits_to_mask(bits)[None, None]
    res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, tile_q=tq, tile_k=tk,
                             softmax_scale=1.3, log_eps=-math.inf, step=0, order="asc")
    allowed = [[not bits[r // tq, c // tk] for c in range(n)] for r in range(n)]
    want = pyref.masked_attention(q, k, v, allowed, 1.3)
    np.testing.assert_allclose(res.out[0, 0], np.array(want), rtol=1e-12, atol=1e-12)
    # rows whose tile allows nothing are zero
    for i in range(tqn):
        if bits[i].all():
            assert np.all(res.out[0, 0, i * tq:(i + 1) * tq] == 0)


# ------------------------------------------------------------------ brute force on tiny inputs
@pytest.mark.parametrize("seed", range(40))
def test_mask_update_matches_brute_force(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(4, 40))
    d = int(rng.integers(1, 5))
    tq = int(rng.choice([1, 2, 3, 4, 8, 16]))
    tk = int(rng.choice([1, 2, 3, 4, 8, 16]))
    scale = float(rng.choice([1.0, 0.5, 2.5]))
    log_eps = float(rng.choice([-0.5, -2.0, -4.0, -8.0]))
    step = int(rng.integers(0, 4))
    order = str(rng.choice(["asc", "alt"]))
    prefix = int(rng.choice([0, 0, 3]))
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, 2)
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    skipped = rng.random((tqn, tkn)) < float(rng.choice([0.0, 0.3]))
    mask = bits_to_mask(skipped)[None, None]
    res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, tile_q=tq, tile_k=tk,
                             softmax_scale=scale, log_eps=log_eps, step=step, order=order,
                             dense_prefix=prefix)
    descending = order == "alt" and step % 2 == 1
    flags, margins = pyref.brute_flags(q, k, skipped.tolist(), tq, tk, scale, log_eps,
                                       descending, prefix)
    got_new = mask_to_bits(res.mask_next, tkn)[0, 0] & ~skipped
    for i in range(tqn):
        for j in range(tkn):
            if skipped[i, j]:
                assert math.isnan(res.margins[0, 0, i, j])
                continue
            mb = margins[i][j]
            mo = res.margins[0, 0, i, j]
            if math.isinf(mb):
                assert mo == mb
            else:
                assert abs(mo - mb) <= 1e-9 * max(1.0, abs(mb))
                if abs(mb) < 1e-9:
                    continue
            assert bool(got_new[i, j]) == flags[i][j], (i, j, mb)
    # old bits are kept
    assert np.all(mask_to_bits(res.mask_next, tkn)[0, 0] | ~skipped)


# ------------------------------------------------------------------ invariants over chains
def _chain_inputs(seed, n, d, steps, spread=1.2):
    rng = np.random.default_rng(seed)
    base_q = rng.standard_normal((2, 3, n, d)) * spread
    base_k = rng.standard_normal((2, 3, n, d)) * spread
    v = rng.standard_normal((2, 3, n, d))
    out = []
    for t in range(steps):
        out.append((base_q + 0.05 * rng.standard_normal(base_q.shape),
                    base_k + 0.05 * rng.standard_normal(base_k.shape), v))
    return out


@pytest.mark.parametrize("order", ["asc", "alt"])
def test_chain_monotone_normalised_first_tile_kept(order):
    n, d, tq, tk, steps = 70, 8, 16, 8, 5
    scale, eps = 1.0, [-math.inf, -6.0, -5.0, -4.0, -4.0]
    inputs = _chain_inputs(7, n, d, steps, spread=1.5)
    mask = empty_mask(2, 3, n, tq, tk)
    _, tkn, _ = mask_geometry(n, tq, tk)
    total_flags = 0
    for t in range(steps):
        q, k, v = inputs[t]
        res = lite_attn_step_ref(q, k, np.ones_like(v), mask, tile_q=tq, tile_k=tk,
                                 softmax_scale=scale, log_eps=eps[t], step=t, order=order)
        # normalisation: with V = 1 every output element is 1
        np.testing.assert_allclose(res.out, 1.0, rtol=0, atol=1e-12)
        old = mask_to_bits(mask, tkn)
        new = mask_to_bits(res.mask_next, tkn)
        assert not np.any(old & ~new), "bits were cleared"
        total_flags += int((new & ~old).sum())
        # first visited tile of every row tile is never flagged
        descending = order == "alt" and t % 2 == 1
        for idx in np.ndindex(old.shape[:3]):
            vis = [j for j in (range(tkn - 1, -1, -1) if descending else range(tkn)) if not old[idx][j]]
            assert vis and not new[idx][vis[0]]
        if t == 0:
            assert total_flags == 0  # log_eps = -inf flags nothing
        mask = res.mask_next
    assert total_flags > 0  # the case is not vacuous


def test_flagged_tiles_carry_little_mass():
    """A tile flagged at step t holds less than tile_k * exp(log_eps) of any of its rows'
    softmax mass at step t (the running max only grows and the normaliser is >= 1)."""
    n, d, tq, tk = 48, 3, 8, 4
    rng = np.random.default_rng(3)
    q = rng.standard_normal((n, d)) * 2
    k = rng.standard_normal((n, d)) * 2
    log_eps = -3.0
    for order, step in (("asc", 0), ("alt", 1)):
        res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(np.zeros((n, 1))),
                                 empty_mask(1, 1, n, tq, tk), tile_q=tq, tile_k=tk,
                                 softmax_scale=1.0, log_eps=log_eps, step=step, order=order)
        s = pyref.scores(q.tolist(), k.tolist(), 1.0)
        _, tkn, _ = mask_geometry(n, tq, tk)
        fl = mask_to_bits(res.mask_next, tkn)[0, 0]
        assert fl.any()
        for i, j in zip(*np.nonzero(fl)):
            for r in range(i * tq, min(n, (i + 1) * tq)):
                mx = max(s[r])
                z = sum(math.exp(x - mx) for x in s[r])
                mass = sum(math.exp(s[r][c] - mx) for c in range(j * tk, min(n, (j + 1) * tk))) / z
                assert mass < tk * math.exp(log_eps)


def test_dense_prefix_exemption_and_orders_agree_on_even_steps():
    inputs = _chain_inputs(11, 50, 4, 1, spread=2.0)
    q, k, v = inputs[0]
    tq, tk, prefix = 8, 4, 12
    mask = empty_mask(2, 3, 50, tq, tk)
    a = lite_attn_step_ref(q, k, v, mask, tile_q=tq, tile_k=tk, softmax_scale=1.0, log_eps=-2.0,
                           step=2, order="asc", dense_prefix=prefix)
    b = lite_attn_step_ref(q, k, v, mask, tile_q=tq, tile_k=tk, softmax_scale=1.0, log_eps=-2.0,
                           step=2, order="alt", dense_prefix=prefix)
    assert np.array_equal(a.mask_next, b.mask_next)
    assert np.array_equal(a.out, b.out)
    c = lite_attn_step_ref(q, k, v, mask, tile_q=tq, tile_k=tk, softmax_scale=1.0, log_eps=-2.0,
                           step=3, order="alt", dense_prefix=prefix)
    for res in (a, c):
        bits = mask_to_bits(res.mask_next, 13)
        assert not bits[:, :, :2, :].any()      # row tiles 0, 1 touch tokens < 12
        assert not bits[:, :, :, :3].any()      # key tiles 0..2 touch tokens < 12
        assert bits.any()
    free = lite_attn_step_ref(q, k, v, mask, tile_q=tq, tile_k=tk, softmax_scale=1.0,
                              log_eps=-2.0, step=3, order="alt")
    assert mask_to_bits(free.mask_next, 13)[:, :, :, :3].any()  # exemption matters here


def test_head_permutation_equivariance_and_determinism():
    q, k, v = _chain_inputs(5, 40, 4, 1, spread=2.0)[0]
    mask = bits_to_mask(np.random.default_rng(0).random((2, 3, 5, 10)) < 0.2)
    kw = dict(tile_q=8, tile_k=4, softmax_scale=1.0, log_eps=-3.0, step=1, order="alt")
    r1 = lite_attn_step_ref(q, k, v, mask, **kw)
    r2 = lite_attn_step_ref(q, k, v, mask, **kw)
    assert np.array_equal(r1.out, r2.out) and np.array_equal(r1.mask_next, r2.mask_next)
    perm = [2, 0, 1]
    rp = lite_attn_step_ref(q[:, perm], k[:, perm], v[:, perm], mask[:, perm], **kw)
    assert np.array_equal(rp.out, r1.out[:, perm])
    assert np.array_equal(rp.mask_next, r1.mask_next[:, perm])
    bp = lite_attn_step_ref(q[::-1], k[::-1], v[::-1], mask[::-1], **kw)
    assert np.array_equal(bp.mask_next, r1.mask_next[::-1])


def test_nan_scores_never_flag_and_log_eps_zero():
    n, d = 16, 2
    rng = np.random.default_rng(9)
    q = rng.standard_normal((n, d)) * 3
    k = rng.standard_normal((n, d)) * 3
    qn = q.copy()
    qn[5, 0] = np.nan
    kw = dict(tile_q=8, tile_k=2, softmax_scale=1.0, step=0, order="asc")
    r = lite_attn_step_ref(_one_head(qn), _one_head(k), _one_head(k), empty_mask(1, 1, n, 8, 2),
                           log_eps=-0.1, **kw)
    assert not mask_to_bits(r.mask_next, 8)[0, 0, 0].any()   # row tile 0 holds the NaN row
    # log_eps = 0 flags exactly the tiles that do not raise any row's running maximum
    r0 = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(k), empty_mask(1, 1, n, 8, 2),
                            log_eps=0.0, **kw)
    s = np.array(pyref.scores(q.tolist(), k.tolist(), 1.0))
    for i in range(2):
        rows = s[i * 8:(i + 1) * 8]
        run = np.full(8, -np.inf)
        for j in range(8):
            mt = rows[:, 2 * j:2 * j + 2].max(axis=1)
            want = bool(np.all(mt < run))
            assert bool(mask_to_bits(r0.mask_next, 8)[0, 0, i, j]) == want
            run = np.maximum(run, mt)


def test_rejects_bad_arguments_and_empty_inputs():
    q = np.zeros((1, 1, 4, 2))
    m = empty_mask(1, 1, 4, 2, 2)
    with pytest.raises(ValueError):
        lite_attn_step_ref(q, q, q, m, tile_q=2, tile_k=2, softmax_scale=1.0, log_eps=0.5, step=0)
    with pytest.raises(ValueError):
        lite_attn_step_ref(q, q, q, m, tile_q=2, tile_k=2, softmax_scale=1.0, log_eps=float("nan"),
                           step=0)
    with pytest.raises(ValueError):
        lite_attn_step_ref(q, q, q, m, tile_q=2, tile_k=2, softmax_scale=1.0, log_eps=-1.0, step=0,
                           order="desc")
    e = np.zeros((1, 1, 0, 2))
    r = lite_attn_step_ref(e, e, e, empty_mask(1, 1, 0, 2, 2), tile_q=2, tile_k=2,
                           softmax_scale=1.0, log_eps=-1.0, step=0)
    assert r.out.shape == (1, 1, 0, 2) and r.mask_next.shape == (1, 1, 0, 0)


# ------------------------------------------------------------------ in-step skip variant
@pytest.mark.parametrize("seed", range(12))
def test_in_step_skip_output_is_block_masked_attention_over_next_mask(seed):
    """With in-step skip the flags are those of the plain step (brute force), and the output is
    block-masked softmax attention over the tiles still clear after the step (closed form,
    pure-Python attention)."""
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.integers(4, 36))
    d = int(rng.integers(1, 5))
    tq = int(rng.choice([1, 2, 3, 4, 8]))
    tk = int(rng.choice([1, 2, 3, 4, 8]))
    scale = float(rng.choice([1.0, 2.5]))
    log_eps = float(rng.choice([-0.5, -2.0, -4.0]))
    step = int(rng.integers(0, 4))
    order = str(rng.choice(["asc", "alt"]))
    prefix = int(rng.choice([0, 0, 3]))
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, 2)
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    skipped = rng.random((tqn, tkn)) < float(rng.choice([0.0, 0.3]))
    mask = bits_to_mask(skipped)[None, None]
    kw = dict(tile_q=tq, tile_k=tk, softmax_scale=scale, log_eps=log_eps, step=step,
              order=order, dense_prefix=prefix)
    plain = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, **kw)
    res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, in_step_skip=True, **kw)
    descending = order == "alt" and step % 2 == 1
    flags, _ = pyref.brute_flags(q, k, skipped.tolist(), tq, tk, scale, log_eps, descending, prefix)
    after = skipped | np.asarray(flags, dtype=bool)
    assert np.array_equal(mask_to_bits(res.mask_next, tkn)[0, 0], after)
    assert np.array_equal(res.mask_next, plain.mask_next)
    np.testing.assert_array_equal(np.nan_to_num(res.margins, nan=7.0), np.nan_to_num(plain.margins, nan=7.0))
    allowed = [[not after[r // tq, c // tk] for c in range(n)] for r in range(n)]
    want = np.array(pyref.masked_attention(q, k, v, allowed, scale))
    for i in range(tqn):
        rows = slice(i * tq, min(n, (i + 1) * tq))
        if after[i].all():
            assert np.all(res.out[0, 0, rows] == 0)
        else:
            np.testing.assert_allclose(res.out[0, 0, rows], want[rows], rtol=1e-12, atol=1e-12)


def test_in_step_skip_changes_output_by_at_most_the_flagged_mass():
    """Leaving out tiles whose scores all lie more than |log_eps| below the row's running
    maximum moves each output row by at most 2 * w * max|v|, where w is the softmax mass of the
    left-out columns (bounded by their count times exp(log_eps)); and without flags the two
    modes agree exactly."""
    rng = np.random.default_rng(77)
    n, d, tq, tk = 48, 3, 8, 4
    x = np.linspace(0, 1, n)[:, None]
    q = np.hstack([np.cos(6 * x), np.sin(6 * x), 0.1 * rng.standard_normal((n, 1))]) * 3
    k = q + 0.05 * rng.standard_normal((n, d))
    v = rng.standard_normal((n, 2))
    mask = empty_mask(1, 1, n, tq, tk)
    kw = dict(tile_q=tq, tile_k=tk, softmax_scale=1.0, step=0, order="asc")
    for log_eps in (-6.0, -3.0):
        plain = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, log_eps=log_eps, **kw)
        ins = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, log_eps=log_eps,
                                 in_step_skip=True, **kw)
        flagged = mask_to_bits(plain.mask_next, -(-n // tk))[0, 0]
        assert flagged.any()
        s = q @ k.T
        for r in range(n):
            cols = np.repeat(flagged[r // tq], tk)[:n]
            p = np.exp(s[r] - s[r].max())
            w = p[cols].sum() / p.sum()
            assert w <= cols.sum() * math.exp(log_eps) + 1e-15
            diff = np.abs(ins.out[0, 0, r] - plain.out[0, 0, r]).max()
            assert diff <= 2 * w * np.abs(v).max() + 1e-12
    same = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, log_eps=-math.inf,
                              in_step_skip=True, **kw)
    base = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, log_eps=-math.inf, **kw)
    assert np.array_equal(same.out, base.out)


# ------------------------------------------------------------------ divergence refresh
def _brute_stat(q, k, skipped, tq, tk, scale, i):
    """Mean over the valid rows of tile i of the largest scaled score over the columns of the
    key tiles that are not skipped (pure Python)."""
    n = len(q)
    rows = range(i * tq, min(n, (i + 1) * tq))
    vals = []
    for r in rows:
        best = -math.inf
        for c in range(n):
            if not skipped[c // tk]:
                best = max(best, scale * sum(a * b for a, b in zip(q[r], k[c])))
        vals.append(best)
    return sum(vals) / len(vals)


@pytest.mark.parametrize("seed", range(8))
def test_refresh_statistic_matches_brute_force_and_infinite_delta_changes_nothing(seed):
    rng = np.random.default_rng(9000 + seed)
    n = int(rng.integers(6, 30))
    d = int(rng.integers(1, 4))
    tq, tk = int(rng.choice([2, 4, 8])), int(rng.choice([2, 3, 4]))
    q, k, v = _rand(rng, n, d, 2.0), _rand(rng, n, d, 2.0), _rand(rng, n, 2)
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    skipped = rng.random((tqn, tkn)) < 0.3
    mask = bits_to_mask(skipped)[None, None]
    kw = dict(tile_q=tq, tile_k=tk, softmax_scale=1.0, log_eps=-2.0, step=seed % 2, order="alt")
    plain = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, **kw)
    ref0 = np.full((1, 1, tqn), np.nan)
    res = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, tile_stats=ref0,
                             refresh_delta=math.inf, **kw)
    for i in range(tqn):
        want = _brute_stat(q, k, skipped[i].tolist(), tq, tk, 1.0, i)
        assert res.stats[0, 0, i] == pytest.approx(want, rel=1e-12, abs=1e-12) or (
            math.isinf(want) and res.stats[0, 0, i] == want)
    # a first step only records the reference; an infinite delta never refreshes
    np.testing.assert_array_equal(res.stats_next, res.stats)
    assert np.array_equal(res.mask_next, plain.mask_next) and not res.refreshed.any()
    np.testing.assert_array_equal(np.nan_to_num(res.out), np.nan_to_num(plain.out))
    again = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask,
                               tile_stats=res.stats_next + 1e9, refresh_delta=math.inf, **kw)
    assert np.array_equal(again.mask_next, plain.mask_next)
    np.testing.assert_array_equal(again.stats_next, res.stats_next + 1e9)


def test_refresh_clears_a_row_when_the_attention_moves_into_skipped_tiles():
    """Local attention (query r looks at key r); step 1 flags far tiles; at step 2 the keys are
    rolled so the best keys of every row lie in tiles that step 1 flagged: the row maxima over
    the computed tiles fall, the statistic moves by more than delta, and the rows are cleared
    (and the reference dropped); with a large delta nothing is cleared."""
    n, tq, tk = 32, 8, 8
    x = np.arange(n)
    q = np.stack([np.cos(2 * np.pi * x / n), np.sin(2 * np.pi * x / n)], axis=1) * 4.0
    k = q.copy()
    v = np.eye(n)[:, :3]
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    kw = dict(tile_q=tq, tile_k=tk, softmax_scale=1.0, order="asc")
    stats = np.full((1, 1, tqn), np.nan)
    mask = empty_mask(1, 1, n, tq, tk)
    r0 = lite_attn_step_ref(_one_head(q), _one_head(k), _one_head(v), mask, log_eps=-8.0, step=0,
                            tile_stats=stats, refresh_delta=2.0, **kw)
    assert not r0.refreshed.any() and not np.isnan(r0.stats_next).any()
    flagged = mask_to_bits(r0.mask_next, tkn)[0, 0]
    assert flagged.any()
    k2 = np.roll(k, n // 2, axis=0)        # every row's best keys move half the circle away
    r1 = lite_attn_step_ref(_one_head(q), _one_head(k2), _one_head(v), r0.mask_next, log_eps=-8.0,
                            step=1, tile_stats=r0.stats_next, refresh_delta=2.0, **kw)
    moved = np.abs(r1.stats - r0.stats_next)[0, 0]
    for i in range(tqn):
        if moved[i] > 2.0:
            assert r1.refreshed[0, 0, i] and not r1.mask_next[0, 0, i].any()
            assert math.isnan(r1.stats_next[0, 0, i])
        else:
            assert not r1.refreshed[0, 0, i]
    assert r1.refreshed.any()
    keep = lite_attn_step_ref(_one_head(q), _one_head(k2), _one_head(v), r0.mask_next, log_eps=-8.0,
                              step=1, tile_stats=r0.stats_next, refresh_delta=1e6, **kw)
    assert not keep.refreshed.any()
    assert np.array_equal(keep.mask_next, keep.mask_next | r0.mask_next)   # bits only grow


# ------------------------------------------------------------------ the chain driver
@pytest.mark.parametrize("order", ["asc", "alt"])
def test_run_chain_ref_matches_a_brute_force_chain(order):
    """run_chain_ref against a chain built by hand from the pure-Python pieces: every step
    starts from the previous step's mask (step 0 from an empty one), the mask it yields is the
    mask at the start of the step, flags follow the brute-force rule in this step's traversal
    direction, and the output is block-masked attention over that start mask."""
    from oracle import run_chain_ref
    rng = np.random.default_rng(77)
    n, d, tq, tk, steps, scale = 23, 3, 4, 3, 5, 1.0
    eps = [-math.inf, -1.0, -1.5, -0.8, -0.8]
    base_q, base_k = rng.standard_normal((n, d)) * 2.0, rng.standard_normal((n, d)) * 2.0
    v = rng.standard_normal((n, 2))
    xs = [(base_q + 0.1 * rng.standard_normal((n, d)), base_k + 0.1 * rng.standard_normal((n, d)))
          for _ in range(steps)]
    inputs = lambda t: (_one_head(xs[t][0]), _one_head(xs[t][1]), _one_head(v))
    tqn, tkn, _ = mask_geometry(n, tq, tk)
    skipped = [[False] * tkn for _ in range(tqn)]     # the hand-built chain's mask
    seen = 0
    for t, start, res in run_chain_ref(inputs, steps, eps, batch=1, heads=1, seq_len=n,
                                       tile_q=tq, tile_k=tk, softmax_scale=scale, order=order):
        assert t == seen
        seen += 1
        assert mask_to_bits(start, tkn)[0, 0].tolist() == skipped, t
        q, k = xs[t][0].tolist(), xs[t][1].tolist()
        descending = order == "alt" and t % 2 == 1
        flags, margins = pyref.brute_flags(q, k, skipped, tq, tk, scale, eps[t], descending)
        allowed = [[not skipped[r // tq][c // tk] for c in range(n)] for r in range(n)]
        want = pyref.masked_attention(q, k, v.tolist(), allowed, scale)
        np.testing.assert_allclose(res.out[0, 0], np.array(want), rtol=1e-12, atol=1e-12)
        got = mask_to_bits(res.mask_next, tkn)[0, 0]
        for i in range(tqn):
            for j in range(tkn):
                if skipped[i][j]:
                    assert got[i, j]
                elif abs(margins[i][j]) > 1e-9:
                    assert bool(got[i, j]) == flags[i][j], (t, i, j)
        skipped = [[bool(x) for x in row] for row in got]
    assert seen == steps
    assert sum(map(sum, skipped)) > 0          # the chain flags something
