"""The seeded synthetic generator: shapes, determinism, per-head independence, schedules."""
import math

import torch

from workloads import CONFIGS, Workload, derive, get_config


def test_config_shapes():
    assert get_config(1).seq_len == 1024
    assert get_config(2).seq_len == 32760
    assert get_config(3).seq_len == 75600
    assert get_config(4).seq_len == 256 + 33 * 45 * 80 == 119056
    assert get_config(5).seq_len == 17408
    assert get_config(3).tiles_q == 591 and get_config(3).tiles_k == 1182
    for c in CONFIGS.values():
        assert len(c.sigmas) == c.steps == len(c.log_eps)
        assert len(c.head_recipes) == c.heads
        # budgets never loosen then tighten: early steps tolerate less error
        eps = [e for e in c.log_eps]
        assert all(a <= b for a, b in zip(eps, eps[1:]))
        assert all(e <= 0 for e in eps)
    bws = [r.bw for r in get_config(3).head_recipes]
    assert min(bws) >= 2 and max(bws) <= 10 and len(set(bws)) == 40
    assert get_config(2).log_eps[0] == -14 and get_config(2).log_eps[-1] == -8
    assert math.isclose(get_config(2).sigmas[-1], 0.01)
    assert get_config(1).log_eps[0] == -math.inf


def test_generator_deterministic_and_per_head():
    cfg = derive(get_config(2), heads=[0, 1, 2], grid=(2, 5, 7))
    a = Workload(cfg).inputs(1)
    b = Workload(cfg).inputs(1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    q, k, v = a
    assert q.shape == (1, 3, 70, 128) and q.dtype == torch.bfloat16 and q.is_contiguous()
    # a single head regenerates alone with the same values
    qh, kh, vh = Workload(cfg).head_inputs(1, 0, 2)
    assert torch.equal(qh.to(torch.bfloat16), q[0, 2])
    # steps differ in Q/K but share V
    q2, k2, v2 = Workload(cfg).inputs(2)
    assert not torch.equal(q2, q) and torch.equal(v2, v)


def test_prefix_is_isotropic_and_video_is_local():
    cfg = derive(get_config(4), heads=[0], grid=(2, 6, 8), prefix=16, dense_prefix=16)
    q0, k0, _ = Workload(cfg).base(0, 0)
    assert q0.shape == (16 + 96, 128)
    # video tokens: q.k of a token with itself is large (RFF kernel), the prefix is not
    vid = (q0[16:] * k0[16:]).sum(1).mean()
    pre = (q0[:16] * k0[:16]).sum(1).mean()
    assert vid > 20 and abs(pre) < 10
