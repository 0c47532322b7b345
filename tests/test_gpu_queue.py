"""Persistent bf16 launches: every step takes its query tiles from a queue owned by its stream.
Steps on concurrent streams, more streams than queues (the fallback to one workgroup per tile)
and back-to-back launches of different sizes on one stream must all give the results of a plain
run on the current stream, bit for bit."""
import numpy as np
import pytest
import torch

import temporally_sparse_attention_amd as tsa
from gpu_util import device, log, to_mask_tensor
from oracle import bits_to_mask, mask_geometry

pytestmark = pytest.mark.gpu


def _case(B, H, N, D, seed, skip=0.4):
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k, v = ((torch.randn(B, H, N, D, generator=g) * 1.5).to(torch.bfloat16).to(dev)
               for _ in range(3))
    tq, tk, w = mask_geometry(N, 128, 64)
    bits = np.random.default_rng(seed).random((B, H, tq, tk)) < skip
    return q, k, v, to_mask_tensor(bits_to_mask(bits), dev)


def _run(att, q, k, v, mask0, eps, step, stream=None):
    out = torch.full_like(q, float("nan"))
    mask = mask0.clone()
    att.step(q, k, v, out, mask, eps, step, stream=stream)
    return out, mask


def test_concurrent_streams_match_serial():
    B, H, N, D = 1, 8, 9000, 128
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1 / 11.3)
    cases = [_case(B, H, N, D, s) for s in (1, 2, 3)]
    ref = [_run(att, *c, -3.0, 1) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        got = []
        for st, c in zip(streams, cases):
            with torch.cuda.stream(st):
                got.append(_run(att, *c, -3.0, 1, stream=st))
        torch.cuda.synchronize()
        for (o, m), (ro, rm) in zip(got, ref):
            assert torch.equal(o, ro) and torch.equal(m, rm), f"repetition {rep}"


def test_more_streams_than_queues():
    B, H, N, D = 1, 2, 3000, 64
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16")
    c = _case(B, H, N, D, 7)
    ro, rm = _run(att, *c, -2.0, 0)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(72)]
    outs = []
    for st in streams:
        with torch.cuda.stream(st):
            outs.append(_run(att, *c, -2.0, 0, stream=st))
    torch.cuda.synchronize()
    for i, (o, m) in enumerate(outs):
        assert torch.equal(o, ro) and torch.equal(m, rm), f"stream {i}"
    log(f"{len(streams)} streams agree")


def test_back_to_back_launches_of_different_sizes():
    """The queue is reset by the last workgroup of each launch; the next launch on the stream
    (here alternating between two tile counts and two head dims) starts from zero."""
    big = tsa.LiteAttention(1, 4, 7000, 128, tile_q=128, dtype="bf16")
    small = tsa.LiteAttention(2, 1, 700, 64, tile_q=64, dtype="bf16")
    cb, cs = _case(1, 4, 7000, 128, 11), _case(2, 1, 700, 64, 12)
    # small's mask geometry uses tile_q 64
    tq, tk, w = mask_geometry(700, 64, 64)
    bits = np.random.default_rng(12).random((2, 1, tq, tk)) < 0.4
    cs = cs[:3] + (to_mask_tensor(bits_to_mask(bits), device()),)
    rb, rs = _run(big, *cb, -2.5, 2), _run(small, *cs, -2.5, 3)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        res = [(_run(big, *cb, -2.5, 2, stream=st), _run(small, *cs, -2.5, 3, stream=st))
               for _ in range(4)]
    torch.cuda.synchronize()
    for (gb, gs) in res:
        assert torch.equal(gb[0], rb[0]) and torch.equal(gb[1], rb[1])
        assert torch.equal(gs[0], rs[0]) and torch.equal(gs[1], rs[1])


def test_graph_replays_match_eager():
    """A step captured in a HIP graph (torch.cuda.graph) replays the persistent launch with the
    queue of the capture stream; the queue is back at zero after every replay, so each replay
    (with eager work on the GPU in between) gives the eager result."""
    B, H, N, D = 1, 4, 6000, 128
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1 / 11.3)
    q, k, v, mask0 = _case(B, H, N, D, 21)
    ro, rm = _run(att, q, k, v, mask0, -3.0, 1)
    torch.cuda.synchronize()
    out = torch.full_like(q, float("nan"))
    mask = mask0.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        att.step(q, k, v, out, mask, -3.0, 1)
    for rep in range(3):
        out.fill_(float("nan"))
        mask.copy_(mask0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(mask, rm), f"replay {rep}"
        _run(att, q, k, v, mask0, -2.0, 0)        # eager work between replays
        torch.cuda.synchronize()
