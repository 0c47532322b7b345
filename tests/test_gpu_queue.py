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


def _hip_runtime():
    """The HIP runtime torch loaded (the library binds to the same one)."""
    import ctypes
    from temporally_sparse_attention_amd.binding import _hip_runtimes_mapped
    paths = _hip_runtimes_mapped()
    assert len(paths) == 1, paths
    hip = ctypes.CDLL(paths[0])
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamCreate.restype = ctypes.c_int
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy.restype = ctypes.c_int
    return hip


def _oracle_check(q, k, v, mask0, out, mask, eps, step, tile_q=128):
    """The launch's output and new mask against the oracle (all query tiles)."""
    from gpu_util import Comparison, from_mask_tensor
    from oracle import lite_attn_step_ref, mask_to_bits
    B, H, N, D = q.shape
    ref = lite_attn_step_ref(q.cpu(), k.cpu(), v.cpu(), from_mask_tensor(mask0), tile_q=tile_q,
                             tile_k=64, softmax_scale=1.0 / D ** 0.5, log_eps=eps, step=step)
    _, tk, _ = mask_geometry(N, tile_q, 64)
    cmp = Comparison()
    cmp.add_out(out.double().cpu().numpy(), ref.out)
    cmp.add_mask(mask_to_bits(from_mask_tensor(mask), tk), mask_to_bits(ref.mask_next, tk),
                 ref.margins, mask_to_bits(from_mask_tensor(mask0), tk))
    cmp.check("fallback vs oracle")


def test_more_streams_than_queues_fall_back_to_one_workgroup_per_tile():
    """Streams made with hipStreamCreate (outside torch's pool of 32 per device), more than the
    64 eager queues: the steps on the streams left without a queue launch one workgroup per
    query tile (lite_attn_last_launch reports queue -1 and a grid of B*H*Tq), and every launch
    matches the oracle."""
    import ctypes
    B, H, N, D = 1, 2, 3000, 64
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16")
    tq, _ = att.tiles
    q, k, v, mask0 = _case(B, H, N, D, 7)
    ro, rm = _run(att, q, k, v, mask0, -2.0, 0)
    torch.cuda.synchronize()
    _oracle_check(q, k, v, mask0, ro, rm, -2.0, 0)
    hip = _hip_runtime()
    handles = []
    for _ in range(72):
        h = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(h)) == 0
        handles.append(h.value)
    try:
        launches, outs = [], []
        for hv in handles:
            st = torch.cuda.ExternalStream(hv, device=q.device)
            with torch.cuda.stream(st):
                outs.append(_run(att, q, k, v, mask0, -2.0, 0, stream=st))
            launches.append(tsa.lite_attn_last_launch())
        torch.cuda.synchronize()
    finally:
        for hv in handles:
            hip.hipStreamDestroy(ctypes.c_void_p(hv))
    fallback = [i for i, (_, qu) in enumerate(launches) if qu == -1]
    log(f"  {len(handles)} streams: queues {[qu for _, qu in launches]}")
    assert len(fallback) >= len(handles) - 64, launches
    for i, (o, m) in enumerate(outs):
        assert torch.equal(o, ro) and torch.equal(m, rm), f"stream {i}"
    for i in fallback:
        assert launches[i][0] == B * H * tq, launches[i]


def test_per_thread_default_stream_falls_back_and_matches_the_oracle():
    """The per-thread default stream has one handle value for many streams, so no queue can be
    tied to it: the step takes one workgroup per query tile. Both head dims and tile_q values
    run that way and are compared with the oracle."""
    per_thread = 2       # hipStreamPerThread
    for (D, tile_q) in ((128, 128), (64, 64), (128, 64), (64, 128)):
        B, H, N = 1, 3, 1100
        att = tsa.LiteAttention(B, H, N, D, tile_q=tile_q, dtype="bf16")
        tq, tk, w = mask_geometry(N, tile_q, 64)
        g = torch.Generator(device="cpu").manual_seed(D + tile_q)
        q, k, v = ((torch.randn(B, H, N, D, generator=g) * 1.5).to(torch.bfloat16).to(device())
                   for _ in range(3))
        bits = np.random.default_rng(D).random((B, H, tq, tk)) < 0.3
        mask0 = to_mask_tensor(bits_to_mask(bits), device())
        torch.cuda.synchronize()
        out = torch.full_like(q, float("nan"))
        mask = mask0.clone()
        torch.cuda.synchronize()
        att.step(q, k, v, out, mask, -2.0, 1, stream=per_thread)
        wg, qu = tsa.lite_attn_last_launch()
        torch.cuda.synchronize()
        assert (wg, qu) == (B * H * tq, -1), (D, tile_q, wg, qu)
        _oracle_check(q, k, v, mask0, out, mask, -2.0, 1, tile_q=tile_q)
        ro, rm = _run(att, q, k, v, mask0, -2.0, 1)
        assert tsa.lite_attn_last_launch()[1] >= 0
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(mask, rm), (D, tile_q)


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


def test_two_graphs_on_one_capture_stream_replay_concurrently():
    """torch.cuda.graph captures every graph on one shared capture stream. Each captured step
    gets a tile queue of its own, so two graphs (two guidance branches, with their own masks)
    replayed at the same time on two streams both give the eager results."""
    B, H, N, D = 1, 4, 6000, 128
    att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1 / 11.3)
    cases = [_case(B, H, N, D, s) for s in (31, 32)]
    refs = [_run(att, *c, -3.0, 1) for c in cases]
    torch.cuda.synchronize()
    bufs = [(torch.full_like(c[0], float("nan")), c[3].clone()) for c in cases]
    graphs, queues = [], []
    for c, (out, mask) in zip(cases, bufs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            att.step(c[0], c[1], c[2], out, mask, -3.0, 1)
        queues.append(tsa.lite_attn_last_launch()[1])
        graphs.append(g)
    log(f"  captured steps use queues {queues}")
    assert queues[0] != queues[1] and min(queues) >= 64
    streams = [torch.cuda.Stream() for _ in graphs]
    for rep in range(4):
        for c, (out, mask) in zip(cases, bufs):
            out.fill_(float("nan"))
            mask.copy_(c[3])
        torch.cuda.synchronize()
        for st, g in zip(streams, graphs):
            with torch.cuda.stream(st):
                g.replay()
        torch.cuda.synchronize()
        for (out, mask), (ro, rm) in zip(bufs, refs):
            assert torch.equal(out, ro) and torch.equal(mask, rm), f"replay {rep}"
        _run(att, *cases[0], -2.0, 0)        # eager work between replays
        torch.cuda.synchronize()
