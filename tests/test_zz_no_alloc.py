"""lite_attn_step_scheduled_static (the entry point that allocates nothing: its schedule
workspace is the library's static device memory) against lite_attn_step_scheduled with a
caller workspace: outputs and masks bit for bit, on two calls in a row, the second with a
smaller problem (the static array keeps the first call's contents; nothing in it may leak into
the second call's result)."""
import numpy as np
import pytest
import torch

import temporally_sparse_attention_amd as tsa
from gpu_util import device, log, to_mask_tensor
from oracle import bits_to_mask, mask_geometry

pytestmark = pytest.mark.gpu


def _case(B, H, N, D, tile_q, seed, skip):
    dev = device()
    g = torch.Generator(device="cpu").manual_seed(seed)
    q, k, v = (torch.randn(B, H, N, D, generator=g) * 1.5 for _ in range(3))
    k[:, :, 64:] *= 0.2         # key tile 0 dominates: the tiles visited after it flag
    q, k, v = (x.to(torch.bfloat16).to(dev) for x in (q, k, v))
    tq, tk, _ = mask_geometry(N, tile_q, 64)
    bits = np.random.default_rng(seed).random((B, H, tq, tk)) < skip
    # a few dense rows, so that the schedule moves them to the front
    bits[:, :, :2] = False
    return q, k, v, to_mask_tensor(bits_to_mask(bits), dev)


@pytest.mark.parametrize("D,tile_q", [(128, 128), (64, 64)])
def test_static_workspace_matches_caller_workspace_on_two_calls(D, tile_q):
    shapes = [(2, 5, 9000), (1, 3, 2500)]          # the second call is smaller
    for call, (B, H, N) in enumerate(shapes):
        log(f"  call {call}: B={B} H={H} N={N} D={D} tile_q={tile_q}")
        att = tsa.LiteAttention(B, H, N, D, tile_q=tile_q, dtype="bf16", softmax_scale=1.0)
        q, k, v, mask0 = _case(B, H, N, D, tile_q, 100 + call, 0.85)
        ws = att.new_workspace(q.device)
        o_ref, m_ref = torch.full_like(q, float("nan")), mask0.clone()
        att.step(q, k, v, o_ref, m_ref, -4.0, 2 * call, workspace=ws)
        o_st, m_st = torch.full_like(q, float("nan")), mask0.clone()
        tsa.lite_attn_step_scheduled_static(att.handle, q, k, v, o_st, m_st, -4.0, 2 * call)
        torch.cuda.synchronize()
        assert not torch.isnan(o_ref).any()
        assert torch.equal(o_st, o_ref), f"call {call}: outputs differ"
        assert torch.equal(m_st, m_ref), f"call {call}: masks differ"
        assert not torch.equal(m_st, mask0), "the case must flag tiles"
