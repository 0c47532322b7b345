"""A process whose first library call is made under HIP graph capture: the library resolves its
static device symbols (tile queues, static workspace) on first use, so that lookup then happens
during capture. Each case runs in a fresh Python process (the state to test is per process) and
compares the graph's replays with the eager results."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys, torch
sys.path.insert(0, {root!r})
import temporally_sparse_attention_amd as tsa
B, H, N, D = 1, 2, 3000, 128
att = tsa.LiteAttention(B, H, N, D, tile_q=128, dtype="bf16", softmax_scale=1.0)
g = torch.Generator(device="cpu").manual_seed(5)
q, k, v = (torch.randn(B, H, N, D, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
k[:, :, 64:] *= 0.2
mask0 = torch.zeros(att.mask_shape, dtype=torch.int32, device="cuda")
out = torch.full_like(q, float("nan"))
mask = mask0.clone()
torch.cuda.synchronize()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):
    if {static!r}:
        tsa.lite_attn_step_scheduled_static(att.handle, q, k, v, out, mask, -4.0, 0)
    else:
        att.step(q, k, v, out, mask, -4.0, 0)
print("captured, queue", tsa.lite_attn_last_launch(), flush=True)
for rep in range(3):
    out.fill_(float("nan")); mask.copy_(mask0); torch.cuda.synchronize()
    graph.replay(); torch.cuda.synchronize()
    ref_out, ref_mask = torch.full_like(q, float("nan")), mask0.clone()
    att.step(q, k, v, ref_out, ref_mask, -4.0, 0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(mask, ref_mask), rep
    assert not torch.equal(mask, mask0)
print("ok", flush=True)
"""


@pytest.mark.parametrize("static", [False, True], ids=["step", "scheduled_static"])
def test_first_call_under_graph_capture(static):
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT, static=static)],
                       capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "ok" in r.stdout
