"""Graph replay (hfa_attn_fwd_graph_create / hfa_graph_launch) on the GPU.

A captured graph must write exactly what the eager call writes, on every
replay.  Between replays the program does eager work of its own (other
attention calls, fills of the output buffers with NaN) and synchronises, so a
replay that skipped or reordered a launch, or read stale arguments, shows up.
"""

import math

import pytest
import torch

import fa2_fwd_amd as hfa
from fa2_fwd_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [("f32", 1, 1, 128, 64), ("f32", 4, 8, 1024, 64), ("bf16", 1, 2, 1000, 128), ("bf16", 2, 2, 300, 64)]


@pytest.mark.parametrize("dtype,B,H,N,d", CASES)
@pytest.mark.parametrize("count", [1, 3])
def test_graph_replays_match_eager(dtype, B, H, N, d, count):
    print(f"[graph] {dtype} B={B} H={H} N={N} d={d} count={count}", flush=True)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(B, H, N, d, dtype, seed=N + d + count))
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = hfa.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    other = [t.to(dev) for t in W.make_inputs(B, H, N, d, dtype, seed=7)]
    with hfa.AttnGraph(q, k, v, scale, count=count) as g:
        for rep in range(3):
            g.out.fill_(float("nan"))
            g.lse.fill_(float("nan"))
            hfa.attn_fwd(*other, scale)  # unrelated eager work between replays
            torch.cuda.synchronize()
            o, lse = g.launch()
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), f"replay {rep}: O differs from the eager call"
            assert torch.equal(lse, lse_ref), f"replay {rep}: LSE differs from the eager call"


def test_graph_on_a_side_stream():
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(1, 4, 512, 128, "bf16", seed=11))
    o_ref, lse_ref = hfa.attn_fwd(q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with hfa.AttnGraph(q, k, v, count=2) as g:
        g.out.zero_()
        torch.cuda.synchronize()
        g.launch(stream=side)
        side.synchronize()
        assert torch.equal(g.out, o_ref) and torch.equal(g.lse, lse_ref)
