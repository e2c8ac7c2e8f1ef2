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
from parity_util import assert_close, run_oracle

pytestmark = pytest.mark.gpu

CASES = [("f32", 1, 1, 128, 64), ("f32", 4, 8, 1024, 64), ("bf16", 1, 2, 1000, 128), ("bf16", 2, 2, 300, 64)]


@pytest.mark.parametrize("dtype,B,H,N,d", CASES)
@pytest.mark.parametrize("count", [1, 3])
def test_graph_replays_match_eager(dtype, B, H, N, d, count):
    print(f"[graph] {dtype} B={B} H={H} N={N} d={d} count={count}", flush=True)
    dev = torch.device("cuda:0")
    hq, hk, hv = W.make_inputs(B, H, N, d, dtype, seed=N + d + count)
    q, k, v = (t.to(dev) for t in (hq, hk, hv))
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = hfa.attn_fwd(q, k, v, scale)
    torch.cuda.synchronize()
    ref_o, ref_lse = run_oracle(hq, hk, hv, scale)
    other = [t.to(dev) for t in W.make_inputs(B, H, N, d, dtype, seed=7)]
    with hfa.AttnGraph(q, k, v, scale, count=count) as g:
        for rep in range(3):
            g.out.fill_(float("nan"))
            g.lse.fill_(float("nan"))
            hfa.attn_fwd(*other, scale)  # unrelated eager work between replays
            torch.cuda.synchronize()
            o, lse = g.launch()
            torch.cuda.synchronize()
            # each replay against the oracle, then bit for bit against the eager call
            assert_close(f"graph replay {rep} {dtype} B={B} H={H} N={N} d={d} count={count}",
                         o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ref_o, ref_lse, dtype)
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


def test_softmax_and_rmsnorm_under_torch_graph_capture():
    # The HBM-bound entry points launch kernels only (no memset, no allocation),
    # so a caller can capture them into a graph: every replay must equal the
    # eager result, with unrelated eager work and fills between replays.
    dev = torch.device("cuda:0")
    g = torch.Generator("cpu").manual_seed(21)
    xs = (torch.randn(64, 70001, generator=g) * 4.0).to(dev)  # wide softmax path (element-wise layout), ragged width
    xs2 = (torch.randn(128, 3000, generator=g) * 4.0).to(dev)  # register-resident path
    rw = W.RmsNormWorkload("graph", 300, 4096, "bf16", 22)
    xr, rr, wr = (t.to(dev) for t in rw.inputs())
    ys, ys2 = torch.empty_like(xs), torch.empty_like(xs2)
    yr, sr = torch.empty_like(xr), torch.empty_like(xr)
    ref = (hfa.softmax_rows(xs), hfa.softmax_rows(xs2), *hfa.rmsnorm(xr, wr, rw.eps, residual=rr))
    torch.cuda.synchronize()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):  # warm-up on the capture stream, as torch's graph docs ask
        hfa.softmax_rows(xs, out=ys)
    side.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        hfa.softmax_rows(xs, out=ys)
        hfa.softmax_rows(xs2, out=ys2)
        hfa.rmsnorm(xr, wr, rw.eps, residual=rr, out=yr, residual_out=sr)
    for rep in range(3):
        for t in (ys, ys2, yr, sr):
            t.fill_(float("nan"))
        hfa.softmax_rows(xs2 * 0.5)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ref[0]) and torch.equal(ys2, ref[1]), f"replay {rep}: softmax differs"
        assert torch.equal(yr.view(torch.int16), ref[2].view(torch.int16)), f"replay {rep}: rmsnorm y differs"
        assert torch.equal(sr.view(torch.int16), ref[3].view(torch.int16)), f"replay {rep}: rmsnorm sum differs"
