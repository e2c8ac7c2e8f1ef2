"""hfa_attn_fwd_split_noalloc (the key split with the library's own scratch array as
workspace) against hfa_attn_fwd_split with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input: the scratch keeps the first
call's partial results, which the second must not read.  Both calls are also
checked against the fp64 oracle at the bf16 tolerance.
"""

import math

import numpy as np
import pytest
import torch

import fa2_fwd_amd as hfa
from fa2_fwd_amd import workloads as W
from parity_util import assert_close, run_oracle

pytestmark = pytest.mark.gpu


def _both(B, H, N, d, splits, seed):
    dev = torch.device("cuda:0")
    hq, hk, hv = W.make_inputs(B, H, N, d, "bf16", seed=seed)
    q, k, v = (t.to(dev) for t in (hq, hk, hv))
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream(dev).cuda_stream
    need = hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, B, H, N, d, splits)
    assert 0 < need <= 64 << 20
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o_ref = torch.empty_like(q)
    l_ref = torch.empty(B, H, N, device=dev)
    st = hfa.hfa_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                                B, H, N, d, scale, hfa.HFA_BF16, splits, ws.data_ptr(), need, stream)
    assert st == hfa.HFA_OK, hfa.hfa_status_str(st)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=dev)
    st = hfa.hfa_attn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        B, H, N, d, scale, hfa.HFA_BF16, splits, stream)
    assert st == hfa.HFA_OK, hfa.hfa_status_str(st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "O differs from hfa_attn_fwd_split"
    assert torch.equal(lse, l_ref), "LSE differs from hfa_attn_fwd_split"
    ro, rl = run_oracle(hq, hk, hv, scale)
    assert_close(f"noalloc split={splits} B={B} H={H} N={N} d={d}", o.float().cpu().double().numpy(),
                 lse.cpu().double().numpy(), ro, rl, "bf16")


def test_noalloc_matches_the_workspace_entry_point_twice():
    print("[noalloc] first call: B=1 H=4 N=3000 d=128 splits=5", flush=True)
    _both(1, 4, 3000, 128, 5, seed=9001)
    print("[noalloc] second call, smaller: B=1 H=2 N=700 d=64 splits=3", flush=True)
    _both(1, 2, 700, 64, 3, seed=9002)


def test_noalloc_rejects_a_split_beyond_its_scratch():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 64, 4096, 128, dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(1, 64, 4096, device=dev)
    # 8 ranges x 64 heads x 4096 rows x 129 fp32 = 1.08 GB > 64 MiB
    st = hfa.hfa_attn_fwd_split_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                        1, 64, 4096, 128, 0.125, hfa.HFA_BF16, 8, None)
    assert st == hfa.HFA_ERR_WORKSPACE


def test_noalloc_replays_from_a_captured_graph():
    """The callers this entry point is for capture it: a graph holding one call, replayed
    three times with new inputs copied in eagerly between replays, each replay equal to
    an eager hfa_attn_fwd_split call on the same inputs and within tolerance of the oracle."""
    dev = torch.device("cuda:0")
    B, H, N, d, splits = 1, 4, 2500, 128, 4
    scale = 1.0 / math.sqrt(d)
    inputs = [W.make_inputs(B, H, N, d, "bf16", seed=9100 + r) for r in range(3)]
    q, k, v = (t.to(dev) for t in inputs[0])
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)

    def call(stream):
        return hfa.hfa_attn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                              lse.data_ptr(), B, H, N, d, scale, hfa.HFA_BF16, splits, stream)

    # one eager call first: the library's per-device set-up happens outside the capture
    assert call(torch.cuda.current_stream(dev).cuda_stream) == hfa.HFA_OK
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            assert call(torch.cuda.current_stream(dev).cuda_stream) == hfa.HFA_OK
    torch.cuda.synchronize()

    need = hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, B, H, N, d, splits)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for r, (hq, hk, hv) in enumerate(inputs):
        print(f"[noalloc graph] replay {r}: B={B} H={H} N={N} d={d} splits={splits}", flush=True)
        q.copy_(hq.to(dev))
        k.copy_(hk.to(dev))
        v.copy_(hv.to(dev))
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        o_ref = torch.empty_like(q)
        l_ref = torch.empty_like(lse)
        st = hfa.hfa_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                                    B, H, N, d, scale, hfa.HFA_BF16, splits, ws.data_ptr(), need,
                                    torch.cuda.current_stream(dev).cuda_stream)
        assert st == hfa.HFA_OK, hfa.hfa_status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {r}: O differs from the eager call"
        assert torch.equal(lse, l_ref), f"replay {r}: LSE differs from the eager call"
        ro, rl = run_oracle(hq, hk, hv, scale)
        assert_close(f"noalloc graph replay {r}", o.float().cpu().double().numpy(), lse.cpu().double().numpy(),
                     ro, rl, "bf16")
