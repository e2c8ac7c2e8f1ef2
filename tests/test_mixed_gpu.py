"""The three operations together on the GPU: seeded random attention shapes
against the oracle, and all three kernels running at once on separate streams
giving the same bytes as when run one after another.

Random shapes: 24 cases drawn from a fixed seed (B, H in 1..3, N in 1..700,
d in {64, 128}, dtype fp32 or bf16, scale 1/sqrt(d) times 0.25..4), each
checked on every row against the fp64 oracle with the tolerances of
test_parity_gpu.py.
"""

import math

import numpy as np
import pytest
import torch

import fa2_fwd_amd as hfa
import oracle
from fa2_fwd_amd import workloads as W
from test_parity_gpu import assert_close, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


def _random_cases(n, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 701))
        d = int(rng.choice([64, 128]))
        dtype = "f32" if rng.random() < 0.5 else "bf16"
        mult = float(2.0 ** rng.uniform(-2, 2))
        cases.append((i, B, H, N, d, dtype, mult))
    return cases


@pytest.mark.parametrize("i,B,H,N,d,dtype,mult", _random_cases(24))
def test_random_shapes(i, B, H, N, d, dtype, mult):
    q, k, v = W.make_inputs(B, H, N, d, dtype, seed=5000 + i)
    scale = mult / math.sqrt(d)
    name = f"random #{i} {dtype} B={B} H={H} N={N} d={d} scale={scale:.4g}"
    print(f"[mixed] {name}", flush=True)
    go, gl = run_gpu(q, k, v, scale)
    ro, rl = run_oracle(q, k, v, scale)
    assert_close(name, go, gl, ro, rl, dtype)


def test_three_kernels_on_three_streams():
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(1, 8, 4096, 128, "bf16", seed=31))
    xs = W.SoftmaxWorkload("t", 512, 40000, 32).inputs().to(dev)
    rw = W.RmsNormWorkload("t", 4096, 4096, "bf16", 33)
    xr, rr, wr = (t.to(dev) for t in rw.inputs())

    def run_all(streams):
        outs = {}
        with torch.cuda.stream(streams[0]):
            outs["attn"] = hfa.attn_fwd(q, k, v, 0.0883883, stream=streams[0])
        with torch.cuda.stream(streams[1]):
            outs["softmax"] = hfa.softmax_rows(xs, stream=streams[1])
        with torch.cuda.stream(streams[2]):
            outs["rmsnorm"] = hfa.rmsnorm(xr, wr, 1e-6, residual=rr, stream=streams[2])
        for s in streams:
            s.synchronize()
        return outs

    torch.cuda.synchronize()
    one = torch.cuda.current_stream(dev)
    serial = run_all([one, one, one])
    streams = [torch.cuda.Stream(dev) for _ in range(3)]
    torch.cuda.synchronize()
    for rep in range(3):
        conc = run_all(streams)
        assert torch.equal(conc["attn"][0].view(torch.int16), serial["attn"][0].view(torch.int16))
        assert torch.equal(conc["attn"][1], serial["attn"][1])
        assert torch.equal(conc["softmax"], serial["softmax"])
        assert torch.equal(conc["rmsnorm"][0].view(torch.int16), serial["rmsnorm"][0].view(torch.int16))
        assert torch.equal(conc["rmsnorm"][1].view(torch.int16), serial["rmsnorm"][1].view(torch.int16))
    # and the serial results are right
    rows = np.array([0, 1, 255, 511])
    ref = oracle.softmax_rows(xs.cpu().numpy(), rows=rows)
    assert np.abs(serial["softmax"].cpu().double().numpy()[rows] - ref).max() <= 1e-5
