"""The fused forward + backward captured in a HIP graph (as the benchmark runs
it) must reproduce the eager results bit for bit on every replay.  The
kernels' split-reduction counters reset themselves, and no call records a
memset, so replays stay independent of each other."""

import numpy as np
import pytest

from tests.gpu_util import bf16_host_bits, host, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d_out,d_in,M,r", [(4096, 4096, 16, 16), (528, 4096, 300, 16),
                                            (1040, 768, 513, 48)])
def test_graph_replays_match_eager(d_out, d_in, M, r):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("g", d_out, d_in, M, r, 2.0)
    inp = make_inputs(wl, seed=3)
    qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), 64, 256)
    x, A, B, dy = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    dev = x.device
    ws = torch.zeros(qb.qlin_workspace_bytes(qw, M, r, 1), dtype=torch.uint8, device=dev)
    y = torch.empty((M, d_out), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, d_in), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, d_in), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((d_out, r), dtype=torch.bfloat16, device=dev)

    def step():
        qb.qlin_fwd(qw, x, A, B, r, 2.0, 1, y=y, u_out=u, ws=ws)
        qb.qlin_bwd(qw, x, A, B, r, 2.0, dy, 1, u_saved=u, dx=dx, dA=dA, dB=dB, ws=ws)

    def snap():
        torch.cuda.synchronize()
        return [bf16_host_bits(t) for t in (y, dx, dA, dB)] + [host(u).view(np.uint32)]

    step()
    eager = snap()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (y, dx, dA, dB, u):
            t.zero_()
        # eager work of the program between replays
        scratch = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        got = snap()
        for name, a, b in zip(("y", "dx", "dA", "dB", "u"), eager, got):
            assert np.array_equal(a, b), f"replay {rep}: {name} differs from eager"
        del scratch
