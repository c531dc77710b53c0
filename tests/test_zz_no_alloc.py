"""The forward entry point that allocates nothing (qlin_fwd_noalloc), called
through the C ABI: its outputs must be bit-identical to qlin_fwd's (the same
kernels on the library's own device array instead of a workspace), and
within the float bounds of the CPU oracle, on calls in a row of decreasing
size (the array keeps the previous call's contents)."""

import numpy as np
import pytest

from tests import parity
from tests.gpu_util import bf16_host_bits, host, to_dev_bf16, to_dev_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    qb._lib.lib()
    return qb


# large-token layer first, then smaller ones: the second call reuses the
# array after a larger one (split partials and counters of another shape)
CASES = [
    ("nf4", 1040, 768, 513, 48, 1),    # MFMA forward, u by the skinny split product
    ("nf4", 512, 4096, 260, 16, 1),    # MFMA forward with split-K (ticketed fix-up)
    ("int4", 256, 1088, 16, 64, 32),   # few tokens, pooled adapter
    ("nf4", 256, 11008, 7, 16, 1),     # few tokens, K split over 3 workgroups, fused u
]


def _run_case(qb, oracle, fmt, d_out, d_in, M, r, pool, seed):
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("na", d_out, d_in, M, r, 2.0, fmt=fmt, block=64 if fmt == "nf4" else 32,
                  dq_block=256 if fmt == "nf4" else 0, pool=pool)
    inp = make_inputs(wl, seed=seed)
    if fmt == "nf4":
        qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), 64, 256)
        codes, am, am2 = oracle.quantize_nf4(inp.W, 64, 256)
        Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2))
    else:
        qw = qb.qlin_quantize_int4_group(to_dev_f32(inp.W), 32)
        codes, sc, zp = oracle.quantize_int4_group(inp.W, 32)
        Wd = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zp, 32))
    x, A, B = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B))
    print(f"[noalloc] {fmt} {d_out}x{d_in} M={M} r={r} pool={pool}", flush=True)
    qb_w = qw
    y0, u0 = qb.qlin_fwd(qb_w, x, A, B, r, 2.0, pool)
    y1, u1 = qb.qlin_fwd_noalloc(qb_w, x, A, B, r, 2.0, pool)
    # without a u output the forward keeps u in the array itself
    y2, _ = qb.qlin_fwd_noalloc(qb_w, x, A, B, r, 2.0, pool, want_u=False)
    assert np.array_equal(bf16_host_bits(y1), bf16_host_bits(y0))
    assert np.array_equal(host(u1).view(np.uint32), host(u0).view(np.uint32))
    assert np.array_equal(bf16_host_bits(y2), bf16_host_bits(y0))
    xf, Af, Bf = (oracle.bf16_bits_to_f64(a) for a in (inp.x, inp.A, inp.B))
    y_ref, u_ref = oracle.lora_forward(Wd, xf, Af, Bf, 2.0, pool)
    parity.check({"y": (oracle.bf16_bits_to_f64(bf16_host_bits(y1)), y_ref),
                  "u": (host(u1).astype(np.float64), u_ref)}, fmts={"u": "f32"})


def test_noalloc_forward_matches_workspace_forward(qb, oracle):
    for i, case in enumerate(CASES):
        _run_case(qb, oracle, *case, seed=20 + i)
    # and once more, the first (largest) case after the smaller ones
    _run_case(qb, oracle, *CASES[0], seed=30)


def test_noalloc_rejects_a_layer_beyond_its_array(qb):
    """The QA-LoRA 4096 x 11008 layer at 2048 tokens needs 64 MiB of split
    partials: refused with QLIN_E_WORKSPACE before anything is enqueued."""
    import torch
    w = qb.QWeight(2, 32, 0, 4096, 11008, torch.empty((4096, 5504), dtype=torch.uint8, device="cuda"),
                   scale=torch.empty((4096, 344), dtype=torch.float16, device="cuda"),
                   zero=torch.empty((4096, 344), dtype=torch.float16, device="cuda"))
    x = torch.empty((2048, 11008), dtype=torch.bfloat16, device="cuda")
    A = torch.empty((64, 344), dtype=torch.bfloat16, device="cuda")
    B = torch.empty((4096, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qb.QlinError) as e:
        qb.qlin_fwd_noalloc(w, x, A, B, 64, 2.0, 32)
    assert e.value.status == 6
