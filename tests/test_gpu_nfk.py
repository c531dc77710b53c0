"""NormalFloat-k weights (k = 2, 3, 4 bits; blocks of 32 to 256) on the GPU,
through the C ABI: packed bit planes, 8-bit and second-level constants and
the decoded bf16 weight bit-exact to the oracle; the layer's forward and
backward (through the transcoded form) within the float bounds."""

import numpy as np
import pytest

from tests import parity
from tests.gpu_util import bf16_host_bits, host, to_dev_bf16, to_dev_f32, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    qb._lib.lib()
    return qb


def _check_packed(qb, oracle, W, bits, block, dq):
    qw = qb.qlin_quantize_nf(to_dev_f32(W), bits, block, dq)
    codes, am, am2 = oracle.quantize_nf(W, bits, block, dq)
    assert np.array_equal(u8(qw.codes), codes)
    if dq:
        assert np.array_equal(host(qw.absmax).view(np.int8), am)
        assert np.array_equal(host(qw.absmax2).view(np.uint32), am2.view(np.uint32))
    else:
        assert np.array_equal(host(qw.absmax).view(np.uint32), am.view(np.uint32))
    ref = oracle.dequant_nf_bf16(codes, am, am2, bits, block, dq)
    assert np.array_equal(bf16_host_bits(qb.qlin_dequant_bf16(qw)), ref)
    return qw


@pytest.mark.parametrize("bits,block,dq", [(2, 32, 256), (3, 64, 256), (3, 128, 0),
                                           (2, 256, 256), (4, 32, 256), (3, 256, 0), (4, 64, 0)])
def test_nf_pack_and_decode_bit_exact(qb, oracle, bits, block, dq):
    from quantized_base_rank_amd.inputs import make_weight
    _check_packed(qb, oracle, make_weight(336, 1536, seed=bits * 100 + block), bits, block, dq)


@pytest.mark.parametrize("bits", [2, 3])
def test_nf_special_blocks(qb, oracle, bits):
    c = oracle.nf_codebook(bits)
    W = np.zeros((16, 512), np.float32)
    W[0, 64:64 + c.size] = c * np.float32(2.0 ** -3)   # the levels themselves
    W[1, 5] = -3.0                                     # single nonzero
    W[2, :64] = np.linspace(-1.0, 0.5, 64, dtype=np.float32)
    W[3, :] = 0.125
    mids = ((c[:-1].astype(np.float64) + c[1:]) / 2).astype(np.float32)
    W[4, 0] = 1.0
    W[4, 1:c.size] = mids                              # near-midpoint values
    W[5, :] = np.float32(1e-30)
    for block, dq in ((32, 256), (64, 0), (256, 256)):
        _check_packed(qb, oracle, W, bits, block, dq)


def test_nf_rejects_nonfinite(qb):
    from quantized_base_rank_amd.inputs import make_weight
    W = make_weight(32, 256, seed=2)
    W[9, 100] = np.inf
    with pytest.raises(qb.QlinError) as e:
        qb.qlin_quantize_nf(to_dev_f32(W), 3, 64, 256)
    assert e.value.status == 4


@pytest.mark.parametrize("bits,block,d_out,d_in,M,r", [
    (3, 64, 512, 1024, 16, 16),     # few tokens, fused u
    (2, 32, 336, 1088, 5, 16),      # few tokens, groups of 32
    (3, 128, 1040, 768, 300, 48),   # MFMA path, ragged tiles
    (2, 256, 528, 1024, 260, 64),   # MFMA path with split-K
    (4, 32, 512, 4160, 16, 64),     # few tokens, K split over 2 workgroups
    (3, 256, 256, 2048, 1, 16),
    (3, 64, 2064, 16448, 16, 16),   # streamed forward, unaligned group rows
    (2, 128, 4160, 8192, 4, 16),    # streamed forward, 16-byte aligned group rows
])
def test_layer_nf(qb, oracle, bits, block, d_out, d_in, M, r):
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("nfk", d_out, d_in, M, r, 2.0)
    inp = make_inputs(wl, seed=bits + block)
    qw = qb.qlin_quantize_nf(to_dev_f32(inp.W), bits, block, 256)
    codes, am, am2 = oracle.quantize_nf(inp.W, bits, block, 256)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf_bf16(codes, am, am2, bits, block, 256))
    x, A, B, dy = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    y, u = qb.qlin_fwd(qw, x, A, B, r, 2.0, 1)
    dx, dA, dB = qb.qlin_bwd(qw, x, A, B, r, 2.0, dy, 1, u_saved=u)
    xf, Af, Bf, dyf = (oracle.bf16_bits_to_f64(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    y_ref, u_ref = oracle.lora_forward(Wd, xf, Af, Bf, 2.0)
    dX_ref, dA_ref, dB_ref, _ = oracle.lora_backward(Wd, xf, Af, Bf, 2.0, dyf)
    g = lambda t: oracle.bf16_bits_to_f64(bf16_host_bits(t))  # noqa: E731
    parity.check({"y": (g(y), y_ref), "u": (host(u).astype(np.float64), u_ref),
                  "dX": (g(dx), dX_ref), "dA": (g(dA), dA_ref), "dB": (g(dB), dB_ref)},
                 fmts={"u": "f32"})


def test_one_hot_inputs_return_nf3_weight_columns_exactly(qb, oracle):
    """As for NF4: with the adapter off and one-hot tokens, y holds columns of
    W_bf16 and dX rows of it, bit for bit (one bf16 x bf16 product each)."""
    import torch
    from quantized_base_rank_amd.inputs import make_weight
    d_out, d_in, M = 512, 1024, 256
    W = make_weight(d_out, d_in, seed=6)
    qw = qb.qlin_quantize_nf(to_dev_f32(W), 3, 128, 256)
    codes, am, am2 = oracle.quantize_nf(W, 3, 128, 256)
    Wb = oracle.dequant_nf_bf16(codes, am, am2, 3, 128, 256)
    cols = np.arange(M) * 37 % d_in
    xh = np.zeros((M, d_in), np.uint16)
    xh[np.arange(M), cols] = 0x3F80
    A = torch.zeros((4, d_in), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((d_out, 4), dtype=torch.bfloat16, device="cuda")
    y, _ = qb.qlin_fwd(qw, to_dev_bf16(xh), A, B, 4, 0.0, 1)
    assert np.array_equal(bf16_host_bits(y), Wb[:, cols].T)
    rows = np.arange(M) * 11 % d_out
    dyh = np.zeros((M, d_out), np.uint16)
    dyh[np.arange(M), rows] = 0x3F80
    dx, _, _ = qb.qlin_bwd(qw, to_dev_bf16(xh), A, B, 4, 0.0, to_dev_bf16(dyh), 1)
    assert np.array_equal(bf16_host_bits(dx), Wb[rows])
