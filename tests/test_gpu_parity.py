"""GPU parity against the CPU oracle, called through the C ABI.

Integer outputs (packed codes, 8-bit absmax, fp16 scale/zero bits, the bf16
decoded weight) must match bit for bit.  Floating outputs (y, dX, dA, dB, u)
must be within relative Frobenius error 2e-3 of the float64 oracle, and
within tighter whole-tensor, per-row and per-tile bounds of the oracle
rounded once to the output format (tests/parity.py).  Shapes span several
tiles of every kernel and end in ragged tails.
"""

import numpy as np
import pytest

from tests.gpu_util import bf16_host_bits, f16_bits, host, to_dev_bf16, to_dev_f32, u8

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    qb._lib.lib()  # must load the HIP library; no fallback exists
    return qb


def _weight(seed, d_out, d_in, std=0.02):
    from quantized_base_rank_amd.inputs import make_weight
    return make_weight(d_out, d_in, seed=seed, std=std)


# ---------------------------------------------------------------- quantizers


@pytest.mark.parametrize("shape,dq", [((256, 256), 256), ((336, 1088), 256), ((16, 64), 256),
                                      ((96, 640), 0), ((4096, 4096), 256)])
def test_nf4_quantizer_bit_exact(qb, oracle, shape, dq):
    W = _weight(1, *shape)
    qw = qb.qlin_quantize_nf4(to_dev_f32(W), 64, dq)
    codes, am, am2 = oracle.quantize_nf4(W, 64, dq)
    assert np.array_equal(u8(qw.codes), codes)
    if dq:
        assert np.array_equal(host(qw.absmax).view(np.int8), am)
        assert np.array_equal(host(qw.absmax2).view(np.uint32), am2.view(np.uint32))
    else:
        assert np.array_equal(host(qw.absmax).view(np.uint32), am.view(np.uint32))


def test_nf4_quantizer_special_blocks(qb, oracle):
    c = oracle.nf4_codebook()
    W = np.zeros((16, 512), np.float32)
    W[0, 64:80] = c * np.float32(2.0 ** -3)          # levels at absmax 2^-3
    W[1, 5] = -3.0                                    # single nonzero
    W[2, :64] = np.linspace(-1.0, 0.5, 64, dtype=np.float32)
    W[3, :] = 0.125
    mids = ((c[:-1].astype(np.float64) + c[1:]) / 2).astype(np.float32)
    W[4, 0] = 1.0
    W[4, 1:16] = mids                                # near-midpoint values
    W[5, :] = np.float32(1e-30)                       # tiny magnitudes
    W[6, 128:192] = -np.float32(7.5)
    for dq in (0, 256):
        qw = qb.qlin_quantize_nf4(to_dev_f32(W), 64, dq)
        codes, am, am2 = oracle.quantize_nf4(W, 64, dq)
        assert np.array_equal(u8(qw.codes), codes)
        if dq:
            assert np.array_equal(host(qw.absmax).view(np.int8), am)
            assert np.array_equal(host(qw.absmax2).view(np.uint32), am2.view(np.uint32))


def test_nf4_quantizer_rejects_nonfinite(qb):
    W = _weight(2, 64, 256)
    W[7, 9] = np.inf
    with pytest.raises(qb.QlinError) as e:
        qb.qlin_quantize_nf4(to_dev_f32(W), 64, 256)
    assert e.value.status == 4
    W[7, 9] = np.nan
    with pytest.raises(qb.QlinError):
        qb.qlin_quantize_nf4(to_dev_f32(W), 64, 0)


@pytest.mark.parametrize("shape", [(64, 1024), (336, 1088), (4096, 11008)])
def test_int4_quantizer_bit_exact(qb, oracle, shape):
    W = _weight(3, *shape)
    qw = qb.qlin_quantize_int4_group(to_dev_f32(W), 32)
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    assert np.array_equal(u8(qw.codes), codes)
    assert np.array_equal(f16_bits(qw.scale), sc)
    assert np.array_equal(f16_bits(qw.zero), zp)


def test_int4_quantizer_rejects_out_of_range(qb):
    W = _weight(4, 32, 64)
    W[3, 3] = 1e6
    with pytest.raises(qb.QlinError) as e:
        qb.qlin_quantize_int4_group(to_dev_f32(W), 32)
    assert e.value.status == 4


# ---------------------------------------------------------- decoded weight


@pytest.mark.parametrize("fmt,dq", [("nf4", 256), ("nf4", 0), ("int4", 0)])
def test_lut_decode_bit_exact(qb, oracle, fmt, dq):
    W = _weight(5, 272, 1152)
    if fmt == "nf4":
        qw = qb.qlin_quantize_nf4(to_dev_f32(W), 64, dq)
        codes, am, am2 = oracle.quantize_nf4(W, 64, dq)
        ref = oracle.dequant_nf4_bf16(codes, am, am2, 64, dq)
    else:
        qw = qb.qlin_quantize_int4_group(to_dev_f32(W), 32)
        codes, sc, zp = oracle.quantize_int4_group(W, 32)
        ref = oracle.dequant_int4_bf16(codes, sc, zp, 32)
    got = bf16_host_bits(qb.qlin_dequant_bf16(qw))
    assert np.array_equal(got, ref)


# ------------------------------------------------------- forward / backward


def _layer_case(qb, oracle, d_out, d_in, M, r, s=2.0, fmt="nf4", seed=0, pool=1, zero_w=False,
                zero_b=False, dq=256):
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("case", d_out, d_in, M, r, s, fmt=fmt, block=64 if fmt == "nf4" else 32,
                  dq_block=dq if fmt == "nf4" else 0, pool=pool)
    inp = make_inputs(wl, seed=seed)
    W = np.zeros_like(inp.W) if zero_w else inp.W
    B = np.zeros_like(inp.B) if zero_b else inp.B
    if fmt == "nf4":
        qw = qb.qlin_quantize_nf4(to_dev_f32(W), 64, dq)
        codes, am, am2 = oracle.quantize_nf4(W, 64, dq)
        Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2, 64, dq))
    else:
        qw = qb.qlin_quantize_int4_group(to_dev_f32(W), 32)
        codes, sc, zp = oracle.quantize_int4_group(W, 32)
        Wd = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zp, 32))
    x, A, Bd, dy = (to_dev_bf16(a) for a in (inp.x, inp.A, B, inp.dy))
    y, u = qb.qlin_fwd(qw, x, A, Bd, r, s, pool)
    dx, dA, dB = qb.qlin_bwd(qw, x, A, Bd, r, s, dy, pool, u_saved=u)
    xf, Af, Bf, dyf = (oracle.bf16_bits_to_f64(a) for a in (inp.x, inp.A, B, inp.dy))
    y_ref, u_ref = oracle.lora_forward(Wd, xf, Af, Bf, s, pool)
    dX_ref, dA_ref, dB_ref, _ = oracle.lora_backward(Wd, xf, Af, Bf, s, dyf, pool)
    got = {
        "y": oracle.bf16_bits_to_f64(bf16_host_bits(y)),
        "u": host(u).astype(np.float64),
        "dX": oracle.bf16_bits_to_f64(bf16_host_bits(dx)),
        "dA": oracle.bf16_bits_to_f64(bf16_host_bits(dA)),
        "dB": oracle.bf16_bits_to_f64(bf16_host_bits(dB)),
    }
    ref = {"y": y_ref, "u": u_ref, "dX": dX_ref, "dA": dA_ref, "dB": dB_ref}
    return qw, (x, A, Bd, dy), got, ref


def _check(oracle, got, ref, keys=("y", "u", "dX", "dA", "dB")):
    from tests import parity
    return parity.check({k: (got[k], ref[k]) for k in keys}, fmts={"u": "f32"})


@pytest.mark.parametrize("d_out,d_in,M,r", [
    (256, 256, 16, 8),        # the tiny layer
    (336, 1088, 1, 16),       # weight-streaming path, ragged splits
    (336, 1088, 5, 16),
    (4096, 4096, 16, 16),     # q_proj shape, decode-sized batch
    (512, 1024, 7, 64),       # weight-streaming, adapter wider than 16 (extra du rounds)
    (256, 512, 16, 128),      # weight-streaming, widest adapter
    (4608, 512, 4, 16),       # weight-streaming, 9 row splits (two fix-up batches)
    (528, 320, 300, 64),      # MFMA path: 2 + ragged tiles, K tail of 64
    (512, 1024, 17, 8),       # just above the weight-streaming threshold
    (1040, 768, 513, 48),
    (512, 4096, 260, 16),     # few tiles, long K: split-K with ticketed fix-up
    (256, 1280, 100, 16),     # split-K with an odd number of K steps per split (a masked pad step)
    (400, 640, 600, 96),      # MFMA path, adapter wider than 64: three-slot ring in the dA / dB
                              # reductions, two token shares of 300 (ragged last stage)
    (272, 1088, 300, 128),    # MFMA path, widest adapter
])
def test_layer_nf4(qb, oracle, d_out, d_in, M, r):
    _, _, got, ref = _layer_case(qb, oracle, d_out, d_in, M, r)
    _check(oracle, got, ref)


@pytest.mark.parametrize("d_out,d_in,M,r,pool", [
    (256, 1024, 8, 16, 1),
    (272, 1088, 300, 64, 1),
    (256, 1024, 16, 16, 32),    # QA-LoRA pooled adapter, weight-streaming
    (528, 1088, 300, 64, 32),   # QA-LoRA pooled adapter, MFMA path (34 groups)
    (272, 2048, 260, 16, 32),   # pooled, MFMA path, group count a multiple of 8
    (256, 1280, 100, 16, 32),   # pooled, split-K with an odd number of K steps per split
])
def test_layer_int4(qb, oracle, d_out, d_in, M, r, pool):
    _, _, got, ref = _layer_case(qb, oracle, d_out, d_in, M, r, fmt="int4", pool=pool)
    _check(oracle, got, ref)


@pytest.mark.parametrize("M", [16, 300])
def test_adapter_dominant_zero_weight(qb, oracle, M):
    """W = 0: the adapter carries the whole output."""
    _, _, got, ref = _layer_case(qb, oracle, 512, 1024, M, 16, zero_w=True)
    _check(oracle, got, ref)


@pytest.mark.parametrize("M", [16, 300])
def test_plain_product_when_adapter_is_zero(qb, oracle, M):
    _, _, got, ref = _layer_case(qb, oracle, 512, 1024, M, 16, zero_b=True)
    _check(oracle, got, ref, keys=("y", "u", "dX", "dA"))
    assert not got["dA"].any()


@pytest.mark.parametrize("M", [16, 256])
def test_one_hot_inputs_return_weight_columns_exactly(qb, oracle, M):
    """With the adapter off (s = 0) and x a one-hot row, y is one column of
    W_bf16: a single bf16 x bf16 product accumulated in fp32 is exact."""
    import torch
    d_out, d_in = 512, 1024
    W = _weight(6, d_out, d_in)
    qw = qb.qlin_quantize_nf4(to_dev_f32(W), 64, 256)
    codes, am, am2 = oracle.quantize_nf4(W, 64, 256)
    Wb = oracle.dequant_nf4_bf16(codes, am, am2)
    cols = np.arange(M) * 37 % d_in
    xh = np.zeros((M, d_in), np.uint16)
    xh[np.arange(M), cols] = 0x3F80  # 1.0
    x = to_dev_bf16(xh)
    A = torch.zeros((4, d_in), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((d_out, 4), dtype=torch.bfloat16, device="cuda")
    y, _ = qb.qlin_fwd(qw, x, A, B, 4, 0.0, 1)
    assert np.array_equal(bf16_host_bits(y), Wb[:, cols].T)
    # and dY one-hot gives rows of W_bf16 through the transposed path
    rows = np.arange(M) * 11 % d_out
    dyh = np.zeros((M, d_out), np.uint16)
    dyh[np.arange(M), rows] = 0x3F80
    dx, _, _ = qb.qlin_bwd(qw, x, A, B, 4, 0.0, to_dev_bf16(dyh), 1)
    assert np.array_equal(bf16_host_bits(dx), Wb[rows])


def test_recompute_u_matches_saved(qb, oracle):
    qw, (x, A, B, dy), got, ref = _layer_case(qb, oracle, 512, 1024, 64, 16)
    dx2, dA2, dB2 = qb.qlin_bwd(qw, x, A, B, 16, 2.0, dy, 1, u_saved=None)
    assert np.array_equal(oracle.bf16_bits_to_f64(bf16_host_bits(dB2)), got["dB"])
    assert np.array_equal(oracle.bf16_bits_to_f64(bf16_host_bits(dA2)), got["dA"])


@pytest.mark.parametrize("M", [16, 300])
def test_runs_are_bit_identical(qb, oracle, M):
    qw, (x, A, B, dy), _, _ = _layer_case(qb, oracle, 528, 1088, M, 16)
    outs = []
    for _ in range(2):
        y, u = qb.qlin_fwd(qw, x, A, B, 16, 2.0, 1)
        dx, dA, dB = qb.qlin_bwd(qw, x, A, B, 16, 2.0, dy, 1, u_saved=u)
        outs.append([bf16_host_bits(t) for t in (y, dx, dA, dB)] + [host(u)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_qa_merge_equivalence(qb, oracle):
    """Fold the pooled adapter into the fp16 zero points on the GPU
    (qlin_qa_merge: zero' = RN16(zero + s B A)) and run the adapter-free
    layer (r = 0).

    (a) The merged zero points equal the oracle's exactly rounded ones bit
        for bit.
    (b) The GPU forward of the merged INT4 model matches the oracle's forward
        of the same merged model (ordinary parity).
    (c) It stays within 2e-3 + e_m of the oracle's *adapted* layer, where
        e_m = |y_merged - y_adapted| / |y_adapted| in float64: merging changes
        which bf16 values the weights decode to (they are re-rounded after the
        zero shift), so the merged model cannot be closer than that; in real
        arithmetic the two models agree to ~4e-4 (fp16 zero rounding)."""
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    from tests import parity
    wl = Workload("qa", 528, 1088, 64, 16, 2.0, fmt="int4", block=32, dq_block=0, pool=32)
    inp = make_inputs(wl, seed=7)
    qw = qb.qlin_quantize_int4_group(to_dev_f32(inp.W), 32)
    x, A, B = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B))
    codes, sc, zp = oracle.quantize_int4_group(inp.W, 32)
    merged = qb.qlin_qa_merge(qw, A, B, 16, 2.0)
    zbits = oracle.qa_merge_zero_f16(zp, inp.A, inp.B, 2.0)
    assert np.array_equal(f16_bits(merged.zero), zbits)
    y_merged, u_none = qb.qlin_fwd(merged, x, None, None, 0, 0.0, 32)
    assert u_none is None
    xf, Af, Bf = (oracle.bf16_bits_to_f64(a) for a in (inp.x, inp.A, inp.B))
    y_gpu = oracle.bf16_bits_to_f64(bf16_host_bits(y_merged))
    Wm = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zbits, 32))
    y_m_ref = xf @ Wm.T
    Wd = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zp, 32))
    y_ad_ref, _ = oracle.lora_forward(Wd, xf, Af, Bf, 2.0, 32)
    parity.check({"y_merged": (y_gpu, y_m_ref)})
    e_m = oracle.rel_fro(y_m_ref, y_ad_ref)
    assert oracle.rel_fro(y_gpu, y_ad_ref) <= TOL + e_m


@pytest.mark.parametrize("M", [4, 300])
def test_adapter_free_forward(qb, oracle, M):
    """r = 0: the plain quantized product, no adapter operands at all."""
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    from tests import parity
    wl = Workload("plain", 512, 1024, M, 4, 2.0)
    inp = make_inputs(wl, seed=8)
    qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), 64, 256)
    y, u = qb.qlin_fwd(qw, to_dev_bf16(inp.x), None, None, 0, 2.0)
    assert u is None
    codes, am, am2 = oracle.quantize_nf4(inp.W, 64, 256)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2))
    ref = oracle.bf16_bits_to_f64(inp.x) @ Wd.T
    parity.check({"y": (oracle.bf16_bits_to_f64(bf16_host_bits(y)), ref)})


def test_workspace_reuse_across_shapes(qb, oracle):
    """One workspace for calls of different shapes: a large-token backward
    that recomputes u into the workspace, then a few-token backward whose
    split reduction takes tickets on 86 column tiles.  The ticket counters
    sit in a region no call writes anything else into, so the second call
    must see them at zero."""
    import torch
    ws = torch.zeros(256 << 20, dtype=torch.uint8, device="cuda")
    qw1, (x1, A1, B1, dy1), _, _ = _layer_case(qb, oracle, 512, 1024, 64, 16)
    qb.qlin_bwd(qw1, x1, A1, B1, 16, 2.0, dy1, 1, u_saved=None, ws=ws)
    qb.qlin_fwd(qw1, x1, A1, B1, 16, 2.0, 1, ws=ws, want_u=False)
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("reuse", 256, 11008, 16, 16, 2.0)
    inp = make_inputs(wl, seed=9)
    qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), 64, 256)
    x, A, B, dy = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    y, u = qb.qlin_fwd(qw, x, A, B, 16, 2.0, 1, ws=ws)
    dx, dA, dB = qb.qlin_bwd(qw, x, A, B, 16, 2.0, dy, 1, u_saved=u, ws=ws)
    codes, am, am2 = oracle.quantize_nf4(inp.W, 64, 256)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2))
    xf, Af, Bf, dyf = (oracle.bf16_bits_to_f64(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    dX_ref, dA_ref, dB_ref, _ = oracle.lora_backward(Wd, xf, Af, Bf, 2.0, dyf)
    got = {"dX": oracle.bf16_bits_to_f64(bf16_host_bits(dx)),
           "dA": oracle.bf16_bits_to_f64(bf16_host_bits(dA)),
           "dB": oracle.bf16_bits_to_f64(bf16_host_bits(dB))}
    _check(oracle, got, {"dX": dX_ref, "dA": dA_ref, "dB": dB_ref}, keys=("dX", "dA", "dB"))


@pytest.mark.parametrize("d_out,d_in,M,r,fmt,pool", [
    (512, 4160, 1, 16, "nf4", 1),     # weight-streaming forward: K split over 2 workgroups
    (512, 4160, 16, 64, "nf4", 1),
    (256, 11008, 16, 16, "nf4", 1),   # 3 K splits, fused u
    (256, 11008, 1, 64, "nf4", 1),
    (512, 11008, 16, 64, "int4", 32), # pooled adapter, 3 K splits
    (8192, 1024, 16, 64, "nf4", 1),   # backward: 16 row splits x r 64 du partials (no LDS stage)
])
def test_layer_few_token_split_paths(qb, oracle, d_out, d_in, M, r, fmt, pool):
    _, _, got, ref = _layer_case(qb, oracle, d_out, d_in, M, r, fmt=fmt, pool=pool)
    _check(oracle, got, ref)


def _poisoned_run(qb, oracle, d_out, d_in, M, r, row, where, cols):
    """Forward + backward twice: clean, and with +Inf written into `cols` of
    token `row` of x (where='x') or dY (where='dy')."""
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    wl = Workload("nan", d_out, d_in, M, r, 2.0)
    inp = make_inputs(wl, seed=13)
    qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), 64, 256)
    outs = []
    for poison in (False, True):
        xh, dyh = inp.x.copy(), inp.dy.copy()
        if poison:
            (xh if where == "x" else dyh)[row, cols] = 0x7F80  # +Inf
        x, A, B, dy = (to_dev_bf16(a) for a in (xh, inp.A, inp.B, dyh))
        y, u = qb.qlin_fwd(qw, x, A, B, r, 2.0, 1)
        dx, _, _ = qb.qlin_bwd(qw, x, A, B, r, 2.0, dy, 1, u_saved=u)
        outs.append((bf16_host_bits(y), bf16_host_bits(dx)))
    return outs


def test_nonfinite_token_does_not_leak_forward(qb, oracle):
    """d_in % 128 == 64: the last K step of the large-token forward holds 64
    columns.  An Inf in the next token's first 64 features must leave every
    other token's y bit-identical."""
    M, bad = 40, 6
    (y0, _), (y1, _) = _poisoned_run(qb, oracle, 256, 320, M, 16, bad, "x", slice(0, 64))
    keep = np.arange(M) != bad
    assert np.array_equal(y1[keep], y0[keep])
    assert not np.all(np.isfinite(oracle.bf16_bits_to_f64(y1[bad])))


def test_nonfinite_token_does_not_leak_backward(qb, oracle):
    """d_out % 64 == 16: the last step of the large-token input gradient
    holds 16 columns of dY.  An Inf in the next token's first 48 values must
    leave every other token's dX bit-identical."""
    M, bad = 40, 6
    (_, d0), (_, d1) = _poisoned_run(qb, oracle, 528, 256, M, 16, bad, "dy", slice(0, 48))
    keep = np.arange(M) != bad
    assert np.array_equal(d1[keep], d0[keep])


@pytest.mark.parametrize("d_out,d_in,M", [
    (256, 1024, 64),     # whole tiles
    (272, 1088, 300),    # ragged tiles in n, k and tokens
    (512, 2048, 1),      # a single token
])
def test_int4_scale_zero_grad(qb, oracle, d_out, d_in, M):
    """Gradients of the INT4 group scales and zero points (fp32 outputs)
    against the float64 oracle, with the fp32 bounds of tests/parity.py."""
    from quantized_base_rank_amd.inputs import Workload, make_inputs
    from tests import parity
    wl = Workload("loqa", d_out, d_in, M, 16, 2.0, fmt="int4", block=32, dq_block=0, pool=32)
    inp = make_inputs(wl, seed=17)
    qw = qb.qlin_quantize_int4_group(to_dev_f32(inp.W), 32)
    ds, dz = qb.qlin_int4_scale_zero_grad(qw, to_dev_bf16(inp.x), to_dev_bf16(inp.dy))
    codes, _, _ = oracle.quantize_int4_group(inp.W, 32)
    da_ref, db_ref = oracle.int4_scale_zero_grads(codes, oracle.bf16_bits_to_f64(inp.x),
                                                  oracle.bf16_bits_to_f64(inp.dy), 32)
    parity.check({"dscale": (host(ds).astype(np.float64), da_ref),
                  "dzero": (host(dz).astype(np.float64), db_ref)},
                 fmts={"dscale": "f32", "dzero": "f32"})


@pytest.mark.parametrize("d_out,d_in,M,r,fmt,pool,dq", [
    (4112, 8192, 16, 16, "nf4", 1, 256),    # streamed forward: ragged last row group
    (4096, 8256, 5, 64, "nf4", 1, 256),     # ragged last chunk (K % 256 == 64), u by the few-token product
    (4096, 8256, 16, 64, "int4", 32, 0),    # INT4 with unaligned group rows, pooled adapter
    (4160, 8192, 16, 32, "int4", 32, 0),    # INT4 with 16-byte aligned group rows
    (4160, 8192, 7, 16, "nf4", 1, 0),       # NF4 with fp32 block constants (no double quantization)
    (2064, 16448, 1, 16, "nf4", 1, 256),    # one token, 17 row groups
])
def test_layer_streamed_few_token(qb, oracle, d_out, d_in, M, r, fmt, pool, dq):
    """Weights above 32 M elements at <= 16 tokens take the streamed forward
    (K split over the resident workgroups, ticketed fixed-order fix-up)."""
    _, _, got, ref = _layer_case(qb, oracle, d_out, d_in, M, r, fmt=fmt, pool=pool, dq=dq)
    _check(oracle, got, ref)


@pytest.mark.parametrize("d_out,d_in,M,r,fmt,pool", [
    (4096, 8256, 5, 64, "nf4", 1),      # streamed backward: dA formed without the dX pass
    (4096, 8256, 16, 64, "int4", 32),   # streamed, pooled adapter
    (336, 1088, 7, 16, "nf4", 1),       # one-shot few-token kernel
    (256, 1280, 100, 16, "nf4", 1),     # large-M path
])
def test_backward_without_input_gradient(qb, oracle, d_out, d_in, M, r, fmt, pool):
    """dX is optional (the first layer of a network needs none); dA and dB
    must come out the same way without it."""
    qw, (x, A, Bd, dy), got, ref = _layer_case(qb, oracle, d_out, d_in, M, r, fmt=fmt, pool=pool)
    _, u = qb.qlin_fwd(qw, x, A, Bd, r, 2.0, pool)
    dx, dA, dB = qb.qlin_bwd(qw, x, A, Bd, r, 2.0, dy, pool, u_saved=u, need_dx=False)
    assert dx is None
    got2 = {"dA": oracle.bf16_bits_to_f64(bf16_host_bits(dA)), "dB": oracle.bf16_bits_to_f64(bf16_host_bits(dB))}
    _check(oracle, got2, ref, keys=("dA", "dB"))
