"""Low-rank plus quantized decomposition on the GPU (qlin_lq_nf4) against the
oracle [LQ-LoRA record, abstract].  What is unique is compared exactly: the
first quantization (of W itself) bit for bit, rank 0 as plain NF4.  Later
quantizations see an fp32 difference W - L computed on a different path, so
a value next to a level midpoint may take the other level: those are
counted, not required equal.  The rank-r part is compared with the oracle's
run on the GPU's own final quantization, and the reported errors with the
oracle's."""

import numpy as np
import pytest

from tests.gpu_util import bf16_host_bits, host, to_dev_f32, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    qb._lib.lib()
    return qb


def _weight(n, k, r_true, seed):
    """A pretrained-like weight: a few strong directions plus Gaussian noise
    (synthetic; no trained weights are available)."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((n, r_true)) @ rng.standard_normal((r_true, k))) * 0.05 / np.sqrt(r_true) \
        + rng.standard_normal((n, k)) * 0.02
    return W.astype(np.float32)


def _omega(r, k, seed):
    return np.random.default_rng(seed).standard_normal((r, k)).astype(np.float32)


def _run(qb, W, r, iters, power, om, dq=256):
    qw, B, A, errs = qb.qlin_lq_nf4(to_dev_f32(W), r, iters, power, to_dev_f32(om) if r else None, dq)
    am = host(qw.absmax)
    return (u8(qw.codes), am.view(np.int8) if dq else am.view(np.float32),
            host(qw.absmax2) if dq else None, bf16_host_bits(B), bf16_host_bits(A), host(errs))


def test_rank_zero_is_the_quantizer(qb, oracle):
    W = _weight(64, 512, 4, 0)
    codes, am, am2, _, _, errs = _run(qb, W, 0, 2, 0, None)
    c0, a0, a20 = oracle.quantize_nf4(W, 64, 256)
    assert np.array_equal(codes, c0) and np.array_equal(am, a0)
    assert np.array_equal(am2.view(np.uint32), a20.view(np.uint32))
    ref = oracle.lq_decompose(W, 0, 2, 0, np.zeros((0, 512)))[-1]
    assert np.allclose(errs, ref, rtol=1e-5)


@pytest.mark.parametrize("n,k,r,iters,power,dq", [
    (256, 1024, 8, 1, 2, 256),    # one iteration: Q is NF4(W) bit for bit
    (256, 1024, 8, 3, 2, 256),
    (528, 768, 16, 2, 1, 0),      # fp32 block constants; ragged 64-tiles
    (1040, 2112, 64, 2, 1, 256),  # the widest adapter the layer kernels are tuned for
    (256, 512, 5, 2, 1, 256),     # a rank that is not a multiple of 4 (padded inverse, ragged tiles)
])
def test_decomposition(qb, oracle, n, k, r, iters, power, dq):
    W = _weight(n, k, 8, 1 + r)
    om = _omega(r, k, 2 + r)
    codes, am, am2, Bb, Ab, errs = _run(qb, W, r, iters, power, om, dq)
    rc, ram, ram2, rU, rC, rerrs = oracle.lq_decompose(W, r, iters, power, om, 64, dq)
    if iters == 1:
        assert np.array_equal(codes, rc)
    # later quantizations: a few values next to a midpoint may differ
    diff = np.count_nonzero(codes != rc) / codes.size
    assert diff < 2e-3, diff
    # the rank-r part of the residual of the GPU's own quantization
    Wq = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2, 64, dq))
    U, C = oracle.lowrank_part(W.astype(np.float64) - Wq, om, power)
    B = oracle.bf16_bits_to_f64(Bb)
    A = oracle.bf16_bits_to_f64(Ab)
    # factors equal the oracle's up to their bf16 rounding
    assert oracle.rel_fro(B, U) < 4e-3
    assert oracle.rel_fro(A, C) < 4e-3
    L = B @ A
    assert oracle.rel_fro(L, U @ C) < 6e-3
    # the reported error is the oracle's, and the low-rank part helps
    assert np.allclose(errs, rerrs, rtol=2e-3)
    got_err = np.linalg.norm(W - Wq - L) / np.linalg.norm(W)
    assert got_err == pytest.approx(errs[-1], rel=5e-3)
    base = oracle.lq_decompose(W, 0, 1, 0, np.zeros((0, k)), 64, dq)[-1][-1]
    assert errs[-1] < base


def test_zero_weight(qb, oracle):
    W = np.zeros((64, 256), np.float32)
    codes, am, am2, Bb, Ab, errs = _run(qb, W, 8, 2, 1, _omega(8, 256, 3))
    rc, ram, ram2 = oracle.quantize_nf4(W, 64, 256)
    assert np.array_equal(codes, rc)
    assert np.all(oracle.bf16_bits_to_f64(Bb) @ oracle.bf16_bits_to_f64(Ab) == 0.0)
    assert np.all(np.isfinite(errs)) and np.all(errs == 0.0)


def test_workspace_and_argument_errors(qb):
    import torch
    W = torch.zeros((64, 256), dtype=torch.float32, device="cuda")
    with pytest.raises(qb.QlinError) as e:
        qb.qlin_lq_nf4(W, 200, 1, 0, torch.zeros((200, 256), dtype=torch.float32, device="cuda"))
    assert e.value.status == 2  # QLIN_E_SHAPE: rank above 128
