"""Pins of the oracle's low-rank plus quantized decomposition
[LQ-LoRA record, abstract: W is split iteratively into a quantized part and
a high-precision low-rank part], each against something other than the
oracle's own formula: numpy's SVD (Eckart-Young), numpy's Cholesky, the
plain NF4 quantizer, and orthogonality."""

import numpy as np
import pytest

from oracle import qlin_oracle as o


def _lowrank_plus_noise(n, k, r, gap=100.0, noise=1e-3, seed=0):
    """A matrix whose r leading singular values sit `gap` times above the
    rest: r orthonormal directions with values 1..2, plus small noise."""
    rng = np.random.default_rng(seed)
    Uq, _ = np.linalg.qr(rng.standard_normal((n, r)))
    Vq, _ = np.linalg.qr(rng.standard_normal((k, r)))
    s = np.linspace(2.0, 1.0, r)
    return (Uq * s) @ Vq.T + noise * rng.standard_normal((n, k)) / np.sqrt(max(n, k)) * gap / 100.0


def test_thin_qr_is_the_unique_positive_diagonal_factorisation():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((300, 12))
    Q, R = o.thin_qr_pos(X)
    assert np.allclose(Q @ R, X, atol=1e-12)
    assert np.allclose(Q.T @ Q, np.eye(12), atol=1e-12)
    assert np.allclose(R, np.triu(R)) and np.all(np.diag(R) > 0)
    # Cholesky QR (a different algorithm) yields the same factors
    Rc = np.linalg.cholesky(X.T @ X).T
    assert np.allclose(R, Rc, rtol=1e-9, atol=1e-10)
    assert np.allclose(Q, X @ np.linalg.inv(Rc), atol=1e-9)


def test_lowrank_part_equals_truncated_svd():
    """Eckart-Young: the best rank-r approximation is the truncated SVD; with a
    clear spectral gap two power steps reach it to rounding."""
    n, k, r = 200, 300, 6
    R = _lowrank_plus_noise(n, k, r)
    om = np.random.default_rng(2).standard_normal((r, k))
    U, C = o.lowrank_part(R, om, power=2)
    u, sv, vt = np.linalg.svd(R, full_matrices=False)
    L_svd = (u[:, :r] * sv[:r]) @ vt[:r]
    assert o.rel_fro(U @ C, L_svd) < 1e-9
    err = np.linalg.norm(R - U @ C)
    assert abs(err - np.sqrt(np.sum(sv[r:] ** 2))) <= 1e-9 * np.linalg.norm(R)


def test_lowrank_part_teeth():
    """A start that ignores the data (no power step, wrong subspace) is far from
    the SVD: the comparison above can fail."""
    n, k, r = 200, 300, 6
    R = _lowrank_plus_noise(n, k, r)
    om = np.random.default_rng(3).standard_normal((r, k))
    U, C = o.lowrank_part(R + np.random.default_rng(4).standard_normal(R.shape), om, power=0)
    u, sv, vt = np.linalg.svd(R, full_matrices=False)
    assert o.rel_fro(U @ C, (u[:, :r] * sv[:r]) @ vt[:r]) > 1e-3


def test_rank_zero_is_plain_nf4():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((64, 256)) * 0.02
    codes, am, am2, U, C, errs = o.lq_decompose(W, 0, 2, 1, np.zeros((0, 256)))
    c0, a0, a20 = o.quantize_nf4(W.astype(np.float32), 64, 256)
    assert np.array_equal(codes, c0) and np.array_equal(am, a0) and np.array_equal(am2, a20)
    Wq = o.bf16_bits_to_f64(o.dequant_nf4_bf16(c0, a0, a20))
    assert errs[-1] == pytest.approx(np.linalg.norm(W - Wq) / np.linalg.norm(W), rel=1e-12)
    assert U.shape == (64, 0) and C.shape == (0, 256)


def _case(seed=6, n=128, k=512, r_true=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, r_true)) @ rng.standard_normal((r_true, k))) * 0.05 \
        + rng.standard_normal((n, k)) * 0.02


def test_decomposition_bookkeeping_and_orthogonality():
    W = _case()
    r = 8
    om = np.random.default_rng(7).standard_normal((r, W.shape[1]))
    codes, am, am2, U, C, errs = o.lq_decompose(W, r, 3, 2, om)
    Wq = o.bf16_bits_to_f64(o.dequant_nf4_bf16(codes, am, am2))
    R = W - Wq
    # the returned error is the reconstruction error of the returned parts
    assert errs[-1] == pytest.approx(np.linalg.norm(R - U @ C) / np.linalg.norm(W), rel=1e-12)
    # U orthonormal, C its coordinates of R, the rest orthogonal to U
    assert np.allclose(U.T @ U, np.eye(r), atol=1e-12)
    assert np.allclose(C, U.T @ R, atol=1e-12)
    assert np.abs(U.T @ (R - U @ C)).max() < 1e-12
    # the last quantization saw W - L of the previous iteration
    _, _, _, U2, C2, _ = o.lq_decompose(W, r, 2, 2, om)
    c_again, _, _ = o.quantize_nf4((W - U2 @ C2).astype(np.float32), 64, 256)
    assert np.array_equal(codes, c_again)


def test_low_rank_part_lowers_the_error():
    W = _case(seed=8)
    k = W.shape[1]
    base = o.lq_decompose(W, 0, 1, 0, np.zeros((0, k)))[-1][-1]
    prev = base
    for r in (2, 4, 8):
        om = np.random.default_rng(9).standard_normal((r, k))
        e = o.lq_decompose(W, r, 3, 2, om)[-1][-1]
        assert e < prev
        prev = e
    assert prev < 0.95 * base
