"""Pins of the oracle's dequantization, INT4 group quantizer, adapter forward /
backward and the QA-LoRA merge.

Checks use library routines of other projects (torch's dtype conversions,
numpy products), finite differences, brute force on tiny inputs and
error bounds that follow from the rounding rules.  Nothing here calls the
HIP library.
"""

import math

import numpy as np
import pytest
import torch
from scipy import integrate
from scipy.stats import norm

from quantized_base_rank_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------ formats


def test_bf16_rounding_matches_torch(oracle):
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(100_000).astype(np.float32) * 3,
        # exact ties: low 16 bits = 0x8000 with even / odd kept bit
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32) * 1,
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38], np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(a), ref)
    back = oracle.bf16_bits_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float64).numpy())


def test_fp16_rounding_matches_torch(oracle):
    a = (np.random.default_rng(6).standard_normal(50_000) * 0.05).astype(np.float32)
    a = np.concatenate([a, np.array([6e-8, 3e-8, 65504.0, -1e-5], np.float32)])
    ref = torch.from_numpy(a).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16_bits(a), ref)


# --------------------------------------------------------- NF4 dequant


def test_dequant_of_power_of_two_blocks_is_level_times_scale(oracle):
    """A block whose absmax is 2^e holding c_i 2^e dequantizes (without
    double quantization) to bf16(c_i) 2^e exactly."""
    c = oracle.nf4_codebook()
    W = np.zeros((2, 64), np.float32)
    W[0, :16] = c * np.float32(2.0 ** -5)
    W[1, :16] = c[::-1] * np.float32(2.0 ** 3)
    codes, a, _ = oracle.quantize_nf4(W, 64, 0)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, a, None, 64, 0))
    cb = torch.from_numpy(c).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(wb[0, :16], cb * 2.0 ** -5)
    assert np.array_equal(wb[1, :16], cb[::-1] * 2.0 ** 3)


@pytest.mark.parametrize("dq", [0, 256])
def test_dequant_error_bound(oracle, dq):
    """|w - w_hat| <= a * gmax/2 + |a - a_hat| + bf16 half-ulp, with gmax the
    largest gap between neighbouring levels."""
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((64, 2048)) * 0.02).astype(np.float32)
    codes, am, am2 = oracle.quantize_nf4(W, 64, dq)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, am, am2, 64, dq))
    _, a, _ = oracle.quantize_nf4(W, 64, 0)
    ahat = oracle.nf4_block_scales(am, am2, dq).astype(np.float64)
    c = oracle.nf4_codebook().astype(np.float64)
    gmax = np.max(np.diff(c))
    a_e = np.repeat(a.astype(np.float64), 64).reshape(W.shape)
    da_e = np.repeat(np.abs(a.astype(np.float64) - ahat), 64).reshape(W.shape)
    bound = a_e * gmax / 2 + da_e + np.abs(wb) * 2.0 ** -8 + 1e-12
    assert np.all(np.abs(W - wb) <= bound)
    rel = oracle.rel_fro(wb, W)
    assert 0.05 < rel < 0.15, rel


def test_row_and_column_dequant_helpers_agree_with_full(oracle):
    rng = np.random.default_rng(8)
    W = (rng.standard_normal((96, 640)) * 0.02).astype(np.float32)
    codes, q, s2 = oracle.quantize_nf4(W, 64, 256)
    full = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, q, s2, 64, 256))
    rows = np.array([0, 5, 95, 40])
    cols = np.array([0, 1, 63, 64, 639, 300])
    assert np.array_equal(oracle.dequant_nf4_rows(codes, q, s2, rows), full[rows])
    assert np.array_equal(oracle.dequant_nf4_cols(codes, q, s2, cols), full[:, cols])


# ----------------------------------------------------------------- INT4


def test_int4_codes_bounds_and_extremes(oracle):
    rng = np.random.default_rng(9)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    q = oracle.unpack_nibbles(codes).reshape(64, 32, 32)
    g = W.reshape(64, 32, 32)
    assert q.max() <= 15
    assert np.all(np.take_along_axis(q, g.argmin(axis=2)[..., None], 2) == 0)
    assert np.all(np.take_along_axis(q, g.argmax(axis=2)[..., None], 2) == 15)
    assert sc.shape == (64, 32) and zp.shape == (64, 32)


def test_int4_error_bound_and_gaussian_level(oracle):
    rng = np.random.default_rng(10)
    W = (rng.standard_normal((128, 2048)) * 0.02).astype(np.float32)
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zp, 32))
    alpha = np.repeat(oracle.f16_bits_to_f32(sc).astype(np.float64), 32, axis=1)
    # round-to-nearest on the grid (alpha/2), fp16 rounding of the zero, bf16 output
    beta_err = np.repeat(np.abs(oracle.f16_bits_to_f32(zp).astype(np.float64)
                                - W.reshape(128, -1, 32).min(axis=2)), 32, axis=1)
    bound = alpha / 2 * (1 + 1e-3) + beta_err + np.abs(wb) * 2.0 ** -8
    assert np.all(np.abs(W - wb) <= bound)
    # relative error of a uniform 16-level grid over the range of 32 normals:
    # alpha = range/15, uniform rounding noise alpha^2/12 on the 30 interior
    # elements of a group (its min and max are reproduced exactly).
    e_range = integrate.quad(
        lambda x: 1 - norm.cdf(x) ** 32 - (1 - norm.cdf(x)) ** 32, -12, 12)[0]
    expect = e_range / 15 / math.sqrt(12) * math.sqrt(30 / 32)
    rel = oracle.rel_fro(wb, W)
    assert abs(rel - expect) / expect < 0.06, (rel, expect)


def test_int4_zero_range_group(oracle):
    W = np.full((1, 64), 0.03125, np.float32)
    W[0, 32:] = np.linspace(-0.1, 0.1, 32, dtype=np.float32)
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    q = oracle.unpack_nibbles(codes)[0]
    assert sc[0, 0] == 0 and np.all(q[:32] == 0)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(codes, sc, zp, 32))
    assert np.all(wb[0, :32] == 0.03125)


# ------------------------------------------------ forward / backward


def _tiny_layer(oracle, pool=1, M=3, N=5, K=64, r=2, seed=11):
    rng = np.random.default_rng(seed)
    Wd = rng.standard_normal((N, K))
    A = rng.standard_normal((r, K // pool))
    B = rng.standard_normal((N, r))
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))
    return Wd, A, B, x, dy


def test_forward_brute_force_loops(oracle):
    """Pure-Python loops on a tiny layer: h = W0 x + s B (A x) for each token."""
    Wd, A, B, x, dy = _tiny_layer(oracle)
    s = 1.5
    y, u = oracle.lora_forward(Wd, x, A, B, s)
    M, N, K, r = x.shape[0], Wd.shape[0], Wd.shape[1], A.shape[0]
    for m in range(M):
        ax = [sum(A[j][k] * x[m][k] for k in range(K)) for j in range(r)]
        for n in range(N):
            ref = sum(Wd[n][k] * x[m][k] for k in range(K)) + s * sum(B[n][j] * ax[j] for j in range(r))
            assert abs(y[m][n] - ref) < 1e-9 * (1 + abs(ref))
        assert np.allclose(u[m], ax, rtol=1e-12, atol=1e-12)


def test_qa_forward_brute_force_loops(oracle):
    """Pooled adapter: the adapter sees the sum of each group of inputs."""
    pool = 16
    Wd, A, B, x, dy = _tiny_layer(oracle, pool=pool)
    s = 0.5
    y, _ = oracle.lora_forward(Wd, x, A, B, s, pool)
    M, N, K, r = x.shape[0], Wd.shape[0], Wd.shape[1], A.shape[0]
    for m in range(M):
        p = [sum(x[m][g * pool + i] for i in range(pool)) for g in range(K // pool)]
        ap = [sum(A[j][g] * p[g] for g in range(K // pool)) for j in range(r)]
        for n in range(N):
            ref = sum(Wd[n][k] * x[m][k] for k in range(K)) + s * sum(B[n][j] * ap[j] for j in range(r))
            assert abs(y[m][n] - ref) < 1e-9 * (1 + abs(ref))


@pytest.mark.parametrize("pool", [1, 16])
def test_backward_matches_finite_differences(oracle, pool):
    """L = <dy, y> is linear in each of x, A and B, so central differences are
    exact up to rounding; every entry of dX, dA and dB is checked."""
    Wd, A, B, x, dy = _tiny_layer(oracle, pool=pool)
    s = 1.75
    dX, dA, dB, du = oracle.lora_backward(Wd, x, A, B, s, dy, pool)

    def loss(x_, A_, B_):
        y, _ = oracle.lora_forward(Wd, x_, A_, B_, s, pool)
        return float(np.sum(dy * y))

    h = 1e-3
    for name, arr, grad in (("x", x, dX), ("A", A, dA), ("B", B, dB)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p = arr.copy(); p[idx] += h
            mth = arr.copy(); mth[idx] -= h
            args = {"x": x, "A": A, "B": B}
            args[name] = p
            lp = loss(args["x"], args["A"], args["B"])
            args[name] = mth
            lm = loss(args["x"], args["A"], args["B"])
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, fd, rtol=1e-7, atol=1e-8), name


def test_special_cases_reduce_to_plain_products(oracle):
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl, seed=0)
    codes, q, s2 = oracle.quantize_nf4(inp.W, 64, 256)
    Wd = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(codes, q, s2))
    x = oracle.bf16_bits_to_f64(inp.x)
    A = oracle.bf16_bits_to_f64(inp.A)
    B = oracle.bf16_bits_to_f64(inp.B)
    dy = oracle.bf16_bits_to_f64(inp.dy)
    # B = 0: plain product
    y, _ = oracle.lora_forward(Wd, x, A, np.zeros_like(B), 2.0)
    assert np.allclose(y, np.einsum("mk,nk->mn", x, Wd), rtol=1e-12, atol=1e-12)
    # s = 0: same, and adapter gradients of A vanish
    y0, _ = oracle.lora_forward(Wd, x, A, B, 0.0)
    assert np.allclose(y0, np.einsum("mk,nk->mn", x, Wd), rtol=1e-12, atol=1e-12)
    dX, dA, dB, _ = oracle.lora_backward(Wd, x, A, B, 0.0, dy)
    assert not dA.any() and not dB.any()
    # W = 0 (all-zero blocks): pure adapter output, W_bf16 is exactly zero
    cz, qz, s2z = oracle.quantize_nf4(np.zeros_like(inp.W), 64, 256)
    Wz = oracle.bf16_bits_to_f64(oracle.dequant_nf4_bf16(cz, qz, s2z))
    assert not Wz.any() and np.all(oracle.unpack_nibbles(cz) == 7)
    yz, u = oracle.lora_forward(Wz, x, A, B, 2.0)
    assert np.allclose(yz, 2.0 * np.einsum("mj,nj->mn", np.einsum("mk,jk->mj", x, A), B),
                       rtol=1e-12, atol=1e-14)
    # M = 1 is a matrix-vector product
    y1, _ = oracle.lora_forward(Wd, x[:1], A, B, 2.0)
    assert np.allclose(y1, y[:1] + 2.0 * (x[:1] @ A.T) @ B.T, rtol=1e-12, atol=1e-12)


def test_qa_merge_folds_adapter_into_zero_points(oracle):
    """Merged INT4 weights (zero' = zero + s B A) without an adapter reproduce
    the adapted layer: exactly in float64, and to 1e-3 with fp16 zeros."""
    rng = np.random.default_rng(12)
    N, K, r, M, G = 48, 512, 4, 6, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, sc, zp = oracle.quantize_int4_group(W, G)
    A = rng.uniform(-0.1, 0.1, (r, K // G))
    B = rng.standard_normal((N, r)) * 0.01
    x = rng.standard_normal((M, K))
    s = 2.0
    q = oracle.unpack_nibbles(codes).astype(np.float64)
    alpha = np.repeat(oracle.f16_bits_to_f32(sc).astype(np.float64), G, axis=1)
    beta = np.repeat(oracle.f16_bits_to_f32(zp).astype(np.float64), G, axis=1)
    W_real = alpha * q + beta
    y_adapted, _ = oracle.lora_forward(W_real, x, A, B, s, G)
    beta_m = oracle.qa_merge_zero(zp, A, B, s)
    W_merged = alpha * q + np.repeat(beta_m, G, axis=1)
    y_merged = x @ W_merged.T
    assert oracle.rel_fro(y_merged, y_adapted) < 1e-12
    beta_m16 = oracle.f16_bits_to_f32(oracle.f32_to_f16_bits(beta_m.astype(np.float32)))
    y_m16 = x @ (alpha * q + np.repeat(beta_m16.astype(np.float64), G, axis=1)).T
    assert oracle.rel_fro(y_m16, y_adapted) < 1e-3
    # average pooling would not fold the same way: the fold would be s B A / G
    assert oracle.rel_fro(x @ (alpha * q + np.repeat(oracle.f16_bits_to_f32(zp) + s * (B @ A) / G,
                                                      G, axis=1)).T, y_adapted) > 1e-3


# ------------------------------------------- INT4 rounding in exact rationals


def _int4_ref_codes(w, alpha, beta):
    """clamp(round_half_even((w - beta)/alpha), 0, 15) in rationals; 0 if alpha = 0."""
    from fractions import Fraction

    from tests.exact_round import round_half_even_int
    a = Fraction(float(alpha))
    if a == 0:
        return 0
    v = round_half_even_int((Fraction(float(w)) - Fraction(float(beta))) / a)
    return min(max(v, 0), 15)


def _near_tie_groups():
    """Groups whose min and max fix dyadic alpha and beta, and whose other
    members sit exactly on the rounding boundaries beta + (k + 1/2) alpha or
    one fp32 step either side of them."""
    rows = []
    for beta, alpha in ((-0.0625, 0.0078125), (-0.04, 0.005859375), (0.5, 0.0009765625),
                        (-1.25, 0.1875)):
        b16 = float(np.float16(beta))
        a16 = float(np.float16(alpha))
        ties = np.array([b16 + (k + 0.5) * a16 for k in range(15)], np.float32)
        assert np.array_equal(ties.astype(np.float64),
                              np.array([b16 + (k + 0.5) * a16 for k in range(15)]))
        lo, hi = np.float32(b16), np.float32(b16 + 15 * a16)
        for variant in (ties, np.nextafter(ties, np.float32(np.inf)),
                        np.nextafter(ties, np.float32(-np.inf))):
            g = np.full(32, lo, np.float32)
            g[1] = hi
            g[2:17] = variant
            g[17:32] = variant
            rows.append(g)
    return np.stack(rows).reshape(-1, 64)


def test_int4_codes_are_the_exact_nearest_integer(oracle):
    """Random groups plus constructed exact ties and one-ulp near-ties: every
    code is the rational round-half-even of (w - beta)/alpha, clamped."""
    rng = np.random.default_rng(22)
    W = np.concatenate([(rng.standard_normal((16, 256)) * 0.02).astype(np.float32).reshape(-1, 64),
                        _near_tie_groups()])
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    q = oracle.unpack_nibbles(codes)
    al = oracle.f16_bits_to_f32(sc)
    be = oracle.f16_bits_to_f32(zp)
    for n in range(W.shape[0]):
        for k in range(W.shape[1]):
            g = k // 32
            assert q[n, k] == _int4_ref_codes(W[n, k], al[n, g], be[n, g]), (n, k)


def test_int4_exact_ties_round_half_to_even(oracle):
    g = _near_tie_groups()[:1]          # first group pair: members 2..16 are exact ties
    codes, sc, zp = oracle.quantize_int4_group(g, 32)
    q = oracle.unpack_nibbles(codes)[0]
    assert q[0] == 0 and q[1] == 15
    assert q[2:17].tolist() == [k if k % 2 == 0 else k + 1 for k in range(15)]


def test_int4_pin_rejects_plausible_other_rules(oracle):
    """The exact pins have teeth: the fp32 chain fl32(fl32(w - beta)/alpha)
    with round-half-even, and the float64 quotient with round-half-up, each
    give a different code somewhere on the near-tie groups."""
    W = _near_tie_groups()
    codes, sc, zp = oracle.quantize_int4_group(W, 32)
    q = oracle.unpack_nibbles(codes).reshape(W.shape)
    al = np.repeat(oracle.f16_bits_to_f32(sc), 32, axis=1)
    be = np.repeat(oracle.f16_bits_to_f32(zp), 32, axis=1)
    chain = np.clip(np.rint(((W - be).astype(np.float32) / al).astype(np.float32)), 0, 15)
    half_up = np.clip(np.floor((W.astype(np.float64) - be) / al + 0.5), 0, 15)
    assert np.any(chain != q)
    assert np.any(half_up != q)


def test_int4_scale_is_the_exactly_rounded_range_over_15(oracle):
    """alpha = RN16((max - min)/15) in exact rationals: random groups, groups
    whose fp64 difference is inexact (tiny min against a large max), and
    groups whose quotient is exactly an fp16 rounding boundary (ties to the
    even significand)."""
    from fractions import Fraction

    from tests.exact_round import FP16, round_rne
    rng = np.random.default_rng(23)
    lo = (rng.standard_normal(3000) * 0.05).astype(np.float32)
    hi = (lo + np.abs(rng.standard_normal(3000)) * 0.1).astype(np.float32)
    # inexact float64 differences
    lo_x = np.array([-1e-30, 1e-30, -3e-25, 2.5e-38], np.float32)
    hi_x = np.array([1.0, 7.5, 0.33, 1000.0], np.float32)
    # exact fp16 boundaries: (hi - lo)/15 = midpoint of two neighbouring fp16
    hs = np.float16(rng.uniform(1e-4, 10.0, 200))
    mid = (hs.astype(np.float64) + np.nextafter(hs, np.float16(np.inf)).astype(np.float64)) / 2
    lo_t = np.zeros(200, np.float32)
    hi_t = (15 * mid).astype(np.float32)
    assert np.array_equal(hi_t.astype(np.float64), 15 * mid)
    L = np.concatenate([lo, lo_x, lo_t])
    H = np.concatenate([hi, hi_x, hi_t])
    got = oracle.f16_bits_to_f32(oracle.int4_group_scale(L, H))
    for i in range(L.size):
        exact = (Fraction(float(H[i])) - Fraction(float(L[i]))) / 15
        assert Fraction(float(got[i])) == round_rne(exact, FP16), (float(L[i]), float(H[i]))
    # and the boundary cases really are ties that went to the even neighbour
    bits = oracle.int4_group_scale(lo_t, hi_t)
    assert np.all(bits & 1 == 0)


# ------------------------------------------------ QA-LoRA merge in fp16


def test_qa_merge_f16_is_the_exactly_rounded_sum(oracle):
    """beta' = RN16(beta + s sum_j B[n][j] A[j][g]) in exact rationals, on a
    random pooled adapter and on constructed sums that land exactly on an fp16
    rounding boundary (ties to the even significand)."""
    from fractions import Fraction

    from quantized_base_rank_amd.inputs import bf16_bits
    from tests.exact_round import FP16, round_rne
    rng = np.random.default_rng(31)
    n, G, r, s = 24, 12, 8, np.float32(2.0)
    zp = oracle.f32_to_f16_bits((rng.standard_normal((n, G)) * 0.03).astype(np.float32))
    A = bf16_bits(rng.uniform(-0.2, 0.2, (r, G)).astype(np.float32))
    B = bf16_bits((rng.standard_normal((n, r)) * 0.01).astype(np.float32))
    got = oracle.qa_merge_zero_f16(zp, A, B, s)
    Af, Bf = oracle.bf16_bits_to_f64(A), oracle.bf16_bits_to_f64(B)
    beta = oracle.f16_bits_to_f32(zp)
    for i in range(n):
        for g in range(G):
            exact = Fraction(float(beta[i, g])) + sum(
                Fraction(float(s)) * Fraction(float(Bf[i, j])) * Fraction(float(Af[j, g]))
                for j in range(r))
            want = round_rne(exact, FP16)
            assert Fraction(float(oracle.f16_bits_to_f32(got[i, g]))) == want, (i, g)
    # ties: 1 + 2^-11 lies half-way between 1 and 1 + 2^-10 (even: 1);
    # (1 + 2^-10) + 2^-11 half-way between it and 1 + 2^-9 (even: the latter)
    zt = oracle.f32_to_f16_bits(np.array([[1.0, 1.0 + 2.0 ** -10]], np.float32))
    At = bf16_bits(np.array([[2.0 ** -6, 2.0 ** -6]], np.float32))
    Bt = bf16_bits(np.array([[2.0 ** -5]], np.float32))
    tie = oracle.qa_merge_zero_f16(zt, At, Bt, np.float32(1.0))
    assert oracle.f16_bits_to_f32(tie).tolist() == [[1.0, 1.0 + 2.0 ** -9]]
    # and the float64 merge it rounds agrees to within half an fp16 step
    ref = oracle.qa_merge_zero(zp, Af, Bf, float(s))
    back = oracle.f16_bits_to_f32(got).astype(np.float64)
    assert np.all(np.abs(back - ref) <= np.abs(ref) * 2.0 ** -11 + 2.0 ** -25)


# ------------------------------------- trainable INT4 scale and zero point


def test_int4_scale_zero_grads_match_finite_differences(oracle):
    """<dy, x W^T> with W = alpha q + beta is linear in every alpha and beta,
    so central differences in float64 equal the gradients up to rounding."""
    rng = np.random.default_rng(51)
    M, N, K, G = 5, 6, 96, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, sc, zp = oracle.quantize_int4_group(W, G)
    q = oracle.unpack_nibbles(codes).astype(np.float64)
    alpha = oracle.f16_bits_to_f32(sc).astype(np.float64)
    beta = oracle.f16_bits_to_f32(zp).astype(np.float64)
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))

    def loss(al, be):
        Wr = np.repeat(al, G, axis=1) * q + np.repeat(be, G, axis=1)
        return float(np.sum(dy * (x @ Wr.T)))

    da, db = oracle.int4_scale_zero_grads(codes, x, dy, G)
    h = 1e-3
    for arr, grad, which in ((alpha, da, 0), (beta, db, 1)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p_, m_ = arr.copy(), arr.copy()
            p_[idx] += h
            m_[idx] -= h
            lp = loss(p_, beta) if which == 0 else loss(alpha, p_)
            lm = loss(m_, beta) if which == 0 else loss(alpha, m_)
            fd[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, fd, rtol=1e-8, atol=1e-9)


def test_int4_scale_zero_grads_loops_and_special_cases(oracle):
    rng = np.random.default_rng(52)
    M, N, K, G = 3, 4, 64, 32
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, _, _ = oracle.quantize_int4_group(W, G)
    q = oracle.unpack_nibbles(codes)
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))
    da, db = oracle.int4_scale_zero_grads(codes, x, dy, G)
    for n in range(N):
        for g in range(K // G):
            ks = range(g * G, (g + 1) * G)
            dw = [sum(dy[m][n] * x[m][k] for m in range(M)) for k in ks]
            assert abs(db[n][g] - sum(dw)) < 1e-12
            assert abs(da[n][g] - sum(int(q[n][k]) * d for k, d in zip(ks, dw))) < 1e-12
    # dbeta is the pooled product dy^T P
    assert np.allclose(db, dy.T @ oracle.pool_sum(x, G), rtol=1e-13, atol=1e-13)
    # every code equal to c: dalpha = c dbeta
    c = 9
    codes_c = oracle.pack_nibbles(np.full((N, K), c, np.uint8))
    da_c, db_c = oracle.int4_scale_zero_grads(codes_c, x, dy, G)
    assert np.allclose(da_c, c * db_c, rtol=1e-13, atol=1e-13)
