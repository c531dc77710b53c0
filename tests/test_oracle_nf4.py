"""Pins of the oracle's NF4 codebook, quantizer and double quantization.

Each test checks the oracle against something other than itself: the forward
normal CDF, independent inverse CDFs, exact rational arithmetic, closed forms
and the figures the QLoRA explainer prints.  Nothing here calls the library.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qlora_page_figures.json")


def _phi(x: float) -> float:
    """Standard normal CDF from erfc (independent of any inverse CDF)."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


# ----------------------------------------------------------------- codebook


def test_codebook_shape_ends_and_zero(oracle):
    c = oracle.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == -1.0 and c[15] == 1.0
    assert c[7] == 0.0 and not np.signbit(c[7])
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert int(np.sum(c < 0)) == 7 and int(np.sum(c > 0)) == 8


def test_codebook_equal_probability_spacing(oracle):
    """Phi(c_i * t) must step by the same probability on each side of zero:
    (delta - 1/2)/7 below, (delta - 1/2)/8 above (forward CDF, not inverse)."""
    c = oracle.nf4_codebook().astype(np.float64)
    delta = oracle.NF4_DELTA
    # recover t = Phi^-1(delta) by bisection on the forward CDF
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if _phi(mid) < delta else (lo, mid)
    t = 0.5 * (lo + hi)
    half = delta - 0.5
    for j in range(1, 8):
        assert abs(_phi(c[7 - j] * t) - (0.5 - j * half / 7)) < 1e-7
    for j in range(1, 9):
        assert abs(_phi(c[7 + j] * t) - (0.5 + j * half / 8)) < 1e-7


def test_codebook_independent_inverse_cdfs_agree_bitwise(oracle):
    import mpmath
    from scipy.special import ndtri

    mpmath.mp.dps = 40
    c_nd = oracle.nf4_codebook()
    c_sp = oracle.nf4_codebook(lambda p: float(ndtri(p)))
    c_mp = oracle.nf4_codebook(
        lambda p: float(mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1)))
    assert np.array_equal(c_nd.view(np.uint32), c_sp.view(np.uint32))
    assert np.array_equal(c_nd.view(np.uint32), c_mp.view(np.uint32))


def test_codebook_bin_occupancy_on_normal_sample(oracle):
    """Bins of the nearest-level quantizer hold (nearly) equal shares of a
    normal sample: counts match the analytic masses within 5 sigma and every
    mass lies within 15% of 1/16 (exact equality is impossible with an exact
    zero and 16 levels, see the design notes)."""
    c = oracle.nf4_codebook().astype(np.float64)
    from scipy.special import ndtri
    t = float(ndtri(oracle.NF4_DELTA))
    n = 2_000_000
    x = np.random.default_rng(0).standard_normal(n)
    # quantize r = x / t with the oracle's nearest-level rule (a = t, scalar)
    idx = oracle.nearest_level_index(x.reshape(-1, 1000), np.full(n // 1000, t), c).ravel()
    counts = np.bincount(idx, minlength=16)
    mids = (c[:-1] + c[1:]) / 2 * t
    edges = np.concatenate([[-np.inf], mids, [np.inf]])
    mass = np.array([_phi(edges[i + 1]) - _phi(edges[i]) for i in range(16)])
    sigma = np.sqrt(n * mass * (1 - mass))
    assert np.all(np.abs(counts - n * mass) < 5 * sigma)
    assert np.all(mass > 0.85 / 16) and np.all(mass < 1.15 / 16)


# ---------------------------------------------------------------- quantizer


def _exact_argmin(w: np.ndarray, a: float, c: np.ndarray) -> np.ndarray:
    """Sketch formulation (argmin of |w/a - c|, first minimum) in exact
    rational arithmetic."""
    levels = [Fraction(float(v)) for v in c]
    fa = Fraction(float(a))
    out = []
    for v in w:
        if fa == 0:
            out.append(7)
            continue
        r = Fraction(float(v)) / fa
        d = [abs(r - lv) for lv in levels]
        out.append(d.index(min(d)))
    return np.array(out)


def test_quantizer_matches_exact_argmin(oracle):
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((8, 64 * 40)) * 0.02).astype(np.float32)
    codes, _, _ = oracle.quantize_nf4(W, 64, 0)
    idx = oracle.unpack_nibbles(codes).reshape(-1, 64)
    blocks = W.reshape(-1, 64)
    c = oracle.nf4_codebook()
    for b in range(blocks.shape[0]):
        a = float(np.abs(blocks[b]).max())
        assert np.array_equal(idx[b], _exact_argmin(blocks[b], a, c))


def test_quantizer_matches_float_argmin_large(oracle):
    """The sketch's fp64 argmin on many random blocks gives the same indices
    (no exact ties occur in continuous random data)."""
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((512, 4096)) * 0.02).astype(np.float32)
    codes, _, _ = oracle.quantize_nf4(W, 64, 0)
    idx = oracle.unpack_nibbles(codes).reshape(-1, 64)
    blocks = W.reshape(-1, 64).astype(np.float64)
    a = np.abs(blocks).max(axis=1, keepdims=True)
    c = oracle.nf4_codebook().astype(np.float64)
    ref = np.argmin(np.abs(blocks[:, :, None] / a[:, :, None] - c[None, None, :]), axis=-1)
    assert np.array_equal(idx, ref)


def test_quantizer_special_cases(oracle):
    c = oracle.nf4_codebook()
    W = np.zeros((4, 128), np.float32)
    # row 0, block 0: +absmax, -absmax... and zeros
    W[0, 0] = 0.5
    W[0, 1] = -0.25
    # row 0, block 1: levels c_i * 2^-3 with absmax 2^-3 present -> exactly i
    e = np.float32(2.0 ** -3)
    W[0, 64:80] = c * e
    # row 1, block 0: single nonzero (negative)
    W[1, 5] = -3.0
    # row 1, block 1: all zero
    # row 2, block 0: -absmax is the extreme
    W[2, :64] = np.linspace(-1.0, 0.5, 64, dtype=np.float32)
    # row 3: every element equal and positive
    W[3, :] = 0.125
    codes, absmax, _ = oracle.quantize_nf4(W, 64, 0)
    idx = oracle.unpack_nibbles(codes)
    assert idx[0, 0] == 15 and idx[0, 2] == 7
    assert np.array_equal(idx[0, 64:80], np.arange(16))
    assert idx[1, 5] == 0 and np.all(np.delete(idx[1, :64], 5) == 7)
    assert np.all(idx[1, 64:] == 7) and absmax[3] == 0.0
    assert idx[2, 0] == 0
    assert np.all(idx[3] == 15)
    # every block with a nonzero element uses an end code
    for b in range(W.size // 64):
        blk = idx.reshape(-1, 64)[b]
        if np.any(W.reshape(-1, 64)[b] != 0):
            assert 0 in blk or 15 in blk


def test_quantizer_tie_goes_to_lower_index(oracle):
    """On a dyadic codebook the midpoints are exact; a value on a midpoint
    takes the lower level (argmin's first minimum)."""
    c = np.array([-1, -0.75, -0.5, -0.375, -0.25, -0.125, -0.0625, 0,
                  0.0625, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 1], np.float32)
    mids = (c[:-1].astype(np.float64) + c[1:]) / 2
    W = np.zeros((1, 64), np.float32)
    W[0, 0] = 1.0
    W[0, 1:16] = mids.astype(np.float32)
    assert np.array_equal(W[0, 1:16].astype(np.float64), mids)
    codes, _, _ = oracle.quantize_nf4(W, 64, 0, codebook=c)
    idx = oracle.unpack_nibbles(codes)[0]
    assert np.array_equal(idx[1:16], np.arange(15))
    assert np.array_equal(idx[1:16], _exact_argmin(W[0, 1:16], 1.0, c))


def test_nibble_packing_order(oracle):
    # byte j of each run of 8 holds element j (low nibble) and j + 4 (high)
    idx = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 0]], np.uint8)
    packed = oracle.pack_nibbles(idx)
    assert packed.tolist() == [[0x51, 0x62, 0x73, 0x84, 0xD9, 0xEA, 0xFB, 0x0C]]
    assert np.array_equal(oracle.unpack_nibbles(packed), idx)
    # the column sampler reads the same layout
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(3, 64), dtype=np.uint8)
    codes = oracle.pack_nibbles(q)
    absmax = np.ones(3, np.float32)
    cols = np.arange(64)
    got = oracle.dequant_nf4_cols(codes, absmax, None, cols, block=64, dq_block=0)
    c = oracle.nf4_codebook()
    assert np.array_equal(got, oracle.bf16_bits_to_f64(oracle.f32_to_bf16_bits(c[q].astype(np.float32))))


def test_quantizer_rejects_nonfinite_and_bad_shape(oracle):
    W = np.zeros((2, 64), np.float32)
    W[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_nf4(W)
    with pytest.raises(ValueError):
        oracle.quantize_nf4(np.zeros((2, 96), np.float32))


# ------------------------------------------------------ double quantization


def test_double_quant_codes_and_bound(oracle):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    _, a, _ = oracle.quantize_nf4(W, 64, 0)
    codes_dq, q, s2 = oracle.quantize_nf4(W, 64, 256)
    codes_nodq, _, _ = oracle.quantize_nf4(W, 64, 0)
    assert np.array_equal(codes_dq, codes_nodq)  # codes use the fp32 absmax
    assert q.dtype == np.int8 and s2.dtype == np.float32
    assert q.size == a.size and s2.size == a.size // 256
    assert np.all(q >= 0) and np.all(q <= 127)
    groups = a.reshape(-1, 256)
    assert np.array_equal(s2, groups.max(axis=1))
    for g in range(groups.shape[0]):
        assert q.reshape(-1, 256)[g][np.argmax(groups[g])] == 127
    # exact rounding rule in rationals: |127 a / s2 - q| <= 1/2, ties even
    for b in range(0, a.size, 37):
        exact = Fraction(127) * Fraction(float(a[b])) / Fraction(float(s2[b // 256]))
        assert abs(exact - int(q[b])) <= Fraction(1, 2)
    ahat = oracle.dq_absmax(q, s2, 256).astype(np.float64)
    s2b = np.repeat(s2, 256).astype(np.float64)
    assert np.all(np.abs(ahat - a) <= s2b / 254 * (1 + 1e-6))
    top = q == 127
    assert np.array_equal(ahat[top], s2b[top])  # the group maximum comes back exactly


def test_double_quant_partial_last_group_and_zero_group(oracle):
    a = np.zeros(300, np.float32)
    a[256:] = np.linspace(0.0, 1.0, 44, dtype=np.float32)
    q, s2 = oracle.double_quantize(a, 256)
    assert s2.tolist() == [0.0, 1.0]
    assert np.all(q[:256] == 0) and q[-1] == 127 and q[256] == 0


def test_storage_accounting_closed_forms(oracle):
    # bits per weight on constants: 32/64 before, 8/64 + 32/(64*256) after
    before = oracle.constant_bits_per_param(64, 0)
    after = oracle.constant_bits_per_param(64, 256)
    assert before == 0.5
    assert after == 0.126953125
    assert before - after == 0.373046875
    # and from the quantizer's actual outputs
    W = (np.random.default_rng(4).standard_normal((256, 1024)) * 0.02).astype(np.float32)
    codes, q, s2 = oracle.quantize_nf4(W, 64, 256)
    bits_const = (q.nbytes + s2.nbytes) * 8 / W.size
    assert bits_const == after and codes.nbytes * 8 / W.size == 4.0
    nb = oracle.nf4_packed_nbytes(256, 1024, 64, 256)
    assert nb["total"] == codes.nbytes + q.nbytes + s2.nbytes


def test_storage_accounting_matches_page_figures(oracle):
    fig = {it["id"]: it for it in json.load(open(GOLDEN))["items"]}
    c = oracle.nf4_codebook()
    assert c.size == fig["levels"]["value"]
    before = oracle.constant_bits_per_param(fig["block"]["value"], 0)
    after = oracle.constant_bits_per_param(fig["block"]["value"], fig["dq_block"]["value"])
    assert before == fig["fp32_constant_overhead_bits"]["value"]
    assert round(after, 3) == fig["dq_overhead_bits"]["value"]
    assert round(before - after, 2) == fig["dq_saving_bits"]["value"]
    n65 = 65e9
    assert round(n65 * before / 8 / 1e9) == fig["fp32_constant_overhead_GB_65B"]["value"]
    assert round(n65 * (before - after) / 8 / 1e9) == fig["dq_saving_GB_65B"]["value"]
    assert n65 * 16 / 8 / 1e9 >= fig["weights_16bit_GB_65B"]["value"]
    bits_nf4 = 4 + after
    assert round(16 / bits_nf4) == fig["nf4_shrink_factor"]["value"]
    # the frozen 4-bit weights of a 65B model fit the single GPU named
    assert n65 * bits_nf4 / 8 / 1e9 < fig["single_gpu_GB"]["value"]
    # LQ-LoRA's 70B at 2.85 bits/param fits its stated footprint
    assert 70e9 * fig["lqlora_70b_avg_bits"]["value"] / 8 / 1e9 < fig["lqlora_70b_GB"]["value"]


def _dq_pairs():
    """Random 8-bit codes against second-level constants over many binades,
    plus edge values: powers of two, the largest fp32, fp32 subnormals."""
    rng = np.random.default_rng(21)
    n = 6000
    q = rng.integers(0, 128, n)
    s2 = (rng.uniform(1.0, 2.0, n) * 2.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    edge_s2 = np.array([1.0, 2.0 ** -20, 3.4028235e38, 1e-40, 1.17549435e-38, 0.0,
                        np.nextafter(np.float32(1), np.float32(2))], np.float32)
    q = np.concatenate([q, np.repeat(np.arange(128), edge_s2.size)])
    s2 = np.concatenate([s2, np.tile(edge_s2, 128)]).astype(np.float32)
    return q.astype(np.int8), s2


def test_dq_reconstruction_is_the_exactly_rounded_quotient(oracle):
    """a_hat = RN32(q s2 / 127) in exact rationals, ties to even [R5]; every
    code 127 reconstructs s2 itself."""
    from tests.exact_round import FP32, round_rne
    q, s2 = _dq_pairs()
    got = oracle.dq_absmax(q, s2, 1)
    for i in range(q.size):
        exact = Fraction(int(q[i])) * Fraction(float(s2[i])) / 127
        assert Fraction(float(got[i])) == round_rne(exact, FP32), (int(q[i]), float(s2[i]))
    top = q == 127
    assert np.array_equal(got[top].view(np.uint32), s2[top].view(np.uint32))


def test_dq_pin_rejects_plausible_other_rules(oracle):
    """The exact-rounding pin above has teeth: rounding twice in fp32 (either
    by a fp32 step 1/127 or by a fp32 product then a quotient) differs from it
    on the same sample, so a mutated oracle would fail that pin."""
    from tests.exact_round import FP32, round_rne
    q, s2 = _dq_pairs()
    step = (s2 * np.float32(1.0 / 127.0)).astype(np.float32)
    alt1 = (q.astype(np.float32) * step).astype(np.float32)
    alt2 = ((q.astype(np.float32) * s2).astype(np.float32) / np.float32(127)).astype(np.float32)
    ref = np.array([float(round_rne(Fraction(int(a)) * Fraction(float(b)) / 127, FP32))
                    for a, b in zip(q, s2)], np.float64)
    assert np.any(alt1.astype(np.float64) != ref)
    assert np.any(alt2.astype(np.float64) != ref)
