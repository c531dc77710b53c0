"""Pins of the oracle's NormalFloat-k generalisation (k = 2, 3, 4 bits,
blocks of 32 to 256): the codebook construction, the quantizer, the bit-plane
packing and the storage accounting.  Checked against the forward normal CDF,
independent inverse CDFs, exact rational arithmetic, hand-computed packings
and closed forms.  Nothing here calls the library."""

import math
from fractions import Fraction

import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _phi(x: float) -> float:
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_k4_is_the_nf4_codebook(oracle):
    assert np.array_equal(oracle.nf_codebook(4).view(np.uint32),
                          oracle.nf4_codebook().view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_ends_zero_and_split(oracle, bits):
    c = oracle.nf_codebook(bits)
    n = 2 ** bits
    assert c.shape == (n,) and c[0] == -1.0 and c[-1] == 1.0
    z = 2 ** (bits - 1) - 1
    assert c[z] == 0.0 and not np.signbit(c[z])
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert int(np.sum(c < 0)) == 2 ** (bits - 1) - 1 and int(np.sum(c > 0)) == 2 ** (bits - 1)


@pytest.mark.parametrize("bits", [2, 3])
def test_codebook_equal_probability_spacing(oracle, bits):
    c = oracle.nf_codebook(bits).astype(np.float64)
    delta = 1.0 - 1.0 / 2 ** (bits + 1)
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if _phi(mid) < delta else (lo, mid)
    t = 0.5 * (lo + hi)
    half = delta - 0.5
    P, Q = 2 ** (bits - 1), 2 ** (bits - 1) - 1
    z = Q
    for j in range(1, Q + 1):
        assert abs(_phi(c[z - j] * t) - (0.5 - j * half / Q)) < 1e-7
    for j in range(1, P + 1):
        assert abs(_phi(c[z + j] * t) - (0.5 + j * half / P)) < 1e-7


@pytest.mark.parametrize("bits", [2, 3])
def test_codebook_independent_inverse_cdfs_agree_bitwise(oracle, bits):
    import mpmath
    from scipy.special import ndtri
    mpmath.mp.dps = 40
    a = oracle.nf_codebook(bits)
    b = oracle.nf_codebook(bits, lambda p: float(ndtri(p)))
    m = oracle.nf_codebook(bits, lambda p: float(mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1)))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), m.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3])
def test_codebook_bin_occupancy(oracle, bits):
    """Counts of a normal sample per bin match the analytic masses (5 sigma)."""
    from scipy.special import ndtri
    c = oracle.nf_codebook(bits).astype(np.float64)
    t = float(ndtri(1.0 - 1.0 / 2 ** (bits + 1)))
    n = 1_000_000
    x = np.random.default_rng(bits).standard_normal(n)
    idx = oracle.nearest_level_index(x.reshape(-1, 1000), np.full(n // 1000, t), c).ravel()
    counts = np.bincount(idx, minlength=c.size)
    edges = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2 * t, [np.inf]])
    mass = np.array([_phi(edges[i + 1]) - _phi(edges[i]) for i in range(c.size)])
    sigma = np.sqrt(n * mass * (1 - mass))
    assert np.all(np.abs(counts - n * mass) < 5 * sigma)


def _exact_argmin(w, a, c):
    levels = [Fraction(float(v)) for v in c]
    fa = Fraction(float(a))
    out = []
    for v in w:
        if fa == 0:
            out.append(int(np.flatnonzero(c == 0)[0]))
            continue
        r = Fraction(float(v)) / fa
        d = [abs(r - lv) for lv in levels]
        out.append(d.index(min(d)))
    return np.array(out)


@pytest.mark.parametrize("bits,block", [(2, 32), (3, 64), (3, 128), (2, 256), (4, 32)])
def test_quantizer_matches_exact_argmin(oracle, bits, block):
    rng = np.random.default_rng(bits * 1000 + block)
    W = (rng.standard_normal((4, 1024)) * 0.02).astype(np.float32)
    codes, a, _ = oracle.quantize_nf(W, bits, block, 0)
    assert codes.shape == (4, 1024 * bits // 8)
    idx = oracle.unpack_bitplanes(codes, bits).reshape(-1, block)
    c = oracle.nf_codebook(bits)
    for b, blk in enumerate(W.reshape(-1, block)):
        assert a[b] == np.abs(blk).max()
        assert np.array_equal(idx[b], _exact_argmin(blk, a[b], c))


def test_quantizer_special_cases_and_ties(oracle):
    c = oracle.nf_codebook(3)
    W = np.zeros((2, 128), np.float32)
    W[0, 0], W[0, 1] = 0.5, -0.5          # both ends
    W[0, 64:72] = c * np.float32(2.0 ** -4)   # the levels themselves (absmax 2^-4 present)
    W[1, 70] = -2.0                       # single nonzero
    codes, a, _ = oracle.quantize_nf(W, 3, 64, 0)
    idx = oracle.unpack_bitplanes(codes, 3)
    assert idx[0, 0] == 7 and idx[0, 1] == 0 and np.all(idx[0, 2:64] == 3)
    assert np.array_equal(idx[0, 64:72], np.arange(8))
    assert np.all(idx[1, :64] == 3) and a[2] == 0.0
    assert idx[1, 70] == 0 and np.all(np.delete(idx[1, 64:], 6) == 3)
    # ties on a dyadic 8-level codebook go to the lower level
    cd = np.array([-1, -0.5, -0.25, 0, 0.125, 0.25, 0.5, 1], np.float32)
    mids = ((cd[:-1].astype(np.float64) + cd[1:]) / 2).astype(np.float32)
    Wt = np.zeros((1, 32), np.float32)
    Wt[0, 0] = 1.0
    Wt[0, 1:8] = mids
    codes, _, _ = oracle.quantize_nf(Wt, 3, 32, 0, codebook=cd)
    assert oracle.unpack_bitplanes(codes, 3)[0, 1:8].tolist() == list(range(7))


def test_bitplane_packing_by_hand(oracle):
    """Element i of a run with index i mod 8 sets bit i of word p exactly when
    bit p of i mod 8 is set: words 0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0."""
    idx = (np.arange(64) % 8).astype(np.uint8).reshape(1, 64)
    words = oracle.pack_bitplanes(idx, 3).view(np.uint32)[0]
    assert words.tolist() == [0xAAAAAAAA, 0xCCCCCCCC, 0xF0F0F0F0] * 2
    two = (np.arange(32) % 4).astype(np.uint8).reshape(1, 32)
    assert oracle.pack_bitplanes(two, 2).view(np.uint32)[0].tolist() == [0xAAAAAAAA, 0xCCCCCCCC]


@pytest.mark.parametrize("bits,block", [(2, 64), (3, 32), (3, 256), (4, 128)])
def test_dequant_error_bound_and_accounting(oracle, bits, block):
    rng = np.random.default_rng(40 + bits)
    W = (rng.standard_normal((64, 2048)) * 0.02).astype(np.float32)
    codes, q, s2 = oracle.quantize_nf(W, bits, block, 256)
    wb = oracle.bf16_bits_to_f64(oracle.dequant_nf_bf16(codes, q, s2, bits, block, 256))
    _, a, _ = oracle.quantize_nf(W, bits, block, 0)
    ahat = oracle.dq_absmax(q, s2, 256).astype(np.float64)
    c = oracle.nf_codebook(bits).astype(np.float64)
    gmax = np.max(np.diff(c))
    a_e = np.repeat(a.astype(np.float64), block).reshape(W.shape)
    da_e = np.repeat(np.abs(a.astype(np.float64) - ahat), block).reshape(W.shape)
    assert np.all(np.abs(W - wb) <= a_e * gmax / 2 + da_e + np.abs(wb) * 2.0 ** -8 + 1e-12)
    # bits per weight: k + 8/block + 32/(256 block)
    nbytes = codes.nbytes + q.nbytes + s2.nbytes
    assert nbytes == oracle.nf_packed_nbytes(64, 2048, bits, block, 256)
    assert nbytes * 8 / W.size == bits + 8 / block + 32 / (256 * block)
