"""CPU oracle for the frozen 4-bit linear layer with a 16-bit low-rank adapter.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously-correct
statement of what the library computes.  Only the test-suite, the smoke check
(``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may import
it.  The library (``quantized_base_rank_amd`` and its HIP code) never imports,
links or calls anything here, and this module imports nothing from the
library: the two share no code, no tables and no helpers.

Everything is numpy in float64 unless a step fixes a narrower format
(fp32 absmax, int8 double-quantized constants, fp16 INT4 scale/zero, bf16
dequantized weights), in which case that format's IEEE rounding is applied
exactly where the step says so.

Sources (web pages on the subject; cited by page title and section):

* [QLoRA] "QLoRA: Efficient Finetuning of Quantized LLMs" explainer
  (azimuth.plus): sections "Background: what is quantization?",
  "Innovation 1: 4-bit NormalFloat (NF4)", "Background: how LoRA works",
  "The QLoRA recipe: quantize, then adapt", "Innovation 2: Double
  Quantization", "The complete QLoRA forward pass" and "The same idea in
  code" (a numpy sketch, captioned as simplified).
* [QA-LoRA] "QA-LoRA: Quantization-Aware Low-Rank Adaptation of Large
  Language Models" (codewithpapers.app record), abstract.
* [LQ-LoRA] "LQ-LoRA: Low-rank Plus Quantized Matrix Decomposition for
  Efficient Language Model Finetuning" (codewithpapers.app record), abstract.

Readings taken where the pages are silent or garbled are tagged [R#] and
listed in the repository's design notes.

Parity status per function
--------------------------
* nf4_codebook ............ pinned (quantile spacing via the forward CDF,
                             two independent inverse CDFs, end/zero levels,
                             bin occupancy on a normal sample)
* quantize_nf4 ............ pinned (brute-force exact argmin, special cases,
                             tie rule on a dyadic codebook, DQ accounting)
* dequant_nf4_bf16 ........ pinned (bf16 rounding vs torch, c_i*2^e blocks,
                             reconstruction error bound)
* dq_absmax ............... pinned (exact rational RN32(q s2 / 127) on
                             random and edge codes; q = 127 gives s2)
* quantize_int4_group ..... pinned (codes against the exact nearest integer
                             in rationals, constructed exact ties and
                             one-ulp near-ties, scale against the exact
                             rational RN16, bounds, min->0, max->15,
                             Gaussian error level)
* dequant_int4_bf16 ....... pinned (error bound vs the input)
* lora_forward / backward . pinned (finite differences, B=0 / W=0 / s=0
                             reductions to plain products, M=1)
* nf_codebook / quantize_nf / dequant_nf_bf16 (NormalFloat-k, k = 2, 3, 4,
  blocks 32..256) ........ pinned (k = 4 reproduces NF4; quantile spacing
                             via the forward CDF; independent inverse CDFs;
                             bin occupancy; exact argmin; special cases;
                             bit-plane packing by hand; storage accounting)
* qa_merge_zero ........... pinned (merged == unmerged forward)
* int4_scale_zero_grads ... pinned (central differences of the real-valued
                             layer in alpha and beta, brute-force loops,
                             dbeta = dy^T pool_sum(x), constant codes); the
                             formula itself is a reading (the page gives
                             none), so its agreement with LoQA's own operator
                             is "parity unpinned"
* qa_merge_zero_f16 ....... pinned (exact rational RN16 of beta + s B A,
                             fp16 boundary ties, merged forward error)
* lq_decompose ............ pinned (rank 0 is plain NF4; on a low-rank plus
                             noise matrix the rank-r part equals numpy's
                             truncated SVD and the error its Eckart-Young
                             value; residual orthogonal to the basis; error
                             below the rank-0 error and falling with r).  The
                             iteration itself is a reading of a one-sentence
                             abstract; agreement with LQ-LoRA's own code is
                             "parity unpinned"
* The absolute values of the NF4 levels beyond the stated construction are
  "parity unpinned": the pages print no table of levels.
"""

from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

F64 = np.float64
F32 = np.float32

# ---------------------------------------------------------------------------
# IEEE format helpers (the oracle's own; nothing here is shared)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16, ties to even; returns the uint16 bit patterns.

    Finite inputs only (the callers never produce NaN or Inf)."""
    u = np.ascontiguousarray(np.asarray(a, dtype=F32)).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(F32).astype(F64)


def f32_to_f16_bits(a) -> np.ndarray:
    """Round fp32 values to IEEE binary16 (ties to even); returns uint16 bits."""
    return np.asarray(a, dtype=F32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(F32)


# ---------------------------------------------------------------------------
# NF4 codebook  [QLoRA, "Innovation 1: 4-bit NormalFloat (NF4)"; "The same
# idea in code"]
# ---------------------------------------------------------------------------

#: Outermost probability used for the levels: the sketch's outermost quantile
#: (15 + 1/2)/16.  [R1]
NF4_DELTA = 31.0 / 32.0
#: Levels below / above the exact zero.  Sixteen levels with an exact zero
#: force an uneven split; the positive side takes the extra level.  [R1]
NF4_NEG, NF4_POS = 7, 8


def nf4_levels_f64(inv_cdf=None) -> list[float]:
    """The 16 NormalFloat levels in float64, before rounding to fp32.

    Construction [R1]: with t = Phi^-1(delta), the positive levels are
    Phi^-1(1/2 + j (delta - 1/2)/8) / t for j = 1..8, the negative levels are
    -Phi^-1(1/2 + j (delta - 1/2)/7) / t for j = 1..7, plus an exact 0.
    Each side therefore sits at equally spaced probabilities of N(0, 1)
    (equal mass between neighbours), the set is normalised to [-1, 1] and
    contains 0 exactly.
    """
    if inv_cdf is None:
        inv_cdf = NormalDist().inv_cdf
    t = inv_cdf(NF4_DELTA)
    half = NF4_DELTA - 0.5
    pos = [inv_cdf(0.5 + j * half / NF4_POS) / t for j in range(1, NF4_POS + 1)]
    neg = [-inv_cdf(0.5 + j * half / NF4_NEG) / t for j in range(1, NF4_NEG + 1)]
    return sorted(neg + [0.0] + pos)


def nf4_codebook(inv_cdf=None) -> np.ndarray:
    """fp32[16] NF4 levels, ascending; c[0] = -1, c[7] = 0, c[15] = +1."""
    return np.array(nf4_levels_f64(inv_cdf), dtype=F32)


# ---------------------------------------------------------------------------
# Blockwise absmax quantization + double quantization
# [QLoRA, "Background: what is quantization?", "Innovation 2: Double
#  Quantization", "The same idea in code"]
# ---------------------------------------------------------------------------

#: Index of the exact-zero level; all-zero blocks encode to it.  [R12]
NF4_ZERO_INDEX = 7


def nearest_level_index(w: np.ndarray, a: np.ndarray, codebook: np.ndarray) -> np.ndarray:
    """Index of the level nearest to w/a, ties to the lower index.  [R2, R3]

    ``w`` has shape (n_blocks, block) and ``a`` (n_blocks,) holds each block's
    absmax.  The nearest level to r = w/a is the number of midpoints
    m_k = (c_k + c_{k+1})/2 that lie strictly below r; a value exactly on a
    midpoint therefore goes to the lower level, as the sketch's argmin (first
    minimum) does.  The comparison r > m_k is evaluated as w > m_k * a, which
    is exact in float64: the midpoints of fp32 levels and the fp32 absmax
    have few enough significant bits that the product is representable.
    """
    w = np.asarray(w, dtype=F64)
    a = np.asarray(a, dtype=F64)
    c = np.asarray(codebook, dtype=F64)
    mids = (c[:-1] + c[1:]) / 2.0
    idx = np.zeros(w.shape, dtype=np.int64)
    for m in mids:
        idx += w > (m * a)[:, None]
    zero_idx = int(np.flatnonzero(c == 0.0)[0]) if np.any(c == 0.0) else NF4_ZERO_INDEX
    idx[a == 0.0] = zero_idx
    return idx


def pack_nibbles(idx: np.ndarray) -> np.ndarray:
    """Two 4-bit indices per byte along each row.  Each run of 8 elements
    fills 4 bytes: byte j of the run holds element j in its low nibble and
    element j + 4 in its high nibble (rows have a multiple of 8 elements).
    [R8]"""
    idx = np.asarray(idx, dtype=np.uint8)
    n = idx.shape[-1]
    assert n % 8 == 0, "rows must hold a multiple of 8 elements"
    g = idx.reshape(idx.shape[:-1] + (n // 8, 8))
    out = g[..., 0:4] | (g[..., 4:8] << 4)
    return out.reshape(idx.shape[:-1] + (n // 2,)).astype(np.uint8)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles.  [R8]"""
    codes = np.asarray(codes, dtype=np.uint8)
    nb = codes.shape[-1]
    assert nb % 4 == 0, "rows must hold a multiple of 4 bytes"
    c = codes.reshape(codes.shape[:-1] + (nb // 4, 4))
    out = np.empty(c.shape[:-1] + (8,), dtype=np.uint8)
    out[..., 0:4] = c & 0x0F
    out[..., 4:8] = c >> 4
    return out.reshape(codes.shape[:-1] + (nb * 2,))


def double_quantize(absmax: np.ndarray, dq_block: int = 256):
    """Second-level quantization of the fp32 first-level constants.  [R4-R6]

    Consecutive flattened block constants are grouped ``dq_block`` at a time
    (the last group may be short).  Each group keeps one fp32 constant, its
    maximum s2; each member a is stored as the 8-bit integer
    q = round_half_even(127 a / s2) in [0, 127] (0 when s2 = 0).
    The division is float64; 127 a is exact there and the quotient cannot
    land on a half-integer by rounding, so this is the exactly rounded value.
    """
    a = np.asarray(absmax, dtype=F32)
    nb = a.size
    ng = -(-nb // dq_block)
    pad = np.zeros(ng * dq_block, dtype=F32)
    pad[:nb] = a
    s2 = pad.reshape(ng, dq_block).max(axis=1).astype(F32)
    s2_per_block = np.repeat(s2, dq_block)[:nb].astype(F64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((127.0 * a.astype(F64)) / s2_per_block)
    q[s2_per_block == 0.0] = 0.0
    return q.astype(np.int8), s2


def dq_absmax(q: np.ndarray, s2: np.ndarray, dq_block: int = 256) -> np.ndarray:
    """fp32 first-level constants reconstructed from their 8-bit codes.  [R5]

    The 8-bit grid of a group runs from 0 to its maximum s2 in 127 equal
    steps, so code q stands for the real number q * s2 / 127.  The stored
    constant is that number rounded once to fp32 (ties to even):
    a_hat = RN32(q * s2 / 127).  Here q * s2 is exact in float64 (7 + 24
    significant bits) and the float64 quotient is rounded again to fp32;
    the quotient either is an fp32 number or lies at least 1/254 of an fp32
    ulp away from every fp32 rounding boundary, far more than the float64
    rounding error, so the two roundings give the single exact one.  For
    q = 127 this returns s2 itself."""
    q = np.asarray(q, dtype=np.int8).astype(F64)
    s2 = np.asarray(s2, dtype=F32).astype(F64)
    s2_b = np.repeat(s2, dq_block)[: q.size]
    return ((q * s2_b) / 127.0).astype(F32)


def _dq_absmax_of_blocks(absmax, absmax2, bids, dq_block: int) -> np.ndarray:
    """dq_absmax for the flat block indices ``bids`` only (same rule)."""
    if not dq_block:
        return np.asarray(absmax, F32)[bids]
    q = np.asarray(absmax, np.int8)[bids].astype(F64)
    s2 = np.asarray(absmax2, F32)[bids // dq_block].astype(F64)
    return ((q * s2) / 127.0).astype(F32)


def quantize_nf4(W, block: int = 64, dq_block: int = 256, codebook=None):
    """NF4 blockwise quantization of an fp32 weight W[d_out][d_in].

    Blocks are ``block`` consecutive elements of a row (row-major flatten of
    W, as the sketch reshapes to (-1, block)).  [R7]  Each block is scaled by
    its fp32 absmax and every element takes the index of the nearest level.
    Codes use the unquantized absmax; double quantization then compresses the
    constants.  [R4]

    Returns ``(codes uint8[d_out][d_in/2], absmax, absmax2)`` where, with
    double quantization (``dq_block > 0``), absmax is int8[n_blocks] and
    absmax2 fp32[ceil(n_blocks/dq_block)]; without it, absmax is
    fp32[n_blocks] and absmax2 is None.
    """
    W = np.asarray(W, dtype=F32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D [d_out][d_in]")
    n, k = W.shape
    if k % block or k % 2:
        raise ValueError("d_in must be a multiple of the block size and even")
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds a non-finite value")  # [R13]
    c = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=F32)
    blocks = W.reshape(-1, block)
    a = np.abs(blocks).max(axis=1).astype(F32)
    idx = nearest_level_index(blocks, a, c).reshape(n, k)
    codes = pack_nibbles(idx)
    if dq_block:
        q, s2 = double_quantize(a, dq_block)
        return codes, q, s2
    return codes, a, None


def nf4_block_scales(absmax, absmax2, dq_block: int) -> np.ndarray:
    """fp32 per-block scale actually used for dequantization."""
    if dq_block:
        return dq_absmax(absmax, absmax2, dq_block)
    return np.asarray(absmax, dtype=F32)


def dequant_nf4_bf16(codes, absmax, absmax2, block: int = 64, dq_block: int = 256,
                     codebook=None) -> np.ndarray:
    """W_bf16 bit patterns uint16[d_out][d_in].  [R9]

    Each element is the fp32 product of its level and its block's scale,
    rounded to bf16 (ties to even): the weight is brought back to BFloat16
    block by block, as the recipe's training stage describes."""
    c = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=F32)
    idx = unpack_nibbles(codes)
    n, k = idx.shape
    scale = nf4_block_scales(absmax, absmax2, dq_block)
    scale_e = np.repeat(scale, block).reshape(n, k)
    prod = (c[idx].astype(F32) * scale_e).astype(F32)
    return f32_to_bf16_bits(prod)


def dequant_nf4_rows(codes, absmax, absmax2, rows, block=64, dq_block=256):
    """W_bf16 (as float64) of selected rows only; for sampled checks at full size."""
    c = nf4_codebook()
    rows = np.asarray(rows, dtype=np.int64)
    k = codes.shape[1] * 2
    nbr = k // block
    idx = unpack_nibbles(codes[rows])
    bids = (rows[:, None] * nbr + np.arange(nbr)[None, :]).reshape(-1)
    sc = _dq_absmax_of_blocks(absmax, absmax2, bids, dq_block)
    sc = np.repeat(sc.reshape(len(rows), nbr), block, axis=1)
    return bf16_bits_to_f64(f32_to_bf16_bits((c[idx] * sc).astype(F32)))


def dequant_nf4_cols(codes, absmax, absmax2, cols, block=64, dq_block=256):
    """W_bf16 (as float64) of selected columns: returns [d_out][len(cols)]."""
    c = nf4_codebook()
    cols = np.asarray(cols, dtype=np.int64)
    n = codes.shape[0]
    k = codes.shape[1] * 2
    nbr = k // block
    byte = codes[:, (cols // 8) * 4 + cols % 4]
    nib = np.where((cols % 8)[None, :] < 4, byte & 0x0F, byte >> 4)
    bids = np.arange(n)[:, None] * nbr + (cols // block)[None, :]
    sc = _dq_absmax_of_blocks(absmax, absmax2, bids, dq_block)
    return bf16_bits_to_f64(f32_to_bf16_bits((c[nib] * sc).astype(F32)))


# ---------------------------------------------------------------------------
# NormalFloat-k with any block size  [LQ-LoRA abstract: per-matrix bit-width
# and block size; QLoRA "Innovation 1: 4-bit NormalFloat (NF4)" for the
# construction]
# ---------------------------------------------------------------------------


def nf_levels_f64(bits: int, inv_cdf=None) -> list[float]:
    """The 2^bits NormalFloat levels in float64, before rounding to fp32.

    The NF4 construction [R1] with 2^bits levels [R22]: with
    delta = 1 - 1/2^(bits+1) (the sketch's outermost quantile
    (2^bits - 1/2)/2^bits) and t = Phi^-1(delta), the positive levels are
    Phi^-1(1/2 + j (delta - 1/2)/P)/t for j = 1..P and the negative levels
    -Phi^-1(1/2 + j (delta - 1/2)/Q)/t for j = 1..Q, with P = 2^(bits-1)
    above and Q = 2^(bits-1) - 1 below an exact zero."""
    if inv_cdf is None:
        inv_cdf = NormalDist().inv_cdf
    delta = 1.0 - 1.0 / 2 ** (bits + 1)
    P, Q = 2 ** (bits - 1), 2 ** (bits - 1) - 1
    t = inv_cdf(delta)
    half = delta - 0.5
    pos = [inv_cdf(0.5 + j * half / P) / t for j in range(1, P + 1)]
    neg = [-inv_cdf(0.5 + j * half / Q) / t for j in range(1, Q + 1)]
    return sorted(neg + [0.0] + pos)


def nf_codebook(bits: int, inv_cdf=None) -> np.ndarray:
    """fp32[2^bits] NormalFloat levels, ascending; c[0] = -1, c[-1] = +1 and
    c[2^(bits-1) - 1] = 0."""
    return np.array(nf_levels_f64(bits, inv_cdf), dtype=F32)


def pack_bitplanes(idx: np.ndarray, bits: int) -> np.ndarray:
    """k-bit indices packed as bit planes along each row [R23]: every run of
    32 elements fills `bits` little-endian 32-bit words, word p holding bit p
    of element i in its bit i.  Rows hold a multiple of 32 elements; the
    result is uint8[rows][d_in * bits / 8]."""
    idx = np.asarray(idx, dtype=np.uint32)
    n = idx.shape[-1]
    assert n % 32 == 0, "rows must hold a multiple of 32 elements"
    runs = idx.reshape(idx.shape[:-1] + (n // 32, 32))
    shifts = np.arange(32, dtype=np.uint32)
    words = np.stack([(((runs >> p) & 1) << shifts).sum(axis=-1, dtype=np.uint64).astype(np.uint32)
                      for p in range(bits)], axis=-1)
    return words.reshape(idx.shape[:-1] + (n // 32 * bits,)).view(np.uint8)


def unpack_bitplanes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_bitplanes."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    words = codes.view(np.uint32)
    nw = words.shape[-1]
    w = words.reshape(words.shape[:-1] + (nw // bits, bits))
    shifts = np.arange(32, dtype=np.uint32)
    out = np.zeros(w.shape[:-1] + (32,), dtype=np.uint32)
    for p in range(bits):
        out |= ((w[..., p:p + 1] >> shifts) & 1) << p
    return out.reshape(words.shape[:-1] + (nw // bits * 32,)).astype(np.uint8)


def quantize_nf(W, bits: int, block: int, dq_block: int = 256, codebook=None):
    """NormalFloat-k blockwise quantization of an fp32 W[d_out][d_in].

    As quantize_nf4 (nearest level of w / absmax with an exact comparison,
    ties to the lower index, an all-zero block to the zero level, double
    quantization of the fp32 constants in groups of ``dq_block``), with
    2^bits levels and blocks of ``block`` consecutive elements of a row, and
    the codes packed as bit planes [R22, R23].  Returns
    ``(codes uint8[d_out][d_in*bits/8], absmax, absmax2)`` as for
    quantize_nf4."""
    W = np.asarray(W, dtype=F32)
    if W.ndim != 2:
        raise ValueError("W must be 2-D [d_out][d_in]")
    n, k = W.shape
    if k % block or k % 32:
        raise ValueError("d_in must be a multiple of the block size and of 32")
    if not np.all(np.isfinite(W)):
        raise ValueError("W holds a non-finite value")
    c = nf_codebook(bits) if codebook is None else np.asarray(codebook, dtype=F32)
    blocks = W.reshape(-1, block)
    a = np.abs(blocks).max(axis=1).astype(F32)
    idx = nearest_level_index(blocks, a, c).reshape(n, k)
    zero_idx = 2 ** (bits - 1) - 1
    idx.reshape(-1, block)[a == 0.0] = zero_idx
    codes = pack_bitplanes(idx, bits)
    if dq_block:
        q, s2 = double_quantize(a, dq_block)
        return codes, q, s2
    return codes, a, None


def dequant_nf_bf16(codes, absmax, absmax2, bits: int, block: int, dq_block: int = 256,
                    codebook=None) -> np.ndarray:
    """W_bf16 bit patterns: bf16(fl32(c[idx] * a_hat)) for NormalFloat-k."""
    c = nf_codebook(bits) if codebook is None else np.asarray(codebook, dtype=F32)
    idx = unpack_bitplanes(codes, bits)
    n, k = idx.shape
    scale = nf4_block_scales(absmax, absmax2, dq_block)
    scale_e = np.repeat(scale, block).reshape(n, k)
    return f32_to_bf16_bits((c[idx].astype(F32) * scale_e).astype(F32))


def nf_packed_nbytes(d_out: int, d_in: int, bits: int, block: int, dq_block: int = 256) -> int:
    n_el = d_out * d_in
    nb = n_el // block
    consts = nb + 4 * (-(-nb // dq_block)) if dq_block else 4 * nb
    return n_el * bits // 8 + consts


# ---------------------------------------------------------------------------
# Group-wise asymmetric INT4  [QA-LoRA abstract: group-wise operators, INT4]
# ---------------------------------------------------------------------------


def nearest_f16_of_rational(x) -> np.float16:
    """The fp16 value nearest to the rational ``x`` (a ``Fraction``), ties to
    the even significand.  ``float(x)`` rounds once to float64; its fp16
    image is within one fp16 step of the answer, so the nearest of that value
    and its two fp16 neighbours, compared in exact rationals, is the answer.
    Finite results only."""
    from fractions import Fraction
    h = np.float16(float(x))
    cands = [np.nextafter(h, np.float16(-np.inf)), h, np.nextafter(h, np.float16(np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - x)
        even = (int(np.array(c).view(np.uint16)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float16(best[1])


def int4_group_scale(lo, hi) -> np.ndarray:
    """fp16 bits of the group scale alpha = RN16((max - min) / 15).  [R16]

    The difference of two fp32 values is computed in float64 together with
    its rounding error (the two-sum error term).  Where the difference is
    exact, the float64 quotient by 15 rounded to fp16 is the exactly rounded
    value: the quotient is either an fp16 rounding boundary itself or lies
    further from every boundary than one float64 rounding can move it.
    Where the difference is not exact (operands of very different
    magnitudes), the rational value is rounded directly."""
    from fractions import Fraction
    lo = np.asarray(lo, dtype=F32).astype(F64)
    hi = np.asarray(hi, dtype=F32).astype(F64)
    d = hi - lo
    bv = d - hi
    err = (hi - (d - bv)) + (-lo - bv)          # hi - lo == d + err exactly
    out = (d / 15.0).astype(np.float16)
    for i in zip(*np.nonzero(err != 0.0)):
        exact = (Fraction(float(hi[i])) - Fraction(float(lo[i]))) / 15
        out[i] = nearest_f16_of_rational(exact)
    return out.view(np.uint16)


def int4_codes(w, alpha, beta) -> np.ndarray:
    """Codes q = clamp(round_half_even((w - beta) / alpha), 0, 15), and q = 0
    where alpha = 0.  [R16]

    ``w`` is fp32, ``alpha`` and ``beta`` fp16 values broadcast against it.
    The rounding is decided exactly: q counts the boundaries
    T_k = beta + (k + 1/2) alpha (k = 0..14) that w exceeds, plus the
    boundaries it equals for odd k (a tie k + 1/2 goes to the even
    neighbour: down for even k, up for odd k).  Each T_k is exact in float64
    (an fp16 value plus (2k + 1) times half an fp16 value), so every
    comparison is exact."""
    w = np.asarray(w, dtype=F32).astype(F64)
    alpha = np.asarray(alpha, dtype=F64)
    beta = np.asarray(beta, dtype=F64)
    q = np.zeros(np.broadcast(w, alpha, beta).shape, dtype=np.int64)
    for k in range(15):
        t = beta + (k + 0.5) * alpha
        q += w > t
        if k % 2 == 1:
            q += w == t
    q[np.broadcast_to(alpha == 0.0, q.shape)] = 0
    return q


def quantize_int4_group(W, group: int = 32):
    """Asymmetric min-max INT4 per (row, group of ``group`` consecutive d_in).
    [R16]

    beta  = RN16(min)                       (the group's additive zero point)
    alpha = RN16((max - min) / 15)          (exact quotient, rounded once)
    q     = 0 if alpha == 0 else clamp(round_half_even((w - beta) / alpha), 0, 15)

    with every rounding taken on the exact real value.  Returns
    ``(codes uint8[d_out][d_in/2], scale_bits uint16[d_out][d_in/group],
    zero_bits uint16[d_out][d_in/group])`` with fp16 bit patterns."""
    W = np.asarray(W, dtype=F32)
    n, k = W.shape
    if k % group or k % 2:
        raise ValueError("d_in must be a multiple of the group size and even")
    if not np.all(np.isfinite(W)) or np.any(np.abs(W) > 65504.0):
        raise ValueError("W holds a non-finite value or one outside fp16 range")
    g = W.reshape(n, k // group, group)
    lo = g.min(axis=2).astype(F32)
    hi = g.max(axis=2).astype(F32)
    beta_b = f32_to_f16_bits(lo)
    alpha_b = int4_group_scale(lo, hi)
    beta = f16_bits_to_f32(beta_b)[..., None]
    alpha = f16_bits_to_f32(alpha_b)[..., None]
    q = int4_codes(g, alpha, beta).astype(np.uint8).reshape(n, k)
    return pack_nibbles(q), alpha_b, beta_b


def dequant_int4_bf16(codes, scale_bits, zero_bits, group: int = 32) -> np.ndarray:
    """W_bf16 bit patterns: bf16(fl32(alpha * q + beta)); alpha * q is exact in
    fp32, so one rounding happens before the bf16 rounding."""
    q = unpack_nibbles(codes).astype(F32)
    alpha = np.repeat(f16_bits_to_f32(scale_bits), group, axis=1)
    beta = np.repeat(f16_bits_to_f32(zero_bits), group, axis=1)
    return f32_to_bf16_bits((alpha * q + beta).astype(F32))


# ---------------------------------------------------------------------------
# Forward / backward of the adapted layer  [QLoRA, "Background: how LoRA
# works", "The QLoRA recipe" stage 3, "The same idea in code"; QA-LoRA]
# ---------------------------------------------------------------------------


def pool_sum(x: np.ndarray, pool: int) -> np.ndarray:
    """Sum over each run of ``pool`` consecutive input features.  [R17]"""
    x = np.asarray(x, dtype=F64)
    if pool == 1:
        return x
    m, k = x.shape
    return x.reshape(m, k // pool, pool).sum(axis=2)


def lora_forward(Wd, x, A, B, s, pool: int = 1):
    """y = x W^T + s (P A^T) B^T with P = x (pool = 1) or the group sums of x.

    All float64.  ``Wd`` is the dequantized weight [d_out][d_in] (float64
    values of the bf16 weights), ``x`` [M][d_in], ``A`` [r][d_in/pool],
    ``B`` [d_out][r].  Returns (y [M][d_out], u [M][r]).  [R11, R19]"""
    x = np.asarray(x, dtype=F64)
    u = pool_sum(x, pool) @ np.asarray(A, dtype=F64).T
    y = x @ np.asarray(Wd, dtype=F64).T + s * (u @ np.asarray(B, dtype=F64).T)
    return y, u


def lora_backward(Wd, x, A, B, s, dy, pool: int = 1, u=None):
    """Gradients of <dy, y> for the frozen-base layer; W receives none.

    du = s dy B ; dB = s dy^T u ; dA = du^T P ; dX = dy W + expand(du A)
    where expand repeats each pooled column ``pool`` times.
    Returns (dX [M][d_in], dA [r][d_in/pool], dB [d_out][r], du [M][r])."""
    x = np.asarray(x, dtype=F64)
    dy = np.asarray(dy, dtype=F64)
    A = np.asarray(A, dtype=F64)
    B = np.asarray(B, dtype=F64)
    P = pool_sum(x, pool)
    if u is None:
        u = P @ A.T
    du = s * (dy @ B)
    dB = s * (dy.T @ u)
    dA = du.T @ P
    g = du @ A
    if pool > 1:
        g = np.repeat(g, pool, axis=1)
    dX = dy @ np.asarray(Wd, dtype=F64) + g
    return dX, dA, dB, du


def qa_merge_zero(zero_bits, A, B, s) -> np.ndarray:
    """QA-LoRA merge: fold the pooled adapter into the per-group zero point.

    With sum pooling, s * (B A)[n, g] is added to every weight of group g in
    row n, i.e. to that group's additive zero: beta' = beta + s * B A (float64).
    [QA-LoRA abstract, point (ii); R17]"""
    beta = f16_bits_to_f32(zero_bits).astype(F64)
    return beta + s * (np.asarray(B, dtype=F64) @ np.asarray(A, dtype=F64))


def qa_merge_zero_f16(zero_bits, A_bits, B_bits, s) -> np.ndarray:
    """fp16 bits of the merged zero points RN16(beta + s * sum_j B[n][j] A[j][g]),
    the exact sum rounded once (ties to even).  [QA-LoRA abstract, point
    (ii); R17]

    ``A_bits`` [r][G] and ``B_bits`` [d_out][r] are bf16 bit patterns and s a
    float32.  Every term s * B * A is exact in float64 (24 + 8 + 8
    significant bits); math.fsum returns the correctly rounded float64 of the
    exact sum, whose fp16 image is within one fp16 step of the answer, and the
    sign of the exact sum minus an fp16 rounding boundary (another fsum, with
    the boundary as one more exact term) decides between the neighbours.
    Slow (pure Python per entry): for test-sized layers."""
    beta = f16_bits_to_f32(zero_bits).astype(F64)
    A = bf16_bits_to_f64(A_bits)
    B = bf16_bits_to_f64(B_bits)
    s = float(np.float32(s))
    n_rows, G = beta.shape
    r = A.shape[0]
    out = np.empty((n_rows, G), dtype=np.uint16)
    inf16 = np.float16(np.inf)
    for n in range(n_rows):
        for g in range(G):
            terms = [float(beta[n, g])] + [s * B[n, j] * A[j, g] for j in range(r)]
            h = np.float16(math.fsum(terms))
            # step down while the exact sum lies below the boundary under h,
            # up while it lies above the boundary over h (ties: even bits)
            for _ in range(2):
                lo = np.nextafter(h, -inf16)
                m = (float(lo) + float(h)) / 2.0
                d = math.fsum(terms + [-m])
                if d < 0 or (d == 0 and int(np.array(h).view(np.uint16)) & 1):
                    h = lo
            for _ in range(2):
                hi = np.nextafter(h, inf16)
                m = (float(h) + float(hi)) / 2.0
                d = math.fsum(terms + [-m])
                if d > 0 or (d == 0 and int(np.array(h).view(np.uint16)) & 1):
                    h = hi
            out[n, g] = np.array(h).view(np.uint16)
    return out


def int4_scale_zero_grads(codes, x, dy, group: int = 32):
    """Gradients of <dy, y> with respect to the INT4 group scales and zero
    points, for y = x W^T with W[n][k] = alpha[n][g] q[n][k] + beta[n][g]
    (g = k / group): the trainable-quantization-parameter reading of LoQA's
    operator [LoQA abstract: the scale and the zero point are fine-tuned;
    R24].  The rounding of W to bf16 is passed straight through.  In float64:

        dW[n][k]     = sum_m dy[m][n] x[m][k]
        dalpha[n][g] = sum_{k in g} q[n][k] dW[n][k]
        dbeta[n][g]  = sum_{k in g} dW[n][k]

    Returns (dalpha, dbeta), each [d_out][d_in / group]."""
    q = unpack_nibbles(codes).astype(F64)
    dW = np.asarray(dy, dtype=F64).T @ np.asarray(x, dtype=F64)
    n, k = dW.shape
    dalpha = (q * dW).reshape(n, k // group, group).sum(axis=2)
    dbeta = dW.reshape(n, k // group, group).sum(axis=2)
    return dalpha, dbeta


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=F64)
    ref = np.asarray(ref, dtype=F64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


# ---------------------------------------------------------------------------
# Storage accounting  [QLoRA, "Innovation 2: Double Quantization",
# "The memory wall", "The QLoRA recipe" stage 1]
# ---------------------------------------------------------------------------


def nf4_packed_nbytes(d_out: int, d_in: int, block: int = 64, dq_block: int = 256) -> dict:
    n_el = d_out * d_in
    nb = n_el // block
    out = {"codes": n_el // 2}
    if dq_block:
        out["absmax"] = nb
        out["absmax2"] = 4 * (-(-nb // dq_block))
    else:
        out["absmax"] = 4 * nb
        out["absmax2"] = 0
    out["total"] = out["codes"] + out["absmax"] + out["absmax2"]
    return out


def constant_bits_per_param(block: int = 64, dq_block: int = 256) -> float:
    """Bits per weight spent on scaling constants: 32/block without double
    quantization, 8/block + 32/(block*dq_block) with it."""
    if not dq_block:
        return 32.0 / block
    return 8.0 / block + 32.0 / (block * dq_block)


# ---------------------------------------------------------------------------
# Low-rank plus quantized decomposition  [LQ-LoRA, abstract: each matrix is
# split iteratively into a quantized part and a high-precision low-rank part]
# ---------------------------------------------------------------------------


def thin_qr_pos(X):
    """Thin QR of a tall matrix X (rows >= columns, full column rank) with a
    positive diagonal in R: the unique factorisation X = Q R with
    Q^T Q = I.  [R27]"""
    X = np.asarray(X, dtype=F64)
    q, rr = np.linalg.qr(X, mode="reduced")
    d = np.sign(np.diag(rr))
    d[d == 0] = 1.0
    return q * d, rr * d[:, None]


def lowrank_part(R, omega_t, power: int):
    """Rank-r part of R [N][K] by subspace iteration from the start
    V0 = omega_t^T (omega_t: r x K, drawn by the caller):
    U = orth(R V0); `power` times V = orth(R^T U), U = orth(R V); then the
    projection L = U (U^T R).  Returns U [N][r] and C = U^T R [r][K].  [R27]"""
    R = np.asarray(R, dtype=F64)
    om = np.asarray(omega_t, dtype=F64)
    U, _ = thin_qr_pos(R @ om.T)
    for _ in range(power):
        V, _ = thin_qr_pos(R.T @ U)
        U, _ = thin_qr_pos(R @ V)
    return U, U.T @ R


def lq_decompose(W, r: int, iters: int, power: int, omega_t, block: int = 64,
                 dq_block: int = 256):
    """W ~ Q + L with Q an NF4 weight and L = U C of rank r.  [LQ-LoRA,
    abstract; R26]

    L starts at zero.  Each iteration quantizes W - L (rounded to fp32, the
    quantizer's input format), takes the residual R = W - W_bf16(Q) against
    the weight the layer computes with, and replaces L by the rank-r part of
    R.  Returns (codes, absmax, absmax2, U, C, errs) where errs[t] is
    ||W - W_bf16(Q_t) - L_t||_F / ||W||_F after iteration t."""
    W = np.asarray(W, dtype=F64)
    n, k = W.shape
    U = np.zeros((n, r), dtype=F64)
    C = np.zeros((r, k), dtype=F64)
    wn = float(np.linalg.norm(W))
    errs = []
    for _ in range(iters):
        D = (W - U @ C).astype(F32)
        codes, am, am2 = quantize_nf4(D, block, dq_block)
        Wq = bf16_bits_to_f64(dequant_nf4_bf16(codes, am, am2, block, dq_block))
        R = W - Wq
        if r > 0:
            U, C = lowrank_part(R, omega_t, power)
        errs.append(float(np.linalg.norm(R - U @ C)) / (wn if wn > 0 else 1.0))
    return codes, am, am2, U, C, errs
