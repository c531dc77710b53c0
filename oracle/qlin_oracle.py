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
* quantize_int4_group ..... pinned (range/bounds, min->0, max->15, error
                             bound, Gaussian error level)
* dequant_int4_bf16 ....... pinned (error bound vs the input)
* lora_forward / backward . pinned (finite differences, B=0 / W=0 / s=0
                             reductions to plain products, M=1)
* qa_merge_zero ........... pinned (merged == unmerged forward)
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


#: fp32 constant multiplying a group's s2 to give the 8-bit grid step.  [R5]
DQ_INV127 = F32(1.0 / 127.0)


def dq_absmax(q: np.ndarray, s2: np.ndarray, dq_block: int = 256) -> np.ndarray:
    """fp32 first-level constants reconstructed from their 8-bit codes.  [R5]

    step_g = fl32(s2_g * fl32(1/127)); a_hat_b = fl32(q_b * step_g)."""
    q = np.asarray(q, dtype=np.int8).astype(F32)
    s2 = np.asarray(s2, dtype=F32)
    step = (s2 * DQ_INV127).astype(F32)
    step_b = np.repeat(step, dq_block)[: q.size]
    return (q * step_b).astype(F32)


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
    if dq_block:
        g = bids // dq_block
        step = (np.asarray(absmax2, F32)[g] * DQ_INV127).astype(F32)
        sc = (np.asarray(absmax, np.int8)[bids].astype(F32) * step).astype(F32)
    else:
        sc = np.asarray(absmax, F32)[bids]
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
    if dq_block:
        step = (np.asarray(absmax2, F32)[bids // dq_block] * DQ_INV127).astype(F32)
        sc = (np.asarray(absmax, np.int8)[bids].astype(F32) * step).astype(F32)
    else:
        sc = np.asarray(absmax, F32)[bids]
    return bf16_bits_to_f64(f32_to_bf16_bits((c[nib] * sc).astype(F32)))


# ---------------------------------------------------------------------------
# Group-wise asymmetric INT4  [QA-LoRA abstract: group-wise operators, INT4]
# ---------------------------------------------------------------------------


def quantize_int4_group(W, group: int = 32):
    """Asymmetric min-max INT4 per (row, group of ``group`` consecutive d_in).
    [R16]

    beta  = fp16(min)                      (the group's additive zero point)
    alpha = fp16(fl32(fl32(max - min) / 15))
    q     = 0 if alpha == 0 else clamp(round_half_even(fl32(fl32(w - beta) / alpha)), 0, 15)

    Returns ``(codes uint8[d_out][d_in/2], scale_bits uint16[d_out][d_in/group],
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
    alpha_b = f32_to_f16_bits(((hi - lo).astype(F32) / F32(15.0)).astype(F32))
    beta = f16_bits_to_f32(beta_b)[..., None]
    alpha = f16_bits_to_f32(alpha_b)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = ((g - beta).astype(F32) / alpha).astype(F32)
        q = np.clip(np.rint(r), 0, 15)
    q = np.where(alpha == 0, 0, q).astype(np.uint8).reshape(n, k)
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
