"""GPU parity at the full sizes of the target workloads, through the C ABI.

The oracle is too slow to run whole 4096-token layers element by element, so
these tests compare exactly what it can afford, at the real shapes and in the
launch configuration the benchmark uses:

* packed weights: the oracle quantizes the same fp32 weight itself, in bands
  of rows that hold whole double-quantization groups, and every packed byte
  and the whole decoded bf16 weight must match bit for bit;
* y on a sample of output features and dX on a sample of input features, for
  every token (the oracle's dequantized rows / columns of its own packed
  weight); u, du-derived dA and dB in full;
* every float output also passes the per-row and per-tile bounds of
  tests/parity.py.

Workloads: LLaMA-7B q_proj 4096x4096 (M = 1 and 16), up_proj 11008x4096
(M = 4096, r = 64), the QA-LoRA INT4 layer 4096x11008 (M = 2048, pooled
r = 64, and M = 16), and LLaMA-2-70B down_proj 8192x28672 (M = 4096, r = 64,
and M = 1, 16 through the weight-streaming kernels with K split across
workgroups).
"""

from __future__ import annotations

import numpy as np
import pytest

from tests import parity
from tests.gpu_util import bf16_host_bits, f16_bits, host, to_dev_bf16, to_dev_f32, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_base_rank_amd as qb
    qb._lib.lib()
    return qb


def _band_rows(wl):
    """Rows per oracle band: a multiple of whole double-quantization groups
    (NF4) and at most ~16 M weights."""
    if wl.fmt != "nf4":
        return max(16, (1 << 24) // wl.d_in // 16 * 16)
    nbr = wl.d_in // wl.block
    step = wl.dq_block // np.gcd(nbr, wl.dq_block)      # rows per whole number of groups
    rows = max(step, (1 << 24) // wl.d_in // step * step)
    return rows


def _oracle_bands(oracle, wl, W):
    """Yield (row0, codes, constants...) of the oracle's own quantization of
    W, one band of rows at a time (bands hold whole DQ groups, so each band
    quantizes exactly as the full matrix does)."""
    rows = _band_rows(wl)
    for r0 in range(0, wl.d_out, rows):
        band = W[r0:r0 + rows]
        if wl.fmt == "nf4":
            yield (r0,) + tuple(oracle.quantize_nf4(band, wl.block, wl.dq_block))
        else:
            yield (r0,) + tuple(oracle.quantize_int4_group(band, wl.block))


def _sample(n, k, rng):
    """k sorted distinct indices in [0, n), always including both ends."""
    idx = set(rng.choice(n, size=min(n, k), replace=False).tolist())
    idx.update([0, n - 1, n - 16 if n > 16 else 0])
    return np.array(sorted(idx))


def _layer_full(qb, oracle, wl, n_cols=192, k_cols=192, seed=0):
    from quantized_base_rank_amd.inputs import make_inputs
    inp = make_inputs(wl, seed=seed)
    r, s, pool = wl.r, wl.s, wl.pool
    if wl.fmt == "nf4":
        qw = qb.qlin_quantize_nf4(to_dev_f32(inp.W), wl.block, wl.dq_block)
    else:
        qw = qb.qlin_quantize_int4_group(to_dev_f32(inp.W), wl.block)
    x, A, B, dy = (to_dev_bf16(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    y, u = qb.qlin_fwd(qw, x, A, B, r, s, pool)
    dx, dA, dB = qb.qlin_bwd(qw, x, A, B, r, s, dy, pool, u_saved=u)
    got = {"y": oracle.bf16_bits_to_f64(bf16_host_bits(y)), "u": host(u).astype(np.float64),
           "dX": oracle.bf16_bits_to_f64(bf16_host_bits(dx)),
           "dA": oracle.bf16_bits_to_f64(bf16_host_bits(dA)),
           "dB": oracle.bf16_bits_to_f64(bf16_host_bits(dB))}
    del x, A, B, dy, y, u, dx, dA, dB, qw

    rng = np.random.default_rng(seed + 100)
    ncols = _sample(wl.d_out, n_cols, rng)
    kcols = _sample(wl.d_in, k_cols, rng)
    w_rows = np.zeros((ncols.size, wl.d_in))       # W_bf16[ncols, :]
    w_cols = np.zeros((wl.d_out, kcols.size))      # W_bf16[:, kcols]
    for r0, *packed in _oracle_bands(oracle, wl, inp.W):
        nb = packed[0].shape[0]
        if wl.fmt == "nf4":
            codes, am, am2 = packed
            sel = ncols[(ncols >= r0) & (ncols < r0 + nb)] - r0
            if sel.size:
                w_rows[np.searchsorted(ncols, sel + r0)] = oracle.dequant_nf4_rows(
                    codes, am, am2, sel, wl.block, wl.dq_block)
            w_cols[r0:r0 + nb] = oracle.dequant_nf4_cols(codes, am, am2, kcols, wl.block,
                                                         wl.dq_block)
        else:
            full = oracle.bf16_bits_to_f64(oracle.dequant_int4_bf16(*packed, wl.block))
            sel = ncols[(ncols >= r0) & (ncols < r0 + nb)]
            w_rows[np.searchsorted(ncols, sel)] = full[sel - r0]
            w_cols[r0:r0 + nb] = full[:, kcols]

    xf = oracle.bf16_bits_to_f64(inp.x)
    Af = oracle.bf16_bits_to_f64(inp.A)
    Bf = oracle.bf16_bits_to_f64(inp.B)
    dyf = oracle.bf16_bits_to_f64(inp.dy)
    P = oracle.pool_sum(xf, pool)
    u_ref = P @ Af.T
    du = s * (dyf @ Bf)
    ref = {"y": xf @ w_rows.T + s * (u_ref @ Bf[ncols].T), "u": u_ref,
           "dX": dyf @ w_cols + du @ Af[:, kcols // pool],
           "dA": du.T @ P, "dB": s * (dyf.T @ u_ref)}
    got["y"] = got["y"][:, ncols]
    got["dX"] = got["dX"][:, kcols]
    return parity.check({k: (got[k], ref[k]) for k in ref}, fmts={"u": "f32"})


FULL = {
    "q_proj_M1": ("q_proj", 1),
    "q_proj_M16": ("q_proj", 16),
    "up_proj_M4096": ("up_proj", None),
    "qa_int4_M2048": ("qa_int4", None),
    "qa_int4_M16": ("qa_int4", 16),
    "down_proj70b_M4096": ("down_proj70b", None),
    "down_proj70b_M16": ("down_proj70b", 16),
    "down_proj70b_M1": ("down_proj70b", 1),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", list(FULL))
def test_layer_full_size(qb, oracle, case):
    from quantized_base_rank_amd.inputs import WORKLOADS
    name, M = FULL[case]
    wl = WORKLOADS[name]
    if M is not None:
        wl = wl.with_m(M)
    print(f"[full-size] {case}: {wl}", flush=True)
    errs = _layer_full(qb, oracle, wl)
    print(f"[full-size] {case}: {errs}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["down_proj70b", "up_proj"])
def test_nf4_pack_and_decode_bit_exact_full(qb, oracle, name):
    """Every packed byte, 8-bit constant and second-level constant, and the
    whole decoded bf16 weight, at the full layer shape (the 70B down_proj
    decode covers 235 M lookup-table entries)."""
    from quantized_base_rank_amd.inputs import WORKLOADS, make_weight
    wl = WORKLOADS[name]
    W = make_weight(wl.d_out, wl.d_in, seed=3)
    qw = qb.qlin_quantize_nf4(to_dev_f32(W), wl.block, wl.dq_block)
    codes_g, am_g, am2_g = u8(qw.codes), host(qw.absmax).view(np.int8), host(qw.absmax2)
    wdec = qb.qlin_dequant_bf16(qw)
    nbr = wl.d_in // wl.block
    for r0, codes, am, am2 in _oracle_bands(oracle, wl, W):
        nb = codes.shape[0]
        b0 = r0 * nbr
        assert np.array_equal(codes_g[r0:r0 + nb], codes), f"codes, band at row {r0}"
        assert np.array_equal(am_g[b0:b0 + am.size], am), f"absmax, band at row {r0}"
        g0 = b0 // wl.dq_block
        assert np.array_equal(am2_g[g0:g0 + am2.size].view(np.uint32), am2.view(np.uint32))
        ref = oracle.dequant_nf4_bf16(codes, am, am2, wl.block, wl.dq_block)
        got = bf16_host_bits(wdec[r0:r0 + nb])
        assert np.array_equal(got, ref), f"decoded weight, band at row {r0}"


@pytest.mark.timeout(900)
def test_int4_pack_and_decode_bit_exact_full(qb, oracle):
    from quantized_base_rank_amd.inputs import WORKLOADS, make_weight
    wl = WORKLOADS["qa_int4"]
    W = make_weight(wl.d_out, wl.d_in, seed=4)
    qw = qb.qlin_quantize_int4_group(to_dev_f32(W), wl.block)
    codes_g, sc_g, zp_g = u8(qw.codes), f16_bits(qw.scale), f16_bits(qw.zero)
    wdec = qb.qlin_dequant_bf16(qw)
    for r0, codes, sc, zp in _oracle_bands(oracle, wl, W):
        nb = codes.shape[0]
        assert np.array_equal(codes_g[r0:r0 + nb], codes), f"codes, band at row {r0}"
        assert np.array_equal(sc_g[r0:r0 + nb], sc) and np.array_equal(zp_g[r0:r0 + nb], zp)
        ref = oracle.dequant_int4_bf16(codes, sc, zp, wl.block)
        assert np.array_equal(bf16_host_bits(wdec[r0:r0 + nb]), ref)


@pytest.mark.timeout(900)
def test_qa_merge_full_size_sampled_rows(qb, oracle):
    """The QA-LoRA merge at the full 4096 x 11008 shape (r = 64): merged fp16
    zero points bit-exact to the oracle's exactly rounded ones on a sample of
    rows, and the adapter-free forward of the merged weight at M = 16 within
    the spec bound plus the merge's own float64 deviation."""
    from quantized_base_rank_amd.inputs import WORKLOADS, make_inputs
    wl = WORKLOADS["qa_int4"].with_m(16)
    inp = make_inputs(wl, seed=5)
    qw = qb.qlin_quantize_int4_group(to_dev_f32(inp.W), 32)
    A, B = to_dev_bf16(inp.A), to_dev_bf16(inp.B)
    merged = qb.qlin_qa_merge(qw, A, B, wl.r, wl.s)
    zg = f16_bits(merged.zero)
    rows = _sample(wl.d_out, 48, np.random.default_rng(6))
    _, _, zp = oracle.quantize_int4_group(inp.W[rows], 32)
    want = oracle.qa_merge_zero_f16(zp, inp.A, inp.B[rows], wl.s)
    assert np.array_equal(zg[rows], want)
