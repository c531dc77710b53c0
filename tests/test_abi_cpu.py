"""C ABI checks that need no GPU: the library loads, exports every symbol
include/qlin.h declares, computes the NF4 levels on the host bit-identically
to the oracle, sizes workspaces, and rejects bad arguments before enqueuing
anything."""

import ctypes
import os
import re

import numpy as np
import pytest

from quantized_base_rank_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libqlin.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in _declared():
        assert hasattr(L, name), name


def test_codebook_bit_identical_to_oracle(oracle):
    from quantized_base_rank_amd import qlin_nf4_codebook
    got = qlin_nf4_codebook()
    ref = oracle.nf4_codebook()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nf_codebook_bit_identical_to_oracle(oracle, bits):
    from quantized_base_rank_amd import qlin_nf_codebook
    got = qlin_nf_codebook(bits)
    assert np.array_equal(got.view(np.uint32), oracle.nf_codebook(bits).view(np.uint32))


def test_status_strings():
    L = _lib.lib()
    for st in range(8):
        assert L.qlin_status_string(st)
    assert L.qlin_status_string(99) == b"unknown status"


def _qw(fmt=1, block=64, dq=256, d_out=4096, d_in=4096, aligned=True):
    p = 0x1000 if aligned else 0x1004
    return _lib.QWeightStruct(fmt, block, dq, 0, d_out, d_in, p, p, p, p, p)


def test_workspace_bytes_host_only():
    L = _lib.lib()
    for M in (1, 16, 4096):
        n = L.qlin_workspace_bytes(ctypes.byref(_qw()), M, 16, 1)
        assert n > 0 and n % 256 == 0
    assert L.qlin_workspace_bytes(ctypes.byref(_qw()), 0, 16, 1) == 0
    assert L.qlin_workspace_bytes(ctypes.byref(_qw()), 16, -1, 1) == 0
    assert L.qlin_workspace_bytes(ctypes.byref(_qw()), 16, 0, 1) > 0   # adapter-free forward
    assert L.qlin_workspace_bytes(ctypes.byref(_qw()), 16, 129, 1) == 0
    # pooled adapter needs the INT4 group format with pool == group
    assert L.qlin_workspace_bytes(ctypes.byref(_qw()), 16, 16, 32) == 0
    q4 = _qw(fmt=2, block=32, dq=0, d_out=4096, d_in=11008)
    assert L.qlin_workspace_bytes(ctypes.byref(q4), 2048, 64, 32) > 0


def test_argument_errors_return_before_any_launch():
    L = _lib.lib()
    ok = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1004)
    ws = ctypes.c_void_p(0x2000)
    big = 1 << 40
    qw = _qw()
    # fwd: null input, misaligned input, bad rank, bad shape, bad pool, no workspace
    assert L.qlin_fwd(ctypes.byref(qw), None, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 1
    assert L.qlin_fwd(ctypes.byref(qw), bad, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 3
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, ok, ok, -1, 2.0, 1, ok, None, ws, big, None) == 2
    # r = 0 (no adapter) returns no u, and still needs x and y
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, None, None, 0, 2.0, 1, ok, ok, ws, big, None) == 2
    assert L.qlin_fwd(ctypes.byref(qw), None, 16, None, None, 0, 2.0, 1, ok, None, ws, big,
                      None) == 1
    assert L.qlin_bwd(ctypes.byref(qw), ok, 16, ok, ok, 0, 2.0, 1, ok, None, ok, ok, ok, ws,
                      big, None) == 2
    assert L.qlin_fwd(ctypes.byref(qw), ok, 0, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 2
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, ok, ok, 16, float("nan"), 1, ok, None, ws, big,
                      None) == 2
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, ok, ok, 16, 2.0, 32, ok, None, ws, big, None) == 5
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, ok, ok, 16, 2.0, 1, ok, None, None, big, None) == 6
    assert L.qlin_fwd(ctypes.byref(qw), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, 16, None) == 6
    assert L.qlin_fwd(None, ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 1
    # descriptor errors
    assert L.qlin_fwd(ctypes.byref(_qw(d_in=100)), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big,
                      None) == 2
    assert L.qlin_fwd(ctypes.byref(_qw(d_out=100)), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big,
                      None) == 2
    assert L.qlin_fwd(ctypes.byref(_qw(block=32)), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big,
                      None) == 5
    assert L.qlin_fwd(ctypes.byref(_qw(fmt=7)), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big,
                      None) == 5
    # the NormalFloat-k workspace holds the transcoded weight as well
    qnf = _lib.QWeightStruct(3, 64, 256, 3, 4096, 4096, 0x1000, 0x1000, 0x1000, 0, 0)
    assert L.qlin_workspace_bytes(ctypes.byref(qnf), 16, 16, 1) >= \
        L.qlin_workspace_bytes(ctypes.byref(_qw()), 16, 16, 1) + 4096 * 4096 * 5 // 8
    assert L.qlin_fwd(ctypes.byref(_qw(aligned=False)), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws,
                      big, None) == 3
    # bwd: missing gradient outputs
    assert L.qlin_bwd(ctypes.byref(qw), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ok, None, ok, ws,
                      big, None) == 1
    assert L.qlin_bwd(ctypes.byref(qw), ok, 16, ok, ok, 16, 2.0, 1, None, None, ok, ok, ok, ws,
                      big, None) == 1
    # quantizers
    assert L.qlin_quantize_nf4(None, 4, 64, 64, 256, ok, ok, ok, None) == 1
    assert L.qlin_quantize_nf4(ok, 4, 64, 32, 256, ok, ok, ok, None) == 5
    assert L.qlin_quantize_nf4(ok, 4, 96, 64, 256, ok, ok, ok, None) == 2
    assert L.qlin_quantize_nf4(ok, 4, 64, 64, 128, ok, ok, ok, None) == 5
    assert L.qlin_quantize_nf4(ok, 4, 64, 64, 256, ok, ok, None, None) == 1
    assert L.qlin_quantize_nf4(bad, 16, 64, 64, 256, ok, ok, ok, None) == 3
    assert L.qlin_quantize_int4_group(ok, 4, 64, 64, ok, ok, ok, None) == 5
    assert L.qlin_quantize_int4_group(ok, 4, 48, 32, ok, ok, ok, None) == 2
    assert L.qlin_quantize_int4_group(ok, 4, 64, 32, ok, None, ok, None) == 1
    # the quantizers accept exactly the shapes the layer accepts: d_out a
    # multiple of 16, d_in a multiple of 64 (also for INT4 groups of 32)
    assert L.qlin_quantize_nf4(ok, 4, 64, 64, 256, ok, ok, ok, None) == 2
    assert L.qlin_quantize_int4_group(ok, 16, 96, 32, ok, ok, ok, None) == 2
    assert L.qlin_quantize_int4_group(ok, 8, 64, 32, ok, ok, ok, None) == 2
    q96 = _qw(fmt=2, block=32, dq=0, d_out=16, d_in=96)
    assert L.qlin_fwd(ctypes.byref(q96), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big,
                      None) == 2
    # QA-LoRA merge: INT4 weights only, rank 1..128, outputs aligned
    q4 = _qw(fmt=2, block=32, dq=0, d_out=64, d_in=1024)
    assert L.qlin_qa_merge(ctypes.byref(qw), ok, ok, 16, 2.0, ok, None) == 5
    assert L.qlin_qa_merge(ctypes.byref(q4), ok, ok, 0, 2.0, ok, None) == 2
    assert L.qlin_qa_merge(ctypes.byref(q4), ok, ok, 16, float("inf"), ok, None) == 2
    assert L.qlin_qa_merge(ctypes.byref(q4), ok, None, 16, 2.0, ok, None) == 1
    assert L.qlin_qa_merge(ctypes.byref(q4), ok, ok, 16, 2.0, bad, None) == 3
    # NormalFloat-k quantizer and codebook
    out16 = (ctypes.c_float * 16)()
    assert L.qlin_nf_codebook(5, out16) == 5 and L.qlin_nf_codebook(3, None) == 1
    assert L.qlin_quantize_nf(ok, 16, 256, 1, 64, 256, ok, ok, ok, None) == 5
    assert L.qlin_quantize_nf(ok, 16, 256, 3, 48, 256, ok, ok, ok, None) == 5
    assert L.qlin_quantize_nf(ok, 16, 256, 3, 64, 128, ok, ok, ok, None) == 5
    assert L.qlin_quantize_nf(ok, 16, 384, 3, 256, 256, ok, ok, ok, None) == 2
    assert L.qlin_quantize_nf(ok, 8, 256, 3, 64, 256, ok, ok, ok, None) == 2
    assert L.qlin_quantize_nf(ok, 16, 256, 3, 64, 256, ok, ok, None, None) == 1
    assert L.qlin_quantize_nf(bad, 16, 256, 3, 64, 256, ok, ok, ok, None) == 3
    qn = _lib.QWeightStruct(3, 64, 256, 5, 64, 256, 0x1000, 0x1000, 0x1000, 0, 0)
    assert L.qlin_fwd(ctypes.byref(qn), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 5
    qn4 = _lib.QWeightStruct(1, 64, 256, 3, 64, 256, 0x1000, 0x1000, 0x1000, 0, 0)
    assert L.qlin_fwd(ctypes.byref(qn4), ok, 16, ok, ok, 16, 2.0, 1, ok, None, ws, big, None) == 5
    # INT4 scale / zero gradients
    assert L.qlin_int4_scale_zero_grad(ctypes.byref(qw), ok, 16, ok, ok, ok, None) == 5
    assert L.qlin_int4_scale_zero_grad(ctypes.byref(q4), ok, 0, ok, ok, ok, None) == 2
    assert L.qlin_int4_scale_zero_grad(ctypes.byref(q4), ok, 16, None, ok, ok, None) == 1
    assert L.qlin_int4_scale_zero_grad(ctypes.byref(q4), ok, 16, ok, bad, ok, None) == 3
    # profiling hook: host only
    assert L.qlin_profile_next_launch(b"k_fwd_gemm", None, None) == 1
    assert L.qlin_profile_next_launch(b"k" * 64, ok, ok) == 2
    assert L.qlin_profile_next_launch(None, None, None) == 0
    # dequant helper
    assert L.qlin_dequant_bf16(ctypes.byref(qw), None, None) == 1
    assert L.qlin_nf4_codebook(None) == 1


def test_binding_raises_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libqlin.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_lq_workspace_bytes_host_only():
    """The decomposition's workspace query is host arithmetic: every rank,
    including 0 (plain NF4), gets a size that holds the fp32 residual."""
    L = ctypes.CDLL(_lib.LIB_PATH)
    f = L.qlin_lq_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    for r in (0, 1, 8, 64, 128):
        n = f(512, 1024, r)
        assert n >= 512 * 1024 * 4 + r * (512 + 1024) * 4
    assert f(512, 1024, 129) == 0 and f(0, 1024, 8) == 0
