"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic work figures its roofline divides by, and the memory-footprint
context it prints against the pages' own storage accounting."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _golden(item):
    with open(os.path.join(ROOT, "tests", "golden", "qlora_page_figures.json")) as f:
        items = {it["id"]: it for it in json.load(f)["items"]}
    return items[item]["value"]


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_kernel_work_is_the_closed_form_count():
    import bench
    from quantized_base_rank_amd.inputs import WORKLOADS
    wl = WORKLOADS["down_proj70b"]
    M, N, K, r = 4096, 8192, 28672, 64
    assert (wl.M, wl.d_out, wl.d_in, wl.r) == (M, N, K, r)
    # dX = dY W (2 M N K) plus the appended du A term (2 M K r)
    assert bench.kernel_work(wl, "k_dx_gemm") == (2 * M * N * K + 2 * M * K * r, "flop")
    assert bench.kernel_work(wl, "k_dx_gemm")[0] == 1_939_177_734_144
    # y = x W^T (2 M N K) plus s u B^T (2 M N r)
    assert bench.kernel_work(wl, "k_fwd_gemm") == (2 * M * N * K + 2 * M * N * r, "flop")
    # packed NF4-64 + DQ-256 weight: 4-bit codes, one byte per 64-block, one
    # fp32 per 256 blocks
    nb = N * K // 64
    packed = N * K // 2 + nb + 4 * (-(-nb // 256))
    assert wl.packed_weight_bytes() == packed == 121_167_872
    m = 16
    w16 = wl.with_m(m)
    # dX pass: W, dY, A, du, dX, and (unpooled adapter) x and dA formed per panel
    assert bench.kernel_work(w16, "k_gemv_dx_stream") == (
        packed + 2 * m * N + 2 * r * K + 4 * m * r + 2 * m * K + 2 * m * K + 2 * r * K, "byte")
    assert bench.kernel_work(w16, "k_gemv_fwd_stream") == (packed + 2 * m * K + 2 * N * r + 4 * m * r + 2 * m * N, "byte")
    assert bench.streamed(w16) and not bench.streamed(wl)


def test_footprint_follows_the_pages_storage_accounting():
    import bench
    from quantized_base_rank_amd.inputs import WORKLOADS
    wl = WORKLOADS["down_proj70b"]
    fp = bench.footprint(wl, wl.packed_weight_bytes())
    # [QLoRA explainer, "Innovation 2: Double Quantization"]: after double
    # quantization the block constants cost about 0.127 bits per weight
    assert abs(fp["bits_per_param"] - 4 - _golden("dq_overhead_bits")) < 1e-3
    assert abs(fp["bits_per_param"] - (4 + 8 / 64 + 32 / (64 * 256))) < 1e-4
    # [QLoRA explainer, "The contribution"]: a 65B model's frozen 4-bit weights
    # leave room on the one 48 GB GPU
    assert fp["weights_65b_gb"] < _golden("single_gpu_GB")
    # [LQ-LoRA record, abstract]: 27 GB for a 70B model at 2.75-2.85 bits; this
    # library's nearest uniform format (NF3 + DQ, 3.127 bits) lands close above
    assert _golden("lqlora_70b_GB") < fp["weights_70b_nf3_dq_gb"] < 1.2 * _golden("lqlora_70b_GB")
    # INT4 groups of 32 with an fp16 scale and zero point: 4 + 32 / 32 bits
    qa = WORKLOADS["qa_int4"]
    assert bench.footprint(qa, qa.packed_weight_bytes())["bits_per_param"] == 5.0
