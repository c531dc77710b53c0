"""Seeded synthetic workloads for the 4-bit + LoRA linear layer.

This module only draws random numbers and stores them in the layer's input
formats (fp32 weights, bf16 activations and adapters).  It holds none of the
method's arithmetic, so both the library's tests and the CPU oracle can be fed
the same bytes from it.

Recipe (per workload, ``numpy.random.default_rng(seed)``, draws in the order
W, A, B, x, dY):

* W  fp32 [d_out][d_in] ~ N(0, 0.02^2)           (standard deviation 0.02)
* A  bf16 [r][d_in/pool] ~ U(-1/sqrt(f), 1/sqrt(f)), f = d_in/pool
* B  bf16 [d_out][r]     ~ N(0, 0.01^2)
* x  bf16 [M][d_in]      ~ N(0, 1)
* dY bf16 [M][d_out]     ~ N(0, 1)

bf16 values are the round-to-nearest-even images of fp32 draws.  Synthetic
Gaussian layers at LLaMA projection shapes stand in for pretrained weights,
which are not used here.
"""

from __future__ import annotations

import dataclasses

import numpy as np


def _bf16_rne_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d_out: int
    d_in: int
    M: int
    r: int
    s: float = 2.0
    fmt: str = "nf4"          # "nf4", "int4" or "nf" (NormalFloat-k, `bits` bits)
    block: int = 64           # NF absmax block, or INT4 group size
    dq_block: int = 256       # NF second-level group (0 = none)
    pool: int = 1             # 1 = plain LoRA; = group for QA-LoRA pooled adapter
    bits: int = 4             # NormalFloat-k bit count (fmt "nf")

    @property
    def k_a(self) -> int:
        return self.d_in // self.pool

    def with_m(self, M: int) -> "Workload":
        return dataclasses.replace(self, M=M)

    def flops_fwd(self) -> int:
        M, N, K, r = self.M, self.d_out, self.d_in, self.r
        return 2 * M * N * K + 2 * M * self.k_a * r + 2 * M * N * r

    def flops_bwd(self) -> int:
        M, N, K, r = self.M, self.d_out, self.d_in, self.r
        return 2 * M * N * K + 4 * M * N * r + 4 * M * self.k_a * r

    def packed_weight_bytes(self) -> int:
        n_el = self.d_out * self.d_in
        if self.fmt in ("nf4", "nf"):
            nb = n_el // self.block
            codes = n_el * (4 if self.fmt == "nf4" else self.bits) // 8
            if self.dq_block:
                return codes + nb + 4 * (-(-nb // self.dq_block))
            return codes + 4 * nb
        ng = n_el // self.block
        return n_el // 2 + 2 * 2 * ng


#: The layer shapes exercised by tests and the benchmark.
WORKLOADS = {
    "tiny": Workload("tiny-256x256-r8", 256, 256, 16, 8),
    "q_proj": Workload("llama7b-q_proj-4096x4096-r16", 4096, 4096, 16, 16),
    "up_proj": Workload("llama7b-up_proj-11008x4096-r64", 11008, 4096, 4096, 64),
    "qa_int4": Workload("qalora-int4g32-4096x11008-r64", 4096, 11008, 2048, 64,
                        fmt="int4", block=32, dq_block=0, pool=32),
    "down_proj70b": Workload("llama2-70b-down_proj-8192x28672-r64", 8192, 28672, 4096, 64),
    # the 70B down_proj with 3-bit NormalFloat weights (LQ-LoRA's sub-4-bit
    # regime; the layer reads them through the per-call transcoded form)
    "down_proj70b_nf3": Workload("llama2-70b-down_proj-8192x28672-r64-nf3", 8192, 28672, 4096, 64,
                                 fmt="nf", bits=3),
}


@dataclasses.dataclass
class Inputs:
    W: np.ndarray    # fp32 [d_out][d_in]
    A: np.ndarray    # uint16 bf16 bits [r][k_a]
    B: np.ndarray    # uint16 bf16 bits [d_out][r]
    x: np.ndarray    # uint16 bf16 bits [M][d_in]
    dy: np.ndarray   # uint16 bf16 bits [M][d_out]


def make_inputs(wl: Workload, seed: int = 0, w_std: float = 0.02, b_std: float = 0.01) -> Inputs:
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((wl.d_out, wl.d_in), dtype=np.float32)
    W *= np.float32(w_std)
    lim = 1.0 / np.sqrt(wl.k_a)
    A = _bf16_rne_bits(rng.uniform(-lim, lim, (wl.r, wl.k_a)).astype(np.float32))
    B = _bf16_rne_bits((rng.standard_normal((wl.d_out, wl.r), dtype=np.float32) * np.float32(b_std)))
    x = _bf16_rne_bits(rng.standard_normal((wl.M, wl.d_in), dtype=np.float32))
    dy = _bf16_rne_bits(rng.standard_normal((wl.M, wl.d_out), dtype=np.float32))
    return Inputs(W, A, B, x, dy)


def make_weight(d_out: int, d_in: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((d_out, d_in), dtype=np.float32)
    W *= np.float32(std)
    return W


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """bf16 (ties-to-even) bit patterns of arbitrary fp32 test data."""
    return _bf16_rne_bits(np.asarray(a, dtype=np.float32))
