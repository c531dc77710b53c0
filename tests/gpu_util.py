"""Helpers shared by the GPU tests: moving seeded inputs to the device and
running the oracle on the same bytes.  No method arithmetic lives here."""

from __future__ import annotations

import numpy as np


def to_dev_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_f32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_host_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def u8(t) -> np.ndarray:
    return host(t).view(np.uint8)


def f16_bits(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
