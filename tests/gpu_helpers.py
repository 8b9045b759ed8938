"""Helpers for the GPU parity tests (device upload/download of seeded inputs)."""
from __future__ import annotations

import numpy as np

import gptdata


def torch_mod():
    import torch
    return torch


def dev():
    return torch_mod().device("cuda:0")


def bf16_dev(a_f32: np.ndarray):
    """Round fp32 to bf16 on the host (RNE) and upload; returns (tensor, exact fp64 values)."""
    torch = torch_mod()
    bits = gptdata.bf16_round_bits(a_f32)
    t = torch.from_numpy(bits.view(np.int16)).to(dev()).view(torch.bfloat16)
    return t, gptdata.bf16_bits_to_f32(bits).astype(np.float64)


def f32_dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a, dtype=np.float32)
    return torch.from_numpy(a).to(dev()), a.astype(np.float64)


def to_host(t) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> fp64 numpy."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return gptdata.bf16_bits_to_f32(bits).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def empty(shape, dtype: str):
    torch = torch_mod()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.empty(shape, dtype=td, device=dev())


def params_of(w: gptdata.Weights) -> dict:
    from helpers import oracle_params
    return oracle_params(w)
