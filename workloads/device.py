"""Staging of a workload's host arrays into device tensors (and bits back).

Plain copies through torch; no computation on the values.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import Workload

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def bits_to_device(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(TORCH_DTYPE[dtype])


def device_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def device_to_float64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


@dataclass
class DeviceWorkload:
    query: torch.Tensor
    key_cache: torch.Tensor
    value_cache: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    new_key: torch.Tensor
    new_value: torch.Tensor
    slot_mapping: torch.Tensor
    copy_pairs: torch.Tensor
    out: torch.Tensor
    query_start: torch.Tensor | None = None


def upload(w: Workload, device="cuda") -> DeviceWorkload:
    q = bits_to_device(w.query, w.dtype, device)
    return DeviceWorkload(
        query=q,
        key_cache=bits_to_device(w.key_cache, w.dtype, device),
        value_cache=bits_to_device(w.value_cache, w.dtype, device),
        block_tables=torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(device),
        context_lens=torch.from_numpy(np.ascontiguousarray(w.context_lens)).to(device),
        new_key=bits_to_device(w.new_key, w.dtype, device),
        new_value=bits_to_device(w.new_value, w.dtype, device),
        slot_mapping=torch.from_numpy(np.ascontiguousarray(w.slot_mapping)).to(device),
        copy_pairs=torch.from_numpy(np.ascontiguousarray(w.copy_pairs)).to(device),
        out=torch.empty_like(q),
        query_start=None if w.query_start is None
        else torch.from_numpy(np.ascontiguousarray(w.query_start)).to(device),
    )
