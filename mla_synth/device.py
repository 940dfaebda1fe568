"""Move a synthetic workload onto the GPU as torch tensors (no arithmetic of
the method: dtype conversion of already-rounded values and layout only)."""
from __future__ import annotations

import numpy as np
import torch

from . import Workload, f32_to_bf16_bits, paged_cache


def to_torch(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        # values are already bf16-representable: the conversion is exact
        bits = f32_to_bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def from_torch(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def upload(w: Workload, device="cuda") -> dict:
    d = w.dims
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    t = {
        "weights": {k: to_torch(v, d.dtype, device) for k, v in w.weights.items()},
        "x": to_torch(w.x, d.dtype, device),
        "cache": (torch.from_numpy(paged_cache(w)).to(device) if w.kv_scale > 0
                  else to_torch(paged_cache(w), d.dtype, device)),
        "block_table": i32(w.block_table),
        "cu_seqlens": i32(w.cu_seqlens),
        "prefix_lens": i32(w.prefix_lens),
        "seq_lens": i32(w.kv_lens),
    }
    if w.row_lo is not None:
        t["row_lo"], t["row_hi"] = i32(w.row_lo), i32(w.row_hi)
    return t
