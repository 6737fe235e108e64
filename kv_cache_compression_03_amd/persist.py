"""Persist and reload the FP4 main-KV cache; park window KV in host memory.

[deep-dive §3.4] Only the FP4 global KV is persisted (to SSD or host memory, kept
for days); the window KV is held in host DRAM for minutes.  Reading: a persisted
cache is its FP4 codes and E4M3 scales, byte for byte as they sit in HBM, plus
how many entries each sequence holds.  The bf16 indexer keys are not stored: on
reload they are formed again from the codes and scales (`csa2_indexer_keys`),
which gives back the same bits, since a key is a function of the dequantised
entry alone.  Window KV (E4M3 bytes) is parked in pinned host memory and put
back with plain copies.

On disk a cache is a directory holding `codes.npy` [B, N, d/2] u8,
`scales.npy` [B, N, d/16] u8 and `meta.json`.  The arrays are written and read
one sequence at a time through memory maps (`allow_pickle=False`), so a cache
larger than host memory streams through.
"""
import json
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import binding as bd

FORMAT = "csa2-fp4-cache-v1"


def _check_cache(codes: torch.Tensor, scales: torch.Tensor) -> Tuple[int, int, int]:
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("codes and scales must be uint8 tensors")
    if codes.dim() != 3 or scales.dim() != 3:
        raise ValueError("codes must be [B, N, d/2] and scales [B, N, d/16]")
    B, N, half = codes.shape
    d = 2 * half
    if d % 16 or tuple(scales.shape) != (B, N, d // 16):
        raise ValueError(f"scales shape {tuple(scales.shape)} does not match codes {tuple(codes.shape)}")
    return B, N, d


def save_cache(path: str, codes: torch.Tensor, scales: torch.Tensor,
               n_valid: Optional[Sequence[int]] = None) -> None:
    """Write a cache (device or host tensors) under directory `path`.
    n_valid[b] = entries sequence b holds (default: all N)."""
    B, N, d = _check_cache(codes, scales)
    valid = [N] * B if n_valid is None else [int(v) for v in n_valid]
    if len(valid) != B or any(v < 0 or v > N for v in valid):
        raise ValueError("n_valid must give 0 <= entries <= N for every sequence")
    os.makedirs(path, exist_ok=True)
    fmt = np.lib.format
    cm = fmt.open_memmap(os.path.join(path, "codes.npy"), mode="w+", dtype=np.uint8, shape=(B, N, d // 2))
    sm = fmt.open_memmap(os.path.join(path, "scales.npy"), mode="w+", dtype=np.uint8, shape=(B, N, d // 16))
    for b in range(B):
        cm[b] = codes[b].cpu().numpy()
        sm[b] = scales[b].cpu().numpy()
    cm.flush()
    sm.flush()
    del cm, sm
    meta = {"format": FORMAT, "sequences": B, "entries": N, "d": d, "n_valid": valid}
    with open(os.path.join(path, "meta.json"), "w") as f:
        json.dump(meta, f)


def load_cache(path: str, W_ik: Optional[torch.Tensor] = None, device="cuda"):
    """Read a cache saved by `save_cache` into `device`.  Returns
    (codes, scales, k_idx, n_valid); k_idx is formed again from the codes and
    scales when W_ik [d, d_i] bf16 is given (device tensors only), else None."""
    with open(os.path.join(path, "meta.json")) as f:
        meta = json.load(f)
    if meta.get("format") != FORMAT:
        raise ValueError(f"{path}: not a {FORMAT} cache")
    B, N, d = int(meta["sequences"]), int(meta["entries"]), int(meta["d"])
    cm = np.load(os.path.join(path, "codes.npy"), mmap_mode="r", allow_pickle=False)
    sm = np.load(os.path.join(path, "scales.npy"), mmap_mode="r", allow_pickle=False)
    if cm.dtype != np.uint8 or cm.shape != (B, N, d // 2) or sm.dtype != np.uint8 or sm.shape != (B, N, d // 16):
        raise ValueError(f"{path}: arrays do not match meta.json")
    codes = torch.empty(B, N, d // 2, dtype=torch.uint8, device=device)
    scales = torch.empty(B, N, d // 16, dtype=torch.uint8, device=device)
    for b in range(B):
        codes[b].copy_(torch.from_numpy(np.array(cm[b])))    # a writable host copy of the mapped rows
        scales[b].copy_(torch.from_numpy(np.array(sm[b])))
    k_idx = None if W_ik is None else bd.csa2_indexer_keys(codes, scales, W_ik)
    return codes, scales, k_idx, list(meta["n_valid"])


def park_windows(swa: Sequence[torch.Tensor]) -> List[torch.Tensor]:
    """Copy each layer's window [B, S, d] (E4M3 bytes) into pinned host memory."""
    out = []
    for w in swa:
        h = torch.empty(w.shape, dtype=w.dtype, pin_memory=True)
        h.copy_(w)
        out.append(h)
    return out


def restore_windows(parked: Sequence[torch.Tensor], swa: Sequence[torch.Tensor]) -> None:
    """Copy parked windows back into the device windows (same shapes)."""
    if len(parked) != len(swa):
        raise ValueError("one parked window per layer")
    for h, w in zip(parked, swa):
        if h.shape != w.shape or h.dtype != w.dtype:
            raise ValueError("parked window does not match the device window")
        w.copy_(h)
