"""Small test-side helpers: bf16 bit conversion and logical gathers."""
from __future__ import annotations

import numpy as np
import torch

PAGE = 16


def bf16_bits(x) -> np.ndarray:
    """float array -> bf16 bit patterns (round to nearest even) as uint16."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_float(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def logical_rows(pool: torch.Tensor, bt: np.ndarray, s: int, N: int, g: int) -> np.ndarray:
    """Rows [N][d] of KV head g of sequence s, in token order, as bf16 bits.

    pool: [num_blocks][16][Hkv][d] bf16 tensor (host or device)."""
    nb = (N + PAGE - 1) // PAGE
    blocks = torch.as_tensor(np.asarray(bt[s, :nb], dtype=np.int64), device=pool.device)
    rows = pool.index_select(0, blocks)[:, :, g, :].reshape(nb * PAGE, -1)[:N]
    return tensor_bits(rows)


def logical_codes(codes: torch.Tensor, bt: np.ndarray, s: int, N: int, g: int) -> np.ndarray:
    """Codes pool [num_blocks][Hkv][16][W] uint32 (as int32 tensor) -> [N][W]."""
    nb = (N + PAGE - 1) // PAGE
    blocks = torch.as_tensor(np.asarray(bt[s, :nb], dtype=np.int64), device=codes.device)
    sel = codes.index_select(0, blocks)[:, g]          # [nb][16][W]
    out = sel.reshape(nb * PAGE, -1)[:N]
    return out.cpu().numpy().view(np.uint32).copy()


def logical_radii(radii: torch.Tensor, bt: np.ndarray, s: int, N: int, g: int) -> np.ndarray:
    """Radii pool [num_blocks][Hkv][16] uint8 -> [N]."""
    nb = (N + PAGE - 1) // PAGE
    blocks = torch.as_tensor(np.asarray(bt[s, :nb], dtype=np.int64), device=radii.device)
    return radii.index_select(0, blocks)[:, g].reshape(-1)[:N].cpu().numpy().copy()
