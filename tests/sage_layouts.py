"""Test-side readers of libsage's documented buffer layouts (include/sage.h),
written from the header's description (independent of the library code)."""
import numpy as np
import torch


def vperm_positions():
    """pos[r] = position of key r inside a tile row: r = 32 kb + 8 b + 4 g + q
    is stored at 64 g + 16 kb + 4 b + q."""
    r = np.arange(128)
    kb, b, g, q = r >> 5, (r >> 3) & 3, (r >> 2) & 1, r & 3
    return 64 * g + 16 * kb + 4 * b + q


def vq_natural(vq: np.ndarray, N: int) -> np.ndarray:
    """[B,H,nblk,d,128] codes (permuted keys) -> [B,H,N,d] in key order."""
    B, H, nblk, d, _ = vq.shape
    x = vq[..., vperm_positions()]                  # [B,H,nblk,d,128 keys]
    x = np.transpose(x, (0, 1, 2, 4, 3)).reshape(B, H, nblk * 128, d)
    return np.ascontiguousarray(x[:, :, :N])


def to_hnd(x: torch.Tensor, layout: str) -> torch.Tensor:
    return x if layout == "HND" else x.permute(0, 2, 1, 3)


def codes(x: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy codes, same shape."""
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
