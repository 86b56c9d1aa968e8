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


def mx6_unpack_blocks(raw: np.ndarray):
    """[..., 32] bytes (one stored MX block each) -> (codes uint8 [..., 32] in
    value order, E8M0 bytes [...], padding bytes [..., 7]).  Layout from the
    header: bits [6p, 6p + 6) of the first 24 bytes (little endian) hold
    element p; element 2i is value i, element 2i + 1 is value 16 + i; byte
    24 is the scale, bytes 25..31 are zero."""
    raw = np.ascontiguousarray(raw, np.uint8)
    bits = np.unpackbits(raw[..., :24], axis=-1, bitorder="little")      # [..., 192]
    el = bits.reshape(raw.shape[:-1] + (32, 6))
    elem = (el * (1 << np.arange(6))).sum(-1).astype(np.uint8)         # element p
    codes = np.empty_like(elem)
    codes[..., :16] = elem[..., 0::2]
    codes[..., 16:] = elem[..., 1::2]
    return codes, raw[..., 24], raw[..., 25:]


def mx4_unpack_blocks(raw: np.ndarray):
    """[..., 32] bytes (one stored E2M1 block each) -> (codes uint8 [..., 32]
    in value order, E8M0 bytes [...], padding bytes [..., 15]).  Layout from
    the header: byte i (i < 16) holds value i in its low nibble and value
    16 + i in its high nibble; bytes 16..23 are zero, byte 24 is the scale,
    bytes 25..31 are zero."""
    raw = np.ascontiguousarray(raw, np.uint8)
    codes = np.empty(raw.shape[:-1] + (32,), np.uint8)
    codes[..., :16] = raw[..., :16] & 0x0F
    codes[..., 16:] = raw[..., :16] >> 4
    pad = np.concatenate([raw[..., 16:24], raw[..., 25:]], axis=-1)
    return codes, raw[..., 24], pad


def _unpack(fmt):
    return mx4_unpack_blocks if fmt == "mxfp4" else mx6_unpack_blocks


def mx6_rows(x6: np.ndarray, N: int, fmt: str = "mxfp6"):
    """q6 / k6 [B,H,N_pad,d] bytes -> (codes [B,H,N,d], E8M0 [B,H,N,d/32], pad)."""
    B, H, Np, d = x6.shape
    c, e, pad = _unpack(fmt)(x6.reshape(B, H, Np, d // 32, 32))
    return c.reshape(B, H, Np, d)[:, :, :N], e[:, :, :N], pad


def mx6_v(v6: np.ndarray, N: int, fmt: str = "mxfp6"):
    """v6 [B,H,nblk,d,128] bytes -> (codes [B,H,N,d] in key order, E8M0
    [B,H,ceil(N/32),d], pad)."""
    B, H, nblk, d, _ = v6.shape
    c, e, pad = _unpack(fmt)(v6.reshape(B, H, nblk, d, 4, 32))
    c = np.transpose(c.reshape(B, H, nblk, d, 128), (0, 1, 2, 4, 3)).reshape(B, H, nblk * 128, d)
    e = np.transpose(e, (0, 1, 2, 4, 3)).reshape(B, H, nblk * 4, d)
    return c[:, :, :N], e[:, :, :-(-N // 32)], pad
