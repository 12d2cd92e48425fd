"""The TILED weight layout of include/moe_mxfp4.h, written out in numpy from
the header's byte formulas (test-side reference; the library converts with
its own kernel)."""
import numpy as np


def tile_packed(packed: np.ndarray) -> np.ndarray:
    """Row-major [rows, K/2] -> tiled bytes (rows*K/2,)."""
    rows, half = packed.shape
    K = 2 * half
    ns = K // 128
    out = np.empty(rows * half, np.uint8)
    blocks = packed.reshape(rows, K // 32, 16)
    n = np.arange(rows)[:, None]
    b = np.arange(K // 32)[None, :]
    off = 16 * (64 * ((n // 16) * ns + b // 4) + (n % 16) + 16 * (b % 4))
    out.reshape(-1, 16)[(off // 16).ravel()] = blocks.reshape(-1, 16)
    return out


def tile_scales(scales: np.ndarray) -> np.ndarray:
    """Row-major [rows, K/32] -> tiled scale bytes ((rows/16) * ng * 256,)."""
    rows, nb = scales.shape
    ns = nb // 4
    ng = (ns + 3) // 4
    out = np.zeros((rows // 16) * ng * 256, np.uint8)
    n = np.arange(rows)[:, None]
    b = np.arange(nb)[None, :]
    off = 4 * (64 * ((n // 16) * ng + b // 16) + (n % 16) + 16 * (b % 4)) + (b // 4) % 4
    out[off.ravel()] = scales.ravel()
    return out
