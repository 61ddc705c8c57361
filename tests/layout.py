"""Packed int8 operand layout, written independently of the library in numpy.

The layout the C ABI documents: a code matrix R[rows][K] is stored as 16-row
x 64-byte fragments of 1 KiB, fragment (row block b, window w) at
(b * KW + w) * 1024 with KW = ceil(K / 64), and element (r, k) of it at
((k % 64) // 16) * 256 + (r % 16) * 16 + k % 16.  Padding is zero.

This is a pure index permutation (no arithmetic of the method), used by the
tests to compare the GPU's packed codes with the oracle's row-major codes.
"""
import numpy as np


def packed_bytes(rows: int, K: int) -> int:
    return -(-rows // 16) * -(-K // 64) * 1024


def pack(codes: np.ndarray) -> np.ndarray:
    """Row-major int8 [rows][K] -> packed flat int8 buffer."""
    rows, K = codes.shape
    RB, KW = -(-rows // 16), -(-K // 64)
    pad = np.zeros((RB * 16, KW * 64), np.int8)
    pad[:rows, :K] = codes
    # [b, r, w, q, e] -> [b, w, q, r, e]
    return np.ascontiguousarray(
        pad.reshape(RB, 16, KW, 4, 16).transpose(0, 2, 3, 1, 4)).reshape(-1)


def unpack(buf: np.ndarray, rows: int, K: int, with_padding: bool = False) -> np.ndarray:
    """Packed flat buffer -> row-major int8 [rows][K] (or the padded matrix)."""
    RB, KW = -(-rows // 16), -(-K // 64)
    b = np.asarray(buf).view(np.int8)[:RB * KW * 1024]
    full = b.reshape(RB, KW, 4, 16, 16).transpose(0, 3, 1, 2, 4).reshape(RB * 16, KW * 64)
    return full if with_padding else np.ascontiguousarray(full[:rows, :K])


def padding_is_zero(buf: np.ndarray, rows: int, K: int) -> bool:
    full = unpack(buf, rows, K, with_padding=True)
    return bool(np.all(full[rows:, :] == 0) and np.all(full[:, K:] == 0))


# ---- packed 4-bit weights ------------------------------------------------------
#
# Same fragment order at half the size: fragment (b, w) at (b * KW + w) * 512;
# the 16 codes of (row r, quarter q) are 8 bytes at q * 128 + (r % 16) * 8;
# code i of them sits in byte (i % 4) + 4 * (i // 8), low nibble when
# i % 8 < 4, else high nibble, as a two's-complement nibble.

def packed4_bytes(rows: int, K: int) -> int:
    return -(-rows // 16) * -(-K // 64) * 512


def _nibble_index():
    i = np.arange(16)
    return (i % 4) + 4 * (i // 8), (i % 8) >= 4       # byte, high?


def pack4(codes: np.ndarray) -> np.ndarray:
    """Row-major codes in [-8, 7] [rows][K] -> packed 4-bit flat uint8 buffer."""
    assert codes.min() >= -8 and codes.max() <= 7
    rows, K = codes.shape
    RB, KW = -(-rows // 16), -(-K // 64)
    pad = np.zeros((RB * 16, KW * 64), np.int64)
    pad[:rows, :K] = codes
    chunks = pad.reshape(RB, 16, KW, 4, 16).transpose(0, 2, 3, 1, 4)   # [b, w, q, r, i]
    nib = chunks & 0xF
    byte, high = _nibble_index()
    out = np.zeros(chunks.shape[:-1] + (8,), np.int64)
    for i in range(16):
        out[..., byte[i]] |= nib[..., i] << (4 if high[i] else 0)
    return np.ascontiguousarray(out.astype(np.uint8)).reshape(-1)


def unpack4(buf: np.ndarray, rows: int, K: int, with_padding: bool = False) -> np.ndarray:
    """Packed 4-bit flat buffer -> row-major int8 codes [rows][K]."""
    RB, KW = -(-rows // 16), -(-K // 64)
    b = np.asarray(buf).view(np.uint8)[:RB * KW * 512].astype(np.int64)
    b = b.reshape(RB, KW, 4, 16, 8)                                     # [b, w, q, r, byte]
    byte, high = _nibble_index()
    nib = np.stack([(b[..., byte[i]] >> (4 if high[i] else 0)) & 0xF for i in range(16)], axis=-1)
    codes = np.where(nib >= 8, nib - 16, nib).astype(np.int8)           # [b, w, q, r, i]
    full = codes.transpose(0, 3, 1, 2, 4).reshape(RB * 16, KW * 64)
    return full if with_padding else np.ascontiguousarray(full[:rows, :K])


def padding4_is_zero(buf: np.ndarray, rows: int, K: int) -> bool:
    full = unpack4(buf, rows, K, with_padding=True)
    return bool(np.all(full[rows:, :] == 0) and np.all(full[:, K:] == 0))
