"""Group-structured bit-plane packing.  TEST INFRASTRUCTURE (oracle).

Page 1, FAQ on storage overhead and the section on deployment: the
group-wise allocation needs no bitmap or codebook index, costs no extra
storage, and dequantization has the same structure as uniform quantization.
Page 3 (abstract) and page 1 report about 5.5-6x memory saving at 2 bits.

Reading (the pages fix no layout): bit-planes, group-major.  Group j
(bit-width b_j) starts at word offset off(j) = n * (g/32) * sum_{j'<j} b_j'.
Word (j, plane p, row i, w) sits at off(j) + (p * n + i) * (g/32) + w, and its
bit c is bit p of the code of row i, column j*g + 32w + c.  The total is
exactly n*m*N/32 words when the bit-widths average N; the only metadata is
the k bit-widths.
"""
import numpy as np


def packed_words(n: int, m: int, avg_bits: int) -> int:
    return n * m * avg_bits // 32


def pack_bitplanes(codes, bits, group: int) -> np.ndarray:
    """codes uint8 [n, m], bits [k] -> uint32 words (length n*g/32*sum(bits))."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, m = codes.shape
    k = m // group
    wps = group // 32
    bits = np.asarray(bits, dtype=np.int64)
    out = np.zeros(n * wps * int(bits.sum()), dtype=np.uint32)
    sh = np.arange(32, dtype=np.uint64)
    off = 0
    for j in range(k):
        blk = codes[:, j * group:(j + 1) * group].reshape(n, wps, 32).astype(np.uint64)
        for p in range(int(bits[j])):
            plane = (((blk >> np.uint64(p)) & np.uint64(1)) << sh).sum(axis=-1)
            out[off + p * n * wps: off + (p + 1) * n * wps] = plane.reshape(-1).astype(np.uint32)
        off += int(bits[j]) * n * wps
    return out


def unpack_bitplanes(words, bits, n: int, m: int, group: int) -> np.ndarray:
    """Inverse of ``pack_bitplanes``: uint8 codes [n, m]."""
    words = np.asarray(words, dtype=np.uint32)
    k = m // group
    wps = group // 32
    bits = np.asarray(bits, dtype=np.int64)
    codes = np.zeros((n, m), dtype=np.uint8)
    sh = np.arange(32, dtype=np.uint32)
    off = 0
    for j in range(k):
        acc = np.zeros((n, wps, 32), dtype=np.uint8)
        for p in range(int(bits[j])):
            plane = words[off + p * n * wps: off + (p + 1) * n * wps].reshape(n, wps, 1)
            acc |= (((plane >> sh) & np.uint32(1)).astype(np.uint8) << np.uint8(p))
        codes[:, j * group:(j + 1) * group] = acc.reshape(n, group)
        off += int(bits[j]) * n * wps
    return codes
