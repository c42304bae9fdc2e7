"""Brute-force reference for Invariant Bit Packing on tiny inputs.

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product path.

A second, independent statement of the same definitions as the C oracle
(oracle/ibp_oracle.c), written with Python lists of 0/1 integers so that every
step can be read against the pages:

  [G-EN] gist.science English explainer of "Reducing the GPU Memory Bottleneck
         with Lossless Compression for ML -- Extended", Technical Summary.
  [JH]   juhe.plus Chinese review of the same paper.

Readings where the pages are silent are the same as the C oracle's header
states (LSB-first bit order, cutoff ceil(T*n) in binary64, participation needs
a full Mask match and at least one Mask bit, unpadded concatenation of chunk
streams).  Pure-Python loops: use only for tensors of a few hundred bytes.
"""
import math


def to_bits(data):
    """Bytes -> list of bits, bit i = bit (i % 8) of byte i // 8."""
    return [(data[i // 8] >> (i % 8)) & 1 for i in range(8 * len(data))]


def from_bits(bits, n_bytes):
    """List of bits -> bytes of length n_bytes (missing bits are zero)."""
    out = bytearray(n_bytes)
    for i, b in enumerate(bits):
        if b:
            out[i // 8] |= 1 << (i % 8)
    return bytes(out)


def cutoff(threshold, n):
    """[G-EN] Preprocessing: a position is invariant if >= ceil(T*n) agree."""
    return math.ceil(threshold * n)


def build_metadata(samples, threshold):
    """[G-EN] Preprocessing.  samples: list of equal-length byte strings.

    Returns (mask, bitval) as byte strings of the tensor size.
    """
    n = len(samples)
    size = len(samples[0])
    m = cutoff(threshold, n)
    cols = [to_bits(s) for s in samples]
    mask, bitval = [], []
    for i in range(8 * size):
        ones = sum(col[i] for col in cols)
        zeros = n - ones
        invariant = max(ones, zeros) >= m
        mask.append(1 if invariant else 0)
        bitval.append(1 if (invariant and ones > zeros) else 0)
    return from_bits(mask, size), from_bits(bitval, size)


def chunk_ranges(tensor_bytes, chunk_bytes):
    """Bit ranges [lo, hi) of the chunks of one tensor."""
    out = []
    start = 0
    while start < tensor_bytes:
        end = min(start + chunk_bytes, tensor_bytes)
        out.append((8 * start, 8 * end))
        start = end
    return out


def compress_one(x, mask, bitval, chunk_bytes):
    """[G-EN] Compression, for one tensor.

    Returns (payload bytes, list of participation bits, payload length in bits).
    """
    xb, mb, vb = to_bits(x), to_bits(mask), to_bits(bitval)
    stream, part = [], []
    for lo, hi in chunk_ranges(len(x), chunk_bytes):
        positions = range(lo, hi)
        matches = all(xb[i] == vb[i] for i in positions if mb[i])
        kept = [i for i in positions if not mb[i]]
        p = matches and len(kept) < hi - lo
        part.append(1 if p else 0)
        if p:
            stream.extend(xb[i] for i in kept)
        else:
            stream.extend(xb[i] for i in positions)
    n_bytes = (len(stream) + 7) // 8
    return from_bits(stream, n_bytes), part, len(stream)


def decompress_one(payload, part, mask, bitval, tensor_bytes, chunk_bytes):
    """[G-EN] Decompression, for one tensor."""
    pb, mb, vb = to_bits(payload), to_bits(mask), to_bits(bitval)
    out = [0] * (8 * tensor_bytes)
    cursor = 0
    for c, (lo, hi) in enumerate(chunk_ranges(tensor_bytes, chunk_bytes)):
        for i in range(lo, hi):
            if part[c] and mb[i]:
                out[i] = vb[i]
            else:
                out[i] = pb[cursor]
                cursor += 1
    return from_bits(out, tensor_bytes)
