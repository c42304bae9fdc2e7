"""numpy front end of the C oracle (oracle/ibp_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product path never does.
It only marshals numpy arrays into the C functions; all arithmetic is in C.

`Oracle(path)` binds one build of the C file (the tests also load deliberately
broken copies of it to show that the pins catch them); the module-level
functions use the default build, oracle/liboracle.so.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i64p = ctypes.POINTER(ctypes.c_int64)
_c = ctypes


def _p(a, t):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def _rows2d(rows):
    rows = np.ascontiguousarray(rows)
    assert rows.ndim == 2
    return rows.view(np.uint8).reshape(rows.shape[0], -1)


class Oracle:
    def __init__(self, path=DEFAULT_LIB):
        L = ctypes.CDLL(path)
        L.orc_cutoff.restype = _c.c_int64
        L.orc_cutoff.argtypes = [_c.c_double, _c.c_uint64]
        L.orc_num_chunks.restype = _c.c_uint32
        L.orc_num_chunks.argtypes = [_c.c_uint32, _c.c_uint32]
        L.orc_build_metadata.restype = _c.c_int
        L.orc_build_metadata.argtypes = [_u8p, _c.c_uint64, _i64p, _c.c_uint64, _c.c_uint32,
                                         _c.c_double, _u8p, _u8p, _u64p]
        L.orc_compress.restype = _c.c_int
        L.orc_compress.argtypes = [_u8p, _c.c_uint64, _c.c_uint64, _c.c_uint64, _c.c_uint32,
                                   _c.c_uint32, _u8p, _u8p, _u8p, _c.c_uint64, _u32p, _u32p]
        L.orc_compact.restype = _c.c_int
        L.orc_compact.argtypes = [_u8p, _c.c_uint64, _u32p, _c.c_uint64, _u64p, _u8p]
        L.orc_compact_aligned.restype = _c.c_int
        L.orc_compact_aligned.argtypes = [_u8p, _c.c_uint64, _u32p, _c.c_uint64, _c.c_uint32,
                                          _u64p, _u8p]
        L.orc_cache_index.restype = _c.c_int
        L.orc_cache_index.argtypes = [_u32p, _c.c_uint64, _u64p]
        L.orc_gather_decompress.restype = _c.c_int
        L.orc_gather_decompress.argtypes = [_u8p, _c.c_uint64, _u64p, _u32p, _c.c_uint64, _i64p,
                                            _c.c_uint64, _c.c_uint32, _c.c_uint32, _u8p, _u8p,
                                            _u8p]
        self.lib = L
        self.path = path

    def cutoff(self, threshold, n):
        return int(self.lib.orc_cutoff(float(threshold), int(n)))

    def num_chunks(self, tensor_bytes, chunk_bytes):
        return int(self.lib.orc_num_chunks(tensor_bytes, chunk_bytes))

    def build_metadata(self, rows, threshold, sample_ids=None, return_ones=False):
        """rows: (N, B) array (any dtype, viewed as bytes).  Returns (mask,
        bitval) as uint32 arrays of B/4 words (plus per-bit one counts)."""
        r = _rows2d(rows)
        B = r.shape[1]
        ids = None if sample_ids is None else np.ascontiguousarray(sample_ids, dtype=np.int64)
        n = r.shape[0] if ids is None else ids.shape[0]
        mask = np.zeros(B, np.uint8)
        bitval = np.zeros(B, np.uint8)
        ones = np.zeros(8 * B, np.uint64)
        rc = self.lib.orc_build_metadata(_p(r, _u8p), B, _p(ids, _i64p), n, B, float(threshold),
                                         _p(mask, _u8p), _p(bitval, _u8p), _p(ones, _u64p))
        if rc != 0:
            raise ValueError("orc_build_metadata rejected its arguments")
        out = (mask.view(np.uint32), bitval.view(np.uint32))
        return out + (ones,) if return_ones else out

    def compress(self, rows, mask, bitval, chunk_bytes, slot_bytes=None, store=None,
                 part_bits=None, first_tensor=0, n_tensors=None):
        """Compresses rows into in-place slots; returns (store, part_bits, lengths).

        store: uint8 array of n_tensors*slot_bytes (allocated if None);
        part_bits: uint32 bitmap of n_tensors*n_c bits (allocated if None)."""
        r = _rows2d(rows)
        n, B = r.shape
        if slot_bytes is None:
            slot_bytes = (B + 127) // 128 * 128
        n_c = self.num_chunks(B, chunk_bytes)
        if n_tensors is None:
            n_tensors = first_tensor + n
        if store is None:
            store = np.zeros(n_tensors * slot_bytes, np.uint8)
        if part_bits is None:
            part_bits = np.zeros((n_tensors * n_c + 31) // 32, np.uint32)
        lengths = np.zeros(n, np.uint32)
        m8 = np.ascontiguousarray(mask).view(np.uint8)
        v8 = np.ascontiguousarray(bitval).view(np.uint8)
        rc = self.lib.orc_compress(_p(r, _u8p), B, n, first_tensor, B, chunk_bytes,
                                   _p(m8, _u8p), _p(v8, _u8p), _p(store, _u8p), slot_bytes,
                                   _p(part_bits, _u32p), _p(lengths, _u32p))
        if rc != 0:
            raise ValueError("orc_compress rejected its arguments")
        return store, part_bits, lengths

    def compact(self, store, slot_bytes, lengths, with_cache=True):
        """Returns (offsets (n+1,) uint64, cache uint8 array or None)."""
        lengths = np.ascontiguousarray(lengths, dtype=np.uint32)
        n = lengths.shape[0]
        offsets = np.zeros(n + 1, np.uint64)
        rc = self.lib.orc_compact(None, slot_bytes, _p(lengths, _u32p), n, _p(offsets, _u64p),
                                  None)
        if rc != 0:
            raise ValueError("orc_compact rejected its arguments")
        if not with_cache:
            return offsets, None
        cache = np.zeros(int(offsets[-1]), np.uint8)
        rc = self.lib.orc_compact(_p(store, _u8p), slot_bytes, _p(lengths, _u32p), n,
                                  _p(offsets, _u64p), _p(cache, _u8p))
        if rc != 0:
            raise ValueError("orc_compact rejected its arguments")
        return offsets, cache

    def compact_aligned(self, store, slot_bytes, lengths, align, with_cache=True):
        """As compact(), each entry rounded up to a multiple of `align` bytes."""
        lengths = np.ascontiguousarray(lengths, dtype=np.uint32)
        n = lengths.shape[0]
        offsets = np.zeros(n + 1, np.uint64)
        rc = self.lib.orc_compact_aligned(None, slot_bytes, _p(lengths, _u32p), n, align,
                                          _p(offsets, _u64p), None)
        if rc != 0:
            raise ValueError("orc_compact_aligned rejected its arguments")
        if not with_cache:
            return offsets, None
        cache = np.zeros(int(offsets[-1]), np.uint8)
        rc = self.lib.orc_compact_aligned(_p(store, _u8p), slot_bytes, _p(lengths, _u32p), n,
                                          align, _p(offsets, _u64p), _p(cache, _u8p))
        if rc != 0:
            raise ValueError("orc_compact_aligned rejected its arguments")
        return offsets, cache

    def cache_index(self, part_bits, n_bits):
        """Rank index (ceil(n_bits / 32),) uint64 of a participation bitmap."""
        pb = np.ascontiguousarray(part_bits, dtype=np.uint32)
        index = np.zeros((n_bits + 31) // 32, np.uint64)
        rc = self.lib.orc_cache_index(_p(pb, _u32p), n_bits, _p(index, _u64p))
        if rc != 0:
            raise ValueError("orc_cache_index rejected its arguments")
        return index

    def gather_decompress(self, store, part_bits, n_tensors, ids, tensor_bytes, chunk_bytes,
                          mask, bitval, slot_bytes=None, offsets=None, out=None):
        """Returns the (n_ids, tensor_bytes) uint8 array of decompressed rows."""
        ids = np.ascontiguousarray(ids, dtype=np.int64)
        if slot_bytes is None:
            slot_bytes = (tensor_bytes + 127) // 128 * 128
        if out is None:
            out = np.empty((ids.shape[0], tensor_bytes), np.uint8)
        m8 = np.ascontiguousarray(mask).view(np.uint8)
        v8 = np.ascontiguousarray(bitval).view(np.uint8)
        offs = None if offsets is None else np.ascontiguousarray(offsets, dtype=np.uint64)
        pb = np.ascontiguousarray(part_bits, dtype=np.uint32)
        rc = self.lib.orc_gather_decompress(_p(store, _u8p), slot_bytes, _p(offs, _u64p),
                                            _p(pb, _u32p), n_tensors, _p(ids, _i64p),
                                            ids.shape[0], tensor_bytes, chunk_bytes,
                                            _p(m8, _u8p), _p(v8, _u8p), _p(out, _u8p))
        if rc != 0:
            raise ValueError("orc_gather_decompress rejected its arguments")
        return out


_default = None


def default():
    """The oracle built from oracle/ibp_oracle.c (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(DEFAULT_LIB):
            from oracle import build as _b
            _b.build()
        _default = Oracle(DEFAULT_LIB)
    return _default


def cutoff(*a, **k):
    return default().cutoff(*a, **k)


def num_chunks(*a, **k):
    return default().num_chunks(*a, **k)


def build_metadata(*a, **k):
    return default().build_metadata(*a, **k)


def compress(*a, **k):
    return default().compress(*a, **k)


def compact(*a, **k):
    return default().compact(*a, **k)


def compact_aligned(*a, **k):
    return default().compact_aligned(*a, **k)


def cache_index(*a, **k):
    return default().cache_index(*a, **k)


def gather_decompress(*a, **k):
    return default().gather_decompress(*a, **k)
