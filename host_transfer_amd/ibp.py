"""Thin ctypes binding of libibp.so (include/ibp.h).

Argument marshalling only: every function forwards to the C entry point of
the same name with raw pointers and sizes; all work runs in the library's HIP
kernels.  Pointers may be given as torch tensors (their data_ptr()), as
HostBuffer objects, or as plain integers.  `stream` defaults to torch's
current HIP stream.  A non-zero status raises IbpError.

There is no fallback: if libibp.so has not been built this module raises on
import (build it with `python -c "import __graft_entry__ as g; g.build()"`).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch  # loaded first: libibp.so then binds to the same HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libibp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                      "(__graft_entry__.build() or host_transfer_amd/csrc/build.py)")

_lib = ctypes.CDLL(LIB_PATH)

OK = 0
ERR_NULL, ERR_SIZE, ERR_CHUNK, ERR_THRESHOLD, ERR_ALIGN, ERR_HIP, ERR_FLAGS = -1, -2, -3, -4, -5, -6, -7
MAX_TENSOR_BYTES = 16384
MAX_CHUNKS = 64
HOST_DEFAULT, HOST_COHERENT, HOST_NONCOHERENT = 0, 1, 2
NOT_CACHED = (1 << 64) - 1

_vp = ctypes.c_void_p
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64
_i = ctypes.c_int

# name -> argument types (all return int status)
_SIGS = {
    "ibp_version": [],
    "ibp_num_chunks": [_u32, _u32],
    "ibp_build_metadata": [_vp, _u64, _vp, _u64, _u32, ctypes.c_double, _vp, _vp, _vp, _vp],
    "ibp_build_metadata_noalloc": [_vp, _u64, _vp, _u64, _u32, ctypes.c_double, _vp, _vp, _vp],
    "ibp_compress": [_vp, _u64, _u64, _u64, _u64, _u32, _u32, _vp, _vp, _vp, _u64, _vp, _vp, _vp],
    "ibp_compress_segments": [_vp, _u64, _vp, _vp, _vp, _u32, _u64, _u32, _u32, _vp, _vp, _vp, _u64,
                              _vp, _vp, _vp],
    "ibp_compact_offsets": [_vp, _u64, _vp, _vp],
    "ibp_compact": [_vp, _u64, _u64, _vp, _vp, _u64, _vp],
    "ibp_compact_offsets_aligned": [_vp, _u64, _u32, _vp, _vp],
    "ibp_cache_index": [_vp, _u64, _vp, _vp],
    "ibp_gather_decompress_indexed": [_vp, _u64, _u32, _vp, _u64, _vp, _u64, _u32, _u32, _vp, _vp,
                                      _vp, _vp],
    "ibp_gather_decompress": [_vp, _u64, _u64, _vp, _vp, _u64, _vp, _u64, _u32, _u32, _vp, _vp,
                              _vp, _vp],
    "ibp_gather_decompress_ex": [_vp, _u64, _u64, _vp, _vp, _u64, _vp, _u64, _u32, _u32, _vp,
                                 _vp, _vp, ctypes.c_uint, _vp],
    "ibp_gather_decompress_segments": [_vp, _u64, _u64, _vp, _vp, _u64, _vp, _vp, _u32, _u32,
                                       _u32, _vp, _vp, _vp, _u32, _vp],
    "ibp_cache_offsets": [_vp, _vp, _u64, _vp, _vp],
    "ibp_cache_fill": [_vp, _u64, _vp, _u64, _vp, _vp, _u64, _vp],
    "ibp_gather_decompress_hybrid": [_vp, _u64, _u64, _vp, _u64, _vp, _vp, _u64, _vp, _u64, _u32,
                                     _u32, _vp, _vp, _vp, _vp],
    "ibp_host_alloc": [_u64, ctypes.c_uint, ctypes.POINTER(_vp)],
    "ibp_host_free": [_vp],
    "ibp_raw_gather": [_vp, _u64, _u64, _vp, _u64, _u32, _vp, ctypes.c_uint, _vp],
    "ibp_stream_read": [_vp, _u64, _u32, _vp, _vp],
    "ibp_stream_copy": [_vp, _vp, _u64, _vp],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _i
_lib.ibp_last_error.argtypes = []
_lib.ibp_last_error.restype = ctypes.c_char_p

EXPORTED = tuple(_SIGS) + ("ibp_last_error",)


class IbpError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libibp status {code}: {msg}")
        self.code = code


def last_error() -> str:
    return _lib.ibp_last_error().decode()


def _check(code):
    if code < 0:
        raise IbpError(code, last_error())
    return code


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    if isinstance(x, HostBuffer):
        return x.ptr
    return int(x)


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def version() -> int:
    return _lib.ibp_version()


def num_chunks(tensor_bytes, chunk_bytes) -> int:
    return _check(_lib.ibp_num_chunks(tensor_bytes, chunk_bytes))


def build_metadata(rows, row_stride, sample_ids, n_samples, tensor_bytes, threshold, mask, bitval,
                   counts, stream=None):
    _check(_lib.ibp_build_metadata(_ptr(rows), row_stride, _ptr(sample_ids), n_samples,
                                   tensor_bytes, threshold, _ptr(mask), _ptr(bitval), _ptr(counts),
                                   _stream(stream)))


NOALLOC_MAX_TENSOR_BYTES = 16384


def build_metadata_noalloc(rows, row_stride, sample_ids, n_samples, tensor_bytes, threshold, mask,
                           bitval, stream=None):
    _check(_lib.ibp_build_metadata_noalloc(_ptr(rows), row_stride, _ptr(sample_ids), n_samples,
                                           tensor_bytes, threshold, _ptr(mask), _ptr(bitval),
                                           _stream(stream)))


def compress(rows, row_stride, n_rows, first_tensor, n_tensors, tensor_bytes, chunk_bytes, mask,
             bitval, store, slot_bytes, part_bits, lengths, stream=None):
    _check(_lib.ibp_compress(_ptr(rows), row_stride, n_rows, first_tensor, n_tensors,
                             tensor_bytes, chunk_bytes, _ptr(mask), _ptr(bitval), _ptr(store),
                             slot_bytes, _ptr(part_bits), _ptr(lengths), _stream(stream)))


def compress_segments(rows, row_stride, seg_row, seg_first, seg_count, n_tensors, tensor_bytes,
                      chunk_bytes, masks, bitvals, store, slot_bytes, part_bits, lengths,
                      stream=None):
    """seg_row, seg_first, seg_count: host sequences of one entry per segment."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.uint64)) for x in (seg_row, seg_first,
                                                                           seg_count)]
    n = arrs[0].size
    if any(a.size != n for a in arrs):
        raise ValueError("seg_row, seg_first and seg_count must have one entry per segment")
    _check(_lib.ibp_compress_segments(
        _ptr(rows), row_stride, *[a.ctypes.data if n else None for a in arrs], n, n_tensors,
        tensor_bytes, chunk_bytes, _ptr(masks), _ptr(bitvals), _ptr(store), slot_bytes,
        _ptr(part_bits), _ptr(lengths), _stream(stream)))


def compact_offsets(lengths, n_tensors, offsets, stream=None):
    _check(_lib.ibp_compact_offsets(_ptr(lengths), n_tensors, _ptr(offsets), _stream(stream)))


def compact_offsets_aligned(lengths, n_tensors, entry_align, offsets, stream=None):
    _check(_lib.ibp_compact_offsets_aligned(_ptr(lengths), n_tensors, entry_align, _ptr(offsets),
                                            _stream(stream)))


def cache_index(part_bits, n_tensors, index, stream=None):
    _check(_lib.ibp_cache_index(_ptr(part_bits), n_tensors, _ptr(index), _stream(stream)))


def gather_decompress_indexed(cache, cache_bytes, entry_align, index, n_tensors, ids, n_ids,
                              tensor_bytes, chunk_bytes, mask, bitval, out, stream=None):
    _check(_lib.ibp_gather_decompress_indexed(_ptr(cache), cache_bytes, entry_align, _ptr(index),
                                              n_tensors, _ptr(ids), n_ids, tensor_bytes,
                                              chunk_bytes, _ptr(mask), _ptr(bitval), _ptr(out),
                                              _stream(stream)))


def compact(store, slot_bytes, n_tensors, offsets, cache, cache_bytes, stream=None):
    _check(_lib.ibp_compact(_ptr(store), slot_bytes, n_tensors, _ptr(offsets), _ptr(cache),
                            cache_bytes, _stream(stream)))


def gather_decompress(store, store_bytes, slot_bytes, offsets, part_bits, n_tensors, ids, n_ids,
                      tensor_bytes, chunk_bytes, mask, bitval, out, stream=None):
    _check(_lib.ibp_gather_decompress(_ptr(store), store_bytes, slot_bytes, _ptr(offsets),
                                      _ptr(part_bits), n_tensors, _ptr(ids), n_ids, tensor_bytes,
                                      chunk_bytes, _ptr(mask), _ptr(bitval), _ptr(out),
                                      _stream(stream)))


GATHER_ROUTE_XCD = 1


def gather_decompress_ex(store, store_bytes, slot_bytes, offsets, part_bits, n_tensors, ids, n_ids,
                         tensor_bytes, chunk_bytes, mask, bitval, out, flags=0, stream=None):
    _check(_lib.ibp_gather_decompress_ex(_ptr(store), store_bytes, slot_bytes, _ptr(offsets),
                                         _ptr(part_bits), n_tensors, _ptr(ids), n_ids,
                                         tensor_bytes, chunk_bytes, _ptr(mask), _ptr(bitval),
                                         _ptr(out), flags, _stream(stream)))


MAX_SEGMENTS = 256


def gather_decompress_segments(store, store_bytes, slot_bytes, offsets, part_bits, n_tensors, ids,
                               seg_ids, tensor_bytes, chunk_bytes, masks, bitvals, out, flags=0,
                               stream=None):
    """seg_ids: host sequence of n_segments + 1 row offsets (numpy uint64 or a list);
    flags: 0 or GATHER_ROUTE_XCD."""
    seg = np.ascontiguousarray(np.asarray(seg_ids, dtype=np.uint64))
    _check(_lib.ibp_gather_decompress_segments(
        _ptr(store), store_bytes, slot_bytes, _ptr(offsets), _ptr(part_bits), n_tensors, _ptr(ids),
        seg.ctypes.data if seg.size else None, max(0, seg.size - 1), tensor_bytes, chunk_bytes,
        _ptr(masks), _ptr(bitvals), _ptr(out), flags, _stream(stream)))


def cache_offsets(lengths, select, n_tensors, offsets, stream=None):
    _check(_lib.ibp_cache_offsets(_ptr(lengths), _ptr(select), n_tensors, _ptr(offsets),
                                  _stream(stream)))


def cache_fill(store, slot_bytes, lengths, n_tensors, offsets, cache, cache_bytes, stream=None):
    _check(_lib.ibp_cache_fill(_ptr(store), slot_bytes, _ptr(lengths), n_tensors, _ptr(offsets),
                               _ptr(cache), cache_bytes, _stream(stream)))


def gather_decompress_hybrid(store, store_bytes, slot_bytes, cache, cache_bytes, offsets,
                             part_bits, n_tensors, ids, n_ids, tensor_bytes, chunk_bytes, mask,
                             bitval, out, stream=None):
    _check(_lib.ibp_gather_decompress_hybrid(_ptr(store), store_bytes, slot_bytes, _ptr(cache),
                                             cache_bytes, _ptr(offsets), _ptr(part_bits),
                                             n_tensors, _ptr(ids), n_ids, tensor_bytes,
                                             chunk_bytes, _ptr(mask), _ptr(bitval), _ptr(out),
                                             _stream(stream)))


RAW_ROUTE_XCD = 1


def raw_gather(src, row_stride, n_rows, ids, n_ids, row_bytes, out, flags=0, stream=None):
    _check(_lib.ibp_raw_gather(_ptr(src), row_stride, n_rows, _ptr(ids), n_ids, row_bytes,
                               _ptr(out), flags, _stream(stream)))


def stream_read(src, nbytes, never, sink, stream=None):
    _check(_lib.ibp_stream_read(_ptr(src), nbytes, never, _ptr(sink), _stream(stream)))


def stream_copy(src, dst, nbytes, stream=None):
    _check(_lib.ibp_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


def host_alloc(nbytes, flags=HOST_DEFAULT) -> int:
    p = _vp()
    _check(_lib.ibp_host_alloc(nbytes, flags, ctypes.byref(p)))
    return p.value


def host_free(ptr):
    _check(_lib.ibp_host_free(ptr))


class HostBuffer:
    """Pinned, GPU-mapped host memory from ibp_host_alloc, with a numpy view."""

    def __init__(self, nbytes, flags=HOST_DEFAULT):
        self.nbytes = int(nbytes)
        self.flags = flags
        self.ptr = host_alloc(self.nbytes, flags)
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        self.array = np.frombuffer(buf, dtype=np.uint8)

    def free(self):
        if self.ptr:
            self.array = None
            host_free(self.ptr)
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
