"""Helpers of the GPU parity tests: run every stage of libibp.so on one input
and compare it with the CPU oracle, bit for bit.

Only host-side checks and marshalling live here; the GPU work is done by the
library through its C ABI (host_transfer_amd.ibp).
"""
import numpy as np
import torch

from host_transfer_amd import ibp
from oracle import oracle as O


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def log(msg):
    print(msg, flush=True)


class Result:
    pass


def gpu_metadata(rows, threshold, sample_ids=None):
    """GPU Mask/Bitval/counts for (N, B) uint8 rows."""
    rows = np.ascontiguousarray(rows)
    N, B = rows.shape
    d_rows = dev(rows)
    d_ids = None if sample_ids is None else dev(np.asarray(sample_ids, np.int64))
    n = N if sample_ids is None else len(sample_ids)
    mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    bitval = torch.zeros_like(mask)
    counts = torch.full((8 * B,), 7, dtype=torch.int32, device="cuda")
    ibp.build_metadata(d_rows, B, d_ids, n, B, threshold, mask, bitval, counts)
    return (host(mask).view(np.uint32), host(bitval).view(np.uint32),
            host(counts).view(np.uint32))


def check_metadata(rows, threshold, sample_ids=None):
    m, v, counts = gpu_metadata(rows, threshold, sample_ids)
    om, ov, ones = O.build_metadata(rows, threshold, sample_ids=sample_ids, return_ones=True)
    assert (counts == ones.astype(np.uint32)).all(), "per-bit counts differ"
    assert (m == om).all(), "Mask differs"
    assert (v == ov).all(), "Bitval differs"
    return om, ov


def gpu_compress(rows, mask, bitval, C, slot, n_tensors=None, first=0, store=None, part=None,
                 lengths=None, pinned=False):
    """Compresses rows on the GPU into a device (or host-mapped) store."""
    rows = np.ascontiguousarray(rows)
    n, B = rows.shape
    n_tensors = n_tensors or first + n
    n_c = ibp.num_chunks(B, C)
    if store is None:
        if pinned:
            store = ibp.HostBuffer(n_tensors * slot)
            store.array[:] = 0xA5
        else:
            store = torch.full((n_tensors * slot,), 0xA5 - 256, dtype=torch.int8, device="cuda")
    if part is None:
        part = torch.zeros((n_tensors * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    if lengths is None:
        lengths = torch.zeros(n_tensors, dtype=torch.int32, device="cuda")
    ibp.compress(dev(rows), B, n, first, n_tensors, B, C, dev(mask), dev(bitval), store, slot, part,
                 lengths)
    torch.cuda.synchronize()
    return store, part, lengths


def store_bytes(store):
    if isinstance(store, ibp.HostBuffer):
        return store.array
    return host(store).view(np.uint8)


def check_store(rows, mask, bitval, C, slot, store, part, lengths, first=0, n_tensors=None):
    """GPU store/bitmap/lengths against the oracle's, on the payload bytes."""
    n, B = rows.shape
    n_tensors = n_tensors or first + n
    n_c = ibp.num_chunks(B, C)
    o_store, o_part, o_len = O.compress(rows, mask, bitval, C, slot_bytes=slot,
                                        first_tensor=first, n_tensors=n_tensors)
    g_len = host(lengths).view(np.uint32)[first:first + n]
    assert (g_len == o_len).all(), "payload lengths differ"
    nbits = n_tensors * n_c
    g_bits = np.unpackbits(host(part).view(np.uint8), bitorder="little")[:nbits]
    o_bits = np.unpackbits(o_part.view(np.uint8), bitorder="little")[:nbits]
    lo, hi = first * n_c, (first + n) * n_c
    assert (g_bits[lo:hi] == o_bits[lo:hi]).all(), "participation bits differ"
    g = store_bytes(store).reshape(n_tensors, slot)[first:first + n]
    o = o_store.reshape(n_tensors, slot)[first:first + n]
    valid = np.arange(slot)[None, :] < o_len[:, None].astype(np.int64)
    assert (g[valid] == o[valid]).all(), "payload bytes differ"
    # bytes between len_t and the next 16 B boundary are written as zeros
    pad = (np.arange(slot)[None, :] >= o_len[:, None]) & \
          (np.arange(slot)[None, :] < ((o_len[:, None] + 15) // 16 * 16))
    assert not g[pad].any(), "padding after the payload is not zero"
    return o_store, o_part, o_len


ROUTE = 1  # IBP_GATHER_ROUTE_XCD


def gpu_gather(store, store_nbytes, slot, offsets, part, n_tensors, ids, B, C, mask, bitval,
               flags=0):
    """ibp_gather_decompress (flags == 0) or ibp_gather_decompress_ex(flags)."""
    ids = np.ascontiguousarray(ids, np.int64)
    out = torch.full((max(1, len(ids)) * B,), -1, dtype=torch.int8, device="cuda")
    d_ids = dev(ids) if len(ids) else torch.zeros(1, dtype=torch.int64, device="cuda")
    if flags:
        ibp.gather_decompress_ex(store, store_nbytes, slot, offsets, part, n_tensors, d_ids,
                                 len(ids), B, C, dev(mask), dev(bitval), out, flags)
    else:
        ibp.gather_decompress(store, store_nbytes, slot, offsets, part, n_tensors, d_ids, len(ids),
                              B, C, dev(mask), dev(bitval), out)
    return host(out).view(np.uint8)[:len(ids) * B].reshape(len(ids), B)


def expected_rows(rows, ids, first=0):
    ids = np.asarray(ids, np.int64)
    n = rows.shape[0]
    out = np.zeros((len(ids), rows.shape[1]), np.uint8)
    ok = (ids >= first) & (ids < first + n)
    out[ok] = rows[ids[ok] - first]
    return out
