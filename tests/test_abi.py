"""The C ABI on the CPU: libibp.so loads, exports every function include/ibp.h
declares, and rejects bad arguments synchronously with the documented status
and a message, before any HIP call.  No compute call is made here."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ibp.h")


@pytest.fixture(scope="module")
def ibp():
    from host_transfer_amd import ibp as mod
    return mod


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ibp_\w+)\s*\(", text, flags=re.M))


def test_every_declared_function_is_exported(ibp):
    names = declared_functions()
    assert len(names) == 23, names
    out = subprocess.run(["nm", "-D", "--defined-only", ibp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ibp_\w+)$", out, flags=re.M))
    assert names <= exported, names - exported
    assert names == set(ibp.EXPORTED)


def test_version_and_chunks(ibp):
    assert ibp.version() == 1
    assert ibp.num_chunks(5732, 1024) == 6
    assert ibp.num_chunks(512, 1024) == 1
    assert ibp.num_chunks(10240, 256) == 40
    assert ibp.num_chunks(16384, 256) == 64
    for tb, cb, code in [(0, 256, ibp.ERR_SIZE), (6, 256, ibp.ERR_SIZE), (16388, 256, ibp.ERR_SIZE),
                         (512, 512, ibp.ERR_CHUNK), (512, 0, ibp.ERR_CHUNK)]:
        with pytest.raises(ibp.IbpError) as e:
            ibp.num_chunks(tb, cb)
        assert e.value.code == code and ibp.last_error()


P = 1 << 20  # a fake, suitably aligned address: validation never dereferences it


def _expect(ibp, code, fn, *args):
    with pytest.raises(ibp.IbpError) as e:
        fn(*args, stream=0)
    assert e.value.code == code, (e.value.code, ibp.last_error())
    assert ibp.last_error()


def test_build_metadata_validation(ibp):
    f = ibp.build_metadata
    _expect(ibp, ibp.ERR_NULL, f, 0, 512, None, 10, 512, 0.99, P, P, P)
    _expect(ibp, ibp.ERR_NULL, f, P, 512, None, 10, 512, 0.99, P, P, None)
    _expect(ibp, ibp.ERR_SIZE, f, P, 512, None, 10, 510, 0.99, P, P, P)
    _expect(ibp, ibp.ERR_SIZE, f, P, 512, None, 0, 512, 0.99, P, P, P)
    _expect(ibp, ibp.ERR_SIZE, f, P, 256, None, 10, 512, 0.99, P, P, P)
    for T in (0.4999, 1.0001, float("nan")):
        _expect(ibp, ibp.ERR_THRESHOLD, f, P, 512, None, 10, 512, T, P, P, P)
    _expect(ibp, ibp.ERR_ALIGN, f, P + 2, 512, None, 10, 512, 0.99, P, P, P)
    _expect(ibp, ibp.ERR_ALIGN, f, P, 512, P + 4, 10, 512, 0.99, P, P, P)


def test_build_metadata_noalloc_validation(ibp):
    f = ibp.build_metadata_noalloc
    _expect(ibp, ibp.ERR_NULL, f, 0, 512, None, 10, 512, 0.99, P, P)
    _expect(ibp, ibp.ERR_NULL, f, P, 512, None, 10, 512, 0.99, P, None)
    _expect(ibp, ibp.ERR_SIZE, f, P, 512, None, 10, 510, 0.99, P, P)
    _expect(ibp, ibp.ERR_SIZE, f, P, 1 << 20, None, 10, ibp.NOALLOC_MAX_TENSOR_BYTES + 4, 0.99,
            P, P)
    assert "16384" in ibp.last_error()
    _expect(ibp, ibp.ERR_SIZE, f, P, 512, None, 0, 512, 0.99, P, P)
    _expect(ibp, ibp.ERR_SIZE, f, P, 256, None, 10, 512, 0.99, P, P)
    for T in (0.4999, 1.0001, float("nan")):
        _expect(ibp, ibp.ERR_THRESHOLD, f, P, 512, None, 10, 512, T, P, P)
    _expect(ibp, ibp.ERR_ALIGN, f, P + 2, 512, None, 10, 512, 0.99, P, P)
    _expect(ibp, ibp.ERR_ALIGN, f, P, 512, P + 4, 10, 512, 0.99, P, P)


def test_compress_validation(ibp):
    f = ibp.compress
    ok = [P, 512, 10, 0, 10, 512, 256, P, P, P, 512, P, P]

    def args(**kw):
        a = list(ok)
        names = ["rows", "stride", "n", "first", "nt", "tb", "cb", "mask", "bv", "store", "slot",
                 "pb", "lens"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return a
    _expect(ibp, ibp.ERR_NULL, f, *args(store=0))
    _expect(ibp, ibp.ERR_NULL, f, *args(pb=0))
    _expect(ibp, ibp.ERR_CHUNK, f, *args(cb=128))
    _expect(ibp, ibp.ERR_SIZE, f, *args(first=5, n=6))
    _expect(ibp, ibp.ERR_SIZE, f, *args(slot=520))
    _expect(ibp, ibp.ERR_SIZE, f, *args(slot=496))
    _expect(ibp, ibp.ERR_SIZE, f, *args(stride=508))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(store=P + 8))
    # ibp_compress_segments: the host segment tables
    fs = ibp.compress_segments

    def seg(row, first, count, nt=10, stride=512, slot=512, store=P):
        return [P, stride, row, first, count, nt, 512, 256, P, P, store, slot, P, P]
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([], [], []))                 # no segment
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0] * 257, [0] * 257, [1] * 257))
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0, 5], [0, 8], [4, 3]))    # 8 + 3 > 10 tensors
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0], [0], [4], stride=0))
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0], [0], [4], slot=520))
    _expect(ibp, ibp.ERR_ALIGN, fs, *seg([0], [0], [4], store=P + 8))
    _expect(ibp, ibp.ERR_NULL, fs, *seg([0], [0], [4], store=0))


def test_gather_validation(ibp):
    f = ibp.gather_decompress
    ok = [P, 10 * 512, 512, None, P, 10, P, 4, 512, 256, P, P, P]

    def args(**kw):
        a = list(ok)
        names = ["store", "sbytes", "slot", "offs", "pb", "nt", "ids", "nids", "tb", "cb", "mask",
                 "bv", "out"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return a
    _expect(ibp, ibp.ERR_NULL, f, *args(ids=0))
    _expect(ibp, ibp.ERR_NULL, f, *args(out=0))
    _expect(ibp, ibp.ERR_SIZE, f, *args(sbytes=10 * 512 - 1))
    _expect(ibp, ibp.ERR_SIZE, f, *args(tb=20000))
    _expect(ibp, ibp.ERR_CHUNK, f, *args(cb=2048))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(out=P + 4))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(ids=P + 4))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(offs=P + 4))
    # the flags of ibp_gather_decompress_ex
    fx = ibp.gather_decompress_ex
    _expect(ibp, ibp.ERR_FLAGS, fx, *args(), 2)
    _expect(ibp, ibp.ERR_FLAGS, fx, *args(offs=P), ibp.GATHER_ROUTE_XCD)
    _expect(ibp, ibp.ERR_SIZE, fx, *args(nids=1 << 32), ibp.GATHER_ROUTE_XCD)
    _expect(ibp, ibp.ERR_SIZE, fx, *args(sbytes=10 * 512 - 1), ibp.GATHER_ROUTE_XCD)
    # ibp_gather_decompress_segments: the host segment table
    fs = ibp.gather_decompress_segments

    def seg(seg_ids, **kw):
        a = args(**kw)
        return a[:7] + [seg_ids] + a[8:]
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0]))                     # no segment
    _expect(ibp, ibp.ERR_SIZE, fs, *seg(list(range(258))))        # 257 segments
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([1, 4]))                  # must start at 0
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0, 5, 3]))               # decreasing
    _expect(ibp, ibp.ERR_NULL, fs, *seg([0, 4], ids=0))
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0, 4], sbytes=10 * 512 - 1))
    _expect(ibp, ibp.ERR_ALIGN, fs, *seg([0, 4], out=P + 4))
    _expect(ibp, ibp.ERR_CHUNK, fs, *seg([0, 4], cb=2048))
    _expect(ibp, ibp.ERR_FLAGS, fs, *seg([0, 4]), 2)
    _expect(ibp, ibp.ERR_FLAGS, fs, *seg([0, 4], offs=P), ibp.GATHER_ROUTE_XCD)
    _expect(ibp, ibp.ERR_SIZE, fs, *seg([0, 1 << 31, 1 << 32]), ibp.GATHER_ROUTE_XCD)


def test_other_validation(ibp):
    _expect(ibp, ibp.ERR_NULL, ibp.compact_offsets, 0, 10, P)
    _expect(ibp, ibp.ERR_NULL, ibp.compact, P, 512, 10, P, 0, 100)
    _expect(ibp, ibp.ERR_SIZE, ibp.compact, P, 500, 10, P, P, 100)
    _expect(ibp, ibp.ERR_SIZE, ibp.raw_gather, P, 512, 10, P, 4, 514, P)
    _expect(ibp, ibp.ERR_SIZE, ibp.raw_gather, P, 514, 10, P, 4, 512, P)
    _expect(ibp, ibp.ERR_ALIGN, ibp.raw_gather, P + 2, 512, 10, P, 4, 512, P)
    _expect(ibp, ibp.ERR_FLAGS, ibp.raw_gather, P, 512, 10, P, 4, 512, P, 2)
    _expect(ibp, ibp.ERR_SIZE, ibp.raw_gather, P, 512, 1 << 56, P, 4, 512, P)
    _expect(ibp, ibp.ERR_SIZE, ibp.raw_gather, P, 512, 10, P, 1 << 56, 512, P)
    _expect(ibp, ibp.ERR_SIZE, ibp.raw_gather, P, 512, 10, P, 1 << 32, 512, P,
            ibp.RAW_ROUTE_XCD)
    _expect(ibp, ibp.ERR_SIZE, ibp.stream_read, P, 100, 0, P)
    _expect(ibp, ibp.ERR_NULL, ibp.stream_copy, 0, P, 1024)
    _expect(ibp, ibp.ERR_NULL, ibp.stream_copy, P, 0, 1024)
    _expect(ibp, ibp.ERR_SIZE, ibp.stream_copy, P, P + 4096, 100)
    _expect(ibp, ibp.ERR_ALIGN, ibp.stream_copy, P + 8, P + 4096, 1024)
    _expect(ibp, ibp.ERR_ALIGN, ibp.stream_copy, P, P + 4104, 1024)
    _expect(ibp, ibp.ERR_SIZE, ibp.stream_copy, P, P + 512, 1024)   # overlap
    _expect(ibp, ibp.ERR_SIZE, ibp.stream_copy, P + 512, P, 1024)   # overlap
    with pytest.raises(ibp.IbpError) as e:
        ibp.host_alloc(1024, 7)
    assert e.value.code == ibp.ERR_FLAGS
    with pytest.raises(ibp.IbpError) as e:
        ibp.host_alloc(0)
    assert e.value.code == ibp.ERR_SIZE
    ibp.host_free(0)


def test_cache_and_hybrid_validation(ibp):
    # ibp_cache_offsets / ibp_cache_fill (partial cache)
    _expect(ibp, ibp.ERR_NULL, ibp.cache_offsets, P, 0, 10, P)
    _expect(ibp, ibp.ERR_NULL, ibp.cache_offsets, 0, P, 10, P)
    _expect(ibp, ibp.ERR_ALIGN, ibp.cache_offsets, P, P, 10, P + 4)
    _expect(ibp, ibp.ERR_ALIGN, ibp.cache_offsets, P + 2, P, 10, P)
    _expect(ibp, ibp.ERR_NULL, ibp.cache_fill, P, 512, P, 10, P, 0, 100)
    _expect(ibp, ibp.ERR_SIZE, ibp.cache_fill, P, 500, P, 10, P, P, 100)
    _expect(ibp, ibp.ERR_SIZE, ibp.cache_fill, P, 0, P, 10, P, P, 100)
    _expect(ibp, ibp.ERR_ALIGN, ibp.cache_fill, P, 512, P, 10, P, P + 8, 100)
    _expect(ibp, ibp.ERR_ALIGN, ibp.cache_fill, P, 512, P, 10, P + 4, P, 100)
    # ibp_gather_decompress_hybrid
    f = ibp.gather_decompress_hybrid
    ok = [P, 10 * 512, 512, P, 4096, P, P, 10, P, 4, 512, 256, P, P, P]
    names = ["store", "sbytes", "slot", "cache", "cbytes", "offs", "pb", "nt", "ids", "nids",
             "tb", "cb", "mask", "bv", "out"]

    def args(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return a
    _expect(ibp, ibp.ERR_NULL, f, *args(cache=0))
    _expect(ibp, ibp.ERR_NULL, f, *args(offs=0))
    _expect(ibp, ibp.ERR_NULL, f, *args(store=0))
    _expect(ibp, ibp.ERR_SIZE, f, *args(sbytes=10 * 512 - 1))
    _expect(ibp, ibp.ERR_SIZE, f, *args(slot=500))
    _expect(ibp, ibp.ERR_SIZE, f, *args(tb=6))
    _expect(ibp, ibp.ERR_CHUNK, f, *args(cb=100))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(cache=P + 8))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(offs=P + 4))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(out=P + 4))


def test_indexed_cache_validation(ibp):
    fa = ibp.compact_offsets_aligned
    _expect(ibp, ibp.ERR_NULL, fa, 0, 10, 128, P)
    for bad in (0, 8, 96, 8192):
        _expect(ibp, ibp.ERR_ALIGN, fa, P, 10, bad, P)
    _expect(ibp, ibp.ERR_ALIGN, fa, P, 10, 128, P + 4)
    fi = ibp.cache_index
    _expect(ibp, ibp.ERR_NULL, fi, 0, 10, P)
    _expect(ibp, ibp.ERR_SIZE, fi, P, 1 << 32, P)
    _expect(ibp, ibp.ERR_ALIGN, fi, P, 10, P + 4)
    f = ibp.gather_decompress_indexed
    ok = [P, 1 << 20, 128, P, 10, P, 4, 512, 1024, P, P, P]
    names = ["cache", "cbytes", "align", "index", "nt", "ids", "nids", "tb", "cb", "mask", "bv",
             "out"]

    def args(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[names.index(k)] = v
        return a
    _expect(ibp, ibp.ERR_NULL, f, *args(index=0))
    _expect(ibp, ibp.ERR_NULL, f, *args(cache=0))
    _expect(ibp, ibp.ERR_CHUNK, f, *args(cb=256))            # two chunks
    _expect(ibp, ibp.ERR_SIZE, f, *args(tb=768, cb=1024))    # no kernel shape for 768 B
    _expect(ibp, ibp.ERR_ALIGN, f, *args(align=100))
    _expect(ibp, ibp.ERR_SIZE, f, *args(nt=1 << 32))
    _expect(ibp, ibp.ERR_SIZE, f, *args(cache=(1 << 48) - 4096, cbytes=8192))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(out=P + 4))
    _expect(ibp, ibp.ERR_ALIGN, f, *args(index=P + 4))


def test_valid_call_without_a_device_reports_hip_error(ibp):
    """With no GPU visible, a call whose arguments are valid fails with
    IBP_ERR_HIP (and the HIP runtime's message) instead of crashing.  The
    calls used enqueue nothing even when a device is present (zero rows or
    bytes), so the test is safe to run anywhere; it only asserts the error
    where no device exists."""
    import torch
    has_device = torch.cuda.device_count() > 0
    calls = [
        (ibp.gather_decompress, (P, 10 * 512, 512, None, P, 10, P, 0, 512, 256, P, P, P)),
        (ibp.raw_gather, (P, 512, 10, P, 0, 512, P)),
        (ibp.stream_read, (P, 0, 0, P)),
        (ibp.stream_copy, (P, P + 4096, 0)),
    ]
    for fn, a in calls:
        if has_device:
            fn(*a, stream=0)
            continue
        with pytest.raises(ibp.IbpError) as e:
            fn(*a, stream=0)
        assert e.value.code == ibp.ERR_HIP, (fn.__name__, e.value.code, ibp.last_error())
        assert "HIP error" in ibp.last_error()
