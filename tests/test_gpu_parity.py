"""GPU parity: every stage of libibp.so against the CPU oracle, bit for bit.

Inputs are the seeded workloads at sizes the oracle finishes in seconds
(several tiles and a ragged tail each), random tensors covering every thread
grouping (tiles of 1..4 words per lane, groups of 64..1024 threads with 1..6
words per thread, 1..64 chunks), and the degenerate cases of the method.
Gathers from slots run both plain and with rows routed to XCDs.  All GPU work
goes through the C ABI.
"""
import numpy as np
import pytest
import torch

from host_transfer_amd import workloads as W
from tests import gpu_case as G

pytestmark = pytest.mark.gpu


def full_roundtrip(name, rows, C, T, sample_ids=None, slot=None, pinned=False, batches=None,
                   rng=None):
    """Metadata -> compress -> gather (slots) -> compact -> gather (cache)."""
    rng = rng or np.random.default_rng(7)
    n, B = rows.shape
    slot = slot or (B + 127) // 128 * 128
    G.log(f"[parity] {name}: n={n} B={B} C={C} T={T} slot={slot} pinned={pinned}")
    mask, bitval = G.check_metadata(rows, T, sample_ids)
    store, part, lengths = G.gpu_compress(rows, mask, bitval, C, slot, pinned=pinned)
    o_store, o_part, o_len = G.check_store(rows, mask, bitval, C, slot, store, part, lengths)
    batches = batches or [rng.integers(0, n, 777), np.arange(n)[::-1].copy(), np.array([0, n - 1, 0])]
    for ids in batches:
        ora = O_gather(o_store, o_part, n, ids, B, C, mask, bitval, slot)
        want = G.expected_rows(rows, ids)
        for flags in (0, G.ROUTE):  # plain, and rows routed to XCDs by tensor
            got = G.gpu_gather(store, n * slot, slot, None, part, n, ids, B, C, mask, bitval, flags)
            assert (got == want).all(), f"{name}: gather from slots is not the original rows ({flags})"
            assert (got == ora).all(), f"{name}: gather differs from the oracle ({flags})"
    # compacted HBM cache
    offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    from host_transfer_amd import ibp
    ibp.compact_offsets(lengths, n, offsets)
    g_off = G.host(offsets).view(np.uint64)
    from oracle import oracle as O
    o_off, o_cache = O.compact(o_store, slot, o_len)
    assert (g_off == o_off).all(), f"{name}: cache offsets differ"
    total = int(g_off[-1])
    cache = torch.full((max(total, 16),), 0x3C, dtype=torch.int8, device="cuda")
    ibp.compact(store, slot, n, offsets, cache, total)
    g_cache = G.host(cache).view(np.uint8)[:total]
    assert (g_cache == o_cache).all(), f"{name}: cache bytes differ"
    ids = batches[0]
    got = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
    assert (got == G.expected_rows(rows, ids)).all(), f"{name}: gather from the cache differs"
    return mask, bitval, o_len


def O_gather(store, part, n, ids, B, C, mask, bitval, slot):
    from oracle import oracle as O
    return O.gather_decompress(store, part, n, ids, B, C, mask, bitval, slot_bytes=slot)


# ------------------------------------------------------------ the workloads

def test_tiny_full():
    w = W.WORKLOADS["tiny"]
    rows = W.rows(w)
    mask, _, lens = full_roundtrip("tiny", rows, w.chunk_bytes, w.threshold,
                                   batches=[W.batch_ids(w, 0), W.batch_ids(w, 1)[:1000],
                                            np.arange(w.n_tensors)])
    assert (mask == 0x78000000).all()


@pytest.mark.parametrize("T", [0.99, 0.95])
def test_sparse_gnn(T):
    w = W.WORKLOADS["sparse_gnn"].scaled(3000)
    rows = W.rows(w)
    full_roundtrip(f"sparse_gnn T={T}", rows, w.chunk_bytes, T, sample_ids=W.sample_ids(
        W.WORKLOADS["sparse_gnn"].scaled(3000 * 40))[:300] % 3000)


def test_dense_gnn_pinned():
    w = W.WORKLOADS["dense_gnn"].scaled(5000)
    rows = W.rows(w)
    full_roundtrip("dense_gnn", rows, w.chunk_bytes, w.threshold, pinned=True)


def test_dlrm_pinned():
    for key, n in (("dlrm_1k", 4000), ("dlrm_2k", 2500)):
        w = W.WORKLOADS[key].scaled(n)
        rows = W.rows(w)
        full_roundtrip(key, rows, w.chunk_bytes, w.threshold, pinned=True)


def test_kv_pair():
    w = W.WORKLOADS["kv_opt13b"]
    prefill = W.kv_prefill_rows(w, 5, 3000)
    rows = W.rows(w, 5 * 2560, 2560)
    # Mask from the prefill sample, applied to the pair's decode rows
    mask, bitval = G.check_metadata(prefill, w.threshold)
    slot = w.slot_bytes
    store, part, lengths = G.gpu_compress(rows, mask, bitval, w.chunk_bytes, slot, pinned=True)
    o_store, o_part, _ = G.check_store(rows, mask, bitval, w.chunk_bytes, slot, store, part,
                                       lengths)
    ids = np.arange(2560)
    got = G.gpu_gather(store, 2560 * slot, slot, None, part, 2560, ids, w.tensor_bytes,
                       w.chunk_bytes, mask, bitval)
    assert (got == rows).all()


# ------------------------------------------------------------ geometry sweep

SHAPES = [(4, 256), (12, 256), (256, 256), (260, 256), (508, 1024), (768, 256), (1024, 256),
          (1024, 1024), (1028, 256), (2052, 1024),
          (4100, 4096), (5732, 1024), (8196, 256), (10240, 256), (16384, 256), (16384, 4096)]


@pytest.mark.parametrize("B,C", SHAPES)
def test_geometry_sweep(B, C):
    rng = np.random.default_rng(B * 7 + C)
    n = 300 if B <= 4096 else 120
    x = (rng.standard_normal((n, B // 4)) * rng.uniform(0.05, 3.0, B // 4)).astype(np.float32)
    x[rng.random((n, B // 4)) < 0.01] = 0.0
    rows = x.view(np.uint8)
    full_roundtrip(f"sweep B={B} C={C}", rows, C, 0.9, batches=[rng.integers(0, n, 257),
                                                                np.array([n - 1])])


@pytest.mark.parametrize("B,C,pinned", [(1028, 256, False), (2052, 1024, False),
                                         (5732, 1024, True), (16384, 4096, True)])
def test_group_first_payload_prefix(B, C, pinned):
    """Group kernel, slot mode: each group requests its first tensor's
    guaranteed payload prefix (ceil(K / 128) units, K = kept bits) before the
    chunk scan and the rest after it.  Batches shorter than the number of
    groups make every row a group's first row.  Tensors with every chunk
    packed, one chunk whole, every chunk whole, and invalid ids; K is not a
    multiple of 128 except for B = 16384."""
    rng = np.random.default_rng(B + C)
    n, W = 240, B // 4
    # bits 23..31 equal in every word (a fixed top byte, bit 23 clear): K = 23 W
    x = rng.integers(0, 1 << 23, (n, W), dtype=np.uint32) | np.uint32(0x3F000000)
    wpc = C // 4
    x[1:5, min(wpc, W - 1)] ^= np.uint32(1 << 30)   # one chunk whole
    for c in range(0, W, wpc):                      # every chunk whole
        x[5:9, c] ^= np.uint32(1 << 30)
    rows = x.view(np.uint8)
    first = np.array([-1, 5, 1, 0, n, 6, 2, 10, 3, 7, 11, 4, 8, 12, 1 << 40, 239])
    mixed = rng.integers(-3, n + 3, 3000)
    mask, _, lens = full_roundtrip(f"first payload B={B} C={C}", rows, C, 0.9, pinned=pinned,
                                   batches=[mixed, first, np.array([5, 6, 7, 8])])
    K = 32 * W - int(np.unpackbits(mask.view(np.uint8)).sum())
    assert K == 23 * W, "the Mask should keep bits 0..22 of every word"
    n_c = -(-B // C)
    assert lens[0] == -(-K // 8) and lens[5] == B and (lens[1] > lens[0]) and (lens[1] < B or n_c == 1)


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(case):
    """Seeded random shapes across the kernel choices: tensor size (tile,
    direct or group kernel), chunk size, threshold, value law, batch size
    (short and long launches), ids with repeats and invalid entries; slots
    (device or pinned) and the compacted cache, against the oracle."""
    from host_transfer_amd import ibp
    from oracle import oracle as O
    rng = np.random.default_rng(1000 + case)
    W_ = int(rng.choice([1, 17, 64, 100, 128, 200, 256, 257, 700, 1433, 2560, 4096]))
    B = 4 * W_
    C = int(rng.choice([256, 1024, 4096]))
    T = float(rng.choice([0.6, 0.9, 0.99, 1.0]))
    n = int(min(1500, max(8, 2_000_000 // B)))
    law = rng.integers(0, 3)
    if law == 0:
        x = (rng.standard_normal((n, W_)) * rng.uniform(0.05, 2.0, W_)).astype(np.float32)
    elif law == 1:
        x = (rng.random((n, W_)) < 0.03).astype(np.float32)
    else:
        x = rng.uniform(-0.05, 0.05, (n, W_)).astype(np.float32)
    rows = x.view(np.uint8).reshape(n, B)
    slot = (B + 127) // 128 * 128
    pinned = bool(rng.integers(0, 2))
    nb = int(rng.choice([1, 333, 4096, 40000 if B <= 1024 else 3000]))
    ids = rng.integers(-2, n + 2, nb)
    G.log(f"[parity] random case {case}: B={B} C={C} T={T} n={n} ids={nb} pinned={pinned}")
    mask, bitval = G.check_metadata(rows, T)
    store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot, pinned=pinned)
    o_store, o_part, o_len = G.check_store(rows, mask, bitval, C, slot, store, part, lens)
    want = G.expected_rows(rows, ids)
    got = G.gpu_gather(store, n * slot, slot, None, part, n, ids, B, C, mask, bitval)
    assert (got == want).all(), "slots"
    ok = (ids >= 0) & (ids < n)
    ora = O.gather_decompress(o_store, o_part, n, ids[ok], B, C, mask, bitval, slot_bytes=slot)
    assert (got[ok] == ora).all(), "oracle"
    offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets(lens, n, offsets)
    total = int(offsets[-1].item())
    cache = torch.zeros(max(total, 16), dtype=torch.uint8, device="cuda")
    ibp.compact(store, slot, n, offsets, cache, total)
    got = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
    assert (got == want).all(), "cache"
    if pinned:
        store.free()


# ------------------------------------------------------------ degenerate cases

def test_mask_zero_and_all_ones():
    from host_transfer_amd import ibp
    rng = np.random.default_rng(3)
    B, C, n = 1024, 256, 200
    rows = rng.integers(0, 256, (n, B), dtype=np.uint8)
    zero = np.zeros(B // 4, np.uint32)
    store, part, lens = G.gpu_compress(rows, zero, zero, C, B)
    G.check_store(rows, zero, zero, C, B, store, part, lens)
    assert (G.host(lens) == B).all() and not G.host(part).any()
    ids = rng.integers(0, n, 99)
    got = G.gpu_gather(store, n * B, B, None, part, n, ids, B, C, zero, zero)
    assert (got == rows[ids]).all()
    # identical tensors: Mask all ones, empty payloads, Bitval restores them
    same = np.tile(rows[:1], (50, 1))
    mask, bitval = G.check_metadata(same, 0.99)
    assert (mask == 0xFFFFFFFF).all()
    store, part, lens = G.gpu_compress(same, mask, bitval, C, B)
    assert not G.host(lens).any()
    got = G.gpu_gather(store, 50 * B, B, None, part, 50, [0, 49, 7], B, C, mask, bitval)
    assert (got == same[:3]).all()


# One-chunk tensors of 256 B, 512 B or 1 KB gathered from an HBM cache through
# the offset table take k_gather_cache (any batch size; the batches here fit
# one round of waves with 1, 2 or 4 steps each, and test_indexed_cache and the
# full-size tests take its grid-stride form).  Ragged tails, repeated and invalid ids, tensors that do and
# do not participate, and both degenerate Masks (all zero: every tensor whole;
# all ones: empty payloads).
STREAM_CASES = [("dense_gnn", 512, 1024, 3000, 40037), ("dlrm_1k", 1024, 4096, 2000, 20011),
                ("tiny-256", 256, 256, 2500, 70001), ("dense_gnn", 512, 4096, 1500, 33000)]


@pytest.mark.parametrize("key,B,C,n,nb", STREAM_CASES)
@pytest.mark.parametrize("law", ["workload", "mask0", "mask1"])
def test_stream_cache_large_batches(key, B, C, n, nb, law):
    from host_transfer_amd import ibp
    from oracle import oracle as O
    rng = np.random.default_rng(B + n + nb)
    if law == "workload" and key != "tiny-256":
        w = W.WORKLOADS[key].scaled(n)
        rows, T = W.rows(w), w.threshold
    elif law == "workload":
        rows = (rng.standard_normal((n, B // 4)) * 0.1).astype(np.float32).view(np.uint8)
        T = 0.99
    elif law == "mask0":
        rows, T = rng.integers(0, 256, (n, B), dtype=np.uint8), 1.0
    else:
        rows, T = np.tile(rng.integers(0, 256, (1, B), dtype=np.uint8), (n, 1)), 0.99
    slot = (B + 127) // 128 * 128
    G.log(f"[parity] one-chunk cache gather: {key} {law} B={B} C={C} n={n} ids={nb}")
    mask, bitval = G.check_metadata(rows, T)
    if law == "mask0":
        assert not mask.any()
    if law == "mask1":
        assert (mask == 0xFFFFFFFF).all()
    store, part, lengths = G.gpu_compress(rows, mask, bitval, C, slot)
    o_store, o_part, o_len = G.check_store(rows, mask, bitval, C, slot, store, part, lengths)
    offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets(lengths, n, offsets)
    total = int(G.host(offsets)[-1])
    cache = torch.full((max(total, 16),), 0x3C, dtype=torch.int8, device="cuda")
    ibp.compact(store, slot, n, offsets, cache, total)
    ids = rng.integers(0, n, nb)
    ids[rng.integers(0, nb, 64)] = rng.choice([-1, n, n + 7, 1 << 40], 64)
    ids[-1] = n - 1
    got = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
    want = O.gather_decompress(o_store, o_part, n, ids, B, C, mask, bitval, slot_bytes=slot)
    assert (got == want).all(), f"{key} {law}: cache gather differs from the oracle"
    assert (got == G.expected_rows(rows, ids)).all()
    # entries marked IBP_NOT_CACHED give zero rows, in large and short batches
    gone = rng.choice(n, 16, replace=False)
    offsets[torch.from_numpy(gone).cuda()] = -1
    hit = np.isin(ids, gone)
    want[hit] = 0
    got = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
    assert (got == want).all(), f"{key} {law}: uncached entries"
    short = np.concatenate([ids[:500], gone[:4]])
    got = G.gpu_gather(cache, total, 0, offsets, part, n, short, B, C, mask, bitval)
    assert (got == np.concatenate([want[:500], np.zeros((4, B), np.uint8)])).all()


def test_batch_edges_and_invalid_ids():
    w = W.WORKLOADS["tiny"].scaled(1000)
    rows = W.rows(w)
    B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    mask, bitval = G.check_metadata(rows, w.threshold)
    store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot)
    for flags in (0, G.ROUTE):
        for nb in (0, 1, 63, 64, 65, 255, 256, 257):
            ids = (np.arange(nb) * 37) % 1000
            got = G.gpu_gather(store, 1000 * slot, slot, None, part, 1000, ids, B, C, mask, bitval,
                               flags)
            assert (got == rows[ids]).all(), (nb, flags)
        ids = np.array([5, -1, 1000, 999, 1 << 40, 5, 5])
        got = G.gpu_gather(store, 1000 * slot, slot, None, part, 1000, ids, B, C, mask, bitval,
                           flags)
        assert (got == G.expected_rows(rows, ids)).all()
        assert not got[[1, 2, 4]].any()


@pytest.mark.parametrize("flags", [0, 1, 2])  # IBP_HOST_DEFAULT, _COHERENT, _NONCOHERENT
def test_host_store_flags(flags):
    """Compression into, and gathers from, pinned stores of every host
    allocation kind (the GPU writes and reads them over PCIe)."""
    from host_transfer_amd import ibp
    w = W.WORKLOADS["sparse_gnn"].scaled(800)
    rows = W.rows(w)
    B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    mask, bitval = G.check_metadata(rows, 0.95)
    store = ibp.HostBuffer(800 * slot, flags)
    store.array[:] = 0xA5
    G.log(f"[parity] host store flags {flags}")
    store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot, store=store)
    G.check_store(rows, mask, bitval, C, slot, store, part, lens)
    ids = np.random.default_rng(flags).integers(0, 800, 1000)
    for route in (0, G.ROUTE):
        got = G.gpu_gather(store, 800 * slot, slot, None, part, 800, ids, B, C, mask, bitval, route)
        assert (got == rows[ids]).all(), (flags, route)
    store.free()


def test_routed_zipf_repeats():
    """Routed gathers of a batch that repeats a few tensors many times (the
    case routing is for), tile and group kernels, device and pinned slots."""
    rng = np.random.default_rng(5)
    for key, n in (("dense_gnn", 3000), ("dlrm_2k", 1200), ("kv_opt13b", 300)):
        w = W.WORKLOADS[key].scaled(n)
        rows = W.rows(w, 0, n)
        B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
        mask, bitval = G.check_metadata(rows, w.threshold)
        for pinned in (False, True):
            store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot, pinned=pinned)
            hot = rng.integers(0, n, 7)
            ids = np.where(rng.random(5000) < 0.6, hot[rng.integers(0, 7, 5000)],
                           rng.integers(-3, n + 3, 5000))
            G.log(f"[parity] routed repeats {key}: n={n} pinned={pinned}")
            got = G.gpu_gather(store, n * slot, slot, None, part, n, ids, B, C, mask, bitval,
                               G.ROUTE)
            assert (got == G.expected_rows(rows, ids)).all(), key
        # one tensor in every row (spread over all XCDs), and invalid ids whose
        # low 32 bits equal a valid id's
        one = np.full(3001, n // 2)
        coll = np.where(np.arange(3001) % 3 == 0, n // 2 + (1 << 32), one)
        for ids in (one, coll):
            G.log(f"[parity] routed single tensor {key}: {len(ids)} ids")
            got = G.gpu_gather(store, n * slot, slot, None, part, n, ids, B, C, mask, bitval,
                               G.ROUTE)
            assert (got == G.expected_rows(rows, ids)).all(), key


def test_side_stream_and_graph_replay():
    """Gathers launched on a side stream, and gathers captured in a HIP graph
    and replayed with the captured ids buffer refilled in between (eager work
    and synchronisations between replays): tile kernel (dense_gnn) and group
    kernel (sparse_gnn), from slots and from a compacted cache.  Every replay
    is checked against an eager launch of the same ids and the original rows."""
    from host_transfer_amd import ibp
    rng = np.random.default_rng(11)
    for key, n in (("dense_gnn", 3000), ("sparse_gnn", 1500)):
        w = W.WORKLOADS[key].scaled(n)
        rows = W.rows(w)
        B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
        mask, bitval = G.check_metadata(rows, w.threshold)
        store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot)
        offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
        ibp.compact_offsets(lens, n, offsets)
        total = int(offsets[-1].item())
        cache = torch.zeros(max(total, 16), dtype=torch.uint8, device="cuda")
        ibp.compact(store, slot, n, offsets, cache, total)
        d_mask, d_bitval = G.dev(mask), G.dev(bitval)
        nb = 700
        ids = torch.zeros(nb, dtype=torch.int64, device="cuda")
        out = torch.zeros(nb * B, dtype=torch.uint8, device="cuda")
        ref = torch.zeros_like(out)
        sources = (("slots", store, n * slot, slot, None), ("cache", cache, total, 0, offsets))
        for name, src, src_bytes, sb, offs in sources:
            def launch(dst):
                ibp.gather_decompress(src, src_bytes, sb, offs, part, n, ids, nb, B, C, d_mask,
                                      d_bitval, dst)
            G.log(f"[parity] side stream + graph {key} from {name}")
            batch = rng.integers(0, n, nb)
            ids.copy_(torch.from_numpy(batch))
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                launch(out)
            side.synchronize()
            assert (G.host(out).reshape(nb, B) == rows[batch]).all(), (key, name, "side stream")
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                launch(out)
            torch.cuda.synchronize()
            for rep in range(3):
                batch = rng.integers(-2, n + 2, nb)
                ids.copy_(torch.from_numpy(batch))
                out.fill_(0x5A)
                launch(ref)  # eager launch of the same ids
                torch.cuda.synchronize()
                graph.replay()
                torch.cuda.synchronize()
                got = G.host(out).reshape(nb, B)
                assert (got == G.host(ref).reshape(nb, B)).all(), (key, name, rep, "eager")
                assert (got == G.expected_rows(rows, batch)).all(), (key, name, rep)
            del graph


def test_two_streams_at_once():
    """Gathers of different batches launched alternately on two streams, so
    that consecutive launches run at the same time (the library keeps no
    state a launch writes): group and tile kernels from pinned slots, and the
    indexed cache gather; every output checked against the original rows."""
    from host_transfer_amd import ibp
    rng = np.random.default_rng(23)
    for key, n in (("sparse_gnn", 1500), ("dense_gnn", 3000)):
        w = W.WORKLOADS[key].scaled(n)
        rows = W.rows(w)
        B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
        G.log(f"[parity] two streams at once: {key}")
        mask, bitval = G.check_metadata(rows, w.threshold)
        store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot, pinned=True)
        d_mask, d_bitval = G.dev(mask), G.dev(bitval)
        launches = [("slots", lambda ids, nb, dst: ibp.gather_decompress(
            store, n * slot, slot, None, part, n, ids, nb, B, C, d_mask, d_bitval, dst))]
        if C >= B:  # one-chunk tensors: also the indexed cache
            offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
            ibp.compact_offsets_aligned(lens, n, 128, offsets)
            total = int(offsets[-1].item())
            cache = torch.zeros(max(total, 16), dtype=torch.uint8, device="cuda")
            ibp.cache_fill(store, slot, lens, n, offsets, cache, total)
            index = torch.zeros((n + 31) // 32, dtype=torch.int64, device="cuda")
            ibp.cache_index(part, n, index)
            launches.append(("indexed cache", lambda ids, nb, dst: ibp.gather_decompress_indexed(
                cache, total, 128, index, n, ids, nb, B, C, d_mask, d_bitval, dst)))
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for name, launch in launches:
            nb = 4096
            batches = [rng.integers(-1, n + 1, nb) for _ in range(8)]
            d_ids = [torch.from_numpy(b).cuda() for b in batches]
            outs = [torch.full((nb * B,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(8)]
            torch.cuda.synchronize()
            for k in range(8):
                with torch.cuda.stream(streams[k % 2]):
                    launch(d_ids[k], nb, outs[k])
            torch.cuda.synchronize()
            for k in range(8):
                got = G.host(outs[k]).reshape(nb, B)
                assert (got == G.expected_rows(rows, batches[k])).all(), (key, name, k)
        store.free()


def _segment_case(rows, masks, bitvals, parts, B, C, S, n, rng, mode, per_seg=300, flags=0,
                  hot=0):
    """One segmented gather over `parts` = [(first, count) of the tensors
    compressed with mask k]; segment order shuffled, plus an empty segment and
    invalid ids.  hot > 0: every segment's ids drawn from its first `hot`
    tensors only (many repeats, as Zipf lookups).  Returns (got, want)."""
    from host_transfer_amd import ibp
    store, part, offsets, store_bytes, slot = mode
    order = list(rng.permutation(len(parts)))
    seg_ids, ids, m_all, v_all = [0], [], [], []
    for k in order + ["empty"]:
        if k == "empty":
            m_all.append(masks[0]), v_all.append(bitvals[0])
            seg_ids.append(seg_ids[-1])
            continue
        first, count = parts[k]
        x = rng.integers(first, first + (min(hot, count) if hot else count), per_seg)
        x[:3] = [first, first + count - 1, -1]
        ids.append(x)
        m_all.append(masks[k]), v_all.append(bitvals[k])
        seg_ids.append(seg_ids[-1] + len(x))
    ids = np.concatenate(ids).astype(np.int64)
    out = torch.full((len(ids) * B,), -1, dtype=torch.int8, device="cuda")
    ibp.gather_decompress_segments(store, store_bytes, slot, offsets, part, n, G.dev(ids), seg_ids,
                                   B, C, G.dev(np.concatenate(m_all)), G.dev(np.concatenate(v_all)),
                                   out, flags)
    got = G.host(out).view(np.uint8).reshape(len(ids), B)
    return got, G.expected_rows(rows, ids)


def test_segments():
    """ibp_gather_decompress_segments: every segment decoded with its own
    Mask/Bitval; the group kernel (K/V rows) and the tile kernel (dense_gnn,
    dlrm_1k rows); from slots and from a compacted cache; XCD-routed from
    slots (with few distinct ids per segment, and long); an empty segment and
    invalid ids."""
    from host_transfer_amd import ibp
    rng = np.random.default_rng(31)
    cases = []
    w = W.WORKLOADS["kv_opt13b"]
    R = 400
    rows = np.concatenate([W.rows(w, p * W.KV_ROWS_PER_PAIR, R) for p in range(3)])
    samples = [W.kv_prefill_rows(w, p, 1500) for p in range(3)]
    cases.append(("kv_opt13b", rows, samples, [w.threshold] * 3, w.chunk_bytes, w.slot_bytes))
    w = W.WORKLOADS["dense_gnn"]
    rows = W.rows(w, 0, 900)
    cases.append(("dense_gnn", rows, [rows[:300], rows[300:600], rows[600:]], [0.99, 0.9, 0.75],
                  w.chunk_bytes, w.slot_bytes))
    w = W.WORKLOADS["dlrm_1k"]
    rows = W.rows(w, 0, 900)
    x = rows.view(np.float32).copy()
    x[300:600] *= 16.0  # a second table with other exponents
    rows = x.view(np.uint8)
    cases.append(("dlrm_1k", rows, [rows[:300], rows[300:600], rows[600:]], [0.99, 0.99, 0.9],
                  w.chunk_bytes, w.slot_bytes))
    for key, rows, samples, Ts, C, S in cases:
        n, B = rows.shape
        k = len(samples)
        per = n // k
        masks, bitvals = [], []
        store = part = lens = None
        for p in range(k):
            m, v = G.check_metadata(samples[p], Ts[p])
            masks.append(m), bitvals.append(v)
            store, part, lens = G.gpu_compress(rows[p * per:(p + 1) * per], m, v, C, S,
                                               n_tensors=n, first=p * per, store=store, part=part,
                                               lengths=lens)
        assert len({m.tobytes() for m in masks}) > 1, "the segments' masks should differ"
        parts = [(p * per, per) for p in range(k)]
        G.log(f"[parity] segments {key}: {k} masks, slots")
        got, want = _segment_case(rows, masks, bitvals, parts, B, C, S, n, rng,
                                  (store, part, None, n * S, S))
        assert (got == want).all(), (key, "slots")
        offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
        ibp.compact_offsets(lens, n, offsets)
        total = int(offsets[-1].item())
        cache = torch.zeros(max(total, 16), dtype=torch.uint8, device="cuda")
        ibp.compact(store, S, n, offsets, cache, total)
        G.log(f"[parity] segments {key}: {k} masks, cache")
        got, want = _segment_case(rows, masks, bitvals, parts, B, C, S, n, rng,
                                  (cache, part, offsets, total, 0))
        assert (got == want).all(), (key, "cache")
        # long launches (the tile kernel's 8-load tiles for small tensors)
        G.log(f"[parity] segments {key}: {k} masks, 15,000 ids per segment")
        got, want = _segment_case(rows, masks, bitvals, parts, B, C, S, n, rng,
                                  (store, part, None, n * S, S), per_seg=15000)
        assert (got == want).all(), (key, "long")
        route = ibp.GATHER_ROUTE_XCD
        for per_seg, hot in ((300, 0), (2000, 40), (15000, 0)):
            G.log(f"[parity] segments {key}: routed, {per_seg} ids per segment, hot {hot}")
            got, want = _segment_case(rows, masks, bitvals, parts, B, C, S, n, rng,
                                      (store, part, None, n * S, S), per_seg=per_seg,
                                      flags=route, hot=hot)
            assert (got == want).all(), (key, "routed", per_seg, hot)


@pytest.mark.parametrize("key", ["kv_opt13b", "dense_gnn"])
def test_compress_segments(key):
    """ibp_compress_segments: each segment compressed with its own Mask and
    Bitval gives the oracle's payloads, bitmap bits and lengths for its
    tensors; an empty segment; rows taken at any offset of a larger buffer."""
    from host_transfer_amd import ibp
    w = W.WORKLOADS[key]
    R = 200
    if key == "kv_opt13b":
        rows = np.concatenate([W.rows(w, p * W.KV_ROWS_PER_PAIR, R) for p in range(3)])
        samples = [W.kv_prefill_rows(w, p, 1500) for p in range(3)]
        Ts = [w.threshold] * 3
    else:
        rows = W.rows(w, 0, 3 * R)
        samples = [rows[:R], rows[R:2 * R], rows[2 * R:]]
        Ts = [0.99, 0.9, 0.75]
    n, B = rows.shape
    C, S = w.chunk_bytes, w.slot_bytes
    masks, bitvals = [], []
    for p in range(3):
        m, v = G.check_metadata(samples[p], Ts[p])
        masks.append(m), bitvals.append(v)
    # segments: tensors [p*R + 7, p*R + 7 + count) from rows at the same index, one empty
    seg_row = [2 * R + 7, 0 * R + 7, 5, 1 * R + 7]
    seg_first = [2 * R + 7, 0 * R + 7, 0, 1 * R + 7]
    seg_count = [150, 120, 0, R - 7]
    seg_mask = [2, 0, 0, 1]
    store = torch.full((n * S,), 0xA5 - 256, dtype=torch.int8, device="cuda")
    part = torch.zeros((n * ibp.num_chunks(B, C) + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(n, dtype=torch.int32, device="cuda")
    G.log(f"[parity] compress segments {key}: {len(seg_row)} segments")
    ibp.compress_segments(G.dev(rows), B, seg_row, seg_first, seg_count, n, B, C,
                          G.dev(np.concatenate([masks[k] for k in seg_mask])),
                          G.dev(np.concatenate([bitvals[k] for k in seg_mask])), store, S, part,
                          lengths)
    torch.cuda.synchronize()
    for r0, f, c, k in zip(seg_row, seg_first, seg_count, seg_mask):
        if c:
            G.check_store(rows[r0:r0 + c], masks[k], bitvals[k], C, S, store, part, lengths,
                          first=f, n_tensors=n)


def test_deterministic_and_store_bound():
    w = W.WORKLOADS["dense_gnn"].scaled(2000)
    rows = W.rows(w)
    B, C, slot = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    mask, bitval = G.check_metadata(rows, w.threshold)
    store, part, lens = G.gpu_compress(rows, mask, bitval, C, slot)
    ids = np.random.default_rng(1).integers(0, 2000, 5000)
    a = G.gpu_gather(store, 2000 * slot, slot, None, part, 2000, ids, B, C, mask, bitval)
    b = G.gpu_gather(store, 2000 * slot, slot, None, part, 2000, ids, B, C, mask, bitval)
    assert (a == b).all() and (a == rows[ids]).all()


def test_compress_in_pieces_matches_whole():
    """Tensors compressed in separate calls (first_tensor) equal one call."""
    w = W.WORKLOADS["kv_opt13b"]
    rows = W.rows(w, 0, 600)
    mask, bitval = G.check_metadata(W.kv_prefill_rows(w, 0, 800), w.threshold)
    slot, C = w.slot_bytes, w.chunk_bytes
    s1, p1, l1 = G.gpu_compress(rows, mask, bitval, C, slot)
    s2, p2, l2 = G.gpu_compress(rows[:250], mask, bitval, C, slot, n_tensors=600)
    s2, p2, l2 = G.gpu_compress(rows[250:], mask, bitval, C, slot, n_tensors=600, first=250,
                                store=s2, part=p2, lengths=l2)
    G.check_store(rows[250:], mask, bitval, C, slot, s2, p2, l2, first=250, n_tensors=600)
    assert (G.host(p1) == G.host(p2)).all() and (G.host(l1) == G.host(l2)).all()
    ln = G.host(l1).view(np.uint32)
    a = G.store_bytes(s1).reshape(600, slot)
    b = G.store_bytes(s2).reshape(600, slot)
    valid = np.arange(slot)[None, :] < ln[:, None].astype(np.int64)
    assert (a[valid] == b[valid]).all()


@pytest.mark.parametrize("B,stride,shift,m", [(5732, 5760, 0, 777), (64, 128, 0, 777),
                                               (64, 128, 0, 140000), (64, 64, 4, 140000),
                                               (4, 4, 0, 600000), (256, 256, 4, 777),
                                               (60, 68, 0, 300000), (4096, 4096, 0, 777),
                                               (16384, 16384, 4, 777)])
@pytest.mark.parametrize("flags", [0, 1])
def test_raw_gather_and_stream_read(B, stride, shift, m, flags):
    """Uncompressed baseline gather: several rows per wave for short rows in
    large batches, 4 B units for rows at a 4 B offset, zero rows for invalid
    ids; with flags = 1 every row is copied on the XCD its id hashes to."""
    from host_transfer_amd import ibp
    rng = np.random.default_rng(11 + B)
    n = 500
    raw = rng.integers(0, 256, (n, stride), dtype=np.uint8)
    hb = ibp.HostBuffer(n * stride + shift)
    hb.array[shift:] = raw.ravel()
    ids = rng.integers(-2, n + 2, m)
    G.log(f"[parity] raw gather B={B} stride={stride} shift={shift} ids={m} flags={flags}")
    out = torch.zeros(m * B, dtype=torch.int8, device="cuda")
    ibp.raw_gather(hb.ptr + shift, stride, n, G.dev(ids), m, B, out, flags)
    got = G.host(out).view(np.uint8).reshape(m, B)
    assert (got == G.expected_rows(raw[:, :B].copy(), ids)).all()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    ibp.stream_read(hb, n * stride, 0x9E3779B9, sink)
    torch.cuda.synchronize()
    hb.free()


@pytest.mark.parametrize("nbytes", [0, 16, 4096, 1 << 20, (77 << 20) + 48])
def test_stream_copy(nbytes):
    """The copy probe copies every byte (device to device, and from pinned
    host memory), with a ragged tail of 16 B units past whole grid strides."""
    from host_transfer_amd import ibp
    rng = np.random.default_rng(nbytes % 1000 + 3)
    src_h = rng.integers(0, 256, nbytes, dtype=np.uint8)
    G.log(f"[parity] stream copy {nbytes} B")
    src = torch.zeros(max(nbytes, 16), dtype=torch.int8, device="cuda")
    src[:nbytes] = torch.from_numpy(src_h.view(np.int8)).cuda()
    dst = torch.full((nbytes + 32,), 7, dtype=torch.int8, device="cuda")
    ibp.stream_copy(src, dst, nbytes)
    got = G.host(dst).view(np.uint8)
    assert (got[:nbytes] == src_h).all()
    assert (got[nbytes:] == 7).all(), "bytes past the copy are untouched"
    if nbytes:
        hb = ibp.HostBuffer(nbytes)
        hb.array[:] = src_h[::-1]
        dst.fill_(7)
        ibp.stream_copy(hb, dst, nbytes)
        got = G.host(dst).view(np.uint8)
        assert (got[:nbytes] == src_h[::-1]).all()
        assert (got[nbytes:] == 7).all()
        hb.free()


# ------------------------------------------------------------ cache + store (hybrid)

@pytest.mark.parametrize("key,n", [("dense_gnn", 5000), ("sparse_gnn", 1500)])
@pytest.mark.parametrize("frac", [0.0, 0.3, 1.0])
def test_hybrid_cache_and_store(key, n, frac):
    """Cached tensors come from the HBM cache, the others from the pinned
    slots; the rows must be the same as from the slots alone."""
    from host_transfer_amd import ibp
    from oracle import oracle as O
    w = W.WORKLOADS[key].scaled(n)
    rows = W.rows(w)
    B, C, S = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    G.log(f"[parity] hybrid {key}: n={n} cached fraction {frac}")
    mask, bitval = G.check_metadata(rows, 0.95)
    store, part, lengths = G.gpu_compress(rows, mask, bitval, C, S, pinned=True)
    rng = np.random.default_rng(int(frac * 10) + n)
    select = (rng.random(n) < frac).astype(np.uint32)
    offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    ibp.cache_offsets(lengths, G.dev(select), n, offsets)
    g_off = G.host(offsets).view(np.uint64)
    ln = G.host(lengths).view(np.uint32).astype(np.uint64)
    pad = np.where(select != 0, (ln + 15) // 16 * 16, 0).astype(np.uint64)
    run = np.concatenate([[0], np.cumsum(pad)]).astype(np.uint64)
    want_off = np.where(select != 0, run[:-1], np.uint64(ibp.NOT_CACHED))
    assert (g_off[:n] == want_off).all() and g_off[n] == run[-1], "cache offsets"
    total = int(run[-1])
    cache = torch.full((max(total, 16),), 0x11, dtype=torch.uint8, device="cuda")
    ibp.cache_fill(store, S, lengths, n, offsets, cache, total)
    g_cache = G.host(cache)
    slots = store.array.reshape(n, S)
    for t in np.nonzero(select)[0][:200]:
        o, L = int(g_off[t]), int(ln[t])
        assert (g_cache[o:o + L] == slots[t, :L]).all(), "cached payload differs"
    ids = rng.integers(0, n, 3000)
    ids[:4] = [-1, n, 0, n - 1]
    out = torch.full((len(ids) * B,), -1, dtype=torch.int8, device="cuda")
    ibp.gather_decompress_hybrid(store, n * S, S, cache, total, offsets, part, n, G.dev(ids),
                                 len(ids), B, C, G.dev(mask), G.dev(bitval), out)
    got = G.host(out).view(np.uint8).reshape(len(ids), B)
    assert (got == G.expected_rows(rows, ids)).all(), "hybrid gather is not the original rows"
    o_store, o_part, _ = O.compress(rows, mask, bitval, C, slot_bytes=S)
    ok_ids = ids[(ids >= 0) & (ids < n)]
    want = O.gather_decompress(o_store, o_part, n, ok_ids, B, C, mask, bitval, slot_bytes=S)
    assert (got[(ids >= 0) & (ids < n)] == want).all(), "hybrid gather differs from the oracle"
    # the cache alone: tensors that are not cached give zero rows
    got2 = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
    cached = np.zeros(len(ids), bool)
    inr = (ids >= 0) & (ids < n)
    cached[inr] = select[ids[inr]] != 0
    assert (got2[cached] == got[cached]).all() and not got2[~cached].any()
    store.free()


# ------------------------------------------- aligned cache, rank index, indexed gather

def _scattered_rows(rng, n, B):
    """Rows whose invariant bits are scattered over each word (kept bits in
    three or more runs), so the indexed gather takes its five-stage expand."""
    W = B // 4
    fixed = rng.integers(0, 1 << 32, W, dtype=np.uint64).astype(np.uint32) & np.uint32(0x5A5A5A5A)
    vals = rng.integers(0, 1 << 32, W, dtype=np.uint64).astype(np.uint32)
    x = rng.integers(0, 1 << 32, (n, W), dtype=np.uint64).astype(np.uint32)
    x = (x & ~fixed) | (vals & fixed)
    flip = rng.random(n) < 0.1  # some tensors break the pattern and stay whole
    x[flip] ^= fixed
    return x.view(np.uint8)


INDEXED_CASES = [("dense_gnn", 512, 1024, 3000), ("dlrm_1k", 1024, 4096, 2000),
                 ("tiny-256", 256, 256, 2500), ("dense_gnn", 512, 4096, 1500)]


@pytest.mark.parametrize("key,B,C,n", INDEXED_CASES)
@pytest.mark.parametrize("law", ["workload", "mask0", "mask1", "scattered"])
def test_indexed_cache(key, B, C, n, law):
    """ibp_compact_offsets_aligned and ibp_cache_index against the oracle, bit
    for bit; ibp_gather_decompress_indexed (and the offset-table gather over
    the same aligned cache) against the oracle's gather and the original rows,
    on short and large batches with ragged tails, repeats and invalid ids."""
    from host_transfer_amd import ibp
    from oracle import oracle as O
    rng = np.random.default_rng(3 * B + n)
    if law == "workload" and key != "tiny-256":
        w = W.WORKLOADS[key].scaled(n)
        rows, T = W.rows(w), w.threshold
    elif law == "workload":
        rows = (rng.standard_normal((n, B // 4)) * 0.1).astype(np.float32).view(np.uint8)
        T = 0.99
    elif law == "mask0":
        rows, T = rng.integers(0, 256, (n, B), dtype=np.uint8), 1.0
    elif law == "mask1":
        rows, T = np.tile(rng.integers(0, 256, (1, B), dtype=np.uint8), (n, 1)), 0.99
    else:
        rows, T = _scattered_rows(rng, n, B), 0.85
    slot = (B + 127) // 128 * 128
    G.log(f"[parity] indexed cache: {key} {law} B={B} C={C} n={n}")
    mask, bitval = G.check_metadata(rows, T)
    store, part, lengths = G.gpu_compress(rows, mask, bitval, C, slot)
    o_store, o_part, o_len = G.check_store(rows, mask, bitval, C, slot, store, part, lengths)
    # rank index
    index = torch.full(((n + 31) // 32,), -1, dtype=torch.int64, device="cuda")
    ibp.cache_index(part, n, index)
    assert (G.host(index).view(np.uint64) == O.cache_index(o_part, n)).all(), "rank index differs"
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rpi = {256: 4, 512: 2, 1024: 1}[B]
    # more rows than one round of resident waves can take (at most 8 waves per
    # SIMD, 4 steps of rpi rows each): the grid-stride form of k_gather_cache
    big = 128 * cus * rpi
    for A in (16, 128):
        offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
        ibp.compact_offsets_aligned(lengths, n, A, offsets)
        o_off, o_cache = O.compact_aligned(o_store, slot, o_len, A)
        g_off = G.host(offsets).view(np.uint64)
        assert (g_off == o_off).all(), f"aligned offsets differ (A={A})"
        total = int(g_off[-1])
        cache = torch.full((max(total, 16),), 0x3C, dtype=torch.int8, device="cuda")
        ibp.cache_fill(store, slot, lengths, n, offsets, cache, total)
        g_cache = G.host(cache).view(np.uint8)
        for t in rng.choice(n, min(n, 300), replace=False):
            o, L = int(o_off[t]), int(o_len[t])
            assert (g_cache[o:o + L] == o_cache[o:o + L]).all(), f"cache entry {t} differs"
        d_mask, d_bv = G.dev(mask), G.dev(bitval)
        for nb in (1, 63, 65, 500, 4097, big + 1237):
            ids = rng.integers(0, n, nb)
            if nb > 3:
                ids[rng.integers(0, nb, max(1, nb // 50))] = rng.choice([-1, n, n + 7, 1 << 40])
                ids[-1] = n - 1
            want = O.gather_decompress(o_cache, o_part, n, ids, B, C, mask, bitval,
                                       offsets=o_off)
            assert (want == G.expected_rows(rows, ids)).all()
            out = torch.full((nb * B,), -1, dtype=torch.int8, device="cuda")
            d_ids = G.dev(ids.astype(np.int64))
            ibp.gather_decompress_indexed(cache, total, A, index, n, d_ids, nb, B, C, d_mask,
                                          d_bv, out)
            got = G.host(out).view(np.uint8).reshape(nb, B)
            assert (got == want).all(), f"{key} {law} A={A} nb={nb}: indexed gather differs"
            # the offset-table gather over the same aligned cache
            got = G.gpu_gather(cache, total, 0, offsets, part, n, ids, B, C, mask, bitval)
            assert (got == want).all(), f"{key} {law} A={A} nb={nb}: table gather differs"
        # a cache_bytes that cuts the last entries: their rows are zero, no read past it
        cut = max(16, total - 3 * slot)
        ids = np.concatenate([np.arange(n - 8, n), rng.integers(0, n, 200)])
        out = torch.full((len(ids) * B,), -1, dtype=torch.int8, device="cuda")
        ibp.gather_decompress_indexed(cache, cut, A, index, n, G.dev(ids), len(ids), B, C, d_mask,
                                      d_bv, out)
        got = G.host(out).view(np.uint8).reshape(len(ids), B)
        units = (o_len[ids].astype(np.int64) + 15) // 16
        inside = o_off[ids].astype(np.int64) + 16 * units <= cut
        want = G.expected_rows(rows, ids)
        want[~inside & (units > 0)] = 0
        assert (got == want).all(), f"{key} {law} A={A}: cut cache"
    # no tensors at all (an empty index): every row is zero, nothing is read
    ids = np.array([0, 1, -1, 5])
    out = torch.full((len(ids) * B,), -1, dtype=torch.int8, device="cuda")
    ibp.gather_decompress_indexed(cache, total, 128, index, 0, G.dev(ids), len(ids), B, C,
                                  G.dev(mask), G.dev(bitval), out)
    assert not G.host(out).any(), "rows of a gather over no tensors must be zero"


@pytest.mark.parametrize("n_seg", [80, 130, 256])
@pytest.mark.parametrize("B,C", [(256, 256), (1040, 256)])
def test_many_segments(n_seg, B, C):
    """ibp_compress_segments and ibp_gather_decompress_segments with 80, 130
    (the compressor splits launches at 128 segments) and 256 segments (the
    most one call takes), each segment with its own Mask and Bitval, empty
    segments among them; tile kernel (256 B tensors) and group kernel
    (1,040 B, five chunks); from slots (plain and XCD-routed) and from a
    compacted cache; element by element against the oracle."""
    from host_transfer_amd import ibp
    from oracle import oracle as O
    rng = np.random.default_rng(n_seg * 7 + B)
    per = 6
    n = n_seg * per
    S = (B + 127) // 128 * 128
    # segment k: floats with exponents shifted by k % 9, so the Masks differ
    x = (rng.standard_normal((n, B // 4)) * 0.1).astype(np.float32)
    x *= (2.0 ** (np.arange(n) // per % 9 - 4)).astype(np.float32)[:, None]
    rows = x.view(np.uint8).reshape(n, B)
    masks, bitvals = [], []
    for k in range(n_seg):
        m, v = O.build_metadata(rows[k * per:(k + 1) * per], 0.8)
        masks.append(m), bitvals.append(v)
    assert len({m.tobytes() for m in masks}) > 4
    empty = set(range(3, n_seg, 17))
    seg_row = [k * per for k in range(n_seg)]
    seg_count = [0 if k in empty else per for k in range(n_seg)]
    store = torch.full((n * S,), 0x5A, dtype=torch.int8, device="cuda")
    part = torch.zeros((n * ibp.num_chunks(B, C) + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(n, dtype=torch.int32, device="cuda")
    G.log(f"[parity] {n_seg} compress segments, B={B} C={C}")
    ibp.compress_segments(G.dev(rows), B, seg_row, seg_row, seg_count, n, B, C,
                          G.dev(np.concatenate(masks)), G.dev(np.concatenate(bitvals)), store, S,
                          part, lengths)
    torch.cuda.synchronize()
    full = [k for k in range(n_seg) if k not in empty]
    o_parts = {}
    for k in full:
        o_store, o_part, o_len = G.check_store(rows[k * per:(k + 1) * per], masks[k], bitvals[k], C,
                                               S, store, part, lengths, first=k * per, n_tensors=n)
        o_parts[k] = (o_store, o_part)
    # the empty segments' tensors were not written
    g_len = G.host(lengths).view(np.uint32)
    for k in empty:
        assert not g_len[k * per:(k + 1) * per].any()
    # gather: segment k takes ids of its own tensors (with repeats and an invalid id)
    ids, seg_ids, m_all, v_all, want = [], [0], [], [], []
    for k in range(n_seg):
        cnt = 0 if k in empty else int(rng.integers(1, 40))
        x = rng.integers(k * per, (k + 1) * per, cnt)
        if cnt > 2:
            x[1] = -1
        ids.append(x)
        seg_ids.append(seg_ids[-1] + cnt)
        m_all.append(masks[k]), v_all.append(bitvals[k])
        if cnt:
            o_store, o_part = o_parts[k]
            want.append(O.gather_decompress(o_store, o_part, n, x, B, C, masks[k], bitvals[k],
                                            slot_bytes=S))
    ids = np.concatenate(ids).astype(np.int64)
    want = np.concatenate(want)
    assert (want == G.expected_rows(rows, ids)).all()
    d_ids, d_m, d_v = G.dev(ids), G.dev(np.concatenate(m_all)), G.dev(np.concatenate(v_all))
    offsets = torch.zeros(n + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets(lengths, n, offsets)
    total = int(offsets[-1].item())
    cache = torch.zeros(max(total, 16), dtype=torch.uint8, device="cuda")
    ibp.compact(store, S, n, offsets, cache, total)
    for name, src, nbytes, slot, offs, flags in (
            ("slots", store, n * S, S, None, 0), ("slots routed", store, n * S, S, None, G.ROUTE),
            ("cache", cache, total, 0, offsets, 0)):
        G.log(f"[parity] {n_seg} gather segments, B={B}: {name}")
        out = torch.full((len(ids) * B,), -1, dtype=torch.int8, device="cuda")
        ibp.gather_decompress_segments(src, nbytes, slot, offs, part, n, d_ids, seg_ids, B, C, d_m,
                                       d_v, out, flags)
        got = G.host(out).view(np.uint8).reshape(len(ids), B)
        assert (got == want).all(), f"{n_seg} segments, B={B}: {name} differs from the oracle"


@pytest.mark.parametrize("n", [64, 1000])
def test_metadata_ties_at_half(n):
    """T = 0.5 with an even sample count: bit positions where exactly half the
    samples are 1 reach the cutoff (Mask 1) and take Bitval 0; positions one
    sample away from the tie take the majority value."""
    rng = np.random.default_rng(n)
    B = 512
    rows = np.zeros((n, B), np.uint8)
    half = n // 2
    bits = np.unpackbits(rows, axis=1, bitorder="little")
    kind = rng.integers(0, 4, 8 * B)   # 0: exact tie, 1: tie + 1 one, 2: tie - 1, 3: random
    for i in range(8 * B):
        ones = {0: half, 1: half + 1, 2: half - 1, 3: int(rng.integers(0, n + 1))}[int(kind[i])]
        col = np.zeros(n, np.uint8)
        col[rng.choice(n, ones, replace=False)] = 1
        bits[:, i] = col
    rows = np.packbits(bits, axis=1, bitorder="little")
    mask, bitval = G.check_metadata(rows, 0.5)
    mb = np.unpackbits(mask.view(np.uint8), bitorder="little")
    vb = np.unpackbits(bitval.view(np.uint8), bitorder="little")
    assert mb.all(), "at T = 0.5 the majority (or a tie) always reaches the cutoff"
    assert not vb[kind == 0].any(), "ties give Bitval 0"
    assert vb[kind == 1].all() and not vb[kind == 2].any()
