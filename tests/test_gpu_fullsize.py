"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times.

At these sizes the oracle cannot redo everything, so each test checks:
  - Mask/Bitval of the GPU against the oracle's on the same sample (exact);
  - compressed bytes, participation bits and lengths of a random sample of
    tensors against the oracle compressing those tensors (exact);
  - the cache offsets against the 16 B-rounded running sum of the lengths, and
    the 128 B-aligned offsets and the rank index against the oracle's;
  - every gathered row against the original row (the method is lossless),
    and a sample of gathered rows against the oracle's gather.
"""
import numpy as np
import pytest
import torch

from host_transfer_amd import ibp
from host_transfer_amd import workloads as W
from oracle import oracle as O
from tests import gpu_case as G

pytestmark = pytest.mark.gpu

SAMPLE = 1024


def build_table(w, where, T=None):
    """Raw rows (pinned host, slot-strided), GPU metadata/compress/compact."""
    T = w.threshold if T is None else T
    N, B, C, S = w.n_tensors, w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    G.log(f"[fullsize] {w.key}: generating {N} x {B} B")
    raw = ibp.HostBuffer(N * S)
    view = raw.array.reshape(N, S)[:, :B]
    W.rows(w, 0, N, out=view)
    sid = W.sample_ids(w)
    n_s = N if sid is None else len(sid)
    mask = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    bitval = torch.zeros_like(mask)
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    ibp.build_metadata(raw, S, None if sid is None else G.dev(sid), n_s, B, T, mask, bitval, counts)
    G.log(f"[fullsize] {w.key}: metadata vs oracle on the {n_s}-tensor sample")
    sample_rows = view if sid is None else view[sid]
    om, ov = O.build_metadata(np.ascontiguousarray(sample_rows), T)
    m, v = G.host(mask).view(np.uint32), G.host(bitval).view(np.uint32)
    assert (m == om).all() and (v == ov).all(), "Mask/Bitval differ from the oracle"
    n_c = ibp.num_chunks(B, C)
    store = ibp.HostBuffer(N * S) if where == "pinned" else \
        torch.empty(N * S, dtype=torch.uint8, device="cuda")
    part = torch.zeros((N * n_c + 31) // 32, dtype=torch.int32, device="cuda")
    lengths = torch.zeros(N, dtype=torch.int32, device="cuda")
    ibp.compress(raw, S, N, 0, N, B, C, mask, bitval, store, S, part, lengths)
    torch.cuda.synchronize()
    return dict(w=w, raw=raw, view=view, mask=om, bitval=ov, d_mask=mask, d_bitval=bitval,
                store=store, part=part, lengths=lengths, n_c=n_c)


def check_sampled_store(t, rng):
    """Compressed bytes, bits and lengths of SAMPLE random tensors vs the oracle."""
    w = t["w"]
    N, B, C, S, n_c = w.n_tensors, w.tensor_bytes, w.chunk_bytes, w.slot_bytes, t["n_c"]
    ids = np.sort(rng.choice(N, SAMPLE, replace=False))
    rows = np.ascontiguousarray(t["view"][ids])
    o_store, o_part, o_len = O.compress(rows, t["mask"], t["bitval"], C, slot_bytes=S)
    g_len = G.host(t["lengths"]).view(np.uint32)
    assert (g_len[ids] == o_len).all(), "lengths differ"
    g_bits = np.unpackbits(G.host(t["part"]).view(np.uint8), bitorder="little")
    o_bits = np.unpackbits(o_part.view(np.uint8), bitorder="little")
    gi = (ids[:, None] * n_c + np.arange(n_c)[None, :]).ravel()
    oi = (np.arange(SAMPLE)[:, None] * n_c + np.arange(n_c)[None, :]).ravel()
    assert (g_bits[gi] == o_bits[oi]).all(), "participation bits differ"
    if isinstance(t["store"], ibp.HostBuffer):
        g_slots = t["store"].array.reshape(N, S)[ids]
    else:
        g_slots = t["store"].view(N, S)[G.dev(ids)].cpu().numpy()
    o_slots = o_store.reshape(SAMPLE, S)
    valid = np.arange(S)[None, :] < o_len[:, None].astype(np.int64)
    assert (g_slots[valid] == o_slots[valid]).all(), "payload bytes differ"
    return g_len


def check_gather(t, ids, store, store_bytes, offsets, rng, label, flags=0):
    """Every row lossless; SAMPLE rows equal to the oracle's gather."""
    w = t["w"]
    N, B, C, S = w.n_tensors, w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    nb = len(ids)
    out = torch.empty(nb * B, dtype=torch.uint8, device="cuda")
    G.log(f"[fullsize] {w.key}: gather {nb} ids ({label}, flags {flags})")
    ibp.gather_decompress_ex(store, store_bytes, S, offsets, t["part"], N, G.dev(ids), nb, B, C,
                             t["d_mask"], t["d_bitval"], out, flags)
    got = G.host(out).reshape(nb, B)
    assert (got == t["view"][ids]).all(), f"{label}: gathered rows are not the original rows"
    pick = rng.choice(nb, min(SAMPLE, nb), replace=False)
    sub = ids[pick]
    uniq, inv = np.unique(sub, return_inverse=True)
    rows = np.ascontiguousarray(t["view"][uniq])
    o_store, o_part, _ = O.compress(rows, t["mask"], t["bitval"], C, slot_bytes=S)
    want = O.gather_decompress(o_store, o_part, len(uniq), inv, B, C, t["mask"], t["bitval"],
                               slot_bytes=S)
    assert (got[pick] == want).all(), f"{label}: gather differs from the oracle"


def test_fullsize_sparse_gnn_pinned():
    rng = np.random.default_rng(101)
    w = W.WORKLOADS["sparse_gnn"]
    t = build_table(w, "pinned")
    check_sampled_store(t, rng)
    for k in (0, 1):
        check_gather(t, W.batch_ids(w, k), t["store"], w.n_tensors * w.slot_bytes, None, rng,
                     f"batch {k}")
    t["raw"].free()
    t["store"].free()


def _hbm_cache(t):
    w = t["w"]
    N, S = w.n_tensors, w.slot_bytes
    offsets = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets(t["lengths"], N, offsets)
    g_off = G.host(offsets).view(np.uint64)
    g_len = G.host(t["lengths"]).view(np.uint32).astype(np.uint64)
    want = np.concatenate([[0], np.cumsum((g_len + 15) // 16 * 16)]).astype(np.uint64)
    assert (g_off == want).all(), "cache offsets are not the rounded running sum"
    total = int(g_off[-1])
    cache = torch.empty(total, dtype=torch.uint8, device="cuda")
    ibp.compact(t["store"], S, N, offsets, cache, total)
    torch.cuda.synchronize()
    return offsets, cache, total


@pytest.mark.parametrize("key", ["dense_gnn", "dlrm_1k"])
def test_fullsize_hbm_cache(key):
    rng = np.random.default_rng(202)
    w = W.WORKLOADS[key]
    t = build_table(w, "hbm")
    check_sampled_store(t, rng)
    offsets, cache, total = _hbm_cache(t)
    del t["store"]
    torch.cuda.empty_cache()
    check_gather(t, W.batch_ids(w, 0), cache, total, offsets, rng, "workload batch")
    big = np.concatenate([W.batch_ids(w, k) for k in range((1 << 20) // w.batch)])
    check_gather(t, big, cache, total, offsets, rng, "1M ids")
    t["raw"].free()


def check_indexed_gather(t, ids, cache, total, align, index, rng, label):
    """ibp_gather_decompress_indexed: every row lossless; SAMPLE rows equal to
    the oracle's gather."""
    w = t["w"]
    N, B, C, S = w.n_tensors, w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    nb = len(ids)
    out = torch.empty(nb * B, dtype=torch.uint8, device="cuda")
    G.log(f"[fullsize] {w.key}: indexed gather {nb} ids ({label}, entries of {align} B)")
    ibp.gather_decompress_indexed(cache, total, align, index, N, G.dev(ids), nb, B, C,
                                  t["d_mask"], t["d_bitval"], out)
    got = G.host(out).reshape(nb, B)
    assert (got == t["view"][ids]).all(), f"{label}: gathered rows are not the original rows"
    pick = rng.choice(nb, min(SAMPLE, nb), replace=False)
    uniq, inv = np.unique(ids[pick], return_inverse=True)
    rows = np.ascontiguousarray(t["view"][uniq])
    o_store, o_part, _ = O.compress(rows, t["mask"], t["bitval"], C, slot_bytes=S)
    want = O.gather_decompress(o_store, o_part, len(uniq), inv, B, C, t["mask"], t["bitval"],
                               slot_bytes=S)
    assert (got[pick] == want).all(), f"{label}: gather differs from the oracle"


@pytest.mark.parametrize("key", ["dense_gnn", "dlrm_1k"])
def test_fullsize_indexed_cache(key):
    """The HBM cache as the benchmark lays it out and times it: entries rounded
    to 128 B lines (ibp_compact_offsets_aligned, ibp_cache_fill) and found
    through the rank index (ibp_cache_index), gathered with the workload's
    batch, 1M Zipf ids and 1M distinct ids."""
    rng = np.random.default_rng(303)
    w = W.WORKLOADS[key]
    N, S, A = w.n_tensors, w.slot_bytes, 128
    t = build_table(w, "hbm")
    check_sampled_store(t, rng)
    offsets = torch.zeros(N + 1, dtype=torch.int64, device="cuda")
    ibp.compact_offsets_aligned(t["lengths"], N, A, offsets)
    g_off = G.host(offsets).view(np.uint64)
    g_len = G.host(t["lengths"]).view(np.uint32)
    o_off, _ = O.compact_aligned(None, S, g_len, A, with_cache=False)
    assert (g_off == o_off).all(), "aligned offsets differ from the oracle's"
    total = int(g_off[-1])
    cache = torch.empty(total, dtype=torch.uint8, device="cuda")
    ibp.cache_fill(t["store"], S, t["lengths"], N, offsets, cache, total)
    index = torch.zeros((N + 31) // 32, dtype=torch.int64, device="cuda")
    ibp.cache_index(t["part"], N, index)
    o_idx = O.cache_index(G.host(t["part"]).view(np.uint32), N)
    assert (G.host(index).view(np.uint64) == o_idx).all(), "rank index differs from the oracle's"
    del t["store"], offsets
    torch.cuda.empty_cache()
    check_indexed_gather(t, W.batch_ids(w, 0), cache, total, A, index, rng, "workload batch")
    big = np.concatenate([W.batch_ids(w, k) for k in range((1 << 20) // w.batch)])
    check_indexed_gather(t, big, cache, total, A, index, rng, "1M Zipf ids")
    distinct = rng.permutation(N)[:1 << 20].astype(np.int64)
    check_indexed_gather(t, distinct, cache, total, A, index, rng, "1M distinct ids")
    t["raw"].free()


@pytest.mark.parametrize("key", ["dense_gnn", "dlrm_1k", "dlrm_2k"])
def test_fullsize_pinned(key):
    rng = np.random.default_rng(303)
    w = W.WORKLOADS[key]
    t = build_table(w, "pinned")
    check_sampled_store(t, rng)
    for flags in (0, G.ROUTE):  # plain, and routed to XCDs (the bench's launch for Zipf ids)
        check_gather(t, W.batch_ids(w, 0), t["store"], w.n_tensors * w.slot_bytes, None, rng,
                     "workload batch", flags)
    t["raw"].free()
    t["store"].free()


def test_fullsize_kv_pair():
    """One (layer, K|V) launch at full size: Mask from the whole 38,400-row
    prefill sample, the pair's 2,560 decode rows, all checked against the oracle."""
    w = W.WORKLOADS["kv_opt13b"]
    B, C, S = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    pair = 7
    G.log("[fullsize] kv_opt13b: prefill sample metadata")
    pre = W.kv_prefill_rows(w, pair)
    mask, bitval = G.check_metadata(pre, w.threshold)
    del pre
    rows = W.rows(w, pair * W.KV_ROWS_PER_PAIR, W.KV_ROWS_PER_PAIR)
    n = rows.shape[0]
    store, part, lengths = G.gpu_compress(rows, mask, bitval, C, S, pinned=True)
    o_store, o_part, _ = G.check_store(rows, mask, bitval, C, S, store, part, lengths)
    ids = np.arange(n)
    got = G.gpu_gather(store, n * S, S, None, part, n, ids, B, C, mask, bitval)
    assert (got == rows).all()
    want = O.gather_decompress(o_store, o_part, n, ids, B, C, mask, bitval, slot_bytes=S)
    assert (got == want).all()
    store.free()
