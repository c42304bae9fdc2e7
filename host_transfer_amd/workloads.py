"""Seeded synthetic inputs shaped like the workloads on the pages.

This module only draws random numbers: it holds none of the compression
method's arithmetic, and both the HIP path's tests/benchmark and the CPU
oracle take their inputs from here.  No dataset is used; every tensor comes
from a numpy PCG64 stream seeded with SeedSequence([workload id, stream,
block]), so a block of rows is the same whatever else is drawn and whatever
the thread count.

Workloads (the pages describe GNN feature rows, DLRM embedding entries and
LLM K/V entries moved from CPU memory to the GPU; [G-EN] = gist.science English
explainer of "Reducing the GPU Memory Bottleneck with Lossless Compression for
ML -- Extended", [JH] = juhe.plus Chinese review of the same paper):

  tiny        4,096 tensors of 128 fp32 drawn from 0.1*N(0,1); 256 B chunks;
              Mask from all tensors, T = 0.99; compressed cache in HBM.
  sparse_gnn  2^20 rows of 1,433 fp32 that are 1.0 with probability 0.013 and
              0.0 otherwise (Cora-like binary features); 1 KB chunks; Mask from
              a 1 % sample; pinned host store; 8,192 uniform ids per batch.
  dense_gnn   2^21 rows of 128 fp32, column j drawn from N(0, s_j^2) with
              s_j ~ U[0.05, 2]; 1 KB chunks; 1 % sample; pinned host store;
              16,384 ids per batch from a bounded Zipf law, alpha = 1.1.
  dlrm_1k     2^23 rows of 256 fp32 ~ U(-0.05, 0.05); 4 KB chunks; 1 % sample;
              pinned host; 8,192 Zipf(1.05) ids per batch ([JH] Figure 10
              discussion: batch 8192 with 1 KB and 2 KB entries).
  dlrm_2k     same with 512 fp32 per row.
  kv_opt13b   OPT-13B K/V shape ([JH] LLM paragraph: 1,920 prompt tokens, 128
              output tokens, batch 20): a tensor is one (layer, K|V, sequence,
              token) row of 40 heads x 128 fp16 = 10,240 B; 256 B chunks (one
              head); channel c of pair p has scale s_c = exp(U(ln 0.1, ln 4)),
              51 channels (1 %) scaled x20, x = fp16(s_c * N(0,1)).  The Mask of
              a (layer, K|V) pair comes from its own prefill sample of
              1,920 x 20 = 38,400 rows ([JH]: Mask/Bitval from the prompt's K/V
              at prefill); a launch gathers that pair's 2,560 decode rows.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np

# stream ids inside a workload's seed sequence
STREAM_DATA = 0
STREAM_SAMPLE = 1
STREAM_BATCH = 2
STREAM_PARAM = 3
STREAM_PERM = 4
STREAM_PREFILL = 5

KV_LAYERS = 40
KV_HEADS = 40
KV_HEAD_DIM = 128
KV_SEQS = 20
KV_PROMPT = 1920
KV_DECODE = 128
KV_PAIRS = KV_LAYERS * 2
KV_ROWS_PER_PAIR = KV_SEQS * KV_DECODE          # 2,560 decode rows per launch
KV_PREFILL_ROWS = KV_SEQS * KV_PROMPT           # 38,400 sampled rows per pair
KV_CHANNELS = KV_HEADS * KV_HEAD_DIM            # 5,120


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    wid: int                 # seed id of the workload
    n_tensors: int
    tensor_bytes: int
    chunk_bytes: int
    threshold: float
    sample_fraction: float   # 1.0 = every tensor; KV uses its prefill sample
    batch: int               # ids per gather launch
    id_law: str              # 'perm' | 'uniform' | 'zipf' | 'kv_block'
    zipf_alpha: float
    store: str               # 'hbm' | 'pinned'
    dtype: str               # 'f32' | 'f16'
    row_block: int           # rows per seeded block

    @property
    def slot_bytes(self) -> int:
        """In-place slot size: the tensor size rounded up to 128 B lines."""
        return (self.tensor_bytes + 127) // 128 * 128

    def scaled(self, n_tensors: int) -> "Workload":
        """Same laws and seeds with fewer tensors (tensor i is unchanged)."""
        return dataclasses.replace(self, n_tensors=int(n_tensors))


WORKLOADS = {
    "tiny": Workload("tiny", 1, 4096, 512, 256, 0.99, 1.0, 4096, "perm", 0.0, "hbm", "f32", 4096),
    "sparse_gnn": Workload("sparse_gnn", 2, 1 << 20, 5732, 1024, 0.99, 0.01, 8192, "uniform", 0.0,
                           "pinned", "f32", 4096),
    "dense_gnn": Workload("dense_gnn", 3, 1 << 21, 512, 1024, 0.99, 0.01, 16384, "zipf", 1.1,
                          "pinned", "f32", 16384),
    "dlrm_1k": Workload("dlrm_1k", 4, 1 << 23, 1024, 4096, 0.99, 0.01, 8192, "zipf", 1.05,
                        "pinned", "f32", 16384),
    "dlrm_2k": Workload("dlrm_2k", 6, 1 << 23, 2048, 4096, 0.99, 0.01, 8192, "zipf", 1.05,
                        "pinned", "f32", 8192),
    "kv_opt13b": Workload("kv_opt13b", 5, KV_PAIRS * KV_ROWS_PER_PAIR, 2 * KV_CHANNELS, 256, 0.99,
                          0.0, KV_ROWS_PER_PAIR, "kv_block", 0.0, "pinned", "f16",
                          KV_ROWS_PER_PAIR),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- parameters

def dense_sigma(w: Workload) -> np.ndarray:
    """Per-column standard deviations of dense_gnn, s_j ~ U[0.05, 2]."""
    return _rng(w.wid, STREAM_PARAM).uniform(0.05, 2.0, w.tensor_bytes // 4).astype(np.float32)


def kv_scales(w: Workload, pair: int) -> np.ndarray:
    """Per-channel scales of one (layer, K|V) pair, with 1 % outlier channels."""
    r = _rng(w.wid, STREAM_PARAM, pair)
    s = np.exp(r.uniform(np.log(0.1), np.log(4.0), KV_CHANNELS))
    n_out = int(round(0.01 * KV_CHANNELS))
    s[r.choice(KV_CHANNELS, n_out, replace=False)] *= 20.0
    return s.astype(np.float32)


# ---------------------------------------------------------------- row blocks

def _draw_block(w: Workload, block: int, stream: int = STREAM_DATA, n_rows: int | None = None):
    rows = w.row_block if n_rows is None else n_rows
    r = _rng(w.wid, stream, block)
    if w.key == "tiny":
        x = r.standard_normal((rows, 128), dtype=np.float32) * np.float32(0.1)
    elif w.key == "sparse_gnn":
        x = (r.random((rows, w.tensor_bytes // 4), dtype=np.float32) < np.float32(0.013))
        x = x.astype(np.float32)
    elif w.key == "dense_gnn":
        x = r.standard_normal((rows, 128), dtype=np.float32) * dense_sigma(w)[None, :]
    elif w.key in ("dlrm_1k", "dlrm_2k"):
        x = r.random((rows, w.tensor_bytes // 4), dtype=np.float32) * np.float32(0.1)
        x -= np.float32(0.05)
    elif w.key == "kv_opt13b":
        # block = one (layer, K|V) pair's decode rows
        s = kv_scales(w, block)
        x = (r.standard_normal((rows, KV_CHANNELS), dtype=np.float32) * s[None, :])
        x = x.astype(np.float16)
    else:
        raise KeyError(w.key)
    return np.ascontiguousarray(x).view(np.uint8).reshape(rows, w.tensor_bytes)


def rows(w: Workload, start: int = 0, count: int | None = None, out: np.ndarray | None = None,
         threads: int | None = None) -> np.ndarray:
    """Tensors [start, start+count) as a (count, B) uint8 array (or into out,
    which may be any writable (count, B) uint8 array, e.g. pinned memory)."""
    if count is None:
        count = w.n_tensors - start
    if out is None:
        out = np.empty((count, w.tensor_bytes), np.uint8)
    if count == 0:
        return out
    b0 = start // w.row_block
    b1 = (start + count - 1) // w.row_block

    def fill(b):
        blk = _draw_block(w, b)
        lo = max(start, b * w.row_block)
        hi = min(start + count, (b + 1) * w.row_block)
        out[lo - start:hi - start] = blk[lo - b * w.row_block:hi - b * w.row_block]

    nt = threads or _threads()
    if nt == 1 or b1 == b0:
        for b in range(b0, b1 + 1):
            fill(b)
    else:
        with cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(b0, b1 + 1)))
    return out


KV_PREFILL_BLOCK = 4096


def kv_prefill_rows(w: Workload, pair: int, n_rows: int = KV_PREFILL_ROWS,
                    threads: int | None = None) -> np.ndarray:
    """Prompt K/V rows of one (layer, K|V) pair: the sample its Mask comes
    from.  Drawn in blocks of 4,096 rows, each from its own seeded stream."""
    s = kv_scales(w, pair)
    out = np.empty((n_rows, w.tensor_bytes), np.uint8)

    def fill(b):
        lo, hi = b * KV_PREFILL_BLOCK, min(n_rows, (b + 1) * KV_PREFILL_BLOCK)
        r = _rng(w.wid, STREAM_PREFILL, pair, b)
        x = r.standard_normal((hi - lo, KV_CHANNELS), dtype=np.float32) * s[None, :]
        out[lo:hi] = x.astype(np.float16).view(np.uint8).reshape(hi - lo, w.tensor_bytes)

    nb = (n_rows + KV_PREFILL_BLOCK - 1) // KV_PREFILL_BLOCK
    nt = threads or _threads()
    if nt == 1 or nb == 1:
        for b in range(nb):
            fill(b)
    else:
        with cf.ThreadPoolExecutor(nt) as ex:
            list(ex.map(fill, range(nb)))
    return out


# ---------------------------------------------------------------- ids

def sample_ids(w: Workload) -> np.ndarray | None:
    """Sorted ids of the metadata sample (None = every tensor)."""
    if w.sample_fraction >= 1.0:
        return None
    n = max(1, int(round(w.sample_fraction * w.n_tensors)))
    ids = _rng(w.wid, STREAM_SAMPLE).choice(w.n_tensors, n, replace=False)
    return np.sort(ids).astype(np.int64)


_zipf_cache: dict = {}


def _zipf_tables(w: Workload):
    key = (w.wid, w.n_tensors, w.zipf_alpha)
    if key not in _zipf_cache:
        r = np.arange(1, w.n_tensors + 1, dtype=np.float64)
        cdf = np.cumsum(r ** (-w.zipf_alpha))
        perm = _rng(w.wid, STREAM_PERM).permutation(w.n_tensors).astype(np.int64)
        _zipf_cache.clear()
        _zipf_cache[key] = (cdf, perm)
    return _zipf_cache[key]


def batch_ids(w: Workload, k: int, batch: int | None = None) -> np.ndarray:
    """The k-th batch of gathered tensor ids (int64)."""
    n = w.batch if batch is None else batch
    r = _rng(w.wid, STREAM_BATCH, k)
    if w.id_law == "perm":
        return r.permutation(w.n_tensors)[:n].astype(np.int64)
    if w.id_law == "uniform":
        return r.integers(0, w.n_tensors, n, dtype=np.int64)
    if w.id_law == "zipf":
        cdf, perm = _zipf_tables(w)
        u = r.random(n) * cdf[-1]
        rank = np.minimum(np.searchsorted(cdf, u, side="right"), w.n_tensors - 1)
        return perm[rank]
    if w.id_law == "kv_block":
        pair = k % KV_PAIRS
        first = pair * KV_ROWS_PER_PAIR
        return np.arange(first, first + min(n, KV_ROWS_PER_PAIR), dtype=np.int64)
    raise KeyError(w.id_law)
