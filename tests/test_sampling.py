"""Metadata from a sample of the tensors ([JH] sampling paragraph: Masks built
from 1 %, 5 % or 10 % of the data give compression ratios close to those of
the full data), on the CPU oracle.

DLRM-like entries, U(-0.05, 0.05) fp32: the Mask has a closed form at every
sample size (each word 0x78000000, Bitval 0x38000000; see test_workloads.py),
so sampled and full-data Masks are identical.  Dense GNN features,
N(0, s_j^2) fp32 with s_j ~ U[0.05, 2] per column: the Mask depends on each
column's scale; the payload ratio of the whole table compressed with the
sampled Mask stays within 1 % of the full-data ratio.  The ratios are printed
(run with -s) for the design notes.
"""
import numpy as np
import pytest

from host_transfer_amd import workloads as W

FRACTIONS = (0.01, 0.05, 0.10, 1.0)


def _ratios(orc, w, rows, seed):
    rng = np.random.default_rng(seed)
    n, B = rows.shape
    out = {}
    for f in FRACTIONS:
        ids = None if f >= 1.0 else np.sort(rng.choice(n, int(round(f * n)), replace=False))
        mask, bitval = orc.build_metadata(rows, w.threshold, sample_ids=ids)
        _, _, lens = orc.compress(rows, mask, bitval, w.chunk_bytes, slot_bytes=w.slot_bytes)
        out[f] = (mask, bitval, float(lens.mean()) / B)
    return out


@pytest.mark.slow
def test_dlrm_sampled_mask_equals_full(orc):
    w = W.WORKLOADS["dlrm_1k"]
    rows = W.rows(w, 0, 32768)
    r = _ratios(orc, w, rows, 5)
    for f, (mask, bitval, ratio) in r.items():
        assert (mask == 0x78000000).all() and (bitval == 0x38000000).all(), f
        assert ratio == r[1.0][2], f
    print("dlrm_1k payload/tensor by sample:", {f: round(v[2], 5) for f, v in r.items()})


@pytest.mark.slow
def test_dense_gnn_sampled_ratio_close_to_full(orc):
    w = W.WORKLOADS["dense_gnn"]
    rows = W.rows(w, 0, 40960)
    r = _ratios(orc, w, rows, 6)
    full = r[1.0][2]
    for f, (mask, _, ratio) in r.items():
        assert abs(ratio / full - 1.0) < 0.01, (f, ratio, full)
    # a small sample may add a bit near the threshold to a few columns' Masks
    print("dense_gnn payload/tensor by sample:", {f: round(v[2], 5) for f, v in r.items()},
          "Mask words differing from the full-data Mask:",
          {f: int((v[0] != r[1.0][0]).sum()) for f, v in r.items()})
