"""ibp_build_metadata_noalloc (the metadata build with the library's own fixed
counter array, for callers that cannot allocate) against ibp_build_metadata
with a caller workspace, and against the CPU oracle, bit for bit.  Two calls
in a row: the second with a smaller tensor and fewer samples, so counters the
first call left behind would show if they were not cleared."""
import numpy as np
import pytest
import torch

from host_transfer_amd import ibp
from host_transfer_amd import workloads as W
from tests import gpu_case as G

pytestmark = pytest.mark.gpu


def both_ways(rows, T, sample_ids=None):
    rows = np.ascontiguousarray(rows)
    N, B = rows.shape
    d_rows = G.dev(rows)
    d_ids = None if sample_ids is None else G.dev(np.asarray(sample_ids, np.int64))
    n = N if sample_ids is None else len(sample_ids)
    m0 = torch.zeros(B // 4, dtype=torch.int32, device="cuda")
    v0 = torch.zeros_like(m0)
    counts = torch.zeros(8 * B, dtype=torch.int32, device="cuda")
    ibp.build_metadata(d_rows, B, d_ids, n, B, T, m0, v0, counts)
    m1 = torch.full((B // 4,), 0x55, dtype=torch.int32, device="cuda")
    v1 = torch.full((B // 4,), 0x33, dtype=torch.int32, device="cuda")
    ibp.build_metadata_noalloc(d_rows, B, d_ids, n, B, T, m1, v1)
    return [G.host(t).view(np.uint32) for t in (m0, v0, m1, v1)]


def test_noalloc_matches_workspace_entry_point_twice():
    from oracle import oracle as O
    rng = np.random.default_rng(11)
    # first call: the largest tensor the fixed array holds, every counter used
    big = rng.integers(0, 256, (300, ibp.NOALLOC_MAX_TENSOR_BYTES), dtype=np.uint8)
    big[:, ::4] = 0x3C  # some invariant bytes
    cases = [("16 KB tensors", big, 0.9, None)]
    # second call: smaller tensors and fewer samples (tiny workload, sampled ids)
    w = W.WORKLOADS["tiny"].scaled(1500)
    rows = W.rows(w)
    ids = rng.choice(w.n_tensors, 700, replace=False)
    cases.append(("tiny, 700 sampled of 1500", rows, w.threshold, ids))
    # third: a tie-prone case at T = 0.5 with an even sample count
    half = np.zeros((64, 64), np.uint8)
    half[:32] = 0xFF
    cases.append(("exact ties at T = 0.5", half, 0.5, None))
    for name, r, T, s in cases:
        G.log(f"[noalloc] {name}: shape {r.shape}, T={T}")
        m0, v0, m1, v1 = both_ways(r, T, s)
        om, ov = O.build_metadata(r, T, sample_ids=s)
        assert (m1 == m0).all() and (v1 == v0).all(), f"{name}: differs from ibp_build_metadata"
        assert (m1 == om).all() and (v1 == ov).all(), f"{name}: differs from the oracle"
    # ties reach the cutoff at T = 0.5 and give Bitval 0
    assert (m1 == 0xFFFFFFFF).all() and (v1 == 0).all()
