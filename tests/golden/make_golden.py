"""Writes tests/golden/oracle_regression.json: the oracle's results on small
seeded cases of every workload, as digests.

Calls only oracle/ (and the seeded input generators).  The pages print no
worked example with concrete bits, so these values are not the pages': they
fix what the oracle computes today, so that any later change to its
arithmetic shows up in tests/test_oracle_golden.py and has to be justified
by a passage of the pages.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from host_transfer_amd import workloads as W  # noqa: E402
from oracle import oracle as O  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")

# (workload, tensors, threshold); K/V takes its Mask from prefill rows
CASES = [("tiny", 512, 0.99), ("sparse_gnn", 96, 0.99), ("sparse_gnn", 96, 0.95),
         ("dense_gnn", 384, 0.99), ("dlrm_1k", 256, 0.99), ("dlrm_2k", 128, 0.99),
         ("kv_opt13b", 64, 0.99)]


def digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def case(key, n, T):
    w = W.WORKLOADS[key].scaled(n)
    B, C, S = w.tensor_bytes, w.chunk_bytes, w.slot_bytes
    rows = W.rows(w, 0, n)
    sample = W.kv_prefill_rows(w, 0, 2000) if key == "kv_opt13b" else rows
    mask, bitval = O.build_metadata(sample, T)
    store, part, lens = O.compress(rows, mask, bitval, C, slot_bytes=S)
    payload = np.concatenate([store[t * S:t * S + int(lens[t])] for t in range(n)])
    offsets, cache = O.compact(store, S, lens)
    ids = np.array([0, n - 1, n // 2, -1, n, 3, 3, n // 3], np.int64)
    got = O.gather_decompress(store, part, n, ids, B, C, mask, bitval, slot_bytes=S)
    got_c = O.gather_decompress(cache, part, n, ids, B, C, mask, bitval, offsets=offsets)
    assert (got == got_c).all()
    return {"workload": key, "tensors": n, "tensor_bytes": B, "chunk_bytes": C, "threshold": T,
            "mask_popcount": int(np.unpackbits(mask.view(np.uint8)).sum()),
            "mask_first_words": [f"{int(x):08x}" for x in mask[:4]],
            "bitval_first_words": [f"{int(x):08x}" for x in bitval[:4]],
            "mask_bitval_sha256": digest(mask, bitval),
            "lengths_sum": int(lens.astype(np.uint64).sum()),
            "lengths_sha256": digest(lens.astype("<u4")),
            "part_bits_sha256": digest(part.astype("<u4")),
            "payload_sha256": digest(payload),
            "cache_bytes": int(offsets[-1]),
            "gather_ids": ids.tolist(),
            "gather_sha256": digest(got)}


def build():
    return {"note": "oracle results on seeded inputs (written by make_golden.py from oracle/ "
                    "only; not values printed by the pages)",
            "cases": [case(*c) for c in CASES]}


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(build(), f, indent=1)
        f.write("\n")
    print("wrote", OUT)
