"""The C oracle against the pure-Python brute force (oracle/ibp_ref.py) on
randomly drawn small cases: tensor and chunk sizes, thresholds, sample
subsets and value laws chosen by hypothesis.  Metadata, participation bits,
payload bytes and lengths must agree exactly, and the brute force's decode
of the C oracle's payload must give the tensor back."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import ibp_ref
from oracle import oracle as O
from tests import oracle_pins as P


@settings(max_examples=200, deadline=None)
@given(words=st.integers(1, 40), chunk_words=st.sampled_from([1, 2, 4, 16, 64]),
       n=st.integers(1, 10), T=st.floats(0.5, 1.0),
       kind=st.sampled_from(["float", "bytes", "sparse", "flips"]),
       seed=st.integers(0, 2 ** 31 - 1), use_sample=st.booleans())
def test_oracle_matches_brute_force(words, chunk_words, n, T, kind, seed, use_sample):
    rng = np.random.default_rng(seed)
    B, C = 4 * words, 4 * chunk_words
    rows = P._random_case(rng, n, words, kind)
    sample = None
    if use_sample and n > 1:
        sample = np.sort(rng.choice(n, size=max(1, n // 2), replace=False)).astype(np.int64)
    samples = [r.tobytes() for r in (rows if sample is None else rows[sample])]
    rm, rv = ibp_ref.build_metadata(samples, T)
    mask, bitval = O.build_metadata(rows, T, sample_ids=sample)
    assert rm == P._bytes(mask) and rv == P._bytes(bitval)
    slot = (B + 127) // 128 * 128
    store, pb, lens = O.compress(rows, mask, bitval, C, slot_bytes=slot)
    bits = P._bits_le(pb)
    n_c = (B + C - 1) // C
    for i in range(n):
        payload, part, _ = ibp_ref.compress_one(rows[i].tobytes(), rm, rv, C)
        assert [int(b) for b in bits[i * n_c:(i + 1) * n_c]] == part
        assert int(lens[i]) == len(payload)
        assert store[i * slot:i * slot + len(payload)].tobytes() == payload
        assert ibp_ref.decompress_one(payload, part, rm, rv, B, C) == rows[i].tobytes()
    ids = rng.integers(-1, n + 1, 7)
    got = O.gather_decompress(store, pb, n, ids, B, C, mask, bitval, slot_bytes=slot)
    for r, t in zip(got, ids):
        want = rows[t].tobytes() if 0 <= t < n else bytes(B)
        assert r.tobytes() == want
