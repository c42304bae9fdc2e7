"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each pin takes an oracle instance (oracle.oracle.Oracle) and raises
AssertionError on a violation, so the same pins run against the real oracle
(tests/test_oracle_pins.py) and against deliberately broken copies of it
(tests/test_oracle_mutants.py).  None of them re-types the oracle's loops:

  - hand-worked examples derived from the definitions ([G-EN] = gist.science
    English explainer of "Reducing the GPU Memory Bottleneck with Lossless
    Compression for ML -- Extended", Technical Summary, Core Algorithm);
  - cutoff boundaries of the threshold rule (Preprocessing);
  - closed forms of the metadata (identical samples, T = 1, ties, order);
  - the payload equals x86 BMI2 PEXT of the tensor's words (a hardware
    instruction's definition pins the bit order), decode equals PDEP;
  - lossless round trip ([G-EN] Methodology: the data comes back unchanged);
  - the payload length is the popcount of the non-invariant bits of the
    participating chunks plus the full size of the others;
  - Mask = 0 reduces gather + decompress to a plain row gather;
  - a second, pure-Python brute-force implementation (oracle/ibp_ref.py).
"""
import numpy as np

from oracle import ibp_ref

U32 = np.uint32


def _w(*words):
    return np.array(words, dtype=U32)


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8).tobytes()


def _bits_le(a):
    return np.unpackbits(np.ascontiguousarray(a).view(np.uint8), bitorder="little")


# --------------------------------------------------------------------------
# hand-worked examples ([G-EN] Core Algorithm, Compression and Decompression)

HAND_EXAMPLES = [
    # (name, tensor words, mask, bitval, chunk bytes, payload, P bits)
    # One word, bits 24..31 invariant with value 0x3F: the word matches, so the
    # 24 low bits 0x123456 are kept, LSB first: bytes 56 34 12.
    ("drop-top-byte", _w(0x3F123456), _w(0xFF000000), _w(0x3F000000), 256,
     bytes([0x56, 0x34, 0x12]), [1]),
    # Same Mask, top byte 0x40 differs from Bitval: the chunk stays raw.
    ("mismatch-raw", _w(0x40ABCDEF), _w(0xFF000000), _w(0x3F000000), 256,
     bytes([0xEF, 0xCD, 0xAB, 0x40]), [0]),
    # Two words, one chunk.  Word 0 keeps bits 4..31 (0x0ABCDEF0, 28 bits),
    # word 1 keeps bits 0..30 (0x7FFFFFFF, 31 bits) right after it:
    # stream = 0x0ABCDEF0 + 0x7FFFFFFF * 2^28 = 0x07FFFFFFFABCDEF0, 59 bits.
    ("two-words-gapless", _w(0xABCDEF05, 0x7FFFFFFF), _w(0x0000000F, 0x80000000), _w(5, 0), 256,
     bytes([0xF0, 0xDE, 0xBC, 0xFA, 0xFF, 0xFF, 0xFF, 0x07]), [1]),
    # Two 4-byte chunks: chunk 0 matches (16 kept bits 0x1234), chunk 1 has bit
    # 16 set against Bitval 0 and stays raw (32 bits) right after chunk 0:
    # stream = 0x1234 + 0x00015678 * 2^16, 48 bits.
    ("chunk-fallback", _w(0x00001234, 0x00015678), _w(0xFFFF0000, 0xFFFF0000), _w(0, 0), 4,
     bytes([0x34, 0x12, 0x78, 0x56, 0x01, 0x00]), [1, 0]),
    # Chunk 0 holds no Mask bit: packing saves nothing, so it does not
    # participate; chunk 1 is all Mask bits and matches: zero payload bits.
    ("no-saving-no-participation", _w(0xDEADBEEF, 0x12345678), _w(0, 0xFFFFFFFF),
     _w(0, 0x12345678), 4, bytes([0xEF, 0xBE, 0xAD, 0xDE]), [0, 1]),
]


def pin_hand_examples(orc):
    for name, x, mask, bitval, C, payload, part in HAND_EXAMPLES:
        B = 4 * x.size
        store = np.full(128, 0xAA, np.uint8)   # garbage: the last byte must be zero-filled
        store, pb, lens = orc.compress(x[None, :], mask, bitval, C, slot_bytes=128, store=store)
        assert int(lens[0]) == len(payload), (name, int(lens[0]))
        assert store[:len(payload)].tobytes() == payload, (name, store[:len(payload)].tobytes())
        got = [int(b) for b in _bits_le(pb)[:len(part)]]
        assert got == part, (name, got)
        y = orc.gather_decompress(store, pb, 1, [0], B, C, mask, bitval, slot_bytes=128)
        assert y.tobytes() == _bytes(x), name

    # The bitmap index of chunk c of tensor t is t*n_c + c: tensor 3 of 4 with
    # two chunks per tensor owns bits 6 and 7 (P = 1, 0): word 0 = 0x40.
    _, x, mask, bitval, C, _, _ = HAND_EXAMPLES[3]
    store, pb, _ = orc.compress(x[None, :], mask, bitval, C, slot_bytes=128, first_tensor=3,
                                n_tensors=4)
    assert int(pb[0]) == 0x40, hex(int(pb[0]))


# --------------------------------------------------------------------------
# metadata ([G-EN] Core Algorithm, Preprocessing)

def _rows_with_counts(n, counts):
    """n one-word tensors where bit b is set in exactly counts[b] of them."""
    rows = np.zeros((n, 1), U32)
    for b, k in counts.items():
        rows[:k, 0] |= U32(1 << b)
    return rows


def pin_metadata_hand(orc):
    # Four tensors 0x1, 0x3, 0x1, 0x0.  T = 0.75 -> cutoff 3: bit 0 is 1 in
    # three of them (invariant, value 1), bit 1 is 0 in three (invariant, 0).
    rows = _w(0x1, 0x3, 0x1, 0x0)[:, None]
    m, v = orc.build_metadata(rows, 0.75)
    assert (int(m[0]), int(v[0])) == (0xFFFFFFFF, 0x1), (hex(int(m[0])), hex(int(v[0])))
    # T = 1: only positions on which all four agree.
    m, v = orc.build_metadata(rows, 1.0)
    assert (int(m[0]), int(v[0])) == (0xFFFFFFFC, 0x0)
    # Tie at T = 0.5 (cutoff 1 of 2): invariant, and the value of a tie is 0.
    m, v = orc.build_metadata(_w(0x1, 0x0)[:, None], 0.5)
    assert (int(m[0]), int(v[0])) == (0xFFFFFFFF, 0x0)


def pin_cutoff_boundaries(orc):
    # n = 100, T = 0.99: cutoff 99.  Bit 0 set in 99 -> invariant 1; bit 1 in
    # 98 -> not; bit 2 in 1 -> invariant 0; bit 3 in 2 -> not.
    rows = _rows_with_counts(100, {0: 99, 1: 98, 2: 1, 3: 2})
    m, v = orc.build_metadata(rows, 0.99)
    assert (int(m[0]), int(v[0])) == (0xFFFFFFF5, 0x1), (hex(int(m[0])), hex(int(v[0])))
    # n = 4096, T = 0.99: T*n = 4055.04 rounds up to the cutoff 4056.
    rows = _rows_with_counts(4096, {0: 4056, 1: 4055, 2: 40, 3: 41})
    m, v = orc.build_metadata(rows, 0.99)
    assert (int(m[0]), int(v[0])) == (0xFFFFFFF5, 0x1), (hex(int(m[0])), hex(int(v[0])))
    assert orc.cutoff(0.99, 4096) == 4056 and orc.cutoff(0.99, 100) == 99


def pin_metadata_closed_forms(orc, rng):
    B = 64
    one = rng.integers(0, 2 ** 32, B // 4, dtype=np.uint64).astype(U32)
    # identical samples: every position is invariant and Bitval is the tensor
    m, v = orc.build_metadata(np.tile(one, (7, 1)), 0.99)
    assert (m == U32(0xFFFFFFFF)).all() and (v == one).all()
    # ... and compressing that tensor leaves an empty payload in every chunk
    _, pb, lens = orc.compress(one[None, :], m, v, 16)
    assert int(lens[0]) == 0 and (_bits_le(pb)[:4] == 1).all()
    # T = 1: Mask = positions where all samples agree, Bitval = their AND
    rows = rng.integers(0, 2 ** 32, (9, B // 4), dtype=np.uint64).astype(U32)
    rows[:, :4] &= U32(0x00FF00FF)
    rows[:, 4:8] |= U32(0xF000000F)
    m, v = orc.build_metadata(rows, 1.0)
    and_all = np.bitwise_and.reduce(rows, axis=0)
    or_all = np.bitwise_or.reduce(rows, axis=0)
    assert (m == (and_all | ~or_all)).all() and (v == and_all).all()
    # invariants: Bitval only on Mask positions; sample order is irrelevant;
    # an explicit id list is the same as those rows
    rows = rng.integers(0, 2 ** 32, (50, B // 4), dtype=np.uint64).astype(U32)
    rows[:45, :] &= U32(0x0FFFFFFF)
    m1, v1 = orc.build_metadata(rows, 0.9)
    assert not (v1 & ~m1).any()
    perm = rng.permutation(50)
    m2, v2 = orc.build_metadata(rows[perm], 0.9)
    assert (m1 == m2).all() and (v1 == v2).all()
    ids = np.sort(rng.choice(50, 20, replace=False))
    m3, v3 = orc.build_metadata(rows, 0.9, sample_ids=ids)
    m4, v4 = orc.build_metadata(rows[ids], 0.9)
    assert (m3 == m4).all() and (v3 == v4).all()


# --------------------------------------------------------------------------
# compression / decompression properties

def _chunk_table(B, C):
    n_c = (B + C - 1) // C
    return [(c * C // 4, min((c + 1) * C, B) // 4) for c in range(n_c)]


def check_store(orc, bmi2, rows, mask, bitval, C, store, pb, lens, slot, first=0):
    """Checks one compressed store against the definitions.

    For every tensor: (1) the participation bit of each chunk is exactly
    'all Mask bits match Bitval and the chunk has a Mask bit'; (2) the payload
    is the BMI2 PEXT stream of the tensor with selector ~Mask on participating
    chunks and all-ones on the others (bit order and gap-free concatenation);
    (3) its length is ceil((sum of kept bits)/8) <= B; (4) decode is lossless.
    """
    n, B = rows.shape[0], 4 * rows.shape[1]
    chunks = _chunk_table(B, C)
    n_c = len(chunks)
    keep_bits = np.unpackbits((~mask).view(np.uint8), bitorder="little")
    k_c = np.array([int(keep_bits[32 * a:32 * b].sum()) for a, b in chunks])
    bits_c = np.array([32 * (b - a) for a, b in chunks])
    P = _bits_le(pb)
    full = U32(0xFFFFFFFF)
    for i in range(n):
        x = rows[i]
        t = first + i
        part = [int(P[t * n_c + c]) for c in range(n_c)]
        for c, (a, b) in enumerate(chunks):
            match = bool(((x[a:b] ^ bitval[a:b]) & mask[a:b] == 0).all())
            assert part[c] == int(match and k_c[c] < bits_c[c]), (t, c)
        sel = np.empty_like(mask)
        for c, (a, b) in enumerate(chunks):
            sel[a:b] = ~mask[a:b] if part[c] else full
        want, nbits = bmi2.pack(_bytes(x), _bytes(sel))
        assert nbits == sum(k_c[c] if part[c] else bits_c[c] for c in range(n_c))
        assert int(lens[i]) == (nbits + 7) // 8 <= B, (t, int(lens[i]), nbits)
        got = store[t * slot:t * slot + int(lens[i])].tobytes()
        assert got == want, ("payload differs from PEXT", t)
        # PDEP of the payload into the kept positions, plus Bitval, is x
        back = np.frombuffer(bmi2.unpack(got, _bytes(sel), B), U32)
        back = back | (bitval & ~sel)
        assert (back == x).all(), ("PDEP decode", t)


def _random_case(rng, n, words, kind):
    if kind == "float":
        x = (rng.standard_normal((n, words)) * rng.uniform(0.01, 3)).astype(np.float32)
        rows = x.view(U32)
    elif kind == "bytes":
        rows = rng.integers(0, 2 ** 32, (n, words), dtype=np.uint64).astype(U32)
    elif kind == "sparse":
        rows = (rng.random((n, words)) < 0.05).astype(np.float32).view(U32)
    else:  # near-constant: a base tensor with rare single-bit flips
        base = rng.integers(0, 2 ** 32, words, dtype=np.uint64).astype(U32)
        rows = np.tile(base, (n, 1))
        flips = rng.random((n, words)) < 0.02
        rows ^= np.where(flips, U32(1) << rng.integers(0, 32, (n, words)).astype(U32), U32(0))
    return np.ascontiguousarray(rows)


CASES = [  # (tensor bytes, chunk bytes) -- chunk > tensor, one partial chunk, many chunks
    (4, 256), (8, 4), (12, 8), (260, 256), (516, 256), (1028, 256), (512, 1024), (5732, 1024),
    (10240, 256), (2048, 4096),
]


def pin_roundtrip_and_format(orc, bmi2, rng):
    for (B, C) in CASES:
        for kind in ("float", "bytes", "sparse", "flips"):
            n = 24 if B > 2048 else 48
            rows = _random_case(rng, n, B // 4, kind)
            T = float(rng.choice([0.5, 0.75, 0.9, 0.99, 1.0]))
            mask, bitval = orc.build_metadata(rows, T)
            assert not (bitval & ~mask).any()
            slot = (B + 127) // 128 * 128
            store = np.full(n * slot, 0x5A, np.uint8)
            store, pb, lens = orc.compress(rows, mask, bitval, C, slot_bytes=slot, store=store)
            check_store(orc, bmi2, rows, mask, bitval, C, store, pb, lens, slot)
            ids = rng.integers(0, n, 2 * n)
            ids[:3] = [0, n - 1, 0]
            y = orc.gather_decompress(store, pb, n, ids, B, C, mask, bitval, slot_bytes=slot)
            assert (y == rows.view(np.uint8)[ids]).all(), (B, C, kind)


def pin_mask_zero_is_plain_gather(orc, rng):
    # Mask = 0: nothing is invariant, no chunk can save space, so the store is
    # the raw rows and gather + decompress is a plain row gather.
    B, C, n = 1024, 256, 40
    rows = _random_case(rng, n, B // 4, "bytes")
    zero = np.zeros(B // 4, U32)
    store, pb, lens = orc.compress(rows, zero, zero, C, slot_bytes=B)
    assert (lens == B).all() and not pb.any()
    assert (store.reshape(n, B) == rows.view(np.uint8)).all()
    ids = rng.integers(0, n, 77)
    y = orc.gather_decompress(store, pb, n, ids, B, C, zero, zero, slot_bytes=B)
    assert (y == np.take(rows.view(np.uint8), ids, axis=0)).all()


def pin_full_participation_independent_of_chunk(orc, bmi2, rng):
    # When every chunk participates the payload is the PEXT of the whole
    # tensor with selector ~Mask, whatever the chunk size.
    B = 4096
    mask = np.full(B // 4, 0x7F800000, U32)
    mask[::7] = 0xFFFF0000
    bitval = mask & U32(0x3C800000)
    rows = _random_case(rng, 8, B // 4, "bytes")
    rows = (rows & ~mask) | bitval
    want = [bmi2.pack(_bytes(r), _bytes(~mask))[0] for r in rows]
    for C in (256, 1024, 4096):
        store, pb, lens = orc.compress(rows, mask, bitval, C, slot_bytes=B)
        for i in range(8):
            assert store[i * B:i * B + int(lens[i])].tobytes() == want[i], C


def pin_compact(orc, rng):
    B, C, n = 520, 256, 30
    rows = _random_case(rng, n, B // 4, "float")
    mask, bitval = orc.build_metadata(rows, 0.9)
    slot = 640
    store, pb, lens = orc.compress(rows, mask, bitval, C, slot_bytes=slot)
    offsets, cache = orc.compact(store, slot, lens)
    # entries are 16-byte aligned and packed back to back
    pad = (lens.astype(np.uint64) + 15) // 16 * 16
    assert (offsets == np.concatenate([[0], np.cumsum(pad)]).astype(np.uint64)).all()
    for t in range(n):
        o, L = int(offsets[t]), int(lens[t])
        assert cache[o:o + L].tobytes() == store[t * slot:t * slot + L].tobytes()
        assert not cache[o + L:int(offsets[t + 1])].any()
    ids = rng.integers(0, n, 50)
    y1 = orc.gather_decompress(cache, pb, n, ids, B, C, mask, bitval, offsets=offsets)
    assert (y1 == rows.view(np.uint8)[ids]).all()


def pin_compact_aligned(orc, rng):
    """Aligned compaction ([G-EN] System Integration, cache compression, laid
    out on 128 B lines) and the rank index: every entry starts at a multiple of
    the alignment and is the smallest such multiple that holds its payload;
    with 16 it is the 16 B layout above; the cache round-trips; and for
    one-chunk tensors the entry offset follows from the index alone,
    t * s_r - r1(t) * (s_r - s_p), with s_p / s_r the aligned sizes of a
    packed payload (ceil(K / 8) bytes, K = bits not in the Mask) and of a
    whole tensor."""
    B, C, n = 512, 1024, 77
    rows = _random_case(rng, n, B // 4, "float")
    mask, bitval = orc.build_metadata(rows, 0.9)
    slot = 512
    store, pb, lens = orc.compress(rows, mask, bitval, C, slot_bytes=slot)
    o16, _ = orc.compact(store, slot, lens, with_cache=False)
    K = int(np.unpackbits(np.ascontiguousarray(~mask).view(np.uint8)).sum())
    P = _bits_le(pb)[:n].astype(bool)
    assert 0 < P.sum() < n, "the case should mix packed and whole tensors"
    # one-chunk tensors: a packed payload is ceil(K / 8) bytes, a whole one B
    assert (lens[P] == (K + 7) // 8).all() and (lens[~P] == B).all()
    for A in (16, 48, 64, 128, 256):
        offs, cache = orc.compact_aligned(store, slot, lens, A)
        size = np.diff(offs).astype(np.int64)
        assert (offs[:-1] % A == 0).all()
        assert (size >= lens).all() and (size - A < lens).all()
        if A == 16:
            assert (offs == o16).all()
        for t in range(n):
            o, L = int(offs[t]), int(lens[t])
            assert cache[o:o + L].tobytes() == store[t * slot:t * slot + L].tobytes()
            assert not cache[o + L:int(offs[t + 1])].any()
        ids = rng.integers(0, n, 40)
        y = orc.gather_decompress(cache, pb, n, ids, B, C, mask, bitval, offsets=offs)
        assert (y == rows.view(np.uint8)[ids]).all()
        # offsets from the rank index
        pb_dirty = pb.copy()
        pb_dirty[-1] |= np.uint32(0xFFFFFFFF << (n % 32) & 0xFFFFFFFF)  # bits past n are ignored
        index = orc.cache_index(pb_dirty, n)
        assert index.shape == ((n + 31) // 32,)
        assert ((index & np.uint64(0xFFFFFFFF)).astype(np.uint32) == pb).all()
        s_p = -(-((K + 7) // 8) // A) * A
        s_r = -(-B // A) * A
        for t in range(n):
            word, rank = int(index[t // 32]) & 0xFFFFFFFF, int(index[t // 32]) >> 32
            r1 = rank + bin(word & ((1 << (t % 32)) - 1)).count("1")
            assert int(offs[t]) == t * s_r - r1 * (s_r - s_p), (A, t)


def pin_invalid_ids(orc, rng):
    B, C, n = 64, 256, 5
    rows = _random_case(rng, n, B // 4, "float")
    mask, bitval = orc.build_metadata(rows, 0.9)
    store, pb, _ = orc.compress(rows, mask, bitval, C, slot_bytes=128)
    y = orc.gather_decompress(store, pb, n, [-1, 2, 5, 1 << 40], B, C, mask, bitval,
                              slot_bytes=128)
    assert not y[[0, 2, 3]].any() and (y[1] == rows.view(np.uint8)[2]).all()


def pin_brute_force(orc, rng):
    """The C oracle against the pure-Python brute force on tiny inputs."""
    for (B, C) in [(4, 256), (8, 4), (12, 8), (36, 16), (132, 64), (260, 256)]:
        for kind in ("float", "bytes", "flips", "sparse"):
            n = 12
            rows = _random_case(rng, n, B // 4, kind)
            T = float(rng.choice([0.5, 0.6, 0.8, 0.95, 1.0]))
            samples = [r.tobytes() for r in rows]
            rm, rv = ibp_ref.build_metadata(samples, T)
            mask, bitval = orc.build_metadata(rows, T)
            assert rm == _bytes(mask) and rv == _bytes(bitval), (B, C, kind, T)
            slot = (B + 127) // 128 * 128
            store, pb, lens = orc.compress(rows, mask, bitval, C, slot_bytes=slot)
            P = _bits_le(pb)
            n_c = (B + C - 1) // C
            for i in range(n):
                payload, part, nbits = ibp_ref.compress_one(samples[i], rm, rv, C)
                assert [int(b) for b in P[i * n_c:(i + 1) * n_c]] == part
                assert int(lens[i]) == len(payload)
                assert store[i * slot:i * slot + len(payload)].tobytes() == payload
                assert ibp_ref.decompress_one(payload, part, rm, rv, B, C) == samples[i]


def run_all(orc, bmi2, seed=1234):
    """Every pin, in order; raises AssertionError on the first violation."""
    rng = np.random.default_rng(seed)
    pin_hand_examples(orc)
    pin_metadata_hand(orc)
    pin_cutoff_boundaries(orc)
    pin_metadata_closed_forms(orc, rng)
    pin_mask_zero_is_plain_gather(orc, rng)
    pin_full_participation_independent_of_chunk(orc, bmi2, rng)
    pin_compact(orc, rng)
    pin_compact_aligned(orc, rng)
    pin_invalid_ids(orc, rng)
    pin_brute_force(orc, rng)
    pin_roundtrip_and_format(orc, bmi2, rng)
