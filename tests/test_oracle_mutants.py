"""Planted mistakes in copies of the oracle must each fail some pin.

Every mutant below is one plausible slip in oracle/ibp_oracle.c (a dropped
term, a wrong comparison, a wrong bit order or index).  The test writes the
mutated source to a temporary directory, builds it with gcc and runs every pin
of tests/oracle_pins.py against it in a child process (so a mutant that
crashes cannot take the test run down); the child must fail.  The real
oracle's source is never modified.
"""
import os
import subprocess
import sys

import pytest

from oracle import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = [
    ("cutoff rounds down", [("return (int64_t)ceil(threshold * (double)n);",
                             "return (int64_t)floor(threshold * (double)n);")]),
    ("strict cutoff", [("const unsigned inv = (int64_t)top >= m;",
                        "const unsigned inv = (int64_t)top > m;")]),
    ("tie counts as one", [("put_bit(bitval, i, inv && n1 > n0);",
                            "put_bit(bitval, i, inv && n1 >= n0);")]),
    ("zero count off by one", [("const uint64_t n0 = n_samples - n1;",
                                "const uint64_t n0 = n_samples - n1 - 1;")]),
    ("participation ignores the saving rule", [("const unsigned p = match && k < hi - lo;",
                                                "const unsigned p = match;")]),
    ("match ignores Bitval", [("if (get_bit(x, b) != get_bit(bitval, b))",
                               "if (get_bit(x, b) != 0)")]),
    ("raw chunk drops invariant bits", [("if (!p || !get_bit(mask, b))",
                                         "if (!get_bit(mask, b))")]),
    ("MSB-first bit order", [("return (p[i / 8] >> (i % 8)) & 1u;",
                              "return (p[i / 8] >> (7 - i % 8)) & 1u;"),
                             ("uint8_t m = (uint8_t)(1u << (i % 8));",
                              "uint8_t m = (uint8_t)(1u << (7 - i % 8));")]),
    ("bitmap index transposed", [("put_map_bit(part_bits, (first_tensor + i) * n_c + c,",
                                  "put_map_bit(part_bits, (first_tensor + i) + c * n_rows,"),
                                 ("get_map_bit(part_bits, (uint64_t)t * n_c + c)",
                                  "get_map_bit(part_bits, (uint64_t)t + c * n_tensors)")]),
    ("decode takes Mask for Bitval", [("v = get_bit(bitval, b);", "v = get_bit(mask, b);")]),
    ("decode ignores participation", [("if (p && get_bit(mask, b))", "if (get_bit(mask, b))")]),
    ("compact aligns to 8 bytes", [("(((uint64_t)lengths[t] + 15) / 16) * 16",
                                    "(((uint64_t)lengths[t] + 7) / 8) * 8")]),
    ("aligned entry one unit too large", [("while (size < lengths[t])", "while (size <= lengths[t])")]),
    ("rank counts its own word", [("index[w] = (before << 32) | word;\n        for (unsigned b = 0; b < 32; b++)\n            before += (word >> b) & 1;",
                                   "for (unsigned b = 0; b < 32; b++)\n            before += (word >> b) & 1;\n        index[w] = (before << 32) | word;")]),
    ("last byte not cleared", [("memset(out, 0, tensor_bytes);", "(void)0;")]),
    ("partial last chunk dropped", [("return (tensor_bytes + chunk_bytes - 1) / chunk_bytes;",
                                     "return tensor_bytes / chunk_bytes;")]),
    ("chunk size read as bits", [("const uint64_t lo = c * chunk_bytes * 8;",
                                  "const uint64_t lo = c * chunk_bytes;"),
                                 ("uint64_t hi = (c + 1) * chunk_bytes * 8;",
                                  "uint64_t hi = (c + 1) * chunk_bytes;")]),
]

CHILD = """
import sys
sys.path.insert(0, {root!r})
from oracle.oracle import Oracle
from tests.helpers import bmi2
from tests import oracle_pins
oracle_pins.run_all(Oracle({lib!r}), bmi2.load({work!r}))
"""


@pytest.mark.slow
@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, edits, tmp_path):
    src = open(build.SRC).read()
    for old, new in edits:
        # every occurrence is edited, so compression and decompression stay consistent
        assert old in src, f"mutant '{name}' no longer matches the oracle source: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = build.build(src=str(path), out=str(tmp_path / "libmutant.so"), werror=False)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=lib, work=str(tmp_path))],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant '{name}' passed every pin"
