"""ctypes front end of tests/helpers/bmi2_helper.c (PEXT/PDEP reference)."""
import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


class Bmi2:
    def __init__(self, path):
        L = ctypes.CDLL(path)
        L.pext_stream.restype = ctypes.c_uint64
        L.pext_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                  ctypes.c_void_p, ctypes.c_uint64]
        L.pdep_stream.restype = None
        L.pdep_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                  ctypes.c_void_p]
        self.lib = L

    @staticmethod
    def _words(b):
        b = np.ascontiguousarray(b).view(np.uint8).ravel()
        pad = (-b.size) % 8
        return np.concatenate([b, np.zeros(pad, np.uint8)]).view(np.uint64)

    def pack(self, x, keep):
        """PEXT-pack the bits of byte string x selected by byte string keep.
        Returns (payload bytes, number of bits)."""
        xs, ks = self._words(x), self._words(keep)
        dst = np.zeros(xs.size * 8 + 8, np.uint8)
        nbits = self.lib.pext_stream(xs.ctypes.data, ks.ctypes.data, xs.size, dst.ctypes.data,
                                     dst.size)
        return dst[:(nbits + 7) // 8].tobytes(), int(nbits)

    def unpack(self, payload, keep, n_bytes):
        """PDEP-unpack a payload into the positions selected by keep."""
        ks = self._words(keep)
        src = np.zeros(len(payload) + 16, np.uint8)
        src[:len(payload)] = np.frombuffer(payload, np.uint8)
        dst = np.zeros(ks.size, np.uint64)
        self.lib.pdep_stream(src.ctypes.data, ks.ctypes.data, ks.size, dst.ctypes.data)
        return dst.view(np.uint8)[:n_bytes].tobytes()


def load(workdir):
    src = os.path.join(HERE, "bmi2_helper.c")
    out = os.path.join(workdir, "libbmi2_helper.so")
    subprocess.run(["gcc", "-O2", "-mbmi2", "-mpopcnt", "-fPIC", "-shared", src, "-o", out],
                   check=True)
    return Bmi2(out)
