"""ctypes front of the fp32 C oracle (``mq_oracle_c.c``).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests and the CPU
baseline of ``bench.py`` call it; nothing on the product path does.  The
functions mirror ``mq_oracle``'s signatures and array layouts (bf16 bit
patterns in uint16, codes in uint32 words) and return the product in fp32,
accumulated in fp32 (k ascending, one fused multiply-add per step).

``load()`` compiles the library with gcc next to its source when it is
missing or older than the source; ``load(mutant=NAME)`` builds a copy with one
planted mistake (``MQ_MUTANT_<NAME>``), for the tests that show the pins
catch it.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mq_oracle_c.c")
LIB = os.path.join(HERE, "libmq_oracle_c.so")
MUTANTS = ("NO_BIAS", "ROUND_AWAY", "GROUP_SHIFT", "UNSTABLE", "SKIP_LAST_K")

_libs: dict = {}


def _compile(out: str, defines=()) -> None:
    gcc = shutil.which("gcc") or shutil.which("cc")
    if not gcc:
        raise RuntimeError("no C compiler (gcc) for the C oracle")
    tmp = out + f".tmp{os.getpid()}"
    cmd = [gcc, "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", *[f"-D{d}" for d in defines], SRC, "-o", tmp, "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C oracle build failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)


def build() -> str:
    """Compile the library in place (always); returns its path."""
    _compile(LIB)
    return LIB


def load(mutant: str | None = None) -> ctypes.CDLL:
    key = mutant or ""
    if key in _libs:
        return _libs[key]
    if mutant is None:
        path = LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
            _compile(path)
    else:
        if mutant not in MUTANTS:
            raise ValueError(mutant)
        path = os.path.join(tempfile.mkdtemp(prefix="mqo_mutant_"), f"libmq_oracle_{mutant}.so")
        _compile(path, [f"MQ_MUTANT_{mutant}"])
    lib = ctypes.CDLL(path)
    P, I64, I32, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.mqo_threads.argtypes, lib.mqo_threads.restype = [I], I
    lib.mqo_quantize.argtypes = [P, I64, I64, I, I, P, P, P]
    lib.mqo_dequantize.argtypes = [P, P, P, I64, I64, I, I, P]
    lib.mqo_route.argtypes = [P, I64, I32, P, P, P]
    lib.mqo_gather_qmm.argtypes = [P, I64, I64, I64, P, P, P, I32, I64, I64, P, I64, I, I, I, P]
    for f in (lib.mqo_quantize, lib.mqo_dequantize, lib.mqo_route, lib.mqo_gather_qmm):
        f.restype = I
    _libs[key] = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """The C oracle's functions (a planted-mistake copy with ``mutant``)."""

    def __init__(self, mutant: str | None = None):
        self.lib = load(mutant)

    def threads(self, n: int = 0) -> int:
        return int(self.lib.mqo_threads(n))

    def quantize(self, w_bits, group_size: int, bits: int):
        w = np.ascontiguousarray(w_bits, dtype=np.uint16)
        K = w.shape[-1]
        if bits not in (4, 8) or K % group_size:
            raise ValueError("unsupported quantisation parameters")
        rows = w.size // K
        lead = w.shape[:-1]
        wq = np.empty(lead + (K * bits // 32,), np.uint32)
        s = np.empty(lead + (K // group_size,), np.uint16)
        b = np.empty_like(s)
        if self.lib.mqo_quantize(_p(w), rows, K, group_size, bits, _p(wq), _p(s), _p(b)):
            raise ValueError("unsupported quantisation parameters")
        return wq, s, b

    def dequantize(self, wq, scales, biases, group_size: int, bits: int):
        wq = np.ascontiguousarray(wq, dtype=np.uint32)
        s = np.ascontiguousarray(scales, dtype=np.uint16)
        b = np.ascontiguousarray(biases, dtype=np.uint16)
        C = wq.shape[-1] * (32 // bits)
        out = np.empty(wq.shape[:-1] + (C,), np.float32)
        if self.lib.mqo_dequantize(_p(wq), _p(s), _p(b), wq.size // wq.shape[-1], C, group_size,
                                   bits, _p(out)):
            raise ValueError("unsupported quantisation parameters")
        return out

    def route(self, idx, E: int):
        flat = np.ascontiguousarray(np.asarray(idx).reshape(-1), dtype=np.int32)
        counts = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        perm = np.empty(flat.size, np.int32)
        st = self.lib.mqo_route(_p(flat), flat.size, E, _p(counts), _p(offsets), _p(perm))
        if st == -1:
            raise ValueError(f"expert index outside [0, {E})")
        if st:
            raise MemoryError("C oracle")
        return counts.astype(np.int64), offsets.astype(np.int64), perm.astype(np.int64)

    def gather_qmm(self, x_bits, wq, scales, biases, rhs_indices, group_size: int, bits: int,
                   transpose: bool = True):
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        wq = np.ascontiguousarray(wq, dtype=np.uint32)
        s = np.ascontiguousarray(scales, dtype=np.uint16)
        b = np.ascontiguousarray(biases, dtype=np.uint16)
        idx = np.ascontiguousarray(rhs_indices, dtype=np.int32)
        T, A = idx.shape
        _, Ax, M, KI = x.shape
        E, R = wq.shape[0], wq.shape[1]
        C = wq.shape[2] * (32 // bits)
        if KI != (C if transpose else R):
            raise ValueError("x's features do not match the stored weight")
        NO = R if transpose else C
        out = np.empty((T, A, M, NO), np.float32)
        st = self.lib.mqo_gather_qmm(_p(x), T, Ax, M, _p(wq), _p(s), _p(b), E, R, C, _p(idx), A,
                                     int(bool(transpose)), group_size, bits, _p(out))
        if st == -1:
            raise ValueError("bad parameters or an expert index outside [0, E)")
        if st:
            raise MemoryError("C oracle")
        return out

    def qmm(self, x_bits, wq, scales, biases, group_size: int, bits: int, transpose: bool = True):
        x = np.asarray(x_bits, dtype=np.uint16)
        M, K = x.shape
        out = self.gather_qmm(x.reshape(M, 1, 1, K), np.asarray(wq)[None], np.asarray(scales)[None],
                              np.asarray(biases)[None], np.zeros((M, 1), np.int32), group_size, bits,
                              transpose)
        return out.reshape(M, -1)
