"""CPU oracle for the W4A8 linear layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The HIP library never does, and this package
never imports the HIP library: the two share nothing but the seeded input
generator.

The arithmetic lives in ``oracle.c`` (plain C loops, see its header for the
passages each step follows).  This module compiles it with gcc and wraps it
with ctypes over numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIBS: dict[int, ctypes.CDLL] = {}

OK = 0
BAD_ARG = -1
NONFINITE = -2
RANGE = -3
P_BOUND = 128 * 127 * 15


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, out: str | None = None) -> str:
    """Compile the oracle (optionally with one planted mistake) with gcc.

    Plain -O2: no fast-math, no FMA contraction, IEEE float division."""
    out = out or lib_path(mutant)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall",
           f"-DORACLE_MUTANT={mutant}", _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(mutant: int = 0) -> ctypes.CDLL:
    if mutant in _LIBS:
        return _LIBS[mutant]
    path = lib_path(mutant)
    if mutant != 0 or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build(mutant)
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_version.restype = ctypes.c_int
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    for name, args in {
        "oracle_quant_act_f32": [vp, i64, i64, vp, vp],
        "oracle_quant_act_bf16": [vp, i64, i64, vp, vp],
        "oracle_group_partials": [vp, vp, vp, i64, i64, i64, i32, i64, i64, vp],
        "oracle_linear": [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, i64, i64, i64, vp],
        "oracle_layout_pack": [vp, vp, vp, i64, i64, vp],
        "oracle_layout_unpack": [vp, i64, i64, vp, vp, vp],
        "oracle_w8a8_totals": [vp, vp, i64, i64, i64, i64, i64, vp],
        "oracle_hadamard_rows": [vp, i32, i64, i64, vp],
        "oracle_w4a16_linear": [vp, i32, vp, vp, vp, i64, i64, i64, i32, i64, i64, i64, i64, vp],
        "oracle_hadamard_quant_act": [vp, i32, i64, i64, vp, vp],
        "oracle_w8a8_linear": [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, vp],
        "oracle_w8_layout_pack": [vp, vp, i64, i64, vp],
        "oracle_w8_layout_unpack": [vp, i64, i64, vp, vp],
    }.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.oracle_layout_bytes.argtypes = [i64, i64]
    lib.oracle_layout_bytes.restype = i64
    lib.oracle_w8_layout_bytes.argtypes = [i64, i64]
    lib.oracle_w8_layout_bytes.restype = i64
    _LIBS[mutant] = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what} returned {rc}")


def quant_act(x: np.ndarray, mutant: int = 0):
    """x: float32 [M][K] or uint16 bf16 bit patterns [M][K] -> (qa int8, sa float32)."""
    lib = load(mutant)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    qa = np.empty((M, K), np.int8)
    sa = np.empty((M,), np.float32)
    if x.dtype == np.float32:
        _check(lib.oracle_quant_act_f32(_ptr(x), M, K, _ptr(qa), _ptr(sa)), "quant_act_f32")
    elif x.dtype == np.uint16:
        _check(lib.oracle_quant_act_bf16(_ptr(x), M, K, _ptr(qa), _ptr(sa)), "quant_act_bf16")
    else:
        raise TypeError(x.dtype)
    return qa, sa


def hadamard_rows(x, mutant: int = 0):
    """Rows rotated group by group by the unnormalised 128 x 128 Walsh-Hadamard
    matrix, in float32 by the butterflies of increasing stride."""
    lib = load(mutant)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    if x.dtype not in (np.float32, np.uint16):
        raise TypeError(x.dtype)
    xr = np.empty((M, K), np.float32)
    _check(lib.oracle_hadamard_rows(_ptr(x), int(x.dtype == np.uint16), M, K, _ptr(xr)),
           "hadamard_rows")
    return xr


def hadamard_quant_act(x, mutant: int = 0):
    """Rotation, then the per-token quantisation: (qa int8, sa float32)."""
    lib = load(mutant)
    x = np.ascontiguousarray(x)
    M, K = x.shape
    if x.dtype not in (np.float32, np.uint16):
        raise TypeError(x.dtype)
    qa = np.empty((M, K), np.int8)
    sa = np.empty((M,), np.float32)
    _check(lib.oracle_hadamard_quant_act(_ptr(x), int(x.dtype == np.uint16), M, K, _ptr(qa),
                                         _ptr(sa)), "hadamard_quant_act")
    return qa, sa


def group_partials(qa, q, z, group=128, m0=0, m1=None, mutant: int = 0):
    """Exact per-group int32 partials P[m1-m0][N][G]."""
    lib = load(mutant)
    qa = np.ascontiguousarray(qa, np.int8)
    q = np.ascontiguousarray(q, np.uint8)
    z = np.ascontiguousarray(z, np.uint8)
    M, K = qa.shape
    N = q.shape[0]
    m1 = M if m1 is None else m1
    P = np.empty((m1 - m0, N, K // group), np.int32)
    _check(lib.oracle_group_partials(_ptr(qa), _ptr(q), _ptr(z), M, N, K, group, m0, m1, _ptr(P)),
           "group_partials")
    return P


def linear(qa, sa, q, z, s, group=128, rows=None, cols=None, mutant: int = 0):
    """Unrounded float64 y[rows][cols] = sa[m] * sum_g s[n,g] * P[m,n,g]."""
    lib = load(mutant)
    qa = np.ascontiguousarray(qa, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    q = np.ascontiguousarray(q, np.uint8)
    z = np.ascontiguousarray(z, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    M, K = qa.shape
    N = q.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    n0, n1 = cols if cols is not None else (0, N)
    y = np.empty((m1 - m0, n1 - n0), np.float64)
    _check(lib.oracle_linear(_ptr(qa), _ptr(sa), _ptr(q), _ptr(z), _ptr(s), M, N, K, group,
                             m0, m1, n0, n1, _ptr(y)), "linear")
    return y


def w8a8_totals(qa, qw, m0=0, m1=None, mutant: int = 0):
    """W8A8: exact integer products over all of K, P[m1-m0][N] (int32)."""
    lib = load(mutant)
    qa = np.ascontiguousarray(qa, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, K = qa.shape
    N = qw.shape[0]
    m1 = M if m1 is None else m1
    P = np.empty((m1 - m0, N), np.int32)
    _check(lib.oracle_w8a8_totals(_ptr(qa), _ptr(qw), M, N, K, m0, m1, _ptr(P)), "w8a8_totals")
    return P


def w8a8_linear(qa, sa, qw, sw, rows=None, cols=None, mutant: int = 0):
    """W8A8: unrounded float64 y[rows][cols] = sa[m] * (sw[n] * P[m][n])."""
    lib = load(mutant)
    qa = np.ascontiguousarray(qa, np.int8)
    sa = np.ascontiguousarray(sa, np.float32)
    qw = np.ascontiguousarray(qw, np.int8)
    sw = np.ascontiguousarray(sw, np.float32)
    M, K = qa.shape
    N = qw.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    n0, n1 = cols if cols is not None else (0, N)
    y = np.empty((m1 - m0, n1 - n0), np.float64)
    _check(lib.oracle_w8a8_linear(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, m0, m1, n0, n1,
                                  _ptr(y)), "w8a8_linear")
    return y


def w8_layout_bytes(N: int, K: int) -> int:
    return int(load().oracle_w8_layout_bytes(N, K))


def w8_layout_pack(qw, sw):
    lib = load()
    qw = np.ascontiguousarray(qw, np.int8)
    sw = np.ascontiguousarray(sw, np.float32)
    N, K = qw.shape
    out = np.empty((w8_layout_bytes(N, K),), np.uint8)
    _check(lib.oracle_w8_layout_pack(_ptr(qw), _ptr(sw), N, K, _ptr(out)), "w8_layout_pack")
    return out


def w8_layout_unpack(buf, N: int, K: int):
    lib = load()
    buf = np.ascontiguousarray(buf, np.uint8)
    qw = np.empty((N, K), np.int8)
    sw = np.empty((N,), np.float32)
    _check(lib.oracle_w8_layout_unpack(_ptr(buf), N, K, _ptr(qw), _ptr(sw)), "w8_layout_unpack")
    return qw, sw


def w4a16_linear(x, q, z, s, group=128, rows=None, cols=None, mutant: int = 0):
    """W4A16: unrounded float64 y = sum_g s * sum_k x * (q - z), x as given
    (float32, or uint16 bf16 bit patterns widened exactly)."""
    lib = load(mutant)
    x = np.ascontiguousarray(x)
    if x.dtype not in (np.float32, np.uint16):
        raise TypeError(x.dtype)
    q = np.ascontiguousarray(q, np.uint8)
    z = np.ascontiguousarray(z, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    M, K = x.shape
    N = q.shape[0]
    m0, m1 = rows if rows is not None else (0, M)
    n0, n1 = cols if cols is not None else (0, N)
    y = np.empty((m1 - m0, n1 - n0), np.float64)
    _check(lib.oracle_w4a16_linear(_ptr(x), int(x.dtype == np.uint16), _ptr(q), _ptr(z), _ptr(s),
                                   M, N, K, group, m0, m1, n0, n1, _ptr(y)), "w4a16_linear")
    return y


def threads() -> int:
    """OpenMP threads the oracle's loops use."""
    return int(load().oracle_threads())


def set_threads(n: int) -> None:
    """Run the oracle's later calls on n OpenMP threads (timing only)."""
    if load().oracle_set_threads(int(n)) != 0:
        raise ValueError(f"oracle: cannot run on {n} threads")


def layout_bytes(N: int, K: int) -> int:
    return int(load().oracle_layout_bytes(N, K))


def layout_pack(q, z, s):
    lib = load()
    q = np.ascontiguousarray(q, np.uint8)
    z = np.ascontiguousarray(z, np.uint8)
    s = np.ascontiguousarray(s, np.float32)
    N, K = q.shape
    out = np.empty((layout_bytes(N, K),), np.uint8)
    _check(lib.oracle_layout_pack(_ptr(q), _ptr(z), _ptr(s), N, K, _ptr(out)), "layout_pack")
    return out


def layout_unpack(buf, N: int, K: int):
    lib = load()
    buf = np.ascontiguousarray(buf, np.uint8)
    G = K // 128
    q = np.empty((N, K), np.uint8)
    z = np.empty((N, G), np.uint8)
    s = np.empty((N, G), np.float32)
    _check(lib.oracle_layout_unpack(_ptr(buf), N, K, _ptr(q), _ptr(z), _ptr(s)), "layout_unpack")
    return q, z, s


def tolerance_ok(y_bf16_as_f32: np.ndarray, y_ref: np.ndarray, rel: float = 4e-3):
    """max|y - y_ref| <= rel * max|y_ref| over the tensor; returns (ok, err, bound)."""
    err = float(np.max(np.abs(y_bf16_as_f32.astype(np.float64) - y_ref))) if y_ref.size else 0.0
    bound = rel * float(np.max(np.abs(y_ref))) if y_ref.size else 0.0
    return err <= bound, err, bound


if __name__ == "__main__":  # pragma: no cover
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else 0))
