"""The oracle for the Engram n-gram memory hot path: a ctypes front end to the
plain C implementation in ``engram_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
imports it and shares no code with it.  The one exception is building it:
``build()`` compiles the C source with gcc, and the package build step calls
that.

Every function here only moves numpy arrays across the C boundary.  The method
itself lives in the C file, where each step cites the page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_OK = 0
ORC_E_ARG = -1
ORC_E_ROWS = -2
ORC_E_VC = -3
ORC_E_NEED_STORE = -4
ORC_E_TOKEN = -5
ORC_E_NAN = -6
ORC_E_NOFIT = -7


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def build() -> str:
    """Compile liboracle.so with gcc: single-threaded, no fast-math, no FMA contraction."""
    cmd = [
        "gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        # ORACLE_LIB names another build of the same source (the sanitizer test runs
        # the pins against an AddressSanitizer / UBSan build this way)
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, u64 = ctypes.c_int64, ctypes.c_int, ctypes.c_uint64
        L.oracle_draw_primes.argtypes = [i32, i32, i32, u64, P]
        L.oracle_fit_layout.argtypes = [P, i32, P, P, P]
        L.oracle_layout_at_floor.argtypes = [P, i32, u64, P, P]
        L.oracle_compress_hash.argtypes = [i64, i64, i64, i32, P, P, P, P, i64, P, i64, P, P,
                                           P, i64, P, P, P]
        L.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_decode.restype = ctypes.c_float
        L.oracle_bf16_rne.argtypes = [ctypes.c_double]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_dequant_rows.argtypes = [P, P, i64, i64, i32, P, P]
        L.oracle_project.argtypes = [P, P, i64, i64, i64, P]
        L.oracle_gate_add.argtypes = [P, P, P, i64, i64, i64, P, P]
        L.oracle_site_layout.argtypes = [i32, i32, u64, i32, P, P]
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_dequant_rows_block32.argtypes = [P, P, i64, i64, P, P]
        _lib = L
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != ORC_OK:
        raise OracleError(rc, what)


def draw_primes(n_layers: int, max_ngram: int, n_heads: int, floor_: int) -> np.ndarray:
    """Primes [layer][order][head] drawn at and above ``floor_``."""
    out = np.zeros(n_layers * (max_ngram - 1) * n_heads, dtype=np.uint64)
    _check(lib().oracle_draw_primes(n_layers, max_ngram, n_heads, floor_, _ptr(out)), "draw_primes")
    return out.reshape(n_layers, max_ngram - 1, n_heads)


@dataclass
class OracleLayout:
    floor: int
    primes: np.ndarray   # uint64 [3][H]
    offsets: np.ndarray  # uint64 [3][H]

    @property
    def heads(self) -> int:
        return self.primes.shape[1]


def fit_layout(rows, n_heads: int) -> OracleLayout:
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint64))
    primes = np.zeros(3 * n_heads, dtype=np.uint64)
    offs = np.zeros(3 * n_heads, dtype=np.uint64)
    fl = np.zeros(1, dtype=np.uint64)
    _check(lib().oracle_fit_layout(_ptr(rows), n_heads, _ptr(fl), _ptr(primes), _ptr(offs)),
           "fit_layout")
    return OracleLayout(int(fl[0]), primes.reshape(3, n_heads), offs.reshape(3, n_heads))


def layout_at_floor(rows, n_heads: int, floor_: int) -> OracleLayout:
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.uint64))
    primes = np.zeros(3 * n_heads, dtype=np.uint64)
    offs = np.zeros(3 * n_heads, dtype=np.uint64)
    _check(lib().oracle_layout_at_floor(_ptr(rows), n_heads, floor_, _ptr(primes), _ptr(offs)),
           "layout_at_floor")
    return OracleLayout(int(floor_), primes.reshape(3, n_heads), offs.reshape(3, n_heads))


def site_layouts(n_sites: int, n_heads: int, floor_: int, per_site_table: bool) -> list:
    """One OracleLayout per site of a shared hash pass (site s draws its primes
    after sites 0..s-1)."""
    primes = np.zeros(n_sites * 3 * n_heads, dtype=np.uint64)
    offs = np.zeros(n_sites * 3 * n_heads, dtype=np.uint64)
    _check(lib().oracle_site_layout(n_sites, n_heads, floor_, 1 if per_site_table else 0,
                                    _ptr(primes), _ptr(offs)), "site_layout")
    p = primes.reshape(n_sites, 3, n_heads)
    o = offs.reshape(n_sites, 3, n_heads)
    return [OracleLayout(int(floor_), p[s].copy(), o[s].copy()) for s in range(n_sites)]


def _opt(a, dtype):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=dtype))


def compress_hash(layout: OracleLayout, *, vocab: int, vc: int, pad_token_id: int,
                  tid2eid, tokens, cu_seqlens, seq_start=None, slots=None, store=None,
                  dead=None):
    """Returns (eids int32[T], row_ids int32[T][3][H]); ``store`` (int32 [slots][3]) is
    updated in place when given."""
    tid2eid = _opt(tid2eid, np.int32)
    tokens = _opt(tokens, np.int32)
    cu = _opt(cu_seqlens, np.int32)
    ss = _opt(seq_start, np.uint8)
    sl = _opt(slots, np.int32)
    dd = _opt(dead, np.uint8)
    if store is not None:
        assert store.dtype == np.int32 and store.flags["C_CONTIGUOUS"]
    T = tokens.shape[0]
    S = cu.shape[0] - 1
    H = layout.heads
    eids = np.zeros(T, dtype=np.int32)
    rows = np.zeros((T, 3, H), dtype=np.int32)
    primes = np.ascontiguousarray(layout.primes.reshape(-1), dtype=np.uint64)
    offs = np.ascontiguousarray(layout.offsets.reshape(-1), dtype=np.uint64)
    rc = lib().oracle_compress_hash(
        vocab, vc, pad_token_id, H, _ptr(primes), _ptr(offs), _ptr(tid2eid), _ptr(tokens), T,
        _ptr(cu), S, _ptr(ss), _ptr(sl), _ptr(store), 0 if store is None else store.shape[0],
        _ptr(dd), _ptr(eids), _ptr(rows))
    _check(rc, "compress_hash")
    return eids, rows


def e4m3fn_decode(b: int) -> float:
    return float(lib().oracle_e4m3fn_decode(b))


def bf16_rne(x: float) -> int:
    return int(lib().oracle_bf16_rne(float(x)))


def dequant_rows(rows, scales, *, bf16_table: bool = False):
    """rows: uint8 [n][D] (fp8) or uint16 [n][D] (bf16 bits); scales: float32 [n] or None.
    Returns (f32 [n][D], bf16 bits uint16 [n][D])."""
    rows = np.ascontiguousarray(rows)
    n, D = rows.shape
    raw = rows.view(np.uint8)
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    f32 = np.zeros((n, D), dtype=np.float32)
    b16 = np.zeros((n, D), dtype=np.uint16)
    rc = lib().oracle_dequant_rows(_ptr(raw), _ptr(sc), n, D, 1 if bf16_table else 0,
                                   _ptr(f32), _ptr(b16))
    _check(rc, "dequant_rows")
    return f32, b16


def e8m0_decode(b: int) -> float:
    return float(lib().oracle_e8m0_decode(b))


def dequant_rows_block32(rows, scales):
    """rows: uint8 [n][D] e4m3fn bytes; scales: uint8 [n][D/32] e8m0 bytes.
    Returns (f32 [n][D], bf16 bits uint16 [n][D])."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    sc = np.ascontiguousarray(scales, dtype=np.uint8)
    n, D = rows.shape
    assert sc.shape == (n, D // 32)
    f32 = np.zeros((n, D), dtype=np.float32)
    b16 = np.zeros((n, D), dtype=np.uint16)
    _check(lib().oracle_dequant_rows_block32(_ptr(rows), _ptr(sc), n, D, _ptr(f32), _ptr(b16)),
           "dequant_rows_block32")
    return f32, b16


def project(E_bf16, W_bf16) -> np.ndarray:
    """E: uint16 bf16 bits [T][K]; W: uint16 bf16 bits [hidden][K] -> fp64 [T][hidden]."""
    E = np.ascontiguousarray(E_bf16, dtype=np.uint16)
    W = np.ascontiguousarray(W_bf16, dtype=np.uint16)
    T, K = E.shape
    hidden, K2 = W.shape
    assert K == K2
    v = np.zeros((T, hidden), dtype=np.float64)
    _check(lib().oracle_project(_ptr(E), _ptr(W), T, K, hidden, _ptr(v)), "project")
    return v


def gate_add(x_bf16, v, keep=None):
    """x: uint16 bf16 bits [T][hc][hidden]; v: fp64 [T][hidden]; keep: [T] or None.
    Returns (y bf16 bits [T][hc][hidden], gates fp64 [T][hc])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.float64)
    T, hc, hidden = x.shape
    kp = _opt(keep, np.uint8)
    y = np.zeros_like(x)
    g = np.zeros((T, hc), dtype=np.float64)
    _check(lib().oracle_gate_add(_ptr(x), _ptr(v), _ptr(kp), T, hc, hidden, _ptr(y), _ptr(g)),
           "gate_add")
    return y, g
