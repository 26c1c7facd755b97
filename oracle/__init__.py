"""CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``etg_oracle.c`` -- plain
scalar loops with float64 accumulation -- through ctypes.  It shares no code
with the HIP library and never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, Q8_0, F16 = 0, 1, 2, 3
WIRE_F32, WIRE_F16, WIRE_I8 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "etg_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# ETG_ORACLE_LIBRARY loads another build of the same source (e.g. with sanitizers)
_LOAD = os.environ.get("ETG_ORACLE_LIBRARY") or _LIB
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-Wall", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LOAD == _LIB and not os.path.exists(_LIB):
        build(force=True)
    L = ctypes.CDLL(_LOAD)
    i64, i32, f32p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    vp = ctypes.c_void_p
    L.orc_row_bytes.restype = i64
    L.orc_row_bytes.argtypes = [ctypes.c_int, i64]
    L.orc_f16_to_f64.restype = ctypes.c_double
    L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_bf16_to_f64.restype = ctypes.c_double
    L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_f16_array.argtypes = [vp, i64, vp]
    L.orc_bf16_array.argtypes = [vp, i64, vp]
    L.orc_dequant_row.argtypes = [vp, ctypes.c_int, i64, vp]
    L.orc_sqrt_d.restype = ctypes.c_float
    L.orc_sqrt_d.argtypes = [i64]
    L.orc_embed_gather.restype = i64
    L.orc_embed_gather.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, ctypes.c_float, ctypes.c_int, vp]
    L.orc_logits.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp]
    L.orc_topk.argtypes = [vp, i64, i64, i32, vp, vp]
    L.orc_logits_at.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp, i64, vp, vp]
    L.orc_log_partition.argtypes = [vp, i64, i64, ctypes.c_double, vp]
    L.orc_probs_at.argtypes = [vp, vp, i64, i64, ctypes.c_double, vp, i32, vp]
    L.orc_wire_row_bytes.restype = i64
    L.orc_wire_row_bytes.argtypes = [ctypes.c_int, i64]
    L.orc_f32_to_f16_sat.restype = ctypes.c_uint16
    L.orc_f32_to_f16_sat.argtypes = [ctypes.c_float]
    L.orc_wire_encode.argtypes = [vp, i64, i64, ctypes.c_int, vp]
    L.orc_wire_decode.argtypes = [vp, i64, i64, ctypes.c_int, vp]
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_max_threads.restype = ctypes.c_int
    _lib = L
    return L


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _bytes(table: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(table).reshape(-1).view(np.uint8)


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


def row_bytes(dtype: int, hidden: int) -> int:
    return int(_load().orc_row_bytes(int(dtype), int(hidden)))


def f16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(b.size, np.float64)
    _load().orc_f16_array(_p(b), b.size, _p(out))
    return out.reshape(np.shape(bits))


def bf16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    out = np.empty(b.size, np.float64)
    _load().orc_bf16_array(_p(b), b.size, _p(out))
    return out.reshape(np.shape(bits))


def dequant_row(row: np.ndarray, dtype: int, hidden: int) -> np.ndarray:
    rb = row_bytes(dtype, hidden)
    raw = _bytes(row)
    if raw.size != rb:
        raise ValueError(f"row has {raw.size} bytes, expected {rb}")
    out = np.empty(hidden, np.float64)
    _load().orc_dequant_row(_p(raw), int(dtype), int(hidden), _p(out))
    return out


def sqrt_d(hidden: int) -> np.float32:
    return np.float32(_load().orc_sqrt_d(int(hidden)))


def _check_table(table, dtype, V, hidden):
    raw = _bytes(table)
    rb = row_bytes(dtype, hidden)
    if rb < 0 or raw.size != V * rb:
        raise ValueError(f"table holds {raw.size} bytes, expected {V}*{rb}")
    return raw


def embed_gather(table, dtype: int, V: int, hidden: int, ids, scale=None):
    """Returns (out f32 [n, hidden], number of bad ids).  scale: None, or an f32 value."""
    raw = _check_table(table, dtype, V, hidden)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
    out = np.empty((ids.size, hidden), np.float32)
    use = 0 if scale is None else 1
    sc = 1.0 if scale is None else float(np.float32(scale))
    bad = _load().orc_embed_gather(_p(raw), int(dtype), int(V), int(hidden), _p(ids), ids.size,
                                   sc, use, _p(out))
    return out, int(bad)


def logits(table, dtype: int, V: int, hidden: int, R):
    """Returns (L, A): float64 [B, V] logits and sum of |products|."""
    raw = _check_table(table, dtype, V, hidden)
    R = np.ascontiguousarray(R, dtype=np.float32).reshape(-1, hidden)
    B = R.shape[0]
    L = np.empty((B, V), np.float64)
    A = np.empty((B, V), np.float64)
    _load().orc_logits(_p(raw), int(dtype), int(V), int(hidden), _p(R), B, _p(L), _p(A))
    return L, A


def topk(L, k: int):
    """Returns (ids int32 [B, k], scores f32 [B, k]) ordered by logit desc, id asc."""
    L = np.ascontiguousarray(L, dtype=np.float64)
    if L.ndim == 1:
        L = L[None, :]
    B, V = L.shape
    if not 1 <= k <= V:
        raise ValueError("k out of range")
    ids = np.empty((B, k), np.int32)
    sc = np.empty((B, k), np.float32)
    _load().orc_topk(_p(L), B, V, int(k), _p(ids), _p(sc))
    return ids, sc


def logits_at(table, dtype: int, V: int, hidden: int, R, bs, vids):
    """Logit and |product| sum at selected (batch row, vocabulary id) pairs."""
    raw = _check_table(table, dtype, V, hidden)
    R = np.ascontiguousarray(R, dtype=np.float32).reshape(-1, hidden)
    bs = np.ascontiguousarray(bs, dtype=np.int64).reshape(-1)
    vids = np.ascontiguousarray(vids, dtype=np.int32).reshape(-1)
    if bs.size != vids.size:
        raise ValueError("bs and vids differ in length")
    if bs.size and (bs.min() < 0 or bs.max() >= R.shape[0]):
        raise ValueError("batch index out of range")
    oL = np.empty(bs.size, np.float64)
    oA = np.empty(bs.size, np.float64)
    _load().orc_logits_at(_p(raw), int(dtype), int(V), int(hidden), _p(R), _p(bs), _p(vids),
                          bs.size, _p(oL), _p(oA))
    return oL, oA


def log_partition(L, T: float) -> np.ndarray:
    """lse[b] = log(sum_v exp(L[b][v] / T)) in float64 (softmax normaliser at temperature T)."""
    L = np.ascontiguousarray(L, dtype=np.float64)
    if L.ndim == 1:
        L = L[None, :]
    if not T > 0:
        raise ValueError("temperature must be > 0")
    B, V = L.shape
    out = np.empty(B, np.float64)
    _load().orc_log_partition(_p(L), B, V, float(T), _p(out))
    return out


def probs_at(L, ids, T: float) -> np.ndarray:
    """prob[b][j] = exp(L[b][ids[b][j]] / T - lse[b]): softmax of L / T over the vocabulary."""
    L = np.ascontiguousarray(L, dtype=np.float64)
    if L.ndim == 1:
        L = L[None, :]
    B, V = L.shape
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(B, -1)
    k = ids.shape[1]
    lse = log_partition(L, T)
    out = np.empty((B, k), np.float64)
    _load().orc_probs_at(_p(L), _p(lse), B, V, float(T), _p(ids), int(k), _p(out))
    return out


def wire_row_bytes(wire: int, hidden: int) -> int:
    return int(_load().orc_wire_row_bytes(int(wire), int(hidden)))


def f32_to_f16_sat(x: float) -> int:
    return int(_load().orc_f32_to_f16_sat(float(np.float32(x))))


def wire_encode(x, wire: int) -> np.ndarray:
    """uint8 [n, wire_row_bytes] encoding of float32 rows x [n, hidden]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    n, hidden = x.shape
    out = np.empty((n, wire_row_bytes(wire, hidden)), np.uint8)
    _load().orc_wire_encode(_p(x), n, hidden, int(wire), _p(out))
    return out


def wire_decode(rows, hidden: int, wire: int) -> np.ndarray:
    """float32 [n, hidden] values of wire rows."""
    rb = wire_row_bytes(wire, hidden)
    raw = np.ascontiguousarray(rows, dtype=np.uint8).reshape(-1, rb)
    out = np.empty((raw.shape[0], hidden), np.float32)
    _load().orc_wire_decode(_p(raw), raw.shape[0], hidden, int(wire), _p(out))
    return out
