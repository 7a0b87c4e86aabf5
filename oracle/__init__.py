"""fp64 CPU oracle for Skip Softmax attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may
import this package.  The product (``long_context_flash_amd``) never does.  The
arithmetic lives in ``oracle.c`` (plain C, fp64); this module only marshals numpy
arrays through ctypes.

Inputs: numpy arrays of dtype uint16 (bf16 bit patterns), float32 or float64.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

UNVISITED, EXECUTED, SKIPPED = 0, 1, 2


def build(extra_flags=(), out_path=None) -> str:
    """Compile oracle.c into a shared library (in-tree by default)."""
    out_path = out_path or _LIB_PATH
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", *extra_flags,
           os.path.join(_HERE, "oracle.c"), "-o", out_path + ".tmp", "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


class _PrefillShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("S", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_double), ("tau", ctypes.c_double),
                ("S_k", ctypes.c_int32), ("weights", ctypes.c_int32)]


class _DecodeShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("smax", ctypes.c_int32), ("tile_k", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("scale", ctypes.c_double), ("tau", ctypes.c_double), ("sink_seed", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_double), ("v_scale", ctypes.c_double)]


def load(path=None):
    """Load the oracle library (``path`` lets tests load a separately built copy)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if path is None and not os.path.exists(p):
        build()
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [ctypes.POINTER(_PrefillShape), vp, vp, vp, ctypes.c_int, vp, ctypes.c_int64,
                                   vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [ctypes.POINTER(_DecodeShape), vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int64,
                                  vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def _dtype_code(*arrays):
    dt = arrays[0].dtype
    for a in arrays:
        if a.dtype != dt:
            raise TypeError("q, k and v must share one dtype")
    if dt == np.uint16:
        return 1
    if dt == np.float32:
        return 0
    if dt == np.float64:
        return 2
    raise TypeError(f"unsupported oracle input dtype {dt}")


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def prefill(q, k, v, *, causal=True, tau=-math.log(1000.0), tile_q=128, tile_k=64, scale=0.0,
            units=None, override=None, form="closed", weights="exp", threads=None, lib=None) -> dict:
    """Skip Softmax prefill on q [B,S,Hq,d], k/v [B,S_k,Hkv,d] with S_k >= S (S_k > S: chunked prefill, the
    queries being the last S of the S_k positions; causal masking is then bottom-right aligned).
    weights: "exp" (softmax) or "rowmax_pot" (a kept key's weight is 2^(rint(log2(e) l) - rint(log2(e) mu)),
    mu the row maximum over the kept keys).

    Returns dict: out [n,tile_q,d], lse [n,tile_q], state/gamma [n,ceil(S_k/tile_k)], dropped [n,tile_q],
    for the listed units (unit = (b*Hq + h)*ceil(S/tile_q) + qt) or all units in that order."""
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    B, S, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Sk, Hkv, d) or v.shape != k.shape or Sk < S:
        raise ValueError("k/v must be [B,S_k,Hkv,d] with S_k >= S")
    nqt, nkt = -(-S // tile_q), -(-Sk // tile_k)
    units_arr = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    n = B * Hq * nqt if units_arr is None else len(units_arr)
    ov = None
    if override is not None:
        ov = np.ascontiguousarray(override, dtype=np.int8).reshape(n, nkt)
    res = {"out": np.empty((n, tile_q, d)), "lse": np.empty((n, tile_q)), "state": np.empty((n, nkt), np.uint8),
           "gamma": np.empty((n, nkt)), "dropped": np.empty((n, tile_q))}
    if weights not in ("exp", "rowmax_pot"):
        raise ValueError("weights must be 'exp' or 'rowmax_pot'")
    shape = _PrefillShape(B, S, Hq, Hkv, d, tile_q, tile_k, int(bool(causal)), float(scale), float(tau), Sk,
                          1 if weights == "rowmax_pot" else 0)
    rc = (lib or load()).oracle_prefill(ctypes.byref(shape), _p(q), _p(k), _p(v), _dtype_code(q, k, v),
                                        _p(units_arr), n, _p(ov), 1 if form == "scan" else 0,
                                        _p(res["out"]), _p(res["lse"]), _p(res["state"]), _p(res["gamma"]),
                                        _p(res["dropped"]), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_prefill failed with code {rc}")
    return res


def decode(q, k, v, kv_lens, *, tau=-math.log(1000.0), tile_k=64, num_splits=16, scale=0.0, units=None,
           override=None, form="closed", sink_seed=False, k_scale=1.0, v_scale=1.0, threads=None,
           lib=None) -> dict:
    """Skip Softmax split-K decode on q [B,Hq,d], contiguous caches k/v [B,Hkv,smax,d], kv_lens [B].
    sink_seed: splits after the first start their running maximum at the first tile's row maxima.
    k and v may be uint8 arrays of OCP fp8 e4m3 codes; keys and values are then k_scale * code and
    v_scale * code (the scales also apply to other k/v dtypes).

    Returns dict: out [n,G,d], lse [n,G], state/gamma [n,ceil(smax/tile_k)], dropped [n,G]
    for the listed units (unit = b*Hkv + g) or all units in that order."""
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    kv_lens = np.ascontiguousarray(kv_lens, dtype=np.int32)
    B, Hq, d = q.shape
    _, Hkv, smax, _ = k.shape
    if k.dtype == np.uint8 or v.dtype == np.uint8:
        if k.dtype != v.dtype:
            raise TypeError("k and v must share one dtype")
        kv_dtype = 3
    else:
        kv_dtype = _dtype_code(k, v)
    q_dtype = _dtype_code(q)
    if k.shape != (B, Hkv, smax, d) or v.shape != k.shape or kv_lens.shape != (B,):
        raise ValueError("k/v must be [B,Hkv,smax,d], kv_lens [B]")
    G = Hq // Hkv
    maxt = -(-smax // tile_k)
    units_arr = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    n = B * Hkv if units_arr is None else len(units_arr)
    ov = None
    if override is not None:
        ov = np.ascontiguousarray(override, dtype=np.int8).reshape(n, maxt)
    res = {"out": np.empty((n, G, d)), "lse": np.empty((n, G)), "state": np.empty((n, maxt), np.uint8),
           "gamma": np.empty((n, maxt)), "dropped": np.empty((n, G))}
    shape = _DecodeShape(B, Hq, Hkv, d, smax, tile_k, num_splits, float(scale), float(tau), 1 if sink_seed else 0,
                         kv_dtype, float(k_scale), float(v_scale))
    rc = (lib or load()).oracle_decode(ctypes.byref(shape), _p(q), _p(k), _p(v), q_dtype,
                                       _p(kv_lens), _p(units_arr), n, _p(ov), 1 if form == "scan" else 0,
                                       _p(res["out"]), _p(res["lse"]), _p(res["state"]), _p(res["gamma"]),
                                       _p(res["dropped"]), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return res
