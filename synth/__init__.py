"""Seeded synthetic inputs for Skip Softmax attention (shared by tests, bench and oracle).

The arrays come from ``synth.c`` (counter-based SplitMix64 + Box-Muller, so the
bytes do not depend on the thread count).  This package holds no attention
arithmetic: it only draws Q/K/V and plants the structure (a sink tile, relevant
tiles, a low-rank shared factor) that makes some key tiles skippable.

bf16 tensors are returned as ``numpy.uint16`` bit patterns; fp32 copies hold the
same values before bf16 rounding.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile synth.c into libsynth.so (in-tree)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH + ".tmp", "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.synth_u64.restype = ctypes.c_uint64
    lib.synth_u64.argtypes = [ctypes.c_uint64] * 3
    lib.synth_uniform.restype = ctypes.c_double
    lib.synth_uniform.argtypes = [ctypes.c_uint64] * 3
    lib.synth_normal.restype = ctypes.c_double
    lib.synth_normal.argtypes = [ctypes.c_uint64] * 3
    lib.synth_f32_to_bf16.restype = ctypes.c_uint16
    lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.synth_gen_a.restype = ctypes.c_int
    lib.synth_gen_b.restype = ctypes.c_int
    lib.synth_num_pages.restype = ctypes.c_int64
    lib.synth_num_pages.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    lib.synth_kv_lens.restype = None
    lib.synth_kv_lens.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    _lib = lib
    return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class _GenAParams(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("B", ctypes.c_int32), ("S", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("shared_scale", ctypes.c_double), ("ar_window", ctypes.c_double),
                ("mu", ctypes.c_double), ("tile_k", ctypes.c_int32), ("sink_tiles", ctypes.c_int32),
                ("sink_amp", ctypes.c_double), ("rel_amp", ctypes.c_double), ("rel_frac", ctypes.c_double),
                ("rel_count", ctypes.c_int32)]


class _GenBParams(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("sink_tiles", ctypes.c_int32), ("sink_amp", ctypes.c_double), ("rel_amp", ctypes.c_double),
                ("rel_frac", ctypes.c_double)]


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


@dataclass(frozen=True)
class PrefillWorkload:
    """GEN-A prefill workload: Q [B,S,Hq,d], K/V [B,S,Hkv,d]."""
    name: str
    seed: int
    B: int
    S: int
    Hq: int
    Hkv: int
    d: int
    causal: bool = True
    tile_q: int = 128
    tile_k: int = 64
    rank: int = 16
    shared_scale: float = 1.5
    ar_window: float = 512.0
    mu: float = -1.0          # < 0: sqrt(d/G)
    sink_tiles: int = 1
    sink_amp: float = 4.0
    rel_amp: float = 2.5
    rel_frac: float = 0.10
    rel_count: int = 0
    taus: tuple = (-math.log(1000.0),)


@dataclass(frozen=True)
class DecodeWorkload:
    """GEN-B decode workload: q [B,Hq,d]; KV cache contiguous [B,Hkv,Smax,d] or paged [pages,Hkv,64,d]."""
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    kv_len: int = 0           # fixed length (kv_len_lo/hi ignored when > 0)
    kv_len_lo: int = 0
    kv_len_hi: int = 0
    paged: bool = False
    tile_k: int = 64
    num_splits: int = 16
    sink_tiles: int = 1
    sink_amp: float = 4.0
    rel_amp: float = 2.5
    rel_frac: float = 0.10
    taus: tuple = (-math.log(1000.0),)


# Workloads with Llama-3.3-70B attention shapes (64 query heads, 8 KV heads, head_dim 128).
# tiny_prefill: rank-0 GEN-A, two planted tiles per head group (+12 logits), no sink.
TINY_PREFILL = PrefillWorkload("tiny_prefill_s512", seed=1001, B=1, S=512, Hq=4, Hkv=1, d=64,
                               tile_q=64, tile_k=64, rank=0, sink_amp=0.0, rel_amp=3.0,
                               rel_frac=0.0, rel_count=2,
                               taus=(-math.log(1000.0), float("-inf")))
DECODE_32K = DecodeWorkload("decode_b8_kv32k", seed=1002, B=8, Hq=64, Hkv=8, d=128, kv_len=32768,
                            paged=False, num_splits=16)
PREFILL_16K = PrefillWorkload("prefill_s16k", seed=1003, B=1, S=16384, Hq=64, Hkv=8, d=128,
                              taus=(float("-inf"), -math.log(100.0), -math.log(1000.0)))
# rel_frac calibrated with the oracle's mask on sampled units for >= 50% skipped tiles at
# tau = -ln 1000 (oracle/calibrate.py writes tests/golden/calibration.json).
PREFILL_128K = PrefillWorkload("prefill_s128k", seed=1004, B=1, S=131072, Hq=64, Hkv=8, d=128,
                               rel_frac=0.4906, taus=(-math.log(1000.0),))
# taus calibrated with the oracle for about 0/30/50/70% skipped tiles with 16 split-local scans
# (same calibration file); taus[2] is the ~50% operating point.
DECODE_128K = DecodeWorkload("decode_b32_kv128k_paged", seed=1005, B=32, Hq=64, Hkv=8, d=128,
                             kv_len_lo=65536, kv_len_hi=131072, paged=True, num_splits=16,
                             taus=(float("-inf"), -7.518, -6.523, -5.267))

WORKLOADS = {w.name: w for w in (TINY_PREFILL, DECODE_32K, PREFILL_16K, PREFILL_128K, DECODE_128K)}


def gen_prefill(w: PrefillWorkload, *, bf16=True, fp32=False, threads=None) -> dict:
    """Draw one GEN-A prefill input set.  Returns dict with q/k/v (uint16 bf16 bits) and/or
    q32/k32/v32 (float32), plus ``relevant`` [B*Hkv, ceil(S/tile_k)] (uint8)."""
    lib = _load()
    p = _GenAParams(w.seed, w.B, w.S, w.Hq, w.Hkv, w.d, w.rank, w.shared_scale, w.ar_window, w.mu,
                    w.tile_k, w.sink_tiles, w.sink_amp, w.rel_amp, w.rel_frac, w.rel_count)
    out = {}
    qs, ks = (w.B, w.S, w.Hq, w.d), (w.B, w.S, w.Hkv, w.d)
    if bf16:
        out["q"], out["k"], out["v"] = (np.empty(s, np.uint16) for s in (qs, ks, ks))
    if fp32:
        out["q32"], out["k32"], out["v32"] = (np.empty(s, np.float32) for s in (qs, ks, ks))
    rel = np.zeros((w.B * w.Hkv, -(-w.S // w.tile_k)), np.uint8)
    rc = lib.synth_gen_a(ctypes.byref(p), _ptr(out.get("q")), _ptr(out.get("k")), _ptr(out.get("v")),
                         _ptr(out.get("q32")), _ptr(out.get("k32")), _ptr(out.get("v32")), _ptr(rel),
                         ctypes.c_int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"synth_gen_a failed with code {rc}")
    out["relevant"] = rel
    return out


# 256 sequences with as many cached keys in all as DECODE_128K (kv_len ~ U[8192, 16384]): a large batch through
# one decode call (timing of the dispatch order's cost; not an oracle-calibrated operating point).
DECODE_B256 = DecodeWorkload("decode_b256_kv16k_paged", seed=1006, B=256, Hq=64, Hkv=8, d=128,
                             kv_len_lo=8192, kv_len_hi=16384, paged=True, num_splits=16,
                             taus=(-math.log(1000.0),))


def kv_lens_for(w: DecodeWorkload) -> np.ndarray:
    lens = np.empty(w.B, np.int32)
    if w.kv_len > 0:
        lens[:] = w.kv_len
    else:
        _load().synth_kv_lens(ctypes.c_uint64(w.seed), w.B, w.kv_len_lo, w.kv_len_hi, _ptr(lens))
    return lens


def gen_decode(w: DecodeWorkload, *, kv_lens=None, contiguous=None, paged=None, fp32=False,
               smax=None, threads=None) -> dict:
    """Draw one GEN-B decode input set.

    Returns q (uint16 bf16) [B,Hq,d]; kv_lens int32 [B]; when ``contiguous``: k_cache/v_cache
    [B,Hkv,smax,d]; when ``paged``: k_pool/v_pool [pages,Hkv,tile_k,d] and page_table
    [B,max_pages]; with ``fp32`` also q32 and (contiguous) k32/v32."""
    lib = _load()
    lens = kv_lens_for(w) if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
    if contiguous is None:
        contiguous = not w.paged
    if paged is None:
        paged = w.paged
    T = w.tile_k
    maxlen = int(lens.max()) if len(lens) else 0
    if smax is None:
        smax = max(T, -(-maxlen // T) * T)
    out = {"kv_lens": lens, "q": np.empty((w.B, w.Hq, w.d), np.uint16)}
    if fp32:
        out["q32"] = np.empty((w.B, w.Hq, w.d), np.float32)
    if contiguous:
        out["k_cache"] = np.empty((w.B, w.Hkv, smax, w.d), np.uint16)
        out["v_cache"] = np.empty((w.B, w.Hkv, smax, w.d), np.uint16)
        if fp32:
            out["k32"] = np.empty((w.B, w.Hkv, smax, w.d), np.float32)
            out["v32"] = np.empty((w.B, w.Hkv, smax, w.d), np.float32)
    max_pages = max(1, -(-maxlen // T))
    if paged:
        npages = int(lib.synth_num_pages(w.B, _ptr(lens), T))
        out["k_pool"] = np.empty((max(npages, 1), w.Hkv, T, w.d), np.uint16)
        out["v_pool"] = np.empty((max(npages, 1), w.Hkv, T, w.d), np.uint16)
        if npages == 0:
            out["k_pool"][:] = 0
            out["v_pool"][:] = 0
        out["page_table"] = np.empty((w.B, max_pages), np.int32)
    rel = np.zeros((w.B * w.Hkv, max_pages), np.uint8)
    p = _GenBParams(w.seed, w.B, w.Hq, w.Hkv, w.d, T, w.sink_tiles, w.sink_amp, w.rel_amp, w.rel_frac)
    rc = lib.synth_gen_b(ctypes.byref(p), _ptr(lens), _ptr(out["q"]), _ptr(out.get("q32")),
                         _ptr(out.get("k_cache")), _ptr(out.get("v_cache")), _ptr(out.get("k32")),
                         _ptr(out.get("v32")), ctypes.c_int64(smax),
                         _ptr(out.get("k_pool")), _ptr(out.get("v_pool")), _ptr(out.get("page_table")),
                         ctypes.c_int32(max_pages), _ptr(rel), ctypes.c_int(threads or default_threads()))
    if rc != 0:
        raise ValueError(f"synth_gen_b failed with code {rc}")
    out["relevant"] = rel
    return out


FP8_E4M3_MAX = 448.0  # largest finite OCP e4m3 value


def _amax_bf16(bits: np.ndarray, chunk: int = 1 << 26) -> float:
    flat = bits.reshape(-1)
    m = 0.0
    for i in range(0, flat.size, chunk):
        m = max(m, float(np.abs(bf16_bits_to_f32(flat[i:i + chunk])).max(initial=0.0)))
    return m


def quantize_fp8_e4m3(bits: np.ndarray, scale: float, chunk: int = 1 << 26) -> np.ndarray:
    """OCP fp8 e4m3 storage codes (uint8) of a bf16 tensor with one per-tensor scale: code = the e4m3 value
    nearest to x / scale (ties to even, torch's float8_e4m3fn conversion), |x / scale| clamped to 448.
    Storage preparation of an input (like the bf16 rounding above); no attention arithmetic."""
    import torch
    flat = bits.reshape(-1)
    out = np.empty(flat.size, np.uint8)
    for i in range(0, flat.size, chunk):
        x = torch.from_numpy(bf16_bits_to_f32(flat[i:i + chunk]) / np.float32(scale))
        out[i:i + chunk] = x.clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return out.reshape(bits.shape)


def fp8_kv(data: dict) -> dict:
    """fp8 e4m3 copies of the K/V of a gen_decode() result with one scale per tensor (amax / 448, as float32):
    k_scale / v_scale, and the codes of whichever of k_pool/v_pool and k_cache/v_cache exist (a pool and a
    contiguous cache hold the same keys and share the scale)."""
    out = {}
    for name in ("k", "v"):
        src = data.get(f"{name}_pool", data.get(f"{name}_cache"))
        amax = _amax_bf16(src)
        scale = float(np.float32(amax / FP8_E4M3_MAX)) if amax > 0 else 1.0
        out[f"{name}_scale"] = scale
        for kind in ("pool", "cache"):
            if f"{name}_{kind}" in data:
                out[f"{name}_{kind}"] = quantize_fp8_e4m3(data[f"{name}_{kind}"], scale)
    return out


def fp8_qk(data: dict) -> dict:
    """fp8 e4m3 copies of the Q and K of a gen_prefill() result with one scale per tensor (amax / 448, as
    float32): q, k (uint8 codes) and q_scale, k_scale."""
    out = {}
    for name in ("q", "k"):
        amax = _amax_bf16(data[name])
        scale = float(np.float32(amax / FP8_E4M3_MAX)) if amax > 0 else 1.0
        out[f"{name}_scale"] = scale
        out[name] = quantize_fp8_e4m3(data[name], scale)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bits (nearest even), matching synth_f32_to_bf16 for finite values."""
    x = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    x = x + 0x7FFF + ((x >> 16) & 1)
    return (x >> 16).astype(np.uint16)


def gen_integer_qk(seed: int, B: int, S: int, Hq: int, Hkv: int, d: int, *, lo: int = -2, hi: int = 2,
                   offset: float = 0.0) -> dict:
    """Queries and keys with integer entries in [lo, hi] (exact in bf16, so every dot product is an exact small
    integer), values standard normal, all as bf16 bits.  offset > 0: the last channel of every query is 1 and
    that of every key uniform in (-offset, offset) (rounded to bf16), so each dot product lies within offset
    (plus bf16 rounding) of an integer."""
    r = np.random.default_rng(seed)
    q = r.integers(lo, hi + 1, (B, S, Hq, d)).astype(np.float32)
    k = r.integers(lo, hi + 1, (B, S, Hkv, d)).astype(np.float32)
    if offset:
        q[..., -1] = 1.0
        k[..., -1] = r.uniform(-offset, offset, (B, S, Hkv)).astype(np.float32)
    v = r.standard_normal((B, S, Hkv, d)).astype(np.float32)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}


__all__ = ["gen_integer_qk", "DECODE_B256", "quantize_fp8_e4m3", "fp8_kv", "fp8_qk", "FP8_E4M3_MAX", "PrefillWorkload", "DecodeWorkload", "WORKLOADS", "TINY_PREFILL", "DECODE_32K", "PREFILL_16K",
           "PREFILL_128K", "DECODE_128K", "gen_prefill", "gen_decode", "kv_lens_for", "bf16_bits_to_f32",
           "f32_to_bf16_bits", "build", "default_threads", "replace"]
