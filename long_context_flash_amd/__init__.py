"""Skip Softmax attention on AMD MI355X: thin Python binding of libssm.so.

Every computation runs in the HIP kernels of ``libssm.so``; this module only turns
torch tensors into the C descriptors of ``include/ssm.h`` (pointers, shapes, strides),
allocates outputs/workspace with torch, and raises on error codes.  There is no
fallback path: if the library is missing or a call fails, an exception is raised.

Entry points (same names as the C ABI):
    ssm_prefill(q, k, v, causal=True, tau=-ln(1000), ...)       -> out [B,S,Hq,d] bf16
    ssm_prefill_fp8qk(q8, q_scale, k8, k_scale, v, ...)         -> out (fp8 e4m3 queries and keys)
    ssm_prefill_paged(q, k_cache, v_cache, page_table, ...)     -> out [total_q,Hq,d] bf16
    ssm_prefill_paged_fp8qk(q8, q_scale, k_cache8, v_cache8, ...) -> out (fp8 e4m3 queries over fp8 pages)
    ssm_decode(q, k_cache, v_cache, kv_lens, tau=..., ...)      -> out [B,Hq,d] bf16
    ssm_decode_noalloc(q, k_cache, v_cache, kv_lens, out=..., ...) -> out (workspace: the library's static scratch)
    ssm_decode_workspace_bytes(B, Hq, d, num_splits)
    ssm_strerror(code), ssm_last_error(), ssm_abi_version()
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm.so")

SSM_OK, SSM_EINVAL, SSM_EUNSUPPORTED, SSM_EWORKSPACE, SSM_EHIP = range(5)
SSM_BF16, SSM_FP32, SSM_FP8_E4M3 = 0, 1, 2
EXPORTED_SYMBOLS = ("ssm_prefill", "ssm_prefill_fp8qk", "ssm_decode", "ssm_decode_noalloc", "ssm_prefill_paged", "ssm_prefill_paged_fp8qk",
                    "ssm_decode_workspace_bytes", "ssm_strerror", "ssm_last_error", "ssm_abi_version")


class SsmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class KvCache(ctypes.Structure):
    _fields_ = [("pool", Tensor), ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("scale", ctypes.c_float)]


class SkipStatsC(ctypes.Structure):
    _fields_ = [("tile_state", ctypes.c_void_p), ("tile_state_len", ctypes.c_int64), ("unit_gap", ctypes.c_void_p),
                ("unit_gap_len", ctypes.c_int64), ("counters", ctypes.c_void_p)]


class Opts(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("tile_q", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("num_splits", ctypes.c_int32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("decode_flags", ctypes.c_int32), ("weights", ctypes.c_int32)]


ABI_VERSION = 10              # the layout above and the entry points match SSM_ABI_VERSION of include/ssm.h
DECODE_SINK_SEED = 1          # SSM_DECODE_SINK_SEED
WEIGHTS = {"exp": 0, "rowmax_pot": 1}  # SSM_WEIGHTS_EXP, SSM_WEIGHTS_ROWMAX_POT


_lib = None


def lib():
    """Load libssm.so (built by ``python -m long_context_flash_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_flash_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    L.ssm_prefill.restype = ctypes.c_int
    L.ssm_prefill.argtypes = [P(Tensor), P(Tensor), P(Tensor), ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                              P(Tensor), P(SkipStatsC), ctypes.c_void_p, P(Opts)]
    L.ssm_prefill_fp8qk.restype = ctypes.c_int
    L.ssm_prefill_fp8qk.argtypes = [P(Tensor), ctypes.c_float, P(Tensor), ctypes.c_float, P(Tensor), ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_float, P(Tensor), P(SkipStatsC), ctypes.c_void_p, P(Opts)]
    L.ssm_decode.restype = ctypes.c_int
    L.ssm_decode.argtypes = [P(Tensor), P(KvCache), P(KvCache), ctypes.c_void_p, ctypes.c_float, P(Tensor),
                             P(SkipStatsC), ctypes.c_void_p, P(Opts)]
    L.ssm_decode_noalloc.restype = ctypes.c_int
    L.ssm_decode_noalloc.argtypes = [P(Tensor), P(KvCache), P(KvCache), ctypes.c_void_p, ctypes.c_float, P(Tensor),
                                     P(SkipStatsC), ctypes.c_void_p, P(Opts)]
    L.ssm_prefill_paged.restype = ctypes.c_int
    L.ssm_prefill_paged.argtypes = [P(Tensor), P(KvCache), P(KvCache), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P(Tensor), P(SkipStatsC),
                                    ctypes.c_void_p, P(Opts)]
    L.ssm_prefill_paged_fp8qk.restype = ctypes.c_int
    L.ssm_prefill_paged_fp8qk.argtypes = [P(Tensor), ctypes.c_float, P(KvCache), P(KvCache), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_float, P(Tensor), P(SkipStatsC), ctypes.c_void_p, P(Opts)]
    L.ssm_decode_workspace_bytes.restype = ctypes.c_size_t
    L.ssm_decode_workspace_bytes.argtypes = [ctypes.c_int32] * 4
    L.ssm_strerror.restype = ctypes.c_char_p
    L.ssm_strerror.argtypes = [ctypes.c_int]
    L.ssm_last_error.restype = ctypes.c_char_p
    L.ssm_last_error.argtypes = []
    L.ssm_abi_version.restype = ctypes.c_int
    L.ssm_abi_version.argtypes = []
    if L.ssm_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.ssm_abi_version()}, this binding expects {ABI_VERSION}: "
                           "rebuild it with `python -m long_context_flash_amd.build`")
    _lib = L
    return L


def describe(t: Optional[torch.Tensor]) -> Tensor:
    """ssm_tensor descriptor of a torch tensor (no copy)."""
    d = Tensor()
    if t is None:
        return d
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d.data = t.data_ptr()
    d.dtype = {torch.bfloat16: SSM_BF16, torch.float32: SSM_FP32, torch.float8_e4m3fn: SSM_FP8_E4M3}.get(t.dtype, -1)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _on_device(device: torch.device, **tensors):
    """Every tensor handed to the library must live on the GPU of the call (the kernels dereference the
    pointers on that device); raise before any library call otherwise."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} is on {t.device}; the call runs on {device} and needs every tensor there")


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int):
    if rc != SSM_OK:
        raise SsmError(rc, f"{ssm_strerror(rc)}: {ssm_last_error()}")


@dataclass
class SkipStats:
    """Device buffers for the optional skip statistics (see ssm_skip_stats in include/ssm.h)."""
    tile_state: Optional[torch.Tensor] = None   # uint8
    unit_gap: Optional[torch.Tensor] = None     # float32
    counters: Optional[torch.Tensor] = None     # int64 [4]: visited, skipped, qk tiles, pv tiles

    def tensors(self) -> dict:
        return {"skip_stats.tile_state": self.tile_state, "skip_stats.unit_gap": self.unit_gap,
                "skip_stats.counters": self.counters}

    def c(self) -> SkipStatsC:
        for t, dt, name in ((self.tile_state, torch.uint8, "tile_state"), (self.unit_gap, torch.float32, "unit_gap"),
                            (self.counters, torch.int64, "counters")):
            if t is not None and (t.dtype != dt or not t.is_contiguous()):
                raise ValueError(f"skip_stats.{name} must be a contiguous {dt} tensor")
        if self.counters is not None and self.counters.numel() < 4:
            raise ValueError("skip_stats.counters needs 4 elements")
        s = SkipStatsC()
        if self.tile_state is not None:
            s.tile_state = self.tile_state.data_ptr()
            s.tile_state_len = self.tile_state.numel()
        if self.unit_gap is not None:
            s.unit_gap = self.unit_gap.data_ptr()
            s.unit_gap_len = self.unit_gap.numel()
        if self.counters is not None:
            s.counters = self.counters.data_ptr()
        return s

    @staticmethod
    def alloc(units: int, tiles: int, device, gaps: bool = False) -> "SkipStats":
        return SkipStats(tile_state=torch.zeros(units, tiles, dtype=torch.uint8, device=device),
                         unit_gap=torch.empty(units, tiles, dtype=torch.float32, device=device) if gaps else None,
                         counters=torch.zeros(4, dtype=torch.int64, device=device))


def _weights_code(weights: str) -> int:
    if weights not in WEIGHTS:
        raise ValueError(f"weights must be one of {sorted(WEIGHTS)}")
    return WEIGHTS[weights]


def prefill_stats_shape(B, S, Hq, tile_q=128, tile_k=64):
    """(units, tiles) of the prefill statistics: unit = (b*Hq + h)*ceil(S/tile_q) + q_tile."""
    return B * Hq * (-(-S // tile_q)), -(-S // tile_k)


def ssm_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                tau: float = -math.log(1000.0), out: Optional[torch.Tensor] = None,
                skip_stats: Optional[SkipStats] = None, stream=None, tile_q: int = 128, tile_k: int = 64,
                scale: float = 0.0, weights: str = "exp") -> torch.Tensor:
    """Skip Softmax prefill: q [B,S,Hq,d], k/v [B,S,Hkv,d] bf16 on the GPU -> out [B,S,Hq,d] bf16.
    weights: "exp" (softmax) or "rowmax_pot" (power-of-two weights anchored at the row maximum)."""
    _on_device(q.device, q=q, k=k, v=v, out=out, **(skip_stats.tensors() if skip_stats else {}))
    if out is None:
        out = torch.empty_like(q)
    qd, kd, vd, od = describe(q), describe(k), describe(v), describe(out)
    opts = Opts(float(scale), int(tile_q), int(tile_k), 0, None, 0, 0, _weights_code(weights))
    st = skip_stats.c() if skip_stats is not None else None
    rc = lib().ssm_prefill(ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd), int(q.shape[1]) if q.dim() == 4 else 0,
                           int(bool(causal)), float(tau), ctypes.byref(od), ctypes.byref(st) if st else None,
                           _stream_handle(stream), ctypes.byref(opts))
    _check(rc)
    return out


def ssm_prefill_fp8qk(q: torch.Tensor, q_scale: float, k: torch.Tensor, k_scale: float, v: torch.Tensor,
                      causal: bool = True, tau: float = -math.log(1000.0), out: Optional[torch.Tensor] = None,
                      skip_stats: Optional[SkipStats] = None, stream=None, tile_q: int = 128, tile_k: int = 64,
                      scale: float = 0.0, weights: str = "exp") -> torch.Tensor:
    """Skip Softmax prefill with 8-bit scores: q [B,S,Hq,d] and k [B,S,Hkv,d] torch.float8_e4m3fn codes (query =
    q_scale * code, key = k_scale * code), v [B,S,Hkv,d] bf16 on the GPU -> out [B,S,Hq,d] bf16."""
    _on_device(q.device, q=q, k=k, v=v, out=out, **(skip_stats.tensors() if skip_stats else {}))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    qd, kd, vd, od = describe(q), describe(k), describe(v), describe(out)
    opts = Opts(float(scale), int(tile_q), int(tile_k), 0, None, 0, 0, _weights_code(weights))
    st = skip_stats.c() if skip_stats is not None else None
    rc = lib().ssm_prefill_fp8qk(ctypes.byref(qd), float(q_scale), ctypes.byref(kd), float(k_scale), ctypes.byref(vd),
                                 int(q.shape[1]) if q.dim() == 4 else 0, int(bool(causal)), float(tau),
                                 ctypes.byref(od), ctypes.byref(st) if st else None, _stream_handle(stream),
                                 ctypes.byref(opts))
    _check(rc)
    return out


def _paged_cache(t: torch.Tensor, pt: torch.Tensor, scale: float = 1.0) -> KvCache:
    c = KvCache()
    c.pool = describe(t)
    c.scale = float(scale)
    if pt.dtype != torch.int32 or pt.dim() != 2 or not pt.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [B, max_pages] tensor")
    c.page_table = pt.data_ptr()
    c.page_size = t.shape[2]
    c.max_pages = pt.shape[1]
    return c


def ssm_prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, page_table: torch.Tensor,
                      q_start: torch.Tensor, kv_lens: torch.Tensor, max_q_len: int, causal: bool = True,
                      tau: float = -math.log(1000.0), out: Optional[torch.Tensor] = None,
                      skip_stats: Optional[SkipStats] = None, stream=None, tile_q: int = 128, scale: float = 0.0,
                      v_page_table: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> torch.Tensor:
    """Chunked prefill against a paged cache: q/out [total_q,Hq,d] bf16 (sequence b's rows q_start[b] ..
    q_start[b+1]-1, the last of its kv_lens[b] cached keys); k_cache/v_cache [pages,Hkv,64,d] bf16, or
    torch.float8_e4m3fn codes (key = k_scale * code, value = v_scale * code), with page_table int32
    [B,max_pages]; q_start int32 [B+1] and kv_lens int32 [B] on the GPU."""
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, v_page_table=v_page_table,
               q_start=q_start, kv_lens=kv_lens, out=out, **(skip_stats.tensors() if skip_stats else {}))
    if out is None:
        out = torch.empty_like(q)
    for name, t in (("q_start", q_start), ("kv_lens", kv_lens)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    B = kv_lens.shape[0]
    if q_start.shape[0] != B + 1:
        raise ValueError("q_start must have batch + 1 entries")
    kc = _paged_cache(k_cache, page_table, k_scale)
    vc = _paged_cache(v_cache, page_table if v_page_table is None else v_page_table, v_scale)
    qd, od = describe(q), describe(out)
    opts = Opts(float(scale), int(tile_q), 64, 0, None, 0, 0)
    st = skip_stats.c() if skip_stats is not None else None
    rc = lib().ssm_prefill_paged(ctypes.byref(qd), ctypes.byref(kc), ctypes.byref(vc), q_start.data_ptr(),
                                 kv_lens.data_ptr(), int(B), int(max_q_len), int(bool(causal)), float(tau),
                                 ctypes.byref(od), ctypes.byref(st) if st else None, _stream_handle(stream),
                                 ctypes.byref(opts))
    _check(rc)
    return out


def ssm_prefill_paged_fp8qk(q: torch.Tensor, q_scale: float, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            page_table: torch.Tensor, q_start: torch.Tensor, kv_lens: torch.Tensor, max_q_len: int,
                            k_scale: float, v_scale: float, causal: bool = True, tau: float = -math.log(1000.0),
                            out: Optional[torch.Tensor] = None, skip_stats: Optional[SkipStats] = None, stream=None,
                            tile_q: int = 128, scale: float = 0.0,
                            v_page_table: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked prefill with 8-bit queries over e4m3 pages: q [total_q,Hq,d] torch.float8_e4m3fn codes (query =
    q_scale * code), k_cache/v_cache [pages,Hkv,64,d] torch.float8_e4m3fn codes with k_scale / v_scale; the rest
    as ssm_prefill_paged.  out [total_q,Hq,d] bf16."""
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table, v_page_table=v_page_table,
               q_start=q_start, kv_lens=kv_lens, out=out, **(skip_stats.tensors() if skip_stats else {}))
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    for name, t in (("q_start", q_start), ("kv_lens", kv_lens)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    B = kv_lens.shape[0]
    if q_start.shape[0] != B + 1:
        raise ValueError("q_start must have batch + 1 entries")
    kc = _paged_cache(k_cache, page_table, k_scale)
    vc = _paged_cache(v_cache, page_table if v_page_table is None else v_page_table, v_scale)
    qd, od = describe(q), describe(out)
    opts = Opts(float(scale), int(tile_q), 64, 0, None, 0, 0)
    st = skip_stats.c() if skip_stats is not None else None
    rc = lib().ssm_prefill_paged_fp8qk(ctypes.byref(qd), float(q_scale), ctypes.byref(kc), ctypes.byref(vc),
                                       q_start.data_ptr(), kv_lens.data_ptr(), int(B), int(max_q_len),
                                       int(bool(causal)), float(tau), ctypes.byref(od),
                                       ctypes.byref(st) if st else None, _stream_handle(stream), ctypes.byref(opts))
    _check(rc)
    return out


def ssm_decode_workspace_bytes(B: int, Hq: int, d: int, num_splits: int) -> int:
    return int(lib().ssm_decode_workspace_bytes(B, Hq, d, num_splits))


def decode_workspace(B, Hq, d, num_splits, device) -> torch.Tensor:
    n = ssm_decode_workspace_bytes(B, Hq, d, num_splits)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def ssm_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
               tau: float = -math.log(1000.0), out: Optional[torch.Tensor] = None,
               page_table: Optional[torch.Tensor] = None, v_page_table: Optional[torch.Tensor] = None,
               num_splits: int = 16, workspace: Optional[torch.Tensor] = None,
               skip_stats: Optional[SkipStats] = None, stream=None, scale: float = 0.0,
               sink_seed: bool = False, k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """Skip Softmax split-K decode.

    q [B,Hq,d] bf16; k_cache/v_cache contiguous [B,Hkv,Smax,d] (page_table None) or paged pools
    [pages,Hkv,64,d] with page_table int32 [B,max_pages]; kv_lens int32 [B] on the GPU.
    sink_seed: splits after the first start their running maximum at the first key tile's row maxima.
    k_cache/v_cache may be torch.float8_e4m3fn tensors of codes; keys and values are then k_scale * code and
    v_scale * code."""
    return _decode(q, k_cache, v_cache, kv_lens, tau, out, page_table, v_page_table, num_splits, workspace, skip_stats,
                   stream, scale, sink_seed, k_scale, v_scale, noalloc=False)


def ssm_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
                       tau: float = -math.log(1000.0), out: Optional[torch.Tensor] = None,
                       page_table: Optional[torch.Tensor] = None, v_page_table: Optional[torch.Tensor] = None,
                       num_splits: int = 16, skip_stats: Optional[SkipStats] = None, stream=None, scale: float = 0.0,
                       sink_seed: bool = False, k_scale: float = 1.0, v_scale: float = 1.0) -> torch.Tensor:
    """ssm_decode whose workspace is the library's static per-GPU scratch array (ssm_decode_noalloc): the C call
    allocates nothing.  Pass ``out`` to keep this wrapper from allocating it.  Calls that overlap on one GPU race
    on the shared scratch."""
    return _decode(q, k_cache, v_cache, kv_lens, tau, out, page_table, v_page_table, num_splits, None, skip_stats,
                   stream, scale, sink_seed, k_scale, v_scale, noalloc=True)


def _decode(q, k_cache, v_cache, kv_lens, tau, out, page_table, v_page_table, num_splits, workspace, skip_stats,
            stream, scale, sink_seed, k_scale, v_scale, noalloc):
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, kv_lens=kv_lens, out=out, page_table=page_table,
               v_page_table=v_page_table, workspace=workspace, **(skip_stats.tensors() if skip_stats else {}))
    if out is None:
        out = torch.empty_like(q)
    B, Hq, d = q.shape
    if workspace is None and not noalloc:
        workspace = decode_workspace(B, Hq, d, num_splits, q.device)
    vpt = page_table if v_page_table is None else v_page_table

    def cache(t, pt, sc):
        c = KvCache()
        c.pool = describe(t)
        c.scale = float(sc)
        if pt is not None:
            if pt.dtype != torch.int32 or pt.dim() != 2 or not pt.is_contiguous():
                raise ValueError("page_table must be a contiguous int32 [B, max_pages] tensor")
            c.page_table = pt.data_ptr()
            c.page_size = t.shape[2]
            c.max_pages = pt.shape[1]
        return c

    if kv_lens.dtype != torch.int32 or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be a contiguous int32 tensor")
    kc, vc = cache(k_cache, page_table, k_scale), cache(v_cache, vpt, v_scale)
    qd, od = describe(q), describe(out)
    ws_ptr, ws_bytes = (None, 0) if noalloc else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    opts = Opts(float(scale), 0, 64, int(num_splits), ws_ptr, ws_bytes, DECODE_SINK_SEED if sink_seed else 0)
    st = skip_stats.c() if skip_stats is not None else None
    fn = lib().ssm_decode_noalloc if noalloc else lib().ssm_decode
    rc = fn(ctypes.byref(qd), ctypes.byref(kc), ctypes.byref(vc), kv_lens.data_ptr(), float(tau), ctypes.byref(od),
            ctypes.byref(st) if st else None, _stream_handle(stream), ctypes.byref(opts))
    _check(rc)
    return out


def ssm_strerror(code: int) -> str:
    return lib().ssm_strerror(code).decode()


def ssm_last_error() -> str:
    return lib().ssm_last_error().decode()


def ssm_abi_version() -> int:
    return int(lib().ssm_abi_version())


def bf16_from_bits(a, device=None) -> torch.Tensor:
    """numpy uint16 bf16 bit patterns -> torch.bfloat16 tensor (optionally moved to ``device``)."""
    t = torch.from_numpy(a.view("int16")).view(torch.bfloat16)
    return t.to(device) if device is not None else t


__all__ = ["ssm_prefill", "ssm_prefill_fp8qk", "ssm_prefill_paged_fp8qk", "ssm_decode", "ssm_decode_noalloc", "ssm_prefill_paged", "ssm_decode_workspace_bytes", "ssm_strerror", "ssm_last_error",
           "ssm_abi_version", "SkipStats", "SsmError", "prefill_stats_shape", "decode_workspace", "bf16_from_bits",
           "lib", "describe", "LIB_PATH", "EXPORTED_SYMBOLS"]
