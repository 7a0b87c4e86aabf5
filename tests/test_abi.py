"""The C ABI library loads, exports every symbol include/ssm.h declares, and rejects invalid
arguments before touching the device (CPU only: no compute call is made)."""
import ctypes
import math
import os
import re
import subprocess

import pytest

import long_context_flash_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssm.LIB_PATH):
        pytest.fail("libssm.so is not built (run __graft_entry__.build())")
    return ssm.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(ssm.EXPORTED_SYMBOLS), names
    out = subprocess.run(["nm", "-D", "--defined-only", ssm.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (ssm_\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, f"{n} not exported"
        assert hasattr(lib, n)


def test_version_and_strings(lib):
    assert ssm.ssm_abi_version() == ssm.ABI_VERSION == 10
    for code in range(5):
        assert ssm.ssm_strerror(code)
    assert "unknown" in ssm.ssm_strerror(99)


def test_workspace_bytes(lib):
    n = ssm.ssm_decode_workspace_bytes(32, 64, 128, 16)
    o_bytes = 32 * 64 * 16 * 128 * 4
    assert n >= o_bytes + 32 * 64 * 16 * 4 + 32 * 4
    assert ssm.ssm_decode_workspace_bytes(1, 1, 128, 0) == 0
    # partial outputs, partial LSEs, (batches up to 8192) the dispatch order and two skip counts per (b, head,
    # split), each on a 256-byte boundary
    r256 = lambda x: (x + 255) // 256 * 256
    for B in (1, 7, 8192, 8193):
        rows = B * 8 * 4
        want = r256(r256(r256(rows * 64 * 4) + rows * 4) + (B * 4 if B <= 8192 else 0)) + rows * 8
        assert ssm.ssm_decode_workspace_bytes(B, 8, 64, 4) == want, B


FAKE = 0x10000  # never dereferenced: validation fails first


def desc(shape, dtype=ssm.SSM_BF16, data=FAKE, stride=None):
    d = ssm.Tensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, s in enumerate(shape):
        d.shape[i] = s
        d.stride[i] = stride[i]
    return d


def call_prefill(lib, q=None, k=None, v=None, o=None, seqlen=256, causal=1, tau=-6.9, opts=None):
    q = q or desc([1, 256, 8, 128])
    k = k or desc([1, 256, 2, 128])
    v = v or desc([1, 256, 2, 128])
    o = o or desc([1, 256, 8, 128])
    return lib.ssm_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), seqlen, causal, tau, ctypes.byref(o),
                           None, None, ctypes.byref(opts) if opts else None)


@pytest.mark.parametrize("case,code", [
    ("nan_tau", ssm.SSM_EINVAL), ("pos_tau", ssm.SSM_EINVAL), ("null_q", ssm.SSM_EINVAL),
    ("seqlen", ssm.SSM_EINVAL), ("gqa", ssm.SSM_EINVAL), ("head_dim", ssm.SSM_EUNSUPPORTED),
    ("dtype", ssm.SSM_EUNSUPPORTED), ("stride", ssm.SSM_EINVAL), ("align", ssm.SSM_EUNSUPPORTED),
    ("tile_q", ssm.SSM_EUNSUPPORTED), ("tile_k", ssm.SSM_EUNSUPPORTED), ("out_shape", ssm.SSM_EINVAL),
    ("slice_offsets", ssm.SSM_EUNSUPPORTED), ("too_many_tiles", ssm.SSM_EUNSUPPORTED),
    ("too_long", ssm.SSM_EUNSUPPORTED),
])
def test_prefill_rejects(lib, case, code):
    kw = {}
    if case in ("slice_offsets", "too_many_tiles", "too_long"):
        # sizes past the limits the kernels' 32-bit offsets and grid allow; nothing is dereferenced
        B, S = {"slice_offsets": (1, 262144), "too_many_tiles": (40000, 1 << 20), "too_long": (1, (1 << 30) + 64)}[case]
        kw["q"], kw["k"], kw["v"], kw["o"] = (desc([B, S, h, 128]) for h in (64, 8, 8, 64))
        kw["seqlen"] = S
    if case == "nan_tau":
        kw["tau"] = math.nan
    elif case == "pos_tau":
        kw["tau"] = 0.5
    elif case == "null_q":
        kw["q"] = desc([1, 256, 8, 128], data=0)
    elif case == "seqlen":
        kw["seqlen"] = 255
    elif case == "gqa":
        kw["k"] = desc([1, 256, 3, 128])
        kw["v"] = desc([1, 256, 3, 128])
    elif case == "head_dim":
        kw["q"], kw["k"], kw["v"], kw["o"] = (desc([1, 256, h, 96]) for h in (8, 2, 2, 8))
    elif case == "dtype":
        kw["q"] = desc([1, 256, 8, 128], dtype=ssm.SSM_FP32)
    elif case == "stride":
        kw["q"] = desc([1, 256, 8, 128], stride=[256 * 8 * 128, 8 * 128, 128, 2])
    elif case == "align":
        kw["q"] = desc([1, 256, 8, 128], data=FAKE + 2)
    elif case == "tile_q":
        kw["opts"] = ssm.Opts(0.0, 32, 0, 0, None, 0)
    elif case == "tile_k":
        kw["opts"] = ssm.Opts(0.0, 0, 128, 0, None, 0)
    elif case == "out_shape":
        kw["o"] = desc([1, 256, 4, 128])
    rc = call_prefill(lib, **kw)
    assert rc == code, (rc, ssm.ssm_last_error())
    assert ssm.ssm_last_error()


def call_prefill_fp8qk(lib, q=None, k=None, v=None, o=None, q_scale=0.05, k_scale=0.02, seqlen=256, tau=-6.9,
                      opts=None):
    q = q or desc([1, 256, 8, 128], dtype=ssm.SSM_FP8_E4M3)
    k = k or desc([1, 256, 2, 128], dtype=ssm.SSM_FP8_E4M3)
    v = v or desc([1, 256, 2, 128])
    o = o or desc([1, 256, 8, 128])
    return lib.ssm_prefill_fp8qk(ctypes.byref(q), q_scale, ctypes.byref(k), k_scale, ctypes.byref(v), seqlen, 1, tau,
                                 ctypes.byref(o), None, None, ctypes.byref(opts) if opts else None)


@pytest.mark.parametrize("case,code", [
    ("bf16_q", ssm.SSM_EUNSUPPORTED), ("bf16_k", ssm.SSM_EUNSUPPORTED), ("fp8_v", ssm.SSM_EUNSUPPORTED),
    ("zero_scale", ssm.SSM_EINVAL), ("nan_scale", ssm.SSM_EINVAL), ("inf_scale", ssm.SSM_EINVAL),
    ("neg_scale", ssm.SSM_EINVAL), ("fp8_stride", ssm.SSM_EUNSUPPORTED), ("head_dim", ssm.SSM_EUNSUPPORTED),
    ("pos_tau", ssm.SSM_EINVAL), ("gqa", ssm.SSM_EINVAL), ("tile_q", ssm.SSM_EUNSUPPORTED),
])
def test_prefill_fp8qk_rejects(lib, case, code):
    kw = {}
    f8 = ssm.SSM_FP8_E4M3
    if case == "bf16_q":
        kw["q"] = desc([1, 256, 8, 128])
    elif case == "bf16_k":
        kw["k"] = desc([1, 256, 2, 128])
    elif case == "fp8_v":
        kw["v"] = desc([1, 256, 2, 128], dtype=f8)
    elif case == "zero_scale":
        kw["q_scale"] = 0.0
    elif case == "nan_scale":
        kw["k_scale"] = math.nan
    elif case == "inf_scale":
        kw["q_scale"] = math.inf
    elif case == "neg_scale":
        kw["k_scale"] = -1.0
    elif case == "fp8_stride":  # 136 codes per row: not a multiple of 16 bytes
        kw["k"] = desc([1, 256, 2, 128], dtype=f8, stride=[256 * 2 * 136, 2 * 136, 136, 1])
    elif case == "head_dim":
        kw["q"], kw["k"] = desc([1, 256, 8, 96], dtype=f8), desc([1, 256, 2, 96], dtype=f8)
        kw["v"], kw["o"] = desc([1, 256, 2, 96]), desc([1, 256, 8, 96])
    elif case == "pos_tau":
        kw["tau"] = 0.1
    elif case == "gqa":
        kw["k"] = desc([1, 256, 3, 128], dtype=f8)
        kw["v"] = desc([1, 256, 3, 128])
    elif case == "tile_q":
        kw["opts"] = ssm.Opts(0.0, 32, 0, 0, None, 0)
    rc = call_prefill_fp8qk(lib, **kw)
    assert rc == code, (rc, ssm.ssm_last_error())
    assert ssm.ssm_last_error()


def _weights_opts(w):
    o = ssm.Opts(0.0, 0, 0, 0, None, 0, 0)
    o.weights = w
    return o


def test_weights_option_is_validated(lib):
    """ssm_opts.weights: unknown values are SSM_EINVAL for both prefills; Rowmax-PoT weights are SSM_EUNSUPPORTED for
    the decode and the chunked prefills (no device call: these run without a GPU)."""
    assert ssm.WEIGHTS == {"exp": ssm_h_define("SSM_WEIGHTS_EXP"), "rowmax_pot": ssm_h_define("SSM_WEIGHTS_ROWMAX_POT")}
    for w in (2, -1):
        assert call_prefill(lib, opts=_weights_opts(w)) == ssm.SSM_EINVAL
        assert "weights" in ssm.ssm_last_error()
        assert call_prefill_fp8qk(lib, opts=_weights_opts(w)) == ssm.SSM_EINVAL
    pot = ssm.WEIGHTS["rowmax_pot"]
    dec = ssm.Opts(0.0, 0, 0, 16, 256 * 1024, 1 << 30)
    dec.weights = pot
    assert call_decode(lib, opts=dec) == ssm.SSM_EUNSUPPORTED and "weights" in ssm.ssm_last_error()
    assert call_prefill_paged(lib, opts=_weights_opts(pot)) == ssm.SSM_EUNSUPPORTED
    assert "weights" in ssm.ssm_last_error()
    with pytest.raises(ValueError):
        ssm._weights_code("softmax")


def ssm_h_define(name):
    m = re.search(rf"#define {name} (\d+)", open(os.path.join(ROOT, "include", "ssm.h")).read())
    return int(m.group(1))


def test_prefill_stats_too_small(lib):
    q, k, v, o = desc([1, 256, 8, 128]), desc([1, 256, 2, 128]), desc([1, 256, 2, 128]), desc([1, 256, 8, 128])
    st = ssm.SkipStatsC()
    st.tile_state = FAKE
    st.tile_state_len = 10
    rc = lib.ssm_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 256, 1, -6.9, ctypes.byref(o),
                         ctypes.byref(st), None, None)
    assert rc == ssm.SSM_EINVAL and "tile_state" in ssm.ssm_last_error()


def cache(shape, paged=False, max_pages=0, dtype=ssm.SSM_BF16, scale=0.0, stride=None):
    c = ssm.KvCache()
    c.pool = desc(shape, dtype=dtype, stride=stride)
    c.scale = scale
    if paged:
        c.page_table = FAKE
        c.page_size = shape[2]
        c.max_pages = max_pages
    return c


def call_decode(lib, q=None, kc=None, vc=None, lens=FAKE, tau=-6.9, o=None, opts="default"):
    q = q or desc([2, 16, 128])
    o = o or desc([2, 16, 128])
    kc = kc or cache([2, 2, 1024, 128])
    vc = vc or cache([2, 2, 1024, 128])
    if opts == "default":
        opts = ssm.Opts(0.0, 0, 0, 16, 256 * 1024, 1 << 30)
    return lib.ssm_decode(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc), lens, tau, ctypes.byref(o), None,
                          None, ctypes.byref(opts) if opts else None)


def test_decode_noalloc_rejects_before_any_device_call(lib):
    """ssm_decode_noalloc validates like ssm_decode, then rejects a request whose workspace exceeds its 32 MiB static
    scratch with SSM_EWORKSPACE (no HIP call, nothing launched: this runs without a GPU)."""
    B, Hq, d, P = 64, 64, 128, 64
    assert ssm.ssm_decode_workspace_bytes(B, Hq, d, P) > 32 << 20
    q, o = desc([B, Hq, d]), desc([B, Hq, d])
    kc, vc = cache([B, 8, 1024, d]), cache([B, 8, 1024, d])
    opts = ssm.Opts(0.0, 0, 0, P, None, 0, 0)
    call = lambda tau, op: lib.ssm_decode_noalloc(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc), FAKE, tau,
                                                  ctypes.byref(o), None, None, ctypes.byref(op) if op else None)
    assert call(-6.9, opts) == ssm.SSM_EWORKSPACE
    assert "static scratch" in ssm.ssm_last_error()
    assert call(1.0, opts) == ssm.SSM_EINVAL          # tau > 0: the same checks as ssm_decode come first
    assert call(-6.9, ssm.Opts(0.0, 0, 0, 65, None, 0, 0)) == ssm.SSM_EUNSUPPORTED


@pytest.mark.parametrize("case,code", [
    ("no_workspace", ssm.SSM_EWORKSPACE), ("small_workspace", ssm.SSM_EWORKSPACE), ("null_lens", ssm.SSM_EINVAL),
    ("pos_tau", ssm.SSM_EINVAL), ("page_size", ssm.SSM_EUNSUPPORTED), ("mixed_paging", ssm.SSM_EINVAL),
    ("group_too_big", ssm.SSM_EUNSUPPORTED), ("splits", ssm.SSM_EUNSUPPORTED), ("batch", ssm.SSM_EINVAL),
    ("head_dim", ssm.SSM_EUNSUPPORTED), ("unknown_flag", ssm.SSM_EINVAL), ("fp8_no_scale", ssm.SSM_EINVAL),
    ("fp8_nan_scale", ssm.SSM_EINVAL), ("mixed_kv_dtypes", ssm.SSM_EINVAL), ("fp8_stride", ssm.SSM_EUNSUPPORTED),
    ("fp32_cache", ssm.SSM_EUNSUPPORTED), ("batch_too_large", ssm.SSM_EUNSUPPORTED),
    ("too_many_pages", ssm.SSM_EUNSUPPORTED),
])
def test_decode_rejects(lib, case, code):
    kw = {}
    if case == "batch_too_large":
        # more sequences than the grid's (b, g, split) numbering allows; nothing is dereferenced
        kw["q"], kw["o"] = desc([70000, 16, 128]), desc([70000, 16, 128])
        kw["kc"], kw["vc"] = cache([70000, 2, 1024, 128]), cache([70000, 2, 1024, 128])
    elif case == "too_many_pages":
        kw["kc"] = cache([100, 2, 64, 128], paged=True, max_pages=(1 << 25))
        kw["vc"] = cache([100, 2, 64, 128], paged=True, max_pages=(1 << 25))
    if case == "no_workspace":
        kw["opts"] = None
    elif case == "small_workspace":
        kw["opts"] = ssm.Opts(0.0, 0, 0, 16, 256 * 1024, 100)
    elif case == "null_lens":
        kw["lens"] = None
    elif case == "pos_tau":
        kw["tau"] = 1.0
    elif case == "page_size":
        kw["kc"] = cache([100, 2, 32, 128], paged=True, max_pages=64)
        kw["vc"] = cache([100, 2, 32, 128], paged=True, max_pages=64)
    elif case == "mixed_paging":
        kw["kc"] = cache([100, 2, 64, 128], paged=True, max_pages=64)
    elif case == "group_too_big":
        kw["q"], kw["o"] = desc([2, 64, 128]), desc([2, 64, 128])
        kw["kc"], kw["vc"] = cache([2, 2, 1024, 128]), cache([2, 2, 1024, 128])
    elif case == "splits":
        kw["opts"] = ssm.Opts(0.0, 0, 0, 65, 256 * 1024, 1 << 30)
    elif case == "batch":
        kw["kc"], kw["vc"] = cache([3, 2, 1024, 128]), cache([3, 2, 1024, 128])
    elif case == "head_dim":
        kw["q"], kw["o"] = desc([2, 16, 80]), desc([2, 16, 80])
        kw["kc"], kw["vc"] = cache([2, 2, 1024, 80]), cache([2, 2, 1024, 80])
    elif case == "unknown_flag":
        kw["opts"] = ssm.Opts(0.0, 0, 0, 16, 256 * 1024, 1 << 30, 2)
    elif case in ("fp8_no_scale", "fp8_nan_scale"):
        sc = 0.0 if case == "fp8_no_scale" else math.nan
        kw["kc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP8_E4M3, scale=sc)
        kw["vc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP8_E4M3, scale=1.0)
    elif case == "mixed_kv_dtypes":
        kw["kc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP8_E4M3, scale=1.0)
    elif case == "fp8_stride":
        st = [2 * 1024 * 136, 1024 * 136, 136, 1]  # 136 fp8 elements: not a multiple of 16 bytes
        kw["kc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP8_E4M3, scale=1.0, stride=st)
        kw["vc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP8_E4M3, scale=1.0, stride=st)
    elif case == "fp32_cache":
        kw["kc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP32)
        kw["vc"] = cache([2, 2, 1024, 128], dtype=ssm.SSM_FP32)
    rc = call_decode(lib, **kw)
    assert rc == code, (rc, ssm.ssm_last_error())
    if case == "batch_too_large":
        assert "too large" in ssm.ssm_last_error()
    if case == "too_many_pages":
        assert "too many pages" in ssm.ssm_last_error()


def test_product_does_not_import_oracle():
    """The binding and the HIP sources never reference the oracle package."""
    pkg = os.path.join(ROOT, "long_context_flash_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text), f"{f} mentions the oracle"


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of the descriptor structs have the C compiler's sizes and field offsets."""
    structs = {"ssm_tensor": ssm.Tensor, "ssm_kv_cache": ssm.KvCache, "ssm_skip_stats": ssm.SkipStatsC,
               "ssm_opts": ssm.Opts}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "ssm.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        cname, field, val = line.split()
        got[(cname, field)] = int(val)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


def call_prefill_paged(lib, q=None, kc=None, vc=None, q_start=FAKE, kv_lens=FAKE, batch=2, max_q=256, tau=-6.9,
                       o=None, opts="default"):
    q = q or desc([300, 16, 128])
    o = o or desc([300, 16, 128])
    kc = kc or cache([100, 2, 64, 128], paged=True, max_pages=64)
    vc = vc or cache([100, 2, 64, 128], paged=True, max_pages=64)
    if opts == "default":
        opts = ssm.Opts(0.0, 0, 0, 0, None, 0, 0)
    return lib.ssm_prefill_paged(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc), q_start, kv_lens, batch, max_q,
                                 1, tau, ctypes.byref(o), None, None, ctypes.byref(opts) if opts else None)


@pytest.mark.parametrize("case,code", [
    ("contiguous_cache", ssm.SSM_EINVAL), ("null_q_start", ssm.SSM_EINVAL), ("null_kv_lens", ssm.SSM_EINVAL),
    ("neg_batch", ssm.SSM_EINVAL), ("pos_tau", ssm.SSM_EINVAL), ("page_tables_differ", ssm.SSM_EINVAL),
    ("fp8_k_bf16_v", ssm.SSM_EINVAL), ("fp8_zero_scale", ssm.SSM_EINVAL), ("fp8_stride", ssm.SSM_EUNSUPPORTED),
    ("head_dim", ssm.SSM_EUNSUPPORTED), ("tile_q", ssm.SSM_EUNSUPPORTED),
    ("gqa", ssm.SSM_EINVAL), ("out_shape", ssm.SSM_EINVAL),
])
def test_prefill_paged_rejects(lib, case, code):
    kw = {}
    if case == "contiguous_cache":
        kw["kc"], kw["vc"] = cache([2, 2, 1024, 128]), cache([2, 2, 1024, 128])
    elif case == "null_q_start":
        kw["q_start"] = None
    elif case == "null_kv_lens":
        kw["kv_lens"] = None
    elif case == "neg_batch":
        kw["batch"] = -1
    elif case == "pos_tau":
        kw["tau"] = 0.5
    elif case == "page_tables_differ":
        kw["vc"] = cache([100, 2, 64, 128], paged=True, max_pages=32)
    elif case == "fp8_k_bf16_v":
        kw["kc"] = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=ssm.SSM_FP8_E4M3, scale=1.0)
    elif case == "fp8_zero_scale":
        kw["kc"] = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=ssm.SSM_FP8_E4M3, scale=1.0)
        kw["vc"] = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=ssm.SSM_FP8_E4M3, scale=0.0)
    elif case == "fp8_stride":  # 136 codes per row: not a multiple of 16 bytes
        st = [2 * 64 * 136, 64 * 136, 136, 1]
        kw["kc"] = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=ssm.SSM_FP8_E4M3, scale=1.0, stride=st)
        kw["vc"] = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=ssm.SSM_FP8_E4M3, scale=1.0, stride=st)
    elif case == "head_dim":
        kw["q"], kw["o"] = desc([300, 16, 96]), desc([300, 16, 96])
        kw["kc"] = cache([100, 2, 64, 96], paged=True, max_pages=64)
        kw["vc"] = cache([100, 2, 64, 96], paged=True, max_pages=64)
    elif case == "tile_q":
        kw["opts"] = ssm.Opts(0.0, 96, 0, 0, None, 0, 0)
    elif case == "gqa":
        kw["q"], kw["o"] = desc([300, 15, 128]), desc([300, 15, 128])
    elif case == "out_shape":
        kw["o"] = desc([299, 16, 128])
    rc = call_prefill_paged(lib, **kw)
    assert rc == code, (case, rc, ssm.ssm_last_error())


@pytest.mark.parametrize("case,code", [
    ("bf16_q", ssm.SSM_EUNSUPPORTED), ("bf16_cache", ssm.SSM_EUNSUPPORTED), ("zero_q_scale", ssm.SSM_EINVAL),
    ("nan_q_scale", ssm.SSM_EINVAL), ("zero_k_scale", ssm.SSM_EINVAL), ("pos_tau", ssm.SSM_EINVAL),
])
def test_prefill_paged_fp8qk_rejects(lib, case, code):
    f8 = ssm.SSM_FP8_E4M3
    q = desc([300, 16, 128], dtype=f8)
    kc = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=f8, scale=0.5)
    vc = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=f8, scale=0.5)
    q_scale, tau = 0.1, -6.9
    if case == "bf16_q":
        q = desc([300, 16, 128])
    elif case == "bf16_cache":
        kc = cache([100, 2, 64, 128], paged=True, max_pages=64)
        vc = cache([100, 2, 64, 128], paged=True, max_pages=64)
    elif case == "zero_q_scale":
        q_scale = 0.0
    elif case == "nan_q_scale":
        q_scale = math.nan
    elif case == "zero_k_scale":
        kc = cache([100, 2, 64, 128], paged=True, max_pages=64, dtype=f8, scale=0.0)
    elif case == "pos_tau":
        tau = 0.3
    o = desc([300, 16, 128])
    opts = ssm.Opts(0.0, 0, 0, 0, None, 0, 0)
    rc = lib.ssm_prefill_paged_fp8qk(ctypes.byref(q), q_scale, ctypes.byref(kc), ctypes.byref(vc), FAKE, FAKE, 2, 256,
                                     1, tau, ctypes.byref(o), None, None, ctypes.byref(opts))
    assert rc == code, (case, rc, ssm.ssm_last_error())


def test_prefill_paged_empty_batch_is_a_no_op(lib):
    assert call_prefill_paged(lib, batch=0) == ssm.SSM_OK
    assert call_prefill_paged(lib, max_q=0) == ssm.SSM_OK


def test_c_program_links_and_validates(tmp_path):
    """A plain C99 program (no C++ or torch) includes ssm.h, links libssm.so and gets error codes and messages
    back from argument validation (which returns before any device call)."""
    src = tmp_path / "use.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "ssm.h"
int main(void) {
  ssm_tensor q, k, v, o;
  memset(&q, 0, sizeof q); memset(&k, 0, sizeof k); memset(&v, 0, sizeof v); memset(&o, 0, sizeof o);
  if (ssm_abi_version() != SSM_ABI_VERSION) return 10;
  /* NULL data pointers: every entry point must refuse without touching the device */
  int rc = ssm_prefill(&q, &k, &v, 1, 1, -6.9f, &o, NULL, NULL, NULL);
  if (rc != SSM_EINVAL || strlen(ssm_last_error()) == 0) return 11;
  rc = ssm_prefill_fp8qk(&q, 1.0f, &k, 1.0f, &v, 1, 1, -6.9f, &o, NULL, NULL, NULL);
  if (rc != SSM_EINVAL) return 12;
  rc = ssm_decode(&q, NULL, NULL, NULL, -6.9f, &o, NULL, NULL, NULL);
  if (rc != SSM_EINVAL) return 13;
  if (ssm_decode_workspace_bytes(1, 8, 128, 16) == 0) return 14;
  printf("%s | %s\n", ssm_strerror(rc), ssm_last_error());
  return 0;
}
''')
    exe = tmp_path / "use"
    libdir = os.path.dirname(ssm.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lssm", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "q" in r.stdout


def test_binding_rejects_host_tensors_before_any_call():
    """The binding refuses tensors that are not on the call's GPU (the kernels would dereference host
    addresses); checked on the host, so it runs without a GPU."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(1, 64, 4, 64, dtype=bf)
    kv = torch.zeros(1, 64, 1, 64, dtype=bf)
    with pytest.raises(ValueError, match="needs every tensor"):
        ssm.ssm_prefill(q, kv, kv)
    with pytest.raises(ValueError, match="needs every tensor"):
        ssm.ssm_prefill_fp8qk(q.to(torch.float8_e4m3fn), 1.0, kv.to(torch.float8_e4m3fn), 1.0, kv)
    pool = torch.zeros(4, 1, 64, 64, dtype=bf)
    pt = torch.zeros(1, 4, dtype=torch.int32)
    qs, kl = torch.tensor([0, 64], dtype=torch.int32), torch.tensor([256], dtype=torch.int32)
    with pytest.raises(ValueError, match="needs every tensor"):
        ssm.ssm_prefill_paged(q[0], pool, pool, pt, qs, kl, 64)
    with pytest.raises(ValueError, match="needs every tensor"):
        ssm.ssm_prefill_paged_fp8qk(q[0].to(torch.float8_e4m3fn), 1.0, pool.to(torch.float8_e4m3fn),
                                    pool.to(torch.float8_e4m3fn), pt, qs, kl, 64, 1.0, 1.0)
    with pytest.raises(ValueError, match="needs every tensor"):
        ssm.ssm_decode(q[0, :1], pool, pool, kl, page_table=pt)


def test_skip_stats_dtypes_are_checked():
    import torch
    with pytest.raises(ValueError, match="tile_state"):
        ssm.SkipStats(tile_state=torch.zeros(4, dtype=torch.int32)).c()
    with pytest.raises(ValueError, match="counters"):
        ssm.SkipStats(counters=torch.zeros(3, dtype=torch.int64)).c()
    with pytest.raises(ValueError, match="unit_gap"):
        ssm.SkipStats(unit_gap=torch.zeros(4, 2, dtype=torch.float32)[:, 0]).c()


def test_empty_problems_are_no_ops_with_null_data(lib):
    """Empty views may carry NULL data (torch's empty tensors do); a call with nothing to compute returns
    SSM_OK without a launch (no GPU needed), and an empty decode needs no workspace or kv_lens."""
    opts = ssm.Opts(0.0, 0, 0, 0, None, 0, 0)
    q, k, v, o = desc([1, 0, 8, 128], data=None), desc([1, 0, 2, 128], data=None), \
        desc([1, 0, 2, 128], data=None), desc([1, 0, 8, 128], data=None)
    rc = lib.ssm_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, 1, -6.9, ctypes.byref(o), None, None,
                         ctypes.byref(opts))
    assert rc == ssm.SSM_OK, ssm.ssm_last_error()
    qd, od = desc([0, 8, 128], data=None), desc([0, 8, 128], data=None)
    kc = cache([0, 2, 64, 128])
    rc = lib.ssm_decode(ctypes.byref(qd), ctypes.byref(kc), ctypes.byref(kc), None, -6.9, ctypes.byref(od), None,
                        None, ctypes.byref(opts))
    assert rc == ssm.SSM_OK, ssm.ssm_last_error()
    # a non-empty view still needs its data
    q = desc([1, 4, 8, 128], data=None)
    rc = lib.ssm_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 4, 1, -6.9, ctypes.byref(o), None, None,
                         ctypes.byref(opts))
    assert rc == ssm.SSM_EINVAL
