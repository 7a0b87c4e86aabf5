"""Host-side logic of bench.py (CPU): the FLOP and byte counts behind the roofline figures, the parity fields of
the bench line, and the board power sampler (on a fake sysfs tree)."""
import math
import os
import time
from types import SimpleNamespace

import numpy as np

import bench


def test_prefill_flops_against_counting():
    """Dense-equivalent FLOP = 4 d per valid (query, key) pair, counted pair by pair; executed = one 128x64x d
    QK^T per visited tile plus one P.V per kept tile."""
    for causal in (True, False):
        w = SimpleNamespace(B=2, Hq=3, d=64, S=300, causal=causal, tile_q=128, tile_k=64)
        pairs = sum((i + 1) if causal else w.S for i in range(w.S))
        dense, executed = bench.prefill_flops(w, visited=17, kept=11)
        assert dense == 4.0 * w.d * pairs * w.B * w.Hq
        assert executed == 2.0 * 128 * 64 * 64 * (17 + 11)


def test_decode_bytes_against_counting():
    """K bytes: every cached row of every KV head; V bytes: the rows of kept tiles only (a partial last tile
    counts its valid rows), counted row by row."""
    rng = np.random.default_rng(5)
    w = SimpleNamespace(d=8, Hkv=2, Hq=4, B=3)
    lens = np.array([1, 64, 130], np.int32)
    nt = -(-lens // 64)
    state = np.zeros((w.B * w.Hkv, int(nt.max())), np.uint8)
    for b in range(w.B):
        state[b * w.Hkv:(b + 1) * w.Hkv, :nt[b]] = rng.integers(1, 3, (w.Hkv, nt[b]))
    k, v_kept, v_all, _ = bench.decode_bytes(w, lens, state, P=2)
    rows_kept = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            for row in range(int(lens[b])):
                rows_kept += state[b * w.Hkv + g, row // 64] == 1
    assert k == float(lens.sum()) * w.Hkv * w.d * 2
    assert v_all == k
    assert v_kept == float(rows_kept) * w.d * 2
    k1, v1, _, _ = bench.decode_bytes(w, lens, state, P=2, kv_elem=1)
    assert (k1, v1) == (k / 2, v_kept / 2)


def test_parity_fields():
    rng = np.random.default_rng(9)
    ref = rng.standard_normal((4, 64))
    ref[0, 0] = 4.0
    got = ref.copy()
    got[1, 3] += 0.009            # under the 1e-2 bar
    got[0, 0] += 0.015            # |o| = 4: bar 2^-8 * 4 + 2e-3 = 0.0176
    st_ref = np.array([[1, 2, 1, 0], [2, 2, 1, 0]], np.uint8)
    gamma = np.array([[np.inf, -9.0, -3.0, np.nan], [-7.0004, -8.0, -1.0, np.nan]])
    tau = -7.0
    st_gpu = st_ref.copy()
    st_gpu[1, 0] = 1              # a flip inside the 1e-3 band around tau
    r = bench.parity_fields(np, got, ref, st_gpu, st_ref, gamma, tau)
    assert math.isclose(r["max_abs"], 0.015, rel_tol=1e-3)
    assert math.isclose(r["rel_l2"], math.hypot(0.009, 0.015) / np.linalg.norm(ref), rel_tol=1e-3)
    assert (r["mask_tiles_off_band"], r["mask_agree_off_band"]) == (5, 5)
    assert (r["ambiguous_tiles"], r["ambiguous_flips"]) == (1, 1)
    assert r["unvisited_agree"] and r["pass"]
    # the oracle re-run takes the GPU's decision on that tile: keep (0) where the GPU kept it
    ov = bench.flip_override(np, st_gpu, st_ref, gamma, tau)
    assert ov[1, 0] == 0 and (np.delete(ov.ravel(), 4) == -1).all()
    assert bench.flip_override(np, st_ref, st_ref, gamma, tau) is None
    # a disagreement off the band, an output error over the bar, an unvisited mismatch: each fails
    bad = st_gpu.copy()
    bad[0, 1] = 1
    assert not bench.parity_fields(np, got, ref, bad, st_ref, gamma, tau)["pass"]
    far = got.copy()
    far[2, 2] += 0.02
    assert not bench.parity_fields(np, far, ref, st_gpu, st_ref, gamma, tau)["pass"]
    unv = st_gpu.copy()
    unv[0, 3] = 2
    assert not bench.parity_fields(np, got, ref, unv, st_ref, gamma, tau)["unvisited_agree"]


def _fake_card(root, n, watts, mhz):
    dev = root / f"card{n}" / "device"
    hw = dev / "hwmon" / f"hwmon{n + 3}"
    hw.mkdir(parents=True)
    (hw / "power1_input").write_text(f"{int(watts * 1e6)}\n")
    (hw / "power1_cap").write_text("1400000000\n")
    (dev / "pp_dpm_sclk").write_text(f"0: 500Mhz\n1: {mhz}Mhz *\n2: 2400Mhz\n")
    return dev


def test_board_sampler_on_fake_sysfs(tmp_path):
    dev = _fake_card(tmp_path, 0, 1234.5, 1900)
    assert bench.gpu_sysfs_dir(root=str(tmp_path)) == str(dev)
    with bench.BoardSampler(str(dev), period=0.001) as smp:
        time.sleep(0.05)
    s = smp.summary()
    assert s["mean_w"] == 1234.5 and s["max_w"] == 1234.5 and s["cap_w"] == 1400.0
    assert s["sclk_mean_mhz"] == 1900 and s["samples"] >= 2 and s["distinct_power_values"] == 1
    assert smp.summary(t0=time.monotonic() + 10) is None
    # no sysfs node: the sampler records nothing and the bench line carries no board figures
    with bench.BoardSampler(None) as none:
        pass
    assert none.summary() is None
    # two cards and no PCI address to tell them apart: no guess
    _fake_card(tmp_path, 1, 500.0, 2000)
    assert bench.gpu_sysfs_dir(root=str(tmp_path)) is None
    assert bench.gpu_sysfs_dir(root=os.path.join(str(tmp_path), "missing")) is None
