#!/usr/bin/env python3
"""Skip Softmax hot path on one MI355X: causal prefill at 128K + paged split-K decode at 128K.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only prefill|decode]

One step = one ssm_prefill call (batch 1, 64 query / 8 KV heads, d 128, S = 131072, causal,
tau = -ln 1000, ~50% skipped tiles) followed by one ssm_decode call (batch 32, 64/8 heads,
d 128, paged KV cache with kv_len ~ U[64K, 128K], 16 splits + log-sum-exp combine, tau
calibrated for ~50% skipped tiles).  Inputs are seeded synthetic tensors with
Llama-3.3-70B attention shapes, resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` is the prefill's dense-equivalent TFLOP/s
(4*Hq*d*S*(S+1)/2 FLOP over the prefill kernel's event-timed duration); the decode's
KV GB/s is reported beside it.  ``roofline`` is the prefill kernel against the bf16 MFMA
peak; ``roofline_decode`` is the decode path against HBM.  ``cpu_baseline`` is the fp64
oracle timed on a bounded sample of the same prefill work on the host cores.

After the timed steps (unless --main-only) the variants are timed on their own on the same inputs:
the sink-seeded and fp8-cache decodes, the fp8-score prefill, the chunked prefill (last 8192 queries
against a paged pool of all keys; bf16 pages, fp8 pages, 8-bit queries over fp8 pages), and the
speedup skipping buys over the dense kernel (the prefill at tau = -inf, the decode over its
calibrated tau sweep).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dense-equiv attn TFLOP/s (prefill 128K) + decode KV GB/s, at ~50% tile sparsity"
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "long_context_flash_amd", "csrc")
KERNEL_SOURCES = {"prefill": ["prefill_pp.hip", "prefill.hip", "ssm_device.h", "ssm_launch.h", "ssm_api.cpp"],
                  "decode": ["decode.hip", "ssm_device.h", "ssm_launch.h", "ssm_api.cpp"]}
COPY_PROBE_BYTES = 1 << 30
# the step's kernels as the profiler names them (d = 128, tile_q = 128, plain prefill, bf16 cache)
PREFILL_KERNEL = "prefill_pp_kernel"
DECODE_SPLIT_KERNEL = "decode_split_kernel<128, 2>"
DECODE_COMBINE_KERNEL = "decode_combine_kernel<128>"
DECODE_ORDER_KERNEL = "decode_order_kernel"


def sources_sha(path_kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path_kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(path_kind):
    """HBM bytes per launch recorded from FETCH_SIZE/WRITE_SIZE counter runs, if taken on the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[path_kind]
    except (OSError, KeyError, ValueError):
        return None
    return rec["bytes_per_launch"] if rec.get("source_sha256") == sources_sha(path_kind) else None


def _recorded(name, key):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        return json.load(f).get(key)


def recorded_mfma_ceiling():
    """Random-operand MFMA rate recorded in profiles/mfma_ceiling.json (None if absent)."""
    return _recorded("mfma_ceiling.json", "random_operands_tflops")


def recorded_read_ceiling():
    """Best streaming-read rate of the decode's load shapes recorded in profiles/read_ceiling.json (None if absent)."""
    return _recorded("read_ceiling.json", "best_gbps")


def summarize_traffic(fetch_dir, write_dir, command):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) into HBM bytes per launch,
    each scaled by what the same counter reads for a device copy of COPY_PROBE_BYTES.  The per-launch figure is
    the median over a kernel's dispatches: the runs take W warmup + K timed steps and then one untimed call that
    records the tile states (a fresh output buffer, byte-wise state writes), whose traffic differs from the
    timed calls' and must not set the figure."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    copy_names = [n for n in fetch if "copy" in n.lower()]
    copy = max(copy_names, key=lambda n: max(fetch[n]))
    kib = COPY_PROBE_BYTES / 1024.0
    f_fac = kib / max(fetch[copy])
    w_fac = kib / max(write[copy])

    def med(v):
        v = sorted(v)
        return v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])

    def launch_bytes(pred):
        tot = 0.0
        for n in fetch:
            if pred(n):
                tot += (med(fetch[n]) * f_fac + med(write[n]) * w_fac) * 1024
        return tot

    rec = {"copy_kernel": copy, "fetch_factor": f_fac, "write_factor": w_fac, "command": command,
           "prefill": {"kernels": PREFILL_KERNEL,
                       "bytes_per_launch": launch_bytes(lambda n: PREFILL_KERNEL in n),
                       "source_sha256": sources_sha("prefill")},
           "decode": {"kernels": "decode_order_kernel + decode_split_kernel + decode_combine_kernel",
                      "bytes_per_launch": launch_bytes(lambda n: DECODE_SPLIT_KERNEL in n or DECODE_COMBINE_KERNEL in n
                                                       or DECODE_ORDER_KERNEL in n),
                      "source_sha256": sources_sha("decode")}}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# HBM traffic from FETCH_SIZE / WRITE_SIZE (rocprofv3 --pmc), prefill_s128k and decode_b32_kv128k_paged",
             "", "Commands (MI355X, one GPU; $REPO is the repository root):", "", "```", command, "```", "",
             f"Normalisation: a device copy of {COPY_PROBE_BYTES} bytes (`{copy}`) reads FETCH_SIZE = "
             f"{max(fetch[copy]):.0f} KiB and WRITE_SIZE = {max(write[copy]):.0f} KiB; factors "
             f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write) scale each kernel's counters to bytes.", "",
             "Each figure is the median over the kernel's dispatches; FETCH_SIZE per dispatch in order, KiB, in the "
             "last column.", "",
             "| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (scaled) "
             "| FETCH_SIZE of each dispatch |",
             "|---|---|---|---|---|---|"]
    for n in sorted(fetch):
        fk = med(fetch[n])
        wk = med(write.get(n, [0]))
        each = " ".join(f"{x:.0f}" for x in fetch[n]) if len(fetch[n]) <= 8 else ""
        lines.append(f"| `{n[:90]}` | {len(fetch[n])} | {fk:.0f} | {wk:.0f} | {(fk * f_fac + wk * w_fac) * 1024:.4g} "
                     f"| {each} |")
    lines += ["", f"Per launch: prefill {rec['prefill']['bytes_per_launch']:.4g} B; decode (order + split + combine) "
              f"{rec['decode']['bytes_per_launch']:.4g} B."]
    with open(os.path.join(ROOT, "profiles", "hbm_traffic__prefill_s128k__decode_b32_kv128k_paged.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


# standalone measurement programs of this benchmark (not part of the library): the MFMA rate this GPU sustains
# with zero and random operands, and the HBM streaming-read rate in the decode's load shapes
CEILING_PROGRAMS = ("mfma_ceiling", "read_ceiling")
CEILING_DIR = os.path.join(ROOT, "_build", "ceilings")


def build_ceiling_programs():
    """Compile mfma_ceiling.hip and read_ceiling.hip (next to this file) into _build/ceilings/."""
    from long_context_flash_amd.build import HIPCC_FLAGS, hipcc
    os.makedirs(CEILING_DIR, exist_ok=True)
    for name in CEILING_PROGRAMS:
        exe = os.path.join(CEILING_DIR, name)
        r = subprocess.run([hipcc(), *HIPCC_FLAGS, os.path.join(ROOT, name + ".hip"), "-o", exe + ".tmp"],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}.hip:\n{r.stdout}\n{r.stderr}")
        os.replace(exe + ".tmp", exe)


def gpu_sysfs_dir(torch=None, root="/sys/class/drm"):
    """The sysfs device directory of cuda:0 that holds a hwmon power reading: matched by PCI address when torch
    reports it, else the only such GPU on the host; None if there is none (or no way to tell which)."""
    import glob
    cands = [d for d in sorted(glob.glob(os.path.join(root, "card*", "device")))
             if glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input"))]
    if torch is not None and cands:
        p = torch.cuda.get_device_properties(0)
        bus = getattr(p, "pci_bus_id", None)
        if bus is not None:
            for d in cands:
                addr = os.path.basename(os.path.realpath(d))  # domain:bus:device.function
                parts = addr.replace(".", ":").split(":")
                try:
                    dom, b, dv = (int(x, 16) for x in parts[:3])
                except ValueError:
                    continue
                if len(parts) == 4 and (dom, b, dv) == (getattr(p, "pci_domain_id", dom), bus,
                                                        getattr(p, "pci_device_id", dv)):
                    return d
    return cands[0] if len(cands) == 1 else None


class BoardSampler:
    """Board power and graphics clock of one GPU, read from sysfs on a host thread every `period` s while
    running: hwmon power1_input (socket power, microwatts; power1_cap is the limit the board holds it to) and
    the current level of pp_dpm_sclk (MHz), each sample stamped with time.monotonic()."""

    def __init__(self, dev_dir, period=0.01):
        import glob
        import threading
        hw = sorted(glob.glob(os.path.join(dev_dir, "hwmon", "hwmon*"))) if dev_dir else []
        self.hwmon = hw[0] if hw else None
        self.sclk = os.path.join(dev_dir, "pp_dpm_sclk") if dev_dir else None
        self.period = period
        self.samples = []  # (t, watts, mhz or None)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _read(path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    def cap_w(self):
        v = self._read(os.path.join(self.hwmon, "power1_cap")) if self.hwmon else None
        return int(v) / 1e6 if v and v.strip().isdigit() else None

    def _clock(self):
        text = self._read(self.sclk) if self.sclk else None
        for line in (text or "").splitlines():
            if line.rstrip().endswith("*"):
                digits = "".join(ch for ch in line.split(":", 1)[-1] if ch.isdigit())
                return int(digits) if digits else None
        return None

    def _run(self):
        pin = os.path.join(self.hwmon, "power1_input")
        while not self._stop.is_set():
            v = self._read(pin)
            if v and v.strip().isdigit():
                self.samples.append((time.monotonic(), int(v) / 1e6, self._clock()))
            self._stop.wait(self.period)

    def __enter__(self):
        if self.hwmon:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.hwmon:
            self._stop.set()
            self._thread.join()

    def summary(self, t0=None, t1=None):
        """Mean and largest power, mean clock and the limit over the samples in [t0, t1]; None without samples."""
        sel = [x for x in self.samples if (t0 is None or x[0] >= t0) and (t1 is None or x[0] <= t1)]
        if not sel:
            return None
        w = [x[1] for x in sel]
        mhz = [x[2] for x in sel if x[2] is not None]
        return {"mean_w": round(sum(w) / len(w), 1), "max_w": round(max(w), 1), "cap_w": self.cap_w(),
                "sclk_mean_mhz": round(sum(mhz) / len(mhz)) if mhz else None, "samples": len(sel),
                "distinct_power_values": len(set(w))}


def mfma_power(seconds):
    """Run mfma_ceiling in its sustained form beside a BoardSampler and print, per phase (idle; zero and random
    operands; random operands with LDS operand reads, transposing LDS reads, VALU work, tile loads, a barrier,
    scalar instructions, or LDS reads, VALU work and tile loads together; the same FLOP as 16x16x32 MFMAs;
    normal operands), the MFMA rate with
    the board's power and clock over the phase's last three quarters, and the energy above idle per
    wave-iteration (16 MFMAs of one wave with that phase's other work) and per executed FLOP."""
    exe = os.path.join(CEILING_DIR, "mfma_ceiling")
    if not os.path.exists(exe):
        sys.exit(f"{exe} is missing: build it with `python -c 'import bench; bench.build_ceiling_programs()'`")
    dev_dir = gpu_sysfs_dir()
    if dev_dir is None:
        sys.exit("no hwmon power reading found for the GPU")
    with BoardSampler(dev_dir) as smp:
        r = subprocess.run([exe, "20000", "sustain", str(seconds)], capture_output=True, text=True)
    if r.returncode != 0:
        sys.exit(f"mfma_ceiling failed ({r.returncode}): {r.stderr}")
    rec = json.loads(r.stdout)
    for ph in rec["phases"]:
        lo = ph["t0"] + 0.25 * (ph["t1"] - ph["t0"])
        ph["board"] = smp.summary(lo, ph["t1"])
    # the idle baseline: the idle phases between work phases (the first one may find the GPU in a deeper sleep)
    idle = [ph["board"]["mean_w"] for ph in rec["phases"][1:] if ph["phase"] == "idle" and ph["board"]]
    if idle:
        rec["idle_w"] = round(sum(idle) / len(idle), 1)
        base = None
        for ph in rec["phases"]:
            if ph["phase"] == "idle" or not ph["board"]:
                continue
            above = ph["board"]["mean_w"] - rec["idle_w"]
            ph["nj_per_wave_iter"] = round(above / ph["wave_iters_per_s"] * 1e9, 1)
            ph["pj_per_flop"] = round(above / (ph["tflops"] * 1e12) * 1e12, 4)
            if ph["phase"] == "random":
                base = ph["nj_per_wave_iter"]
            elif base is not None and (ph["phase"].startswith("random+") or ph["phase"] == "normal"):
                ph["nj_over_random"] = round(ph["nj_per_wave_iter"] - base, 1)
    rec["sysfs"] = dev_dir
    print(json.dumps(rec), flush=True)


def prefill_flops(w, visited, kept):
    dense = 4.0 * w.B * w.Hq * w.d * (w.S * (w.S + 1) / 2 if w.causal else w.S * w.S)
    per_tile = 2.0 * w.tile_q * w.tile_k * w.d
    return dense, per_tile * (visited + kept)


def decode_bytes(w, lens, state, P, kv_elem=2):
    """Algorithmic HBM bytes of one decode call (see the design notes for the accounting); kv_elem: bytes per
    cached K/V element (2 bf16, 1 fp8)."""
    import numpy as np
    d, Hkv, Hq, B = w.d, w.Hkv, w.Hq, w.B
    k_bytes = float(lens.astype(np.int64).sum()) * Hkv * d * kv_elem
    nt = -(-lens // 64)
    kept_rows = 0
    for b in range(B):
        last_rows = int(lens[b]) - (int(nt[b]) - 1) * 64
        st = state[b * Hkv:(b + 1) * Hkv, :nt[b]]
        kept = st == 1
        kept_rows += int(kept[:, :-1].sum()) * 64 + int(kept[:, -1].sum()) * last_rows
    v_kept = float(kept_rows) * d * kv_elem
    v_all = float(lens.astype(np.int64).sum()) * Hkv * d * kv_elem
    small = 2 * B * Hq * d * 2 + 2 * float(nt.sum()) * 4 + 2 * B * Hq * P * (d + 1) * 4
    return k_bytes, v_kept, v_all, small


def time_sink_seeded_decode(ssm, torch, np, w, data, dq, kp, vp, pt, lens, dout, ws, dstate, tau, steps, dev):
    """The sink-seeded split-K variant on the same decode workload and tau, timed on its own (after the step
    timing): HIP events around each call, counters in the timed calls, tile states from one more call."""
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    stats = ssm.SkipStats(counters=cnt)
    run = lambda st: ssm.ssm_decode(dq, kp, vp, lens, tau=tau, out=dout, page_table=pt, num_splits=w.num_splits,
                                    workspace=ws, skip_stats=st, sink_seed=True)
    run(stats)
    torch.cuda.synchronize()
    cnt.zero_()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        run(stats)
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    dstate.zero_()
    run(ssm.SkipStats(tile_state=dstate))
    state = dstate.cpu().numpy()
    c = cnt.cpu().numpy() / steps
    if not (int((state != 0).sum()) == c[0] and int((state == 2).sum()) == c[1]):
        raise RuntimeError("sink-seeded decode: tile states disagree with the timed counters")
    kb, vk, va, small = decode_bytes(w, data["kv_lens"], state, w.num_splits)
    nt = -(-data["kv_lens"] // 64)
    seeded_splits = 0  # non-empty splits after the first: ceil(n / ceil(n / P)) - 1 per sequence of n tiles
    for n in (int(x) for x in nt if x > 0):
        tps = -(-n // w.num_splits)
        seeded_splits += -(-n // tps) - 1
    seed_bytes = float(seeded_splits) * w.Hkv * 64 * w.d * 2  # key tile 0 once more per seeded split
    t = ms / 1e3
    tot = kb + vk + small + seed_bytes
    return {"ms": round(ms, 4), "tau": tau, "sparsity": round(float(c[1]) / float(c[0]), 4),
            "kv_gbps": round((kb + vk) / t / 1e9, 1), "total_gbps": round(tot / t / 1e9, 1),
            "hbm_frac": round(tot / t / 1e9 / HBM_PEAK_GBPS, 4), "per_launch_bytes": tot,
            "speedup_vs_split_local": None}


def time_fp8_decode(ssm, torch, np, w, data, dq, kp, vp, pt, lens, dout, ws, dstate, tau, steps, dev):
    """The decode over an fp8 e4m3 copy of the same paged cache (per-tensor scales amax/448, quantised on the
    GPU before timing), same tau and splits, timed on its own after the step timing."""
    def quant(pool):
        amax = float(pool.abs().max().float())
        scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
        codes = torch.empty(pool.shape, dtype=torch.float8_e4m3fn, device=dev)
        for i in range(0, pool.shape[0], 4096):
            codes[i:i + 4096] = (pool[i:i + 4096].float() / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        return codes, scale
    k8, ks = quant(kp)
    v8, vs = quant(vp)
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda st: ssm.ssm_decode(dq, k8, v8, lens, tau=tau, out=dout, page_table=pt, num_splits=w.num_splits,
                                    workspace=ws, skip_stats=st, k_scale=ks, v_scale=vs)
    run(ssm.SkipStats(counters=cnt))
    torch.cuda.synchronize()
    cnt.zero_()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        run(ssm.SkipStats(counters=cnt))
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    dstate.zero_()
    run(ssm.SkipStats(tile_state=dstate))
    state = dstate.cpu().numpy()
    c = cnt.cpu().numpy() / steps
    if not (int((state != 0).sum()) == c[0] and int((state == 2).sum()) == c[1]):
        raise RuntimeError("fp8 decode: tile states disagree with the timed counters")
    kb, vk, va, small = decode_bytes(w, data["kv_lens"], state, w.num_splits, kv_elem=1)
    t = ms / 1e3
    del k8, v8
    return {"ms": round(ms, 4), "tau": tau, "k_scale": ks, "v_scale": vs,
            "sparsity": round(float(c[1]) / float(c[0]), 4), "kv_gbps": round((kb + vk) / t / 1e9, 1),
            "total_gbps": round((kb + vk + small) / t / 1e9, 1),
            "hbm_frac": round((kb + vk + small) / t / 1e9 / HBM_PEAK_GBPS, 4), "per_launch_bytes": kb + vk + small,
            "speedup_vs_bf16": None}


def _timed(torch, np, fn, steps, before=None):
    """mean ms of `steps` calls of fn between HIP events on the current stream, after one untimed call; `before`
    (untimed) runs ahead of each timed call"""
    fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        if before is not None:
            before()
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))


def _graph_timed(torch, np, fn, steps, before=None):
    """mean ms of `steps` replays of a HIP graph holding one call of fn (captured after one eager call on a side
    stream), between HIP events on the current stream"""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    ms = _timed(torch, np, g.replay, steps, before)
    del g
    return ms


def time_prefill_vs_dense(ssm, torch, np, w, q, k, v, out, skip_ms, sparsity, steps, dev):
    """The same prefill launch at tau = -inf (no tile skipped: the dense kernel) against the timed skip launch:
    the speedup skipping buys on this input, the quantity the Skip Softmax pages report (as context: 1.4x for
    prefill of Llama 3.3 70B at 128K on GB200)."""
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    with BoardSampler(gpu_sysfs_dir(torch)) as board:
        ms = _timed(torch, np, lambda: ssm.ssm_prefill(q, k, v, causal=True, tau=-math.inf, out=out,
                                                       skip_stats=ssm.SkipStats(counters=cnt), tile_q=w.tile_q),
                    steps)
    c = cnt.cpu().numpy()
    if int(c[1]) != 0:
        raise RuntimeError("tau = -inf skipped tiles")
    res = {"dense_ms": round(ms, 3), "skip_ms": skip_ms, "skip_sparsity": sparsity,
           "speedup_vs_dense": round(ms / skip_ms, 3), "pages_prefill_speedup": 1.4}
    if board.summary() is not None:
        res["board_power"] = board.summary()
    return res


def time_pot_prefill(ssm, torch, np, w, q, k, v, out, tau, exp_ms, exp_dense_ms, steps, dev):
    """Rowmax-PoT weights ("Approximating Softmax in Pretrained LLMs", Abstract: powers of two anchored at the row
    maximum in place of the exponentials) on the same input: the launch at tau and at tau = -inf (every tile's
    weights computed) against the exponential-weight launches, and how far the output moves from the
    exponential one (max abs and relative L2 over the whole output; the page reports the effect as a perplexity
    change, which needs a trained model)."""
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda t: ssm.ssm_prefill(q, k, v, causal=True, tau=t, out=out, skip_stats=ssm.SkipStats(counters=cnt),
                                    tile_q=w.tile_q, weights="rowmax_pot")
    with BoardSampler(gpu_sysfs_dir(torch)) as board:
        ms = _timed(torch, np, lambda: run(tau), steps)
    c = cnt.cpu().numpy() / (steps + 1)
    cnt.zero_()
    dense_ms = _timed(torch, np, lambda: run(-math.inf), steps)
    if int(cnt[1]) != 0:
        raise RuntimeError("tau = -inf skipped tiles")
    out_e = torch.empty_like(out)
    ssm.ssm_prefill(q, k, v, causal=True, tau=tau, out=out_e, tile_q=w.tile_q)
    run(tau)
    torch.cuda.synchronize()
    mx, dd, ee = 0.0, 0.0, 0.0
    for i in range(0, w.S, 8192):
        e = out_e[:, i:i + 8192].float()
        dlt = out[:, i:i + 8192].float() - e
        mx = max(mx, float(dlt.abs().max()))
        dd += float((dlt * dlt).sum())
        ee += float((e * e).sum())
    del out_e
    visited, skipped = float(c[0]), float(c[1])
    dense, executed = prefill_flops(w, visited, visited - skipped)
    return {"workload": f"{w.name}, weights 2^(rint(log2e*l) - rint(log2e*rowmax))", "ms": round(ms, 3),
            "dense_tflops": round(dense / (ms / 1e3) / 1e12, 2),
            "executed_tflops": round(executed / (ms / 1e3) / 1e12, 2), "sparsity": round(skipped / visited, 4),
            "speedup_vs_exp": round(exp_ms / ms, 3), "no_skip_ms": round(dense_ms, 3),
            "no_skip_speedup_vs_exp": round(exp_dense_ms / dense_ms, 3),
            "vs_exp_output": {"max_abs": float("%.4g" % mx), "rel_l2": float("%.4g" % math.sqrt(dd / max(ee, 1e-300)))},
            "pages_speedup": {"causal_8k_fp8": 1.124, "noncausal_8k_fp8": 1.258, "hardware": "B200"},
            "board_power": board.summary()}


def time_decode_tau_sweep(ssm, torch, np, w, dq, kp, vp, pt, lens, dout, ws, steps, dev):
    """The decode at each calibrated tau of its workload (tau = -inf, written as null, is the dense kernel): time,
    sparsity and the speedup over tau = -inf (as context: the pages project 1.36x for decode of Llama 3.3 70B)."""
    rows = []
    for tau in w.taus:
        cnt = torch.zeros(4, dtype=torch.int64, device=dev)
        ms = _timed(torch, np, lambda: ssm.ssm_decode(dq, kp, vp, lens, tau=tau, out=dout, page_table=pt,
                                                      num_splits=w.num_splits, workspace=ws,
                                                      skip_stats=ssm.SkipStats(counters=cnt)), steps)
        c = cnt.cpu().numpy()
        # tau = -inf is written as null (JSON has no infinities)
        rows.append({"tau": None if math.isinf(tau) else round(float(tau), 4), "ms": round(ms, 4),
                     "sparsity": round(float(c[1]) / float(c[0]), 4)})
    dense = rows[0]["ms"]
    for r in rows:
        r["speedup_vs_dense"] = round(dense / r["ms"], 3)
    return {"sweep": rows, "pages_decode_speedup": 1.36}


def recorded_fp8_mfma_ceiling():
    """Random-operand fp8 MFMA rate recorded in profiles/mfma_ceiling.json (None if absent)."""
    rec = _recorded("mfma_ceiling.json", "fp8")
    return rec.get("random_operands_tflops") if rec else None


def time_fp8qk_prefill(ssm, torch, np, w, q, k, v, out, tau, bf16_ms, steps, dev):
    """The same prefill with 8-bit queries and keys (NEXT row, FP8 MFMA): q and k quantised on the GPU to OCP
    e4m3 codes with amax/448 scales before timing, v bf16; timed on its own after the steps with HIP events,
    skip counters in the timed calls.  The MFMA work splits into fp8 QK^T (every visited tile) and bf16 P.V
    (kept tiles); `mfma_frac` is the time those would take at the published peaks over the measured time."""
    def quant(x):
        amax = float(x.abs().max().float())
        scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
        codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=dev)
        for i in range(0, x.shape[1], 8192):
            codes[:, i:i + 8192] = (x[:, i:i + 8192].float() / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        return codes, scale
    q8, qs = quant(q)
    k8, ks = quant(k)
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda: ssm.ssm_prefill_fp8qk(q8, qs, k8, ks, v, causal=True, tau=tau, out=out,
                                        skip_stats=ssm.SkipStats(counters=cnt), tile_q=w.tile_q)
    run()
    torch.cuda.synchronize()
    cnt.zero_()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    with BoardSampler(gpu_sysfs_dir(torch)) as board:
        for i in range(steps):
            ev[i][0].record()
            run()
            ev[i][1].record()
        torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    c = cnt.cpu().numpy() / steps
    visited, skipped = float(c[0]), float(c[1])
    dense, executed = prefill_flops(w, visited, visited - skipped)
    qk_flop = 2.0 * w.tile_q * w.tile_k * w.d * visited
    pv_flop = executed - qk_flop
    t = ms / 1e3
    ideal = qk_flop / (2 * MFMA_BF16_PEAK_TFLOPS * 1e12) + pv_flop / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    res = {"workload": f"{w.name} with e4m3 q/k (amax/448 scales), bf16 v", "ms": round(ms, 3),
           "dense_tflops": round(dense / t / 1e12, 2), "executed_tflops": round(executed / t / 1e12, 2),
           "qk_fp8_tflops": round(qk_flop / t / 1e12, 2), "pv_bf16_tflops": round(pv_flop / t / 1e12, 2),
           "mfma_frac": round(ideal / t, 4), "sparsity": round(skipped / visited, 4), "tau": tau,
           "q_scale": qs, "k_scale": ks, "speedup_vs_bf16": round(bf16_ms / ms, 3), "board_power": board.summary()}
    c8, c16 = recorded_fp8_mfma_ceiling(), recorded_mfma_ceiling()
    if c8 and c16:
        res["mfma_frac_of_measured_ceilings"] = round((qk_flop / (c8 * 1e12) + pv_flop / (c16 * 1e12)) / t, 4)
    del q8, k8
    return res


CHUNK_Q = 8192  # the chunked-prefill leg: the last 8192 queries of the 128K input against all of its keys


def time_chunked_prefill(ssm, torch, np, w, data, tau, steps, dev):
    """Chunked prefill against a paged cache (NEXT row): the last CHUNK_Q queries of the 128K prefill input
    attend to all S keys held in a 64-token-page pool at a seeded random page order; timed on its own after
    the steps with HIP events, skip counters in the timed calls."""
    S, nq = w.S, CHUNK_Q
    npages = -(-S // 64)
    perm = np.random.default_rng(w.seed).permutation(npages).astype(np.int32)
    k = torch.from_numpy(data["k"][0].view(np.int16)).view(torch.bfloat16)      # [S, Hkv, d] host
    v = torch.from_numpy(data["v"][0].view(np.int16)).view(torch.bfloat16)
    pool_k = torch.empty(npages, w.Hkv, 64, w.d, dtype=torch.bfloat16, device=dev)
    pool_v = torch.empty_like(pool_k)
    kd = k.to(dev).view(npages, 64, w.Hkv, w.d).transpose(1, 2)
    vd = v.to(dev).view(npages, 64, w.Hkv, w.d).transpose(1, 2)
    idx = torch.from_numpy(perm.astype(np.int64)).to(dev)
    pool_k[idx] = kd
    pool_v[idx] = vd
    del kd, vd
    pt = torch.from_numpy(perm[None, :]).to(dev)
    q = torch.from_numpy(data["q"][0, S - nq:].view(np.int16)).view(torch.bfloat16).to(dev)   # [nq, Hq, d]
    qs = torch.tensor([0, nq], dtype=torch.int32, device=dev)
    kl = torch.tensor([S], dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda: ssm.ssm_prefill_paged(q, pool_k, pool_v, pt, qs, kl, nq, causal=True, tau=tau, out=out,
                                        skip_stats=ssm.SkipStats(counters=cnt), tile_q=w.tile_q)
    run()
    torch.cuda.synchronize()
    cnt.zero_()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    with BoardSampler(gpu_sysfs_dir(torch)) as board:
        for i in range(steps):
            ev[i][0].record()
            run()
            ev[i][1].record()
        torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    c = cnt.cpu().numpy() / steps
    visited, skipped = float(c[0]), float(c[1])
    off = S - nq
    dense = 4.0 * w.Hq * w.d * (nq * off + nq * (nq + 1) / 2)  # query i sees off + i + 1 keys
    executed = 2.0 * w.tile_q * w.tile_k * w.d * (2 * visited - skipped)
    t = ms / 1e3
    res = {"workload": f"chunk q{nq} of kv{S} (paged, 64-token pages)", "ms": round(ms, 3),
           "dense_tflops": round(dense / t / 1e12, 2), "executed_tflops": round(executed / t / 1e12, 2),
           "mfma_frac": round(executed / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4), "sparsity": round(skipped / visited, 4),
           "tau": tau}
    # the same chunk over an fp8 e4m3 copy of the pools (amax/448 scales, quantised on the GPU before timing)
    def quant(pool):
        amax = float(pool.abs().max().float())
        scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
        codes = torch.empty(pool.shape, dtype=torch.float8_e4m3fn, device=dev)
        for i in range(0, pool.shape[0], 4096):
            codes[i:i + 4096] = (pool[i:i + 4096].float() / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
        return codes, scale
    k8, ks = quant(pool_k)
    v8, vs = quant(pool_v)
    cnt8 = torch.zeros(4, dtype=torch.int64, device=dev)
    run8 = lambda: ssm.ssm_prefill_paged(q, k8, v8, pt, qs, kl, nq, causal=True, tau=tau, out=out,
                                         skip_stats=ssm.SkipStats(counters=cnt8), tile_q=w.tile_q, k_scale=ks,
                                         v_scale=vs)
    run8()
    torch.cuda.synchronize()
    cnt8.zero_()
    for i in range(steps):
        ev[i][0].record()
        run8()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms8 = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    c8 = cnt8.cpu().numpy() / steps
    res["fp8_cache"] = {"ms": round(ms8, 3), "dense_tflops": round(dense / (ms8 / 1e3) / 1e12, 2),
                        "sparsity": round(float(c8[1]) / float(c8[0]), 4), "k_scale": ks, "v_scale": vs,
                        "speedup_vs_bf16_cache": round(ms / ms8, 3)}
    # and with the queries as e4m3 codes too (amax/448), QK^T on the fp8 MFMA (ssm_prefill_paged_fp8qk)
    qamax = float(q.abs().max().float())
    qsc = float(np.float32(qamax / 448.0)) if qamax > 0 else 1.0
    q8 = (q.float() / qsc).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    cnt88 = torch.zeros(4, dtype=torch.int64, device=dev)
    run88 = lambda: ssm.ssm_prefill_paged_fp8qk(q8, qsc, k8, v8, pt, qs, kl, nq, k_scale=ks, v_scale=vs, causal=True,
                                                tau=tau, out=out, skip_stats=ssm.SkipStats(counters=cnt88),
                                                tile_q=w.tile_q)
    run88()
    torch.cuda.synchronize()
    cnt88.zero_()
    for i in range(steps):
        ev[i][0].record()
        run88()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms88 = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    c88 = cnt88.cpu().numpy() / steps
    res["fp8_qk_fp8_cache"] = {"ms": round(ms88, 3), "dense_tflops": round(dense / (ms88 / 1e3) / 1e12, 2),
                               "sparsity": round(float(c88[1]) / float(c88[0]), 4), "q_scale": qsc,
                               "speedup_vs_bf16_cache": round(ms / ms88, 3)}
    del pool_k, pool_v, k8, v8, q, q8, out
    return res


def leg_decode_32k(ssm, torch, np, steps, dev, threads, cpu=True):
    """decode_b8_kv32k (batch 8, 64/8 heads, d 128, contiguous 32K caches, tau = -ln 1000) with 16 split-local
    scans, one scan, and 16 sink-seeded scans: GPU time, sparsity and HBM rate of each, beside the oracle's time
    on all 8 sequences of the same input and the parity of the timed output."""
    import synth
    w = synth.DECODE_32K
    tau = w.taus[0]
    data = synth.gen_decode(w, threads=threads)
    dq = ssm.bf16_from_bits(data["q"], dev)
    kc, vc = ssm.bf16_from_bits(data["k_cache"], dev), ssm.bf16_from_bits(data["v_cache"], dev)
    lens = torch.from_numpy(data["kv_lens"]).to(dev)
    out = torch.empty_like(dq)
    max_tiles = -(-kc.shape[2] // 64)
    state = torch.zeros(w.B * w.Hkv, max_tiles, dtype=torch.uint8, device=dev)
    # the caches (1.07 GB) are 4x the last-level cache: each timed call follows an untimed read of 1 GiB, so no call
    # finds the previous one's lines there (a read leaves no dirty lines to write back during the timed call)
    scratch = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    flush = lambda: scratch.max()
    rows = []
    for name, P, seeded in (("split_local_p16", 16, False), ("one_scan_p1", 1, False), ("sink_seeded_p16", 16, True)):
        ws = ssm.decode_workspace(w.B, w.Hq, w.d, P, dev)
        cnt = torch.zeros(4, dtype=torch.int64, device=dev)
        run = lambda st: ssm.ssm_decode(dq, kc, vc, lens, tau=tau, out=out, num_splits=P, workspace=ws,
                                        skip_stats=st, sink_seed=seeded)
        ms = _timed(torch, np, lambda: run(ssm.SkipStats(counters=cnt)), steps, flush)
        got = out.float().cpu().numpy()
        c = cnt.cpu().numpy() / (steps + 1)
        # the same call replayed from a HIP graph (its three kernels launched as one graph)
        cnt_g = torch.zeros_like(cnt)
        graph_ms = _graph_timed(torch, np, lambda: run(ssm.SkipStats(counters=cnt_g)), steps, flush) if P > 1 else None
        state.zero_()
        run(ssm.SkipStats(tile_state=state))
        st = state.cpu().numpy()
        if not (int((st != 0).sum()) == c[0] and int((st == 2).sum()) == c[1]):
            raise RuntimeError(f"decode 32K {name}: tile states disagree with the timed counters")
        kb, vk, va, small = decode_bytes(w, data["kv_lens"], st, P)
        nt = -(-data["kv_lens"] // 64)
        seed_bytes = 0.0
        if seeded:
            for n in (int(x) for x in nt if x > 0):
                tps = -(-n // P)
                seed_bytes += (-(-n // tps) - 1) * w.Hkv * 64 * w.d * 2
        t = ms / 1e3
        tot = kb + vk + small + seed_bytes
        row = {"variant": name, "num_splits": P, "sink_seed": seeded, "ms": round(ms, 4),
               "sparsity": round(float(c[1]) / float(c[0]), 4), "kv_gbps": round((kb + vk) / t / 1e9, 1),
               "total_gbps": round(tot / t / 1e9, 1), "hbm_frac": round(tot / t / 1e9 / HBM_PEAK_GBPS, 4)}
        if graph_ms is not None:
            row["graph_ms"] = round(graph_ms, 4)
        if cpu:
            base, par = cpu_baseline_decode(np, w, data, tau, threads, P, got, st, sink_seed=seeded)
            row["oracle_kv_gbps"] = round(base["value"], 3)
            row["oracle_seconds"] = base["seconds"]
            row["gpu_over_oracle"] = round(row["kv_gbps"] / base["value"], 1)
            row["parity"] = par
        rows.append(row)
        del ws
    del kc, vc, scratch
    return {"workload": f"{w.name} (contiguous, kv_len {w.kv_len}, tau -ln 1000)", "tau": tau,
            "timing": "each timed call after an untimed 1 GiB read (the last-level cache holds none of the caches)",
            "oracle_threads": threads, "variants": rows}


def leg_decode_b256(ssm, torch, np, steps, dev, threads, cpu=True, n_seq=8):
    """decode_b256_kv16k_paged: 256 sequences (kv_len ~ U[8K, 16K], as many keys in all as the 128K decode) through
    one ssm_decode call: the longest-first ordering kernel (one pass over the 256 lengths), the split kernel over
    256 x 8 x 16 workgroups and the combine.  GPU time and HBM rate, and the parity of the timed outputs on
    sampled sequences (the longest, the shortest and n_seq - 2 others) against the oracle."""
    import synth
    w = synth.DECODE_B256
    tau = w.taus[0]
    P = w.num_splits
    data = synth.gen_decode(w, threads=threads)
    dq = ssm.bf16_from_bits(data["q"], dev)
    kp, vp = ssm.bf16_from_bits(data["k_pool"], dev), ssm.bf16_from_bits(data["v_pool"], dev)
    pt = torch.from_numpy(data["page_table"]).to(dev)
    lens = torch.from_numpy(data["kv_lens"]).to(dev)
    out = torch.empty_like(dq)
    ws = ssm.decode_workspace(w.B, w.Hq, w.d, P, dev)
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    run = lambda st: ssm.ssm_decode(dq, kp, vp, lens, tau=tau, out=out, page_table=pt, num_splits=P, workspace=ws,
                                    skip_stats=st)
    ms = _timed(torch, np, lambda: run(ssm.SkipStats(counters=cnt)), steps)
    got = out.float().cpu().numpy()
    c = cnt.cpu().numpy() / (steps + 1)
    state = torch.zeros(w.B * w.Hkv, pt.shape[1], dtype=torch.uint8, device=dev)
    run(ssm.SkipStats(tile_state=state))
    st = state.cpu().numpy()
    if not (int((st != 0).sum()) == c[0] and int((st == 2).sum()) == c[1]):
        raise RuntimeError("decode B=256: tile states disagree with the timed counters")
    kb, vk, va, small = decode_bytes(w, data["kv_lens"], st, P)
    t = ms / 1e3
    tot = kb + vk + small
    res = {"workload": f"{w.name} (B {w.B}, paged, kv_len U[{w.kv_len_lo}, {w.kv_len_hi}], P {P}, tau -ln 1000)",
           "ms": round(ms, 4), "sparsity": round(float(c[1]) / float(c[0]), 4),
           "kv_gbps": round((kb + vk) / t / 1e9, 1), "total_gbps": round(tot / t / 1e9, 1),
           "hbm_frac": round(tot / t / 1e9 / HBM_PEAK_GBPS, 4)}
    del kp, vp, ws
    if cpu:
        import oracle
        L = data["kv_lens"]
        order = np.argsort(-L, kind="stable")
        rng = np.random.default_rng(256)
        others = rng.choice(order[1:-1], n_seq - 2, replace=False)
        pick = np.array([order[0], order[-1], *others], np.int64)
        kc, vc = paged_to_contiguous(np, w, data, pick)
        r = oracle.decode(data["q"][pick], kc, vc, L[pick], tau=tau, num_splits=P, threads=threads)
        maxt = r["state"].shape[1]
        rows = (pick[:, None] * w.Hkv + np.arange(w.Hkv)[None, :]).ravel()
        stg = st[rows][:, :maxt]
        if st[rows][:, maxt:].any():
            raise RuntimeError("decode B=256: tiles past the sequences marked visited")
        ov = flip_override(np, stg, r["state"], r["gamma"], tau)
        ro = r["out"] if ov is None else oracle.decode(data["q"][pick], kc, vc, L[pick], tau=tau, num_splits=P,
                                                       override=ov, threads=threads)["out"]
        G = w.Hq // w.Hkv
        res["parity"] = parity_fields(np, got[pick].reshape(len(pick) * w.Hkv, G, w.d), ro, stg.ravel(),
                                      r["state"].ravel(), r["gamma"].ravel(), tau)
        res["parity"]["sequences"] = [int(x) for x in pick]
    return res


def leg_prefill_16k(ssm, torch, np, steps, dev, threads, cpu=True, n_units=64):
    """prefill_s16k (batch 1, 64/8 heads, d 128, S 16384 causal) at tau = -inf, -ln 100 and -ln 1000: GPU time,
    sparsity, dense-equivalent and executed TFLOP/s and the MFMA roofline fraction at each tau, beside the
    oracle's time on n_units sampled units of the same input and the parity of the timed output there."""
    import synth
    w = synth.PREFILL_16K
    data = synth.gen_prefill(w, threads=threads)
    q, k, v = (ssm.bf16_from_bits(data[x], dev) for x in ("q", "k", "v"))
    out = torch.empty_like(q)
    units_n, nkt = ssm.prefill_stats_shape(w.B, w.S, w.Hq, w.tile_q)
    state = torch.zeros(units_n, nkt, dtype=torch.uint8, device=dev)
    units, heads, qts = prefill_sample_units(np, w, n_units)
    rows = []
    for tau in w.taus:
        cnt = torch.zeros(4, dtype=torch.int64, device=dev)
        run = lambda st: ssm.ssm_prefill(q, k, v, causal=True, tau=tau, out=out, skip_stats=st, tile_q=w.tile_q)
        ms = _timed(torch, np, lambda: run(ssm.SkipStats(counters=cnt)), steps)
        got = gather_prefill_rows(torch, np, out, w, heads, qts)
        c = cnt.cpu().numpy() / (steps + 1)
        state.zero_()
        run(ssm.SkipStats(tile_state=state))
        st = state.cpu().numpy()
        if not (int((st != 0).sum()) == c[0] and int((st == 2).sum()) == c[1]):
            raise RuntimeError("prefill 16K: tile states disagree with the timed counters")
        visited, skipped = float(c[0]), float(c[1])
        dense, executed = prefill_flops(w, visited, visited - skipped)
        t = ms / 1e3
        row = {"tau": None if math.isinf(tau) else round(tau, 4), "ms": round(ms, 4),
               "sparsity": round(skipped / visited, 4), "dense_tflops": round(dense / t / 1e12, 2),
               "executed_tflops": round(executed / t / 1e12, 2),
               "mfma_frac": round(executed / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        if cpu:
            base, par = cpu_baseline_prefill(np, w, data, tau, threads, units, got, st[units])
            row["oracle_dense_tflops"] = round(base["value"], 5)
            row["oracle_seconds"] = base["seconds"]
            row["gpu_over_oracle"] = round(row["dense_tflops"] / base["value"], 1)
            row["parity"] = par
        rows.append(row)
    del q, k, v, out, state
    return {"workload": f"{w.name} (causal, GEN-A rel_frac {w.rel_frac})", "oracle_units": n_units,
            "oracle_threads": threads, "taus": rows}


PARITY_MAX_ABS, PARITY_REL_L2, PARITY_BAND = 1e-2, 3e-3, 1e-3
PARITY_BF16_OUT, PARITY_ACC_ABS = 2.0 ** -8, 2e-3  # where |o| > 2.05: bf16 output rounding + accumulated error


def host_info(threads):
    """The host the CPU legs ran on: logical CPUs (nproc), those this process may use, the CPU model, and the
    threads the oracle was given."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model, "threads": threads,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def oracle_threads():
    """Threads for the oracle: the CPU share this process is given (OMP_NUM_THREADS where the launcher sets
    it, else every CPU the process may run on)."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(usable, share) if share > 0 else usable)


def parity_fields(np, got, ref_out, st_gpu, st_ref, gamma_ref, tau):
    """The timed launch against the oracle on the same units: output max-abs and relative L2 error, and the skip
    decisions compared on every visited tile whose oracle unit gap lies at least PARITY_BAND from tau (closer
    tiles may go either way; ref_out must then be the oracle re-run with the GPU's decisions there)."""
    got = np.asarray(got, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    diff = got - ref_out
    den = float(np.linalg.norm(ref_out.ravel()))
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff.ravel()) / den) if den > 0 else 0.0
    within = bool((np.abs(diff) <= np.maximum(PARITY_MAX_ABS, PARITY_BF16_OUT * np.abs(ref_out) + PARITY_ACC_ABS)).all())
    vis = st_ref > 0
    if math.isinf(tau):
        amb = np.zeros(st_ref.shape, bool)
    else:
        with np.errstate(invalid="ignore"):
            amb = vis & (np.abs(gamma_ref - tau) < PARITY_BAND)
    off = vis & ~amb
    agree = int((off & (st_gpu == st_ref)).sum())
    return {"max_abs": float("%.4g" % max_abs), "rel_l2": float("%.4g" % rel),
            "mask_tiles_off_band": int(off.sum()), "mask_agree_off_band": agree,
            "ambiguous_tiles": int(amb.sum()), "ambiguous_flips": int((amb & (st_gpu != st_ref)).sum()),
            "unvisited_agree": bool(((st_gpu == 0) == (st_ref == 0)).all()),
            "pass": bool(within and rel <= PARITY_REL_L2 and agree == int(off.sum()))}


def flip_override(np, st_gpu, st_ref, gamma_ref, tau):
    """Oracle mask override that takes the GPU's decision on ambiguous tiles where the two differ (else None)."""
    if math.isinf(tau):
        return None
    with np.errstate(invalid="ignore"):
        flips = (st_ref > 0) & (np.abs(gamma_ref - tau) < PARITY_BAND) & (st_gpu != st_ref)
    if not flips.any():
        return None
    return np.where(flips, np.where(st_gpu == 2, 1, 0), -1).astype(np.int8)


def prefill_sample_units(np, w, n_units):
    """n_units prefill units (q-tiles spread evenly over the sequence, heads rotating), as unit ids and (h, qt)."""
    nqt = -(-w.S // w.tile_q)
    qts = np.linspace(0, nqt - 1, n_units).round().astype(np.int64)
    heads = (np.arange(n_units) * 11) % w.Hq
    return heads * nqt + qts, heads, qts


def gather_prefill_rows(torch, np, out, w, heads, qts):
    """[n, tile_q, d] float64 rows of a [1, S, Hq, d] output for units (h, qt) (rows past S are 0)."""
    rows = []
    for h, qt in zip(heads.tolist(), qts.tolist()):
        r0, r1 = qt * w.tile_q, min(w.S, (qt + 1) * w.tile_q)
        x = torch.zeros(w.tile_q, w.d, dtype=torch.float32, device=out.device)
        x[:r1 - r0] = out[0, r0:r1, h].float()
        rows.append(x)
    return torch.stack(rows).cpu().numpy().astype(np.float64)


def cpu_baseline_prefill(np, w, data, tau, threads, units, got, st_gpu):
    """Time the fp64 oracle on a bounded sample of prefill units (dense-equivalent TFLOP/s on the host) and
    compare it with the timed launch's outputs and decisions on those units."""
    import oracle
    nqt = -(-w.S // w.tile_q)
    qts = units % nqt
    rows_keys = 0.0
    for qt in qts:  # dense-equivalent work of these units: sum over rows of visible keys
        r0, r1 = qt * w.tile_q, min(w.S, (qt + 1) * w.tile_q)
        rows_keys += (r1 * (r1 + 1) - r0 * (r0 + 1)) / 2 if w.causal else (r1 - r0) * w.S
    flops = 4.0 * w.d * rows_keys
    t0 = time.perf_counter()
    ref = oracle.prefill(data["q"], data["k"], data["v"], causal=w.causal, tau=tau, tile_q=w.tile_q,
                         tile_k=w.tile_k, units=units, threads=threads)
    dt = time.perf_counter() - t0
    ov = flip_override(np, st_gpu, ref["state"], ref["gamma"], tau)
    ref_out = ref["out"] if ov is None else oracle.prefill(
        data["q"], data["k"], data["v"], causal=w.causal, tau=tau, tile_q=w.tile_q, tile_k=w.tile_k, units=units,
        override=ov, threads=threads)["out"]
    return ({"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
             "sample": f"{len(units)} prefill units (q-tiles spread evenly over 0..{nqt - 1}, heads rotating) of "
                       f"{w.name}, {flops / 1e9:.1f} dense-equiv GFLOP in {dt:.1f} s",
             "seconds": round(dt, 3)},
            parity_fields(np, got, ref_out, st_gpu, ref["state"], ref["gamma"], tau))


def paged_to_contiguous(np, w, data, b):
    """Sequences b of a paged gen_decode() input as contiguous [len(b), Hkv, smax, d] caches (layout only)."""
    lens = data["kv_lens"]
    nt = -(-lens[b] // 64)
    smax = int(max(nt.max(), 1)) * 64
    kc = np.zeros((len(b), w.Hkv, smax, w.d), np.uint16)
    vc = np.zeros_like(kc)
    for i, bb in enumerate(b):
        pages = data["page_table"][bb, :nt[i]]
        kc[i, :, :nt[i] * 64] = data["k_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
        vc[i, :, :nt[i] * 64] = data["v_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
    return kc, vc


def cpu_baseline_decode(np, w, data, tau, threads, num_splits, got, st_gpu, sink_seed=False, chunk=4):
    """The oracle on every sequence of a decode workload (KV GB/s on the host, timed per chunk of sequences;
    paged inputs are gathered into contiguous caches outside the timed region), compared with the timed
    launch's outputs got [B, Hq, d] and tile states st_gpu [B*Hkv, max_tiles]."""
    import oracle
    lens = data["kv_lens"]
    G = w.Hq // w.Hkv
    dt = kv = 0.0
    outs, refs, sg, sr, gr = [], [], [], [], []
    for c0 in range(0, w.B, chunk):
        b = np.arange(c0, min(w.B, c0 + chunk))
        if "k_pool" in data:
            kc, vc = paged_to_contiguous(np, w, data, b)
        else:
            kc, vc = data["k_cache"][b], data["v_cache"][b]
        t0 = time.perf_counter()
        r = oracle.decode(data["q"][b], kc, vc, lens[b], tau=tau, num_splits=num_splits, sink_seed=sink_seed,
                          threads=threads)
        dt += time.perf_counter() - t0
        kept = r["state"] == 1
        kv += float(lens[b].astype(np.int64).sum()) * w.Hkv * w.d * 2 + float(kept.sum()) * 64 * w.d * 2
        maxt = r["state"].shape[1]
        stg = st_gpu[c0 * w.Hkv:(c0 + len(b)) * w.Hkv]
        if stg[:, maxt:].any():
            raise RuntimeError("decode: tiles past the sequences marked visited")
        stg = stg[:, :maxt]
        ov = flip_override(np, stg, r["state"], r["gamma"], tau)
        ro = r["out"] if ov is None else oracle.decode(data["q"][b], kc, vc, lens[b], tau=tau,
                                                       num_splits=num_splits, sink_seed=sink_seed, override=ov,
                                                       threads=threads)["out"]
        outs.append(got[b].reshape(len(b) * w.Hkv, G, w.d))
        refs.append(ro)
        sg.append(stg.ravel())
        sr.append(r["state"].ravel())
        gr.append(r["gamma"].ravel())
    par = parity_fields(np, np.concatenate(outs), np.concatenate(refs), np.concatenate(sg), np.concatenate(sr),
                        np.concatenate(gr), tau)
    return ({"value": kv / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
             "sample": f"all {w.B} sequences of {w.name} (every KV group), {chunk} sequences per oracle call",
             "seconds": round(dt, 3)}, par)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "decode"], default=None)
    ap.add_argument("--main-only", action="store_true",
                    help="time only the step (prefill + decode); skip the chunked-prefill, sink-seeded and fp8 legs "
                         "(used for the profiler runs, so each kernel name is one configuration)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy a 1 GiB device buffer (normalises FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output directories and exit")
    ap.add_argument("--traffic-command", default="", help="command line recorded with --summarize-traffic")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="run the standalone MFMA-rate program (zero vs random bf16 operands), print its JSON and exit")
    ap.add_argument("--mfma-power", type=float, default=None, metavar="SECONDS",
                    help="run the MFMA-rate program in its sustained form (idle / zero / idle / random operands, "
                         "SECONDS each) beside a board power and clock sampler, print the JSON and exit")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="run the standalone HBM streaming-read program (the decode's load shapes), print its JSON "
                         "and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.traffic_command)
        return
    if args.mfma_power is not None:
        mfma_power(args.mfma_power)
        return
    if args.mfma_ceiling or args.read_ceiling:
        exe = os.path.join(CEILING_DIR, "mfma_ceiling" if args.mfma_ceiling else "read_ceiling")
        if not os.path.exists(exe):
            sys.exit(f"{exe} is missing: build it with `python -c 'import bench; bench.build_ceiling_programs()'` "
                     "(__graft_entry__.build() does)")
        sys.exit(subprocess.run([exe]).returncode)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each GPU would run the same "
              "kernels on its shard of KV groups or sequence). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_flash_amd as ssm
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    threads = synth.default_threads()   # input generation
    cpu_threads = oracle_threads()      # the oracle legs: this process's CPU share
    run_prefill = args.only in (None, "prefill")
    run_decode = args.only in (None, "decode")

    pw = synth.PREFILL_128K
    dw = synth.DECODE_128K
    tau_p = pw.taus[0]
    tau_d = dw.taus[2]  # oracle-calibrated for ~50% skipped tiles

    if run_prefill:
        log(f"generating {pw.name} (threads={threads})")
        pdata = synth.gen_prefill(pw, threads=threads)
        q, k, v = (ssm.bf16_from_bits(pdata[x], dev) for x in ("q", "k", "v"))
        pout = torch.empty_like(q)
        pcnt = torch.zeros(4, dtype=torch.int64, device=dev)
        pstats = ssm.SkipStats(counters=pcnt)
    if run_decode:
        log(f"generating {dw.name}")
        ddata = synth.gen_decode(dw, threads=threads)
        dq = ssm.bf16_from_bits(ddata["q"], dev)
        kp, vp = ssm.bf16_from_bits(ddata["k_pool"], dev), ssm.bf16_from_bits(ddata["v_pool"], dev)
        pt = torch.from_numpy(ddata["page_table"]).to(dev)
        lens = torch.from_numpy(ddata["kv_lens"]).to(dev)
        dout = torch.empty_like(dq)
        ws = ssm.decode_workspace(dw.B, dw.Hq, dw.d, dw.num_splits, dev)
        dstate = torch.zeros(dw.B * dw.Hkv, pt.shape[1], dtype=torch.uint8, device=dev)
        dcnt = torch.zeros(4, dtype=torch.int64, device=dev)
        # timed calls report the skip counters; the per-tile states (for the exact byte count) come from one
        # more call on the same inputs after the timed region (the skip decisions are deterministic)
        dstats = ssm.SkipStats(counters=dcnt)
    torch.cuda.synchronize()

    def step(i, ev):
        ev[i][0].record()
        if run_prefill:
            ssm.ssm_prefill(q, k, v, causal=True, tau=tau_p, out=pout, skip_stats=pstats, tile_q=pw.tile_q)
        ev[i][1].record()
        if run_decode:
            ssm.ssm_decode(dq, kp, vp, lens, tau=tau_d, out=dout, page_table=pt, num_splits=dw.num_splits,
                           workspace=ws, skip_stats=dstats)
        ev[i][2].record()

    mk = lambda n: [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
    log(f"warmup {args.warmup}")
    wev = mk(max(args.warmup, 1))
    for i in range(args.warmup):
        step(i, wev)
    torch.cuda.synchronize()
    if run_prefill:
        pcnt.zero_()
    if run_decode:
        dcnt.zero_()
    ev = mk(args.steps)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    with BoardSampler(gpu_sysfs_dir(torch)) as board:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, ev)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    p_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    d_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    step_ms = wall * 1e3 / args.steps
    log(f"prefill ms {['%.2f' % x for x in p_ms]}  decode ms {['%.3f' % x for x in d_ms]}  wall/step {step_ms:.2f}")
    # the timed launches' outputs (before the later legs reuse the output buffers), for the parity check of the
    # CPU-baseline legs; and the prefill's per-tile decisions from one more, untimed call on the same inputs
    if run_prefill:
        p_units, p_heads, p_qts = prefill_sample_units(np, pw, 256)
        p_got = gather_prefill_rows(torch, np, pout, pw, p_heads, p_qts)
        n_units, nkt = ssm.prefill_stats_shape(pw.B, pw.S, pw.Hq, pw.tile_q)
        pstate = torch.zeros(n_units, nkt, dtype=torch.uint8, device=dev)
        ssm.ssm_prefill(q, k, v, causal=True, tau=tau_p, out=torch.empty_like(pout),
                        skip_stats=ssm.SkipStats(tile_state=pstate), tile_q=pw.tile_q)
        pst_all = pstate.cpu().numpy()
        c_t = pcnt.cpu().numpy() / args.steps
        if not (int((pst_all != 0).sum()) == c_t[0] and int((pst_all == 2).sum()) == c_t[1]):
            raise RuntimeError("prefill tile states disagree with the timed counters")
        p_st = pst_all[p_units]
        del pstate, pst_all
    if run_decode:
        d_got = dout.float().cpu().numpy()

    res = {"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic: seeded GEN-A prefill / GEN-B decode inputs with Llama-3.3-70B "
                                    "attention shapes (no weights, no dataset)"}
    cfg = {"workload": ("prefill_s128k+decode_b32_kv128k_paged" if args.only is None else
                        (pw.name if run_prefill else dw.name))}
    if run_prefill:
        c = pcnt.cpu().numpy() / args.steps
        visited, skipped = float(c[0]), float(c[1])
        kept = visited - skipped
        dense, executed = prefill_flops(pw, visited, kept)
        t = float(np.mean(p_ms)) / 1e3
        res["value"] = round(dense / t / 1e12, 2)
        res["prefill_ms"] = round(t * 1e3, 3)
        res["prefill_ms_median_min"] = [round(float(np.median(p_ms)), 3), round(float(np.min(p_ms)), 3)]
        res["prefill_executed_tflops"] = round(executed / t / 1e12, 2)
        res["prefill_sparsity"] = round(skipped / visited, 4)
        cfg["prefill"] = {"batch": pw.B, "seq_len": pw.S, "q_heads": pw.Hq, "kv_heads": pw.Hkv, "head_dim": pw.d,
                          "causal": True, "tau": round(tau_p, 4), "tile_q": pw.tile_q, "tile_k": pw.tile_k,
                          "relevant_tile_frac": pw.rel_frac, "seed": pw.seed}
        res["roofline"] = {"bound": "mfma", "achieved": round(executed / t / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(executed / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                           "traffic": recorded_traffic("prefill"), "kernel": PREFILL_KERNEL,
                           "per_launch_flop": executed, "note": "executed = 2*128*64*128 FLOP per visited "
                           "tile (QK^T) + the same per kept tile (PV)"}
        ceiling = recorded_mfma_ceiling()
        if ceiling:
            # the rate this GPU sustains on random bf16 operands (power-limited clock), recorded by
            # `bench.py --mfma-ceiling`; reported beside the published peak, which stays the roofline's peak
            res["roofline"]["measured_ceiling"] = {
                "random_operands_tflops": ceiling, "frac": round(executed / t / 1e12 / ceiling, 4),
                "source": "profiles/mfma_ceiling.json"}
    if run_prefill and not args.main_only:
        res["prefill_chunked_paged"] = time_chunked_prefill(ssm, torch, np, pw, pdata, tau_p, args.steps, dev)
        res["prefill_fp8_qk"] = time_fp8qk_prefill(ssm, torch, np, pw, q, k, v, pout, tau_p, res["prefill_ms"],
                                                   args.steps, dev)
        res["prefill_vs_dense"] = time_prefill_vs_dense(ssm, torch, np, pw, q, k, v, pout, res["prefill_ms"],
                                                        res["prefill_sparsity"], args.steps, dev)
        res["prefill_rowmax_pot"] = time_pot_prefill(ssm, torch, np, pw, q, k, v, pout, tau_p, res["prefill_ms"],
                                                     res["prefill_vs_dense"]["dense_ms"], args.steps, dev)
    if run_decode:
        c = dcnt.cpu().numpy() / args.steps
        ssm.ssm_decode(dq, kp, vp, lens, tau=tau_d, out=dout, page_table=pt, num_splits=dw.num_splits,
                       workspace=ws, skip_stats=ssm.SkipStats(tile_state=dstate))
        state = dstate.cpu().numpy()
        dstate_timed = state
        if not (int((state != 0).sum()) == c[0] and int((state == 2).sum()) == c[1]):
            raise RuntimeError(f"decode tile states {int((state != 0).sum())}/{int((state == 2).sum())} disagree "
                               f"with the timed counters {c[0]}/{c[1]}")
        lens_np = ddata["kv_lens"]
        kb, vk, va, small = decode_bytes(dw, lens_np, state, dw.num_splits)
        t = float(np.mean(d_ms)) / 1e3
        res["decode_ms"] = round(t * 1e3, 4)
        res["decode_ms_median_min"] = [round(float(np.median(d_ms)), 4), round(float(np.min(d_ms)), 4)]
        res["decode_kv_gbps"] = round((kb + vk) / t / 1e9, 1)
        res["decode_total_gbps"] = round((kb + vk + small) / t / 1e9, 1)
        res["decode_dense_equiv_kv_gbps"] = round((kb + va) / t / 1e9, 1)
        res["decode_sparsity"] = round(float(c[1]) / float(c[0]), 4)
        cfg["decode"] = {"batch": dw.B, "q_heads": dw.Hq, "kv_heads": dw.Hkv, "head_dim": dw.d, "paged": True,
                         "page": 64, "kv_len_range": [dw.kv_len_lo, dw.kv_len_hi],
                         "kv_len_mean": float(lens_np.mean()), "num_splits": dw.num_splits, "tau": tau_d,
                         "seed": dw.seed}
        res["roofline_decode"] = {"bound": "hbm", "achieved": round((kb + vk + small) / t / 1e9, 1),
                                  "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                  "frac": round((kb + vk + small) / t / 1e9 / HBM_PEAK_GBPS, 4),
                                  "traffic": recorded_traffic("decode"),
                                  "kernel": f"{DECODE_ORDER_KERNEL} + {DECODE_SPLIT_KERNEL} + {DECODE_COMBINE_KERNEL}",
                                  "per_launch_bytes": kb + vk + small}
        read_ceiling = recorded_read_ceiling()
        if read_ceiling:
            # the best rate at which this GPU streams reads in the decode's load shapes (no compute), recorded by
            # `bench.py --read-ceiling`; reported beside the published peak, which stays the roofline's peak
            res["roofline_decode"]["measured_ceiling"] = {
                "read_gbps": read_ceiling, "frac": round((kb + vk + small) / t / 1e9 / read_ceiling, 4),
                "source": "profiles/read_ceiling.json"}
        if "value" not in res:
            res["value"] = res["decode_kv_gbps"]
            res["unit"] = "GB/s"
    if run_decode and not args.main_only:
        res["decode_sink_seeded"] = time_sink_seeded_decode(ssm, torch, np, dw, ddata, dq, kp, vp, pt, lens, dout, ws,
                                                            dstate, tau_d, args.steps, dev)
        res["decode_sink_seeded"]["speedup_vs_split_local"] = round(res["decode_ms"] / res["decode_sink_seeded"]["ms"], 3)
        res["decode_fp8_kv"] = time_fp8_decode(ssm, torch, np, dw, ddata, dq, kp, vp, pt, lens, dout, ws, dstate, tau_d,
                                               args.steps, dev)
        res["decode_fp8_kv"]["speedup_vs_bf16"] = round(res["decode_ms"] / res["decode_fp8_kv"]["ms"], 3)
        res["decode_tau_sweep"] = time_decode_tau_sweep(ssm, torch, np, dw, dq, kp, vp, pt, lens, dout, ws, args.steps,
                                                        dev)
        read_ceiling = recorded_read_ceiling()
        if read_ceiling:
            for leg in ("decode_sink_seeded", "decode_fp8_kv"):
                res[leg]["read_ceiling_frac"] = round(res[leg]["total_gbps"] / read_ceiling, 4)
        log("decode 32K legs")
        res["decode_32k"] = leg_decode_32k(ssm, torch, np, args.steps, dev, cpu_threads, cpu=not args.no_cpu_baseline)
        res["decode_b256"] = leg_decode_b256(ssm, torch, np, args.steps, dev, cpu_threads,
                                             cpu=not args.no_cpu_baseline)
    if run_prefill and not args.main_only:
        log("prefill 16K legs")
        res["prefill_16k"] = leg_prefill_16k(ssm, torch, np, args.steps, dev, cpu_threads,
                                             cpu=not args.no_cpu_baseline)
    res["config"] = cfg
    bp = board.summary()
    if bp is not None:
        # almost all of a step's time is the prefill (the decode is under 1% of it)
        bp["what"] = "board power (hwmon power1_input) and graphics clock (pp_dpm_sclk) sampled every 10 ms " \
                     "over the timed steps"
        res["board_power"] = bp
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        host = host_info(cpu_threads)
        if run_prefill:
            log("cpu baseline: oracle on sampled prefill units")
            base, par = cpu_baseline_prefill(np, pw, pdata, tau_p, cpu_threads, p_units, p_got, p_st)
            base["host"] = host
            res["cpu_baseline"] = base
            res["parity"] = {"prefill": par}
        if run_decode:
            log("cpu baseline: oracle on every decode sequence")
            base, par = cpu_baseline_decode(np, dw, ddata, tau_d, cpu_threads, dw.num_splits, d_got,
                                            dstate_timed)
            base["host"] = host
            res["cpu_baseline" if not run_prefill else "cpu_baseline_decode"] = base
            res.setdefault("parity", {})["decode"] = par
        res["parity"]["bar"] = {"max_abs": PARITY_MAX_ABS, "max_abs_large_o": "2^-8 |o| + 2e-3 where larger",
                                "rel_l2": PARITY_REL_L2, "mask_band": PARITY_BAND,
                                "what": "the timed launches' outputs and skip decisions against the fp64 oracle "
                                        "on the cpu_baseline samples"}
    print(json.dumps(res, allow_nan=False), flush=True)


if __name__ == "__main__":
    main()
