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
KERNEL_SOURCES = {"prefill": ["prefill.hip", "ssm_device.h", "ssm_launch.h", "ssm_api.cpp"],
                  "decode": ["decode.hip", "ssm_device.h", "ssm_launch.h", "ssm_api.cpp"]}
COPY_PROBE_BYTES = 1 << 30
# the step's kernels as the profiler names them (d = 128, tile_q = 128, plain prefill, bf16 cache)
PREFILL_KERNEL = "prefill_kernel<128, 128, false, 0>"
DECODE_SPLIT_KERNEL = "decode_split_kernel<128, 2>"
DECODE_COMBINE_KERNEL = "decode_combine_kernel<128>"


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
    each scaled by what the same counter reads for a device copy of COPY_PROBE_BYTES."""
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

    def launch_bytes(pred):
        tot = 0.0
        for n in fetch:
            if pred(n):
                tot += (sum(fetch[n]) / len(fetch[n]) * f_fac + sum(write[n]) / len(write[n]) * w_fac) * 1024
        return tot

    rec = {"copy_kernel": copy, "fetch_factor": f_fac, "write_factor": w_fac, "command": command,
           "prefill": {"kernels": PREFILL_KERNEL,
                       "bytes_per_launch": launch_bytes(lambda n: PREFILL_KERNEL in n),
                       "source_sha256": sources_sha("prefill")},
           "decode": {"kernels": "decode_split_kernel + decode_combine_kernel",
                      "bytes_per_launch": launch_bytes(lambda n: DECODE_SPLIT_KERNEL in n or DECODE_COMBINE_KERNEL in n),
                      "source_sha256": sources_sha("decode")}}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    lines = ["# HBM traffic from FETCH_SIZE / WRITE_SIZE (rocprofv3 --pmc), prefill_s128k and decode_b32_kv128k_paged",
             "", "Commands (MI355X, one GPU; $REPO is the repository root):", "", "```", command, "```", "",
             f"Normalisation: a device copy of {COPY_PROBE_BYTES} bytes (`{copy}`) reads FETCH_SIZE = "
             f"{max(fetch[copy]):.0f} KiB and WRITE_SIZE = {max(write[copy]):.0f} KiB; factors "
             f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write) scale each kernel's counters to bytes.", "",
             "| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | HBM bytes/dispatch (scaled) |",
             "|---|---|---|---|---|"]
    for n in sorted(fetch):
        fk = sum(fetch[n]) / len(fetch[n])
        wk = sum(write.get(n, [0])) / max(len(write.get(n, [0])), 1)
        lines.append(f"| `{n[:90]}` | {len(fetch[n])} | {fk:.0f} | {wk:.0f} | {(fk * f_fac + wk * w_fac) * 1024:.4g} |")
    lines += ["", f"Per launch: prefill {rec['prefill']['bytes_per_launch']:.4g} B; decode (split + combine) "
              f"{rec['decode']['bytes_per_launch']:.4g} B."]
    with open(os.path.join(ROOT, "profiles", "hbm_traffic__prefill_s128k__decode_b32_kv128k_paged.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def _timed(torch, np, fn, steps):
    """mean ms of `steps` calls of fn between HIP events on the current stream, after one untimed call"""
    fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        fn()
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))


def time_prefill_vs_dense(ssm, torch, np, w, q, k, v, out, skip_ms, sparsity, steps, dev):
    """The same prefill launch at tau = -inf (no tile skipped: the dense kernel) against the timed skip launch:
    the speedup skipping buys on this input, the quantity the Skip Softmax pages report (as context: 1.4x for
    prefill of Llama 3.3 70B at 128K on GB200)."""
    cnt = torch.zeros(4, dtype=torch.int64, device=dev)
    ms = _timed(torch, np, lambda: ssm.ssm_prefill(q, k, v, causal=True, tau=-math.inf, out=out,
                                                   skip_stats=ssm.SkipStats(counters=cnt), tile_q=w.tile_q), steps)
    c = cnt.cpu().numpy()
    if int(c[1]) != 0:
        raise RuntimeError("tau = -inf skipped tiles")
    return {"dense_ms": round(ms, 3), "skip_ms": skip_ms, "skip_sparsity": sparsity,
            "speedup_vs_dense": round(ms / skip_ms, 3), "pages_prefill_speedup": 1.4}


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
           "q_scale": qs, "k_scale": ks, "speedup_vs_bf16": round(bf16_ms / ms, 3)}
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


def cpu_baseline_prefill(w, data, threads, n_units=256):
    """Time the fp64 oracle on a bounded sample of prefill units; dense-equivalent TFLOP/s."""
    import numpy as np
    import oracle
    nqt = -(-w.S // w.tile_q)
    qts = np.linspace(0, nqt - 1, n_units).round().astype(np.int64)
    heads = (np.arange(n_units) * 11) % w.Hq
    units = heads * nqt + qts
    rows_keys = 0.0
    for qt in qts:  # dense-equivalent work of these units: sum over rows of visible keys
        r0, r1 = qt * w.tile_q, min(w.S, (qt + 1) * w.tile_q)
        rows_keys += sum(i + 1 for i in range(r0, r1))
    flops = 4.0 * w.d * rows_keys
    t0 = time.perf_counter()
    oracle.prefill(data["q"], data["k"], data["v"], causal=True, tau=w.taus[0], tile_q=w.tile_q, tile_k=w.tile_k,
                   units=units, threads=threads)
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_units} prefill units (q-tiles spread evenly over 0..{nqt - 1}, heads rotating) of the "
                      f"128K prefill, {flops / 1e9:.1f} dense-equiv GFLOP in {dt:.1f} s",
            "seconds": dt}


def cpu_baseline_decode(w, data, tau, threads, chunk=4):
    """The oracle on every sequence of the decode workload (timed per chunk of sequences, gathered from the
    page pool into contiguous caches outside the timed region)."""
    import numpy as np
    import oracle
    lens = data["kv_lens"]
    dt = 0.0
    kv = 0.0
    for c0 in range(0, w.B, chunk):
        b = np.arange(c0, min(w.B, c0 + chunk))
        nt = -(-lens[b] // 64)
        smax = int(nt.max()) * 64
        kc = np.zeros((len(b), w.Hkv, smax, w.d), np.uint16)
        vc = np.zeros_like(kc)
        for i, bb in enumerate(b):
            pages = data["page_table"][bb, :nt[i]]
            kc[i, :, :nt[i] * 64] = data["k_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
            vc[i, :, :nt[i] * 64] = data["v_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
        t0 = time.perf_counter()
        r = oracle.decode(data["q"][b], kc, vc, lens[b], tau=tau, num_splits=w.num_splits, threads=threads)
        dt += time.perf_counter() - t0
        kept = r["state"] == 1
        kv += float(lens[b].astype(np.int64).sum()) * w.Hkv * w.d * 2 + float(kept.sum()) * 64 * w.d * 2
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"all {w.B} decode sequences (every KV group), {chunk} sequences per oracle call",
            "seconds": dt}


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
    ap.add_argument("--read-ceiling", action="store_true",
                    help="run the standalone HBM streaming-read program (the decode's load shapes), print its JSON "
                         "and exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.traffic_command)
        return
    if args.mfma_ceiling or args.read_ceiling:
        exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_flash_amd",
                           "mfma_ceiling" if args.mfma_ceiling else "read_ceiling")
        if not os.path.exists(exe):
            sys.exit(f"{exe} is missing: build with `python -m long_context_flash_amd.build`")
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
    threads = synth.default_threads()
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
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    p_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    d_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    step_ms = wall * 1e3 / args.steps
    log(f"prefill ms {['%.2f' % x for x in p_ms]}  decode ms {['%.3f' % x for x in d_ms]}  wall/step {step_ms:.2f}")

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
    if run_decode:
        c = dcnt.cpu().numpy() / args.steps
        ssm.ssm_decode(dq, kp, vp, lens, tau=tau_d, out=dout, page_table=pt, num_splits=dw.num_splits,
                       workspace=ws, skip_stats=ssm.SkipStats(tile_state=dstate))
        state = dstate.cpu().numpy()
        if not (int((state != 0).sum()) == c[0] and int((state == 2).sum()) == c[1]):
            raise RuntimeError(f"decode tile states {int((state != 0).sum())}/{int((state == 2).sum())} disagree "
                               f"with the timed counters {c[0]}/{c[1]}")
        lens_np = ddata["kv_lens"]
        kb, vk, va, small = decode_bytes(dw, lens_np, state, dw.num_splits)
        t = float(np.mean(d_ms)) / 1e3
        res["decode_ms"] = round(t * 1e3, 4)
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
                                  "kernel": f"{DECODE_SPLIT_KERNEL} + {DECODE_COMBINE_KERNEL}",
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
    res["config"] = cfg
    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        if run_prefill:
            log("cpu baseline: oracle on sampled prefill units")
            res["cpu_baseline"] = cpu_baseline_prefill(pw, pdata, threads)
            if run_decode:
                res["cpu_baseline_decode"] = cpu_baseline_decode(dw, ddata, tau_d, threads)
        elif run_decode:
            res["cpu_baseline"] = cpu_baseline_decode(dw, ddata, tau_d, threads)
    print(json.dumps(res, allow_nan=False), flush=True)


if __name__ == "__main__":
    main()
