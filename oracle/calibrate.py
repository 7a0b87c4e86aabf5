"""Calibrate the synthetic workloads' sparsity knobs with the oracle (test infrastructure).

    python -m oracle.calibrate [--threads N] [--out tests/golden/calibration.json]

* Prefill 128K: the relevant-tile fraction rho for about 50% skipped tiles at tau = -ln 1000.
* Decode 128K: the taus giving about 0 / 30 / 50 / 70% skipped tiles with 16 split-local scans.

Both use the oracle's closed form on sampled units.  The unit gap Gamma of a tile does not
depend on tau (the prefix maximum covers every visited tile), so one oracle pass per input
yields the skip fraction at every tau: a tile is skipped iff Gamma < tau.
The chosen values are written to a JSON record; the workload definitions in synth/ carry them.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def sampled_prefill_units(w, n, seed):
    rng = np.random.default_rng(seed)
    nqt = -(-w.S // w.tile_q)
    heads = rng.integers(0, w.Hq, n)
    qts = rng.integers(0, nqt, n)
    return np.unique(heads * nqt + qts)


def prefill_sparsity(w, units, tau, threads):
    data = synth.gen_prefill(w, threads=threads)
    r = oracle.prefill(data["q"], data["k"], data["v"], causal=w.causal, tau=-math.inf, tile_q=w.tile_q,
                       tile_k=w.tile_k, units=units, threads=threads)
    vis = r["state"] > 0
    return float((r["gamma"][vis] < tau).sum() / vis.sum())


def calibrate_prefill(threads, n_units=48, target=0.5, tau=-math.log(1000.0), iters=6):
    w0 = synth.PREFILL_128K
    units = sampled_prefill_units(w0, n_units, seed=4004)
    lo, hi = 0.2, 0.8   # sparsity falls as rho grows
    history = []
    for _ in range(iters):
        rho = 0.5 * (lo + hi)
        t0 = time.time()
        sp = prefill_sparsity(synth.replace(w0, rel_frac=rho), units, tau, threads)
        history.append({"rel_frac": rho, "sparsity": sp})
        print(f"prefill rho={rho:.4f} sparsity={sp:.4f} ({time.time() - t0:.1f}s)", flush=True)
        if sp > target:
            lo = rho
        else:
            hi = rho
    # the largest rho that still reaches the target sparsity
    best = max((h for h in history if h["sparsity"] >= target), key=lambda h: h["rel_frac"],
               default=min(history, key=lambda h: abs(h["sparsity"] - target)))
    return {"workload": w0.name, "tau": tau, "target_sparsity": target, "units_sampled": int(len(units)),
            "chosen_rel_frac": round(best["rel_frac"], 4), "sparsity_at_chosen": best["sparsity"], "history": history}


def calibrate_decode(threads, batches=tuple(range(32)), targets=(0.3, 0.5, 0.7)):
    w = synth.DECODE_128K
    data = synth.gen_decode(w, contiguous=False, paged=True, threads=threads)
    lens = data["kv_lens"]
    b = np.array(batches)
    nt = -(-lens[b] // 64)
    smax = int(nt.max()) * 64
    kc = np.zeros((len(b), w.Hkv, smax, w.d), np.uint16)
    vc = np.zeros_like(kc)
    for i, bb in enumerate(b):
        pages = data["page_table"][bb, :nt[i]]
        kc[i, :, :nt[i] * 64] = data["k_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
        vc[i, :, :nt[i] * 64] = data["v_pool"][pages].transpose(1, 0, 2, 3).reshape(w.Hkv, -1, w.d)
    t0 = time.time()
    r = oracle.decode(data["q"][b], kc, vc, lens[b], tau=-math.inf, num_splits=w.num_splits, threads=threads)
    g = r["gamma"][r["state"] > 0]
    print(f"decode oracle pass {time.time() - t0:.1f}s over {len(g)} tiles", flush=True)
    taus = {}
    for tgt in targets:
        tau = float(np.quantile(g, tgt))  # fraction of tiles with Gamma < tau
        taus[str(tgt)] = round(tau, 3)
        print(f"decode target {tgt}: tau={tau:.4f} sparsity={(g < round(tau, 3)).mean():.4f}", flush=True)
    return {"workload": w.name, "num_splits": w.num_splits, "batches_sampled": list(map(int, b)),
            "taus_for_sparsity": taus, "sparsity_at_listed_taus": {str(t): float((g < t).mean()) for t in w.taus}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--threads", type=int, default=oracle.default_threads())
    ap.add_argument("--out", default=os.path.join(ROOT, "tests", "golden", "calibration.json"))
    ap.add_argument("--skip-prefill", action="store_true")
    args = ap.parse_args()
    rec = {"generated_by": "python -m oracle.calibrate", "decode": calibrate_decode(args.threads)}
    if not args.skip_prefill:
        rec["prefill"] = calibrate_prefill(args.threads)
    os.makedirs(os.path.dirname(args.out), exist_ok=True)
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
