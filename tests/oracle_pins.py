"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle (optionally a separately
built copy, passed as ``lib``) disagrees with:
  * a library routine: torch's scaled_dot_product_attention in float64 on the CPU
    (the dense special case tau = -inf, and the output given a key mask);
  * brute force in numpy long double on tiny inputs;
  * closed forms: uniform scores give exact means of V; hand-built worked examples
    whose outputs and masks are derived by hand below;
  * invariants: closed form == scan form, monotone skip set in tau, the first tile of
    every scan is kept, tau = -inf skips nothing, the dropped-mass bound, split-count
    invariance at tau = -inf.

The rule being pinned (recap of "Accelerating Long-Context Inference with Skip Softmax in
NVIDIA TensorRT-LLM", Key Points / Detailed Analysis / Skip Softmax Mechanism; news item
"Understanding Skip Softmax"): a key tile is skipped when its local score maximum falls
below the running maximum by more than tau, for every row of the unit.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

LN1000 = math.log(1000.0)


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- references
def sdpa_prefill(q, k, v, causal, scale=None, key_mask=None):
    """torch SDPA in float64; q [B,S,Hq,d], k/v [B,S,Hkv,d] -> [B,S,Hq,d].  key_mask [B,Hq,S,S] bool."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(np.asarray(k, np.float64)).permute(0, 2, 1, 3)
    vt = torch.from_numpy(np.asarray(v, np.float64)).permute(0, 2, 1, 3)
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    if key_mask is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale)
    else:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(key_mask),
                                                             scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def sdpa_decode(q, k, v, kv_lens, scale=None):
    """q [B,Hq,d], k/v [B,Hkv,smax,d] -> [B,Hq,d] over keys j < kv_len[b]."""
    B, Hq, d = q.shape
    G = Hq // k.shape[1]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        n = int(kv_lens[b])
        if n == 0:
            continue
        qt = torch.from_numpy(np.asarray(q[b], np.float64))[:, None, :]
        kt = torch.from_numpy(np.asarray(k[b, :, :n], np.float64)).repeat_interleave(G, dim=0)
        vt = torch.from_numpy(np.asarray(v[b, :, :n], np.float64)).repeat_interleave(G, dim=0)
        out[b] = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0].numpy()
    return out


def brute_prefill_longdouble(q, k, v, causal):
    """Two-pass safe softmax attention with explicit loops in numpy long double (tiny inputs only)."""
    B, S, Hq, d = q.shape
    G = Hq // k.shape[2]
    ld = np.longdouble
    out = np.zeros((B, S, Hq, d), dtype=ld)
    sc = ld(1) / np.sqrt(ld(d))
    for b in range(B):
        for h in range(Hq):
            for i in range(S):
                n = i + 1 if causal else S
                logits = [sc * sum(ld(q[b, i, h, c]) * ld(k[b, j, h // G, c]) for c in range(d)) for j in range(n)]
                m = max(logits)
                w = [np.exp(x - m) for x in logits]
                z = sum(w)
                for c in range(d):
                    out[b, i, h, c] = sum(w[j] * ld(v[b, j, h // G, c]) for j in range(n)) / z
    return out


def unit_rows(res_out, B, S, Hq, tile_q):
    """Reassemble oracle per-unit prefill output [n,Tq,d] (all units) into [B,S,Hq,d]."""
    nqt = -(-S // tile_q)
    d = res_out.shape[-1]
    o = res_out.reshape(B, Hq, nqt * tile_q, d)[:, :, :S]
    return o.transpose(0, 2, 1, 3)


def prefill_inputs(seed, B, S, Hq, Hkv, d, planted=0, amp=12.0):
    """Random fp64 inputs; ``planted`` key tiles (of 64) per KV head get +amp logits along a common direction."""
    r = rng(seed)
    q = r.standard_normal((B, S, Hq, d))
    k = r.standard_normal((B, S, Hkv, d))
    v = r.standard_normal((B, S, Hkv, d))
    if planted:
        u = r.standard_normal(d)
        u /= np.linalg.norm(u)
        mu = math.sqrt(d)
        q = q - np.einsum("bshd,d->bsh", q, u)[..., None] * u + mu * u  # common mode mu along u
        nt = -(-S // 64)
        for b in range(B):
            for g in range(Hkv):
                for t in r.choice(np.arange(1, nt), size=min(planted, nt - 1), replace=False):
                    k[b, t * 64:(t + 1) * 64, g] += amp * math.sqrt(d) / mu * u
    return q, k, v


# ----------------------------------------------------------------- pins
def pin_dense_prefill(lib=None):
    """tau = -inf equals dense softmax attention (SDPA float64), causal and not, GQA, ragged S."""
    cases = [(1, 1, 1, 1, 64, 64, 64), (1, 63, 2, 1, 64, 64, 64), (1, 65, 4, 2, 64, 128, 64),
             (2, 130, 4, 1, 128, 128, 64), (1, 200, 8, 2, 64, 64, 64), (1, 64, 2, 2, 16, 64, 64)]
    for seed, (B, S, Hq, Hkv, d, Tq, Tk) in enumerate(cases):
        q, k, v = prefill_inputs(seed, B, S, Hq, Hkv, d)
        for causal in (True, False):
            r = oracle.prefill(q, k, v, causal=causal, tau=-math.inf, tile_q=Tq, tile_k=Tk, lib=lib)
            got = unit_rows(r["out"], B, S, Hq, Tq)
            ref = sdpa_prefill(q, k, v, causal)
            err = np.abs(got - ref).max()
            assert err < 1e-12, f"dense prefill mismatch {err} case {(B, S, Hq, Hkv, d, causal)}"
            assert (r["state"] != oracle.SKIPPED).all()


def pin_dense_decode(lib=None):
    """tau = -inf decode equals dense single-query attention for every split count, incl. kv_len edge cases."""
    r0 = rng(7)
    B, Hq, Hkv, d, smax = 6, 8, 2, 64, 200
    q = r0.standard_normal((B, Hq, d))
    k = r0.standard_normal((B, Hkv, smax, d))
    v = r0.standard_normal((B, Hkv, smax, d))
    lens = np.array([0, 1, 63, 64, 65, 200], np.int32)
    ref = sdpa_decode(q, k, v, lens)
    for P in (1, 3, 16):
        r = oracle.decode(q, k, v, lens, tau=-math.inf, num_splits=P, lib=lib)
        got = r["out"].reshape(B, Hq, d)
        err = np.abs(got - ref).max()
        assert err < 1e-12, f"dense decode mismatch {err} P={P}"
        lse = r["lse"].reshape(B, Hq)
        assert np.isneginf(lse[0]).all() and np.all(got[0] == 0), "kv_len = 0 must give 0 and lse = -inf"


def pin_longdouble_bruteforce(lib=None):
    """Dense oracle vs explicit-loop long double softmax on tiny inputs."""
    q, k, v = prefill_inputs(11, 1, 9, 2, 1, 4)
    for causal in (True, False):
        r = oracle.prefill(q, k, v, causal=causal, tau=-math.inf, tile_q=4, tile_k=4, lib=lib)
        got = unit_rows(r["out"], 1, 9, 2, 4)
        ref = brute_prefill_longdouble(q, k, v, causal).astype(np.float64)
        assert np.abs(got - ref).max() < 1e-13


def pin_forms_agree(lib=None):
    """Closed form and scan form: identical masks and gammas, outputs within 1e-12 (prefill and split decode)."""
    for seed, (S, Hq, Hkv, d, causal, tau) in enumerate([(512, 4, 1, 64, True, -LN1000), (300, 4, 2, 32, False, -4.0),
                                                          (640, 8, 2, 64, True, -2.0)]):
        q, k, v = prefill_inputs(100 + seed, 1, S, Hq, Hkv, d, planted=2)
        a = oracle.prefill(q, k, v, causal=causal, tau=tau, tile_q=128, tile_k=64, lib=lib)
        b = oracle.prefill(q, k, v, causal=causal, tau=tau, tile_q=128, tile_k=64, form="scan", lib=lib)
        assert np.array_equal(a["state"], b["state"]), "closed vs scan mask"
        vis = a["state"] > 0
        assert np.array_equal(a["gamma"][vis], b["gamma"][vis])
        assert np.abs(a["out"] - b["out"]).max() < 1e-12
        assert np.abs(a["lse"][np.isfinite(a["lse"])] - b["lse"][np.isfinite(b["lse"])]).max() < 1e-12
    q, k, v, lens = decode_planted(5)
    for P in (1, 4, 16):
        for seeded in (False, True):
            a = oracle.decode(q, k, v, lens, tau=-LN1000, num_splits=P, sink_seed=seeded, lib=lib)
            b = oracle.decode(q, k, v, lens, tau=-LN1000, num_splits=P, form="scan", sink_seed=seeded, lib=lib)
            assert np.array_equal(a["state"], b["state"]), f"decode closed vs scan mask P={P} seeded={seeded}"
            vis = a["state"] > 0
            assert np.array_equal(a["gamma"][vis], b["gamma"][vis]), f"decode gammas P={P} seeded={seeded}"
            assert np.abs(a["out"] - b["out"]).max() < 1e-12


def decode_planted(seed, B=3, Hq=16, Hkv=2, d=64, smax=4096):
    """Decode inputs with a sink tile (+16 logits) and 10% relevant tiles (+10 logits)."""
    r = rng(seed)
    q = r.standard_normal((B, Hq, d))
    k = r.standard_normal((B, Hkv, smax, d))
    v = r.standard_normal((B, Hkv, smax, d))
    G = Hq // Hkv
    for b in range(B):
        for g in range(Hkv):
            qh = q[b, g * G:(g + 1) * G].sum(0)
            qh /= np.linalg.norm(qh)
            k[b, g, :64] += 4 * math.sqrt(d) * qh
            for t in range(1, smax // 64):
                if r.random() < 0.1:
                    k[b, g, t * 64:(t + 1) * 64] += 2.5 * math.sqrt(d) * qh
    lens = np.array([smax, smax - 100, 1000][:B], np.int32)
    return q, k, v, lens


def pin_mask_invariants(lib=None):
    """Monotone in tau, tau=-inf skips nothing, first tile of each scan kept, tau=0 keeps tiles with Gamma>=0."""
    q, k, v = prefill_inputs(21, 1, 768, 4, 1, 64, planted=3)
    taus = [-math.inf, -20.0, -LN1000, -4.0, -1.0, -0.1, 0.0]
    prev = None
    for tau in taus:
        r = oracle.prefill(q, k, v, causal=True, tau=tau, tile_q=128, tile_k=64, lib=lib)
        sk = r["state"] == oracle.SKIPPED
        if tau == -math.inf:
            assert not sk.any()
        if prev is not None:
            assert not (prev & ~sk).any(), f"skip set not monotone at tau={tau}"
        assert not sk[:, 0].any(), "first tile of a scan skipped"
        if tau == 0.0:
            assert not (sk & (r["gamma"] >= 0)).any()
        prev = sk
    assert prev.any(), "the planted input must skip something at tau = 0"
    qd, kd, vd, lens = decode_planted(22)
    P = 4
    for tau in (-LN1000, -2.0):
        r = oracle.decode(qd, kd, vd, lens, tau=tau, num_splits=P, lib=lib)
        for u in range(r["state"].shape[0]):
            b = u // kd.shape[1]
            nt = -(-int(lens[b]) // 64)
            tps = -(-nt // P)
            for s in range(P):
                if s * tps < nt:
                    assert r["state"][u, s * tps] == oracle.EXECUTED, "first tile of a split skipped"
            assert (r["state"][u, nt:] == oracle.UNVISITED).all()
            assert (r["state"][u, :nt] != oracle.UNVISITED).all()


def pin_uniform_scores(lib=None):
    """q = 0 gives logits 0, so nothing is skipped and each output is the exact mean of the visible V rows."""
    r0 = rng(31)
    S, d = 200, 64
    q = np.zeros((1, S, 2, d))
    k = r0.standard_normal((1, S, 1, d))
    v = r0.standard_normal((1, S, 1, d))
    for tau in (0.0, -1.0, -LN1000):
        r = oracle.prefill(q, k, v, causal=True, tau=tau, tile_q=64, tile_k=64, lib=lib)
        assert not (r["state"] == oracle.SKIPPED).any()
        got = unit_rows(r["out"], 1, S, 2, 64)
        prefix_mean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
        for h in range(2):
            assert np.abs(got[0, :, h] - prefix_mean).max() < 1e-12
    qd = np.zeros((2, 4, d))
    kd = r0.standard_normal((2, 1, 300, d))
    vd = r0.standard_normal((2, 1, 300, d))
    lens = np.array([300, 129], np.int32)
    r = oracle.decode(qd, kd, vd, lens, tau=0.0, num_splits=16, lib=lib)
    for b in range(2):
        m = vd[b, 0, :lens[b]].mean(0)
        assert np.abs(r["out"][b] - m).max() < 1e-12


def pin_dropped_mass(lib=None):
    """Each skipped tile drops at most tile_k*e^tau of a row's kept mass; the output moves by at most
    2*delta/(1+delta)*max|v| from dense attention."""
    q, k, v = prefill_inputs(41, 1, 1024, 4, 1, 64, planted=4)
    for tau in (-LN1000, -4.0, -1.0):
        r = oracle.prefill(q, k, v, causal=True, tau=tau, tile_q=128, tile_k=64, lib=lib)
        dense = oracle.prefill(q, k, v, causal=True, tau=-math.inf, tile_q=128, tile_k=64, lib=lib)
        nskip = (r["state"] == oracle.SKIPPED).sum(1)
        bound = nskip[:, None] * 64 * math.exp(tau)
        assert (r["dropped"] <= bound * (1 + 1e-12) + 1e-300).all()
        delta = r["dropped"]
        dev = np.abs(r["out"] - dense["out"]).max(-1)
        vmax = np.abs(v).max()
        assert (dev <= 2 * delta / (1 + delta) * vmax + 1e-12).all()
        assert nskip.sum() > 0


def pin_split_invariance(lib=None):
    """At tau = -inf the split-K combine is exact: the output does not depend on the split count."""
    q, k, v, lens = decode_planted(51)
    base = oracle.decode(q, k, v, lens, tau=-math.inf, num_splits=1, lib=lib)
    for P in (2, 7, 16, 64):
        r = oracle.decode(q, k, v, lens, tau=-math.inf, num_splits=P, lib=lib)
        assert np.abs(r["out"] - base["out"]).max() < 1e-12
        assert np.abs(r["lse"] - base["lse"]).max() < 1e-12


def pin_output_given_mask(lib=None):
    """With the oracle's own mask, the output equals softmax restricted to the kept keys (SDPA + boolean mask)."""
    B, S, Hq, Hkv, d = 1, 384, 4, 2, 32
    q, k, v = prefill_inputs(61, B, S, Hq, Hkv, d, planted=2)
    Tq, Tk = 128, 64
    r = oracle.prefill(q, k, v, causal=True, tau=-2.0, tile_q=Tq, tile_k=Tk, lib=lib)
    nqt = S // Tq
    mask = np.zeros((B, Hq, S, S), bool)
    for h in range(Hq):
        for qt in range(nqt):
            st = r["state"][h * nqt + qt]
            for i in range(qt * Tq, (qt + 1) * Tq):
                for t in range(S // Tk):
                    if st[t] == oracle.EXECUTED:
                        mask[0, h, i, t * Tk:min((t + 1) * Tk, i + 1)] = True
    assert (r["state"] == oracle.SKIPPED).any()
    ref = sdpa_prefill(q, k, v, False, key_mask=mask)
    got = unit_rows(r["out"], B, S, Hq, Tq)
    assert np.abs(got - ref).max() < 1e-12
    # forcing a mask through the override gives the same restricted softmax
    ov = np.full(r["state"].shape, -1, np.int8)
    ov[:, 1] = 1
    r2 = oracle.prefill(q, k, v, causal=True, tau=-math.inf, tile_q=Tq, tile_k=Tk, override=ov, lib=lib)
    mask2 = np.tril(np.ones((S, S), bool))[None, None].repeat(Hq, 1)
    mask2[:, :, :, Tk:2 * Tk] = False
    mask2[:, :, :Tk, :Tk] = np.tril(np.ones((Tk, Tk), bool))
    ref2 = sdpa_prefill(q, k, v, False, key_mask=mask2)
    got2 = unit_rows(r2["out"], B, S, Hq, Tq)
    assert np.abs(got2 - ref2).max() < 1e-12


def pin_sink_seed(lib=None):
    """Sink-seeded split-K decode.  Each split's running maximum is max(first-tile maxima, earlier tiles of
    the split), which lies between the split-local one (earlier tiles of the split only) and the sequential
    one (every earlier tile), so the skip sets nest: split-local <= seeded <= sequential (P = 1).  With one
    split, seeding changes nothing; at tau = -inf nothing is skipped and the output is dense attention; the
    dropped-mass bound holds, since tile 0 (the seed) is always kept by the first split."""
    q, k, v, lens = decode_planted(71)
    dense = sdpa_decode(q, k, v, lens)
    for tau in (-LN1000, -4.0, -2.0):
        seq = oracle.decode(q, k, v, lens, tau=tau, num_splits=1, lib=lib)
        one = oracle.decode(q, k, v, lens, tau=tau, num_splits=1, sink_seed=True, lib=lib)
        assert np.array_equal(seq["state"], one["state"]) and np.abs(seq["out"] - one["out"]).max() == 0.0
        for P in (4, 16):
            loc = oracle.decode(q, k, v, lens, tau=tau, num_splits=P, lib=lib)
            sd = oracle.decode(q, k, v, lens, tau=tau, num_splits=P, sink_seed=True, lib=lib)
            s_loc, s_sd, s_seq = (x["state"] == oracle.SKIPPED for x in (loc, sd, seq))
            assert not (s_loc & ~s_sd).any(), f"split-local skip not kept skipped by seeding (tau={tau}, P={P})"
            assert not (s_sd & ~s_seq).any(), f"seeded skip not skipped sequentially (tau={tau}, P={P})"
            assert np.array_equal(loc["state"] > 0, sd["state"] > 0), "visited tiles differ"
            assert (sd["state"][:, 0] == oracle.EXECUTED).all(), "tile 0 skipped"
            if tau == -LN1000 and P == 16:
                assert s_sd.sum() > s_loc.sum(), "seeding must recover sparsity on the planted input"
            nskip = s_sd.sum(1)
            assert (sd["dropped"] <= nskip[:, None] * 64 * math.exp(tau) * (1 + 1e-12) + 1e-300).all()
            delta = sd["dropped"]
            dev = np.abs(sd["out"] - dense.reshape(sd["out"].shape)).max(-1)
            assert (dev <= 2 * delta / (1 + delta) * np.abs(v).max() + 1e-12).all()
    r = oracle.decode(q, k, v, lens, tau=-math.inf, num_splits=16, sink_seed=True, lib=lib)
    assert not (r["state"] == oracle.SKIPPED).any()
    assert np.abs(r["out"] - dense.reshape(r["out"].shape)).max() < 1e-12


def fp8_e4m3_codes_to_f64(codes):
    """torch's OCP float8_e4m3fn conversion of uint8 codes to float64 (the library routine of the fp8 pin)."""
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_fp8_kv(lib=None):
    """K/V given as OCP fp8 e4m3 codes with per-tensor scales: the oracle must equal the same decode on the
    values torch decodes from the codes (times the scales), in both forms, split-local and seeded, and
    dense SDPA at tau = -inf.  Every finite code (subnormals, both zeros, +-448) appears in K and V."""
    r0 = rng(81)
    B, Hq, Hkv, d, smax = 3, 8, 2, 64, 1100
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    kc = r0.choice(finite, size=(B, Hkv, smax, d))
    vc = r0.choice(finite, size=(B, Hkv, smax, d))
    kc[0, 0, :len(finite), 0] = finite
    vc[0, 0, :len(finite), 0] = finite
    q = r0.standard_normal((B, Hq, d)) * 2e-3          # keeps logits of order 1 for |k| up to 448 * k_scale
    q[:, :, 1] = 1.0                                     # channel 1 carries a sink: code 0x7E = 448 on tile 0,
    kc[:, :, :, 1] = 0                                   # zero elsewhere (+20.7 logits on the sink tile)
    kc[:, :, :64, 1] = 0x7E
    ks, vs = 0.37, 1.9
    kf, vf = fp8_e4m3_codes_to_f64(kc) * ks, fp8_e4m3_codes_to_f64(vc) * vs
    assert np.isfinite(kf).all() and np.isfinite(vf).all()
    lens = np.array([smax, 777, 64], np.int32)
    for P, seeded in ((1, False), (16, False), (16, True)):
        for tau in (-LN1000, -2.0, -math.inf):
            for form in ("closed", "scan"):
                a = oracle.decode(q, kc, vc, lens, tau=tau, num_splits=P, sink_seed=seeded, k_scale=ks, v_scale=vs,
                                  form=form, lib=lib)
                b = oracle.decode(q, kf, vf, lens, tau=tau, num_splits=P, sink_seed=seeded, form=form, lib=lib)
                assert np.array_equal(a["state"], b["state"]), f"fp8 mask P={P} seeded={seeded} tau={tau} {form}"
                assert np.abs(a["out"] - b["out"]).max() < 1e-12, f"fp8 output P={P} seeded={seeded} tau={tau}"
            if tau == -LN1000 and P == 16:
                assert (a["state"] == oracle.SKIPPED).any(), "the fp8 input must skip something"
    dense = sdpa_decode(q, kf, vf, lens)
    r = oracle.decode(q, kc, vc, lens, tau=-math.inf, num_splits=16, k_scale=ks, v_scale=vs, lib=lib)
    assert np.abs(r["out"] - dense.reshape(r["out"].shape)).max() < 1e-12
    # one key per sequence: the output is that key's value, so every code's value is observed directly
    lens1 = np.ones(len(finite), np.int32)
    v1 = np.zeros((len(finite), 1, 1, 1), np.uint8); v1[:, 0, 0, 0] = finite
    k1 = np.zeros_like(v1)
    r = oracle.decode(np.zeros((len(finite), 1, 1)), k1, v1, lens1, tau=-math.inf, num_splits=1, k_scale=1.0,
                      v_scale=1.0, lib=lib)
    assert np.array_equal(r["out"][:, 0, 0], fp8_e4m3_codes_to_f64(finite)), "fp8 code values"


def chunk_inputs(seed, B, S, Sk, Hq, Hkv, d, planted=2):
    """Chunked-prefill inputs: q [B,S,Hq,d] are the queries of the last S of Sk positions; k/v [B,Sk,Hkv,d]."""
    q, k, v = prefill_inputs(seed, B, Sk, Hq, Hkv, d, planted=planted)
    return np.ascontiguousarray(q[:, Sk - S:]), k, v


def bottom_right_mask(B, Hq, S, Sk, causal):
    m = np.ones((B, Hq, S, Sk), bool)
    if causal:
        off = Sk - S
        m &= np.arange(Sk)[None, :] <= (off + np.arange(S))[:, None]
    return m


def pin_chunked_prefill(lib=None):
    """Chunked prefill (S queries = the last S of Sk positions, bottom-right causal).  At tau = -inf it is SDPA
    with the bottom-right mask; when the chunk starts on a query-tile boundary its units are exactly units of the
    full prefill over all Sk positions (same rows, same key tiles), so masks and outputs must be identical."""
    for seed, (S, Sk, Hq, Hkv, d, causal, Tq) in enumerate([(64, 200, 4, 2, 32, True, 64), (77, 301, 4, 1, 64, True, 64),
                                                           (130, 130, 2, 1, 16, True, 128), (5, 9, 2, 1, 2, True, 64),
                                                           (100, 250, 4, 2, 32, False, 128), (1, 190, 4, 4, 64, True, 128)]):
        q, k, v = chunk_inputs(90 + seed, 1, S, Sk, Hq, Hkv, d)
        r = oracle.prefill(q, k, v, causal=causal, tau=-math.inf, tile_q=Tq, tile_k=64, lib=lib)
        ref = sdpa_prefill(q, k, v, False, key_mask=bottom_right_mask(1, Hq, S, Sk, causal))
        got = unit_rows(r["out"], 1, S, Hq, Tq)
        assert np.abs(got - ref).max() < 1e-12, f"chunk S={S} Sk={Sk} causal={causal} vs SDPA"
        nkt = -(-Sk // 64)
        nqt = -(-S // Tq)
        last = (Sk - S + np.minimum(S, (np.arange(nqt) + 1) * Tq) - 1) // 64 if causal else np.full(nqt, nkt - 1)
        for h in range(Hq):
            for qt in range(nqt):
                st = r["state"][h * nqt + qt]
                assert (st[:last[qt] + 1] == oracle.EXECUTED).all() and (st[last[qt] + 1:] == 0).all(), "visited tiles"
    for Tq in (64, 128):
        S, Sk = 3 * Tq, 3 * Tq + 2 * Tq
        q, k, v = chunk_inputs(97, 1, S, Sk, 4, 2, 64, planted=3)
        qfull, _, _ = chunk_inputs(97, 1, Sk, Sk, 4, 2, 64, planted=3)
        for tau in (-LN1000, -2.0):
            a = oracle.prefill(q, k, v, causal=True, tau=tau, tile_q=Tq, tile_k=64, lib=lib)
            f = oracle.prefill(qfull, k, v, causal=True, tau=tau, tile_q=Tq, tile_k=64, lib=lib)
            nq, nf = S // Tq, Sk // Tq
            units_f = np.array([h * nf + (Sk - S) // Tq + qt for h in range(4) for qt in range(nq)])
            assert np.array_equal(a["state"], f["state"][units_f]), f"aligned chunk mask Tq={Tq} tau={tau}"
            assert np.abs(a["out"] - f["out"][units_f]).max() < 1e-12
            assert (a["state"] == oracle.SKIPPED).any(), "the planted input must skip something"


def pin_worked_example_chunk(lib=None):
    """W7: W1's keys (tile 0 logit 0, tile 1 logit -10; v = (j, 1) then (1000, -1)) with the queries at positions
    64..127 only (S = 64, Sk = 128, causal, bottom-right).  Query i sees keys 0..64+i, so tile 1 is visited
    (partially) by every row and trails by 10: skipped at tau = -ln 1000 (every row gets (31.5, 1)); at tau = -inf
    row i gets (2016 + 1000 (i+1) e^-10, 64 - (i+1) e^-10) / (64 + (i+1) e^-10)."""
    q1, k1, v1 = _w1_inputs()
    q = np.ascontiguousarray(q1[:, 64:])
    e = math.exp(-10.0)
    for tau, skipped in ((-LN1000, True), (-math.inf, False)):
        r = oracle.prefill(q, k1, v1, causal=True, tau=tau, tile_q=64, tile_k=64, scale=1.0, lib=lib)
        assert list(r["state"][0]) == [1, 2 if skipped else 1], f"W7 mask tau={tau}"
        i = np.arange(64)
        if skipped:
            want = np.stack([np.full(64, 31.5), np.ones(64)], 1)
        else:
            n = i + 1
            want = np.stack([(2016 + 1000 * n * e) / (64 + n * e), (64 - n * e) / (64 + n * e)], 1)
        assert np.abs(r["out"][0] - want).max() < 1e-12, f"W7 output tau={tau}"


# ----------------------------------------------------------------- worked examples
def _w1_inputs():
    """d=2, S=128, q_i=(1,0); tile-0 keys (0,0) -> logit 0; tile-1 keys (-10,0) -> logit -10 (scale 1).
    v_j = (j, 1) on tile 0 and (1000, -1) on tile 1."""
    S, d = 128, 2
    q = np.zeros((1, S, 1, d)); q[..., 0] = 1.0
    k = np.zeros((1, S, 1, d)); k[0, 64:, 0, 0] = -10.0
    v = np.zeros((1, S, 1, d))
    v[0, :64, 0, 0] = np.arange(64); v[0, :64, 0, 1] = 1.0
    v[0, 64:, 0, 0] = 1000.0; v[0, 64:, 0, 1] = -1.0
    return q, k, v


def pin_worked_examples(lib=None):
    """Hand-built examples with outputs derived by hand."""
    # W1: tile 1 trails the running max by exactly 10.
    q, k, v = _w1_inputs()
    e = math.exp(-10.0)
    dense = np.array([(31.5 + 1000 * e) / (1 + e), (1 - e) / (1 + e)])
    for tau, skipped in ((-LN1000, True), (-10.0, False), (-11.0, False), (-math.inf, False), (-9.999, True)):
        r = oracle.prefill(q, k, v, causal=False, tau=tau, tile_q=64, tile_k=64, scale=1.0, lib=lib)
        want = np.array([31.5, 1.0]) if skipped else dense
        assert np.abs(r["out"][:, :, :] - want).max() < 1e-12, f"W1 tau={tau}"
        assert list(r["state"][0]) == [1, 2 if skipped else 1], f"W1 mask tau={tau}"
        assert abs(r["gamma"][0, 1] - (-10.0)) == 0.0
        if skipped:
            assert np.abs(r["dropped"] - e).max() < 1e-15
    # W1 in decode form: the 128 keys as one sequence, G=2 identical query heads, one split.
    qd = np.zeros((1, 2, 2)); qd[..., 0] = 1.0
    kd = k[0, :, 0][None, None]; vd = v[0, :, 0][None, None]
    r = oracle.decode(qd, kd, vd, np.array([128], np.int32), tau=-LN1000, num_splits=1, scale=1.0, lib=lib)
    assert np.abs(r["out"] - np.array([31.5, 1.0])).max() < 1e-12 and list(r["state"][0]) == [1, 2]
    # W1 with two splits: tile 1 starts its own scan, so it is never skipped.
    r = oracle.decode(qd, kd, vd, np.array([128], np.int32), tau=-LN1000, num_splits=2, scale=1.0, lib=lib)
    assert np.abs(r["out"] - dense).max() < 1e-12 and list(r["state"][0]) == [1, 1]

    # W2: the comparison is against the running maximum, not against tile 0.
    # Tile logits: tile0 = 0, tile1 = 8 (new max, kept), tile2 = 3 (5 below the running max 8).
    S = 192
    q = np.zeros((1, S, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, S, 1, 2)); k[0, 64:128, 0, 0] = 8.0; k[0, 128:, 0, 0] = 3.0
    v = np.zeros((1, S, 1, 2)); v[0, :64, 0, 0] = 1.0; v[0, 64:128, 0, 1] = 1.0; v[0, 128:, 0, :] = -1.0
    r = oracle.prefill(q, k, v, causal=False, tau=-4.0, tile_q=64, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 1, 2], "W2 mask"
    z = 1 + math.exp(8)
    assert np.abs(r["out"][0] - np.array([1 / z, math.exp(8) / z])).max() < 1e-12
    r = oracle.prefill(q, k, v, causal=False, tau=-6.0, tile_q=64, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 1, 1], "W2 kept at tau=-6"

    # W3: every row must agree.  Row 0 trails by 10 on tile 1, row 1 gains 2: the tile is kept.
    q = np.zeros((1, 128, 1, 2)); q[0, :, 0, 0] = 1.0; q[0, 1, 0] = (0.0, 1.0)
    k = np.zeros((1, 128, 1, 2)); k[0, 64:, 0] = (-10.0, 2.0)
    v = np.ones((1, 128, 1, 2))
    r = oracle.prefill(q, k, v, causal=False, tau=-LN1000, tile_q=64, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 1], "W3 agreement rule"
    assert r["gamma"][0, 1] == 2.0
    q[0, 1, 0] = (1.0, 0.0)
    r = oracle.prefill(q, k, v, causal=False, tau=-LN1000, tile_q=64, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 2], "W3 skipped once all rows trail"

    # W4: causal abstention.  Tq=128, Tk=64, S=128: rows 0..63 have no valid key in tile 1 and abstain;
    # rows 64..127 trail the running max by 10 there, so the tile is skipped and those rows attend
    # only to tile 0 (keys 0..63, logit 0): output = mean of v over keys 0..63.
    q = np.zeros((1, 128, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, 128, 1, 2)); k[0, 64:, 0, 0] = -10.0
    v = np.zeros((1, 128, 1, 2)); v[0, :, 0, 0] = np.arange(128); v[0, :, 0, 1] = 1.0
    r = oracle.prefill(q, k, v, causal=True, tau=-LN1000, tile_q=128, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 2], "W4 mask"
    assert r["gamma"][0, 1] == -10.0
    rows = np.arange(64, 128)
    assert np.abs(r["out"][0, rows, 0] - 31.5).max() < 1e-12
    assert np.abs(r["out"][0, :64, 0] - np.arange(64) / 2.0).max() < 1e-12  # row i: mean of 0..i

    # W5: the first tile of a scan is kept even when its logits are far below tau.
    q = np.zeros((1, 128, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, 128, 1, 2)); k[0, :64, 0, 0] = -30.0; k[0, 64:, 0, 0] = -45.0
    v = np.zeros((1, 128, 1, 2)); v[0, :64, 0, 0] = 2.0; v[0, 64:, 0, 0] = 5.0
    r = oracle.prefill(q, k, v, causal=False, tau=-LN1000, tile_q=64, tile_k=64, scale=1.0, lib=lib)
    assert list(r["state"][0]) == [1, 2], "W5 mask"
    assert np.abs(r["out"][0, :, 0] - 2.0).max() < 1e-12


def pin_worked_example_sink_seed(lib=None):
    """W6 (decode, d = 2, scale 1, two query heads q = (1, 0), kv_len = 256, four tiles): the keys of tile t
    give the logit L_t = (0, 5, -2, -10)[t] and v_j = (t, 1).  At tau = -ln 1000 (about -6.91):
      split-local, P = 4: every tile is the first of its split            -> kept {0, 1, 2, 3}
      seeded,      P = 4: tile t > 0 is compared with L_0 = 0: gaps 5, -2, -10       -> kept {0, 1, 2}
      sequential,  P = 1: running maxima 0, 5, 5: gaps 5, -7, -15                   -> kept {0, 1}
    and the output is (sum_K t e^L_t / sum_K e^L_t, 1) over the kept set K."""
    L = [0.0, 5.0, -2.0, -10.0]
    k = np.zeros((1, 1, 256, 2)); v = np.zeros((1, 1, 256, 2))
    for t in range(4):
        k[0, 0, 64 * t:64 * (t + 1), 0] = L[t]
        v[0, 0, 64 * t:64 * (t + 1)] = (t, 1.0)
    q = np.zeros((1, 2, 2)); q[..., 0] = 1.0
    lens = np.array([256], np.int32)

    def want(kept):
        w = np.array([math.exp(L[t]) for t in kept])
        return np.array([(w * np.array(kept)).sum() / w.sum(), 1.0])

    for P, seeded, kept in ((4, False, [0, 1, 2, 3]), (4, True, [0, 1, 2]), (1, False, [0, 1]), (1, True, [0, 1]),
                            (2, True, [0, 1, 2])):
        # P = 2: splits {0, 1} and {2, 3}; the second starts from L_0 = 0, keeps tile 2 (gap -2), then
        # compares tile 3 with max(0, -2) = 0 (gap -10): skipped
        for form in ("closed", "scan"):
            r = oracle.decode(q, k, v, lens, tau=-LN1000, num_splits=P, scale=1.0, sink_seed=seeded, form=form,
                              lib=lib)
            st = [1 if t in kept else 2 for t in range(4)]
            assert list(r["state"][0]) == st, f"W6 mask P={P} seeded={seeded} {form}: {list(r['state'][0])}"
            assert np.abs(r["out"][0] - want(kept)).max() < 1e-12, f"W6 output P={P} seeded={seeded} {form}"
    r = oracle.decode(q, k, v, lens, tau=-LN1000, num_splits=4, scale=1.0, sink_seed=True, lib=lib)
    assert list(r["gamma"][0]) == [math.inf, 5.0, -2.0, -10.0], "W6 gaps against the seed"


def _bf16_bits_and_values(x):
    """torch's round-to-nearest-even bf16 of x: (uint16 bit patterns, their values as float64 via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16), t.to(torch.float64).numpy()


def pin_input_widening(lib=None):
    """The oracle's bf16 and fp32 inputs are the values they encode: on bf16 bit patterns it must give exactly
    (bit for bit: outputs, unit gaps, masks) what it gives on torch's float64 decoding of the same bf16 values,
    and on fp32 arrays exactly what it gives on numpy's float64 widening of them.  Both prefill and decode, with
    planted tiles so that some tiles are skipped and the masks are compared too."""
    q, k, v = prefill_inputs(21, 1, 300, 4, 2, 64, planted=2)
    for causal in (True, False):
        ref = None
        for variant in ("bf16", "fp32"):
            if variant == "bf16":
                (qb, qd), (kb, kd), (vb, vd) = (_bf16_bits_and_values(x) for x in (q, k, v))
                a = oracle.prefill(qb, kb, vb, causal=causal, tau=-LN1000, tile_q=64, lib=lib)
                b = oracle.prefill(qd, kd, vd, causal=causal, tau=-LN1000, tile_q=64, lib=lib)
            else:
                q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
                a = oracle.prefill(q32, k32, v32, causal=causal, tau=-LN1000, tile_q=64, lib=lib)
                b = oracle.prefill(*(x.astype(np.float64) for x in (q32, k32, v32)), causal=causal, tau=-LN1000,
                                   tile_q=64, lib=lib)
            for key in ("out", "gamma", "state"):
                assert np.array_equal(a[key], b[key], equal_nan=True), f"prefill {variant} widening differs in {key}"
            assert (a["state"] == oracle.SKIPPED).any(), "the case must skip some tiles"
            ref = a["out"] if ref is None else ref
        # bf16 rounding moves the output by far less than the output itself
        assert np.abs(ref - a["out"]).max() < 0.05
    qd_, kd_, vd_, lens = decode_planted(22, B=2, Hq=8, Hkv=2, d=64, smax=1024)
    for variant in ("bf16", "fp32"):
        if variant == "bf16":
            (qb, qd), (kb, kd), (vb, vd) = (_bf16_bits_and_values(x) for x in (qd_, kd_, vd_))
            a = oracle.decode(qb, kb, vb, lens, tau=-LN1000, num_splits=4, lib=lib)
            b = oracle.decode(qd, kd, vd, lens, tau=-LN1000, num_splits=4, lib=lib)
        else:
            x32 = [x.astype(np.float32) for x in (qd_, kd_, vd_)]
            a = oracle.decode(*x32, lens, tau=-LN1000, num_splits=4, lib=lib)
            b = oracle.decode(*(x.astype(np.float64) for x in x32), lens, tau=-LN1000, num_splits=4, lib=lib)
        for key in ("out", "gamma", "state"):
            assert np.array_equal(a[key], b[key], equal_nan=True), f"decode {variant} widening differs in {key}"
        assert (a["state"] == oracle.SKIPPED).any(), "the decode case must skip some tiles"


def _integer_logit_inputs(seed, S=200, Hq=4, Hkv=2, d=16, delta=0.0):
    """Integer-valued q, k (entries in -2..2) so that with the logit scale ln 2 the base-2 log weights
    log2(e) * ln2 * q.k are the integers q.k; with delta > 0 an extra channel (q: 1, k: uniform in
    (-delta, delta)) moves each of them off its integer by less than delta."""
    r = rng(seed)
    q = r.integers(-2, 3, (1, S, Hq, d)).astype(np.float64)
    k = r.integers(-2, 3, (1, S, Hkv, d)).astype(np.float64)
    v = r.standard_normal((1, S, Hkv, d))
    if delta:
        q = np.concatenate([q, np.ones((1, S, Hq, 1))], -1)
        k = np.concatenate([k, r.uniform(-delta, delta, (1, S, Hkv, 1))], -1)
        v = np.concatenate([v, np.zeros((1, S, Hkv, 1))], -1)
    return q, k, v


def pin_rowmax_pot(lib=None):
    """Rowmax-PoT weights ("Approximating Softmax in Pretrained LLMs", Abstract: powers of two anchored at the
    row maximum; the oracle's reading: 2^(rint(log2(e) l) - rint(log2(e) mu))):
      * logits whose base-2 log weights are integers (scale ln 2, integer q.k) have exact power-of-two weights,
        so the PoT output equals SDPA float64 at that scale (causal and not, tau = -inf), and equals the exact
        softmax of the oracle at a finite tau with identical masks;
      * moving every such log weight by less than 0.45 (one extra channel) leaves the PoT weights unchanged:
        the PoT output equals SDPA on the unmoved integer logits while the exact softmax moves;
      * both forms agree."""
    ln2 = math.log(2.0)
    for causal in (True, False):
        q, k, v = _integer_logit_inputs(31)
        got = oracle.prefill(q, k, v, causal=causal, tau=-math.inf, tile_q=64, scale=ln2, weights="rowmax_pot",
                             lib=lib)
        ref = sdpa_prefill(q, k, v, causal, scale=ln2)
        err = np.abs(unit_rows(got["out"], 1, 200, 4, 64) - ref).max()
        assert err < 1e-12, f"integer log weights: PoT differs from softmax by {err}"
        a = oracle.prefill(q, k, v, causal=causal, tau=-2.0, tile_q=64, scale=ln2, weights="rowmax_pot", lib=lib)
        b = oracle.prefill(q, k, v, causal=causal, tau=-2.0, tile_q=64, scale=ln2, lib=lib)
        assert np.array_equal(a["state"], b["state"]) and (a["state"] == oracle.SKIPPED).any()
        assert np.abs(a["out"] - b["out"]).max() < 1e-12
        qp, kp, vp = _integer_logit_inputs(31, delta=0.45)
        got = oracle.prefill(qp, kp, vp, causal=causal, tau=-math.inf, tile_q=64, scale=ln2, weights="rowmax_pot",
                             lib=lib)
        err = np.abs(unit_rows(got["out"], 1, 200, 4, 64)[..., :16] - ref).max()
        assert err < 1e-12, f"log weights moved by < 0.45: PoT output moved by {err}"
        exact = oracle.prefill(qp, kp, vp, causal=causal, tau=-math.inf, tile_q=64, scale=ln2, lib=lib)
        assert np.abs(unit_rows(exact["out"], 1, 200, 4, 64)[..., :16] - ref).max() > 1e-3
        for form_in in ((q, k, v, -2.0), (qp, kp, vp, -math.inf)):
            x, y, z, tau = form_in
            c = oracle.prefill(x, y, z, causal=causal, tau=tau, tile_q=64, scale=ln2, weights="rowmax_pot", lib=lib)
            sc = oracle.prefill(x, y, z, causal=causal, tau=tau, tile_q=64, scale=ln2, weights="rowmax_pot",
                                form="scan", lib=lib)
            assert np.array_equal(c["state"], sc["state"]) and np.abs(c["out"] - sc["out"]).max() < 1e-12


def pin_worked_example_rowmax_pot(lib=None):
    """W8 (hand-derived): logit scale ln 2, one query (1, 0) per row, three keys whose base-2 log weights are 0,
    -1.3, -2.6 (keys (0, 0), (-1.3, 0), (-2.6, 0)), values (1, 0), (0, 1), (4, 4), non-causal: the PoT weights
    are 1, 2^-1, 2^-3 (nearest integers 0, -1, -3), so o = ((1, 0) + (0, 1/2) + (1/2, 1/2)) / (13/8)
    = (12/13, 8/13).  W9: 64 keys at log weight 0 with values (j, 1), then 64 keys at -12.4 with values
    (1000, -1): at tau = -ln 1000 the second tile is skipped (gap -12.4 ln2 = -8.6 < tau) and o = (31.5, 1); at
    tau = -inf it is kept with weights 2^-12 each: o = (sum_j j + 64 * 1000 / 4096, 64 - 64 / 4096)
    / (64 + 64 / 4096)."""
    ln2 = math.log(2.0)
    q = np.zeros((1, 3, 1, 2)); q[..., 0] = 1.0
    k = np.array([[0.0, 0.0], [-1.3, 0.0], [-2.6, 0.0]]).reshape(1, 3, 1, 2)
    v = np.array([[1.0, 0.0], [0.0, 1.0], [4.0, 4.0]]).reshape(1, 3, 1, 2)
    for form in ("closed", "scan"):
        r = oracle.prefill(q, k, v, causal=False, tau=-math.inf, tile_q=64, scale=ln2, weights="rowmax_pot",
                           form=form, lib=lib)
        got = unit_rows(r["out"], 1, 3, 1, 64)[0, :, 0]
        assert np.abs(got - np.array([12 / 13, 8 / 13])).max() < 1e-14, f"W8 {form}: {got}"
    S = 128
    q = np.zeros((1, S, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, S, 1, 2)); k[0, 64:, 0, 0] = -12.4
    v = np.zeros((1, S, 1, 2))
    v[0, :64, 0, 0] = np.arange(64); v[0, :64, 0, 1] = 1.0
    v[0, 64:, 0, 0] = 1000.0; v[0, 64:, 0, 1] = -1.0
    w = 2.0 ** -12
    for form in ("closed", "scan"):
        r = oracle.prefill(q, k, v, causal=False, tau=-LN1000, tile_q=64, scale=ln2, weights="rowmax_pot",
                           form=form, lib=lib)
        got = unit_rows(r["out"], 1, S, 1, 64)[0, :, 0]
        assert np.abs(got - np.array([31.5, 1.0])).max() < 1e-12 and (r["state"][:, 1] == oracle.SKIPPED).all()
        r = oracle.prefill(q, k, v, causal=False, tau=-math.inf, tile_q=64, scale=ln2, weights="rowmax_pot",
                           form=form, lib=lib)
        got = unit_rows(r["out"], 1, S, 1, 64)[0, :, 0]
        want = np.array([2016 + 64 * 1000 * w, 64 - 64 * w]) / (64 + 64 * w)
        assert np.abs(got - want).max() < 1e-12, f"W9 {form}: {got[0]} vs {want}"


ALL_PINS = [pin_dense_prefill, pin_dense_decode, pin_longdouble_bruteforce, pin_forms_agree, pin_mask_invariants,
            pin_uniform_scores, pin_dropped_mass, pin_split_invariance, pin_output_given_mask, pin_worked_examples,
            pin_sink_seed, pin_worked_example_sink_seed, pin_fp8_kv, pin_chunked_prefill, pin_worked_example_chunk,
            pin_input_widening, pin_rowmax_pot, pin_worked_example_rowmax_pot]


def run_all(lib=None):
    """Run every pin; return the names of those that failed."""
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:  # ValueError: the oracle refused or crashed a case
            failed.append((pin.__name__, str(e)[:200]))
    return failed
