"""The seeded input generators (CPU only)."""
import math

import numpy as np
import torch

import oracle
import synth


def test_determinism_and_thread_independence():
    w = synth.replace(synth.PREFILL_16K, S=1024, Hq=16, Hkv=2)
    a = synth.gen_prefill(w, threads=1)
    b = synth.gen_prefill(w, threads=7)
    for key in ("q", "k", "v", "relevant"):
        assert np.array_equal(a[key], b[key]), key
    d = synth.replace(synth.DECODE_128K, B=2, kv_len_lo=300, kv_len_hi=5000)
    x = synth.gen_decode(d, contiguous=True, paged=True, threads=1)
    y = synth.gen_decode(d, contiguous=True, paged=True, threads=5)
    for key in ("q", "k_cache", "v_cache", "k_pool", "v_pool", "page_table", "kv_lens"):
        assert np.array_equal(x[key], y[key]), key


def test_seed_changes_values():
    w = synth.replace(synth.TINY_PREFILL)
    a = synth.gen_prefill(w)
    b = synth.gen_prefill(synth.replace(w, seed=w.seed + 1))
    assert not np.array_equal(a["q"], b["q"])


def test_bf16_rounding_matches_torch():
    w = synth.TINY_PREFILL
    a = synth.gen_prefill(w, fp32=True)
    ref = torch.from_numpy(a["q32"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref, a["q"])
    assert np.array_equal(synth.f32_to_bf16_bits(a["k32"]), a["k"])
    assert np.array_equal(synth.bf16_bits_to_f32(a["v"]),
                          torch.from_numpy(a["v32"]).to(torch.bfloat16).float().numpy())


def test_normal_moments():
    w = synth.replace(synth.PREFILL_16K, S=2048, Hq=8, Hkv=1, rank=0, sink_amp=0.0, rel_frac=0.0)
    a = synth.gen_prefill(w, bf16=False, fp32=True)
    v = a["v32"].astype(np.float64).ravel()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    # exact common mode mu = sqrt(d/G) along u (before bf16 rounding)
    k = synth.gen_prefill(synth.replace(w, rel_count=0), bf16=False, fp32=True)
    assert np.allclose(k["q32"], a["q32"])


def test_paged_and_contiguous_hold_same_tokens():
    d = synth.replace(synth.DECODE_128K, B=3, kv_len_lo=1, kv_len_hi=3000)
    x = synth.gen_decode(d, contiguous=True, paged=True)
    lens, pt = x["kv_lens"], x["page_table"]
    nt = -(-lens // 64)
    used = np.concatenate([pt[b, :nt[b]] for b in range(d.B)])
    assert np.array_equal(np.sort(used), np.arange(nt.sum())), "page table must be a permutation"
    for b in range(d.B):
        pool = x["k_pool"][pt[b, :nt[b]]].transpose(1, 0, 2, 3).reshape(d.Hkv, nt[b] * 64, d.d)
        assert np.array_equal(pool, x["k_cache"][b, :, :nt[b] * 64])
        vpool = x["v_pool"][pt[b, :nt[b]]].transpose(1, 0, 2, 3).reshape(d.Hkv, nt[b] * 64, d.d)
        assert np.array_equal(vpool, x["v_cache"][b, :, :nt[b] * 64])
        assert not x["k_cache"][b, :, lens[b]:].any(), "tokens past kv_len must be zero"


def test_kv_lens_range():
    lens = synth.kv_lens_for(synth.DECODE_128K)
    assert lens.min() >= 65536 and lens.max() <= 131072 and len(lens) == 32
    assert len(set(lens.tolist())) > 20


def test_sink_shift_direction_decode():
    """Sink keys are shifted along the group's mean query direction by 4*sqrt(d) (about +16 logits)."""
    d = synth.replace(synth.DECODE_32K, B=1, kv_len=2048, rel_frac=0.0)
    x = synth.gen_decode(d, fp32=True)
    q = x["q32"][0].astype(np.float64)
    k = x["k32"][0].astype(np.float64)
    G = d.Hq // d.Hkv
    logits_sink = np.einsum("hd,jd->hj", q[:G], k[0, :64]) / math.sqrt(d.d)
    logits_rest = np.einsum("hd,jd->hj", q[:G], k[0, 64:]) / math.sqrt(d.d)
    assert 12 < logits_sink.mean() - logits_rest.mean() < 20


def test_tiny_workload_has_skipped_and_kept_tiles():
    w = synth.TINY_PREFILL
    a = synth.gen_prefill(w)
    r = oracle.prefill(a["q"], a["k"], a["v"], causal=True, tau=-math.log(1000.0), tile_q=w.tile_q,
                       tile_k=w.tile_k)
    st = r["state"]
    assert (st == oracle.SKIPPED).sum() >= 1
    assert (st[:, 1:] == oracle.EXECUTED).sum() >= 1
