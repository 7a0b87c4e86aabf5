"""HIP chunked prefill against a paged KV cache (ragged batch, bottom-right causal) vs the fp64 oracle (GPU)."""
import math

import numpy as np
import pytest

import synth
from parity import chunk_batch, check_prefill_paged, fp8_pools, fp8_q_packed, run_prefill_paged_gpu

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu

SMALL = synth.replace(synth.PREFILL_16K, S=0, Hq=8, Hkv=2, rank=8, seed=300)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile_q", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_batch(d, tile_q, causal):
    """Chunks of 1, 63, 129 and 300 queries after prefixes that are and are not multiples of 64, a whole-sequence
    chunk (no prefix) and an empty one."""
    w = synth.replace(SMALL, d=d)
    seqs = [(129, 700), (1, 65), (300, 300), (63, 1000), (0, 77), (200, 263)]
    cb = chunk_batch(w, seqs, seed=1)
    for tau in (-LN1000, -math.inf):
        check_prefill_paged(cb, Hq=w.Hq, causal=causal, tau=tau, tile_q=tile_q,
                            where=f"chunked d={d} tq={tile_q} causal={causal} tau={tau}")


def test_whole_sequence_chunk_matches_prefill():
    """A chunk holding every position of a sequence is the plain prefill: same decisions, same output."""
    import long_context_flash_amd as ssm
    import torch
    w = synth.replace(SMALL, d=128)
    cb = chunk_batch(w, [(512, 512)], seed=2)
    out_p, st_p, _, _ = run_prefill_paged_gpu(cb, Hq=w.Hq, causal=True, tau=-LN1000, tile_q=128)
    dat = cb["per"][0]
    q, k, v = (ssm.bf16_from_bits(dat[x], "cuda") for x in ("q", "k", "v"))
    stats = ssm.SkipStats.alloc(*ssm.prefill_stats_shape(1, 512, w.Hq, 128), "cuda")
    out = ssm.ssm_prefill(q, k, v, causal=True, tau=-LN1000, skip_stats=stats, tile_q=128)
    torch.cuda.synchronize()
    assert np.array_equal(out[0].float().cpu().numpy(), out_p)
    assert np.array_equal(stats.tile_state.cpu().numpy(), st_p)


def test_llama_shape_long_context_chunk():
    """64 query / 8 KV heads, d = 128: a 2K chunk after a 14K prefix and a 1K chunk after a 3K prefix."""
    w = synth.replace(synth.PREFILL_16K, S=0, seed=310)
    cb = chunk_batch(w, [(2048, 16384), (1024, 4096)], seed=3)
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[2], tile_q=128, where="chunked llama 16k")
    assert r["sparsity"] > 0.3


def test_chunk_8k_of_128k_sampled():
    """The benchmark's chunked workload: the last 8192 queries of the 128K prefill input against all 131072
    keys in a paged pool; the oracle checks sampled units (the first and last query tiles among them)."""
    w = synth.PREFILL_128K
    cb = chunk_batch(w, [(8192, w.S)], seed=4)
    sample = {0: [(0, 0), (9, 1), (17, 31), (40, 62), (63, 63)]}
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[0], tile_q=128, sample=sample,
                            where="chunked 8k of 128k")
    assert r["sparsity"] > 0.3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile_q", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_batch_fp8_cache(d, tile_q, causal):
    """The ragged batch over an fp8 e4m3 cache (amax/448 scales, the pools a decode reads); the oracle reads
    the dequantised pools."""
    w = synth.replace(SMALL, d=d)
    seqs = [(129, 700), (1, 65), (300, 300), (63, 1000), (0, 77), (200, 263)]
    cb = chunk_batch(w, seqs, seed=5)
    f8 = fp8_pools(cb)
    for tau in (-LN1000, -math.inf):
        check_prefill_paged(cb, Hq=w.Hq, causal=causal, tau=tau, tile_q=tile_q, fp8=f8,
                            where=f"chunked fp8 d={d} tq={tile_q} causal={causal} tau={tau}")


def test_llama_shape_long_context_chunk_fp8_cache():
    w = synth.replace(synth.PREFILL_16K, S=0, seed=311)
    cb = chunk_batch(w, [(2048, 16384), (1024, 4096)], seed=6)
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[2], tile_q=128, fp8=fp8_pools(cb),
                            where="chunked fp8 llama 16k")
    assert r["sparsity"] > 0.3


def test_chunk_8k_of_128k_sampled_fp8_cache():
    """The benchmark's chunked workload over an fp8 cache; sampled units."""
    w = synth.PREFILL_128K
    cb = chunk_batch(w, [(8192, w.S)], seed=4)
    sample = {0: [(0, 0), (17, 31), (63, 63)]}
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[0], tile_q=128, sample=sample, fp8=fp8_pools(cb),
                            where="chunked fp8 8k of 128k")
    assert r["sparsity"] > 0.3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile_q", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_batch_fp8_qk(d, tile_q, causal):
    """The ragged batch with 8-bit queries (amax/448 scale) scored on the fp8 MFMA against the fp8 pools; the
    oracle reads the dequantised queries and pools."""
    w = synth.replace(SMALL, d=d)
    seqs = [(129, 700), (1, 65), (300, 300), (63, 1000), (0, 77), (200, 263)]
    cb = chunk_batch(w, seqs, seed=7)
    f8, f8q = fp8_pools(cb), fp8_q_packed(cb)
    for tau in (-LN1000, -math.inf):
        check_prefill_paged(cb, Hq=w.Hq, causal=causal, tau=tau, tile_q=tile_q, fp8=f8, fp8q=f8q,
                            where=f"chunked fp8qk d={d} tq={tile_q} causal={causal} tau={tau}")


def test_llama_shape_long_context_chunk_fp8_qk():
    w = synth.replace(synth.PREFILL_16K, S=0, seed=312)
    cb = chunk_batch(w, [(2048, 16384), (1024, 4096)], seed=8)
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[2], tile_q=128, fp8=fp8_pools(cb),
                            fp8q=fp8_q_packed(cb), where="chunked fp8qk llama 16k")
    assert r["sparsity"] > 0.3


def test_chunk_8k_of_128k_sampled_fp8_qk():
    """The benchmark's chunked workload with 8-bit queries over an fp8 cache; sampled units."""
    w = synth.PREFILL_128K
    cb = chunk_batch(w, [(8192, w.S)], seed=4)
    sample = {0: [(0, 0), (17, 31), (40, 62), (63, 63)]}
    r = check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=w.taus[0], tile_q=128, sample=sample, fp8=fp8_pools(cb),
                            fp8q=fp8_q_packed(cb), where="chunked fp8qk 8k of 128k")
    assert r["sparsity"] > 0.3


def test_fp8_qk_whole_sequence_chunk_matches_plain_fp8qk_prefill_decisions():
    """A whole-sequence chunk with 8-bit queries over 8-bit pages takes the same skip decisions as the
    non-paged 8-bit-score prefill on the same q/k codes (the scores are the same fp8 products; only V differs,
    e4m3 pages here and bf16 there)."""
    import long_context_flash_amd as ssm
    import torch
    from parity import fp8_device
    w = synth.replace(SMALL, d=128)
    cb = chunk_batch(w, [(512, 512)], seed=9)
    f8, f8q = fp8_pools(cb), fp8_q_packed(cb)
    _, st_p, _, _ = run_prefill_paged_gpu(cb, Hq=w.Hq, causal=True, tau=-LN1000, tile_q=128, fp8=f8, fp8q=f8q)
    # the same k codes as the pool, in [1, S, Hkv, d] order
    pages = cb["page_table"][0, :8]
    k8 = np.ascontiguousarray(f8["k_pool"][pages].transpose(0, 2, 1, 3).reshape(1, 512, w.Hkv, w.d))
    q8 = fp8_device(f8q["q"][None], "cuda")
    v = ssm.bf16_from_bits(cb["per"][0]["v"], "cuda")
    stats = ssm.SkipStats.alloc(*ssm.prefill_stats_shape(1, 512, w.Hq, 128), "cuda")
    ssm.ssm_prefill_fp8qk(q8, f8q["q_scale"], fp8_device(k8, "cuda"), f8["k_scale"], v, causal=True, tau=-LN1000,
                          skip_stats=stats, tile_q=128)
    torch.cuda.synchronize()
    assert np.array_equal(stats.tile_state.cpu().numpy(), st_p)


@pytest.mark.parametrize("mode", ["bf16", "fp8_cache", "fp8_qk"])
def test_strided_views_match_contiguous(mode):
    """q, out and both pools as views into wider buffers (rows padded by 32 elements, one spare head): the
    same output bits and tile states as contiguous tensors, for bf16 pages, fp8 pages and 8-bit queries."""
    import long_context_flash_amd as ssm
    import torch
    from parity import fp8_device
    w = synth.replace(SMALL, d=128)
    cb = chunk_batch(w, [(129, 700), (1, 65), (300, 300), (200, 263)], seed=10)
    f8 = fp8_pools(cb) if mode != "bf16" else None
    f8q = fp8_q_packed(cb) if mode == "fp8_qk" else None
    dev = "cuda"
    if f8q is not None:
        q = fp8_device(f8q["q"], dev)
    else:
        q = ssm.bf16_from_bits(cb["q"], dev)
    if f8 is not None:
        kc, vc = fp8_device(f8["k_pool"], dev), fp8_device(f8["v_pool"], dev)
        scales = dict(k_scale=f8["k_scale"], v_scale=f8["v_scale"])
    else:
        kc, vc = ssm.bf16_from_bits(cb["k_pool"], dev), ssm.bf16_from_bits(cb["v_pool"], dev)
        scales = {}
    pt = torch.from_numpy(cb["page_table"]).to(dev)
    qs = torch.from_numpy(cb["q_start"]).to(dev)
    kl = torch.from_numpy(cb["kv_lens"]).to(dev)
    B, nqt = len(cb["seqs"]), -(-cb["max_q"] // 128)

    def padded(t, head_dim):
        """a view of t inside a buffer with one more head (dim head_dim) and 32 more elements per row"""
        shape = list(t.shape)
        shape[head_dim] += 1
        shape[-1] += 32
        raw = torch.zeros(shape, dtype=torch.uint8 if t.dtype == torch.float8_e4m3fn else t.dtype, device=dev)
        big = raw.view(torch.float8_e4m3fn) if t.dtype == torch.float8_e4m3fn else raw
        idx = [slice(None)] * t.dim()
        idx[head_dim] = slice(0, t.shape[head_dim])
        idx[-1] = slice(0, t.shape[-1])
        view = big[tuple(idx)]
        view.copy_(t)
        return view

    def run(q_, kc_, vc_, out_):
        stats = ssm.SkipStats.alloc(B * w.Hq * nqt, pt.shape[1], dev, gaps=True)
        if f8q is not None:
            ssm.ssm_prefill_paged_fp8qk(q_, f8q["q_scale"], kc_, vc_, pt, qs, kl, cb["max_q"], causal=True,
                                        tau=-LN1000, out=out_, skip_stats=stats, **scales)
        else:
            ssm.ssm_prefill_paged(q_, kc_, vc_, pt, qs, kl, cb["max_q"], causal=True, tau=-LN1000, out=out_,
                                  skip_stats=stats, **scales)
        torch.cuda.synchronize()
        return out_.float().cpu().numpy(), stats.tile_state.cpu().numpy()

    out_c, st_c = run(q, kc, vc, torch.zeros(q.shape, dtype=torch.bfloat16, device=dev))
    out_v = padded(torch.zeros(q.shape, dtype=torch.bfloat16, device=dev), 1)
    out_s, st_s = run(padded(q, 1), padded(kc, 1), padded(vc, 1), out_v)
    assert (st_c == 2).any(), "no tile skipped: the case does not exercise the skip path"
    assert np.array_equal(st_s, st_c), "strided views changed the decisions"
    assert np.array_equal(out_s, out_c), "strided views changed the result"


def test_separate_value_page_table_matches_shared():
    """The chunked prefill with V pages under their own page table gives the same bits as one shared table."""
    import long_context_flash_amd as ssm
    import torch
    w = synth.replace(SMALL, d=128)
    cb = chunk_batch(w, [(129, 700), (300, 300), (63, 1000)], seed=11)
    dev = "cuda"
    pt = cb["page_table"]
    sigma = np.random.default_rng(6).permutation(cb["v_pool"].shape[0]).astype(np.int32)
    v_pool2 = np.empty_like(cb["v_pool"])
    v_pool2[sigma] = cb["v_pool"]
    v_pt2 = np.where(pt >= 0, sigma[np.maximum(pt, 0)], pt).astype(np.int32)
    q = ssm.bf16_from_bits(cb["q"], dev)
    kp, vp = ssm.bf16_from_bits(cb["k_pool"], dev), ssm.bf16_from_bits(cb["v_pool"], dev)
    vp2 = ssm.bf16_from_bits(v_pool2, dev)
    qs, kl = torch.from_numpy(cb["q_start"]).to(dev), torch.from_numpy(cb["kv_lens"]).to(dev)
    pt_d, v_pt2_d = torch.from_numpy(pt).to(dev), torch.from_numpy(v_pt2).to(dev)
    ref = ssm.ssm_prefill_paged(q, kp, vp, pt_d, qs, kl, cb["max_q"], tau=-LN1000)
    got = ssm.ssm_prefill_paged(q, kp, vp2, pt_d, qs, kl, cb["max_q"], tau=-LN1000, v_page_table=v_pt2_d)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), "separate V page table changed the output"


def test_empty_inputs_are_no_ops():
    """Empty torch tensors (NULL data) through every entry point: nothing launched, no error, outputs untouched."""
    import long_context_flash_amd as ssm
    import torch
    dev = "cuda"
    bf, f8 = torch.bfloat16, torch.float8_e4m3fn
    q = torch.empty(1, 0, 8, 128, dtype=bf, device=dev)
    kv = torch.empty(1, 0, 2, 128, dtype=bf, device=dev)
    assert ssm.ssm_prefill(q, kv, kv).shape == (1, 0, 8, 128)
    assert ssm.ssm_prefill_fp8qk(q.to(f8), 1.0, kv.to(f8), 1.0, kv).shape == (1, 0, 8, 128)
    pool = torch.zeros(4, 2, 64, 128, dtype=bf, device=dev)
    lens0 = torch.empty(0, dtype=torch.int32, device=dev)
    out = ssm.ssm_decode(torch.empty(0, 8, 128, dtype=bf, device=dev), pool, pool, lens0,
                         page_table=torch.empty(0, 4, dtype=torch.int32, device=dev))
    assert out.shape == (0, 8, 128)
    # a batch of chunks with no queries at all, and an empty batch
    pt = torch.zeros(2, 4, dtype=torch.int32, device=dev)
    qs = torch.zeros(3, dtype=torch.int32, device=dev)
    kl = torch.full((2,), 100, dtype=torch.int32, device=dev)
    q0 = torch.empty(0, 8, 128, dtype=bf, device=dev)
    assert ssm.ssm_prefill_paged(q0, pool, pool, pt, qs, kl, 0).shape == (0, 8, 128)
    assert ssm.ssm_prefill_paged_fp8qk(q0.to(f8), 1.0, pool.to(f8), pool.to(f8), pt, qs, kl, 0, 1.0, 1.0).shape == \
        (0, 8, 128)
    assert ssm.ssm_prefill_paged(q0, pool, pool, torch.empty(0, 4, dtype=torch.int32, device=dev),
                                 torch.zeros(1, dtype=torch.int32, device=dev), lens0, 0).shape == (0, 8, 128)
    torch.cuda.synchronize()


@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_custom_logit_scale(scale):
    """A logit scale other than 1/sqrt(d) (opts.scale) through the chunked prefill, bf16 and fp8 pages."""
    w = synth.replace(SMALL, d=128)
    cb = chunk_batch(w, [(129, 700), (300, 300), (63, 1000)], seed=12)
    for f8 in (None, fp8_pools(cb)):
        check_prefill_paged(cb, Hq=w.Hq, causal=True, tau=-math.log(100.0), tile_q=128, fp8=f8, scale=scale,
                            where=f"chunked scale={scale} fp8={f8 is not None}")
