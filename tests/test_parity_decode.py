"""HIP split-K decode vs the fp64 oracle (GPU)."""
import math

import numpy as np
import pytest

import synth
from parity import check_decode, run_decode_gpu, errors

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(B=3, Hq=16, Hkv=2, d=128, kv_len=0, kv_len_lo=900, kv_len_hi=5000, seed=9)
    base.update(kw)
    return synth.replace(synth.DECODE_32K, **base)


@pytest.mark.parametrize("P", [1, 4, 16])
@pytest.mark.parametrize("tau", [-LN1000, -math.inf, -4.0])
def test_small_contiguous(P, tau):
    data = synth.gen_decode(_small(), contiguous=True, paged=False)
    check_decode(data, tau=tau, num_splits=P, paged=False, where=f"small contig P={P} tau={tau}")


@pytest.mark.parametrize("P", [1, 16])
def test_small_paged_matches_contiguous(P):
    data = synth.gen_decode(_small(), contiguous=True, paged=True)
    a = check_decode(data, tau=-LN1000, num_splits=P, paged=True, where=f"small paged P={P}")
    b = run_decode_gpu(data, tau=-LN1000, num_splits=P, paged=False)
    assert np.array_equal(a["out"], b[0]), "paged and contiguous layouts must give identical outputs"
    assert np.array_equal(a["state"][:, :b[1].shape[1]], b[1])


def test_kv_len_edge_cases():
    """kv_len 0, 1, 63, 64, 65, 129 with 16 splits (many empty splits)."""
    w = _small(B=6, Hq=8, Hkv=1)
    lens = np.array([0, 1, 63, 64, 65, 129], np.int32)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=True)
    for paged in (False, True):
        r = check_decode(data, tau=-LN1000, num_splits=16, paged=paged, where=f"edge paged={paged}")
        assert np.all(r["out"][0] == 0), "kv_len 0 gives a zero output"


@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_group_sizes_d64(G):
    w = _small(Hq=2 * G, Hkv=2, d=64, seed=10 + G)
    data = synth.gen_decode(w, contiguous=True, paged=False)
    check_decode(data, tau=-LN1000, num_splits=8, paged=False, where=f"d64 G={G}")


@pytest.mark.parametrize("paged", [False, True])
def test_largest_group_and_split_count(paged):
    """The largest supported configuration per unit: 16 query heads per KV head at d = 128 and 64 splits (the
    upper bound of num_splits), kv_len from 1 to 9000 (from more splits than tiles to 2-3 tiles per split),
    split-local and sink-seeded."""
    w = _small(B=4, Hq=32, Hkv=2, d=128, seed=21)
    lens = np.array([1, 700, 4097, 9000], np.int32)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=True)
    for seeded in (False, True):
        for tau in (-LN1000, -1.0):  # -1: a split of 2-3 tiles skips too
            r = check_decode(data, tau=tau, num_splits=64, paged=paged, sink_seed=seeded,
                             where=f"G16 d128 P64 paged={paged} seeded={seeded} tau={tau}")
            if tau == -1.0:
                assert r["sparsity"] > 0.05, "the case must exercise the skip path"


def test_decode_32k_full():
    """The 32K workload at full size, split-K (16) and the sequential definition (1 split)."""
    w = synth.DECODE_32K
    data = synth.gen_decode(w)
    for P in (16, 1):
        check_decode(data, tau=w.taus[0], num_splits=P, paged=False, where=f"32k P={P}")


def test_decode_128k_paged_sampled():
    """The 128K paged workload (random page table, variable lengths) at the calibrated taus; the oracle
    checks four sequences."""
    w = synth.DECODE_128K
    data = synth.gen_decode(w)
    batches = np.array([0, 7, 19, 31])
    for tau in w.taus:
        check_decode(data, tau=tau, num_splits=w.num_splits, paged=True, batches=batches, where=f"128k tau={tau}")


def test_decode_b256_paged_sampled():
    """256 sequences (kv_len 8K-16K, paged, as many keys as the 128K workload) in one call: the ordering kernel's
    longest-first dispatch over a large batch; the oracle checks the longest, the shortest and four others."""
    w = synth.DECODE_B256
    data = synth.gen_decode(w)
    order = np.argsort(-data["kv_lens"], kind="stable")
    batches = np.unique([order[0], order[-1], 3, 100, 177, 255])
    check_decode(data, tau=w.taus[0], num_splits=w.num_splits, paged=True, batches=batches, where="B=256 paged")


def test_batch_beyond_dispatch_sort():
    """Batches above 8192 sequences skip the longest-first dispatch order (plain workgroup order, no order array
    in the workspace): the outputs of such a batch equal those of its first 8192 sequences run as a sorted batch
    bit for bit, and a sample of its sequences (both sides of the 8192 boundary) agrees with the oracle."""
    import torch
    import long_context_flash_amd as ssm
    B, SORT_MAX = 8200, 8192
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 200, size=B).astype(np.int32)
    w = _small(B=B, Hq=8, Hkv=1, d=64, seed=77)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=False)
    sample = np.array([0, 1, 500, 4097, 8191, 8192, 8193, 8199])
    r = check_decode(data, tau=-LN1000, num_splits=4, paged=False, batches=sample, where="B=8200 unsorted dispatch")
    dev = "cuda"
    q = ssm.bf16_from_bits(data["q"][:SORT_MAX], dev)
    kc = ssm.bf16_from_bits(data["k_cache"][:SORT_MAX], dev)
    vc = ssm.bf16_from_bits(data["v_cache"][:SORT_MAX], dev)
    out = ssm.ssm_decode(q, kc, vc, torch.from_numpy(lens[:SORT_MAX]).to(dev), tau=-LN1000, num_splits=4)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), r["out"][:SORT_MAX]), "dispatch order changed the outputs"


def test_strided_query_and_output_match_contiguous():
    """q and out as views with padded head and batch strides give the same bits as contiguous tensors."""
    import torch
    import long_context_flash_amd as ssm
    data = synth.gen_decode(_small(B=2, Hq=16, Hkv=2, d=128, seed=21), contiguous=True, paged=False)
    dev = "cuda"
    q = ssm.bf16_from_bits(data["q"], dev)
    kc, vc = ssm.bf16_from_bits(data["k_cache"], dev), ssm.bf16_from_bits(data["v_cache"], dev)
    lens = torch.from_numpy(data["kv_lens"]).to(dev)
    ref = ssm.ssm_decode(q, kc, vc, lens, tau=-LN1000, num_splits=8)
    big_q = torch.zeros(2, 20, 144, dtype=q.dtype, device=dev)
    qv = big_q[:, :16, :128]
    qv.copy_(q)
    big_o = torch.zeros(2, 20, 144, dtype=q.dtype, device=dev)
    ov = big_o[:, :16, :128]
    ssm.ssm_decode(qv, kc, vc, lens, tau=-LN1000, num_splits=8, out=ov)
    torch.cuda.synchronize()
    assert torch.equal(ov, ref), "strided q/out changed the result"


def test_separate_value_page_table_matches_shared():
    """V pages under their own page table (the pool permuted differently from K's) give the same bits as one
    shared table: each cache is addressed through its own table."""
    import torch
    import long_context_flash_amd as ssm
    w = _small()
    data = synth.gen_decode(w, contiguous=False, paged=True)
    dev = "cuda"
    pt = data["page_table"]
    sigma = np.random.default_rng(5).permutation(data["v_pool"].shape[0]).astype(np.int32)
    v_pool2 = np.empty_like(data["v_pool"])
    v_pool2[sigma] = data["v_pool"]                      # page p of the old pool is page sigma[p] of the new one
    v_pt2 = np.where(pt >= 0, sigma[np.maximum(pt, 0)], pt).astype(np.int32)
    q = ssm.bf16_from_bits(data["q"], dev)
    kp, vp = ssm.bf16_from_bits(data["k_pool"], dev), ssm.bf16_from_bits(data["v_pool"], dev)
    vp2 = ssm.bf16_from_bits(v_pool2, dev)
    lens = torch.from_numpy(data["kv_lens"]).to(dev)
    pt_d, v_pt2_d = torch.from_numpy(pt).to(dev), torch.from_numpy(v_pt2).to(dev)
    for seeded in (False, True):
        ref = ssm.ssm_decode(q, kp, vp, lens, tau=-4.0, page_table=pt_d, num_splits=8, sink_seed=seeded)
        got = ssm.ssm_decode(q, kp, vp2, lens, tau=-4.0, page_table=pt_d, v_page_table=v_pt2_d, num_splits=8,
                             sink_seed=seeded)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"separate V page table changed the output (seeded={seeded})"


@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_custom_logit_scale(scale):
    """A logit scale other than 1/sqrt(d) on both sides, contiguous and paged, split-local and seeded, and over
    an fp8 cache."""
    data = synth.gen_decode(_small(seed=32), contiguous=True, paged=True)
    for paged in (False, True):
        for seeded in (False, True):
            check_decode(data, tau=-4.0, num_splits=8, paged=paged, sink_seed=seeded, scale=scale,
                         where=f"decode scale={scale} paged={paged} seeded={seeded}")
    # over an fp8 cache the key scale multiplies the logit scale
    check_decode(data, tau=-4.0, num_splits=8, paged=True, scale=scale, fp8=synth.fp8_kv(data),
                 where=f"decode scale={scale} fp8")
