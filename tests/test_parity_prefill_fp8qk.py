"""HIP prefill with 8-bit queries and keys (ssm_prefill_fp8qk) vs the fp64 oracle on the same codes (GPU).

q and k are quantised to OCP e4m3 codes with one amax/448 scale each (synth.fp8_qk); the oracle scores the
dequantised values (torch's float8_e4m3fn decoding times the scales) in fp64 with the bf16 values, so both
sides compute the method on identical inputs and only the arithmetic differs."""
import math

import numpy as np
import pytest

import synth
from parity import check_prefill, log

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu


def _case(w):
    data = synth.gen_prefill(w)
    return data, synth.fp8_qk(data)


@pytest.mark.parametrize("tau", [-LN1000, -math.inf])
@pytest.mark.parametrize("tile_q", [64, 128])
def test_tiny(tau, tile_q):
    w = synth.TINY_PREFILL
    data, f8 = _case(w)
    r = check_prefill(data, B=w.B, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=tau, tile_q=tile_q,
                      fp8qk=f8, where=f"fp8qk tiny tq{tile_q}")
    if tau == -LN1000 and tile_q == 64:
        assert r["sparsity"] > 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [1, 63, 65, 200, 1000])
def test_ragged_lengths(d, causal, S):
    """Partial query and key tiles, a single token, both head sizes and both query tiles."""
    w = synth.replace(synth.PREFILL_16K, S=S, Hq=8, Hkv=2, d=d, rank=8, seed=78)
    data, f8 = _case(w)
    for tile_q in (64, 128):
        check_prefill(data, B=1, S=S, Hq=8, Hkv=2, d=d, causal=causal, tau=-LN1000, tile_q=tile_q, fp8qk=f8,
                      where=f"fp8qk ragged S={S} d={d} causal={causal} tq={tile_q}")


@pytest.mark.parametrize("tau", [-math.inf, -math.log(100.0), -LN1000, 0.0])
def test_llama_shape_2k(tau):
    w = synth.replace(synth.PREFILL_16K, S=2048, seed=2049)
    data, f8 = _case(w)
    check_prefill(data, B=1, S=2048, Hq=64, Hkv=8, d=128, causal=True, tau=tau, tile_q=128, fp8qk=f8,
                  where=f"fp8qk llama 2k tau={tau}")


def test_batch2_noncausal_gqa4():
    w = synth.replace(synth.PREFILL_16K, B=2, S=777, Hq=16, Hkv=4, d=128, seed=6)
    data, f8 = _case(w)
    check_prefill(data, B=2, S=777, Hq=16, Hkv=4, d=128, causal=False, tau=-4.0, tile_q=128, fp8qk=f8,
                  where="fp8qk b2 noncausal")


def test_prefill_128k_sampled():
    """The 128K benchmark workload with 8-bit q/k, in the launch configuration the benchmark's fp8 leg times;
    the oracle checks sampled units including the first and the longest query tiles."""
    w = synth.PREFILL_128K
    data, f8 = _case(w)
    nqt = w.S // 128
    units = np.array([0 * nqt + 0, 9 * nqt + 1, 33 * nqt + 512, 63 * nqt + nqt - 1, 58 * nqt + 1000])
    r = check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=w.taus[0], tile_q=128,
                      units=units, fp8qk=f8, where="fp8qk 128k")
    log(f"fp8qk 128k: sparsity {r['sparsity']:.3f}")
    assert r["sparsity"] >= 0.45


def test_strided_views_match_contiguous():
    """e4m3 q/k and bf16 v/out as views into wider buffers (rows padded by 32 elements, one spare head): the
    same bits as contiguous tensors."""
    import torch
    import long_context_flash_amd as ssm
    from parity import fp8_device
    w = synth.replace(synth.PREFILL_16K, S=600, Hq=8, Hkv=2, d=128, seed=13)
    data, f8 = _case(w)
    dev = "cuda"
    q8, k8 = fp8_device(f8["q"], dev), fp8_device(f8["k"], dev)
    v = ssm.bf16_from_bits(data["v"], dev)
    ref = ssm.ssm_prefill_fp8qk(q8, f8["q_scale"], k8, f8["k_scale"], v, causal=True, tau=-LN1000)

    def padded(t):
        B, S, H, d = t.shape
        big = torch.zeros(B, S, H + 1, d + 32, dtype=torch.uint8 if t.dtype == torch.float8_e4m3fn else t.dtype,
                          device=dev)
        if t.dtype == torch.float8_e4m3fn:
            big = big.view(torch.float8_e4m3fn)
        view = big[:, :, :H, :d]
        view.copy_(t)
        return view

    out = padded(torch.zeros(ref.shape, dtype=ref.dtype, device=dev))
    ssm.ssm_prefill_fp8qk(padded(q8), f8["q_scale"], padded(k8), f8["k_scale"], padded(v), causal=True, tau=-LN1000,
                          out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "strided views changed the result"
