"""HIP prefill vs the fp64 oracle, element by element (GPU)."""
import math

import numpy as np
import pytest

import synth
from parity import check_prefill, log

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu


def _data(w, **kw):
    return synth.gen_prefill(synth.replace(w, **kw) if kw else w)


@pytest.mark.parametrize("tau", [-LN1000, -math.inf])
@pytest.mark.parametrize("tile_q", [64, 128])
def test_tiny_prefill(tau, tile_q):
    w = synth.TINY_PREFILL
    r = check_prefill(_data(w), B=w.B, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=tau, tile_q=tile_q,
                      where=f"tiny tq{tile_q}")
    if tau == -LN1000 and tile_q == 64:
        assert r["sparsity"] > 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("S", [1, 63, 65, 200, 1000])
def test_ragged_lengths(d, causal, S):
    """Sequence lengths that leave partial query and key tiles, incl. a single token."""
    w = synth.replace(synth.PREFILL_16K, S=S, Hq=8, Hkv=2, d=d, rank=8, seed=77)
    for tile_q in (64, 128):
        check_prefill(_data(w), B=1, S=S, Hq=8, Hkv=2, d=d, causal=causal, tau=-LN1000, tile_q=tile_q,
                      where=f"ragged S={S} d={d} causal={causal} tq={tile_q}")


@pytest.mark.parametrize("tau", [-math.inf, -math.log(100.0), -LN1000, -2.0, 0.0])
def test_llama_shape_2k(tau):
    """64 query heads / 8 KV heads (exercises the XCD-aware unit order), several dozen key tiles."""
    w = synth.replace(synth.PREFILL_16K, S=2048, seed=2048)
    check_prefill(_data(w), B=1, S=2048, Hq=64, Hkv=8, d=128, causal=True, tau=tau, tile_q=128,
                  where=f"llama 2k tau={tau}")


def test_batch2_noncausal_gqa4():
    w = synth.replace(synth.PREFILL_16K, B=2, S=777, Hq=16, Hkv=4, d=128, seed=5)
    check_prefill(_data(w), B=2, S=777, Hq=16, Hkv=4, d=128, causal=False, tau=-4.0, tile_q=128,
                  where="b2 noncausal")


def test_prefill_16k_sampled():
    """The 16K workload at full size; the oracle checks sampled units (first, last and spread q-tiles)."""
    w = synth.PREFILL_16K
    data = synth.gen_prefill(w)
    nqt = w.S // 128
    rng = np.random.default_rng(3)
    heads = rng.choice(w.Hq, 6, replace=False)
    qts = [0, 1, nqt // 2, nqt - 1]
    units = np.array([h * nqt + qt for h in heads for qt in qts])
    for tau in w.taus:
        r = check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=tau, tile_q=128, units=units,
                          where=f"16k tau={tau}")
        log(f"16k tau={tau}: sparsity {r['sparsity']:.3f}")


def test_prefill_128k_sampled():
    """The 128K benchmark workload in the launch configuration the benchmark times; the oracle checks
    sampled units including the first and the longest query tiles."""
    w = synth.PREFILL_128K
    data = synth.gen_prefill(w)
    nqt = w.S // 128
    units = np.array([0 * nqt + 0, 9 * nqt + 1, 17 * nqt + 255, 33 * nqt + 512, 40 * nqt + 777, 63 * nqt + nqt - 1,
                      5 * nqt + nqt - 2, 58 * nqt + 1000])
    r = check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=w.taus[0], tile_q=128,
                      units=units, where="128k")
    assert r["sparsity"] >= 0.45, "the calibrated workload skips about half of its tiles"


def test_prefill_128k_dense_sampled():
    """The same workload at tau = -inf (the dense launch the benchmark times for its speedup): no tile skipped,
    sampled units against the oracle."""
    w = synth.PREFILL_128K
    data = synth.gen_prefill(w)
    nqt = w.S // 128
    units = np.array([0 * nqt + 0, 21 * nqt + 300, 63 * nqt + nqt - 1])
    r = check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=-math.inf, tile_q=128,
                      units=units, where="128k dense")
    assert r["sparsity"] == 0.0


def test_batch3_causal_gqa2_odd_length():
    w = synth.replace(synth.PREFILL_16K, B=3, S=515, Hq=8, Hkv=4, d=64, seed=8)
    check_prefill(_data(w), B=3, S=515, Hq=8, Hkv=4, d=64, causal=True, tau=-LN1000, tile_q=64,
                  where="b3 causal gqa2")


def test_strided_views_match_contiguous():
    """q/k/v/out as views into wider buffers (row strides padded by 16 elements, heads interleaved with a gap):
    the kernels address through the descriptors' strides, so the outputs equal the contiguous run bit for bit."""
    import torch
    import long_context_flash_amd as ssm
    w = synth.replace(synth.PREFILL_16K, S=700, Hq=8, Hkv=2, d=128, seed=12)
    data = _data(w)
    dev = "cuda"
    q, k, v = (ssm.bf16_from_bits(data[x], dev) for x in ("q", "k", "v"))
    ref = ssm.ssm_prefill(q, k, v, causal=True, tau=-LN1000)

    def padded(t):
        B, S, H, d = t.shape
        big = torch.zeros(B, S, H + 1, d + 16, dtype=t.dtype, device=dev)
        view = big[:, :, :H, :d]
        view.copy_(t)
        return view

    qv, kv, vv = padded(q), padded(k), padded(v)
    out = padded(torch.zeros_like(q))
    assert qv.stride(1) == 9 * 144 and not qv.is_contiguous()
    ssm.ssm_prefill(qv, kv, vv, causal=True, tau=-LN1000, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "strided views changed the result"


@pytest.mark.parametrize("scale", [0.05, 0.3])
def test_custom_logit_scale(scale):
    """A logit scale other than 1/sqrt(d) (opts.scale) on both sides: the gaps, the decisions and the outputs
    follow it (0.05 flattens the scores, 0.3 sharpens them)."""
    w = synth.replace(synth.PREFILL_16K, S=700, Hq=8, Hkv=2, d=128, rank=8, seed=31)
    r = check_prefill(_data(w), B=1, S=700, Hq=8, Hkv=2, d=128, causal=True, tau=-math.log(100.0), tile_q=128,
                      scale=scale, where=f"prefill scale={scale}")
    if scale == 0.3:
        assert r["sparsity"] > 0
