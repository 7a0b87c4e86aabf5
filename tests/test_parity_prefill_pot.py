"""HIP prefill with Rowmax-PoT weights vs the fp64 oracle's Rowmax-PoT prefill (GPU).

Rowmax-PoT ("Approximating Softmax in Pretrained LLMs: Model Sensitivity and Kernel Acceleration", Abstract):
each kept key's weight is 2^(rint(log2(e) l) - rint(log2(e) mu)).  The rounding decides an integer from a
floating-point value, so the comparison has two parts:
  * designed inputs whose base-2 log weights sit at least 0.05 from every half-integer (integer q.k with the
    logit scale ln 2, optionally moved by less than 0.45): the kernel's fp32 scores cannot round differently, no
    row is ambiguous, and every row meets the plain bar;
  * seeded workload-shaped inputs: rows holding a key whose log weight lies within the kernel's error band of a
    half-integer are held to the bound that rounding can move them by (parity.pot_tie_bound), all others to the
    plain bar.
Both kernels are covered: the paired-head kernel (d = 128, 128-row tiles, even GQA groups) and the general one
(d = 64, 64-row tiles, odd groups), plus the fp8-score prefill."""
import math

import numpy as np
import pytest

import synth
from parity import check_prefill, log, run_prefill_gpu

LN1000 = math.log(1000.0)
LN2 = math.log(2.0)
pytestmark = pytest.mark.gpu

# (d, tile_q, Hq, Hkv): the first runs the paired-head kernel, the others the general one
SHAPES = [(128, 128, 8, 2), (128, 128, 6, 2), (128, 64, 8, 2), (64, 128, 4, 4), (64, 64, 6, 2)]


@pytest.mark.parametrize("d,tile_q,Hq,Hkv", SHAPES)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("offset", [0.0, 0.45])
def test_pot_designed_logits_no_ambiguous_row(d, tile_q, Hq, Hkv, causal, offset):
    """Integer q.k (entries -1..1) at logit scale ln 2: base-2 log weights are integers (offset 0) or within 0.45
    of one; S = 333 leaves partial query and key tiles."""
    S = 333
    data = synth.gen_integer_qk(40 + d + Hq, 1, S, Hq, Hkv, d, lo=-1, hi=1, offset=offset)
    for tau in (-math.inf, -2.0):
        r = check_prefill(data, B=1, S=S, Hq=Hq, Hkv=Hkv, d=d, causal=causal, tau=tau, tile_q=tile_q, scale=LN2,
                          weights="rowmax_pot", where=f"pot designed d={d} tq={tile_q} G={Hq // Hkv} off={offset} "
                                                      f"causal={causal} tau={tau}")
        assert r["ties"] == 0


@pytest.mark.parametrize("d,tile_q,Hq,Hkv", SHAPES)
@pytest.mark.parametrize("tau", [-math.inf, -LN1000, -2.0])
def test_pot_workload_inputs(d, tile_q, Hq, Hkv, tau):
    """The 16K workload's generator (low-rank queries and keys, sink and relevant tiles) at 1000 tokens."""
    w = synth.replace(synth.PREFILL_16K, S=1000, Hq=Hq, Hkv=Hkv, d=d, rank=8, seed=911)
    check_prefill(synth.gen_prefill(w), B=1, S=1000, Hq=Hq, Hkv=Hkv, d=d, causal=True, tau=tau, tile_q=tile_q,
                  weights="rowmax_pot", where=f"pot workload d={d} tq={tile_q} G={Hq // Hkv} tau={tau}")


def test_pot_batch2_noncausal():
    w = synth.replace(synth.PREFILL_16K, B=2, S=777, Hq=16, Hkv=4, d=128, seed=6)
    check_prefill(synth.gen_prefill(w), B=2, S=777, Hq=16, Hkv=4, d=128, causal=False, tau=-4.0, tile_q=128,
                  weights="rowmax_pot", where="pot b2 noncausal")


@pytest.mark.parametrize("S", [1, 65])
def test_pot_tiny_lengths(S):
    w = synth.replace(synth.PREFILL_16K, S=S, Hq=8, Hkv=2, d=128, rank=8, seed=78)
    check_prefill(synth.gen_prefill(w), B=1, S=S, Hq=8, Hkv=2, d=128, causal=True, tau=-LN1000, tile_q=128,
                  weights="rowmax_pot", where=f"pot S={S}")


def test_pot_fp8_scores():
    """Rowmax-PoT on the fp8-score prefill (the tie band widens by the fp8 MFMA's score error bound)."""
    w = synth.replace(synth.PREFILL_16K, S=1000, Hq=8, Hkv=2, d=128, rank=8, seed=912)
    data = synth.gen_prefill(w)
    check_prefill(data, B=1, S=1000, Hq=8, Hkv=2, d=128, causal=True, tau=-LN1000, tile_q=128,
                  fp8qk=synth.fp8_qk(data), weights="rowmax_pot", where="pot fp8 scores")


def test_pot_skips_the_same_tiles_as_exp():
    """The weights do not enter the skip rule: both kernels leave the same tiles out, with the same unit gaps, on
    the 2K llama-shaped input."""
    w = synth.replace(synth.PREFILL_16K, S=2048, seed=2048)
    data = synth.gen_prefill(w)
    kw = dict(B=1, S=2048, Hq=64, Hkv=8, d=128, causal=True, tau=-LN1000, tile_q=128)
    out_e, st_e, gap_e, cnt_e = run_prefill_gpu(data, **kw)
    out_p, st_p, gap_p, cnt_p = run_prefill_gpu(data, weights="rowmax_pot", **kw)
    assert np.array_equal(st_e, st_p) and np.array_equal(cnt_e, cnt_p)
    assert np.array_equal(gap_e, gap_p, equal_nan=True)
    diff = np.abs(out_e - out_p)
    log(f"pot vs exp (2K): max |o_pot - o_exp| {diff.max():.3e}, mean {diff.mean():.3e}, skipped "
        f"{int(cnt_e[1])} of {int(cnt_e[0])} tiles")
    assert 0 < diff.max() < 1.0


def test_pot_16k_sampled():
    """The 16K workload at full size with Rowmax-PoT weights; the oracle checks sampled units."""
    w = synth.PREFILL_16K
    data = synth.gen_prefill(w)
    nqt = w.S // 128
    rng = np.random.default_rng(4)
    heads = rng.choice(w.Hq, 3, replace=False)
    qts = [0, nqt // 3, nqt - 1]
    units = [(0 * w.Hq + int(h)) * nqt + qt for h in heads for qt in qts]
    check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=-LN1000, tile_q=128, units=units,
                  weights="rowmax_pot", where="pot 16k sampled")


@pytest.mark.parametrize("tau", [-LN1000, -math.inf])
def test_pot_128k_sampled(tau):
    """Rowmax-PoT on the 128K benchmark workload in the launch configuration the benchmark times (at its tau and
    with nothing skipped); the oracle checks sampled units including the first and the longest query tiles."""
    w = synth.PREFILL_128K
    data = synth.gen_prefill(w)
    nqt = w.S // 128
    units = np.array([0 * nqt + 0, 17 * nqt + 255, 40 * nqt + 777, 63 * nqt + nqt - 1])
    r = check_prefill(data, B=1, S=w.S, Hq=w.Hq, Hkv=w.Hkv, d=w.d, causal=True, tau=tau, tile_q=128, units=units,
                      weights="rowmax_pot", where=f"pot 128k tau={tau}")
    assert r["sparsity"] >= 0.45 if tau > -math.inf else r["sparsity"] == 0.0
