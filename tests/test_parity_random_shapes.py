"""Seeded random shapes through every entry point against the fp64 oracle (GPU): batch, lengths, head counts,
head size, query tile, causality, tau and split counts drawn from a fixed generator, small enough for the
oracle to check every unit; every third prefill also with Rowmax-PoT weights."""
import math

import numpy as np
import pytest

import synth
from parity import check_decode, check_prefill, check_prefill_paged, chunk_batch, fp8_pools, fp8_q_packed

pytestmark = pytest.mark.gpu
TAUS = [-math.inf, -math.log(1000.0), -math.log(100.0), -3.0, 0.0]


def _draw(rng):
    d = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    return d, hkv, g, float(rng.choice(TAUS))


@pytest.mark.parametrize("case", range(40))
def test_prefill_random(case):
    rng = np.random.default_rng(1000 + case)
    d, hkv, g, tau = _draw(rng)
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 900))
    causal, tile_q = bool(rng.integers(0, 2)), int(rng.choice([64, 128]))
    w = synth.replace(synth.PREFILL_16K, B=B, S=S, Hq=hkv * g, Hkv=hkv, d=d, rank=8, seed=2000 + case)
    data = synth.gen_prefill(w)
    check_prefill(data, B=B, S=S, Hq=hkv * g, Hkv=hkv, d=d, causal=causal, tau=tau, tile_q=tile_q,
                  where=f"random prefill {case}: B={B} S={S} Hkv={hkv} G={g} d={d} causal={causal} tq={tile_q}")
    if case % 2 == 0:
        check_prefill(data, B=B, S=S, Hq=hkv * g, Hkv=hkv, d=d, causal=causal, tau=tau, tile_q=tile_q,
                      fp8qk=synth.fp8_qk(data), where=f"random fp8qk prefill {case}")
    if case % 3 == 0:  # Rowmax-PoT weights, on bf16 scores or (every other one) fp8 scores
        check_prefill(data, B=B, S=S, Hq=hkv * g, Hkv=hkv, d=d, causal=causal, tau=tau, tile_q=tile_q,
                      fp8qk=synth.fp8_qk(data) if case % 2 == 1 else None, weights="rowmax_pot",
                      where=f"random pot prefill {case}")


@pytest.mark.parametrize("case", range(30))
def test_decode_random(case):
    rng = np.random.default_rng(3000 + case)
    d, hkv, g, tau = _draw(rng)
    g = min(g * int(rng.choice([1, 2])), 16)
    B = int(rng.integers(1, 6))
    lens = rng.integers(0, 1500, size=B).astype(np.int32)
    P = int(rng.choice([1, 2, 5, 16, 33]))
    w = synth.replace(synth.DECODE_32K, B=B, Hq=hkv * g, Hkv=hkv, d=d, kv_len=0, kv_len_lo=1, kv_len_hi=1500,
                      seed=4000 + case)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=True)
    paged, seeded = bool(rng.integers(0, 2)), bool(rng.integers(0, 2))
    fp8 = synth.fp8_kv(data) if case % 3 == 0 else None
    check_decode(data, tau=tau, num_splits=P, paged=paged, sink_seed=seeded, fp8=fp8,
                 where=f"random decode {case}: B={B} lens={lens.tolist()} Hkv={hkv} G={g} d={d} P={P} "
                       f"paged={paged} seeded={seeded} fp8={fp8 is not None}")


@pytest.mark.parametrize("case", range(20))
def test_chunked_random(case):
    rng = np.random.default_rng(5000 + case)
    d, hkv, g, tau = _draw(rng)
    n = int(rng.integers(1, 5))
    seqs = []
    for _ in range(n):
        nk = int(rng.integers(1, 1200))
        seqs.append((int(rng.integers(0, nk + 1)), nk))
    w = synth.replace(synth.PREFILL_16K, S=0, Hq=hkv * g, Hkv=hkv, d=d, rank=8, seed=6000 + case)
    cb = chunk_batch(w, seqs, seed=case)
    causal, tile_q = bool(rng.integers(0, 2)), int(rng.choice([64, 128]))
    fp8 = fp8_pools(cb) if case % 2 == 1 else None
    fp8q = fp8_q_packed(cb) if case % 4 == 3 else None  # and 8-bit queries (ssm_prefill_paged_fp8qk)
    check_prefill_paged(cb, Hq=hkv * g, causal=causal, tau=tau, tile_q=tile_q, fp8=fp8, fp8q=fp8q,
                        where=f"random chunked {case}: seqs={seqs} Hkv={hkv} G={g} d={d} causal={causal} "
                              f"tq={tile_q} fp8={fp8 is not None} fp8q={fp8q is not None}")
