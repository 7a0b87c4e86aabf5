"""HIP prefill vs the fp64 oracle on inputs whose key tiles carry designed logits (GPU).

Every key of tile t has logit TILE_LOGITS[t] against every query (plus small noise), so the scan of a unit
goes through a fixed sequence of decisions (tau = -ln 1000): the first tile kept; two skipped; a new
maximum right after a skip (the reference max moves while no P.V is pending); a kept tile below the max;
a skip right after a kept tile; another jump after a skip; a kept tile; a jump while the previous tile's
P.V is still pending; a skip; a kept tile; a skip as last tile (T = 12) or a kept jump as last tile
(T = 13, T = 11 ends on a kept tile).  These are the transitions of the prefill kernel's pipeline, where
the exponentials of one tile run between the P.V MFMAs of the previous kept tile.
"""
import math

import numpy as np
import pytest

import synth
from parity import check_prefill, run_prefill_gpu

pytestmark = pytest.mark.gpu
LN1000 = math.log(1000.0)

TILE_LOGITS = [0, -20, -20, 10, 9, -15, 30, 29, 45, -10, 44, -30, 60]
# decisions at tau = -ln 1000 for a unit that sees every tile (1 kept, 2 skipped): the gap to the running
# max is +inf, -20, -20, +10, -1, -25, +20, -1, +15, -55, -1, -75, +15
EXPECTED = [1, 2, 2, 1, 1, 2, 1, 1, 1, 2, 1, 2, 1]


def designed(T, Hq, Hkv, d, seed):
    """q . k * d^-1/2 = TILE_LOGITS[tile of k] + noise: component 0 of every query is sqrt(d), component 0
    of a key is its tile's logit, the other components are small Gaussians (noise ~0.1 logits)."""
    S = 64 * T
    rng = np.random.default_rng(seed)
    q = 0.3 * rng.standard_normal((1, S, Hq, d))
    q[..., 0] = math.sqrt(d)
    k = 0.3 * rng.standard_normal((1, S, Hkv, d))
    k[..., 0] = np.repeat(np.asarray(TILE_LOGITS[:T], np.float64), 64)[None, :, None]
    v = rng.standard_normal((1, S, Hkv, d))
    return {x: synth.f32_to_bf16_bits(a.astype(np.float32)) for x, a in (("q", q), ("k", k), ("v", v))}


@pytest.mark.parametrize("T", [11, 12, 13])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile_q", [64, 128])
def test_designed_transitions_full(T, d, tile_q):
    """Non-causal: every unit sees every tile, so its decisions are the designed sequence exactly."""
    data = designed(T, Hq=4, Hkv=1, d=d, seed=100 + T)
    S = 64 * T
    _, st, _, _ = run_prefill_gpu(data, B=1, S=S, Hq=4, Hkv=1, d=d, causal=False, tau=-LN1000, tile_q=tile_q)
    assert (st == np.asarray(EXPECTED[:T], np.uint8)[None, :]).all(), f"tile states {st[0].tolist()}"
    check_prefill(data, B=1, S=S, Hq=4, Hkv=1, d=d, causal=False, tau=-LN1000, tile_q=tile_q,
                  where=f"designed full T={T} d={d} tq={tile_q}")


@pytest.mark.parametrize("T", [11, 12, 13])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("tile_q", [64, 128])
def test_designed_transitions_causal(T, d, tile_q):
    """Causal: each query tile's scan is a prefix of the sequence (ending on its diagonal tiles)."""
    data = designed(T, Hq=4, Hkv=1, d=d, seed=200 + T)
    check_prefill(data, B=1, S=64 * T, Hq=4, Hkv=1, d=d, causal=True, tau=-LN1000, tile_q=tile_q,
                  where=f"designed causal T={T} d={d} tq={tile_q}")


@pytest.mark.parametrize("T", [12, 13])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_designed_transitions_fp8qk(T, d, causal):
    """The same designed scans through the 8-bit-score prefill (q and k quantised with amax/448 scales; the
    designed tile logits keep their decisions after quantisation, so non-causal units show the sequence).  The
    whole logit sits in channel 0 here, the worst case for the fp8 MFMA's truncated in-group sums (logit errors
    near 0.008 at logit 60), so the outputs are held to the bar derived from that error bound only."""
    data = designed(T, Hq=4, Hkv=1, d=d, seed=300 + T)
    f8 = synth.fp8_qk(data)
    S = 64 * T
    if not causal:
        _, st, _, _ = run_prefill_gpu(data, B=1, S=S, Hq=4, Hkv=1, d=d, causal=False, tau=-LN1000, tile_q=128,
                                      fp8qk=f8)
        assert (st == np.asarray(EXPECTED[:T], np.uint8)[None, :]).all(), f"tile states {st[0].tolist()}"
    check_prefill(data, B=1, S=S, Hq=4, Hkv=1, d=d, causal=causal, tau=-LN1000, tile_q=128, fp8qk=f8, fp8_slack=True,
                  where=f"designed fp8qk causal={causal} T={T} d={d}")
