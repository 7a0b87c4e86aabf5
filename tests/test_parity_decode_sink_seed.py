"""HIP sink-seeded split-K decode vs the fp64 oracle with the same option (GPU).

Every split after the first starts its running maximum at key tile 0's row maxima."""
import math

import numpy as np
import pytest

import synth
from parity import check_decode, log

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(B=3, Hq=16, Hkv=2, d=128, kv_len=0, kv_len_lo=900, kv_len_hi=5000, seed=19)
    base.update(kw)
    return synth.replace(synth.DECODE_32K, **base)


@pytest.mark.parametrize("P", [1, 2, 4, 16])
@pytest.mark.parametrize("tau", [-LN1000, -math.inf, -4.0])
def test_small_contiguous(P, tau):
    data = synth.gen_decode(_small(), contiguous=True, paged=False)
    check_decode(data, tau=tau, num_splits=P, paged=False, sink_seed=True, where=f"seeded small P={P} tau={tau}")


def test_kv_len_edge_cases_paged():
    """kv_len 0, 1, 63, 64, 65, 129 and 16 splits: one-tile units have no seeded split."""
    w = _small(B=6, Hq=8, Hkv=1)
    lens = np.array([0, 1, 63, 64, 65, 129], np.int32)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=True)
    for paged in (False, True):
        r = check_decode(data, tau=-LN1000, num_splits=16, paged=paged, sink_seed=True,
                         where=f"seeded edge paged={paged}")
        assert np.all(r["out"][0] == 0)


@pytest.mark.parametrize("G", [1, 8, 16])
def test_group_sizes_d64(G):
    w = _small(Hq=2 * G, Hkv=2, d=64, seed=30 + G)
    data = synth.gen_decode(w, contiguous=True, paged=False)
    check_decode(data, tau=-LN1000, num_splits=8, paged=False, sink_seed=True, where=f"seeded d64 G={G}")


def test_decode_32k_full_recovers_sparsity():
    """The 32K workload with 16 splits: seeding skips more tiles than split-local scans."""
    w = synth.DECODE_32K
    data = synth.gen_decode(w)
    local = check_decode(data, tau=w.taus[0], num_splits=16, paged=False, where="32k P=16 split-local")
    seeded = check_decode(data, tau=w.taus[0], num_splits=16, paged=False, sink_seed=True, where="32k P=16 seeded")
    log(f"32k sparsity: split-local {local['sparsity']:.3f}, seeded {seeded['sparsity']:.3f}")
    assert seeded["sparsity"] > local["sparsity"] + 0.2
    s_loc, s_sd = local["state"] == 2, seeded["state"] == 2
    assert (s_loc & ~s_sd).sum() <= 0.001 * s_loc.sum(), "seeding keeps (almost) every split-local skip"


def test_decode_128k_paged_sampled():
    """The 128K paged workload in the benchmark's launch configuration, seeded; four sequences checked."""
    w = synth.DECODE_128K
    data = synth.gen_decode(w)
    for tau in (w.taus[2], w.taus[0]):
        check_decode(data, tau=tau, num_splits=w.num_splits, paged=True, batches=np.array([3, 12, 30]),
                     sink_seed=True, where=f"seeded 128k tau={tau}")
