"""HIP decode over an fp8 e4m3 KV cache (per-tensor scales) vs the fp64 oracle on the same codes (GPU)."""
import math

import numpy as np
import pytest

import synth
from parity import check_decode, run_decode_gpu, log

LN1000 = math.log(1000.0)
pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(B=3, Hq=16, Hkv=2, d=128, kv_len=0, kv_len_lo=900, kv_len_hi=5000, seed=29)
    base.update(kw)
    return synth.replace(synth.DECODE_32K, **base)


@pytest.mark.parametrize("P", [1, 4, 16])
@pytest.mark.parametrize("tau", [-LN1000, -math.inf, -4.0])
def test_small_contiguous(P, tau):
    data = synth.gen_decode(_small(), contiguous=True, paged=False)
    check_decode(data, tau=tau, num_splits=P, paged=False, fp8=synth.fp8_kv(data), where=f"fp8 small P={P} tau={tau}")


def test_paged_matches_contiguous_and_seeded():
    data = synth.gen_decode(_small(), contiguous=True, paged=True)
    f8 = synth.fp8_kv(data)
    a = check_decode(data, tau=-LN1000, num_splits=16, paged=True, fp8=f8, where="fp8 paged")
    b = run_decode_gpu(data, tau=-LN1000, num_splits=16, paged=False, fp8=f8)
    assert np.array_equal(a["out"], b[0]), "paged and contiguous fp8 layouts must give identical outputs"
    check_decode(data, tau=-LN1000, num_splits=16, paged=True, fp8=f8, sink_seed=True, where="fp8 paged seeded")


def test_kv_len_edge_cases():
    w = _small(B=6, Hq=8, Hkv=1)
    lens = np.array([0, 1, 63, 64, 65, 129], np.int32)
    data = synth.gen_decode(w, kv_lens=lens, contiguous=True, paged=True)
    f8 = synth.fp8_kv(data)
    for paged in (False, True):
        r = check_decode(data, tau=-LN1000, num_splits=16, paged=paged, fp8=f8, where=f"fp8 edge paged={paged}")
        assert np.all(r["out"][0] == 0)


@pytest.mark.parametrize("G", [1, 8, 16])
def test_group_sizes_d64(G):
    w = _small(Hq=2 * G, Hkv=2, d=64, seed=40 + G)
    data = synth.gen_decode(w, contiguous=True, paged=False)
    check_decode(data, tau=-LN1000, num_splits=8, paged=False, fp8=synth.fp8_kv(data), where=f"fp8 d64 G={G}")


def test_decode_32k_full():
    w = synth.DECODE_32K
    data = synth.gen_decode(w)
    check_decode(data, tau=w.taus[0], num_splits=16, paged=False, fp8=synth.fp8_kv(data), where="fp8 32k P=16")


def test_decode_128k_paged_sampled():
    """The 128K paged workload with an fp8 cache in the benchmark's launch configuration; three sequences."""
    w = synth.DECODE_128K
    data = synth.gen_decode(w)
    f8 = synth.fp8_kv(data)
    for tau in (w.taus[2], -math.inf):
        r = check_decode(data, tau=tau, num_splits=w.num_splits, paged=True, batches=np.array([2, 17, 29]), fp8=f8,
                         where=f"fp8 128k tau={tau}")
        log(f"fp8 128k tau={tau}: sparsity {r['sparsity']:.3f}")


def test_every_value_code_exact():
    """Each finite e4m3 code reaches the output exactly: one key per sequence (its softmax weight is 1), V rows
    holding all 254 finite codes (the two NaN codes replaced by 0), scale 1.  The output in bf16 must equal
    torch's float8_e4m3fn decoding of the code, which bf16 represents exactly."""
    import torch
    import long_context_flash_amd as ssm
    B, Hq, Hkv, d = 2, 8, 1, 128
    codes = np.arange(256, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    v = np.zeros((B, Hkv, 64, d), np.uint8)
    v[:, 0, 0, :] = codes.reshape(B, d)
    k = np.zeros((B, Hkv, 64, d), np.uint8)
    rng = np.random.default_rng(7)
    q = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, d)).astype(np.float32))
    dev = "cuda"
    vc = torch.from_numpy(v).to(dev).view(torch.float8_e4m3fn)
    kc = torch.from_numpy(k).to(dev).view(torch.float8_e4m3fn)
    lens = torch.ones(B, dtype=torch.int32, device=dev)
    for P in (1, 16):
        out = ssm.ssm_decode(ssm.bf16_from_bits(q, dev), kc, vc, lens, tau=-LN1000, num_splits=P, k_scale=1.0,
                             v_scale=1.0)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        want = torch.from_numpy(codes.reshape(B, d)).view(torch.float8_e4m3fn).to(torch.float32).numpy()
        for h in range(Hq):
            assert np.array_equal(got[:, h, :], want), f"P={P} head {h}: {np.argwhere(got[:, h, :] != want)[:8]}"
