"""ssm_decode_noalloc (the decode whose workspace is the library's static per-GPU scratch array) against ssm_decode
with a caller workspace (GPU).  Two calls in a row, the second on a smaller problem than the first, each must give
ssm_decode's outputs, tile states and counters bit for bit (same kernels; only the workspace differs).  The first
call fills most of the 32 MiB scratch (batch 32, 64 query heads, d 128, 16 splits: 16.9 MB), so the second runs
over what the first left behind."""
import math

import numpy as np
import pytest
import torch

import long_context_flash_amd as ssm
import synth
from parity import log

pytestmark = pytest.mark.gpu
LN1000 = math.log(1000.0)


def run_both(data, *, paged, num_splits, sink_seed, tau):
    dev = "cuda"
    q = ssm.bf16_from_bits(data["q"], dev)
    lens = torch.from_numpy(data["kv_lens"]).to(dev)
    kind = "pool" if paged else "cache"
    kc, vc = ssm.bf16_from_bits(data[f"k_{kind}"], dev), ssm.bf16_from_bits(data[f"v_{kind}"], dev)
    pt = torch.from_numpy(data["page_table"]).to(dev) if paged else None
    B, Hq, d = q.shape
    Hkv = kc.shape[1]
    max_tiles = pt.shape[1] if paged else -(-kc.shape[2] // 64)
    outs, stats = [], []
    for noalloc in (False, True):
        st = ssm.SkipStats.alloc(B * Hkv, max_tiles, dev, gaps=True)
        out = torch.full_like(q, float("nan"))
        fn = ssm.ssm_decode_noalloc if noalloc else ssm.ssm_decode
        fn(q, kc, vc, lens, tau=tau, out=out, page_table=pt, num_splits=num_splits, skip_stats=st,
           sink_seed=sink_seed)
        torch.cuda.synchronize()
        outs.append(out)
        stats.append(st)
    assert torch.equal(outs[0], outs[1]), "outputs differ"
    assert torch.equal(stats[0].tile_state, stats[1].tile_state), "tile states differ"
    assert torch.equal(stats[0].counters, stats[1].counters), "counters differ"
    assert torch.equal(stats[0].unit_gap.nan_to_num(), stats[1].unit_gap.nan_to_num()), "unit gaps differ"
    assert not torch.isnan(outs[1].float()).any()
    return stats[1].counters.cpu().numpy()


def test_noalloc_decode_matches_decode_on_two_calls():
    big = synth.replace(synth.DECODE_32K, B=32, kv_len=0, kv_len_lo=600, kv_len_hi=3000, seed=91, paged=True)
    assert ssm.ssm_decode_workspace_bytes(32, 64, 128, 16) > 16 << 20
    log("noalloc: call 1, B=32 Hq=64 d=128 paged 16 splits")
    c1 = run_both(synth.gen_decode(big, contiguous=False, paged=True), paged=True, num_splits=16, sink_seed=False,
                  tau=-LN1000)
    small = synth.replace(synth.DECODE_32K, B=3, Hq=8, Hkv=1, d=64, kv_len=0, kv_len_lo=1, kv_len_hi=900, seed=92)
    log("noalloc: call 2, B=3 Hq=8 d=64 contiguous 4 splits, sink-seeded")
    c2 = run_both(synth.gen_decode(small, contiguous=True, paged=False), paged=False, num_splits=4, sink_seed=True,
                  tau=-4.0)
    assert c1[1] > 0 and c2[0] > 0, "the calls must visit (and the first skip) tiles"


def test_noalloc_rejects_more_than_its_scratch():
    dev = "cuda"
    B, Hq, Hkv, d = 64, 64, 8, 128
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device=dev)
    kc = torch.zeros(B, Hkv, 64, d, dtype=torch.bfloat16, device=dev)
    lens = torch.full((B,), 64, dtype=torch.int32, device=dev)
    out = torch.zeros_like(q)
    with pytest.raises(ssm.SsmError) as e:
        ssm.ssm_decode_noalloc(q, kc, kc, lens, out=out, num_splits=64)
    assert e.value.code == ssm.SSM_EWORKSPACE
    torch.cuda.synchronize()
    assert not out.any(), "nothing may be launched on an error"
