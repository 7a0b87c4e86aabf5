"""The entry points under HIP graph capture (GPU).

The library allocates nothing, writes no memory with memset, never synchronises and reads no device memory on the
host. A call can therefore be captured once, with torch.cuda.graph, and replayed. Between replays, eager work
rewrites the inputs in place: new queries, keys and values for the prefill; new queries and longer kv_lens
for the decode, as in a serving loop. Each replay's outputs and tile states must equal, bit for bit, an eager
call on the same inputs."""
import math

import numpy as np
import pytest
import torch

import long_context_flash_amd as ssm
import synth
from parity import log

pytestmark = pytest.mark.gpu
LN1000 = math.log(1000.0)


def _capture(fn):
    """fn once eagerly on a side stream (first-call set-up), then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("d,Hq,Hkv,tile_q", [(128, 8, 2, 128), (64, 6, 2, 64)])
def test_prefill_graph_replays(d, Hq, Hkv, tile_q):
    """The paired-head kernel (d 128, even groups) and the general one (d 64, odd groups)."""
    dev = "cuda"
    S = 1000
    inputs = [synth.gen_prefill(synth.replace(synth.PREFILL_16K, S=S, Hq=Hq, Hkv=Hkv, d=d, rank=8, seed=700 + i))
              for i in range(3)]
    q, k, v = (ssm.bf16_from_bits(inputs[0][x], dev) for x in ("q", "k", "v"))
    out = torch.empty_like(q)
    units, tiles = ssm.prefill_stats_shape(1, S, Hq, tile_q)
    st = ssm.SkipStats.alloc(units, tiles, dev, gaps=True)
    call = lambda o, s: ssm.ssm_prefill(q, k, v, causal=True, tau=-LN1000, out=o, skip_stats=s, tile_q=tile_q)
    g = _capture(lambda: call(out, st))
    for rep, data in enumerate(inputs[1:] + inputs[:1]):
        log(f"prefill graph d={d} Hq={Hq} tile_q={tile_q}: replay {rep}")
        for name, t in (("q", q), ("k", k), ("v", v)):
            t.copy_(ssm.bf16_from_bits(data[name], dev))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_out = torch.empty_like(out)
        ref_st = ssm.SkipStats.alloc(units, tiles, dev, gaps=True)
        call(ref_out, ref_st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: outputs differ from the eager call"
        assert torch.equal(st.tile_state, ref_st.tile_state), f"replay {rep}: tile states differ"
        assert torch.equal(st.unit_gap.nan_to_num(), ref_st.unit_gap.nan_to_num()), f"replay {rep}: unit gaps differ"
        assert int((ref_st.tile_state == 2).sum()) > 0, "the inputs must skip tiles"


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays_as_kv_lens_grow(noalloc):
    """A paged decode captured once; between replays the queries change and every sequence grows by a few
    tokens (its new keys and values are already in the pool), including across a 64-token tile boundary."""
    dev = "cuda"
    w = synth.replace(synth.DECODE_32K, B=6, kv_len=0, kv_len_lo=3000, kv_len_hi=9000, seed=77, paged=True)
    steps = (1, 63, 200)
    # the pool holds every sequence at its final length; the loop starts sum(steps) tokens short of it
    final = synth.kv_lens_for(w).astype(np.int64) + sum(steps)
    data = synth.gen_decode(w, kv_lens=final, contiguous=False, paged=True)
    kp, vp = ssm.bf16_from_bits(data["k_pool"], dev), ssm.bf16_from_bits(data["v_pool"], dev)
    pt = torch.from_numpy(data["page_table"]).to(dev)
    lens0 = final - sum(steps)
    lens = torch.from_numpy(lens0.astype(np.int32)).to(dev)
    q = ssm.bf16_from_bits(data["q"], dev)
    B, Hq, d = q.shape
    out = torch.empty_like(q)
    st = ssm.SkipStats.alloc(B * w.Hkv, pt.shape[1], dev, gaps=True)
    ws = None if noalloc else ssm.decode_workspace(B, Hq, d, 16, dev)
    fn = ssm.ssm_decode_noalloc if noalloc else ssm.ssm_decode
    kw = dict(tau=-LN1000, page_table=pt, num_splits=16)
    if not noalloc:
        kw["workspace"] = ws
    g = _capture(lambda: fn(q, kp, vp, lens, out=out, skip_stats=st, **kw))
    rng = np.random.default_rng(3)
    grown = lens0.copy()
    for rep, step in enumerate(steps):
        grown = grown + step
        log(f"decode graph noalloc={noalloc}: replay {rep}, kv_len {grown.min()}..{grown.max()}")
        lens.copy_(torch.from_numpy(grown.astype(np.int32)))
        q.copy_(torch.from_numpy(rng.standard_normal(q.shape).astype(np.float32)).to(dev).to(torch.bfloat16))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_out = torch.empty_like(out)
        ref_st = ssm.SkipStats.alloc(B * w.Hkv, pt.shape[1], dev, gaps=True)
        ref_kw = dict(kw)
        if not noalloc:
            ref_kw["workspace"] = ssm.decode_workspace(B, Hq, d, 16, dev)
        fn(q, kp, vp, lens, out=ref_out, skip_stats=ref_st, **ref_kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: outputs differ from the eager call"
        assert torch.equal(st.tile_state, ref_st.tile_state), f"replay {rep}: tile states differ"
        assert torch.equal(st.unit_gap.nan_to_num(), ref_st.unit_gap.nan_to_num()), f"replay {rep}: unit gaps differ"
        visited = int((st.tile_state.cpu() != 0).sum())
        assert visited == int(sum(-(-int(n) // 64) for n in grown)) * w.Hkv, "every tile of the grown lengths"
