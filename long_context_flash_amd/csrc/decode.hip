// decode.hip -- Skip Softmax single-token GQA decode for gfx950: split-K + log-sum-exp combine.
//
// Method: the online-softmax forward of the recap "Accelerating Long-Context
// Inference with Skip Softmax in NVIDIA TensorRT-LLM" (Key Points, Detailed
// Analysis, Skip Softmax Mechanism) applied to the generation phase; the news
// item (Benefits and Implementation) attributes the decode gain to lower memory
// traffic, so here a skipped tile's V rows are never read from HBM.
//
// Unit = (batch b, KV group g): the G query heads of the group vote together.
// The unit's ceil(kv_len/64) key tiles are cut into num_splits consecutive
// chunks; each chunk is an independent scan (running maximum starts at -inf)
// handled by one workgroup that writes a partial (o_s, lse_s).  A second
// kernel combines the partials per (b, query head).
//
// Workgroup = 4 waves.  Tiles of the split are processed four at a time, one
// per wave.  Skipping depends only on the prefix maximum of the tile maxima
// (tau <= 0 means a skipped tile never raises it), so the four tiles' S = Q.K^T
// are computed in parallel, their per-query maxima exchanged through LDS, and
// each wave decides its own tile against max(previous chunks, earlier waves).
//
// Per wave and tile (64 keys):
//   S^T (16 keys x 16 query columns, G <= 16 used) = K . Q^T on
//   v_mfma_f32_16x16x32_bf16, four key blocks.  K comes straight from HBM into
//   the A operand (16 bytes per lane per MFMA, no LDS).  Each lane owns one
//   query column.
//   O^T += V^T . P^T on the same MFMA: P^T is the S^T accumulator converted to
//   bf16 in place.  For the V^T operand each lane loads 8 keys x 8 channels
//   (eight 16-byte rows) and transposes them in registers; MFMA j uses channel
//   j of each loaded chunk, so its 16 output rows are channels 8m + j.
//   V is loaded only after the vote keeps the tile (a skipped tile's loads read an
//   empty buffer resource: no memory traffic), with the non-temporal cache policy:
//   its rows are read whole and once, and must not evict the K lines that each
//   K load instruction leaves half-read for the next one.
//
// FP8 cache (optional): K and V stored as OCP e4m3 codes with one dequantisation
// scale per tensor.  Half the bytes of a bf16 cache are read; each code is
// converted exactly to bf16 in registers and the same bf16 MFMAs run.  The key
// scale is folded into the logit scale, the value scale into the split output.
// The QK^T contraction takes the channels in an order where each lane's 16-byte
// key load holds two k-steps, so a key row is fetched in 64-byte pieces as for
// bf16 (8-byte loads fetch 32-byte pieces and cap the read rate well below HBM's).
//
// Sink-seeded split-K (optional): a split after the first starts its prefix
// maximum at key tile 0's per-query maxima instead of -inf; each wave scores
// tile 0 once before its scan.  The combined output stays the exact softmax
// over the kept keys; the seed only changes which tiles are skipped.
#include <mutex>

#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

constexpr int kDecTK = 64;
constexpr int kDecWaves = 4;
constexpr int kDecMaxG = 16;

// Buffer resource over the valid rows of key tile t of (b, g) in a pool of ES-byte elements: rows past
// kv_len, and every row of a tile whose page id is outside the pool, read as zero.
template <int ES>
__device__ __forceinline__ rsrc_t decode_tile_rsrc(const void* pool, const int32_t* pages, int max_pages,
                                                   int64_t pool_pages, int64_t sb, int64_t sh, int64_t ss, int b,
                                                   int g, int t, int len, int d) {
  const int rows = min(kDecTK, len - t * kDecTK);
  const uint8_t* p8 = static_cast<const uint8_t*>(pool);
  int64_t elem;
  if (pages) {
    // the page id is wave-uniform: keep it (and the resource) in scalar registers
    const int pg = __builtin_amdgcn_readfirstlane(load_uniform_i32(pages, (int64_t)b * max_pages + t));
    if (pg < 0 || pg >= pool_pages) return make_rsrc(pool, 0u);
    elem = (int64_t)pg * sb + (int64_t)g * sh;
  } else {
    elem = (int64_t)b * sb + (int64_t)g * sh + (int64_t)t * kDecTK * ss;
  }
  return make_rsrc(p8 + elem * ES, rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * ss + d) * ES));
}

// kv_cap: keys the cache can hold (contiguous Smax, paged max_pages*64);
// pool_pages: number of pages in the pools (paged only).
// ES: bytes per K/V element (2: bf16 cache; 1: fp8 e4m3 cache, converted to bf16 in registers).
template <int D, int ES>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(DecodeArgs a, int kv_cap, int64_t k_pool_pages,
                                                              int64_t v_pool_pages) {
  constexpr int KS = D / 32;            // k-steps of the QK^T MFMA
  static_assert(ES == 1 || ES == 2, "bf16 or fp8 cache");
  __shared__ float mt[2][kDecWaves][kDecMaxG];  // per-chunk tile maxima (double-buffered by chunk parity)
  __shared__ float cm[kDecWaves][kDecMaxG];
  __shared__ float cl[kDecWaves][kDecMaxG];
  __shared__ __attribute__((aligned(16))) float cacc[kDecWaves][kDecMaxG][D];

  __shared__ unsigned cnt_lds[kDecWaves][2];

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform: the tile index, its page id and its buffer resource then live in scalar registers
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qc = lane & 15, grp = lane >> 4;  // query column, lane group (key group for operands)
  const int P = a.num_splits;
  const int split = blockIdx.x % P;
  const int rg = blockIdx.x / P;
  const int rank = rg / a.Hkv, g = rg - rank * a.Hkv;
  const int G = a.G;
  auto clamp_len = [&](int l) { return l < 0 ? 0 : (l > kv_cap ? kv_cap : l); };

  // Longest sequences first: workgroups are dispatched in index order, so the rank-th longest sequence
  // (decode_order_kernel's order; plain order for batches above kDecSortMax) takes the rank-th group of
  // Hkv * P workgroups and the short ones fill the tail.
  const int b = a.order ? __builtin_amdgcn_readfirstlane(load_uniform_i32(a.order, rank)) : rank;
  const int bg = b * a.Hkv + g;
  const int len = clamp_len(__builtin_amdgcn_readfirstlane(a.kv_lens[b]));
  const int nt = (len + kDecTK - 1) / kDecTK;
  const int tps = (nt + P - 1) / P;
  const int s_begin = min(nt, split * tps), s_end = min(nt, s_begin + tps);
  const int64_t srow = (int64_t)bg * a.max_tiles;

  // statistics rows: this split owns tiles [split*tps, split*tps + tps); the last split also owns the tail
  {
    const int own_lo = min(a.max_tiles, split * tps);
    const int own_hi = split == P - 1 ? a.max_tiles : min(a.max_tiles, split * tps + tps);
    for (int t = max(own_lo, s_end) + tid; t < own_hi; t += 256) {
      if (a.tile_state) a.tile_state[srow + t] = 0;
      if (a.unit_gap) a.unit_gap[srow + t] = __builtin_nanf("");
    }
  }

  const int64_t part_row = ((int64_t)b * a.Hq + g * G) * P + split;  // + q*P for query q of the group
  if (s_begin >= s_end) {  // empty split: lse = -inf, o = 0
    if (a.counters && tid == 0) *reinterpret_cast<u32x2*>(a.wg_cnt + ((int64_t)bg * P + split) * 2) = u32x2{0u, 0u};
    for (int i = tid; i < G * D; i += 256) {
      const int q = i / D, c = i - q * D;
      a.part_o[(part_row + (int64_t)q * P) * D + c] = 0.f;
      if (c == 0) a.part_lse[part_row + (int64_t)q * P] = neg_inf();
    }
    return;
  }

  // Channel order of the QK^T contraction: k-step ks, lane group grp, element e covers channel
  // ks*32 + grp*8 + e for a bf16 cache, and (ks/2)*64 + grp*16 + (ks%2)*8 + e for an fp8 cache, so that one
  // 16-byte load per lane brings two k-steps of fp8 codes and a key row is read in 64-byte pieces (any
  // order of the channels gives the same dot products; Q and K use the same one).
  auto chan = [&](int ks) { return ES == 2 ? ks * 32 + grp * 8 : (ks >> 1) * 64 + grp * 16 + (ks & 1) * 8; };
  // Q^T operand: lane (qc, grp) holds Q[qc][chan(ks) .. +8]; columns >= G are zero
  bf16x8 qreg[KS];
  {
    const rsrc_t rq = make_rsrc(a.q + (int64_t)b * a.q_sb + (int64_t)g * G * a.q_sh, rows_bytes(G, a.q_sh, D));
    const uint32_t qoff = qc < G ? (uint32_t)(qc * a.q_sh * 2) : 0xffffffffu;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = as_bf16x8(buffer_load_16(rq, qc < G ? qoff + chan(ks) * 2 : qoff));
  }

  // lane offsets inside a tile (bytes), fixed for the whole scan
  uint32_t kvo[4];  // K: row kb*16 + qc, channel chan(0) (the other k-steps add immediates)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) kvo[kb] = (uint32_t)(((kb * 16 + qc) * a.k_ss + chan(0)) * ES);
  // V: lane (m = qc, grp) loads keys st*32 + 16*(e/4) + 4*grp + (e%4), channels 8m .. 8m+7 (zero for 8m >= D)
  const bool v_ch_ok = qc * 8 < D;
  uint32_t vvo[2][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int eh = 0; eh < 2; ++eh)
      vvo[st][eh] = v_ch_ok ? (uint32_t)(((st * 32 + 16 * eh + 4 * grp) * a.v_ss + qc * 8) * ES) : 0xffffffffu;
  const uint32_t vrow = (uint32_t)(a.v_ss * ES);

  const int nchunks = (s_end - s_begin + kDecWaves - 1) / kDecWaves;
  // A operand of the QK^T MFMAs, key block kb, k-step ks: bf16 as loaded, or fp8 codes converted at use
  u32x4 kreg[4][KS];       // bf16: one k-step per register
  u32x4 kraw[4][KS / 2];   // fp8: k-steps 2j and 2j+1 in register j (bytes 0-7 and 8-15)
  auto k_rsrc = [&](int t) {
    return decode_tile_rsrc<ES>(a.k, a.k_pages, a.k_max_pages, k_pool_pages, a.k_sb, a.k_sh, a.k_ss, b, g, t, len, D);
  };
  // key block kb of a K tile (16 key rows) into its operand registers
  auto load_k_block = [&](rsrc_t r, int kb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (ES == 2) kreg[kb][ks] = buffer_load_16(r, kvo[kb] + ks * 64);
      else if (ks % 2 == 0) kraw[kb][ks / 2] = buffer_load_16(r, kvo[kb] + ks * 32);
    }
  };
  auto load_k = [&](int t) {
    const rsrc_t r = k_rsrc(t);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) load_k_block(r, kb);
  };
  auto k_operand = [&](int kb, int ks) {
    if constexpr (ES == 2) return as_bf16x8(kreg[kb][ks]);
    else return as_bf16x8(fp8x8_to_bf16x8(u32x2{kraw[kb][ks / 2][2 * (ks % 2)], kraw[kb][ks / 2][2 * (ks % 2) + 1]}));
  };
  u32x4 vreg[2][8];  // 8 key rows x 8 channels per st (bf16), converted from vraw for an fp8 cache
  u32x2 vraw[2][8];
  // V rows of tile t if `real`, else 16 loads from an empty resource (zeros, no memory traffic): the loop issues
  // the same loads on every path, so the compiler's wait counts stay exact and never drain the next K tile.
  // Each V row is read whole and once, with the non-temporal policy: its lines do not displace the K tile's,
  // which every 64-byte K load leaves half-read in L2 for the next instruction (8% faster at half the tiles
  // kept, 10% with every tile kept; the same policy on the K loads makes the decode slower).
  auto load_v = [&](int t, bool real) {
    const rsrc_t r = real ? decode_tile_rsrc<ES>(a.v, a.v_pages, a.v_max_pages, v_pool_pages, a.v_sb, a.v_sh,
                                                 a.v_ss, b, g, t, len, D)
                          : make_rsrc(a.v, 0u);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // lanes whose channels lie past D (D = 64) read outside the resource, i.e. zeros
        const uint32_t off = v_ch_ok ? vvo[st][e >> 2] + (e & 3) * vrow : 0xffffffffu;
        if constexpr (ES == 2) vreg[st][e] = buffer_load_16_nt(r, off);
        else vraw[st][e] = buffer_load_8_nt(r, off);
      }
  };

  f32x4 acc[8];  // acc[j][i] = O[query qc][channel 32*grp + 8*i + j]
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{};
  float m_run = neg_inf(), l_part = 0.f;
  unsigned n_exec = 0, n_vis = 0;

  // S^T of key tile t (its K operand in kreg): s[kb][i] = S^T[key t*64 + kb*16 + 4*grp + i][query qc],
  // -inf for invalid keys and padding columns; returns the tile maximum of this lane's query.  Each key
  // block's registers are refilled with tile t_next's block as soon as its MFMAs have read them, so the next
  // tile is in flight through this tile's vote, barrier and P.V; t_next < 0 loads zeros from an empty resource
  // (no memory traffic), so every path issues the same loads.
  auto score = [&](int t, f32x4 (&s)[4], int t_next) {
    const rsrc_t r_next = t_next >= 0 ? k_rsrc(t_next) : make_rsrc(a.k, 0u);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 x = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(kb, ks), qreg[ks], x, 0, 0, 0);
      s[kb] = x;
      __builtin_amdgcn_sched_barrier(0);
      load_k_block(r_next, kb);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int lim = qc < G ? len - 1 - t * kDecTK : -1;  // key offset o in the tile is valid iff o <= lim
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = kb * 16 + 4 * grp + i;
        if (o > lim) s[kb][i] = neg_inf();
        mx = fmaxf(mx, s[kb][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    return fmaxf(mx, __shfl_xor(mx, 32, 64));
  };

  // prefix max of tile maxima over earlier chunks (this lane's query).  A split scan starts at -inf;
  // with sink seeding, a split after the first starts at key tile 0's maxima (every wave scores it)
  float r_prev = neg_inf();
  if (a.sink_seed && s_begin > 0) {
    load_k(0);
    f32x4 s0[4];
    r_prev = score(0, s0, -1);
  }
  {
    const int t0 = s_begin + w;
    if (t0 < s_end) load_k(t0);
  }
  // the Q operand and the first K tile have landed before the loop (keeps the wait-count pass from
  // treating the Q registers as pending inside it)
  wait_vmem_all();

  // P.V of a kept tile runs one chunk later, when its V rows (loaded after the vote) have arrived
  bf16x8 pend[2];        // that tile's P^T operands (keys st*32 .. st*32+31)
  bool pending = false;  // wave-uniform
  auto pv = [&]() {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // this st's 8 key rows as bf16 (an fp8 cache is converted here, one st at a time)
      u32x4 vr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (ES == 2) vr[e] = vreg[st][e];
        else vr[e] = fp8x8_to_bf16x8(vraw[st][e]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // A_j: channel 8m + j of the 8 loaded key rows, packed two keys per dword
        const int dw = j >> 1;
        u32x4 av;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t x0 = vr[2 * u][dw], x1 = vr[2 * u + 1][dw];
          av[u] = (j & 1) ? pack_hi16(x0, x1) : pack_lo16(x0, x1);
        }
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), pend[st], acc[j], 0, 0, 0);
      }
    }
  };

  for (int c = 0; c < nchunks; ++c) {
    const int t = s_begin + c * kDecWaves + w;
    const bool has = t < s_end;
    f32x4 s[4];
    float mx = neg_inf();
    const int tn = t + kDecWaves;
    {
      // every wave scores (a wave past the split end scores the zeros it loaded) and issues the next loads
      const float mxs = score(t, s, c + 1 < nchunks && tn < s_end ? tn : -1);
      if (has) mx = mxs;
    }
    if (lane < kDecMaxG) mt[c & 1][w][lane] = mx;
    __syncthreads();
    float r = r_prev, r_all = r_prev;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) {
      const float x = mt[c & 1][w2][qc];
      if (w2 < w) r = fmaxf(r, x);
      r_all = fmaxf(r_all, x);
    }
    r_prev = r_all;

    const bool abstain = mx == neg_inf();
    const float gap = mx - r;  // +inf on the scan's first tile
    const bool keep = has && wave_ballot(!abstain && !(gap < a.tau_raw)) != 0;
    if (has) {
      ++n_vis;
      if (a.unit_gap) {
        float gg = abstain ? neg_inf() : gap;
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) gg = fmaxf(gg, __shfl_xor(gg, off, 64));
        if (lane == 0) a.unit_gap[srow + t] = gg == __builtin_inff() ? gg : gg * a.scale;
      }
      if (lane == 0 && a.tile_state) a.tile_state[srow + t] = keep ? 1 : 2;
    }
    // the previous kept tile's V rows were loaded one chunk ago and arrived while this tile was scored
    // and voted on; its P.V goes in before this tile can rescale the accumulators
    if (pending) pv();
    // bf16: every path issues the 16 V loads (see load_v); fp8: only a kept tile's, whose 16 eight-byte loads
    // per wave cost more issue time than the exact wait counts save (5% at half the tiles kept, same-call A/B)
    if constexpr (ES == 1) {
      if (keep) load_v(t, true);
    } else {
      load_v(t, keep);
    }
    pending = keep;
    if (keep) {
      ++n_exec;
      const float m_new = fmaxf(m_run, mx);
      if (wave_ballot(m_new > m_run)) {
        const float alpha = m_new > m_run ? exp2_fast((m_run - m_new) * a.scale_log2) : 1.f;
        l_part *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= alpha;
        m_run = m_new;
      }
      const float moff = (m_run == neg_inf() ? 0.f : m_run) * a.scale_log2;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // P^T operand: keys st*32 + 16*(e/4) + 4*grp + (e%4) = s[2st + e/4][e%4]
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = exp2_fast(fmaf(s[2 * st + (e >> 2)][e & 3], a.scale_log2, -moff));
          const float p1 = exp2_fast(fmaf(s[2 * st + (e >> 2)][(e & 3) + 1], a.scale_log2, -moff));
          pk[e >> 1] = pack_bf16x2(p0, p1);
          l_part = dot2_bf16_sum(pk[e >> 1], l_part);
        }
        pend[st] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
    }
  }
  if (pending) pv();

  // ---- combine the four waves' partial softmax states
  float l_tot = l_part + __shfl_xor(l_part, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (grp == 0) {
    cm[w][qc] = m_run;
    cl[w][qc] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = 32 * grp + 8 * i + j;
      if (ch < D) cacc[w][qc][ch] = acc[j][i];
    }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int q = idx / D, ch = idx - q * D;
    float mstar = neg_inf();
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) mstar = fmaxf(mstar, cm[w2][q]);
    float lsum = 0.f, o = 0.f;
    if (mstar != neg_inf()) {
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) {
        const float f = cm[w2][q] == neg_inf() ? 0.f : exp2_fast((cm[w2][q] - mstar) * a.scale_log2);
        lsum += f * cl[w2][q];
        o += f * cacc[w2][q][ch];
      }
    }
    const bool ok = lsum > 0.f;
    a.part_o[(part_row + (int64_t)q * P) * D + ch] = ok ? o / lsum * a.v_scale : 0.f;
    if (ch == 0) a.part_lse[part_row + (int64_t)q * P] = ok ? mstar * a.scale_log2 + __builtin_log2f(lsum) : neg_inf();
  }
  // skip counts: this workgroup's totals into its workspace slot (the combine adds them up per sequence, so the
  // four global counters take one set of atomics per sequence instead of one per workgroup)
  if (a.counters) {
    if (lane == 0) {
      cnt_lds[w][0] = n_vis;
      cnt_lds[w][1] = n_exec;
    }
    __syncthreads();
    if (tid == 0) {
      unsigned vis = 0, ex = 0;
#pragma unroll
      for (int w2 = 0; w2 < kDecWaves; ++w2) vis += cnt_lds[w2][0], ex += cnt_lds[w2][1];
      *reinterpret_cast<u32x2*>(a.wg_cnt + ((int64_t)bg * P + split) * 2) = u32x2{vis, ex};
    }
  }
}

// order[r] = the sequence with the r-th longest kv_len (ties by index), lengths clamped to [0, kv_cap]: the
// dispatch order of decode_split_kernel.  One thread per sequence counts the sequences that precede it; every
// workgroup stages all B lengths in LDS (B <= kDecSortMax).
__global__ __launch_bounds__(256) void decode_order_kernel(const int32_t* kv_lens, int B, int kv_cap, int32_t* order) {
  __shared__ int lens[kDecSortMax];
  for (int i = threadIdx.x; i < B; i += 256) {
    const int l = kv_lens[i];
    lens[i] = l < 0 ? 0 : (l > kv_cap ? kv_cap : l);
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= B) return;
  const int lc = lens[c];
  int r = 0;
  for (int j = 0; j < B; ++j) {
    const int lj = lens[j];
    r += lj > lc || (lj == lc && j < c);
  }
  order[r] = c;
}

// out[b, h, :] = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M); 0 when every split is empty.  Lane s of each
// wave holds split s's weight (num_splits <= 64), every thread reads its channel of eight partials at a time,
// and both sums run over the splits in order.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int bh = blockIdx.x, ch = threadIdx.x, lane = ch & 63;
  const int b = bh / a.Hq, h = bh - b * a.Hq;
  const int P = a.num_splits;
  const float* po = a.part_o + (int64_t)bh * P * D;
  const float ls = lane < P ? a.part_lse[(int64_t)bh * P + lane] : neg_inf();
  float M = ls;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float wl = M == neg_inf() ? 0.f : exp2_fast(ls - M);  // 0 for empty splits and lanes >= P
  float wsum = 0.f, o = 0.f;
  for (int s0 = 0; s0 < P; s0 += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = s0 + j < P ? po[(int64_t)(s0 + j) * D + ch] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < P) {
        const float wgt = __shfl(wl, s0 + j, 64);
        wsum += wgt;
        o += wgt * x[j];
      }
    }
  }
  const float r = wsum > 0.f ? o / wsum : 0.f;
  const __bf16 y = (__bf16)r;
  a.o[(int64_t)b * a.o_sb + (int64_t)h * a.o_sh + ch] = __builtin_bit_cast(uint16_t, y);
  // skip counters: the workgroup of each sequence's first query head adds up the counts of the sequence's
  // Hkv * P split workgroups (all threads, then the waves' sums), so the global counters take one set of
  // atomics per sequence
  if (a.counters && h == 0) {
    __shared__ unsigned long long red[D / 64][2];
    const int n = a.Hkv * P;
    const u32x2* wc = reinterpret_cast<const u32x2*>(a.wg_cnt) + (int64_t)b * n;
    unsigned long long vis = 0, ex = 0;
    for (int i = ch; i < n; i += D) {
      const u32x2 x = wc[i];
      vis += x[0];
      ex += x[1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      vis += __shfl_xor(vis, off, 64);
      ex += __shfl_xor(ex, off, 64);
    }
    if (lane == 0) {
      red[ch >> 6][0] = vis;
      red[ch >> 6][1] = ex;
    }
    __syncthreads();
    if (ch == 0) {
      vis = ex = 0;
#pragma unroll
      for (int wv = 0; wv < D / 64; ++wv) vis += red[wv][0], ex += red[wv][1];
      atomicAdd(&a.counters[0], vis);
      atomicAdd(&a.counters[1], vis - ex);
      atomicAdd(&a.counters[2], vis);
      atomicAdd(&a.counters[3], ex);
    }
  }
}

// The decode workspace of ssm_decode_noalloc: one statically sized array in each GPU's memory, held until the
// process ends.  Host code never uses the array's name as an address: its device address is taken once per
// device with that device current (hipGetSymbolAddress) and kept here.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (stream) {  // the kernels run on the stream's device: it must be the current one, whose array is used
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_decode_impl(const DecodeArgs& a, int d, int kv_cap, int64_t k_pool_pages, int64_t v_pool_pages,
                              hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hkv * a.num_splits);
  const unsigned cgrid = (unsigned)((int64_t)a.B * a.Hq);
  if (grid == 0) return hipSuccess;
  if (a.order) {
    if (a.B > kDecSortMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(decode_order_kernel, dim3((a.B + 255) / 256), dim3(256), 0, stream, a.kv_lens, a.B, kv_cap,
                       a.order);
  }
  const dim3 blk(256);
  if (d == 128 && !a.kv_fp8)
    hipLaunchKernelGGL((decode_split_kernel<128, 2>), dim3(grid), blk, 0, stream, a, kv_cap, k_pool_pages, v_pool_pages);
  else if (d == 128)
    hipLaunchKernelGGL((decode_split_kernel<128, 1>), dim3(grid), blk, 0, stream, a, kv_cap, k_pool_pages, v_pool_pages);
  else if (d == 64 && !a.kv_fp8)
    hipLaunchKernelGGL((decode_split_kernel<64, 2>), dim3(grid), blk, 0, stream, a, kv_cap, k_pool_pages, v_pool_pages);
  else if (d == 64)
    hipLaunchKernelGGL((decode_split_kernel<64, 1>), dim3(grid), blk, 0, stream, a, kv_cap, k_pool_pages, v_pool_pages);
  else
    return hipErrorInvalidValue;
  if (d == 128) hipLaunchKernelGGL((decode_combine_kernel<128>), dim3(cgrid), dim3(128), 0, stream, a);
  else hipLaunchKernelGGL((decode_combine_kernel<64>), dim3(cgrid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ssm
