// prefill.hip -- Skip Softmax prefill forward for gfx950.
//
// Method (recap of "Accelerating Long-Context Inference with Skip Softmax in
// NVIDIA TensorRT-LLM": Key Points, Detailed Analysis, Skip Softmax Mechanism;
// NVIDIA Skip Softmax news item: Understanding Skip Softmax): an online-softmax
// attention forward that streams key tiles in ascending order and, for each
// tile, compares the tile's score maximum with the running maximum; a tile
// whose gap is below tau for every row of the query tile skips its
// exponentials and its P*V product.
//
// One workgroup owns one unit (batch b, query head h, query tile qt) of TQ rows
// and scans its key tiles of 64.  Each wave owns 32 query rows.
//
//   S^T (64 keys x 32 queries) = K_tile . Q^T on v_mfma_f32_32x32x16_bf16,
//   so each lane holds ONE query column: the row statistics (max, sum, the
//   rescale factor) are per-lane scalars and the only cross-lane step is the
//   swap with lane^32 (v_permlane32_swap) that holds the other 32 keys.
//   O^T (d x 32 queries) += V^T . P^T on the same MFMA.  The accumulator layout
//   of S^T is consumed directly as the P^T operand (converted to bf16 in
//   registers); V is staged in LDS transposed ([channel][key]) with the keys of
//   each 16-key group stored in the order that matches that accumulator layout,
//   so each operand is a single 16-byte LDS read.
//
// Skip vote: every lane votes "keep" unless its row abstains (no valid key in
// the tile) or its gap (tile max - running max) is below tau; a wave ballot
// and one LDS word per wave give the unit's decision at the tile barrier.  The
// running maximum only advances on kept tiles; because tau <= 0 a skipped tile
// never holds a new maximum, so this equals the prefix maximum over all
// visited tiles.
//
// Pipeline: K and V tiles are double-buffered in LDS; the buffer loads of tile
// t+1 are issued before tile t's MFMAs and written to LDS after them.  Rows
// past the sequence end fall outside the buffer resource and read as zero, so
// loads carry no predication.  Tiles wholly inside the causal triangle run a
// step without any masking code; only the diagonal/ragged tiles mask.
//
// Exponentials use a lazily moved reference maximum: P = 2^(S*c - m_ref*c) with
// m_ref only raised when the true running maximum exceeds it by more than 8
// (log2 units), which bounds P by 256 and makes the rescale of the output
// accumulator rare.  The row sums add the same bf16-rounded P that enters the
// P*V product (v_dot2 against (1, 1)).  The skip vote always uses the true
// running maximum.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

constexpr int kTK = 64;
constexpr float kRefSlack = 8.f;  // log2 units the reference max may trail the true max

__device__ __forceinline__ void map_prefill_unit(int bid, const PrefillArgs& a, int& b, int& h, int& qt) {
  int level, rem;
  if (a.xcd_groups > 0) {
    // Workgroups are dispatched round-robin over the 8 XCDs: block i runs on XCD i % 8.
    // XCD x owns KV groups {x, x+8, ...}; all query heads of a group and neighbouring
    // query tiles run together on one XCD and share its L2 for the K/V stream.
    const int x = bid & 7, slot = bid >> 3;
    const int per_level = a.xcd_groups * a.G;
    level = slot / per_level;
    rem = slot - level * per_level;
    const int gi = rem / a.G, hh = rem - gi * a.G;
    const int grp = x + 8 * gi;
    b = grp / a.Hkv;
    h = (grp - b * a.Hkv) * a.G + hh;
  } else {
    const int per_level = a.B * a.Hq;
    level = bid / per_level;
    rem = bid - level * per_level;
    b = rem / a.Hq;
    h = rem - b * a.Hq;
  }
  qt = a.nqt - 1 - level;  // longest causal units first
}

// CHUNKED: queries of each sequence are the last ones of its cached keys (bottom-right causal), packed
// ragged rows of q/o, K/V read through a page table (see PrefillArgs).
template <int D, int TQ, bool CHUNKED>
__global__ __launch_bounds__(TQ * 2, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int NW = TQ / 32;             // waves per workgroup
  constexpr int NT = NW * 64;             // threads
  constexpr int KROW = D + 8;             // K tile row stride in LDS (elements); +16 B avoids bank conflicts
  constexpr int VROW = kTK + 8;           // V^T row stride in LDS (elements)
  constexpr int KSTEPS = D / 16;          // k-steps of the QK^T MFMA
  constexpr int CB = D / 32;              // 32-channel blocks of the output
  constexpr int KPT = kTK * D / 8 / NT;   // 16-byte K chunks per thread per tile
  constexpr int CPT = kTK * D / (NT * 4); // V channels per thread (4 keys each)
  constexpr int VW = CPT / 2;             // dwords per key row per thread
  static_assert(KPT >= 1 && CPT >= 4 && CPT % 4 == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VROW];
  __shared__ uint32_t votes[2][NW];
  __shared__ float wave_gap[2][NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  int b, h, qt;
  map_prefill_unit(blockIdx.x, a, b, h, qt);
  const int g = h / a.G;
  const int64_t unit = ((int64_t)b * a.Hq + h) * a.nqt + qt;
  const int q0 = qt * TQ;
  // S queries against Sk keys; query i sits at key position off + i; q/o rows start at qrow0
  int S = a.S, Sk = a.S, off = 0, qrow0 = 0;
  bool keys_ok = true;
  if constexpr (CHUNKED) {
    qrow0 = __builtin_amdgcn_readfirstlane(a.q_start[b]);
    S = __builtin_amdgcn_readfirstlane(a.q_start[b + 1]) - qrow0;
    Sk = __builtin_amdgcn_readfirstlane(a.kv_lens[b]);
    if (qrow0 < 0 || S < 0 || S > a.S || qrow0 + S > a.total_q) S = 0;  // malformed offsets: no rows touched
    keys_ok = Sk >= S && Sk <= a.max_pages * kTK;                // otherwise its rows are written as zeros
    off = Sk - S;
    if (q0 >= S) {  // a query tile past this sequence's queries: only its statistics row is written
      if (tid == 0)
        for (int t = 0; t < a.nkt; ++t) {
          if (a.tile_state) a.tile_state[unit * a.nkt + t] = 0;
          if (a.unit_gap) a.unit_gap[unit * a.nkt + t] = __builtin_nanf("");
        }
      return;
    }
  }
  const int q_end = min(S, q0 + TQ);
  const int T = !keys_ok ? 0 : (a.causal ? (q_end - 1 + off) / kTK + 1 : (Sk + kTK - 1) / kTK);  // visited key tiles
  // tiles [0, T_in) have every (row, key) pair valid: no masking code runs for them
  const int full_tiles = Sk / kTK;
  const int T_in = q_end < q0 + TQ ? 0 : min(T, a.causal ? min((q0 + off + 1) / kTK, full_tiles) : full_tiles);
  const float c2 = a.scale_log2;

  // ---- buffer resources: one (b, head) slice each (chunked: K/V per tile, below); bytes past the last row
  // read as zero
  const rsrc_t rq = CHUNKED ? make_rsrc(a.q + (int64_t)qrow0 * a.q_ss + (int64_t)h * a.q_sh, rows_bytes(S, a.q_ss, D))
                            : make_rsrc(a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh, rows_bytes(S, a.q_ss, D));
  const rsrc_t rk = make_rsrc(a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh, CHUNKED ? 0u : rows_bytes(S, a.k_ss, D));
  const rsrc_t rv = make_rsrc(a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh, CHUNKED ? 0u : rows_bytes(S, a.v_ss, D));
  // chunked: the resource of key tile t of this KV head (rows past Sk and bad page ids read as zero)
  auto page_rsrc = [&](const uint16_t* pool, const int32_t* pages, int64_t pool_pages, int64_t sb, int64_t sh,
                       int64_t ss, int t) {
    const int pg = __builtin_amdgcn_readfirstlane(pages[(int64_t)b * a.max_pages + t]);
    if (pg < 0 || pg >= pool_pages) return make_rsrc(pool, 0u);
    return make_rsrc(pool + (int64_t)pg * sb + (int64_t)g * sh, rows_bytes(min(kTK, Sk - t * kTK), ss, D));
  };

  // ---- Q operand: lane (col, half) holds Q[row][ks*16 + half*8 .. +8] for every k-step
  const int iq = q0 + w * 32 + col;
  const bool row_ok = iq < S;
  bf16x8 qreg[KSTEPS];
  {
    const uint32_t qoff = row_ok ? (uint32_t)iq * (uint32_t)(a.q_ss * 2) + half * 16 : 0xffffffffu;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qreg[ks] = as_bf16x8(buffer_load_16(rq, row_ok ? qoff + ks * 32 : qoff));
  }

  // ---- tile staging: per-thread byte offsets inside a tile never change; tile t adds t*64 rows.
  // K: thread tid moves 16-byte chunk (tid % (D/8)) of key rows tid/(D/8) + i*KSTRIDE, i < KPT.
  constexpr int KSTRIDE = NT / (D / 8);
  const int key0 = tid / (D / 8), ch0 = (tid % (D / 8)) * 8;
  const uint32_t koff0 = (uint32_t)(key0 * a.k_ss * 2 + ch0 * 2), kstep = (uint32_t)(KSTRIDE * a.k_ss * 2);
  const int klds0 = key0 * KROW + ch0;
  const uint32_t k_tile_bytes = (uint32_t)(kTK * a.k_ss * 2), v_tile_bytes = (uint32_t)(kTK * a.v_ss * 2);
  // V: thread moves keys 4*vkq .. 4*vkq+3 x channels vcg*CPT .. +CPT and writes them transposed;
  // within each 16-key group the 4-key chunks are stored as 0, 2, 1, 3 (the P^T operand order)
  const int vkq = tid & 15, vcg = tid >> 4;
  const uint32_t voff = (uint32_t)(4 * vkq * a.v_ss * 2 + vcg * CPT * 2), vrow = (uint32_t)(a.v_ss * 2);
  const int vpos = 16 * (vkq >> 2) + 4 * (((vkq & 1) << 1) | ((vkq >> 1) & 1));
  u32x4 kst[KPT];
  uint32_t vst[4][VW];

  auto load_tile = [&](int t) {
    rsrc_t rkt = rk, rvt = rv;
    uint32_t tk = (uint32_t)t * k_tile_bytes, tv = (uint32_t)t * v_tile_bytes;
    if constexpr (CHUNKED) {
      rkt = page_rsrc(a.k, a.k_pages, a.k_pool_pages, a.k_sb, a.k_sh, a.k_ss, t);
      rvt = page_rsrc(a.v, a.v_pages, a.v_pool_pages, a.v_sb, a.v_sh, a.v_ss, t);
      tk = tv = 0;
    }
    const uint32_t kb = koff0 + tk;
#pragma unroll
    for (int i = 0; i < KPT; ++i) kst[i] = buffer_load_16(rkt, kb + i * kstep);
    const uint32_t vb = voff + tv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (VW % 4 == 0) {
#pragma unroll
        for (int c4 = 0; c4 < VW; c4 += 4) {
          const u32x4 x = buffer_load_16(rvt, vb + r * vrow + c4 * 4);
          vst[r][c4] = x[0]; vst[r][c4 + 1] = x[1]; vst[r][c4 + 2] = x[2]; vst[r][c4 + 3] = x[3];
        }
      } else {
        static_assert(VW == 2, "4 channels per thread use one 8-byte load");
        const u32x2 x = buffer_load_8(rvt, vb + r * vrow);
        vst[r][0] = x[0]; vst[r][1] = x[1];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) *reinterpret_cast<u32x4*>(&k_lds[buf][klds0 + i * KSTRIDE * KROW]) = kst[i];
#pragma unroll
    for (int p = 0; p < VW; ++p) {
      const int c0 = vcg * CPT + 2 * p;
      const u32x2 even = {pack_lo16(vst[0][p], vst[1][p]), pack_lo16(vst[2][p], vst[3][p])};
      const u32x2 odd = {pack_hi16(vst[0][p], vst[1][p]), pack_hi16(vst[2][p], vst[3][p])};
      *reinterpret_cast<u32x2*>(&v_lds[buf][c0 * VROW + vpos]) = even;
      *reinterpret_cast<u32x2*>(&v_lds[buf][(c0 + 1) * VROW + vpos]) = odd;
    }
  };

  // ---- running state of this lane's query row
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  float m_true = neg_inf();  // running max of raw scores over kept tiles (the skip rule's m_{i-1})
  float m_ref = neg_inf();   // reference max of the exponentials (trails m_true by at most 8/c2)
  float l_part = 0.f;        // this lane's half of the softmax denominator
  int n_exec = 0;

  auto step = [&](int t, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int buf = t & 1;
    if (t + 1 < T) load_tile(t + 1);

    // S^T for keys t*64 .. t*64+63 (two 32-key blocks) x this wave's 32 query columns.  The two blocks'
    // MFMA chains alternate k-step by k-step and each k-step's K operands are read from LDS two k-steps
    // ahead, so neither an MFMA result nor an LDS read is waited for back to back.
    f32x16 s[2] = {f32x16{}, f32x16{}};
    {
      const uint16_t* kl = &k_lds[buf][col * KROW + half * 8];
      auto kop = [&](int kb, int ks) { return *reinterpret_cast<const u32x4*>(kl + kb * 32 * KROW + ks * 16); };
      u32x4 x[KSTEPS][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) x[ks][0] = kop(0, ks), x[ks][1] = kop(1, ks);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + 2 < KSTEPS) x[ks + 2][0] = kop(0, ks + 2), x[ks + 2][1] = kop(1, ks + 2);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's MFMAs
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x[ks][0]), qreg[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x[ks][1]), qreg[ks], s[1], 0, 0, 0);
      }
    }
    if constexpr (MASK) {
      // key offset o inside the tile is valid for this row iff o <= lim
      const int key_base = t * kTK;
      const int lim = !row_ok ? -1 : (a.causal ? iq + off - key_base : Sk - 1 - key_base);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int o = kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
          s[kb][i] = o <= lim ? s[kb][i] : neg_inf();
        }
    }
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmax3(mx, s[kb][i], s[kb][i + 1]);
    mx = pair_max(mx);

    // ---- the skip vote against the running max of the kept tiles so far
    const bool abstain = mx == neg_inf();
    const float gap = mx - m_true;  // +inf while the row has seen no valid key
    const uint64_t ball = wave_ballot(!abstain && !(gap < a.tau_raw));
    if (lane == 0) votes[buf][w] = ball != 0;
    if (a.unit_gap) {
      float gg = abstain ? neg_inf() : gap;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) gg = fmaxf(gg, __shfl_xor(gg, off, 64));
      if (lane == 0) wave_gap[buf][w] = gg;
    }
    __syncthreads();
    bool keep = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) keep |= votes[buf][i] != 0;
    if (tid == 0) {
      if (a.tile_state) a.tile_state[unit * a.nkt + t] = keep ? 1 : 2;
      if (a.unit_gap) {
        float gg = wave_gap[buf][0];
#pragma unroll
        for (int i = 1; i < NW; ++i) gg = fmaxf(gg, wave_gap[buf][i]);
        a.unit_gap[unit * a.nkt + t] = gg == __builtin_inff() ? gg : gg * a.scale;
      }
    }

    if (keep) {
      ++n_exec;
      // online softmax: advance the true max; move the reference max (and rescale) only when it trails by > 8
      m_true = fmaxf(m_true, mx);
      const bool move = (m_true - m_ref) * c2 > kRefSlack;  // also true while m_ref = -inf and m_true finite
      if (wave_ballot(move)) {
        const float alpha = move ? exp2_fast((m_ref - m_true) * c2) : 1.f;  // 0 when m_ref = -inf
        l_part *= alpha;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
        m_ref = move ? m_true : m_ref;
      }
      const float moff = (m_ref == neg_inf() ? 0.f : m_ref) * c2;
      // V^T operands of the first 16-key step, read now so that they land during the exponentials
      const uint16_t* vl = &v_lds[buf][col * VROW + 8 * half];
      auto vop = [&](int cb, int st) { return *reinterpret_cast<const u32x4*>(vl + cb * 32 * VROW + 16 * st); };
      u32x4 vx[4][CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) vx[0][cb] = vop(cb, 0);
      bf16x8 pb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float p0 = exp2_fast(fmaf(s[st >> 1][8 * (st & 1) + e], c2, -moff));
          const float p1 = exp2_fast(fmaf(s[st >> 1][8 * (st & 1) + e + 1], c2, -moff));
          pk[e >> 1] = pack_bf16x2(p0, p1);
          l_part = dot2_bf16_sum(pk[e >> 1], l_part);
        }
        pb[st] = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
      // O^T += V^T . P^T: the CB accumulator chains alternate step by step; the next step's operands are
      // read while the current step's MFMAs issue
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if (st + 1 < 4)
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) vx[st + 1][cb] = vop(cb, st + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's MFMAs
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vx[st][cb]), pb[st], acc[cb], 0, 0, 0);
      }
    }
    if (t + 1 < T) store_tile(buf ^ 1);
    __syncthreads();
  };

  load_tile(0);
  store_tile(0);
  // every load issued so far (Q operand, tile 0) has landed: without this the wait-count pass treats
  // the Q registers as pending inside the loop and stalls each QK^T MFMA on the next tile's prefetch
  wait_vmem_all();
  __syncthreads();
  for (int t = 0; t < T_in; ++t) step(t, false_type{});
  for (int t = T_in; t < T; ++t) step(t, true_type{});

  // ---- epilogue: O = acc / l, bf16
  const float l_tot = pair_sum(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* op = a.o + (CHUNKED ? (int64_t)(qrow0 + iq) * a.o_ss : (int64_t)b * a.o_sb + (int64_t)iq * a.o_ss) +
                   (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = cb * 32 + 8 * gq + 4 * half;
        const u32x2 x = {pack_bf16x2(acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv),
                         pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + ch) = x;
      }
  }
  if (tid == 0) {
    for (int t = T; t < a.nkt; ++t) {
      if (a.tile_state) a.tile_state[unit * a.nkt + t] = 0;
      if (a.unit_gap) a.unit_gap[unit * a.nkt + t] = __builtin_nanf("");
    }
    if (a.counters) {
      const unsigned long long visited = T;
      atomicAdd(&a.counters[0], visited);
      atomicAdd(&a.counters[1], visited - n_exec);
      atomicAdd(&a.counters[2], visited);
      atomicAdd(&a.counters[3], (unsigned long long)n_exec);
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int tile_q, bool chunked, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hq * a.nqt);
  if (grid == 0) return hipSuccess;
  const dim3 blk(tile_q * 2);
#define SSM_PREFILL_LAUNCH(D, TQ)                                                                        \
  if (d == D && tile_q == TQ) {                                                                          \
    if (chunked) hipLaunchKernelGGL((prefill_kernel<D, TQ, true>), dim3(grid), blk, 0, stream, a);       \
    else hipLaunchKernelGGL((prefill_kernel<D, TQ, false>), dim3(grid), blk, 0, stream, a);              \
    return hipGetLastError();                                                                            \
  }
  SSM_PREFILL_LAUNCH(128, 128)
  SSM_PREFILL_LAUNCH(128, 64)
  SSM_PREFILL_LAUNCH(64, 128)
  SSM_PREFILL_LAUNCH(64, 64)
#undef SSM_PREFILL_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssm
