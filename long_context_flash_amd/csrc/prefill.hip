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
//   exchange with lane^32 that holds the other 32 keys of the same query.
//   O^T (d x 32 queries) += V^T . P^T on the same MFMA.  The accumulator layout
//   of S^T is consumed directly as the P^T operand (converted to bf16 in
//   registers); V is staged in LDS transposed ([channel][key]) with the keys of
//   each 16-key group stored in the order that matches that accumulator layout,
//   so each operand is a single 16-byte LDS read.
//
// Skip vote: every lane votes "keep" unless its row abstains (no valid key in
// the tile) or its gap (tile max - running max) is below tau; a wave ballot
// and one LDS word per wave give the unit's decision at the tile barrier.  The
// running maximum only advances on kept tiles, which equals the prefix maximum
// over all visited tiles because tau <= 0 (a skipped tile is below it).
//
// Pipeline: K and V tiles are double-buffered in LDS; the global loads of tile
// t+1 are issued before tile t's MFMAs and written to LDS after them.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

constexpr int kTK = 64;

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

template <int D, int TQ>
__global__ __launch_bounds__(TQ * 2, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int NW = TQ / 32;          // waves per workgroup
  constexpr int NT = NW * 64;          // threads
  constexpr int KROW = D + 8;          // K tile row stride in LDS (elements); +16 B avoids bank conflicts
  constexpr int VROW = kTK + 8;        // V^T row stride in LDS (elements)
  constexpr int KSTEPS = D / 16;       // k-steps of the QK^T MFMA
  constexpr int CB = D / 32;           // 32-channel blocks of the output
  constexpr int KPT = kTK * D / 8 / NT;   // 16-byte K chunks per thread per tile
  constexpr int CPT = kTK * D / (NT * 4); // V channels per thread (4 keys each)
  constexpr int VW = CPT / 2;             // dwords per key row per thread
  static_assert(KPT >= 1 && CPT >= 4 && CPT % 4 == 0, "tile split");

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VROW];
  __shared__ uint32_t votes[NW];
  __shared__ float wave_gap[NW];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  int b, h, qt;
  map_prefill_unit(blockIdx.x, a, b, h, qt);
  const int g = h / a.G;
  const int S = a.S;
  const int q0 = qt * TQ;
  const int q_end = min(S, q0 + TQ);
  const int t_last = a.causal ? (q_end - 1) / kTK : a.nkt - 1;
  const int64_t unit = ((int64_t)b * a.Hq + h) * a.nqt + qt;

  // ---- Q operand: lane (col, half) holds Q[row][ks*16 + half*8 .. +8] for every k-step
  const int iq = q0 + w * 32 + col;
  const bool row_ok = iq < S;
  bf16x8 qreg[KSTEPS];
  {
    const uint16_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)(row_ok ? iq : 0) * a.q_ss + (int64_t)h * a.q_sh;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 x = row_ok ? ld_global_16(qp + ks * 16 + half * 8) : u32x4{0, 0, 0, 0};
      qreg[ks] = as_bf16x8(x);
    }
  }
  const int wave_q_lo = q0 + w * 32, wave_q_hi = min(q0 + w * 32 + 31, S - 1);

  // ---- tile staging (global -> registers -> LDS)
  const uint16_t* kb_ptr = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh;
  const uint16_t* vb_ptr = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh;
  u32x4 kst[KPT];
  uint32_t vst[4][VW];
  const int vkq = tid & 15, vcg = tid >> 4;  // 4-key group, channel group
  // keys 4*vkq..4*vkq+3 go to V^T positions in the order the P^T operand expects:
  // within each 16-key group the 4-key chunks are stored as 0, 2, 1, 3
  const int vpos = 16 * (vkq >> 2) + 4 * (((vkq & 1) << 1) | ((vkq >> 1) & 1));

  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT, key = c / (D / 8), ch = (c % (D / 8)) * 8;
      const int j = t * kTK + key;
      kst[i] = j < S ? ld_global_16(kb_ptr + (int64_t)j * a.k_ss + ch) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = t * kTK + 4 * vkq + r;
      const uint16_t* p = vb_ptr + (int64_t)(j < S ? j : 0) * a.v_ss + vcg * CPT;
      if constexpr (VW % 4 == 0) {
#pragma unroll
        for (int c4 = 0; c4 < VW; c4 += 4) {
          u32x4 x = j < S ? ld_global_16(p + c4 * 2) : u32x4{0, 0, 0, 0};
          vst[r][c4] = x[0]; vst[r][c4 + 1] = x[1]; vst[r][c4 + 2] = x[2]; vst[r][c4 + 3] = x[3];
        }
      } else {
        static_assert(VW == 2, "4 channels per thread use one 8-byte load");
        u32x2 x = j < S ? ld_global_8(p) : u32x2{0, 0};
        vst[r][0] = x[0]; vst[r][1] = x[1];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT, key = c / (D / 8), ch = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&k_lds[buf][key * KROW + ch]) = kst[i];
    }
#pragma unroll
    for (int p = 0; p < VW; ++p) {
      const int c0 = vcg * CPT + 2 * p;
      u32x2 even = {(vst[0][p] & 0xffffu) | (vst[1][p] << 16), (vst[2][p] & 0xffffu) | (vst[3][p] << 16)};
      u32x2 odd = {(vst[0][p] >> 16) | (vst[1][p] & 0xffff0000u), (vst[2][p] >> 16) | (vst[3][p] & 0xffff0000u)};
      *reinterpret_cast<u32x2*>(&v_lds[buf][c0 * VROW + vpos]) = even;
      *reinterpret_cast<u32x2*>(&v_lds[buf][(c0 + 1) * VROW + vpos]) = odd;
    }
  };

  // ---- running state of this lane's query row
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  float m_run = neg_inf();  // running max of raw scores over kept tiles
  float l_part = 0.f;       // this lane's half of the softmax denominator
  int n_exec = 0;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t <= t_last; ++t) {
    const int buf = t & 1;
    if (t < t_last) load_tile(t + 1);

    // S^T for this wave: keys t*64 .. t*64+63 (two 32-key blocks) x 32 query columns
    const int key0 = t * kTK;
    const bool wave_dead = !(wave_q_lo < S) || (a.causal && key0 > wave_q_hi);
    f32x16 s[2];
    float mx = neg_inf();
    if (!wave_dead) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 c = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          u32x4 x = *reinterpret_cast<const u32x4*>(&k_lds[buf][(kb * 32 + col) * KROW + ks * 16 + half * 8]);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x), qreg[ks], c, 0, 0, 0);
        }
        s[kb] = c;
      }
      // masking: causal diagonal tiles, the ragged last tile, padding rows
      const bool need_mask = (a.causal && key0 + kTK - 1 > wave_q_lo) || (key0 + kTK > S) || (wave_q_lo + 31 >= S);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = key0 + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool ok = row_ok && j < S && (!a.causal || j <= iq);
            if (!ok) s[kb][i] = neg_inf();
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = fmaxf(mx, swap_halves(mx));
    }

    // ---- the skip vote
    const bool abstain = mx == neg_inf();
    const float gap = mx - m_run;  // +inf on the first tile with a valid key
    const bool keep_vote = !abstain && !(gap < a.tau_raw);
    const uint64_t ball = wave_ballot(keep_vote);
    if (lane == 0) votes[w] = ball != 0;
    if (a.unit_gap) {
      float gg = abstain ? neg_inf() : gap;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) gg = fmaxf(gg, __shfl_xor(gg, off, 64));
      if (lane == 0) wave_gap[w] = gg;
    }
    __syncthreads();
    bool keep = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) keep |= votes[i] != 0;
    if (tid == 0) {
      if (a.tile_state) a.tile_state[unit * a.nkt + t] = keep ? 1 : 2;
      if (a.unit_gap) {
        float gg = wave_gap[0];
#pragma unroll
        for (int i = 1; i < NW; ++i) gg = fmaxf(gg, wave_gap[i]);
        a.unit_gap[unit * a.nkt + t] = gg == __builtin_inff() ? gg : gg * a.scale;
      }
    }

    if (keep) {
      ++n_exec;
      if (!wave_dead) {
        // online softmax update; rescale only when some row's maximum moved
        const float m_new = fmaxf(m_run, mx);
        if (wave_ballot(m_new > m_run)) {
          const float alpha = m_new > m_run ? exp2_fast((m_run - m_new) * a.scale_log2) : 1.f;
          l_part *= alpha;
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
          m_run = m_new;
        }
        const float moff = (m_run == neg_inf() ? 0.f : m_run) * a.scale_log2;
        bf16x8 pb[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = exp2_fast(s[st >> 1][8 * (st & 1) + e] * a.scale_log2 - moff);
            l_part += p[e];
          }
          u32x4 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
          pb[st] = as_bf16x8(pk);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            u32x4 x = *reinterpret_cast<const u32x4*>(&v_lds[buf][(cb * 32 + col) * VROW + 16 * st + 8 * half]);
            acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x), pb[st], acc[cb], 0, 0, 0);
          }
      }
    }
    if (t < t_last) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16
  const float l_tot = l_part + swap_halves(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)iq * a.o_ss + (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int ch = cb * 32 + 8 * gq + 4 * half;
        u32x2 x = {pack_bf16x2(acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv),
                   pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + ch) = x;
      }
  }
  if (tid == 0) {
    for (int t = t_last + 1; t < a.nkt; ++t) {
      if (a.tile_state) a.tile_state[unit * a.nkt + t] = 0;
      if (a.unit_gap) a.unit_gap[unit * a.nkt + t] = __builtin_nanf("");
    }
    if (a.counters) {
      const unsigned long long visited = t_last + 1;
      atomicAdd(&a.counters[0], visited);
      atomicAdd(&a.counters[1], visited - n_exec);
      atomicAdd(&a.counters[2], visited);
      atomicAdd(&a.counters[3], (unsigned long long)n_exec);
    }
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int d, int tile_q, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hq * a.nqt);
  if (grid == 0) return hipSuccess;
  if (d == 128 && tile_q == 128) hipLaunchKernelGGL((prefill_kernel<128, 128>), dim3(grid), dim3(256), 0, stream, a);
  else if (d == 128 && tile_q == 64) hipLaunchKernelGGL((prefill_kernel<128, 64>), dim3(grid), dim3(128), 0, stream, a);
  else if (d == 64 && tile_q == 128) hipLaunchKernelGGL((prefill_kernel<64, 128>), dim3(grid), dim3(256), 0, stream, a);
  else if (d == 64 && tile_q == 64) hipLaunchKernelGGL((prefill_kernel<64, 64>), dim3(grid), dim3(128), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ssm
