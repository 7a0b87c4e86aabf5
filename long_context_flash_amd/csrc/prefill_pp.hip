// prefill_pp.hip -- Skip Softmax prefill for gfx950, two units per workgroup in ping-pong.
//
// Same method and results as prefill_kernel (recap of "Accelerating Long-Context Inference with Skip Softmax
// in NVIDIA TensorRT-LLM": Key Points, Detailed Analysis, Skip Softmax Mechanism; news item: Understanding Skip
// Softmax): key tiles of 64 are scanned in ascending order; a tile whose score maximum trails the running
// maximum by more than tau in every row of the unit skips its exponentials and its P*V product.
//
// Shape served: head_dim 128, query tiles of 128 rows, an even number of query heads per KV head; bf16 Q and K,
// or (QK8) OCP e4m3 codes scored on v_mfma_f32_32x32x64_f8f6f4 as in prefill_kernel's QK8 form (K tiles as
// 8-bit rows in LDS, 4 MFMAs per tile instead of 16); V and P.V are bf16 either way.  One
// workgroup of 8 waves owns two units: query heads 2j and 2j+1 of one KV group on the same query tile, which
// scan the same key tiles.  Waves 0-3 (group A) own unit A's rows, waves 4-7 (group B) unit B's, 32 rows per
// wave; wave w runs on SIMD w % 4, so each SIMD holds one wave of each group.
//
// Every barrier interval is a phase.  In a matrix phase G(t) a wave issues the P.V MFMAs of tile t-2 (if its
// unit kept it) and the QK^T MFMAs of tile t; in a vector phase V(t) it decides tile t-1 from the votes its
// group wrote one vector phase earlier, computes that tile's exponentials if the unit keeps it, and takes tile
// t's row maxima and its vote.  Group B runs one phase behind group A, so on every SIMD one wave issues MFMAs
// while the other issues the VALU work (the two overlap: the MFMA rate is unchanged and the VALU slows by
// about a tenth):
//
//   phase 2t:    A: G(t)    B: V(t-1)
//   phase 2t+1:  A: V(t)    B: G(t)
//
// The vote of tile t compares its maxima with the running maximum of tiles < t; because tau <= 0 a skipped
// tile never holds a new maximum, so that is the prefix maximum of all visited tiles and does not depend on
// the decision of tile t-1.  The group's four vote words of tile t are written in V(t), published by the two
// barriers that follow and read behind the MFMAs at the end of G(t+1), so the decision in V(t+1) waits for
// nothing.
//
// The two units share every K and V tile in LDS (4 buffers each, 16 KB per tile; 8 KB per 8-bit K tile).  Group A's waves load the
// K tiles (K(t+3) behind the MFMAs of G(t)), group B's waves the V tiles (V(t+1) behind those of G(t); every
// visited tile, since either unit may keep it); a wave waits for its loads of a tile in the vector phase whose
// closing barrier publishes it (K(t+1) in V_A(t), V(t) in V_B(t)).  Tiles go HBM/L2 -> LDS with direct-to-LDS
// buffer loads in the swizzled layout of prefill_kernel; operands are read as there (K: ds_read_b128; V^T:
// ds_read_b64_tr_b16).
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

namespace {

constexpr int kTKpp = 64;
constexpr float kRefSlackPP = 8.f;  // log2 units the reference max may trail the true max
constexpr int kD = 128;
constexpr int kRowB = 2 * kD;       // bytes per key row in LDS
constexpr int kKS = kD / 16;        // k-steps of the QK^T MFMA
constexpr int kCB = kD / 32;        // 32-channel blocks of the output

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// LDS layout of a tile (as prefill_kernel at D = 128): key row r holds 256 bytes; its 16-byte chunk c sits at
// position c ^ swz(r).
__device__ __forceinline__ int pp_swz_k(int r) { return r & 15; }
// 8-bit K rows (128 bytes, QK8): chunk c of row r sits at position c ^ ((r >> 1) & 7)
__device__ __forceinline__ int pp_swz_k8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int pp_swz_v(int r) { return 4 * (r & 3); }

// Barrier without a memory fence: LDS writes of this wave are complete (lgkmcnt(0)); outstanding tile loads
// stay in flight (each wave waits for its own with vmcnt before the barrier that publishes them).
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// s_waitcnt vmcnt(n) with the other counters at their maxima
template <int N> __device__ __forceinline__ void pp_wait_vmem() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

__device__ __forceinline__ void pp_map_unit(int bid, const PrefillArgs& a, int& b, int& h0, int& qt) {
  const int pairs = a.G / 2;  // head pairs per KV group
  const int ngroups = a.B * a.Hkv;
  int level;
  if (((int64_t)ngroups * a.nqt) % 8 == 0) {
    // Block i runs on XCD i % 8.  Units go KV group by KV group, longest query tiles first inside a group: the
    // (group, level) pairs in that order are dealt round-robin to the 8 XCDs, and the head pairs of one (group,
    // level) run on one XCD in consecutive slots, so they share its L2 for the K/V stream.  At any time the
    // whole chip streams one group's K and V (64 MB at 128K keys), which the last-level cache holds.
    const int x = bid & 7, slot = bid >> 3;
    const int row = slot / pairs, pj = slot - row * pairs;
    const int m = row * 8 + x;  // = group * nqt + level
    const int grp = m / a.nqt;
    level = m - grp * a.nqt;
    b = grp / a.Hkv;
    h0 = (grp - b * a.Hkv) * a.G + 2 * pj;
  } else {
    const int per_level = a.B * (a.Hq / 2);
    level = bid / per_level;
    const int rem = bid - level * per_level;
    b = rem / (a.Hq / 2);
    h0 = 2 * (rem - b * (a.Hq / 2));
  }
  qt = a.nqt - 1 - level;  // longest causal units first
}

}  // namespace

// POT: Rowmax-PoT weights 2^(rint(c2*S) - kref) in place of the exponentials (kref an integer reference that
// trails the rounded row maximum by at most kRefSlackPP; the output and row sums are invariant to its choice).
// QK8: q and k hold e4m3 codes (strides count bytes); their scales are folded into the logit scale.
template <bool POT, bool QK8>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillArgs a) {
  constexpr int ESK = QK8 ? 1 : 2;  // bytes per Q and K element
  constexpr int KS8 = kD / 64;      // k-steps of the fp8 QK^T MFMA
  constexpr int LK = QK8 ? 2 : 4;   // K tile loads per wave of group A
  // four K and four V tile buffers, each one array so that a buffer's offset from the first is a constant
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf[4][kTKpp * kD];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf[4][kTKpp * kD];
  // per tile parity and group: one word whose byte w is wave w's keep vote (0 or 1), so that one read gives the
  // group's decision; and, only when unit gaps are recorded, each wave's unit gap
  __shared__ __attribute__((aligned(16))) uint32_t votes[2][2];
  __shared__ __attribute__((aligned(16))) float vgaps[2][2][4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w >> 2, wl = w & 3;
  const int col = lane & 31, half = lane >> 5;

  int b, h0, qt;
  pp_map_unit(blockIdx.x, a, b, h0, qt);
  const int h = h0 + grp;
  const int g = h0 / a.G;
  const int64_t unit = ((int64_t)b * a.Hq + h) * a.nqt + qt;
  const int q0 = qt * 128;
  const int S = a.S;
  const int q_end = min(S, q0 + 128);
  const int T = a.causal ? (q_end - 1) / kTKpp + 1 : (S + kTKpp - 1) / kTKpp;  // visited key tiles (both units)
  const int full_tiles = S / kTKpp;
  // tiles [0, T_in) have every (row, key) pair valid: no masking code runs for them
  const int T_in = q_end < q0 + 128 ? 0 : min(T, a.causal ? min((q0 + 1) / kTKpp, full_tiles) : full_tiles);
  const float c2 = a.scale_log2;

  auto qk_rows_bytes = [&](int n, int64_t ss, int es) {
    return n <= 0 ? 0u : (uint32_t)(((int64_t)(n - 1) * ss + kD) * es);
  };
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q);
  const uint8_t* k8 = reinterpret_cast<const uint8_t*>(a.k);
  const rsrc_t rq = make_rsrc(q8 + ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh) * ESK, qk_rows_bytes(S, a.q_ss, ESK));
  const rsrc_t rk = make_rsrc(k8 + ((int64_t)b * a.k_sb + (int64_t)g * a.k_sh) * ESK, qk_rows_bytes(S, a.k_ss, ESK));
  const rsrc_t rv = make_rsrc(a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh, qk_rows_bytes(S, a.v_ss, 2));

  // ---- Q operand: lane (col, half) holds Q[row][ks*16 + half*8 .. +8] (QK8: the 32 codes Q[row][ks*64 +
  // half*32 .. +32])
  const int iq = q0 + wl * 32 + col;
  const bool row_ok = iq < S;
  bf16x8 qreg[QK8 ? 1 : kKS];
  i32x8 qreg8[QK8 ? KS8 : 1];
  {
    const uint32_t qoff = row_ok ? (uint32_t)iq * (uint32_t)(a.q_ss * ESK) + half * (QK8 ? 32 : 16) : 0xffffffffu;
    if constexpr (QK8) {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const u32x4 lo = buffer_load_16(rq, row_ok ? qoff + ks * 64 : qoff);
        const u32x4 hi = buffer_load_16(rq, row_ok ? qoff + ks * 64 + 16 : qoff);
        qreg8[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) qreg[ks] = as_bf16x8(buffer_load_16(rq, row_ok ? qoff + ks * 32 : qoff));
    }
  }

  // ---- tile loads straight into LDS.  The four waves of a group fill one 16 KB tile: load i of wave wl fills
  // LDS bytes [(wl*4 + i) KB, +1 KB), i.e. key rows 4(wl*4 + i) .. +3; lane l the 16 bytes at l*16 of it
  // (row 4(wl*4+i) + l/16, chunk position l%16, which holds the logical chunk (l%16) ^ swz(row)).
  const int lrow = lane >> 4, lpos = lane & 15;
  const uint32_t k_row_bytes = (uint32_t)(a.k_ss * ESK), v_row_bytes = (uint32_t)(a.v_ss * 2);
  const uint32_t k_tile_bytes = kTKpp * k_row_bytes, v_tile_bytes = kTKpp * v_row_bytes;
  // K: swz_k(row) = row & 15 = (4(wl*4+i)) & 15 | lrow -> chunk = lpos ^ lrow ^ (that load's part).  QK8: the
  // 8 KB tile in 2 loads per wave, load i of wave wl holding rows 16wl + 8i + lane/8, chunk position lane%8;
  // swz_k8(row) = (4(i & 1)) | (lane >> 4), so chunk = (lane%8) ^ (lane >> 4) ^ 4(i & 1)
  uint32_t k_dma = QK8 ? (uint32_t)(wl * 16 + (lane >> 3)) * k_row_bytes : (uint32_t)(wl * 16 + lrow) * k_row_bytes;
  uint32_t k_dmx = QK8 ? (uint32_t)((lane & 7) ^ (lane >> 4)) * 16 : (uint32_t)(lpos ^ pp_swz_k(lrow)) * 16;
  // V: swz_v(row) = 4 (row & 3) = 4 lrow: no load-index part
  uint32_t v_dma = (uint32_t)(wl * 16 + lrow) * v_row_bytes + (uint32_t)(lpos ^ pp_swz_v(lrow)) * 16;
  // this wave's part of a tile buffer (key rows 16 wl .. 16 wl + 15) starts wl * LK KB in (4 KB of bf16 rows,
  // 2 KB of 8-bit rows); an opaque copy per call keeps the compiler from holding every buffer's destination
  // addresses in scalar registers across the loop
  auto load_k = [&](uint16_t* dst, int t) {
    const uint32_t toff = (uint32_t)t * k_tile_bytes;
    int wofs = wl * LK * 1024;
    asm volatile("" : "+s"(wofs));
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      // wave-uniform part of the swizzle
      const uint32_t cx = QK8 ? (uint32_t)(4 * (i & 1)) * 16 : (uint32_t)pp_swz_k((wl * 4 + i) * 4) * 16;
      const uint32_t vo = k_dma + (k_dmx ^ cx) + (uint32_t)(i * (QK8 ? 8 : 4)) * k_row_bytes + toff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)((char*)dst + wofs + i * 1024), 16, vo, 0, 0, 0);
    }
  };
  auto load_v = [&](uint16_t* dst, int t) {
    const uint32_t toff = (uint32_t)t * v_tile_bytes;
    int wofs = wl * 4096;
    asm volatile("" : "+s"(wofs));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t vo = v_dma + (uint32_t)(i * 4) * v_row_bytes + toff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)((char*)dst + wofs + i * 1024), 16, vo, 0, 0, 0);
    }
  };

  // ---- operand reads (prefill_kernel's bf16 forms at D = 128)
  // K (S^T's A operand): lane (col, half) reads row kb*32 + col, logical chunk 2ks + half:
  // byte (kb*32 + col)*256 + 16*((2ks + half) ^ (col & 15)) = (k_opb ^ 32 ks) + kb*32*256
  // QK8: lane (col, half) reads row kb*32 + col, logical chunks 4ks + 2half and 4ks + 2half + 1 (32 codes):
  // bytes (kb*32 + col)*128 + 16*((4ks + 2half + j) ^ swz_k8(col)) = (k_opb ^ 16*(4ks + j)) + kb*32*128
  const int xk = QK8 ? pp_swz_k8(col) : (col & 15);
  uint32_t k_opb = QK8 ? (uint32_t)(col * kD + 16 * ((2 * half) ^ xk))
                       : (uint32_t)(col * kRowB + 32 * (xk >> 1) + 16 * (half ^ (xk & 1)));
  // V^T (O^T's A operand) by transposing reads: in each 16-lane group, lane 4j + m names channels 4m..4m+3 of
  // the group's 16 and key row k0 + j, and receives channel (lane & 15) of the 4 rows
  const int gq = lane >> 4, li = lane & 15;
  const int vrow = li >> 2;
  const int vch = 16 * (gq & 1) + 4 * (li & 3);
  uint32_t v_opb = (uint32_t)(vrow * kRowB + 64 * (pp_swz_v(vrow) >> 2) + 16 * (vch >> 3) + 2 * (vch & 7));
  // the lane's operand offsets for every k-step and channel block, computed once: the buffer and key-block
  // parts of each address are then constants that the LDS reads take as immediate offsets (the V buffers lie
  // past 64 KB, so their first buffer's address is folded into the register)
  // (QK8: k-step ks, 16-byte half j at kxo[2 ks + j])
  constexpr int NKX = QK8 ? 2 * KS8 : kKS;
  uint32_t kxo[NKX], vxo[kCB];
#pragma unroll
  for (int i = 0; i < NKX; ++i) kxo[i] = QK8 ? k_opb ^ (64u * (i >> 1) + 16u * (i & 1)) : k_opb ^ (32u * i);
  const uint32_t vbuf0 = (uint32_t)(uintptr_t)(lds_ptr_t)(&vbuf[0][0]);
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) vxo[cb] = vbuf0 + (v_opb ^ (64u * cb)) + 4 * (gq >> 1) * kRowB;
  auto kop = [&](const uint16_t* kl, int ks, int kb) {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kl) + (kxo[ks] + kb * 32 * kRowB));
  };
  auto kop8 = [&](const uint16_t* kl, int ks, int kb) {
    const char* base = reinterpret_cast<const char*>(kl) + kb * 32 * kD;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + kxo[2 * ks]);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + kxo[2 * ks + 1]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto vop = [&](const uint16_t* vl, int cb, int st) {
    // half hf of the S^T accumulator holds keys 4hf..4hf+3 and 8+4hf..8+4hf+3 of each 16-key step
    typedef __attribute__((address_space(3))) char lds_char;
    const int boff = (int)(reinterpret_cast<const char*>(vl) - reinterpret_cast<const char*>(&vbuf[0][0]));
    lds_char* base = (lds_char*)(uintptr_t)vxo[cb] + (boff + 16 * st * kRowB);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)base);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(base + 8 * kRowB));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto refresh = [&]() {
    asm volatile("" : "+v"(k_opb), "+v"(k_dma), "+v"(k_dmx), "+v"(v_dma));
#pragma unroll
    for (int i = 0; i < NKX; ++i) asm volatile("" : "+v"(kxo[i]));
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) asm volatile("" : "+v"(vxo[cb]));
  };

  // ---- running state of this lane's query row
  f32x16 acc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = f32x16{};
  float m_run = neg_inf();  // max of the row's scores over the tiles voted on so far (the skip rule's m_{i-1})
  float m_ref = neg_inf();  // reference max of the exponentials (trails the true max by at most 8/c2); POT: the
                            // integer reference in base-2 log-weight units (trails rint(c2*max) by at most 8)
  // this lane's half of the softmax denominator in two chains, weight pairs alternating, exactly as
  // prefill_kernel sums it, so the two kernels give the same bits
  float l_part[2] = {0.f, 0.f};
  // the weights' offset: c2 * m_ref (POT: m_ref), 0 while m_ref = -inf
  float moff = 0.f;
  int n_exec = 0;
  f32x16 s[2][2];           // S^T of the tiles of parity 0 / 1, key blocks 0 / 1
  uint32_t pk[4][4];        // P^T operands of the pending tile
  bool pv_pending = false;  // the tile decided in the last vector phase was kept: its P.V is due
  bool pv_resc = false;
  float pv_alpha = 1.f;
  uint32_t vw_in = 0u;      // the group's vote word on the tile before the current one, read at the end of G
  float vg_in[4];           // the waves' unit gaps on it (read only when recorded)

  // S^T(t) = K(t) Q^T: two independent chains (key blocks), operands read two MFMAs ahead
  auto qk = [&](const uint16_t* kl, f32x16 (&st)[2]) {
    if constexpr (QK8) {
      constexpr int NM = 2 * KS8;
      i32x8 x[NM];
#pragma unroll
      for (int j = 0; j < NM; ++j) x[j] = kop8(kl, j >> 1, j & 1);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        const int ks = j >> 1, kb = j & 1;
        st[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x[j], qreg8[ks], ks == 0 ? f32x16{} : st[kb], 0, 0, 0,
                                                                 0, 0, 0);
      }
      return;
    }
    constexpr int NM = 2 * kKS;
    u32x4 x[NM];
    x[0] = kop(kl, 0, 0);
    x[1] = kop(kl, 0, 1);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (j + 2 < NM) x[j + 2] = kop(kl, (j + 2) >> 1, (j + 2) & 1);
      __builtin_amdgcn_sched_barrier(0);
      const int ks = j >> 1, kb = j & 1;
      st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x[j]), qreg[ks], ks == 0 ? f32x16{} : st[kb], 0, 0, 0);
    }
  };
  // O^T += V^T P^T: four chains (channel blocks)
  auto pv = [&](const uint16_t* vl) {
    constexpr int NM = 4 * kCB;
    if (pv_resc) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) acc[cb] *= pv_alpha;
    }
    bf16x8 vx[NM];
    vx[0] = vop(vl, 0, 0);
    vx[1] = vop(vl, 1, 0);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (j + 2 < NM) vx[j + 2] = vop(vl, (j + 2) % kCB, (j + 2) / kCB);
      __builtin_amdgcn_sched_barrier(0);
      const int st = j / kCB, cb = j % kCB;
      const bf16x8 pb = as_bf16x8(u32x4{pk[st][0], pk[st][1], pk[st][2], pk[st][3]});
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vx[j], pb, acc[cb], 0, 0, 0);
    }
  };
  // key offset o inside tile t is valid for this row iff o <= lim
  auto mask = [&](f32x16 (&st)[2], int t) {
    const int lim = (!row_ok ? -1 : (a.causal ? iq - t * kTKpp : S - 1 - t * kTKpp)) - 4 * half;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kb][i] = kb * 32 + 8 * (i >> 2) + (i & 3) <= lim ? st[kb][i] : neg_inf();
  };
  auto row_max = [&](const f32x16 (&st)[2]) {
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmax3(mx, st[kb][i], st[kb][i + 1]);
    return pair_max_nonan(mx);
  };

  // ---- phase bodies (the LDS buffers and score buffers are static in every instance).
  typedef volatile __attribute__((address_space(3))) uint32_t lds_u32;
  typedef volatile __attribute__((address_space(3))) uint8_t lds_u8;
  typedef volatile __attribute__((address_space(3))) float lds_f32;
  // G(t): the P.V of tile t-2 if kept, then S(t); behind the MFMAs, the read of the group's votes on tile t-1
  // (written in V(t-1)) and this group's tile loads: group A K(t+3) (into K(t-1)'s buffer), group B V(t+1) (into
  // V(t-3)'s); the last readers of those buffers finished in earlier phases.
  auto gemm = [&](int t, f32x16 (&st)[2], const uint16_t* kl, const uint16_t* vl_pv, uint16_t* k_dst, uint16_t* v_dst) {
    refresh();
    __builtin_amdgcn_s_setprio(1);
    if (pv_pending) pv(vl_pv);
    pv_pending = false;
    if (t < T) qk(kl, st);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (t >= 1 && t - 1 < T) {
      vw_in = *(lds_u32*)&votes[(t - 1) & 1][grp];
      if (a.unit_gap) {
        lds_f32* vg = (lds_f32*)&vgaps[(t - 1) & 1][grp][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) vg_in[i] = vg[i];
      }
    }
    if (grp == 0) {
      if (t + 3 < T) load_k(k_dst, t + 3);
    } else {
      if (t + 1 < T && t + 1 >= 2) load_v(v_dst, t + 1);
    }
  };
  // V(t): the unit's decision on tile t-1 from the votes the group wrote in the previous vector phase (published
  // by the barriers since and read at the end of G(t)), its exponentials if kept; then tile t's maxima and this
  // wave's vote; then this wave's wait for the tile loads the barrier ending the phase publishes.
  auto vec = [&](int t, f32x16 (&sprev)[2], f32x16 (&scur)[2]) {
    refresh();
    const int tp = t - 1;
    if (tp >= 0 && tp < T) {
      // every lane read the same words: made wave-uniform, so the keep branch is a scalar branch
      const bool keep = __builtin_amdgcn_readfirstlane(vw_in) != 0;
      if (wl == 0 && lane == 0) {
        if (a.tile_state) a.tile_state[unit * a.nkt + tp] = keep ? 1 : 2;
        if (a.unit_gap) {
          const float ug = fmaxf(fmaxf(vg_in[0], vg_in[1]), fmaxf(vg_in[2], vg_in[3]));
          a.unit_gap[unit * a.nkt + tp] = ug == __builtin_inff() ? ug : ug * a.scale;
        }
      }
      if (keep) {
        ++n_exec;
        // m_run includes tile tp (updated at its vote) and no later tile; move the reference max only when it
        // trails by more than the slack (rare: the rescale, and the weights' offset moff, change only then)
        float kn = 0.f;
        bool move;
        if constexpr (POT) {
          kn = rintf(m_run * c2);              // -inf while the row has no valid key
          move = kn - m_ref > kRefSlackPP;      // also true while m_ref = -inf and kn finite
        } else {
          move = (m_run - m_ref) * c2 > kRefSlackPP;  // also true while m_ref = -inf and m_run finite
        }
        pv_resc = wave_ballot(move) != 0;
        if (pv_resc) {
          float alpha;
          if constexpr (POT) {
            alpha = move ? (m_ref == neg_inf() ? 0.f : ldexpf(1.f, (int)(m_ref - kn))) : 1.f;  // exact
            m_ref = move ? kn : m_ref;
            moff = m_ref == neg_inf() ? 0.f : m_ref;
          } else {
            alpha = move ? exp2_fast((m_ref - m_run) * c2) : 1.f;  // 0 when m_ref = -inf
            m_ref = move ? m_run : m_ref;
            moff = (m_ref == neg_inf() ? 0.f : m_ref) * c2;
          }
          pv_alpha = alpha;
          l_part[0] *= alpha;
          l_part[1] *= alpha;
        }
#pragma unroll
        for (int n = 0; n < 32; n += 2) {
          const int stp = n >> 3, e = n & 7;  // 16-key step, position inside it (P^T operand order)
          const float s0 = sprev[stp >> 1][8 * (stp & 1) + e], s1 = sprev[stp >> 1][8 * (stp & 1) + e + 1];
          if constexpr (POT) {
            pk[stp][e >> 1] = pot_pack_sum_bf16x2(s0, s1, c2, moff, l_part[(n >> 1) & 1]);
          } else {
            // the row sums add the fp32 weights (two plain adds cost less energy than one bf16 dot product)
            const float p0 = exp2_fast(fmaf(s0, c2, -moff)), p1 = exp2_fast(fmaf(s1, c2, -moff));
            pk[stp][e >> 1] = pack_bf16x2(p0, p1);
            l_part[(n >> 1) & 1] += p0 + p1;
          }
        }
        pv_pending = true;
      }
    }
    if (t >= 0 && t < T) {  // group B's first phase is V(-1): nothing to vote on yet
      if (t >= T_in) mask(scur, t);
      const float mx = row_max(scur);
      const bool abstain = mx == neg_inf();
      const float gap = mx - m_run;  // +inf while the row has seen no valid key
      // the vote: 1 iff some lane votes to keep, i.e. is not abstaining and has !(gap < tau) (the lane masks of
      // the two comparisons ANDed in scalar registers); the wave's unit gap only when it is recorded
      const uint64_t bal = __builtin_amdgcn_fcmpf(mx, neg_inf(), 6 /* ordered, not equal */) &
                           __builtin_amdgcn_fcmpf(gap, a.tau_raw, 11 /* unordered or >= */);
      // (every lane stores the same byte to the same address: no divergent branch around the store)
      ((lds_u8*)&votes[t & 1][grp])[wl] = bal != 0 ? 1 : 0;
      if (a.unit_gap) {
        float gg = abstain ? neg_inf() : gap;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) gg = fmaxf(gg, __shfl_xor(gg, o, 64));
        if (lane == 0) ((lds_f32*)&vgaps[t & 1][grp][0])[wl] = gg;
      }
      m_run = max_nonan(m_run, mx);  // tau <= 0: a skipped tile never raises it, so this is the running max
    }
    // this wave's loads of the tile the barrier ending the phase publishes have landed.  Group A: K(t+1) (issued
    // in G(t-2); K(t+2), K(t+3) may stay in flight).  Group B: V(t) (issued in G(t-1); V(t+1) may stay in flight).
    if (grp == 0) {
      if (t + 3 < T) pp_wait_vmem<2 * LK>();
      else if (t + 2 < T) pp_wait_vmem<LK>();
      else pp_wait_vmem<0>();
    } else {
      if (t + 1 < T) pp_wait_vmem<4>();
      else pp_wait_vmem<0>();
    }
  };

  // ---- prologue: K(0..2) by group A, V(0..1) by group B, all visible before the first phase (V(2) onward are
  // issued in the matrix phases)
  if (T > 0) {
    if (grp == 0) {
      load_k(kbuf[0], 0);
      if (T > 1) load_k(kbuf[1], 1);
      if (T > 2) load_k(kbuf[2], 2);
    } else {
      load_v(vbuf[0], 0);
      if (T > 1) load_v(vbuf[1], 1);
    }
  }
  wait_vmem_all();  // Q and the first tiles
  pp_barrier();

  // ---- phases p = 0 .. 2T+3: A runs G(t) at p = 2t and V(t) at p = 2t+1; B one phase later (the last P.V, of
  // tile T-1, runs in G(T+1)).  Unrolled by four tiles so that the LDS buffers (tile t: buffer t % 4) and the
  // score buffers (tile t: s[t % 2]) of every body are static; each group runs its own copy of the loop, so
  // that the compiler sees the strict alternation of its phases; both copies pass the same barriers.
  const int nphase = 2 * T + 4;
#define K_BUF(o) (kbuf[((o) + 4) & 3])
#define V_BUF(o) (vbuf[((o) + 4) & 3])
  // A: G(t0 + SUB/2) for even SUB, V(t0 + SUB/2) for odd
#define SSM_PP_PHASE_A(SUB)                                                                     \
    if (p0 + SUB < nphase) {                                                                      \
      constexpr int tt = SUB / 2;                                                                 \
      if (SUB % 2 == 0) gemm(t0 + tt, s[tt & 1], K_BUF(tt), V_BUF(tt + 2), K_BUF(tt + 3), V_BUF(tt + 1)); \
      else vec(t0 + tt, s[(tt + 1) & 1], s[tt & 1]);                                              \
      pp_barrier();                                                                               \
    }
  // B: G(t0 + SUB/2) for odd SUB, V(t0 + SUB/2 - 1) for even
#define SSM_PP_PHASE_B(SUB)                                                                     \
    if (p0 + SUB < nphase) {                                                                      \
      constexpr int tt = SUB % 2 ? SUB / 2 : SUB / 2 - 1;                                         \
      if (SUB % 2 == 1) gemm(t0 + tt, s[(tt + 2) & 1], K_BUF(tt), V_BUF(tt + 2), K_BUF(tt + 3), V_BUF(tt + 1)); \
      else vec(t0 + tt, s[(tt + 3) & 1], s[(tt + 2) & 1]);                                        \
      pp_barrier();                                                                               \
    }
  if (grp == 0) {
    for (int p0 = 0; p0 < nphase; p0 += 8) {
      const int t0 = p0 >> 1;  // multiple of 4
      SSM_PP_PHASE_A(0) SSM_PP_PHASE_A(1) SSM_PP_PHASE_A(2) SSM_PP_PHASE_A(3)
      SSM_PP_PHASE_A(4) SSM_PP_PHASE_A(5) SSM_PP_PHASE_A(6) SSM_PP_PHASE_A(7)
    }
  } else {
    for (int p0 = 0; p0 < nphase; p0 += 8) {
      const int t0 = p0 >> 1;
      SSM_PP_PHASE_B(0) SSM_PP_PHASE_B(1) SSM_PP_PHASE_B(2) SSM_PP_PHASE_B(3)
      SSM_PP_PHASE_B(4) SSM_PP_PHASE_B(5) SSM_PP_PHASE_B(6) SSM_PP_PHASE_B(7)
    }
  }
#undef SSM_PP_PHASE_A
#undef SSM_PP_PHASE_B
#undef K_BUF
#undef V_BUF

  // ---- epilogue: O = acc / l, bf16
  const float l_tot = pair_sum(l_part[0] + l_part[1]);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)iq * a.o_ss + (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int gq4 = 0; gq4 < 4; ++gq4) {
        const int ch = cb * 32 + 8 * gq4 + 4 * half;
        const u32x2 x = {pack_bf16x2(acc[cb][4 * gq4] * inv, acc[cb][4 * gq4 + 1] * inv),
                         pack_bf16x2(acc[cb][4 * gq4 + 2] * inv, acc[cb][4 * gq4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + ch) = x;
      }
  }
  if (wl == 0 && lane == 0) {
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

hipError_t launch_prefill_pp(const PrefillArgs& a, bool qk8, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * (a.Hq / 2) * a.nqt);
  if (grid == 0) return hipSuccess;
  if (a.G % 2 != 0) return hipErrorInvalidValue;
  if (qk8 && a.pot) hipLaunchKernelGGL((prefill_pp_kernel<true, true>), dim3(grid), dim3(512), 0, stream, a);
  else if (qk8) hipLaunchKernelGGL((prefill_pp_kernel<false, true>), dim3(grid), dim3(512), 0, stream, a);
  else if (a.pot) hipLaunchKernelGGL((prefill_pp_kernel<true, false>), dim3(grid), dim3(512), 0, stream, a);
  else hipLaunchKernelGGL((prefill_pp_kernel<false, false>), dim3(grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ssm
