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
//   registers).
//
// Tiles go from HBM straight into LDS (buffer loads with an LDS destination,
// no registers): key-row major, 16-byte chunks XOR-swizzled per row.  The K
// operand is one 16-byte read per lane; the V^T operand is gathered by two
// transposing reads (ds_read_b64_tr_b16) in the key order of the S^T
// accumulator.  Rows past the sequence end fall outside the buffer resource and
// land as zeros, so loads carry no predication.
//
// Skip vote: every lane votes "keep" unless its row abstains (no valid key in
// the tile) or its gap (tile max - running max) is below tau; a wave ballot
// and one LDS word per wave give the unit's decision at the tile barrier.  The
// running maximum only advances on kept tiles; because tau <= 0 a skipped tile
// never holds a new maximum, so this equals the prefix maximum over all
// visited tiles.
//
// Pipeline (one barrier per tile): S(t) and the vote on tile t; barrier; the
// decision; the loads of K(t+2) and, only for a kept tile, V(t); then the
// exponentials of tile t issued between the P*V MFMAs of the previous kept
// tile t-1, so the transcendental work of one tile overlaps the matrix work of
// the other inside each wave.  Tiles wholly inside the causal triangle run
// without masking code; only the diagonal/ragged tiles mask.
//
// FP8 cache for the chunked prefill (KV8): K and V pages hold e4m3 codes; their tiles sit in LDS as 8-bit
// rows and every operand read converts its 8 codes exactly to bf16 (K: one 8-byte read; V^T: one 8-bit
// transposing read, ds_read_b64_tr_b8, of 8 key rows), so the bf16 MFMAs and the rest are unchanged.  The
// key scale joins the logit scale, the value scale multiplies the output.
//
// FP8 scores (QK8): Q and K as OCP e4m3 codes with one dequantisation scale each (folded into the logit
// scale); S^T on v_mfma_f32_32x32x64_f8f6f4, twice the bf16 rate, for the QK^T that every visited tile
// pays.  K tiles sit in LDS as 8-bit rows (D bytes); each lane reads 32 bytes of one key row per MFMA, and
// Q and K use the same channel order (any order gives the same dot products).  V, P and P.V stay bf16.
// Both together (the chunked prefill with 8-bit queries over fp8 pages): the K pages already sit in LDS as
// the QK8 rows, so the scores take the QK8 reads and MFMA, and V takes the KV8 reads and conversions.
//
// Exponentials use a lazily moved reference maximum: P = 2^(S*c - m_ref*c) with
// m_ref only raised when the true running maximum exceeds it by more than 8
// (log2 units), which bounds P by 256 and makes the rescale of the output
// accumulator rare.  The row sums add the fp32 weights, before their rounding
// to the bf16 P that enters the P*V product: two plain adds per pair draw less
// energy than one bf16 dot product of the rounded pair, and on this
// power-limited board that is 3% of the launch.  Rowmax-PoT weights are exact
// powers of two, built in fp32 and summed the same way.  The skip vote always
// uses the true running maximum.
#include "ssm_device.h"
#include "ssm_launch.h"

namespace ssm {

constexpr int kTK = 64;
constexpr float kRefSlack = 8.f;  // log2 units the reference max may trail the true max

__device__ __forceinline__ void map_prefill_unit(int bid, const PrefillArgs& a, int& b, int& h, int& qt) {
  const int ngroups = a.B * a.Hkv;
  int level;
  if (((int64_t)ngroups * a.nqt) % 8 == 0) {
    // Workgroups are dispatched round-robin over the 8 XCDs: block i runs on XCD i % 8.  Units go KV group
    // by KV group, longest query tiles first inside a group: the (group, level) pairs in that order are dealt
    // round-robin to the XCDs, and the query heads of one (group, level) run on one XCD in consecutive slots,
    // sharing its L2 for the K/V stream.  At any time the chip streams one group's K and V, which the
    // last-level cache holds.
    const int x = bid & 7, slot = bid >> 3;
    const int row = slot / a.G, hh = slot - row * a.G;
    const int m = row * 8 + x;  // = group * nqt + level
    const int grp = m / a.nqt;
    level = m - grp * a.nqt;
    b = grp / a.Hkv;
    h = (grp - b * a.Hkv) * a.G + hh;
  } else {
    const int per_level = a.B * a.Hq;
    level = bid / per_level;
    const int rem = bid - level * per_level;
    b = rem / a.Hq;
    h = rem - b * a.Hq;
  }
  qt = a.nqt - 1 - level;  // longest causal units first
}

// LDS tile layout: key row r of a K or V tile occupies 2*D bytes; its 16-byte chunk c (channels 8c..8c+7)
// sits at chunk position c ^ swz(r).  K: 16 consecutive rows read at one logical chunk (one 16-lane
// phase of an operand read) land on 16 distinct positions.  V: the 4 rows gathered by one transposing
// read land on 4 distinct 4-chunk groups.
template <int D> __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
// 8-bit K tile (rows of D bytes): the 16 rows of one 16-lane phase of an operand read hit 16 distinct 4-bank groups
template <int D> __device__ __forceinline__ int swz_k8(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
// 8-bit V tile: the 8 key rows r0..r0+3, r0+8..r0+11 (r0 % 4 == 0) that one 16-lane group of a transposing read
// gathers land on distinct 4-bank groups
template <int D> __device__ __forceinline__ int swz_v8(int r) {
  return D == 128 ? (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) : ((r >> 3) & 1);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// CHUNKED: queries of each sequence are the last ones of its cached keys (bottom-right causal), packed
// ragged rows of q/o, K/V read through a page table (see PrefillArgs).  MODE 0: bf16; 1 (QK8): q and k hold
// e4m3 codes, QK^T on the fp8 MFMA; 2 (KV8, chunked only): the K/V pages hold e4m3 codes; 3 (chunked only):
// both, i.e. e4m3 queries scored on the fp8 MFMA against e4m3 key pages, V pages converted as in 2.
// POT: Rowmax-PoT weights 2^(rint(c2*S) - kref) in place of the exponentials, kref an integer reference moved
// like m_ref (the output and row sums are invariant to its choice, and the rescale is an exact power of two).
template <int D, int TQ, bool CHUNKED, int MODE, bool POT>
__global__ __launch_bounds__(TQ * 2, 2) void prefill_kernel(PrefillArgs a) {
  constexpr bool QK8 = MODE == 1 || MODE == 3, KV8 = MODE == 2 || MODE == 3;
  static_assert(!(CHUNKED && QK8 && !KV8), "8-bit scores over bf16 pages are not implemented");
  static_assert(!KV8 || CHUNKED, "the 8-bit cache is implemented for the chunked prefill");
  constexpr int NW = TQ / 32;             // waves per workgroup
  constexpr int ROWB = (KV8 ? 1 : 2) * D; // bytes per key row of a V tile in LDS
  constexpr int ESK = QK8 || KV8 ? 1 : 2; // bytes per K element
  constexpr int ESQ = QK8 ? 1 : 2;        // bytes per Q element
  constexpr int ROWK = ESK * D;           // bytes per key row of a K tile in LDS
  constexpr int KSTEPS = QK8 ? D / 64 : D / 16;  // k-steps of the QK^T MFMA
  constexpr int CB = D / 32;              // 32-channel blocks of the output
  constexpr int IPW = kTK * ROWB / 1024 / NW;   // 1 KB direct-to-LDS loads per wave and V tile
  constexpr int IPWK = kTK * ROWK / 1024 / NW;  // the same per K tile
  static_assert(IPW >= 1 && kTK * ROWB % (1024 * NW) == 0, "tile split");
  static_assert(IPWK >= 1 && kTK * ROWK % (1024 * NW) == 0, "tile split");
  constexpr int AHEAD = 2;                // MFMAs an LDS operand read runs ahead of its use
  auto swzk = [](int r) { return QK8 || KV8 ? swz_k8<D>(r) : swz_k<D>(r); };
  auto swzv = [](int r) { return KV8 ? swz_v8<D>(r) : swz_v<D>(r); };

  // separate arrays per buffer: the wait-count pass then sees that a load into one buffer does not
  // alias reads of the other
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds0[kTK * ROWK / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds1[kTK * ROWK / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds0[kTK * ROWB / 2];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds1[kTK * ROWB / 2];
  __shared__ uint32_t votes[2];  // per tile parity: byte w is wave w's keep vote (0 or 1)
  static_assert(NW <= 4, "one vote byte per wave");
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
  // read as zero (also for the direct-to-LDS loads)
  // bytes spanned by rows [0, n) of a Q/K slice with row stride ss elements
  auto qk_rows_bytes = [&](int n, int64_t ss, int es) {
    return n <= 0 ? 0u : (uint32_t)(((int64_t)(n - 1) * ss + D) * es);
  };
  const uint8_t* q8 = reinterpret_cast<const uint8_t*>(a.q);
  const uint8_t* k8 = reinterpret_cast<const uint8_t*>(a.k);
  const rsrc_t rq = CHUNKED ? make_rsrc(q8 + ((int64_t)qrow0 * a.q_ss + (int64_t)h * a.q_sh) * ESQ, qk_rows_bytes(S, a.q_ss, ESQ))
                            : make_rsrc(q8 + ((int64_t)b * a.q_sb + (int64_t)h * a.q_sh) * ESQ, qk_rows_bytes(S, a.q_ss, ESQ));
  const rsrc_t rk = make_rsrc(k8 + ((int64_t)b * a.k_sb + (int64_t)g * a.k_sh) * ESK,
                              CHUNKED ? 0u : qk_rows_bytes(S, a.k_ss, ESK));
  const rsrc_t rv = make_rsrc(a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh, CHUNKED ? 0u : rows_bytes(S, a.v_ss, D));
  // chunked: the resource of key tile t of this KV head (rows past Sk and bad page ids read as zero)
  auto page_rsrc = [&](const uint16_t* pool, const int32_t* pages, int64_t pool_pages, int64_t sb, int64_t sh,
                       int64_t ss, int t) {
    const int pg = __builtin_amdgcn_readfirstlane(load_uniform_i32(pages, (int64_t)b * a.max_pages + t));
    if (pg < 0 || pg >= pool_pages) return make_rsrc(pool, 0u);
    if constexpr (KV8) {  // pools of e4m3 codes: strides count bytes
      const int n = min(kTK, Sk - t * kTK);
      return make_rsrc(reinterpret_cast<const uint8_t*>(pool) + (int64_t)pg * sb + (int64_t)g * sh,
                       n <= 0 ? 0u : (uint32_t)((int64_t)(n - 1) * ss + D));
    } else {
      return make_rsrc(pool + (int64_t)pg * sb + (int64_t)g * sh, rows_bytes(min(kTK, Sk - t * kTK), ss, D));
    }
  };

  // ---- Q operand: lane (col, half) holds Q[row][ks*16 + half*8 .. +8] for every k-step (QK8: the 32
  // codes Q[row][ks*64 + half*32 .. +32])
  const int iq = q0 + w * 32 + col;
  const bool row_ok = iq < S;
  bf16x8 qreg[QK8 ? 1 : KSTEPS];
  i32x8 qreg8[QK8 ? KSTEPS : 1];
  {
    const uint32_t qoff = row_ok ? (uint32_t)iq * (uint32_t)(a.q_ss * ESQ) + half * (QK8 ? 32 : 16) : 0xffffffffu;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if constexpr (QK8) {
        const u32x4 lo = buffer_load_16(rq, row_ok ? qoff + ks * 64 : qoff);
        const u32x4 hi = buffer_load_16(rq, row_ok ? qoff + ks * 64 + 16 : qoff);
        qreg8[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      } else {
        qreg[ks] = as_bf16x8(buffer_load_16(rq, row_ok ? qoff + ks * 32 : qoff));
      }
    }
  }

  // ---- tile loads, straight into LDS: load i of wave w fills LDS bytes [(w*IPW + i) KB, +1 KB) of the
  // tile, lane l the 16 bytes at l*16 of it, i.e. chunk position p of row r; it fetches the logical chunk
  // p ^ swz(r) of that key row.
  constexpr int RPL = 1024 / ROWB;   // key rows per load (V)
  constexpr int RPLK = 1024 / ROWK;  // the same for K
  const int lrow = lane / (ROWB / 16), lpos = lane % (ROWB / 16);
  const int lrowk = lane / (ROWK / 16), lposk = lane % (ROWK / 16);
  const uint32_t k_row_bytes = (uint32_t)(a.k_ss * ESK), v_row_bytes = (uint32_t)(a.v_ss * (KV8 ? 1 : 2));
  const uint32_t k_tile_bytes = kTK * k_row_bytes, v_tile_bytes = kTK * v_row_bytes;
  // Row (w*IPW + i)*RPL + lrow: every swizzle splits into a per-lane part and a part of the load index
  // (their bit fields do not overlap), so the chunk offset is (lane part) ^ (uniform part).
  uint32_t k_dma = (uint32_t)(w * IPWK * RPLK + lrowk) * k_row_bytes;   // row part of this lane's K loads
  uint32_t k_dmx = (uint32_t)(lposk ^ swzk(lrowk)) * 16;                // chunk part
  // bf16: row part + chunk part in one offset (the V swizzle has no load-index part); KV8: kept apart
  uint32_t v_dma = (uint32_t)(w * IPW * RPL + lrow) * v_row_bytes + (KV8 ? 0u : (uint32_t)(lpos ^ swzv(lrow)) * 16);
  uint32_t v_dmx = KV8 ? (uint32_t)(lpos ^ swzv(lrow)) * 16 : 0u;
  auto load_k_rsrc = [&](uint16_t* dst, rsrc_t r, uint32_t toff) {
#pragma unroll
    for (int i = 0; i < IPWK; ++i) {
      const uint32_t cx = (uint32_t)swzk((w * IPWK + i) * RPLK) * 16;  // wave-uniform
      const uint32_t vo = k_dma + (k_dmx ^ cx) + (uint32_t)(i * RPLK) * k_row_bytes + toff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + (w * IPWK + i) * 512), 16, vo, 0, 0, 0);
    }
  };
  auto load_v_rsrc = [&](uint16_t* dst, rsrc_t r, uint32_t toff) {
    static_assert(D == 128 || D == 64, "the bf16 V swizzle has no load-index part for these widths");
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      // 8-bit V tiles at D = 128: the swizzle's bit 1 comes from the load index (wave-uniform)
      const uint32_t cx = KV8 ? (uint32_t)swzv((w * IPW + i) * RPL) * 16 : 0u;
      const uint32_t vo = v_dma + (KV8 ? (v_dmx ^ cx) : 0u) + (uint32_t)(i * RPL) * v_row_bytes + toff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + (w * IPW + i) * 512), 16, vo, 0, 0, 0);
    }
  };
  auto load_k = [&](uint16_t* dst, int t) {
    if constexpr (CHUNKED) load_k_rsrc(dst, page_rsrc(a.k, a.k_pages, a.k_pool_pages, a.k_sb, a.k_sh, a.k_ss, t), 0u);
    else load_k_rsrc(dst, rk, (uint32_t)t * k_tile_bytes);
  };
  auto load_v = [&](uint16_t* dst, int t) {
    if constexpr (CHUNKED) load_v_rsrc(dst, page_rsrc(a.v, a.v_pages, a.v_pool_pages, a.v_sb, a.v_sh, a.v_ss, t), 0u);
    else load_v_rsrc(dst, rv, (uint32_t)t * v_tile_bytes);
  };

  // ---- operand reads.  Byte offsets inside a tile buffer: per lane one base, per operand an XOR with a
  // constant on bits that neither the base's row part nor the added constants touch.
  // K (S^T's A operand): lane (col, half) reads row kb*32 + col, logical chunk 2*ks + half, i.e. byte
  // (kb*32 + col)*ROWB + 16*((2ks + half) ^ swz_k(col)) = (k_opb ^ 32*ks) + kb*32*ROWB.
  // QK8: lane (col, half) reads row kb*32 + col, logical chunks 4ks + 2half and 4ks + 2half + 1 (32 codes),
  // i.e. bytes (kb*32 + col)*D + 16*((4ks + 2half + j) ^ swz_k8(col)) = (k_opb ^ 16*(4ks + j)) + kb*32*D.
  // KV8: lane (col, half) reads 8 codes of row kb*32 + col, channels ks*16 + half*8 .. +8, i.e. byte
  // (kb*32 + col)*D + 16*(ks ^ swz_k8(col)) + 8*half = (k_opb ^ 16*ks) + kb*32*D.
  const int xk = swzk(col);
  uint32_t k_opb = QK8 ? (uint32_t)(col * ROWK + 16 * ((2 * half) ^ xk))
                 : KV8 ? (uint32_t)(col * ROWK + 16 * xk + 8 * half)
                       : (uint32_t)(col * ROWB + 32 * (xk >> 1) + 16 * (half ^ (xk & 1)));
  // V^T (O^T's A operand) by transposing reads: in each 16-lane group, lane 4j + m names 4 channels
  // (4m .. 4m+3 of the group's 16) of key row k0 + j and receives channel (lane & 15) of the 4 rows.
  // Group gq covers channels 16*(gq & 1) of each 32-channel block and the keys of half gq >> 1.  The
  // logical chunk of channel block cb is 4cb + vch/8, and swz_v(k0 + vrow) = swz_v(vrow) is a multiple of
  // 4, so the byte is (v_opb ^ 64*cb) + k0*ROWB.
  const int gq = lane >> 4, li = lane & 15;
  const int vrow = li >> 2;                       // row inside the 4-row gather
  const int vch = 16 * (gq & 1) + 4 * (li & 3);   // channel inside the 32-channel block
  // KV8: an 8-bit transposing read gathers 8 rows per 16-lane group; lane 2j + m names row vkey(j) (the S^T
  // accumulator's key order: 4hf + j, then 8 + 4hf + j - 4) and codes 8m..8m+7 of the group's 16 channels
  // (logical chunk 2cb + (gq & 1)); byte (v_opb ^ 32*cb) + 16*st*D.
  const int vj = li >> 1, vkey = (vj < 4 ? 0 : 4) + 4 * (gq >> 1) + vj;
  uint32_t v_opb = KV8 ? (uint32_t)(vkey * ROWB + 16 * ((gq & 1) ^ swz_v8<D>(vkey)) + 8 * (li & 1))
                       : (uint32_t)(vrow * ROWB + 64 * (swz_v<D>(vrow) >> 2) + 16 * (vch >> 3) + 2 * (vch & 7));
  auto kop = [&](const uint16_t* kl, int ks, int kb) {
    if constexpr (KV8) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(reinterpret_cast<const char*>(kl) + ((k_opb ^ (16u * ks)) + kb * 32 * ROWK));
      return fp8x8_to_bf16x8(x);
    } else {
      return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(kl) + ((k_opb ^ (32u * ks)) + kb * 32 * ROWB));
    }
  };
  auto kop8 = [&](const uint16_t* kl, int ks, int kb) {
    const char* base = reinterpret_cast<const char*>(kl) + kb * 32 * ROWK;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + (k_opb ^ (64u * ks)));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + (k_opb ^ (64u * ks + 16u)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto vop = [&](const uint16_t* vl, int cb, int st) {
    if constexpr (KV8) {
      typedef int v2i __attribute__((ext_vector_type(2)));
      const char* base = reinterpret_cast<const char*>(vl) + (v_opb ^ (32u * cb)) + 16 * st * ROWB;
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)base);
      return as_bf16x8(fp8x8_to_bf16x8(u32x2{(uint32_t)x[0], (uint32_t)x[1]}));
    } else {
      // the S^T accumulator layout that P^T comes from: half hf holds keys 4hf..4hf+3 and 8+4hf..8+4hf+3
      // of each 16-key step
      const char* base = reinterpret_cast<const char*>(vl) + (v_opb ^ (64u * cb)) + (16 * st + 4 * (gq >> 1)) * ROWB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)base);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(base + 8 * ROWB));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  // opaque copies of the per-lane bases, taken once per tile, so that the addresses derived from them are
  // formed next to their use instead of being kept in registers across the loop
  auto refresh = [&]() {
    asm volatile("" : "+v"(k_opb), "+v"(v_opb), "+v"(k_dma), "+v"(k_dmx), "+v"(v_dma));
    if constexpr (KV8) asm volatile("" : "+v"(v_dmx));
  };

  // ---- running state of this lane's query row
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  float m_true = neg_inf();  // running max of raw scores over kept tiles (the skip rule's m_{i-1})
  float m_ref = neg_inf();   // reference max of the exponentials (trails m_true by at most 8/c2)
  float moff = 0.f;          // m_ref * c2 (0 while m_ref = -inf)
  // this lane's half of the softmax denominator, in two chains (weight pairs alternate between them) so that
  // consecutive row-sum updates do not wait for each other; added in the epilogue
  float l_part[2] = {0.f, 0.f};
  int n_exec = 0;

  // S^T for keys t*64 .. t*64+63 (two 32-key blocks) x this wave's 32 query columns from the K tile at
  // `kl`; MFMA j is (k-step j/2, key block j%2): the two chains alternate and each operand is read
  // AHEAD MFMAs before its use.
  // Both MFMA streams (QK^T and P.V) raise the wave's issue priority: of the two waves sharing a SIMD,
  // the one with MFMAs to issue goes first and the other's VALU work fills the MFMA shadow.
  auto qk = [&](const uint16_t* kl, f32x16 (&s)[2]) {
    constexpr int NM = 2 * KSTEPS;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (QK8) {
      i32x8 x[NM];
#pragma unroll
      for (int j = 0; j < NM; ++j) x[j] = kop8(kl, j >> 1, j & 1);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        const int ks = j >> 1, kb = j & 1;
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x[j], qreg8[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0, 0,
                                                                0, 0);
      }
    } else {
      u32x4 x[NM];
#pragma unroll
      for (int j = 0; j < AHEAD; ++j) x[j] = kop(kl, j >> 1, j & 1);
#pragma unroll
      for (int j = 0; j < NM; ++j) {
        if (j + AHEAD < NM) x[j + AHEAD] = kop(kl, (j + AHEAD) >> 1, (j + AHEAD) & 1);
        __builtin_amdgcn_sched_barrier(0);
        const int ks = j >> 1, kb = j & 1;
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(x[j]), qreg[ks], ks == 0 ? f32x16{} : s[kb], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // exponential pair n/2 (n even, P^T operand order) of the scores s
  auto exp_pair = [&](const f32x16 (&s)[2], uint32_t (&pk)[4][4], int n, float eo) {
    const int st = n >> 3, e = n & 7;  // 16-key step, position inside it
    const float s0 = s[st >> 1][8 * (st & 1) + e], s1 = s[st >> 1][8 * (st & 1) + e + 1];
    if constexpr (POT) {
      pk[st][e >> 1] = pot_pack_sum_bf16x2(s0, s1, c2, eo, l_part[(n >> 1) & 1]);
    } else {
      const float p0 = exp2_fast(fmaf(s0, c2, -eo)), p1 = exp2_fast(fmaf(s1, c2, -eo));
      pk[st][e >> 1] = pack_bf16x2(p0, p1);
      l_part[(n >> 1) & 1] += p0 + p1;
    }
  };
  // keep the exponentials where they are issued (next to the MFMAs they overlap) instead of letting
  // them sink towards their use one iteration later
  auto pin = [&](uint32_t (&pk)[4][4]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) asm volatile("" ::"v"(pk[st][0]), "v"(pk[st][1]), "v"(pk[st][2]), "v"(pk[st][3]));
    asm volatile("" : "+v"(l_part[0]), "+v"(l_part[1]));
  };
  // O^T += V^T . P^T from the V tile at `vl`; MFMA j is (16-key step j/CB, channel block j%CB).  The
  // exponentials of the current tile's scores `s` against offset `eo` (into `pk_out`) are spread over
  // the MFMAs.  One instance per tile serves kept and skipped current tiles (a skipped one uses
  // eo = +inf: every exponential is exactly 0 and the row sums do not change), so the accumulators keep
  // a single register home.
  auto pv = [&](const uint16_t* vl, const uint32_t (&pk)[4][4], float alpha, bool rescale, const f32x16 (&s)[2],
                float eo, uint32_t (&pk_out)[4][4]) {
    constexpr int NM = 4 * CB;
    constexpr int PPM = 16 / NM;  // exponential pairs per MFMA
    if (rescale) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) acc[cb] *= alpha;
    }
    __builtin_amdgcn_s_setprio(1);
    bf16x8 vx[NM];
#pragma unroll
    for (int j = 0; j < AHEAD; ++j) vx[j] = vop(vl, j % CB, j / CB);
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      if (j + AHEAD < NM) vx[j + AHEAD] = vop(vl, (j + AHEAD) % CB, (j + AHEAD) / CB);
      __builtin_amdgcn_sched_barrier(0);
      const int st = j / CB, cb = j % CB;
      const bf16x8 pb = as_bf16x8(u32x4{pk[st][0], pk[st][1], pk[st][2], pk[st][3]});
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vx[j], pb, acc[cb], 0, 0, 0);
#pragma unroll
      for (int q = 0; q < PPM; ++q) exp_pair(s, pk_out, 2 * (j * PPM + q), eo);
    }
    pin(pk_out);
    __builtin_amdgcn_s_setprio(0);
  };
  // key offset o inside tile t is valid for this row iff o <= lim
  auto mask = [&](f32x16 (&s)[2], int t) {
    const int key_base = t * kTK;
    // offset o = kb*32 + 8*(i/4) + 4*half + i%4; the lane's part 4*half moves into the limit so that
    // each comparison is against a constant
    const int lim = (!row_ok ? -1 : (a.causal ? iq + off - key_base : Sk - 1 - key_base)) - 4 * half;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = kb * 32 + 8 * (i >> 2) + (i & 3) <= lim ? s[kb][i] : neg_inf();
  };
  auto row_max = [&](const f32x16 (&s)[2]) {
    float mx = neg_inf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmax3(mx, s[kb][i], s[kb][i + 1]);
    return pair_max_nonan(mx);
  };

  // ---- one iteration per key tile t (parity P = t & 1, known at compile time):
  //  (1) S(t) = K(t) Q^T; row max; the skip vote against the running max of the kept tiles so far
  //      (tau <= 0: the prefix max); wait for this wave's loads of the previous iteration; barrier;
  //  (2) the unit's decision; statistics; online-softmax update (the output factor is applied before
  //      the next P.V, after the previous one);
  //  (3) loads of K(t+2) into K(t)'s buffer and, if the tile is kept, of V(t) into V(t-2)'s;
  //  (4) the exponentials of tile t (if kept) spread over the P.V MFMAs of tile t-1 (if kept).
  // The barrier of iteration t makes the loads issued in iteration t-1 (K(t+1), V(t-1)) visible and
  // ends every read of the buffers that iteration t's loads replace (K(t) in step 1 of this iteration,
  // V(t-2) in step 4 of the previous one).
  uint32_t pka[4][4], pkb[4][4];
  bool keep_prev = false;  // tile t-1 was kept: its P.V is pending
  float alpha_prev = 1.f;  // output factor to apply before that P.V
  bool resc_prev = false;
  auto iteration = [&](int t, uint32_t (&pk_cur)[4][4], uint32_t (&pk_prev)[4][4], auto parity) {
    constexpr int P = decltype(parity)::value ? 1 : 0;
    uint16_t* k_cur = P ? k_lds1 : k_lds0;
    uint16_t* v_cur = P ? v_lds1 : v_lds0;
    const uint16_t* v_prev = P ? v_lds0 : v_lds1;
    f32x16 s[2];
    bool keep = false;
    float alpha = 1.f;
    bool resc = false;
    if (t < T) {
      refresh();
      qk(k_cur, s);
      if (t >= T_in) mask(s, t);
      const float mx = row_max(s);
      const int vb = t & 1;
      {
        const bool abstain = mx == neg_inf();
        const float gap = mx - m_true;  // +inf while the row has seen no valid key
        // the lane masks of !abstain and !(gap < tau) ANDed in scalar registers; the wave's vote is byte w of
        // the tile parity's word
        const uint64_t ball = __builtin_amdgcn_fcmpf(mx, neg_inf(), 6 /* ordered, not equal */) &
                              __builtin_amdgcn_fcmpf(gap, a.tau_raw, 11 /* unordered or >= */);
        // (every lane stores the same byte to the same address: no divergent branch around the store)
        reinterpret_cast<volatile uint8_t*>(&votes[vb])[w] = ball != 0 ? 1 : 0;
        if (a.unit_gap) {
          float gg = abstain ? neg_inf() : gap;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) gg = fmaxf(gg, __shfl_xor(gg, o, 64));
          if (lane == 0) wave_gap[vb][w] = gg;
        }
      }
      wait_vmem_all();
      __syncthreads();
      keep = __builtin_amdgcn_readfirstlane(votes[vb]) != 0;
      if (tid == 0) {
        if (a.tile_state) a.tile_state[unit * a.nkt + t] = keep ? 1 : 2;
        if (a.unit_gap) {
          float gg = wave_gap[vb][0];
#pragma unroll
          for (int i = 1; i < NW; ++i) gg = fmaxf(gg, wave_gap[vb][i]);
          a.unit_gap[unit * a.nkt + t] = gg == __builtin_inff() ? gg : gg * a.scale;
        }
      }
      if (t + 2 < T) load_k(k_cur, t + 2);
      if (keep) {
        load_v(v_cur, t);
        ++n_exec;
        // advance the true max; move the reference max only when it trails by > 8
        m_true = max_nonan(m_true, mx);
        // the rescale and the weights' offset change only when some row's reference moves (rare)
        float kn = 0.f;
        bool move;
        if constexpr (POT) {
          // m_ref: the integer reference in base-2 log-weight units
          kn = rintf(m_true * c2);           // -inf while the row has no valid key
          move = kn - m_ref > kRefSlack;      // also true while m_ref = -inf and kn finite
        } else {
          move = (m_true - m_ref) * c2 > kRefSlack;  // also true while m_ref = -inf and m_true finite
        }
        resc = wave_ballot(move) != 0;
        if (resc) {
          if constexpr (POT) {
            alpha = move ? (m_ref == neg_inf() ? 0.f : ldexpf(1.f, (int)(m_ref - kn))) : 1.f;  // exact
            m_ref = move ? kn : m_ref;
            moff = m_ref == neg_inf() ? 0.f : m_ref;
          } else {
            alpha = move ? exp2_fast((m_ref - m_true) * c2) : 1.f;  // 0 when m_ref = -inf
            m_ref = move ? m_true : m_ref;
            moff = (m_ref == neg_inf() ? 0.f : m_ref) * c2;
          }
          l_part[0] *= alpha;
          l_part[1] *= alpha;
        }
      }
    } else {
      // past the last tile: only the pending P.V; its V tile was loaded in the previous iteration
      wait_vmem_all();
      __syncthreads();
      s[0] = f32x16{};
      s[1] = f32x16{};
    }
    // exponentials of a skipped tile use offset +inf: exactly 0, so they add nothing to the row sums and
    // give the zero P^T that the next tile's P.V must not accumulate
    // the P.V of the previous tile (if kept) with this tile's exponentials between its MFMAs, else this
    // tile's exponentials alone
    if (keep_prev) {
      pv(v_prev, pk_prev, alpha_prev, resc_prev, s, keep ? moff : __builtin_inff(), pk_cur);
    } else if (keep) {
#pragma unroll
      for (int n = 0; n < 32; n += 2) exp_pair(s, pk_cur, n, moff);
      pin(pk_cur);
    }
    keep_prev = keep;
    alpha_prev = alpha;
    resc_prev = resc;
  };

  if (T > 0) {
    // vote bytes of waves that do not exist (fewer than four waves) stay zero
    if (tid == 0) votes[0] = votes[1] = 0u;
    load_k(k_lds0, 0);
    if (T > 1) load_k(k_lds1, 1);
    wait_vmem_all();  // Q and the first key tiles
    __syncthreads();
    // iterations t = 0 .. T; iteration T only completes the P.V of tile T-1
    for (int t = 0; t <= T; t += 2) {
      iteration(t, pka, pkb, false_type{});
      if (t + 1 <= T) iteration(t + 1, pkb, pka, true_type{});
    }
  }

  // ---- epilogue: O = acc / l, bf16
  const float l_tot = pair_sum(l_part[0] + l_part[1]);
  // KV8: the values are v_scale * code
  const float inv = l_tot > 0.f ? (KV8 ? a.v_scale : 1.f) / l_tot : 0.f;
  if (row_ok) {
    uint16_t* op = a.o + (CHUNKED ? (int64_t)(qrow0 + iq) * a.o_ss : (int64_t)b * a.o_sb + (int64_t)iq * a.o_ss) +
                   (int64_t)h * a.o_sh;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int gq4 = 0; gq4 < 4; ++gq4) {
        const int ch = cb * 32 + 8 * gq4 + 4 * half;
        const u32x2 x = {pack_bf16x2(acc[cb][4 * gq4] * inv, acc[cb][4 * gq4 + 1] * inv),
                         pack_bf16x2(acc[cb][4 * gq4 + 2] * inv, acc[cb][4 * gq4 + 3] * inv)};
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

hipError_t launch_prefill(const PrefillArgs& a, int d, int tile_q, bool chunked, int mode, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)a.B * a.Hq * a.nqt);
  if (grid == 0) return hipSuccess;
  if (chunked ? mode == 1 : (mode == 2 || mode == 3)) return hipErrorInvalidValue;
  if (chunked && a.pot) return hipErrorInvalidValue;
  if (!chunked && (mode == 0 || mode == 1) && d == 128 && tile_q == 128 && a.G % 2 == 0)
    return launch_prefill_pp(a, mode == 1, stream);
  const dim3 blk(tile_q * 2);
#define SSM_PREFILL_LAUNCH(D, TQ)                                                                                   \
  if (d == D && tile_q == TQ) {                                                                                     \
    if (chunked && mode == 2) hipLaunchKernelGGL((prefill_kernel<D, TQ, true, 2, false>), dim3(grid), blk, 0, stream, a); \
    else if (chunked && mode == 3) hipLaunchKernelGGL((prefill_kernel<D, TQ, true, 3, false>), dim3(grid), blk, 0, stream, a); \
    else if (chunked) hipLaunchKernelGGL((prefill_kernel<D, TQ, true, 0, false>), dim3(grid), blk, 0, stream, a);  \
    else if (mode == 1 && a.pot) hipLaunchKernelGGL((prefill_kernel<D, TQ, false, 1, true>), dim3(grid), blk, 0, stream, a); \
    else if (mode == 1) hipLaunchKernelGGL((prefill_kernel<D, TQ, false, 1, false>), dim3(grid), blk, 0, stream, a); \
    else if (a.pot) hipLaunchKernelGGL((prefill_kernel<D, TQ, false, 0, true>), dim3(grid), blk, 0, stream, a);    \
    else hipLaunchKernelGGL((prefill_kernel<D, TQ, false, 0, false>), dim3(grid), blk, 0, stream, a);              \
    return hipGetLastError();                                                                                       \
  }
  SSM_PREFILL_LAUNCH(128, 128)
  SSM_PREFILL_LAUNCH(128, 64)
  SSM_PREFILL_LAUNCH(64, 128)
  SSM_PREFILL_LAUNCH(64, 64)
#undef SSM_PREFILL_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssm
