// ssm_launch.h -- kernel argument blocks and launchers (internal to libssm.so).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

struct PrefillArgs {
  const uint16_t* q;         // bf16, or e4m3 codes (prefill_kernel<..., QK8 = true>; strides then count bytes)
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int64_t q_sb, q_ss, q_sh;  // element strides of batch, position, head (last dim contiguous)
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int32_t B, S, Hq, Hkv, G;
  int32_t nqt, nkt;          // query tiles, key tiles
  int32_t causal;
  float scale;               // softmax scale (natural-log logits = scale * q.k)
  float scale_log2;          // scale * log2(e)
  float tau_raw;             // tau / scale: threshold on raw q.k gaps; -inf never skips
  float v_scale;             // e4m3 V pages (mode 2): value = v_scale * code
  int32_t pot;               // 1: Rowmax-PoT weights (non-chunked prefill only), 0: exponentials
  uint8_t* tile_state;       // nullable [units, nkt]
  float* unit_gap;           // nullable [units, nkt]
  unsigned long long* counters;  // nullable [4]
  // chunked prefill against a paged cache (prefill_kernel<..., true>): S is the longest query count;
  // sequence b's queries are q rows q_start[b] .. q_start[b+1]-1 (o likewise; q_sb/o_sb unused), the last
  // of its kv_lens[b] cached keys; key tile t of (b, KV head g) is page k_pages[b*max_pages + t]
  const int32_t* q_start;
  const int32_t* kv_lens;
  const int32_t* k_pages;
  const int32_t* v_pages;
  int32_t max_pages;         // row length of the page tables (= nkt)
  int32_t total_q;           // rows of q/o
  int64_t k_pool_pages, v_pool_pages;
};

struct DecodeArgs {
  const uint16_t* q;         // [B, Hq, d]
  const void* k;             // pool of bf16 or fp8 e4m3 elements (kv_fp8)
  const void* v;
  const int32_t* kv_lens;    // [B]
  const int32_t* k_pages;    // nullable: paged
  const int32_t* v_pages;
  int64_t q_sb, q_sh;
  // contiguous: element offset of key j of (b, g) = b*sb + g*sh + j*ss
  // paged:      element offset = page*sb + g*sh + (j % 64)*ss, page = table[b*max_pages + j/64]
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int32_t k_max_pages, v_max_pages;
  int32_t B, Hq, Hkv, G;
  int32_t max_tiles;         // row length of tile_state / unit_gap
  int32_t num_splits;
  int32_t sink_seed;         // 1: splits after the first start their running max at tile 0's row maxima
  int32_t kv_fp8;            // 1: K/V pools hold fp8 e4m3 codes; scale includes the key scale
  float v_scale;             // value dequantisation scale (1 for bf16)
  float scale, scale_log2, tau_raw;  // scale: logit scale per raw q.k product (softmax scale x key scale)
  float* part_o;             // workspace [B, Hq, P, d] fp32
  float* part_lse;           // workspace [B, Hq, P] fp32 (base-2 log-sum-exp of raw-scaled logits)
  int32_t* order;            // workspace [B]: dispatch order, longest sequence first (NULL: plain order)
  uint32_t* wg_cnt;          // workspace [B, Hkv, P, 2]: (visited, executed) tiles of each split workgroup
  uint16_t* o;               // [B, Hq, d]
  int64_t o_sb, o_sh;
  uint8_t* tile_state;
  float* unit_gap;
  unsigned long long* counters;
};

// mode 0: bf16; 1: e4m3 q/k scores (contiguous only); 2: e4m3 K/V pages (chunked only); 3: e4m3 queries
// scored against e4m3 K pages, e4m3 V pages (chunked only)
hipError_t launch_prefill(const PrefillArgs& a, int d, int tile_q, bool chunked, int mode, hipStream_t stream);
// d = 128, tile_q = 128, contiguous, an even number of query heads per KV head, bf16 or (qk8) e4m3 Q and K: two
// units per workgroup in ping-pong (prefill_pp.hip)
hipError_t launch_prefill_pp(const PrefillArgs& a, bool qk8, hipStream_t stream);
constexpr int kDecSortMax = 8192;  // batches up to this size are dispatched longest sequence first
// size of the static device array that serves as ssm_decode_noalloc's workspace (one per GPU)
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;

// the current device's address of that array (the first call on a device looks it up); hipErrorInvalidDevice when
// `stream` belongs to another device
hipError_t decode_scratch(hipStream_t stream, void** ptr);

hipError_t launch_decode_impl(const DecodeArgs& a, int d, int kv_cap, int64_t k_pool_rows, int64_t v_pool_rows,
                              hipStream_t stream);

}  // namespace ssm
