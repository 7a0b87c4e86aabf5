/*
 * ssm.h -- C ABI of libssm.so: Skip Softmax attention forward on AMD MI355X (gfx950).
 *
 * Skip Softmax is a FlashAttention-style forward pass with an online (running
 * maximum) softmax over streamed key tiles.  For each key tile the local score
 * maximum is compared with the running maximum of the earlier tiles; when it
 * trails by more than a threshold tau, for every row of the unit, the tile's
 * exponentials and its P*V product are skipped.  Sources: the recap of
 * "Accelerating Long-Context Inference with Skip Softmax in NVIDIA
 * TensorRT-LLM" (Key Points; Detailed Analysis; Skip Softmax Mechanism;
 * Impact on Accuracy vs. Speed) and the NVIDIA Skip Softmax news item
 * (Understanding Skip Softmax; Benefits and Implementation).
 *
 * Conventions shared by every entry point
 *  - Pointers inside descriptors are DEVICE pointers unless noted; descriptor
 *    structs themselves live in host memory and are read during the call only.
 *  - The caller owns every buffer.  The library never allocates device memory
 *    and keeps no state between calls.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  No call synchronises or reads device memory on the
 *    host.  Outputs and statistics are valid once the stream has passed them.
 *  - A call enqueues kernel launches only (no memset or copy nodes), so it can
 *    be captured into a HIP graph and replayed; each replay reads the buffers'
 *    contents at that time (kv_lens and page tables included).
 *  - Return codes: SSM_OK, or an error code; on any error nothing is launched
 *    and ssm_last_error() (thread-local) holds a message.
 *  - Units of tau: natural-log ratio of softmax weights (tau = -ln 1000 skips a
 *    tile whose best weight is below 1/1000 of the running best).  tau = -inf
 *    disables skipping (dense attention).  tau must be -inf or in (-inf, 0];
 *    tau > 0 or NaN is SSM_EINVAL (a skipped tile could then hold a new maximum).
 */
#ifndef SSM_H
#define SSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSM_ABI_VERSION 10

enum {
  SSM_OK = 0,
  SSM_EINVAL = 1,        /* NULL pointer, shape/stride/dtype mismatch, bad tau, Hq % Hkv != 0, ... */
  SSM_EUNSUPPORTED = 2,  /* valid request outside what the kernels implement (head_dim, tiles, alignment) */
  SSM_EWORKSPACE = 3,    /* decode workspace missing or too small */
  SSM_EHIP = 4           /* a HIP runtime call or kernel launch failed */
};

enum { SSM_BF16 = 0, SSM_FP32 = 1, SSM_FP8_E4M3 = 2 /* OCP 8-bit float, 4 exponent / 3 mantissa bits */ };

/* Strided tensor view.  stride[] is in elements; the last dimension must be
 * contiguous (stride 1).  data must be 16-byte aligned and every other stride
 * a multiple of 16 bytes (8 bf16 or 16 fp8 elements), so rows can be moved in
 * 16-byte pieces.  An empty view (some extent 0) may have data == NULL.
 * A call with nothing to compute (prefill B, S or Hq 0; decode B or Hq 0;
 * chunked prefill batch 0 or max_q_len 0) checks its descriptors and returns
 * SSM_OK without launching; an empty decode needs no workspace, and an empty
 * batch needs no kv_lens, q_start or page tables. */
typedef struct {
  void* data;
  int32_t dtype;    /* SSM_BF16, SSM_FP32 or SSM_FP8_E4M3 (where an entry point accepts it) */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} ssm_tensor;

/* Decode KV cache.
 *   contiguous: page_table == NULL, pool = [B, Hkv, Smax, d]
 *   paged:      pool = [num_pages, Hkv, page_size, d]; page_table is a device
 *               int32 [B, max_pages] row-major array; logical key tile t of
 *               sequence b lives in page page_table[b*max_pages + t].  Only
 *               entries t < ceil(kv_len[b]/page_size) are read and they must be
 *               in [0, num_pages).  page_size must equal the key tile (64).
 *   pool.dtype: SSM_BF16, or SSM_FP8_E4M3 with `scale` the per-tensor
 *               dequantisation factor (element value = scale * code; finite, > 0;
 *               ignored for bf16).  K and V caches must share one dtype. */
typedef struct {
  ssm_tensor pool;
  const int32_t* page_table;
  int32_t page_size;
  int32_t max_pages;
  float scale;
} ssm_kv_cache;

/* Optional skip statistics (every member may be NULL / 0).
 *   tile_state: uint8 per (unit, key tile): 0 not visited, 1 executed, 2 skipped.
 *     prefill: unit = (b*Hq + h)*ceil(S/tile_q) + q_tile, row length ceil(S/tile_k)
 *     decode:  unit = b*Hkv + g, row length = max key tiles (Smax/64 or max_pages)
 *   unit_gap:   float per (unit, key tile), same indexing: the unit gap (max
 *     over the unit's rows of tile max minus running max, natural-log units);
 *     +inf on the first tile of a scan, NaN where not visited.
 *   counters:   uint64 [4] = visited tiles, skipped tiles, QK^T tiles issued,
 *     P*V tiles issued.  Accumulated with atomics: zero them before the call. */
typedef struct {
  uint8_t* tile_state;
  int64_t tile_state_len;       /* elements available at tile_state */
  float* unit_gap;
  int64_t unit_gap_len;         /* elements available at unit_gap */
  unsigned long long* counters;
} ssm_skip_stats;

/* Optional tuning / workspace (NULL selects every default). */
typedef struct {
  float scale;             /* softmax scale; 0 selects 1/sqrt(d) */
  int32_t tile_q;          /* prefill query tile: 0 -> 128; 64 or 128 */
  int32_t tile_k;          /* key tile: 0 -> 64; only 64 */
  int32_t num_splits;      /* decode split-K chunks: 0 -> 16; 1..64 */
  void* workspace;         /* decode: device buffer of >= ssm_decode_workspace_bytes() bytes */
  size_t workspace_bytes;
  int32_t decode_flags;    /* decode: 0 or SSM_DECODE_SINK_SEED; other bits are SSM_EINVAL */
  int32_t weights;         /* SSM_WEIGHTS_EXP (0) or SSM_WEIGHTS_ROWMAX_POT: ssm_prefill and ssm_prefill_fp8qk;
                              the other entry points return SSM_EUNSUPPORTED for anything but 0; other
                              values are SSM_EINVAL */
} ssm_opts;

/* Softmax weights of the prefill ("Approximating Softmax in Pretrained LLMs: Model Sensitivity and Kernel
 * Acceleration", AI Summary and Abstract: Rowmax-PoT replaces the exponential by powers of two, a coarse
 * logarithmic weight anchored at each row maximum).  With SSM_WEIGHTS_ROWMAX_POT a kept key's weight is
 * 2^(rint(log2(e) * l) - rint(log2(e) * mu)) for its logit l and the row maximum mu over the kept keys (ties
 * to even), so the weights are exact powers of two and no exponential is evaluated; the output is
 * sum_j w_j v_j / sum_j w_j over the kept keys.  Which tiles are skipped does not change.  The rounding is
 * decided on the fp32 logits, so a logit within a few fp32 ulps of a half-integer base-2 log weight may round
 * either way. */
#define SSM_WEIGHTS_EXP 0
#define SSM_WEIGHTS_ROWMAX_POT 1

/* Sink-seeded split-K decode.  By default every split-K chunk is an independent
 * scan whose running maximum starts at -inf, so the first tile of every chunk
 * is kept.  With this flag a chunk after the first starts its running maximum
 * at the unit's first-tile (tile 0) row maxima: the comparison the recap's Key
 * Points and Skip Softmax Mechanism make against the running maximum then
 * includes the score a single sequential scan would already have seen (tile 0
 * is always kept by the first chunk).  Costs one extra read of key tile 0 per
 * chunk; skips at least the tiles the default skips.  The output remains the
 * exact softmax over the kept keys. */
#define SSM_DECODE_SINK_SEED 1

/* Causal or full prefill (self-attention, S_q = S_k = seqlen): the context phase of the recap of
 * "Accelerating Long-Context Inference with Skip Softmax in NVIDIA TensorRT-LLM" (Detailed Analysis: a key
 * block whose local maximum trails the running maximum by more than tau is skipped whole; Skip Softmax
 * Mechanism) and of the news item (Benefits and Implementation: the prefill phase).
 *   q   [B, S, Hq, d]  bf16    k, v [B, S, Hkv, d] bf16    out [B, S, Hq, d] bf16
 *   d in {64, 128}; Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv).
 *   causal != 0: query i attends to keys j <= i (top-left aligned).
 * The unit of the skip decision is one query tile of one head (tile_q rows);
 * its key tiles are scanned in ascending order and the first is never skipped. */
int ssm_prefill(const ssm_tensor* q, const ssm_tensor* k, const ssm_tensor* v, int32_t seqlen, int32_t causal,
                float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream, const ssm_opts* opts);

/* ssm_prefill with 8-bit queries and keys: the scores QK^T, which every visited tile needs (a skipped tile
 * still needs them to decide), run on the FP8 matrix instructions at twice the bf16 rate, while V, the
 * softmax weights and P*V stay bf16.  Follows the FP8 attention context of the "Approximating Softmax in
 * Pretrained LLMs" page (Abstract) as applied to the Skip Softmax forward above.
 *   q [B, S, Hq, d] and k [B, S, Hkv, d]: SSM_FP8_E4M3 codes (OCP e4m3: bias 7, subnormals, no infinities,
 *     S.1111.111 is NaN) with per-tensor dequantisation factors: query = q_scale * code, key = k_scale * code
 *     (finite, > 0); strides multiples of 16 elements, data 16-byte aligned.
 *   v [B, S, Hkv, d] bf16, out [B, S, Hq, d] bf16; everything else as ssm_prefill (same units, statistics,
 *   options and errors).  The skip rule and the softmax apply to the logits scale * query . key. */
int ssm_prefill_fp8qk(const ssm_tensor* q, float q_scale, const ssm_tensor* k, float k_scale, const ssm_tensor* v,
                      int32_t seqlen, int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats,
                      void* stream, const ssm_opts* opts);

/* Single-token GQA decode with split-K and a log-sum-exp combine: the generation phase of the same rule (recap,
 * Key Points and Detailed Analysis; news item, Benefits and Implementation: in decode the saving is the memory
 * traffic of the skipped blocks, so a skipped tile's V rows are never read).
 *   q [B, Hq, d] bf16; out [B, Hq, d] bf16; K/V caches bf16 or fp8 e4m3 (see ssm_kv_cache: an fp8
 *   cache is read at half the bytes and each code is converted exactly to bf16 for the MFMAs); kv_lens device int32 [B], each in [0, Smax or
 *   max_pages*page_size]; query b attends to keys j < kv_lens[b].  kv_len 0 gives 0.
 * The unit of the skip decision is one KV group (its Hq/Hkv query heads vote
 * together).  The unit's n = ceil(kv_len/64) key tiles are cut into num_splits
 * chunks of ceil(n/num_splits) tiles; each chunk is an independent scan whose
 * running maximum starts at -inf, so the first tile of every chunk is kept
 * (see SSM_DECODE_SINK_SEED for the seeded variant).
 * Needs opts->workspace (see ssm_decode_workspace_bytes). */
int ssm_decode(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
               const int32_t* kv_lens, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
               const ssm_opts* opts);

/* ssm_decode without a caller workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same arguments, semantics, outputs and
 * errors as ssm_decode, except that opts->workspace and opts->workspace_bytes are ignored: the workspace is a
 * statically sized array in each GPU's memory (32 MiB, held by every GPU the library runs on until the process
 * ends), whose device address the first call on a device looks up.  The call allocates nothing.
 *   - Returns SSM_EWORKSPACE when ssm_decode_workspace_bytes(B, Hq, d, num_splits) exceeds 32 MiB (e.g. batch
 *     32, 64 query heads, d 128 needs 16.9 MB at 16 splits), and SSM_EINVAL when `stream` belongs to a device
 *     other than the current one; nothing is launched then.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents (nothing in it needs
 *     clearing: each call writes every byte it reads).  Calls that overlap in time on one GPU (different
 *     streams, or host threads) race on it: serialise them, e.g. on one stream. */
int ssm_decode_noalloc(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                       const int32_t* kv_lens, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                       const ssm_opts* opts);

/* Chunked prefill against a paged KV cache (a serving context phase: new tokens attend to the cached
 * context and to each other); the skip rule of ssm_prefill (recap, Detailed Analysis and Skip Softmax
 * Mechanism) applied to the context phase the news item's Benefits and Implementation names, over the
 * decode's paged cache.  A ragged batch of `batch` sequences:
 *   q, out [total_q, Hq, d] bf16: sequence b's n_b = q_start[b+1] - q_start[b] query rows are rows
 *     q_start[b] .. q_start[b+1]-1 (q_start: device int32 [batch+1], 0 <= n_b <= max_q_len);
 *   k_cache, v_cache: paged pools [pages, Hkv, 64, d] with page tables of equal length (see ssm_kv_cache),
 *     both bf16 or both SSM_FP8_E4M3 with their scales (the same cache the decode reads; each code is
 *     converted exactly to bf16 for the bf16 MFMAs); sequence b has kv_lens[b] (device int32 [batch]) keys,
 *     the last n_b of which are its
 *     new tokens (already written to the cache): query i of sequence b sits at key position
 *     kv_lens[b] - n_b + i and, with causal != 0, attends to keys j <= that position (bottom-right
 *     aligned); otherwise to all kv_lens[b] keys.
 * The unit of the skip decision is one query tile (tile_q rows) of one head of one sequence; its
 * statistics row is unit (b*Hq + h)*ceil(max_q_len/tile_q) + q_tile with max_pages key tiles.  A
 * sequence whose offsets are malformed (n_b < 0, n_b > max_q_len, rows past total_q) is not touched;
 * one with kv_lens[b] < n_b or more keys than its page table holds gets zero outputs.  With
 * kv_lens[b] = n_b this is ssm_prefill on one sequence. */
int ssm_prefill_paged(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                      const int32_t* q_start, const int32_t* kv_lens, int32_t batch, int32_t max_q_len,
                      int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                      const ssm_opts* opts);

/* ssm_prefill_paged with 8-bit queries over e4m3 pages (the serving path of an fp8 cache): q [total_q, Hq, d]
 * holds SSM_FP8_E4M3 codes with dequantisation factor q_scale (finite, > 0); the K and V pools must be
 * SSM_FP8_E4M3 (see ssm_kv_cache).  The scores run on the FP8 matrix instructions straight from the 8-bit key
 * pages (as ssm_prefill_fp8qk); V and P*V stay bf16.  Everything else as ssm_prefill_paged. */
int ssm_prefill_paged_fp8qk(const ssm_tensor* q, float q_scale, const ssm_kv_cache* k_cache,
                            const ssm_kv_cache* v_cache, const int32_t* q_start, const int32_t* kv_lens, int32_t batch,
                            int32_t max_q_len, int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats,
                            void* stream, const ssm_opts* opts);

/* Bytes of device workspace ssm_decode needs: fp32 partial outputs and log-sum-exps per (b, query head,
 * split), for batches up to 8192 the longest-first dispatch order of the sequences (int32 per sequence,
 * written by the call), and two uint32 skip counts per (b, head, split) (used when skip counters are asked
 * for).  0 for invalid arguments. */
size_t ssm_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int32_t num_splits);

const char* ssm_strerror(int code);   /* static text for a return code */
const char* ssm_last_error(void);     /* thread-local detail of the last failed call on this thread */
int ssm_abi_version(void);            /* SSM_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif
