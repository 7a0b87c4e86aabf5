/*
 * oracle.h -- fp64 CPU oracle for Skip Softmax attention (TEST INFRASTRUCTURE).
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path never calls it.  It shares no code
 * with the HIP library.
 *
 * All buffers are host memory owned by the caller.  Inputs are read as fp32,
 * bf16 bit patterns, fp64 or (decode K/V only) OCP fp8 e4m3 codes
 * (ORACLE_F32 / ORACLE_BF16 / ORACLE_F64 / ORACLE_FP8E4M3) and widened to
 * double; all arithmetic is in double.
 *
 * Return codes: 0 ok, 1 invalid argument, 2 allocation failure,
 *               3 internal assertion failed (a visited tile with no valid key).
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2, ORACLE_FP8E4M3 = 3 };
enum { ORACLE_CLOSED_FORM = 0, ORACLE_SCAN_FORM = 1 };
enum { ORACLE_TILE_UNVISITED = 0, ORACLE_TILE_EXECUTED = 1, ORACLE_TILE_SKIPPED = 2 };
enum { ORACLE_WEIGHTS_EXP = 0, ORACLE_WEIGHTS_ROWMAX_POT = 1 };

typedef struct {
  int32_t B, S, Hq, Hkv, d;   /* q [B,S,Hq,d]; k, v [B,S,Hkv,d]; contiguous */
  int32_t tile_q, tile_k;
  int32_t causal;             /* 1: query i sees keys j <= i; 0: all j < S */
  double scale;               /* <= 0 selects 1/sqrt(d) */
  double tau;                 /* -inf: never skip; otherwise must be <= 0 */
  int32_t S_k;                /* chunked prefill: keys per sequence (k, v are [B,S_k,Hkv,d]); the S
                                 queries are the last S of S_k positions, so query i sees keys
                                 j <= S_k - S + i (bottom-right causal).  0 means S_k = S. */
  int32_t weights;            /* ORACLE_WEIGHTS_EXP, or ORACLE_WEIGHTS_ROWMAX_POT: a kept key's weight is
                                 2^(rint(log2(e) l) - rint(log2(e) mu)), mu the row maximum over the kept
                                 keys; lse is then the log of the sum of the 2^rint(log2(e) l) */
} oracle_prefill_shape;

/* Prefill units are u = (b*Hq + h)*ceil(S/tile_q) + qt.  units == NULL means all
 * units in that order.  Per listed unit (index n), with nkt = ceil(S_k/tile_k):
 *   out      [n][tile_q][d]   rows past S are 0
 *   lse      [n][tile_q]      natural log; rows past S are -inf
 *   state    [n][nkt]   0 unvisited, 1 executed, 2 skipped
 *   gamma    [n][nkt]   unit gap; NaN when unvisited
 *   dropped  [n][tile_q]      mass of valid keys outside the kept set (closed form only; NaN in scan form)
 *   override [n][nkt]   -1 decide by the rule, 0 force keep, 1 force skip (may be NULL)
 * Any output may be NULL. */
int oracle_prefill(const oracle_prefill_shape* s, const void* q, const void* k, const void* v, int in_dtype,
                   const int64_t* units, int64_t n_units, const int8_t* override, int form,
                   double* out, double* lse, uint8_t* state, double* gamma, double* dropped, int threads);

typedef struct {
  int32_t B, Hq, Hkv, d;      /* q [B,Hq,d]; k, v [B,Hkv,smax,d]; contiguous */
  int32_t smax;
  int32_t tile_k, num_splits;
  double scale, tau;
  int32_t sink_seed;          /* 1: every split after the first starts its running maximum at the
                                 unit's first-tile maxima instead of -inf (sink-seeded split-K) */
  int32_t kv_dtype;           /* dtype of k and v; < 0: the same as q's (in_dtype) */
  double k_scale, v_scale;    /* per-tensor dequantisation factors: key = k_scale * stored value,
                                 value = v_scale * stored value; <= 0 means 1 */
} oracle_decode_shape;

/* Decode units are u = b*Hkv + g (rows: the G = Hq/Hkv query heads of group g).
 *   out [n][G][d], lse [n][G], dropped [n][G],
 *   state / gamma / override [n][ceil(smax/tile_k)]. */
int oracle_decode(const oracle_decode_shape* s, const void* q, const void* k, const void* v, int in_dtype,
                  const int32_t* kv_lens, const int64_t* units, int64_t n_units, const int8_t* override,
                  int form, double* out, double* lse, uint8_t* state, double* gamma, double* dropped,
                  int threads);

#ifdef __cplusplus
}
#endif
#endif
