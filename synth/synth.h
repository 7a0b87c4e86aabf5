/*
 * synth.h -- seeded synthetic inputs shared by the HIP path's tests/benchmark
 * and the CPU oracle.  Holds no attention arithmetic.  All buffers are host
 * memory owned by the caller; every output pointer may be NULL to skip it.
 * Functions return 0 on success, 1 on invalid arguments, 2 on allocation
 * failure.
 */
#ifndef SYNTH_H
#define SYNTH_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index);
double synth_uniform(uint64_t seed, uint64_t stream, uint64_t index);
double synth_normal(uint64_t seed, uint64_t stream, uint64_t index);
uint16_t synth_f32_to_bf16(float f);

/* GEN-A, prefill layout: Q [B,S,Hq,d], K/V [B,S,Hkv,d], contiguous. */
typedef struct {
  uint64_t seed;
  int32_t B, S, Hq, Hkv, d;
  int32_t rank;          /* r: rank of the shared factor (0 = none) */
  double shared_scale;   /* a: amplitude of the shared factor */
  double ar_window;      /* W: AR(1) correlation length in positions, phi = exp(-1/W) */
  double mu;             /* exact query component along u; < 0 selects sqrt(d/G) */
  int32_t tile_k;        /* key-tile length used for planting */
  int32_t sink_tiles;    /* leading key tiles that get sink_amp */
  double sink_amp;       /* keys += sink_amp*sqrt(d)*u on sink tiles */
  double rel_amp;        /* keys += rel_amp*sqrt(d)*u on relevant tiles */
  double rel_frac;       /* each tile t >= 1 relevant with this probability (if rel_count == 0) */
  int32_t rel_count;     /* > 0: exactly this many distinct relevant tiles t >= 1 per (b, group) */
} synth_gen_a_params;

int synth_gen_a(const synth_gen_a_params* p, uint16_t* q_bf16, uint16_t* k_bf16, uint16_t* v_bf16,
                float* q_f32, float* k_f32, float* v_f32,
                uint8_t* relevant_out /* [B*Hkv, ceil(S/tile_k)] */, int threads);

/* GEN-B, decode layout: q [B,Hq,d]; contiguous caches [B,Hkv,smax,d];
 * paged pools [num_pages,Hkv,tile_k,d] addressed through page_table [B,max_pages]
 * (page size = tile_k; unused entries hold 0). */
typedef struct {
  uint64_t seed;
  int32_t B, Hq, Hkv, d;
  int32_t tile_k;
  int32_t sink_tiles;
  double sink_amp, rel_amp, rel_frac;
} synth_gen_b_params;

void synth_kv_lens(uint64_t seed, int B, int lo, int hi, int32_t* out);
int64_t synth_num_pages(int B, const int32_t* kv_lens, int page);
int synth_gen_b(const synth_gen_b_params* p, const int32_t* kv_lens,
                uint16_t* q_bf16, float* q_f32,
                uint16_t* kc_bf16, uint16_t* vc_bf16, float* kc_f32, float* vc_f32, int64_t smax,
                uint16_t* kpool_bf16, uint16_t* vpool_bf16, int32_t* page_table, int32_t max_pages,
                uint8_t* relevant_out /* [B*Hkv, max_tiles] */, int threads);

#ifdef __cplusplus
}
#endif
#endif
