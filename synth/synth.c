/*
 * synth.c -- seeded synthetic inputs for Skip Softmax attention.
 *
 * This module produces Q/K/V tensors (and decode KV caches with page tables)
 * for both the HIP path and the CPU oracle.  It contains none of the
 * attention method's arithmetic: no logits, no maxima, no softmax, no skip
 * rule.  Only random numbers and the structure that makes some key tiles
 * skippable are produced here.
 *
 * Randomness is counter based, so every value depends only on
 * (seed, stream, index) and the bytes are identical for any thread count:
 *   - SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014): state_n = base + (n+1)*0x9e3779b97f4a7c15,
 *     output = mix(state_n) with the published finaliser constants.
 *   - 53-bit uniforms, then Box-Muller (Box and Muller 1958) normals: the pair
 *     (2m, 2m+1) shares two uniforms; even indices take the cosine branch, odd
 *     indices the sine branch.
 * Values are formed in double, rounded to fp32 (round to nearest even) and
 * then to bf16 (round to nearest even).  The fp32 copy is what a caller gets
 * as "unrounded" input; the bf16 copy is what the GPU consumes.
 *
 * Two workload families (the reading of the pages' workloads is documented in
 * the repository's design notes):
 *   GEN-A (prefill): per (batch, KV group) an orthonormal basis [U | u] from
 *     Gram-Schmidt of a Gaussian matrix; a rank-r factor c_i that follows an
 *     AR(1) process over positions (phi = exp(-1/window)); queries
 *     q = a*U*c_i + noise with the u-component then set to exactly mu; keys
 *     k = a*U*c_j + noise, plus amp*sqrt(d)*u on "sink" keys (tile 0) and on
 *     "relevant" key tiles.  V is standard normal.
 *   GEN-B (decode): q ~ N(0, I); per group the unit vector qhat along the sum
 *     of the group's queries; keys ~ N(0, I) plus amp*sqrt(d)*qhat on the sink
 *     tile and on relevant tiles; V ~ N(0, I).  Keys are indexed by logical
 *     position, so a contiguous cache and a paged pool hold identical content.
 */
#include "synth.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA64 0x9e3779b97f4a7c15ULL

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

uint64_t synth_u64(uint64_t seed, uint64_t stream, uint64_t index) {
  /* one SplitMix64 sequence per (seed, stream); index n picks its n-th output */
  uint64_t base = mix64(seed * GAMMA64 + 0x632be59bd9b4e019ULL) ^ mix64((stream + 1) * 0xd1b54a32d192ed03ULL);
  return mix64(base + (index + 1) * GAMMA64);
}

double synth_uniform(uint64_t seed, uint64_t stream, uint64_t index) {
  return (double)(synth_u64(seed, stream, index) >> 11) * (1.0 / 9007199254740992.0);
}

/* both normals of the Box-Muller pair that holds indices 2*pair and 2*pair+1 */
static void normal_pair(uint64_t seed, uint64_t stream, uint64_t pair, double* z0, double* z1) {
  /* u1 in (0, 1] so the logarithm is finite */
  double u1 = ((double)(synth_u64(seed, stream, 2 * pair) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
  double u2 = (double)(synth_u64(seed, stream, 2 * pair + 1) >> 11) * (1.0 / 9007199254740992.0);
  double rad = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586476925286766559 * u2;
  *z0 = rad * cos(ang);
  *z1 = rad * sin(ang);
}

double synth_normal(uint64_t seed, uint64_t stream, uint64_t index) {
  double z0, z1;
  normal_pair(seed, stream, index >> 1, &z0, &z1);
  return (index & 1) ? z1 : z0;
}

/* out[e] = normal(index0 + e) for e < n; index0 and n even */
static void normals(uint64_t seed, uint64_t stream, uint64_t index0, int n, double* out) {
  for (int e = 0; e < n; e += 2) normal_pair(seed, stream, (index0 + (uint64_t)e) >> 1, &out[e], &out[e + 1]);
}

uint16_t synth_f32_to_bf16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  if ((x & 0x7f800000u) == 0x7f800000u) /* inf or nan: truncate, keep nan quiet */
    return (uint16_t)((x >> 16) | ((x & 0xffffu) ? 0x40u : 0u));
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7fffu + lsb;
  return (uint16_t)(x >> 16);
}

static void store(int64_t i, double val, uint16_t* bf, float* f32) {
  float f = (float)val;
  if (f32) f32[i] = f;
  if (bf) bf[i] = synth_f32_to_bf16(f);
}

/* ------------------------------------------------------------------ threads */
typedef struct {
  void (*fn)(void* ctx, int64_t lo, int64_t hi);
  void* ctx;
  int64_t n, chunk;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* p = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t lo = p->next;
    p->next += p->chunk;
    pthread_mutex_unlock(&p->mu);
    if (lo >= p->n) break;
    int64_t hi = lo + p->chunk < p->n ? lo + p->chunk : p->n;
    p->fn(p->ctx, lo, hi);
  }
  return NULL;
}

static void parallel_for(int64_t n, int64_t chunk, int threads, void (*fn)(void*, int64_t, int64_t), void* ctx) {
  if (n <= 0) return;
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pool_t p;
  p.fn = fn; p.ctx = ctx; p.n = n; p.chunk = chunk < 1 ? 1 : chunk; p.next = 0;
  pthread_mutex_init(&p.mu, NULL);
  pthread_t tid[256];
  int started = 0;
  for (int t = 1; t < threads; ++t)
    if (pthread_create(&tid[started], NULL, pool_worker, &p) == 0) ++started;
  pool_worker(&p);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------ GEN-A */
enum { ST_Q = 1, ST_K = 2, ST_V = 3, ST_PLANT = 4, ST_KVLEN = 5, ST_PAGES = 6, ST_BASIS = 7, ST_AR = 8 };

typedef struct {
  const synth_gen_a_params* p;
  int G;
  double mu;
  double* basis;   /* [B*Hkv][(r+1)][d]: columns 0..r-1 = U, column r = u */
  double* factor;  /* [B*Hkv][S][r] */
  uint8_t* rel;    /* [B*Hkv][ntiles] 1 = relevant key tile */
  uint16_t *q_bf, *k_bf, *v_bf;
  float *q_f, *k_f, *v_f;
} gen_a_ctx;

static void gram_schmidt(double* cols, int ncol, int d) {
  for (int c = 0; c < ncol; ++c) {
    double* x = cols + (int64_t)c * d;
    for (int p = 0; p < c; ++p) {
      const double* y = cols + (int64_t)p * d;
      double dot = 0;
      for (int i = 0; i < d; ++i) dot += x[i] * y[i];
      for (int i = 0; i < d; ++i) x[i] -= dot * y[i];
    }
    double nrm = 0;
    for (int i = 0; i < d; ++i) nrm += x[i] * x[i];
    nrm = sqrt(nrm);
    for (int i = 0; i < d; ++i) x[i] /= nrm;
  }
}

static void gen_a_rows(void* vctx, int64_t lo, int64_t hi) {
  gen_a_ctx* c = (gen_a_ctx*)vctx;
  const synth_gen_a_params* p = c->p;
  const int d = p->d, r = p->rank, Hq = p->Hq, Hkv = p->Hkv, S = p->S;
  const int ntiles = (S + p->tile_k - 1) / p->tile_k;
  double* w = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t row = lo; row < hi; ++row) { /* row = b*S + i */
    const int b = (int)(row / S), i = (int)(row % S);
    for (int g = 0; g < Hkv; ++g) {
      const int64_t bg = (int64_t)b * Hkv + g;
      const double* U = c->basis + bg * (int64_t)(r + 1) * d;
      const double* u = U + (int64_t)r * d;
      const double* ci = c->factor + (bg * S + i) * (int64_t)r;
      /* shared low-rank part a*U*c_i */
      for (int e = 0; e < d; ++e) {
        double s = 0;
        for (int j = 0; j < r; ++j) s += U[(int64_t)j * d + e] * ci[j];
        w[e] = p->shared_scale * s;
      }
      /* queries of this group */
      for (int hh = 0; hh < c->G; ++hh) {
        const int h = g * c->G + hh;
        const int64_t base = (row * Hq + h) * (int64_t)d;
        double qv[1024];
        double dot = 0;
        normals(p->seed, ST_Q, (uint64_t)base, d, qv);
        for (int e = 0; e < d; ++e) {
          qv[e] += w[e];
          dot += qv[e] * u[e];
        }
        for (int e = 0; e < d; ++e) store(base + e, qv[e] + (c->mu - dot) * u[e], c->q_bf, c->q_f);
      }
      /* key and value of this group */
      const int64_t kbase = (row * Hkv + g) * (int64_t)d;
      const int t = i / p->tile_k;
      double shift = 0;
      if (t < p->sink_tiles) shift += p->sink_amp * sqrt((double)d);
      if (c->rel[bg * ntiles + t]) shift += p->rel_amp * sqrt((double)d);
      double kn[1024], vn[1024];
      normals(p->seed, ST_K, (uint64_t)kbase, d, kn);
      normals(p->seed, ST_V, (uint64_t)kbase, d, vn);
      for (int e = 0; e < d; ++e) {
        store(kbase + e, w[e] + kn[e] + shift * u[e], c->k_bf, c->k_f);
        store(kbase + e, vn[e], c->v_bf, c->v_f);
      }
    }
  }
  free(w);
}

int synth_gen_a(const synth_gen_a_params* p, uint16_t* q_bf16, uint16_t* k_bf16, uint16_t* v_bf16,
                float* q_f32, float* k_f32, float* v_f32, uint8_t* relevant_out, int threads) {
  if (!p || p->B < 1 || p->S < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 2 || p->d > 1024 || p->d % 2 != 0 ||
      p->Hq % p->Hkv != 0 || p->rank < 0 || p->rank >= p->d || p->tile_k < 1)
    return 1;
  gen_a_ctx c;
  memset(&c, 0, sizeof c);
  c.p = p;
  c.G = p->Hq / p->Hkv;
  c.mu = p->mu >= 0 ? p->mu : sqrt((double)p->d / c.G);
  c.q_bf = q_bf16; c.k_bf = k_bf16; c.v_bf = v_bf16;
  c.q_f = q_f32; c.k_f = k_f32; c.v_f = v_f32;
  const int d = p->d, r = p->rank, S = p->S;
  const int64_t ngroups = (int64_t)p->B * p->Hkv;
  const int ntiles = (S + p->tile_k - 1) / p->tile_k;
  c.basis = (double*)malloc(sizeof(double) * (size_t)(ngroups * (r + 1) * d));
  c.factor = (double*)malloc(sizeof(double) * (size_t)(ngroups * S * (r > 0 ? r : 1)));
  c.rel = (uint8_t*)calloc((size_t)(ngroups * ntiles), 1);
  if (!c.basis || !c.factor || !c.rel) { free(c.basis); free(c.factor); free(c.rel); return 2; }
  for (int64_t bg = 0; bg < ngroups; ++bg) {
    double* cols = c.basis + bg * (r + 1) * d;
    for (int64_t e = 0; e < (int64_t)(r + 1) * d; ++e) cols[e] = synth_normal(p->seed, ST_BASIS, (uint64_t)(bg * (r + 1) * d + e));
    gram_schmidt(cols, r + 1, d);
    /* AR(1) factor, stationary N(0, I_r) */
    if (r > 0) {
      const double phi = exp(-1.0 / p->ar_window), inn = sqrt(1.0 - phi * phi);
      double* f = c.factor + bg * S * r;
      for (int i = 0; i < S; ++i)
        for (int j = 0; j < r; ++j) {
          double eps = synth_normal(p->seed, ST_AR, (uint64_t)((bg * S + i) * r + j));
          f[(int64_t)i * r + j] = i == 0 ? eps : phi * f[(int64_t)(i - 1) * r + j] + inn * eps;
        }
    }
    /* relevant key tiles (never tile 0): either a fixed count or a Bernoulli fraction */
    uint8_t* rel = c.rel + bg * ntiles;
    if (p->rel_count > 0) {
      int n = ntiles - 1, want = p->rel_count < n ? p->rel_count : n;
      int* idx = (int*)malloc(sizeof(int) * (size_t)(n > 0 ? n : 1));
      for (int t = 0; t < n; ++t) idx[t] = t + 1;
      for (int t = 0; t < want; ++t) { /* partial Fisher-Yates */
        int j = t + (int)(synth_uniform(p->seed, ST_PLANT, (uint64_t)(bg * ntiles + t)) * (n - t));
        int tmp = idx[t]; idx[t] = idx[j]; idx[j] = tmp;
        rel[idx[t]] = 1;
      }
      free(idx);
    } else if (p->rel_frac > 0) {
      for (int t = 1; t < ntiles; ++t)
        rel[t] = synth_uniform(p->seed, ST_PLANT, (uint64_t)(bg * ntiles + t)) < p->rel_frac;
    }
  }
  parallel_for((int64_t)p->B * S, 256, threads, gen_a_rows, &c);
  if (relevant_out) memcpy(relevant_out, c.rel, (size_t)(ngroups * ntiles));
  free(c.basis); free(c.factor); free(c.rel);
  return 0;
}

/* ------------------------------------------------------------------ GEN-B */
#define LOGICAL_STRIDE ((int64_t)1 << 24) /* positions per sequence in the key index space */

void synth_kv_lens(uint64_t seed, int B, int lo, int hi, int32_t* out) {
  for (int b = 0; b < B; ++b) {
    double u = synth_uniform(seed, ST_KVLEN, (uint64_t)b);
    int64_t v = lo + (int64_t)(u * (double)(hi - lo + 1));
    out[b] = (int32_t)(v > hi ? hi : v);
  }
}

int64_t synth_num_pages(int B, const int32_t* kv_lens, int page) {
  int64_t n = 0;
  for (int b = 0; b < B; ++b) n += (kv_lens[b] + page - 1) / page;
  return n;
}

typedef struct {
  const synth_gen_b_params* p;
  const int32_t* kv_lens;
  int G, max_tiles;
  double* qhat;   /* [B*Hkv][d] */
  uint8_t* rel;   /* [B*Hkv][max_tiles] */
  const int32_t* page_table;
  int32_t max_pages;
  int64_t smax;
  uint16_t *kc_bf, *vc_bf, *kp_bf, *vp_bf;
  float *kc_f, *vc_f;
} gen_b_ctx;

static void gen_b_tokens(void* vctx, int64_t lo, int64_t hi) {
  gen_b_ctx* c = (gen_b_ctx*)vctx;
  const synth_gen_b_params* p = c->p;
  const int d = p->d, Hkv = p->Hkv, T = p->tile_k;
  for (int64_t bt = lo; bt < hi; ++bt) { /* bt = b*max_tiles + tile */
    const int b = (int)(bt / c->max_tiles), t = (int)(bt % c->max_tiles);
    const int len = c->kv_lens[b];
    if ((int64_t)t * T >= len) continue;
    for (int g = 0; g < Hkv; ++g) {
      const int64_t bg = (int64_t)b * Hkv + g;
      double shift = 0;
      if (t < p->sink_tiles) shift += p->sink_amp * sqrt((double)d);
      if (c->rel[bg * c->max_tiles + t]) shift += p->rel_amp * sqrt((double)d);
      const double* qh = c->qhat + bg * d;
      for (int jj = 0; jj < T; ++jj) {
        const int64_t j = (int64_t)t * T + jj;
        const int valid = j < len;
        const int64_t lidx = ((b * LOGICAL_STRIDE + j) * Hkv + g) * (int64_t)d;
        double kn[1024], vn[1024];
        if (valid) {
          normals(p->seed, ST_K, (uint64_t)lidx, d, kn);
          normals(p->seed, ST_V, (uint64_t)lidx, d, vn);
        }
        for (int e = 0; e < d; ++e) {
          double kv = 0, vv = 0;
          if (valid) {
            kv = kn[e] + shift * qh[e];
            vv = vn[e];
          }
          if (c->kc_bf || c->kc_f) {
            if (j < c->smax) {
              int64_t ci = ((bg * c->smax) + j) * d + e;
              store(ci, kv, c->kc_bf, c->kc_f);
              store(ci, vv, c->vc_bf, c->vc_f);
            }
          }
          if (c->kp_bf) {
            int64_t page = c->page_table[(int64_t)b * c->max_pages + t];
            int64_t pi = ((page * Hkv + g) * T + jj) * d + e;
            store(pi, kv, c->kp_bf, NULL);
            store(pi, vv, c->vp_bf, NULL);
          }
        }
      }
    }
  }
}

int synth_gen_b(const synth_gen_b_params* p, const int32_t* kv_lens,
                uint16_t* q_bf16, float* q_f32,
                uint16_t* kc_bf16, uint16_t* vc_bf16, float* kc_f32, float* vc_f32, int64_t smax,
                uint16_t* kpool_bf16, uint16_t* vpool_bf16, int32_t* page_table, int32_t max_pages,
                uint8_t* relevant_out, int threads) {
  if (!p || !kv_lens || p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->d < 2 || p->d > 1024 || p->d % 2 != 0 ||
      p->Hq % p->Hkv != 0 || p->tile_k < 1)
    return 1;
  gen_b_ctx c;
  memset(&c, 0, sizeof c);
  c.p = p;
  c.kv_lens = kv_lens;
  c.G = p->Hq / p->Hkv;
  const int d = p->d, T = p->tile_k;
  int maxlen = 0;
  for (int b = 0; b < p->B; ++b) {
    if (kv_lens[b] < 0) return 1;
    if (kv_lens[b] > maxlen) maxlen = kv_lens[b];
  }
  c.max_tiles = (maxlen + T - 1) / T;
  if (c.max_tiles < 1) c.max_tiles = 1;
  if ((kc_bf16 || kc_f32) && smax < maxlen) return 1;
  if (kpool_bf16 && (!vpool_bf16 || !page_table || max_pages < c.max_tiles)) return 1;
  c.smax = smax;
  c.kc_bf = kc_bf16; c.vc_bf = vc_bf16; c.kc_f = kc_f32; c.vc_f = vc_f32;
  c.kp_bf = kpool_bf16; c.vp_bf = vpool_bf16;
  c.max_pages = max_pages;
  const int64_t ngroups = (int64_t)p->B * p->Hkv;
  c.qhat = (double*)calloc((size_t)(ngroups * d), sizeof(double));
  c.rel = (uint8_t*)calloc((size_t)(ngroups * c.max_tiles), 1);
  if (!c.qhat || !c.rel) { free(c.qhat); free(c.rel); return 2; }
  /* queries and the group direction qhat */
  for (int b = 0; b < p->B; ++b)
    for (int h = 0; h < p->Hq; ++h) {
      double* qh = c.qhat + ((int64_t)b * p->Hkv + h / c.G) * d;
      for (int e = 0; e < d; ++e) {
        int64_t i = ((int64_t)b * p->Hq + h) * d + e;
        double x = synth_normal(p->seed, ST_Q, (uint64_t)i);
        store(i, x, q_bf16, q_f32);
        qh[e] += x;
      }
    }
  for (int64_t bg = 0; bg < ngroups; ++bg) {
    double* qh = c.qhat + bg * d, n = 0;
    for (int e = 0; e < d; ++e) n += qh[e] * qh[e];
    n = sqrt(n);
    for (int e = 0; e < d; ++e) qh[e] /= n;
    for (int t = 1; t < c.max_tiles; ++t)
      c.rel[bg * c.max_tiles + t] = synth_uniform(p->seed, ST_PLANT, (uint64_t)(bg * c.max_tiles + t)) < p->rel_frac;
  }
  /* page table: a seeded permutation of all pages, handed out in sequence order */
  if (page_table) {
    int64_t np = synth_num_pages(p->B, kv_lens, T);
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(np > 0 ? np : 1));
    for (int64_t i = 0; i < np; ++i) perm[i] = (int32_t)i;
    for (int64_t i = np - 1; i > 0; --i) { /* Fisher-Yates */
      int64_t j = (int64_t)(synth_uniform(p->seed, ST_PAGES, (uint64_t)i) * (double)(i + 1));
      if (j > i) j = i;
      int32_t tmp = perm[i]; perm[i] = perm[j]; perm[j] = tmp;
    }
    int64_t off = 0;
    for (int b = 0; b < p->B; ++b) {
      int nt = (kv_lens[b] + T - 1) / T;
      for (int t = 0; t < max_pages; ++t) page_table[(int64_t)b * max_pages + t] = t < nt ? perm[off + t] : 0;
      off += nt;
    }
    free(perm);
    c.page_table = page_table;
  }
  /* zero the contiguous caches past each sequence's length (tokens never generated) */
  if (kc_bf16 || kc_f32) {
    for (int b = 0; b < p->B; ++b)
      for (int g = 0; g < p->Hkv; ++g) {
        int64_t start = ((int64_t)b * p->Hkv + g) * smax * d;
        int64_t from = (int64_t)((kv_lens[b] + T - 1) / T) * T;
        if (from > smax) from = smax;
        for (int64_t j = from * d; j < smax * d; ++j) {
          if (kc_bf16) { kc_bf16[start + j] = 0; vc_bf16[start + j] = 0; }
          if (kc_f32) { kc_f32[start + j] = 0; vc_f32[start + j] = 0; }
        }
      }
  }
  parallel_for((int64_t)p->B * c.max_tiles, 16, threads, gen_b_tokens, &c);
  if (relevant_out) memcpy(relevant_out, c.rel, (size_t)(ngroups * c.max_tiles));
  free(c.qhat); free(c.rel);
  return 0;
}
