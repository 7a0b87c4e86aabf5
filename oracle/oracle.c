/*
 * oracle.c -- plain fp64 CPU oracle for Skip Softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the HIP kernels are
 * checked against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; it shares no code with the HIP library.  It is slow
 * on purpose: every step is written the way the method defines it, with no
 * blocking, fusion or reordering.
 *
 * Sources (the pages that describe the method):
 *   [recap]  "Accelerating Long-Context Inference with Skip Softmax in NVIDIA
 *            TensorRT-LLM" (video recap): Key Points; Detailed Analysis;
 *            Skip Softmax Mechanism; Impact on Accuracy vs. Speed; screenshot
 *            caption at 05:54.
 *   [news]   NVIDIA Skip Softmax news item: Understanding Skip Softmax;
 *            Benefits and Implementation; Accuracy and Sparsity Trade-offs.
 *   [topic]  "context length" topic page, Skip Softmax entry.
 *
 * What is computed (readings where the pages are silent are marked READING):
 *   1. Logits l_rj = scale * <q_r, k_j> for every visited (row, key) pair.
 *   2. Validity: causal prefill j <= i (top-left aligned, READING);
 *      non-causal j < S; decode j < kv_len (the new token is already in the
 *      cache, READING).  Chunked prefill (S new queries against S_k >= S keys
 *      whose last S positions are the queries' own): query i sees keys
 *      j <= S_k - S + i (bottom-right aligned, READING), non-causal j < S_k.
 *   3. Units and scans: a prefill unit is (b, h, q-tile) with one ascending
 *      scan over its visited key tiles; a decode unit is (b, KV group) whose
 *      rows are the group's query heads, scanned as num_splits consecutive
 *      chunks of ceil(n_tiles/num_splits) tiles (READING: each split-K chunk
 *      starts its own running maximum at -inf, as a split kernel does).
 *   4. Tile max M_r(t) over the row's valid keys in tile t; -inf means the
 *      row has no valid key there and abstains.
 *   5. The running maximum before tile t ("m_{i-1}", written "MI-1" in the
 *      recap's Key Points and Skip Softmax Mechanism): the max of M_r over the
 *      earlier tiles of the same scan, -inf for the scan's first tile.
 *      Sink-seeded split-K (decode option, READING): a split after the first
 *      starts from the unit's first-tile maxima M_r(0) instead of -inf, so its
 *      running maximum is max(M_r(0), earlier tiles of the split).  Tile 0 is
 *      the first tile of split 0 and is always kept, so the seed is a score the
 *      combined softmax contains, as the running maximum of one sequential scan
 *      would be.
 *   6. Gap g_r(t) = M_r(t) - running max (+inf when the running max is -inf);
 *      unit gap Gamma(t) = max over non-abstaining rows (every row of the
 *      tile must agree before the block is skipped, READING of "block").
 *   7. Skip iff tau > -inf and Gamma(t) < tau (recap, Detailed Analysis:
 *      the block is skipped when its local max falls below the running max
 *      by more than the threshold; Impact on Accuracy vs. Speed fixes the
 *      direction: a larger tau skips more).  A skipped tile contributes
 *      neither exponentials nor P*V ([news], Understanding Skip Softmax:
 *      blocks with negligible contribution are pruned early).
 *   8. Output: softmax over the kept keys, o_r = sum_j e^{l-mu} v_j / Z,
 *      lse_r = mu + ln Z.
 *   9. Diagnostics: tile state, Gamma per tile, dropped mass per row.
 *   Decode K/V may be stored as OCP fp8 e4m3 codes with per-tensor scales
 *   (key = k_scale * code, value = v_scale * code); steps 1-10 then apply to
 *   those dequantised values.
 *  10. A second, independent form: the online (running-max) softmax scan the
 *      pages describe, with the split-K log-sum-exp combine.  Because
 *      tau <= 0, a skipped tile never holds a new maximum, so the scan's
 *      running maximum equals step 5's prefix maximum and both forms produce
 *      the same mask.
 *  Rowmax-PoT weights (prefill option; "Approximating Softmax in Pretrained
 *  LLMs: Model Sensitivity and Kernel Acceleration", AI Summary and Abstract:
 *  the exponential is replaced by powers of two, a coarse logarithmic weight
 *  representation anchored at each row maximum).  READING: the base-2 log
 *  weight log2(e) * l of a kept key is rounded to the nearest integer k (ties
 *  to even) and its weight is 2^(k - K), K the rounded log weight of the row
 *  maximum over the kept keys (whose weight is therefore exactly 1).  Step 8
 *  then uses these weights in place of e^(l - mu); steps 1-7 (which tiles are
 *  skipped) are unchanged.  In the scan form the reference is the rounded log
 *  weight of the running maximum, so it moves by whole powers of two and both
 *  forms compute the same weights.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ input access */
/* OCP 8-bit float E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0
 * is subnormal (m * 2^-9); no infinities; S.1111.111 is NaN; largest finite value 448. */
static double fp8_e4m3_value(uint8_t b) {
  const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);  /* (1 + m/8) 2^(e-7) */
  return sign ? -mag : mag;
}

static double widen(const void* base, int dt, int64_t i) {
  if (dt == ORACLE_F64) return ((const double*)base)[i];
  if (dt == ORACLE_F32) return (double)((const float*)base)[i];
  if (dt == ORACLE_FP8E4M3) return fp8_e4m3_value(((const uint8_t*)base)[i]);
  /* bf16: the 16 stored bits are the top half of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Rowmax-PoT: the rounded base-2 log weight of a logit (see the header). */
static double pot_exponent(double logit) { return nearbyint(logit * 1.4426950408889634074); }

/* ------------------------------------------------------------ one unit */
typedef struct {
  int nr, d, tile_k, ntiles, nkeys;
  const double* q;          /* [nr][d] */
  const void* k;
  const void* v;
  int dt;                   /* dtype of k and v */
  double k_mul, v_mul;      /* per-tensor dequantisation factors of k and v */
  int64_t kv_base, kv_stride; /* key j, channel c at element kv_base + j*kv_stride + c */
  const int64_t* limit;     /* key j valid for row r iff j < limit[r] */
  int nscans;
  const int* scan_first;    /* [nscans + 1] */
  int seed_scans;           /* scans after the first start from the first tile's row maxima */
  double scale, tau;
  const int8_t* override;   /* [ntiles] or NULL */
  int pot;                  /* 1: Rowmax-PoT weights in place of the exponentials */
} unit_t;

typedef struct {
  double* out;      /* [nr][d] */
  double* lse;      /* [nr] */
  uint8_t* state;   /* [ntiles] */
  double* gamma;    /* [ntiles] */
  double* dropped;  /* [nr] */
} unit_out;

static void load_row(const unit_t* u, const void* src, int j, double* dst) {
  const double mul = src == u->k ? u->k_mul : u->v_mul;
  for (int c = 0; c < u->d; ++c) dst[c] = mul * widen(src, u->dt, u->kv_base + (int64_t)j * u->kv_stride + c);
}

static double dot(const double* a, const double* b, int d) {
  double s = 0;
  for (int c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Step 7: the decision for one tile from its unit gap. */
static int decide(const unit_t* u, int t, double unit_gap) {
  if (u->override && u->override[t] >= 0) return u->override[t] ? 1 : 0;
  return u->tau > -INFINITY && unit_gap < u->tau;
}

/* Step 6 for one row: the gap, or NaN when the row abstains. */
static double row_gap(double tile_max, double running_max) {
  if (tile_max == -INFINITY) return NAN;          /* no valid key: abstain */
  if (running_max == -INFINITY) return INFINITY;  /* first tile with a valid key */
  return tile_max - running_max;
}

/* Closed form: steps 1-9 exactly as listed above. */
static int unit_closed(const unit_t* u, unit_out* o) {
  const int nr = u->nr, d = u->d, nk = u->nkeys, T = u->tile_k, nt = u->ntiles;
  double* L = (double*)malloc(sizeof(double) * ((size_t)nr * (nk > 0 ? nk : 1)));
  double* M = (double*)malloc(sizeof(double) * ((size_t)nr * (nt > 0 ? nt : 1)));
  double* R = (double*)malloc(sizeof(double) * (size_t)nr);
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* mu = (double*)malloc(sizeof(double) * (size_t)nr);
  double* Z = (double*)malloc(sizeof(double) * (size_t)nr);
  double* lost = (double*)malloc(sizeof(double) * (size_t)nr);
  int* skip = (int*)malloc(sizeof(int) * (size_t)(nt > 0 ? nt : 1));
  int rc = 0;
  if (!L || !M || !R || !row || !mu || !Z || !lost || !skip) { rc = 2; goto done; }

  /* 1-2: logits of every visited pair; -inf marks an invalid pair */
  for (int j = 0; j < nk; ++j) {
    load_row(u, u->k, j, row);
    for (int r = 0; r < nr; ++r)
      L[(int64_t)r * nk + j] = j < u->limit[r] ? u->scale * dot(u->q + (int64_t)r * d, row, d) : -INFINITY;
  }
  /* 4: tile maxima */
  for (int r = 0; r < nr; ++r)
    for (int t = 0; t < nt; ++t) {
      double m = -INFINITY;
      for (int j = t * T; j < (t + 1) * T && j < nk; ++j)
        if (L[(int64_t)r * nk + j] > m) m = L[(int64_t)r * nk + j];
      M[(int64_t)r * nt + t] = m;
    }
  /* 5-7: per scan, prefix maxima, gaps, unit gap, decision */
  for (int s = 0; s < u->nscans; ++s) {
    for (int r = 0; r < nr; ++r) R[r] = u->seed_scans && s > 0 && nt > 0 ? M[(int64_t)r * nt] : -INFINITY;
    for (int t = u->scan_first[s]; t < u->scan_first[s + 1]; ++t) {
      double G = -INFINITY;
      int voters = 0;
      for (int r = 0; r < nr; ++r) {
        double g = row_gap(M[(int64_t)r * nt + t], R[r]);
        if (isnan(g)) continue;
        ++voters;
        if (g > G) G = g;
      }
      if (voters == 0) { rc = 3; goto done; }
      skip[t] = decide(u, t, G);
      if (o->gamma) o->gamma[t] = G;
      if (o->state) o->state[t] = skip[t] ? ORACLE_TILE_SKIPPED : ORACLE_TILE_EXECUTED;
      for (int r = 0; r < nr; ++r)
        if (M[(int64_t)r * nt + t] > R[r]) R[r] = M[(int64_t)r * nt + t];
    }
  }
  /* 8: softmax restricted to the kept keys; 9: dropped mass */
  for (int r = 0; r < nr; ++r) {
    const double* Lr = L + (int64_t)r * nk;
    double m = -INFINITY;
    for (int j = 0; j < nk; ++j)
      if (!skip[j / T] && Lr[j] > m) m = Lr[j];
    mu[r] = m;
    double z = 0, dz = 0;
    if (m > -INFINITY)
      for (int j = 0; j < nk; ++j) {
        if (Lr[j] == -INFINITY) continue;
        const double w = u->pot ? ldexp(1.0, (int)(pot_exponent(Lr[j]) - pot_exponent(m))) : exp(Lr[j] - m);
        if (!skip[j / T]) z += w;
        else dz += w;
      }
    Z[r] = z;
    lost[r] = dz;
  }
  if (o->out) memset(o->out, 0, sizeof(double) * (size_t)nr * d);
  for (int j = 0; j < nk; ++j) {
    if (skip[j / T]) continue;
    load_row(u, u->v, j, row);
    for (int r = 0; r < nr; ++r) {
      double l = L[(int64_t)r * nk + j];
      if (l == -INFINITY || !o->out) continue;
      double w = (u->pot ? ldexp(1.0, (int)(pot_exponent(l) - pot_exponent(mu[r]))) : exp(l - mu[r])) / Z[r];
      for (int c = 0; c < d; ++c) o->out[(int64_t)r * d + c] += w * row[c];
    }
  }
  for (int r = 0; r < nr; ++r) {
    int empty = mu[r] == -INFINITY;
    /* log of the sum of the kept weights before normalisation (PoT: of the 2^k) */
    if (o->lse) o->lse[r] = empty ? -INFINITY : (u->pot ? pot_exponent(mu[r]) * 0.6931471805599453094 : mu[r]) + log(Z[r]);
    if (o->dropped) o->dropped[r] = empty ? 0.0 : lost[r] / Z[r];
  }
done:
  free(L); free(M); free(R); free(row); free(mu); free(Z); free(lost); free(skip);
  return rc;
}

/* Scan form: the online softmax over each scan, then the log-sum-exp combine (step 10). */
static int unit_scan(const unit_t* u, unit_out* o) {
  const int nr = u->nr, d = u->d, nk = u->nkeys, T = u->tile_k;
  const int ns = u->nscans;
  double* m = (double*)malloc(sizeof(double) * (size_t)nr);
  double* l = (double*)malloc(sizeof(double) * (size_t)nr);
  double* a = (double*)malloc(sizeof(double) * (size_t)nr * d);
  double* os = (double*)malloc(sizeof(double) * (size_t)ns * nr * d);
  double* ls = (double*)malloc(sizeof(double) * (size_t)ns * nr);
  double* lt = (double*)malloc(sizeof(double) * (size_t)nr * T);
  double* Mt = (double*)malloc(sizeof(double) * (size_t)nr);
  double* row = (double*)malloc(sizeof(double) * (size_t)d);
  double* seed = (double*)malloc(sizeof(double) * (size_t)nr);
  double* kref = (double*)malloc(sizeof(double) * (size_t)nr);  /* PoT: rounded log weight of the running max */
  int rc = 0;
  if (!m || !l || !a || !os || !ls || !lt || !Mt || !row || !seed || !kref) { rc = 2; goto done; }
  /* sink seeding: the row maxima of the unit's first tile, from its own logits */
  for (int r = 0; r < nr; ++r) seed[r] = -INFINITY;
  if (u->seed_scans)
    for (int j = 0; j < T && j < nk; ++j) {
      load_row(u, u->k, j, row);
      for (int r = 0; r < nr; ++r) {
        if (j >= u->limit[r]) continue;
        double x = u->scale * dot(u->q + (int64_t)r * d, row, d);
        if (x > seed[r]) seed[r] = x;
      }
    }
  for (int s = 0; s < ns; ++s) {
    for (int r = 0; r < nr; ++r) { m[r] = -INFINITY; l[r] = 0; kref[r] = -INFINITY; }
    memset(a, 0, sizeof(double) * (size_t)nr * d);
    for (int t = u->scan_first[s]; t < u->scan_first[s + 1]; ++t) {
      const int j0 = t * T, j1 = (t + 1) * T < nk ? (t + 1) * T : nk;
      /* this tile's logits and row maxima */
      for (int r = 0; r < nr; ++r) Mt[r] = -INFINITY;
      for (int j = j0; j < j1; ++j) {
        load_row(u, u->k, j, row);
        for (int r = 0; r < nr; ++r) {
          double x = j < u->limit[r] ? u->scale * dot(u->q + (int64_t)r * d, row, d) : -INFINITY;
          lt[(int64_t)r * T + (j - j0)] = x;
          if (x > Mt[r]) Mt[r] = x;
        }
      }
      /* the gap against the running maximum of this scan, and the vote */
      double G = -INFINITY;
      int voters = 0;
      for (int r = 0; r < nr; ++r) {
        /* the scan's running maximum; a seeded split also counts the first tile's maximum */
        double run = s > 0 && seed[r] > m[r] ? seed[r] : m[r];
        double g = row_gap(Mt[r], run);
        if (isnan(g)) continue;
        ++voters;
        if (g > G) G = g;
      }
      if (voters == 0) { rc = 3; goto done; }
      int sk = decide(u, t, G);
      if (o->gamma) o->gamma[t] = G;
      if (o->state) o->state[t] = sk ? ORACLE_TILE_SKIPPED : ORACLE_TILE_EXECUTED;
      if (sk) continue;
      /* kept: rescale and accumulate */
      for (int r = 0; r < nr; ++r) {
        if (Mt[r] == -INFINITY) continue;
        double mn = Mt[r] > m[r] ? Mt[r] : m[r];
        double c;
        if (u->pot) {  /* the reference moves by whole powers of two */
          const double kn = pot_exponent(mn);
          c = kref[r] == -INFINITY ? 0.0 : ldexp(1.0, (int)(kref[r] - kn));
          kref[r] = kn;
        } else {
          c = exp(m[r] - mn);
        }
        l[r] *= c;
        for (int e = 0; e < d; ++e) a[(int64_t)r * d + e] *= c;
        m[r] = mn;
      }
      for (int j = j0; j < j1; ++j) {
        load_row(u, u->v, j, row);
        for (int r = 0; r < nr; ++r) {
          double x = lt[(int64_t)r * T + (j - j0)];
          if (x == -INFINITY) continue;
          double p = u->pot ? ldexp(1.0, (int)(pot_exponent(x) - kref[r])) : exp(x - m[r]);
          l[r] += p;
          for (int e = 0; e < d; ++e) a[(int64_t)r * d + e] += p * row[e];
        }
      }
    }
    for (int r = 0; r < nr; ++r) {
      double* osr = os + ((int64_t)s * nr + r) * d;
      if (l[r] > 0) {
        for (int e = 0; e < d; ++e) osr[e] = a[(int64_t)r * d + e] / l[r];
        ls[(int64_t)s * nr + r] = (u->pot ? kref[r] * 0.6931471805599453094 : m[r]) + log(l[r]);
      } else {
        for (int e = 0; e < d; ++e) osr[e] = 0;
        ls[(int64_t)s * nr + r] = -INFINITY;
      }
    }
  }
  /* log-sum-exp combine of the scans */
  for (int r = 0; r < nr; ++r) {
    double big = -INFINITY;
    for (int s = 0; s < ns; ++s)
      if (ls[(int64_t)s * nr + r] > big) big = ls[(int64_t)s * nr + r];
    double wsum = 0;
    if (o->out) for (int e = 0; e < d; ++e) o->out[(int64_t)r * d + e] = 0;
    if (big > -INFINITY) {
      for (int s = 0; s < ns; ++s) {
        double w = exp(ls[(int64_t)s * nr + r] - big);
        wsum += w;
        if (o->out)
          for (int e = 0; e < d; ++e) o->out[(int64_t)r * d + e] += w * os[((int64_t)s * nr + r) * d + e];
      }
      if (o->out) for (int e = 0; e < d; ++e) o->out[(int64_t)r * d + e] /= wsum;
    }
    if (o->lse) o->lse[r] = big > -INFINITY ? big + log(wsum) : -INFINITY;
    if (o->dropped) o->dropped[r] = NAN;
  }
done:
  free(m); free(l); free(a); free(os); free(ls); free(lt); free(Mt); free(row); free(seed); free(kref);
  return rc;
}

/* ------------------------------------------------------------ thread pool */
typedef struct {
  int (*fn)(void* ctx, int64_t i);
  void* ctx;
  int64_t n, next;
  int rc;
  pthread_mutex_t mu;
} jobs_t;

static void* jobs_worker(void* arg) {
  jobs_t* J = (jobs_t*)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t i = J->next++;
    int stop = J->rc != 0;
    pthread_mutex_unlock(&J->mu);
    if (i >= J->n || stop) break;
    int rc = J->fn(J->ctx, i);
    if (rc) {
      pthread_mutex_lock(&J->mu);
      if (!J->rc) J->rc = rc;
      pthread_mutex_unlock(&J->mu);
    }
  }
  return NULL;
}

static int run_jobs(int64_t n, int threads, int (*fn)(void*, int64_t), void* ctx) {
  jobs_t J;
  J.fn = fn; J.ctx = ctx; J.n = n; J.next = 0; J.rc = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if (threads > n) threads = n > 0 ? (int)n : 1;
  pthread_t tid[256];
  int started = 0;
  for (int t = 1; t < threads; ++t)
    if (pthread_create(&tid[started], NULL, jobs_worker, &J) == 0) ++started;
  jobs_worker(&J);
  for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
  pthread_mutex_destroy(&J.mu);
  return J.rc;
}

static int valid_tau(double tau) { return !isnan(tau) && (tau == -INFINITY || tau <= 0.0); }

/* ------------------------------------------------------------ prefill */
typedef struct {
  const oracle_prefill_shape* s;
  const void *q, *k, *v;
  int dt, form, nqt, nkt, Sk;
  double scale;
  const int64_t* units;
  const int8_t* override;
  double *out, *lse, *gamma, *dropped;
  uint8_t* state;
} prefill_job;

static int prefill_one(void* vctx, int64_t n) {
  prefill_job* P = (prefill_job*)vctx;
  const oracle_prefill_shape* s = P->s;
  const int64_t uid = P->units ? P->units[n] : n;
  const int qt = (int)(uid % P->nqt), h = (int)((uid / P->nqt) % s->Hq), b = (int)(uid / P->nqt / s->Hq);
  const int G = s->Hq / s->Hkv, g = h / G, Tq = s->tile_q, d = s->d;
  const int i0 = qt * Tq, i1 = (qt + 1) * Tq < s->S ? (qt + 1) * Tq : s->S;
  const int Sk = P->Sk, off = Sk - s->S;  /* keys per sequence; position of query 0 among them */
  double* q = (double*)malloc(sizeof(double) * (size_t)Tq * d);
  int64_t* limit = (int64_t*)malloc(sizeof(int64_t) * (size_t)Tq);
  if (!q || !limit) { free(q); free(limit); return 2; }
  for (int r = 0; r < Tq; ++r) {
    const int i = i0 + r;
    limit[r] = i < s->S ? (s->causal ? off + i + 1 : Sk) : 0;
    for (int c = 0; c < d; ++c)
      q[(int64_t)r * d + c] = i < s->S ? widen(P->q, P->dt, (((int64_t)b * s->S + i) * s->Hq + h) * d + c) : 0.0;
  }
  unit_t u;
  memset(&u, 0, sizeof u);
  u.nr = Tq; u.d = d; u.tile_k = s->tile_k;
  u.ntiles = s->causal ? (off + i1 - 1) / s->tile_k + 1 : P->nkt;
  u.nkeys = u.ntiles * s->tile_k < Sk ? u.ntiles * s->tile_k : Sk;
  u.q = q; u.k = P->k; u.v = P->v; u.dt = P->dt;
  u.k_mul = 1.0; u.v_mul = 1.0;
  u.kv_base = ((int64_t)b * Sk * s->Hkv + g) * d;
  u.kv_stride = (int64_t)s->Hkv * d;
  u.limit = limit;
  int scan_first[2] = {0, u.ntiles};
  u.nscans = 1; u.scan_first = scan_first;
  u.scale = P->scale; u.tau = s->tau;
  u.override = P->override ? P->override + n * P->nkt : NULL;
  u.pot = s->weights == ORACLE_WEIGHTS_ROWMAX_POT;
  unit_out o;
  o.out = P->out ? P->out + n * Tq * d : NULL;
  o.lse = P->lse ? P->lse + n * Tq : NULL;
  o.state = P->state ? P->state + n * P->nkt : NULL;
  o.gamma = P->gamma ? P->gamma + n * P->nkt : NULL;
  o.dropped = P->dropped ? P->dropped + n * Tq : NULL;
  if (o.state) memset(o.state, ORACLE_TILE_UNVISITED, (size_t)P->nkt);
  if (o.gamma) for (int t = 0; t < P->nkt; ++t) o.gamma[t] = NAN;
  int rc = P->form == ORACLE_SCAN_FORM ? unit_scan(&u, &o) : unit_closed(&u, &o);
  /* rows past the end of the sequence are padding */
  for (int r = i1 - i0; r < Tq; ++r) {
    if (o.out) memset(o.out + (int64_t)r * d, 0, sizeof(double) * (size_t)d);
    if (o.lse) o.lse[r] = -INFINITY;
    if (o.dropped) o.dropped[r] = P->form == ORACLE_SCAN_FORM ? NAN : 0.0;
  }
  free(q); free(limit);
  return rc;
}

int oracle_prefill(const oracle_prefill_shape* s, const void* q, const void* k, const void* v, int in_dtype,
                   const int64_t* units, int64_t n_units, const int8_t* override, int form,
                   double* out, double* lse, uint8_t* state, double* gamma, double* dropped, int threads) {
  if (!s || !q || !k || !v || s->B < 1 || s->S < 1 || s->Hq < 1 || s->Hkv < 1 || s->d < 1 ||
      s->Hq % s->Hkv || s->tile_q < 1 || s->tile_k < 1 || !valid_tau(s->tau) || in_dtype < 0 || in_dtype > 2 ||
      (s->S_k != 0 && s->S_k < s->S) || (s->weights != ORACLE_WEIGHTS_EXP && s->weights != ORACLE_WEIGHTS_ROWMAX_POT))
    return 1;
  prefill_job P;
  memset(&P, 0, sizeof P);
  P.s = s; P.q = q; P.k = k; P.v = v; P.dt = in_dtype; P.form = form;
  P.nqt = (s->S + s->tile_q - 1) / s->tile_q;
  P.Sk = s->S_k ? s->S_k : s->S;
  P.nkt = (P.Sk + s->tile_k - 1) / s->tile_k;
  P.scale = s->scale > 0 ? s->scale : 1.0 / sqrt((double)s->d);
  const int64_t total = (int64_t)s->B * s->Hq * P.nqt;
  if (units) {
    for (int64_t n = 0; n < n_units; ++n)
      if (units[n] < 0 || units[n] >= total) return 1;
  } else {
    n_units = total;
  }
  P.units = units; P.override = override;
  P.out = out; P.lse = lse; P.state = state; P.gamma = gamma; P.dropped = dropped;
  return run_jobs(n_units, threads, prefill_one, &P);
}

/* ------------------------------------------------------------ decode */
typedef struct {
  const oracle_decode_shape* s;
  const void *q, *k, *v;
  int dt, kvdt, form, maxt;
  double scale;
  const int32_t* kv_lens;
  const int64_t* units;
  const int8_t* override;
  double *out, *lse, *gamma, *dropped;
  uint8_t* state;
} decode_job;

static int decode_one(void* vctx, int64_t n) {
  decode_job* D = (decode_job*)vctx;
  const oracle_decode_shape* s = D->s;
  const int64_t uid = D->units ? D->units[n] : n;
  const int b = (int)(uid / s->Hkv), g = (int)(uid % s->Hkv);
  const int G = s->Hq / s->Hkv, d = s->d, T = s->tile_k, P = s->num_splits;
  const int len = D->kv_lens[b];
  const int nt = (len + T - 1) / T;
  double* q = (double*)malloc(sizeof(double) * (size_t)G * d);
  int64_t* limit = (int64_t*)malloc(sizeof(int64_t) * (size_t)G);
  int* first = (int*)malloc(sizeof(int) * (size_t)(P + 1));
  if (!q || !limit || !first) { free(q); free(limit); free(first); return 2; }
  for (int r = 0; r < G; ++r) {
    limit[r] = len;
    for (int c = 0; c < d; ++c) q[(int64_t)r * d + c] = widen(D->q, D->dt, ((int64_t)b * s->Hq + g * G + r) * d + c);
  }
  /* split s covers tiles [s*tps, (s+1)*tps) clipped to the unit's tiles */
  const int tps = (nt + P - 1) / P;
  for (int sp = 0; sp <= P; ++sp) first[sp] = sp * tps < nt ? sp * tps : nt;
  unit_t u;
  memset(&u, 0, sizeof u);
  u.nr = G; u.d = d; u.tile_k = T; u.ntiles = nt; u.nkeys = len;
  u.q = q; u.k = D->k; u.v = D->v; u.dt = D->kvdt;
  u.k_mul = s->k_scale > 0 ? s->k_scale : 1.0;
  u.v_mul = s->v_scale > 0 ? s->v_scale : 1.0;
  u.kv_base = ((int64_t)b * s->Hkv + g) * (int64_t)s->smax * d;
  u.kv_stride = d;
  u.limit = limit;
  u.nscans = P; u.scan_first = first;
  u.seed_scans = s->sink_seed != 0;
  u.scale = D->scale; u.tau = s->tau;
  u.override = D->override ? D->override + n * D->maxt : NULL;
  unit_out o;
  o.out = D->out ? D->out + n * G * d : NULL;
  o.lse = D->lse ? D->lse + n * G : NULL;
  o.state = D->state ? D->state + n * D->maxt : NULL;
  o.gamma = D->gamma ? D->gamma + n * D->maxt : NULL;
  o.dropped = D->dropped ? D->dropped + n * G : NULL;
  if (o.state) memset(o.state, ORACLE_TILE_UNVISITED, (size_t)D->maxt);
  if (o.gamma) for (int t = 0; t < D->maxt; ++t) o.gamma[t] = NAN;
  int rc = D->form == ORACLE_SCAN_FORM ? unit_scan(&u, &o) : unit_closed(&u, &o);
  free(q); free(limit); free(first);
  return rc;
}

int oracle_decode(const oracle_decode_shape* s, const void* q, const void* k, const void* v, int in_dtype,
                  const int32_t* kv_lens, const int64_t* units, int64_t n_units, const int8_t* override,
                  int form, double* out, double* lse, uint8_t* state, double* gamma, double* dropped,
                  int threads) {
  const int kvdt = s && s->kv_dtype >= 0 ? s->kv_dtype : in_dtype;
  if (!s || !q || !k || !v || !kv_lens || s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->d < 1 ||
      s->Hq % s->Hkv || s->smax < 0 || s->tile_k < 1 || s->num_splits < 1 || !valid_tau(s->tau) ||
      in_dtype < 0 || in_dtype > 2 || kvdt < 0 || kvdt > 3 || isnan(s->k_scale) || isnan(s->v_scale))
    return 1;
  for (int b = 0; b < s->B; ++b)
    if (kv_lens[b] < 0 || kv_lens[b] > s->smax) return 1;
  decode_job D;
  memset(&D, 0, sizeof D);
  D.s = s; D.q = q; D.k = k; D.v = v; D.dt = in_dtype; D.kvdt = kvdt; D.form = form;
  D.maxt = (s->smax + s->tile_k - 1) / s->tile_k;
  D.scale = s->scale > 0 ? s->scale : 1.0 / sqrt((double)s->d);
  D.kv_lens = kv_lens;
  const int64_t total = (int64_t)s->B * s->Hkv;
  if (units) {
    for (int64_t n = 0; n < n_units; ++n)
      if (units[n] < 0 || units[n] >= total) return 1;
  } else {
    n_units = total;
  }
  D.units = units; D.override = override;
  D.out = out; D.lse = lse; D.state = state; D.gamma = gamma; D.dropped = dropped;
  return run_jobs(n_units, threads, decode_one, &D);
}
