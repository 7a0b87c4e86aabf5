// ssm_api.cpp -- C ABI of libssm.so: argument validation, defaults, launch.
//
// Every check runs on the host before any HIP call, so invalid requests return
// an error code without touching the device.  Nothing here allocates device
// memory, synchronises, or reads device data.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/ssm.h"
#include "ssm_launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

// An empty tensor (some extent 0) may carry a NULL data pointer: nothing is read or written through it.
int check_tensor(const ssm_tensor* t, const char* name, int ndim, int dtype) {
  if (!t) return fail(SSM_EINVAL, "%s: NULL descriptor", name);
  if (t->ndim != ndim) return fail(SSM_EINVAL, "%s: expected %d dims, got %d", name, ndim, (int)t->ndim);
  bool empty = false;
  for (int i = 0; i < ndim; ++i) empty = empty || t->shape[i] == 0;
  if (!t->data && !empty) return fail(SSM_EINVAL, "%s: NULL data pointer", name);
  if (t->dtype != dtype)
    return fail(SSM_EUNSUPPORTED, "%s: dtype %d not supported here (%s required)", name, (int)t->dtype,
                dtype == SSM_BF16 ? "bf16" : "fp8 e4m3");
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(SSM_EINVAL, "%s: negative extent in dim %d", name, i);
  if (t->stride[ndim - 1] != 1) return fail(SSM_EINVAL, "%s: last dimension must be contiguous", name);
  const int gran = dtype == SSM_FP8_E4M3 ? 16 : 8;  // elements per 16 bytes
  for (int i = 0; i < ndim - 1; ++i)
    if (t->stride[i] < 0 || t->stride[i] % gran != 0)
      return fail(SSM_EUNSUPPORTED, "%s: stride[%d]=%lld must be a non-negative multiple of %d elements", name, i,
                  (long long)t->stride[i], gran);
  if (!empty && reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(SSM_EUNSUPPORTED, "%s: data must be 16-byte aligned", name);
  return SSM_OK;
}

int check_tau(float tau) {
  if (std::isnan(tau)) return fail(SSM_EINVAL, "tau is NaN");
  if (tau > 0.f) return fail(SSM_EINVAL, "tau must be -inf or <= 0 (got %g)", (double)tau);
  return SSM_OK;
}

int resolve_scale(const ssm_opts* opts, int d, float* scale) {
  float s = opts ? opts->scale : 0.f;
  if (std::isnan(s) || s < 0.f || std::isinf(s)) return fail(SSM_EINVAL, "scale must be finite and >= 0");
  *scale = s > 0.f ? s : 1.f / std::sqrt((float)d);
  return SSM_OK;
}

int launch_status(hipError_t e) {
  if (e != hipSuccess) return fail(SSM_EHIP, "HIP launch failed: %s", hipGetErrorString(e));
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_strerror(int code) {
  switch (code) {
    case SSM_OK: return "ok";
    case SSM_EINVAL: return "invalid argument";
    case SSM_EUNSUPPORTED: return "unsupported configuration";
    case SSM_EWORKSPACE: return "workspace missing or too small";
    case SSM_EHIP: return "HIP runtime error";
    default: return "unknown error code";
  }
}

const char* ssm_last_error(void) { return g_last_error; }

namespace {
// decode workspace layout: partial outputs [B, Hq, P, d] fp32 | partial LSEs [B, Hq, P] fp32 | dispatch order [B]
// int32 (batches up to kDecSortMax) | skip counts per split workgroup [B, Hkv, P, 2] uint32 (sized for Hkv = Hq),
// each part starting on a 256-byte boundary
struct DecodeWs {
  size_t lse_off, order_off, cnt_off, bytes;
};
DecodeWs decode_ws_layout(size_t B, size_t Hq, size_t d, size_t P) {
  const size_t rows = B * Hq * P;
  DecodeWs w;
  w.lse_off = (rows * d * sizeof(float) + 255) & ~(size_t)255;
  w.order_off = (w.lse_off + rows * sizeof(float) + 255) & ~(size_t)255;
  w.cnt_off = (w.order_off + (B <= (size_t)ssm::kDecSortMax ? B * sizeof(int32_t) : 0) + 255) & ~(size_t)255;
  w.bytes = w.cnt_off + rows * 2 * sizeof(uint32_t);
  return w;
}
}  // namespace

size_t ssm_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t d, int32_t num_splits) {
  if (B < 0 || Hq < 0 || d <= 0 || num_splits <= 0) return 0;
  return decode_ws_layout((size_t)B, (size_t)Hq, (size_t)d, (size_t)num_splits).bytes;
}

// qk8: q and k hold e4m3 codes with dequantisation factors q_scale, k_scale (ssm_prefill_fp8qk)
static int prefill_impl(const ssm_tensor* q, const ssm_tensor* k, const ssm_tensor* v, int32_t seqlen, int32_t causal,
                        float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream, const ssm_opts* opts,
                        bool qk8, float q_scale, float k_scale) {
  int rc;
  const int qk_dt = qk8 ? SSM_FP8_E4M3 : SSM_BF16;
  if ((rc = check_tensor(q, "q", 4, qk_dt)) || (rc = check_tensor(k, "k", 4, qk_dt)) ||
      (rc = check_tensor(v, "v", 4, SSM_BF16)) || (rc = check_tensor(out, "out", 4, SSM_BF16)))
    return rc;
  if ((rc = check_tau(tau))) return rc;
  if (qk8 && !(q_scale > 0.f && std::isfinite(q_scale) && k_scale > 0.f && std::isfinite(k_scale)))
    return fail(SSM_EINVAL, "q_scale and k_scale must be finite and > 0");
  const int64_t B = q->shape[0], S = q->shape[1], Hq = q->shape[2], d = q->shape[3];
  const int64_t Hkv = k->shape[2];
  if (seqlen != S) return fail(SSM_EINVAL, "seqlen %d != q.shape[1] %lld", (int)seqlen, (long long)S);
  for (int i = 0; i < 4; ++i) {
    const int64_t want_kv = i == 2 ? Hkv : q->shape[i];
    if (k->shape[i] != want_kv || v->shape[i] != want_kv)
      return fail(SSM_EINVAL, "k/v shape mismatch in dim %d", i);
    if (out->shape[i] != q->shape[i]) return fail(SSM_EINVAL, "out shape mismatch in dim %d", i);
  }
  if (Hkv <= 0 || Hq % Hkv != 0) return fail(SSM_EINVAL, "Hq (%lld) must be a positive multiple of Hkv (%lld)",
                                             (long long)Hq, (long long)Hkv);
  if (d != 64 && d != 128) return fail(SSM_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  const int tile_q = (opts && opts->tile_q) ? opts->tile_q : 128;
  const int tile_k = (opts && opts->tile_k) ? opts->tile_k : 64;
  if (tile_q != 64 && tile_q != 128) return fail(SSM_EUNSUPPORTED, "tile_q %d not supported (64 or 128)", tile_q);
  if (tile_k != 64) return fail(SSM_EUNSUPPORTED, "tile_k %d not supported (64)", tile_k);
  float scale;
  if ((rc = resolve_scale(opts, (int)d, &scale))) return rc;
  const int32_t weights = opts ? opts->weights : SSM_WEIGHTS_EXP;
  if (weights != SSM_WEIGHTS_EXP && weights != SSM_WEIGHTS_ROWMAX_POT)
    return fail(SSM_EINVAL, "unknown weights %d", (int)weights);
  if (B > INT32_MAX || S > (1 << 30) || Hq > 65536) return fail(SSM_EUNSUPPORTED, "problem too large");
  const int64_t nqt = (S + tile_q - 1) / tile_q, nkt = (S + tile_k - 1) / tile_k;
  const int64_t units = B * Hq * nqt;
  if (units > INT32_MAX) return fail(SSM_EUNSUPPORTED, "too many query tiles");
  // the kernels address each (batch, head) slice with 32-bit byte offsets
  for (const ssm_tensor* t : {q, k, v}) {
    const int64_t es = t->dtype == SSM_FP8_E4M3 ? 1 : 2;
    if ((S + 128) * t->stride[1] * es + d * es > (int64_t)UINT32_MAX)
      return fail(SSM_EUNSUPPORTED, "sequence too long for 32-bit slice offsets (S=%lld, row stride %lld)",
                  (long long)S, (long long)t->stride[1]);
  }
  if (skip_stats) {
    if (skip_stats->tile_state && skip_stats->tile_state_len < units * nkt)
      return fail(SSM_EINVAL, "tile_state needs %lld elements", (long long)(units * nkt));
    if (skip_stats->unit_gap && skip_stats->unit_gap_len < units * nkt)
      return fail(SSM_EINVAL, "unit_gap needs %lld elements", (long long)(units * nkt));
  }
  if (B == 0 || S == 0 || Hq == 0) return SSM_OK;

  ssm::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q->data);
  a.k = static_cast<const uint16_t*>(k->data);
  a.v = static_cast<const uint16_t*>(v->data);
  a.o = static_cast<uint16_t*>(out->data);
  a.q_sb = q->stride[0]; a.q_ss = q->stride[1]; a.q_sh = q->stride[2];
  a.k_sb = k->stride[0]; a.k_ss = k->stride[1]; a.k_sh = k->stride[2];
  a.v_sb = v->stride[0]; a.v_ss = v->stride[1]; a.v_sh = v->stride[2];
  a.o_sb = out->stride[0]; a.o_ss = out->stride[1]; a.o_sh = out->stride[2];
  a.B = (int)B; a.S = (int)S; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  a.nqt = (int)nqt; a.nkt = (int)nkt;
  a.causal = causal != 0;
  // the kernels score raw code products; the dequantisation factors join the logit scale
  const float lscale = qk8 ? scale * q_scale * k_scale : scale;
  if (!(lscale > 0.f) || !std::isfinite(lscale)) return fail(SSM_EINVAL, "scale * q_scale * k_scale out of range");
  a.scale = lscale;
  a.scale_log2 = lscale * 1.4426950408889634f;
  a.tau_raw = std::isinf(tau) ? tau : tau / lscale;
  a.v_scale = 1.f;
  a.pot = weights == SSM_WEIGHTS_ROWMAX_POT;
  if (skip_stats) {
    a.tile_state = skip_stats->tile_state;
    a.unit_gap = skip_stats->unit_gap;
    a.counters = skip_stats->counters;
  }
  return launch_status(ssm::launch_prefill(a, (int)d, tile_q, false, qk8 ? 1 : 0, static_cast<hipStream_t>(stream)));
}

int ssm_prefill(const ssm_tensor* q, const ssm_tensor* k, const ssm_tensor* v, int32_t seqlen, int32_t causal,
                float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream, const ssm_opts* opts) {
  return prefill_impl(q, k, v, seqlen, causal, tau, out, skip_stats, stream, opts, false, 1.f, 1.f);
}

int ssm_prefill_fp8qk(const ssm_tensor* q, float q_scale, const ssm_tensor* k, float k_scale, const ssm_tensor* v,
                      int32_t seqlen, int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats,
                      void* stream, const ssm_opts* opts) {
  return prefill_impl(q, k, v, seqlen, causal, tau, out, skip_stats, stream, opts, true, q_scale, k_scale);
}

static int check_cache(const ssm_kv_cache* c, const char* name, int64_t B, int64_t d, int* kv_cap, int64_t* pool_rows,
                       int64_t* heads) {
  if (!c) return fail(SSM_EINVAL, "%s: NULL descriptor", name);
  const int dt = c->pool.dtype == SSM_FP8_E4M3 ? SSM_FP8_E4M3 : SSM_BF16;
  int rc = check_tensor(&c->pool, name, 4, dt);
  if (rc) return rc;
  if (dt == SSM_FP8_E4M3 && !(c->scale > 0.f && std::isfinite(c->scale)))
    return fail(SSM_EINVAL, "%s: an fp8 cache needs a finite scale > 0", name);
  if (c->pool.shape[3] != d) return fail(SSM_EINVAL, "%s: head_dim mismatch", name);
  *heads = c->pool.shape[1];
  if (c->page_table) {
    if (c->page_size != 64) return fail(SSM_EUNSUPPORTED, "%s: page_size must equal the key tile (64)", name);
    if (c->pool.shape[2] != 64) return fail(SSM_EINVAL, "%s: pool dim 2 must equal page_size", name);
    if (c->max_pages <= 0) return fail(SSM_EINVAL, "%s: max_pages must be positive", name);
    if ((int64_t)c->max_pages * 64 > INT32_MAX) return fail(SSM_EUNSUPPORTED, "%s: too many pages", name);
    *kv_cap = c->max_pages * 64;
    *pool_rows = c->pool.shape[0];
  } else {
    if (c->pool.shape[0] != B) return fail(SSM_EINVAL, "%s: contiguous cache dim 0 must equal batch", name);
    if (c->pool.shape[2] > INT32_MAX) return fail(SSM_EUNSUPPORTED, "%s: cache too long", name);
    *kv_cap = (int)c->pool.shape[2];
    *pool_rows = 0;
  }
  return SSM_OK;
}

// noalloc: the workspace is this GPU's static scratch array (ssm_decode_noalloc) instead of opts->workspace
static int decode_impl(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                       const int32_t* kv_lens, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                       const ssm_opts* opts, bool noalloc) {
  int rc;
  if ((rc = check_tensor(q, "q", 3, SSM_BF16)) || (rc = check_tensor(out, "out", 3, SSM_BF16))) return rc;
  if ((rc = check_tau(tau))) return rc;
  const int64_t B = q->shape[0], Hq = q->shape[1], d = q->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(SSM_EINVAL, "out shape mismatch in dim %d", i);
  if (B == 0 || Hq == 0) return SSM_OK;  // nothing to compute (the caches, kv_lens and workspace may be empty)
  if (!kv_lens) return fail(SSM_EINVAL, "kv_lens: NULL");
  int kcap, vcap;
  int64_t krows, vrows, hk, hv;
  if ((rc = check_cache(k_cache, "k_cache", B, d, &kcap, &krows, &hk)) ||
      (rc = check_cache(v_cache, "v_cache", B, d, &vcap, &vrows, &hv)))
    return rc;
  if ((k_cache->page_table == nullptr) != (v_cache->page_table == nullptr))
    return fail(SSM_EINVAL, "k_cache and v_cache must both be paged or both contiguous");
  if (k_cache->pool.dtype != v_cache->pool.dtype) return fail(SSM_EINVAL, "k_cache and v_cache dtypes differ");
  const bool fp8 = k_cache->pool.dtype == SSM_FP8_E4M3;
  if (hk != hv) return fail(SSM_EINVAL, "k/v head counts differ");
  const int64_t Hkv = hk;
  if (Hkv <= 0 || Hq % Hkv != 0) return fail(SSM_EINVAL, "Hq (%lld) must be a positive multiple of Hkv (%lld)",
                                             (long long)Hq, (long long)Hkv);
  if (d != 64 && d != 128) return fail(SSM_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  if (Hq / Hkv > 16) return fail(SSM_EUNSUPPORTED, "query heads per KV head must be <= 16");
  const int tile_k = (opts && opts->tile_k) ? opts->tile_k : 64;
  if (tile_k != 64) return fail(SSM_EUNSUPPORTED, "tile_k %d not supported (64)", tile_k);
  const int P = (opts && opts->num_splits) ? opts->num_splits : 16;
  if (P < 1 || P > 64) return fail(SSM_EUNSUPPORTED, "num_splits %d not supported (1..64)", P);
  const int32_t flags = opts ? opts->decode_flags : 0;
  if (flags & ~SSM_DECODE_SINK_SEED) return fail(SSM_EINVAL, "unknown decode_flags bits 0x%x", (unsigned)flags);
  if (opts && opts->weights != SSM_WEIGHTS_EXP)
    return fail(SSM_EUNSUPPORTED, "the decode takes only exponential weights (weights = 0)");
  float scale;
  if ((rc = resolve_scale(opts, (int)d, &scale))) return rc;
  if (B > 65535 || Hq > 65536 || B * Hkv * P > INT32_MAX) return fail(SSM_EUNSUPPORTED, "problem too large");
  const int kv_cap = kcap < vcap ? kcap : vcap;
  const int64_t max_tiles = k_cache->page_table ? k_cache->max_pages : ((int64_t)kcap + 63) / 64;
  if (skip_stats) {
    const int64_t need = B * Hkv * max_tiles;
    if (skip_stats->tile_state && skip_stats->tile_state_len < need)
      return fail(SSM_EINVAL, "tile_state needs %lld elements", (long long)need);
    if (skip_stats->unit_gap && skip_stats->unit_gap_len < need)
      return fail(SSM_EINVAL, "unit_gap needs %lld elements", (long long)need);
  }
  const size_t ws = ssm_decode_workspace_bytes((int)B, (int)Hq, (int)d, P);
  void* ws_ptr = nullptr;
  if (noalloc) {
    if (ws > ssm::kDecodeScratchBytes)
      return fail(SSM_EWORKSPACE, "this decode needs %zu bytes of workspace; the static scratch of "
                  "ssm_decode_noalloc holds %zu (use ssm_decode with a caller workspace)", ws, ssm::kDecodeScratchBytes);
    const hipError_t e = ssm::decode_scratch(static_cast<hipStream_t>(stream), &ws_ptr);
    if (e == hipErrorInvalidDevice)
      return fail(SSM_EINVAL, "ssm_decode_noalloc: the stream's device must be the current device");
    if (e != hipSuccess) return fail(SSM_EHIP, "device scratch lookup failed: %s", hipGetErrorString(e));
  } else {
    if (!opts || !opts->workspace) return fail(SSM_EWORKSPACE, "decode needs opts->workspace of %zu bytes", ws);
    if (opts->workspace_bytes < ws)
      return fail(SSM_EWORKSPACE, "workspace has %zu bytes, needs %zu", opts->workspace_bytes, ws);
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 256 != 0)
      return fail(SSM_EINVAL, "workspace must be 256-byte aligned");
    ws_ptr = opts->workspace;
  }

  ssm::DecodeArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q->data);
  a.k = k_cache->pool.data;
  a.v = v_cache->pool.data;
  a.kv_lens = kv_lens;
  a.k_pages = k_cache->page_table;
  a.v_pages = v_cache->page_table;
  a.q_sb = q->stride[0]; a.q_sh = q->stride[1];
  a.k_sb = k_cache->pool.stride[0]; a.k_sh = k_cache->pool.stride[1]; a.k_ss = k_cache->pool.stride[2];
  a.v_sb = v_cache->pool.stride[0]; a.v_sh = v_cache->pool.stride[1]; a.v_ss = v_cache->pool.stride[2];
  a.k_max_pages = k_cache->max_pages; a.v_max_pages = v_cache->max_pages;
  a.B = (int)B; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  a.max_tiles = (int)max_tiles;
  a.num_splits = P;
  a.sink_seed = (flags & SSM_DECODE_SINK_SEED) ? 1 : 0;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.v_scale = fp8 ? v_cache->scale : 1.f;
  // logits = scale * k_scale * (q . code): the key scale joins the softmax scale
  const float lscale = fp8 ? scale * k_cache->scale : scale;
  a.scale = lscale;
  a.scale_log2 = lscale * 1.4426950408889634f;
  a.tau_raw = std::isinf(tau) ? tau : tau / lscale;
  char* ws_base = static_cast<char*>(ws_ptr);
  const DecodeWs lay = decode_ws_layout((size_t)B, (size_t)Hq, (size_t)d, (size_t)P);
  a.part_o = reinterpret_cast<float*>(ws_base);
  a.part_lse = reinterpret_cast<float*>(ws_base + lay.lse_off);
  a.order = B <= ssm::kDecSortMax ? reinterpret_cast<int32_t*>(ws_base + lay.order_off) : nullptr;
  a.wg_cnt = reinterpret_cast<uint32_t*>(ws_base + lay.cnt_off);
  a.o = static_cast<uint16_t*>(out->data);
  a.o_sb = out->stride[0]; a.o_sh = out->stride[1];
  if (skip_stats) {
    a.tile_state = skip_stats->tile_state;
    a.unit_gap = skip_stats->unit_gap;
    a.counters = skip_stats->counters;
  }
  return launch_status(ssm::launch_decode_impl(a, (int)d, kv_cap, krows, vrows, static_cast<hipStream_t>(stream)));
}

int ssm_decode(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
               const int32_t* kv_lens, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
               const ssm_opts* opts) {
  return decode_impl(q, k_cache, v_cache, kv_lens, tau, out, skip_stats, stream, opts, false);
}

int ssm_decode_noalloc(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                       const int32_t* kv_lens, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                       const ssm_opts* opts) {
  return decode_impl(q, k_cache, v_cache, kv_lens, tau, out, skip_stats, stream, opts, true);
}

// qk8: q holds e4m3 codes with dequantisation factor q_scale and the caches must be e4m3 (ssm_prefill_paged_fp8qk)
static int prefill_paged_impl(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                              const int32_t* q_start, const int32_t* kv_lens, int32_t batch, int32_t max_q_len,
                              int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                              const ssm_opts* opts, bool qk8, float q_scale) {
  int rc;
  if ((rc = check_tensor(q, "q", 3, qk8 ? SSM_FP8_E4M3 : SSM_BF16)) || (rc = check_tensor(out, "out", 3, SSM_BF16)))
    return rc;
  if (qk8 && !(q_scale > 0.f && std::isfinite(q_scale))) return fail(SSM_EINVAL, "q_scale must be finite and > 0");
  if ((rc = check_tau(tau))) return rc;
  if (batch < 0 || max_q_len < 0) return fail(SSM_EINVAL, "batch and max_q_len must be >= 0");
  if (batch == 0) return SSM_OK;  // nothing to compute (kv_lens and the page tables may be empty)
  if (!q_start || !kv_lens) return fail(SSM_EINVAL, "q_start and kv_lens must be device arrays");
  const int64_t total_q = q->shape[0], Hq = q->shape[1], d = q->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(SSM_EINVAL, "out shape mismatch in dim %d", i);
  if (!k_cache || !v_cache || !k_cache->page_table || !v_cache->page_table)
    return fail(SSM_EINVAL, "k_cache and v_cache must be paged");
  int kcap, vcap;
  int64_t krows, vrows, hk, hv;
  if ((rc = check_cache(k_cache, "k_cache", batch, d, &kcap, &krows, &hk)) ||
      (rc = check_cache(v_cache, "v_cache", batch, d, &vcap, &vrows, &hv)))
    return rc;
  if (k_cache->pool.dtype != v_cache->pool.dtype) return fail(SSM_EINVAL, "k and v caches must share one dtype");
  const bool kv8 = k_cache->pool.dtype == SSM_FP8_E4M3;
  if (qk8 && !kv8) return fail(SSM_EUNSUPPORTED, "8-bit queries need e4m3 caches");
  if (k_cache->max_pages != v_cache->max_pages) return fail(SSM_EINVAL, "k and v page tables differ in length");
  if (hk != hv) return fail(SSM_EINVAL, "k/v head counts differ");
  const int64_t Hkv = hk;
  if (Hkv <= 0 || Hq % Hkv != 0) return fail(SSM_EINVAL, "Hq (%lld) must be a positive multiple of Hkv (%lld)",
                                             (long long)Hq, (long long)Hkv);
  if (d != 64 && d != 128) return fail(SSM_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)d);
  const int tile_q = (opts && opts->tile_q) ? opts->tile_q : 128;
  const int tile_k = (opts && opts->tile_k) ? opts->tile_k : 64;
  if (tile_q != 64 && tile_q != 128) return fail(SSM_EUNSUPPORTED, "tile_q %d not supported (64 or 128)", tile_q);
  if (tile_k != 64) return fail(SSM_EUNSUPPORTED, "tile_k %d not supported (64)", tile_k);
  float scale;
  if ((rc = resolve_scale(opts, (int)d, &scale))) return rc;
  if (opts && opts->weights != SSM_WEIGHTS_EXP)
    return fail(SSM_EUNSUPPORTED, "the chunked prefill takes only exponential weights (weights = 0)");
  if (total_q > INT32_MAX || max_q_len > (1 << 30) || Hq > 65536) return fail(SSM_EUNSUPPORTED, "problem too large");
  const int64_t nqt = ((int64_t)max_q_len + tile_q - 1) / tile_q, nkt = k_cache->max_pages;
  const int64_t units = (int64_t)batch * Hq * nqt;
  if (units > INT32_MAX) return fail(SSM_EUNSUPPORTED, "too many query tiles");
  if (((int64_t)max_q_len + 128) * q->stride[0] * (qk8 ? 1 : 2) + d * 2 > (int64_t)UINT32_MAX)
    return fail(SSM_EUNSUPPORTED, "max_q_len too long for 32-bit slice offsets");
  if (skip_stats) {
    if (skip_stats->tile_state && skip_stats->tile_state_len < units * nkt)
      return fail(SSM_EINVAL, "tile_state needs %lld elements", (long long)(units * nkt));
    if (skip_stats->unit_gap && skip_stats->unit_gap_len < units * nkt)
      return fail(SSM_EINVAL, "unit_gap needs %lld elements", (long long)(units * nkt));
  }
  if (batch == 0 || max_q_len == 0 || Hq == 0) return SSM_OK;

  ssm::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q->data);
  a.k = static_cast<const uint16_t*>(k_cache->pool.data);
  a.v = static_cast<const uint16_t*>(v_cache->pool.data);
  a.o = static_cast<uint16_t*>(out->data);
  a.q_ss = q->stride[0]; a.q_sh = q->stride[1];
  a.o_ss = out->stride[0]; a.o_sh = out->stride[1];
  a.k_sb = k_cache->pool.stride[0]; a.k_sh = k_cache->pool.stride[1]; a.k_ss = k_cache->pool.stride[2];
  a.v_sb = v_cache->pool.stride[0]; a.v_sh = v_cache->pool.stride[1]; a.v_ss = v_cache->pool.stride[2];
  a.B = batch; a.S = max_q_len; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.G = (int)(Hq / Hkv);
  a.nqt = (int)nqt; a.nkt = (int)nkt;
  a.causal = causal != 0;
  // an fp8 cache: the key scale joins the logit scale, the value scale the output
  // same product order as ssm_prefill_fp8qk, so equal codes and scales give equal scores and decisions
  const float lscale = qk8 ? scale * q_scale * k_cache->scale : (kv8 ? scale * k_cache->scale : scale);
  if (!(lscale > 0.f) || !std::isfinite(lscale)) return fail(SSM_EINVAL, "scale * q_scale * k_scale out of range");
  a.scale = lscale;
  a.scale_log2 = lscale * 1.4426950408889634f;
  a.tau_raw = std::isinf(tau) ? tau : tau / lscale;
  a.v_scale = kv8 ? v_cache->scale : 1.f;
  if (skip_stats) {
    a.tile_state = skip_stats->tile_state;
    a.unit_gap = skip_stats->unit_gap;
    a.counters = skip_stats->counters;
  }
  a.q_start = q_start;
  a.kv_lens = kv_lens;
  a.k_pages = k_cache->page_table;
  a.v_pages = v_cache->page_table;
  a.max_pages = k_cache->max_pages;
  a.total_q = (int)total_q;
  a.k_pool_pages = krows;
  a.v_pool_pages = vrows;
  return launch_status(
      ssm::launch_prefill(a, (int)d, tile_q, true, qk8 ? 3 : (kv8 ? 2 : 0), static_cast<hipStream_t>(stream)));
}

int ssm_prefill_paged(const ssm_tensor* q, const ssm_kv_cache* k_cache, const ssm_kv_cache* v_cache,
                      const int32_t* q_start, const int32_t* kv_lens, int32_t batch, int32_t max_q_len,
                      int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats, void* stream,
                      const ssm_opts* opts) {
  return prefill_paged_impl(q, k_cache, v_cache, q_start, kv_lens, batch, max_q_len, causal, tau, out, skip_stats,
                            stream, opts, false, 1.f);
}

int ssm_prefill_paged_fp8qk(const ssm_tensor* q, float q_scale, const ssm_kv_cache* k_cache,
                            const ssm_kv_cache* v_cache, const int32_t* q_start, const int32_t* kv_lens, int32_t batch,
                            int32_t max_q_len, int32_t causal, float tau, ssm_tensor* out, ssm_skip_stats* skip_stats,
                            void* stream, const ssm_opts* opts) {
  return prefill_paged_impl(q, k_cache, v_cache, q_start, kv_lens, batch, max_q_len, causal, tau, out, skip_stats,
                            stream, opts, true, q_scale);
}

}  // extern "C"
