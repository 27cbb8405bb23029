// C ABI of the ParisKV decode path (include/pariskv.h): argument validation,
// context scratch, launch plans and per-kernel event timing.
#include "pariskv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "pk_kernels.hpp"
#include "pk_tables.hpp"


struct pk_context {
  pk_config cfg;
  int group = 1, units = 0, qheads = 0;
  int device = 0;
  pk::Tables tb;
  pk::TierSpec tiers;
  int64_t max_tiles = 0;          // collide / select workgroups per unit at most
  int64_t max_subs = 0;           // 4 sub-tiles (one per wave) per tile
  // scratch (device)
  uint32_t* lut = nullptr;        // [units][16][256]
  float* rq = nullptr;            // [qheads][128]
  uint32_t* scores = nullptr;     // [units][n_cap]
  uint32_t* tile_hist = nullptr;  // per unit [4 heads][bins + 1][max_subs] sub-tile suffix counts (64 or 128 bins)
  int32_t* cand_idx = nullptr;    // [qheads][C]
  float* cand_est = nullptr;      // [qheads][C]
  uint32_t* unit_tot = nullptr;   // [units][4][bins] bin totals of the collision scores
  uint32_t* dev_err = nullptr;    // device error flags (PK_DEVICE_ERR_*)
  std::string err;
  // timing
  int timing_cap = 0;
  std::vector<hipEvent_t> ev[PK_N_KERNELS];
  int ev_used[PK_N_KERNELS] = {0};
};

namespace {

// encode launch arguments for rows [row0, row0 + t) of every unit
template <typename KT>
pk::EncodeArgs<KT> encode_args(const pk_config& cfg, const void* keys, const int64_t* st, int64_t t,
                                      int64_t row0, const pk_summaries* s) {
  return pk::EncodeArgs<KT>{(const KT*)keys, st[0], st[1], st[2], cfg.n_kv_heads, t,
                            (int)((t + pk::ENC_KEYS - 1) / pk::ENC_KEYS), row0, s->n_capacity,
                            s->codes, s->records, s->norms, s->counts};
}


thread_local std::string g_err;

pk_status fail(pk_context* ctx, pk_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  if (ctx) ctx->err = buf;
  return st;
}

#define PK_HIP(ctx, call)                                                                 \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess)                                                                 \
      return fail((ctx), PK_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Keys per collide / select workgroup: about kTargetWG workgroups over all
// units, 256 threads each doing 1..kMaxKPL keys.
constexpr int64_t kTargetWG = 512, kMaxKPL = 64;
constexpr int64_t kFuseTile = 4096;
// select runs one workgroup per sub-tile from this many 64-key rows per wave
// (sub-tiles of >= 4 * 64 * kSelectSubMinRows keys) on
constexpr int kSelectSubMinRows = 4;
// rerank and top-k run as one workgroup per head while its rounds of 1024
// candidates are few: up to four when there are enough heads to fill the chip
// (at 256 heads, fused wins at 4096 candidates and the split kernels at 13108),
// one otherwise (at 32 heads the split kernels win from 2048 on)
constexpr int kFusedTopkHeads = 128;
constexpr int kFusedTopkSlotsMany = 4 * pk::RT_THREADS;
constexpr int kFusedTopkSlots = pk::RT_THREADS;
// README "Parameters": candidate / collision ratio (per mille) by retrieval-zone length
void adaptive_permille(int64_t zone, int* beta, int* rho) {
  if (zone < 5000) { *beta = 500; *rho = 500; }
  else if (zone < 10000) { *beta = 250; *rho = 300; }
  else if (zone < 30000) { *beta = 200; *rho = 250; }
  else { *beta = 100; *rho = 200; }
}

// ceil(permille / 1000 * n), exact
int64_t ceil_permille(int permille, int64_t n) { return ((int64_t)permille * n + 999) / 1000; }

int tile_size(int units, int64_t n) {
  const int64_t want = ((int64_t)units * n + kTargetWG * 256 - 1) / (kTargetWG * 256);
  const int64_t kpl = want < 1 ? 1 : (want > kMaxKPL ? kMaxKPL : want);
  return (int)(256 * kpl);
}
// Upper bound of ceil(n / tile_size(units, n)) over 0 < n <= n_cap: the tile
// holds >= 256 keys, >= units * n / kTargetWG keys, or is at its maximum.
int64_t max_tiles_for(int units, int64_t n_cap) {
  const int64_t by_min = (n_cap + 255) / 256;
  const int64_t by_target = (kTargetWG + units - 1) / units;
  const int64_t by_max = (n_cap + 256 * kMaxKPL - 1) / (256 * kMaxKPL);
  const int64_t m = by_target > by_max ? by_target : by_max;
  return (by_min < m ? by_min : m) + 2;
}

// HIP events around one launch when the context is timing (ctx may be NULL)
struct Launch {
  pk_context* ctx;
  int kid;
  hipStream_t s;
  Launch(pk_context* c, int k, hipStream_t st) : ctx(c), kid(k), s(st) {
    if (ctx && ctx->timing_cap && ctx->ev_used[kid] < ctx->timing_cap)
      (void)hipEventRecord(ctx->ev[kid][2 * ctx->ev_used[kid]], s);
  }
  ~Launch() {
    if (ctx && ctx->timing_cap && ctx->ev_used[kid] < ctx->timing_cap) {
      (void)hipEventRecord(ctx->ev[kid][2 * ctx->ev_used[kid] + 1], s);
      ctx->ev_used[kid]++;
    }
  }
};

pk_status check_launch(pk_context* ctx, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ctx, PK_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PK_OK;
}

void free_scratch(pk_context* c) {
  void* ptrs[] = {c->lut, c->rq, c->scores, c->tile_hist, c->cand_idx, c->cand_est, c->unit_tot, c->dev_err};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  for (int k = 0; k < PK_N_KERNELS; ++k) {
    for (hipEvent_t e : c->ev[k]) (void)hipEventDestroy(e);
    c->ev[k].clear();
  }
}

pk_status check_strides(pk_context* ctx, const void* base, pk_dtype dt, const int64_t* st,
                        const char* what) {
  if (!base) return fail(ctx, PK_ERR_INVALID_ARG, "%s pointer is NULL", what);
  if (!st) return fail(ctx, PK_ERR_INVALID_ARG, "%s strides are NULL", what);
  const int64_t vec = (dt == PK_BF16) ? 8 : 4;   // elements per 16 bytes
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] % vec != 0)
      return fail(ctx, PK_ERR_INVALID_ARG, "%s stride %d (%lld) must be a non-negative multiple of %lld elements",
                  what, i, (long long)st[i], (long long)vec);
  if (st[2] < PK_HEAD_DIM)
    return fail(ctx, PK_ERR_INVALID_ARG, "%s token stride %lld < 128", what, (long long)st[2]);
  if (!aligned(base, 16)) return fail(ctx, PK_ERR_INVALID_ARG, "%s must be 16-byte aligned", what);
  return PK_OK;
}

}  // namespace

// ===========================================================================
extern "C" {

const char* pk_status_str(pk_status s) {
  switch (s) {
    case PK_OK: return "PK_OK";
    case PK_ERR_INVALID_ARG: return "PK_ERR_INVALID_ARG";
    case PK_ERR_UNSUPPORTED: return "PK_ERR_UNSUPPORTED";
    case PK_ERR_CAPACITY: return "PK_ERR_CAPACITY";
    case PK_ERR_OUT_OF_MEMORY: return "PK_ERR_OUT_OF_MEMORY";
    case PK_ERR_HIP: return "PK_ERR_HIP";
    default: break;
  }
  return "PK_ERR_UNKNOWN";
}

const char* pk_last_error(const pk_context* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

pk_status pk_validate_config(const pk_config* c) {
  if (!c) return fail(nullptr, PK_ERR_INVALID_ARG, "config is NULL");
  if (c->head_dim != PK_HEAD_DIM || c->n_sub != PK_N_SUB || c->sub_dim != PK_SUB_DIM)
    return fail(nullptr, PK_ERR_UNSUPPORTED, "geometry must be head_dim 128, n_sub 16, sub_dim 8 (got %d, %d, %d)",
                c->head_dim, c->n_sub, c->sub_dim);
  if (c->tier_mode != PK_TIERS_RANK && c->tier_mode != PK_TIERS_PERCENTILE)
    return fail(nullptr, PK_ERR_INVALID_ARG, "tier_mode must be PK_TIERS_RANK or PK_TIERS_PERCENTILE (got %d)",
                c->tier_mode);
  if (c->tier_mode == PK_TIERS_RANK) {
    if (c->n_tiers < 1 || c->n_tiers > 4)
      return fail(nullptr, PK_ERR_INVALID_ARG, "n_tiers must be 1..4 (got %d)", c->n_tiers);
    int maxw = 0;
    for (int t = 0; t < c->n_tiers; ++t) {
      const int top = c->tier_top[t], prev = t ? c->tier_top[t - 1] : 0;
      if (top <= prev || top > 256)
        return fail(nullptr, PK_ERR_INVALID_ARG, "tier_top must increase strictly within 1..256 (tier %d: %d)", t,
                    top);
      if (c->tier_weight[t] < 0 || c->tier_weight[t] > 255)
        return fail(nullptr, PK_ERR_INVALID_ARG, "tier_weight[%d] = %d out of range", t, c->tier_weight[t]);
      if (c->tier_weight[t] > maxw) maxw = c->tier_weight[t];
    }
    if (maxw * PK_N_SUB > 64)
      return fail(nullptr, PK_ERR_UNSUPPORTED, "n_sub * max tier weight must be <= 64 (got %d)", maxw * PK_N_SUB);
  }
  if (c->n_candidates < 1 || c->n_candidates > PK_MAX_CANDIDATES)
    return fail(nullptr, PK_ERR_INVALID_ARG, "n_candidates must be 1..%d (got %d)", PK_MAX_CANDIDATES, c->n_candidates);
  if (c->top_k < 1 || c->top_k > PK_MAX_TOPK || c->top_k > c->n_candidates)
    return fail(nullptr, PK_ERR_INVALID_ARG, "top_k must be 1..min(n_candidates, %d) (got %d)", PK_MAX_TOPK, c->top_k);
  if (!(std::isfinite(c->softmax_scale)))
    return fail(nullptr, PK_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1)
    return fail(nullptr, PK_ERR_INVALID_ARG, "batch, n_kv_heads and n_q_heads must be >= 1");
  if (c->n_q_heads % c->n_kv_heads != 0)
    return fail(nullptr, PK_ERR_INVALID_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_q_heads,
                c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > PK_MAX_GROUP)
    return fail(nullptr, PK_ERR_UNSUPPORTED, "at most %d query heads per KV head (got %d)", PK_MAX_GROUP,
                c->n_q_heads / c->n_kv_heads);
  if (c->n_capacity < 1 || c->n_capacity > 0x7FFFFFFFll)
    return fail(nullptr, PK_ERR_INVALID_ARG, "n_capacity must be 1..2^31-1 (got %lld)", (long long)c->n_capacity);
  if ((int64_t)c->batch * c->n_q_heads > 0x7FFFFFFFll / 2)
    return fail(nullptr, PK_ERR_INVALID_ARG, "too many heads");
  if (c->adaptive_ratios != 0 && c->adaptive_ratios != 1)
    return fail(nullptr, PK_ERR_INVALID_ARG, "adaptive_ratios must be 0 or 1 (got %d)", c->adaptive_ratios);
  if (c->tier_mode == PK_TIERS_PERCENTILE && !c->adaptive_ratios &&
      (c->collision_permille < 1 || c->collision_permille > 1000))
    return fail(nullptr, PK_ERR_INVALID_ARG, "collision_permille must be 1..1000 (got %d)", c->collision_permille);
  return PK_OK;
}

pk_status pk_summary_bytes(const pk_config* cfg, size_t* codes, size_t* records, size_t* norms, size_t* counts) {
  pk_status st = pk_validate_config(cfg);
  if (st != PK_OK) return st;
  const size_t units = (size_t)cfg->batch * cfg->n_kv_heads;
  const size_t rows = units * (size_t)cfg->n_capacity;
  if (codes) *codes = rows * 16;
  if (records) *records = rows * PK_RECORD_BYTES;
  if (norms) *norms = rows * sizeof(float);
  if (counts) *counts = units * 16 * 256 * sizeof(uint32_t);
  return PK_OK;
}

pk_status pk_tables(uint64_t seed, int8_t signs[128], float levels[8], float thresholds[7]) {
  if (!signs || !levels || !thresholds) return fail(nullptr, PK_ERR_INVALID_ARG, "NULL table pointer");
  pk::srht_signs(seed, signs);
  struct Quantiser {
    float L[8], T[7];
    Quantiser() { pk::magnitude_tables(L, T); }
  };
  static const Quantiser q;   // seed-independent; computed once, thread-safe initialisation
  std::memcpy(levels, q.L, sizeof(q.L));
  std::memcpy(thresholds, q.T, sizeof(q.T));
  return PK_OK;
}

}  // extern "C"

// The constant kernel arguments of a configuration (host only).
static void kernel_tables(const pk_config& cfg, pk::Tables* tb, pk::TierSpec* tiers) {
  int8_t signs[128];
  float L[8], T[7];
  pk_tables(cfg.srht_seed, signs, L, T);
  std::memset(tb, 0, sizeof(*tb));
  for (int j = 0; j < 128; ++j)
    if (signs[j] < 0) tb->neg_bits[j >> 5] |= 1u << (j & 31);
  std::memcpy(tb->levels, L, sizeof(L));
  std::memcpy(tb->thresholds, T, sizeof(T));
  tb->inv_sqrt_d = (float)(1.0 / std::sqrt(128.0));
  tiers->n_tiers = cfg.n_tiers;
  for (int t = 0; t < 4; ++t) {
    tiers->top[t] = t < cfg.n_tiers ? cfg.tier_top[t] : 0;
    tiers->weight[t] = t < cfg.n_tiers ? cfg.tier_weight[t] : 0;
  }
}

extern "C" {

pk_status pk_create(const pk_config* cfg, pk_context** out) {
  if (!out) return fail(nullptr, PK_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  pk_status st = pk_validate_config(cfg);
  if (st != PK_OK) return st;
  pk_context* c = new (std::nothrow) pk_context();
  if (!c) return fail(nullptr, PK_ERR_OUT_OF_MEMORY, "host allocation failed");
  c->cfg = *cfg;
  c->group = cfg->n_q_heads / cfg->n_kv_heads;
  c->units = cfg->batch * cfg->n_kv_heads;
  c->qheads = cfg->batch * cfg->n_q_heads;

  kernel_tables(*cfg, &c->tb, &c->tiers);
  c->max_tiles = max_tiles_for(c->units, cfg->n_capacity);
  c->max_subs = 4 * c->max_tiles;

  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    return fail(nullptr, PK_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  }
  struct Alloc { void** p; size_t bytes; };
  const size_t U = c->units, Q = c->qheads, C = cfg->n_candidates, N = cfg->n_capacity, MS = c->max_subs;
  Alloc allocs[] = {
      {(void**)&c->lut, U * 16 * 256 * 4},
      {(void**)&c->rq, Q * 128 * 4},
      {(void**)&c->scores, U * N * 4},
      {(void**)&c->tile_hist, U * MS * pk::MAXG * (pk::NBIN_MAX + 1) * 4},
      {(void**)&c->cand_idx, Q * C * 4},
      {(void**)&c->cand_est, Q * C * 4},
      {(void**)&c->unit_tot, U * pk::MAXG * pk::NBIN_MAX * 4},
      {(void**)&c->dev_err, 4},
  };
  for (Alloc& a : allocs) {
    e = hipMalloc(a.p, a.bytes);
    if (e != hipSuccess) {
      *a.p = nullptr;
      free_scratch(c);
      delete c;
      return fail(nullptr, e == hipErrorOutOfMemory ? PK_ERR_OUT_OF_MEMORY : PK_ERR_HIP,
                  "hipMalloc(%zu) failed: %s", a.bytes, hipGetErrorString(e));
    }
  }
  // LUT bytes of absent query heads stay zero
  if (hipMemset(c->lut, 0, U * 16 * 256 * 4) != hipSuccess || hipMemset(c->dev_err, 0, 4) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess) {
    free_scratch(c);
    delete c;
    return fail(nullptr, PK_ERR_HIP, "scratch initialisation failed");
  }
  *out = c;
  return PK_OK;
}

void pk_destroy(pk_context* ctx) {
  if (!ctx) return;
  free_scratch(ctx);
  delete ctx;
}

// ---------------------------------------------------------------------------
static pk_status encode_rows(pk_context* ctx, const void* keys, pk_dtype dt, const int64_t* st,
                             int64_t t, int64_t row0, pk_summaries* s, hipStream_t stream) {
  if (t == 0) return PK_OK;
  const int64_t chunks = (t + pk::ENC_KEYS - 1) / pk::ENC_KEYS;   // t <= n_capacity < 2^31
  const int64_t blocks = (int64_t)ctx->units * chunks;
  Launch L(ctx, PK_KERNEL_ENCODE, stream);
  if (dt == PK_BF16)
    hipLaunchKernelGGL(pk::encode_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       encode_args<uint16_t>(ctx->cfg, keys, st, t, row0, s), ctx->tb);
  else
    hipLaunchKernelGGL(pk::encode_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       encode_args<float>(ctx->cfg, keys, st, t, row0, s), ctx->tb);
  return check_launch(ctx, "encode");
}

static pk_status fill_words(pk_context* ctx, uint32_t* p, uint32_t value, int64_t count, hipStream_t stream) {
  if (count <= 0) return PK_OK;
  hipLaunchKernelGGL(pk::fill_u32_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, p, value,
                     count);
  return check_launch(ctx, "fill");
}

static pk_status check_summaries(pk_context* ctx, const pk_config& cfg, const pk_summaries* s) {
  if (!s) return fail(ctx, PK_ERR_INVALID_ARG, "summaries pointer is NULL");
  if (!s->codes || !s->records || !s->norms) return fail(ctx, PK_ERR_INVALID_ARG, "summary array is NULL");
  if (!aligned(s->codes, 16) || !aligned(s->records, 128) || !aligned(s->norms, 4))
    return fail(ctx, PK_ERR_INVALID_ARG, "codes must be 16-byte and records 128-byte aligned");
  if (s->n_capacity != cfg.n_capacity)
    return fail(ctx, PK_ERR_INVALID_ARG, "summaries n_capacity (%lld) differs from the context's (%lld)",
                (long long)s->n_capacity, (long long)cfg.n_capacity);
  if (s->n < 0 || s->n > s->n_capacity)
    return fail(ctx, PK_ERR_INVALID_ARG, "summaries n (%lld) outside 0..n_capacity", (long long)s->n);
  if (s->counts && !aligned(s->counts, 4)) return fail(ctx, PK_ERR_INVALID_ARG, "counts must be 4-byte aligned");
  if (cfg.tier_mode == PK_TIERS_PERCENTILE && !s->counts)
    return fail(ctx, PK_ERR_INVALID_ARG, "percentile tiers need the summaries' centroid counts");
  return PK_OK;
}

pk_status pk_encode_keys(pk_context* ctx, const void* keys, pk_dtype dt, const int64_t key_strides[3],
                         int64_t n, pk_summaries* inout, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  if (dt != PK_F32 && dt != PK_BF16) return fail(ctx, PK_ERR_UNSUPPORTED, "key dtype %d", (int)dt);
  pk_status st = check_summaries(ctx, ctx->cfg, inout);
  if (st != PK_OK) return st;
  if (n < 0) return fail(ctx, PK_ERR_INVALID_ARG, "n < 0");
  if (n > inout->n_capacity)
    return fail(ctx, PK_ERR_CAPACITY, "n (%lld) exceeds n_capacity (%lld)", (long long)n, (long long)inout->n_capacity);
  if (n > 0 && (st = check_strides(ctx, keys, dt, key_strides, "keys")) != PK_OK) return st;
  if (inout->counts &&
      (st = fill_words(ctx, inout->counts, 0u, (int64_t)ctx->units * 16 * 256, (hipStream_t)hip_stream)) != PK_OK)
    return st;
  st = encode_rows(ctx, keys, dt, key_strides, n, 0, inout, (hipStream_t)hip_stream);
  if (st == PK_OK) inout->n = n;
  return st;
}

pk_status pk_append_keys(pk_context* ctx, const void* keys, pk_dtype dt, const int64_t key_strides[3],
                         int64_t t, pk_summaries* inout, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  if (dt != PK_F32 && dt != PK_BF16) return fail(ctx, PK_ERR_UNSUPPORTED, "key dtype %d", (int)dt);
  pk_status st = check_summaries(ctx, ctx->cfg, inout);
  if (st != PK_OK) return st;
  if (t < 0) return fail(ctx, PK_ERR_INVALID_ARG, "t < 0");
  if (inout->n + t > inout->n_capacity)
    return fail(ctx, PK_ERR_CAPACITY, "n + t (%lld) exceeds n_capacity (%lld)", (long long)(inout->n + t),
                (long long)inout->n_capacity);
  if (t > 0 && (st = check_strides(ctx, keys, dt, key_strides, "new_keys")) != PK_OK) return st;
  st = encode_rows(ctx, keys, dt, key_strides, t, inout->n, inout, (hipStream_t)hip_stream);
  if (st == PK_OK) inout->n += t;
  return st;
}

}  // extern "C"

namespace {

pk_status check_retrieve_args(pk_context* ctx, const pk_config& cfg, const void* q, pk_dtype q_dtype,
                              const pk_summaries* s, const int32_t* topk_idx, const float* topk_est) {
  pk_status st = check_summaries(ctx, cfg, s);
  if (st != PK_OK) return st;
  if (!q || !topk_idx) return fail(ctx, PK_ERR_INVALID_ARG, "q and topk_idx must be non-NULL");
  if (q_dtype != PK_F32 && q_dtype != PK_BF16) return fail(ctx, PK_ERR_UNSUPPORTED, "q dtype %d", (int)q_dtype);
  if (!aligned(q, 16) || !aligned(topk_idx, 4) || (topk_est && !aligned(topk_est, 4)))
    return fail(ctx, PK_ERR_INVALID_ARG, "q must be 16-byte aligned, topk_idx / topk_est 4-byte aligned");
  return PK_OK;
}

pk_status check_attend_args(pk_context* ctx, const void* q, pk_dtype q_dtype, const void* k, const void* v,
                            pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows, const int32_t* topk_idx,
                            const void* out, pk_dtype out_dtype) {
  if (!q || !topk_idx || !out) return fail(ctx, PK_ERR_INVALID_ARG, "q, topk_idx and out must be non-NULL");
  for (pk_dtype d : {q_dtype, kv_dtype, out_dtype})
    if (d != PK_F32 && d != PK_BF16) return fail(ctx, PK_ERR_UNSUPPORTED, "dtype %d", (int)d);
  pk_status st = check_strides(ctx, k, kv_dtype, kv_strides, "k");
  if (st != PK_OK) return st;
  if ((st = check_strides(ctx, v, kv_dtype, kv_strides, "v")) != PK_OK) return st;
  if (n_rows < 0) return fail(ctx, PK_ERR_INVALID_ARG, "n_rows < 0");
  if (!aligned(q, 16) || !aligned(out, 4) || !aligned(topk_idx, 4))
    return fail(ctx, PK_ERR_INVALID_ARG, "q must be 16-byte aligned, out / topk_idx 4-byte aligned");
  return PK_OK;
}

// The retrieval chain.  With `att` (q, K/V and output of one dtype) the kernel
// that selects each head's Top-k (rerank + top-k, or top-k after the spread
// rerank) also computes the attention and *attended is set; otherwise the
// caller still has to attend.
// Sizes of one retrieval over n > 0 keys per unit: candidates C and, with
// percentile tiers, the kept positions M (Slides Sec. 4.2.2: C = ceil(beta n);
// README "Parameters": adaptive ratios), and the collide / select tiling.
struct CallShape {
  int C = 0, n_sel = 0, tile = 0, tiles = 0;
  uint32_t keep_m = 0;
  bool pct = false;
};

pk_status call_shape(pk_context* ctx, const pk_config& cfg, int units, int64_t n, CallShape* cs) {
  int64_t C64 = cfg.n_candidates;
  if (cfg.adaptive_ratios) {
    int beta = 0, rho = 0;
    adaptive_permille(n, &beta, &rho);
    C64 = ceil_permille(beta, n);
    if (cfg.tier_mode == PK_TIERS_PERCENTILE) cs->keep_m = (uint32_t)ceil_permille(rho, n);
  } else if (cfg.tier_mode == PK_TIERS_PERCENTILE) {
    cs->keep_m = (uint32_t)ceil_permille(cfg.collision_permille, n);
  }
  if (C64 > cfg.n_candidates)
    return fail(ctx, PK_ERR_CAPACITY, "adaptive candidate count %lld exceeds n_candidates %d", (long long)C64,
                cfg.n_candidates);
  cs->C = (int)C64;
  cs->n_sel = (int)(n < C64 ? n : C64);
  cs->pct = cfg.tier_mode == PK_TIERS_PERCENTILE;
  // rank tiers: tiles of up to kFuseTile keys when a unit has few keys
  // (at most 16 tiles), fewer sub-tiles for the selection parameters to sum
  int tile = tile_size(units, n);
  if (!cs->pct) {
    const int64_t want = ((n + 15) / 16 + 255) / 256 * 256;
    if (want > tile && want <= kFuseTile) tile = (int)want;
  }
  cs->tile = tile;
  cs->tiles = (int)((n + tile - 1) / tile);
  return PK_OK;
}

// What a retrieval runs on: the configuration, constant tables, scratch
// arrays, and the context (nullable: it only receives timings and error text).
struct Scratch {
  uint32_t* lut = nullptr;        // [units][16][256]
  float* rq = nullptr;            // [qheads][128]
  uint32_t* scores = nullptr;     // [units][score_stride]
  int64_t score_stride = 0;
  uint32_t* tile_hist = nullptr;  // per unit: sub-tile suffix counts
  int64_t max_subs = 0;
  uint32_t* unit_tot = nullptr;   // [units][4][bins]
  int32_t* cand_idx = nullptr;    // [qheads][C]
  float* cand_est = nullptr;      // [qheads][C]
  uint32_t* dev_err = nullptr;    // nullable
};

// Rows of one decode step that the retrieval's first launch also encodes
// (pk_append_retrieve_attend): rank tiers, 1..ENC_DIRECT rows per unit,
// written at row0 of the summaries.
struct PendingAppend {
  const void* keys;
  pk_dtype dt;
  const int64_t* strides;
  int64_t t, row0;
};

struct Plan {
  const pk_config* cfg;
  int group, units, qheads;
  pk::Tables tb;
  pk::TierSpec tiers;
  pk_context* ctx;
};

Plan context_plan(pk_context* ctx) {
  return Plan{&ctx->cfg, ctx->group, ctx->units, ctx->qheads, ctx->tb, ctx->tiers, ctx};
}

// Outputs of a retrieval over no keys: every Top-k slot (and candidate slot
// of the debug copies) -1 / -inf.
pk_status retrieve_empty(const Plan& pl, int32_t* topk_idx, float* topk_est, const pk_debug* dbg,
                         hipStream_t stream) {
  const int64_t cnt = (int64_t)pl.qheads * pl.cfg->top_k;
  hipLaunchKernelGGL(pk::fill_empty_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream, topk_idx,
                     topk_est, cnt);
  pk_status st = check_launch(pl.ctx, "fill");
  if (st != PK_OK) return st;
  if (dbg && dbg->cand_idx) {
    const int64_t cc = (int64_t)pl.qheads * pl.cfg->n_candidates;
    hipLaunchKernelGGL(pk::fill_empty_kernel, dim3((unsigned)((cc + 255) / 256)), dim3(256), 0, stream,
                       dbg->cand_idx, dbg->cand_est, cc);
    st = check_launch(pl.ctx, "fill");
  }
  return st;
}

Scratch context_scratch(pk_context* ctx) {
  Scratch sc;
  sc.lut = ctx->lut;
  sc.rq = ctx->rq;
  sc.scores = ctx->scores;
  sc.score_stride = ctx->cfg.n_capacity;
  sc.tile_hist = ctx->tile_hist;
  sc.max_subs = ctx->max_subs;
  sc.cand_idx = ctx->cand_idx;
  sc.cand_est = ctx->cand_est;
  sc.unit_tot = ctx->unit_tot;
  sc.dev_err = ctx->dev_err;
  return sc;
}

// The retrieval chain.  With `att` (q, K/V and output of one dtype) the kernel
// that selects each head's Top-k (rerank + top-k, or top-k after the spread
// rerank) also computes the attention and *attended is set; otherwise the
// caller still has to attend.  n > 0; `cs` is call_shape's result for n, and
// the scratch holds max_subs >= 4 * cs.tiles.
pk_status retrieve_impl(const Plan& pl, const Scratch& sc, const CallShape& cs, const void* q, pk_dtype q_dtype,
                        const pk_summaries* s, int32_t* topk_idx, float* topk_est, const pk_debug* dbg,
                        hipStream_t stream, const pk::AttendArgs* att, bool* attended,
                        const PendingAppend* app = nullptr) {
  pk_status st = PK_OK;
  if (attended) *attended = false;
  pk_context* ctx = pl.ctx;
  const pk_config& cfg = *pl.cfg;
  const int64_t n = s->n;
  const int k = cfg.top_k, C_cap = cfg.n_candidates;
  const int C = cs.C, tile = cs.tile, tiles = cs.tiles, n_sel = cs.n_sel;
  const uint32_t keep_m = cs.keep_m;
  const bool pct = cs.pct;
  const unsigned grid = (unsigned)((int64_t)pl.units * tiles);

  {
    Launch L(ctx, PK_KERNEL_QPREP, stream);
    const int qblocks = pl.qheads * pk::QP_PARTS;
#define PK_QA(QT)                                                                                             \
  pk::QprepArgs<QT>{(const QT*)q, cfg.n_q_heads, cfg.n_kv_heads, pl.group, sc.rq, (uint8_t*)sc.lut, s->counts, \
                    keep_m, sc.unit_tot}
    if (app) {
      // the step's appended rows are encoded by extra workgroups of the same
      // launch (one per unit: t <= ENC_DIRECT)
      const unsigned blocks = (unsigned)(qblocks + pl.units);
#define PK_AQ(QT, KT)                                                                                         \
  hipLaunchKernelGGL((pk::append_qprep_kernel<QT, KT>), dim3(blocks), dim3(64 * pk::QP_WAVES), 0, stream,    \
                     PK_QA(QT), encode_args<KT>(cfg, app->keys, app->strides, app->t, app->row0, s), pl.tb,  \
                     pl.tiers, qblocks)
      if (q_dtype == PK_BF16 && app->dt == PK_BF16) PK_AQ(uint16_t, uint16_t);
      else if (q_dtype == PK_BF16) PK_AQ(uint16_t, float);
      else if (app->dt == PK_BF16) PK_AQ(float, uint16_t);
      else PK_AQ(float, float);
#undef PK_AQ
    } else if (q_dtype == PK_BF16) {
      hipLaunchKernelGGL(pk::qprep_kernel<uint16_t>, dim3(qblocks), dim3(64 * pk::QP_WAVES), 0, stream,
                         PK_QA(uint16_t), pl.tb, pl.tiers);
    } else {
      hipLaunchKernelGGL(pk::qprep_kernel<float>, dim3(qblocks), dim3(64 * pk::QP_WAVES), 0, stream,
                         PK_QA(float), pl.tb, pl.tiers);
    }
#undef PK_QA
  }
  if ((st = check_launch(ctx, "qprep")) != PK_OK) return st;
  {
    Launch L(ctx, PK_KERNEL_COLLIDE, stream);
#define PK_COLLIDE(GG, NB)                                                                                    \
  hipLaunchKernelGGL((pk::collide_kernel<GG, NB>), dim3(grid), dim3(256), 0, stream, (const uint4*)s->codes,      \
                     sc.lut, sc.scores, sc.tile_hist, sc.unit_tot, n, s->n_capacity, sc.score_stride, tiles,      \
                     (int)sc.max_subs, tile)
#define PK_COLLIDE_G(NB)                   \
  switch (pl.group) {                    \
    case 1: PK_COLLIDE(1, NB); break;      \
    case 2: PK_COLLIDE(2, NB); break;      \
    case 3: PK_COLLIDE(3, NB); break;      \
    default: PK_COLLIDE(4, NB); break;     \
  }
    if (pct) {
      PK_COLLIDE_G(pk::NBIN_MAX);
    } else {
      PK_COLLIDE_G(pk::NBIN);
    }
#undef PK_COLLIDE_G
#undef PK_COLLIDE
  }
  if ((st = check_launch(ctx, "collide")) != PK_OK) return st;
  {
    // every select workgroup derives theta and its prefix counts itself from
    // the unit's bin totals and the sub-tiles' suffix counts
    Launch L(ctx, PK_KERNEL_SELECT, stream);
#define PK_SELECT(GG, NB)                                                                                      \
  hipLaunchKernelGGL((pk::select_kernel<GG, NB>), dim3(grid), dim3(256), 0, stream, sc.scores, sc.cand_idx, n, \
                     sc.score_stride, tiles, (int)sc.max_subs, tile, cfg.n_q_heads, cfg.n_kv_heads, C,        \
                     sc.unit_tot, sc.tile_hist, sc.dev_err)
#define PK_SELECT_G(NB)                    \
  switch (pl.group) {                    \
    case 1: PK_SELECT(1, NB); break;       \
    case 2: PK_SELECT(2, NB); break;       \
    case 3: PK_SELECT(3, NB); break;       \
    default: PK_SELECT(4, NB); break;      \
  }
    // one workgroup per sub-tile once a sub-tile is long enough to split
    // over the four waves (more resident waves hide the score loads)
    const int rpw = (tile / 256 + 3) / 4;         // 64-key rows per wave
    if (rpw >= kSelectSubMinRows) {
      const int subs = 4 * tiles;
      const unsigned sgrid = (unsigned)((int64_t)pl.units * subs);
#define PK_SELSUB(GG, NB, RW)                                                                                    \
  hipLaunchKernelGGL((pk::select_sub_kernel<GG, NB, RW>), dim3(sgrid), dim3(256), 0, stream, sc.scores,        \
                     sc.cand_idx, n, sc.score_stride, subs, (int)sc.max_subs, tile / 4, cfg.n_q_heads,       \
                     cfg.n_kv_heads, C, sc.unit_tot, sc.tile_hist, sc.dev_err)
#define PK_SELSUB_R(GG, NB)                  \
  do {                                       \
    if (rpw <= 4) PK_SELSUB(GG, NB, 4);      \
    else if (rpw <= 8) PK_SELSUB(GG, NB, 8); \
    else PK_SELSUB(GG, NB, 16);              \
  } while (0)
#define PK_SELSUB_G(NB)                       \
  switch (pl.group) {                       \
    case 1: PK_SELSUB_R(1, NB); break;        \
    case 2: PK_SELSUB_R(2, NB); break;        \
    case 3: PK_SELSUB_R(3, NB); break;        \
    default: PK_SELSUB_R(4, NB); break;       \
  }
      if (pct) {
        PK_SELSUB_G(pk::NBIN_MAX);
      } else {
        PK_SELSUB_G(pk::NBIN);
      }
#undef PK_SELSUB_G
#undef PK_SELSUB_R
#undef PK_SELSUB
    } else if (pct) {
      PK_SELECT_G(pk::NBIN_MAX);
    } else {
      PK_SELECT_G(pk::NBIN);
    }
#undef PK_SELECT_G
#undef PK_SELECT
  }
  if ((st = check_launch(ctx, "select")) != PK_OK) return st;
  if (n_sel <= (pl.qheads >= kFusedTopkHeads ? kFusedTopkSlotsMany : kFusedTopkSlots)) {
    // one workgroup per head: rerank and top-k together, estimates in LDS
    Launch L(ctx, PK_KERNEL_RERANK_TOPK, stream);
    const int R = (n_sel + pk::RT_THREADS - 1) / pk::RT_THREADS;   // <= 4
    float* est_out = (dbg && dbg->cand_est) ? sc.cand_est : nullptr;
    const pk::AttendArgs none{};
#define PK_RTK_LAUNCH(RR, T, MR, A)                                                                               \
  hipLaunchKernelGGL((pk::rerank_topk_kernel<RR, T, MR, A>), dim3(pl.qheads), dim3(pk::RT_THREADS), 0, stream,   \
                     s->records, sc.rq, sc.cand_idx, est_out, s->n_capacity, n_sel, C, cfg.n_q_heads,           \
                     cfg.n_kv_heads, pl.group, pl.tb, k, topk_idx, topk_est, A ? *att : none)
#define PK_RTK_R(T, MR, A)                         \
  do {                                             \
    if (R <= 1) PK_RTK_LAUNCH(1, T, MR, A);        \
    else if (R <= 2) PK_RTK_LAUNCH(2, T, MR, A);   \
    else PK_RTK_LAUNCH(4, T, MR, A);               \
  } while (0)
    if (att) {
      const int np = k <= 2 * (pk::RT_THREADS / 16) ? 2 : 4;   // passes of 64 rows
      if (q_dtype == PK_BF16 && np == 2) PK_RTK_R(uint16_t, 2, true);
      else if (q_dtype == PK_BF16) PK_RTK_R(uint16_t, 4, true);
      else if (np == 2) PK_RTK_R(float, 2, true);
      else PK_RTK_R(float, 4, true);
      if (attended) *attended = true;
    } else {
      PK_RTK_R(float, 1, false);
    }
#undef PK_RTK_R
#undef PK_RTK_LAUNCH
    if ((st = check_launch(ctx, "rerank_topk")) != PK_OK) return st;
  } else {
    // few heads: spread the rerank over several workgroups per head, then select
    {
      // one candidate per lane while that keeps the grid within ~2048
      // workgroups, else two or four (fewer tables to build)
      Launch L(ctx, PK_KERNEL_RERANK, stream);
      const int64_t total = (int64_t)pl.qheads * n_sel;
      const int rr = total <= (int64_t)1 << 19 ? 1 : (total <= (int64_t)1 << 21 ? 2 : 4);
      const int chunks = (n_sel + 256 * rr - 1) / (256 * rr);
#define PK_RR(RRR)                                                                                               \
  hipLaunchKernelGGL(pk::rerank_kernel<RRR>, dim3((unsigned)((int64_t)pl.qheads * chunks)), dim3(256), 0, stream, \
                     s->records, sc.rq, sc.cand_idx, sc.cand_est, s->n_capacity, n_sel, C, chunks,          \
                     cfg.n_q_heads, cfg.n_kv_heads, pl.group, pl.tb)
      if (rr == 1) PK_RR(1);
      else if (rr == 2) PK_RR(2);
      else PK_RR(4);
#undef PK_RR
    }
    if ((st = check_launch(ctx, "rerank")) != PK_OK) return st;
    {
      // with attention of matching dtypes, the top-k workgroup attends over its
      // head's rows as well (no separate attention launch)
      Launch L(ctx, PK_KERNEL_TOPK, stream);
      const int R = (n_sel + pk::TK_THREADS - 1) / pk::TK_THREADS;
      const pk::AttendArgs none{};
#define PK_TOPK(RR, T, MR, A)                                                                                   \
  hipLaunchKernelGGL((pk::topk_kernel<RR, T, MR, A>), dim3(pl.qheads), dim3(pk::TK_THREADS), 0, stream,        \
                     sc.cand_idx, sc.cand_est, n_sel, C, k, topk_idx, topk_est, cfg.n_q_heads, pl.group,   \
                     A ? *att : none)
#define PK_TOPK_R(T, MR, A)                    \
  do {                                         \
    if (R <= 2) PK_TOPK(2, T, MR, A);          \
    else if (R <= 4) PK_TOPK(4, T, MR, A);     \
    else if (R <= 8) PK_TOPK(8, T, MR, A);     \
    else PK_TOPK(16, T, MR, A);                \
  } while (0)
      if (att) {
        const int np = k <= 2 * (pk::TK_THREADS / 16) ? 2 : 4;   // passes of 64 rows
        if (q_dtype == PK_BF16 && np == 2) PK_TOPK_R(uint16_t, 2, true);
        else if (q_dtype == PK_BF16) PK_TOPK_R(uint16_t, 4, true);
        else if (np == 2) PK_TOPK_R(float, 2, true);
        else PK_TOPK_R(float, 4, true);
        if (attended) *attended = true;
      } else {
        PK_TOPK_R(float, 1, false);
      }
#undef PK_TOPK_R
#undef PK_TOPK
    }
    if ((st = check_launch(ctx, "topk")) != PK_OK) return st;
  }

  if (dbg) {
    const size_t U = pl.units, Q = pl.qheads;
    if (dbg->rot_q) PK_HIP(ctx, hipMemcpyAsync(dbg->rot_q, sc.rq, Q * 128 * 4, hipMemcpyDeviceToDevice, stream));
    if (dbg->lut) PK_HIP(ctx, hipMemcpyAsync(dbg->lut, sc.lut, U * 16 * 256 * 4, hipMemcpyDeviceToDevice, stream));
    if (dbg->scores)
      PK_HIP(ctx, hipMemcpy2DAsync(dbg->scores, (size_t)n * 4, sc.scores, (size_t)sc.score_stride * 4, (size_t)n * 4,
                                   U, hipMemcpyDeviceToDevice, stream));
    // candidate lists are [heads][C] inside, [heads][n_candidates] in the debug copies
    if (C < C_cap && (dbg->cand_idx || dbg->cand_est)) {
      const int64_t cc = (int64_t)Q * C_cap;
      if (dbg->cand_idx) {
        hipLaunchKernelGGL(pk::fill_empty_kernel, dim3((unsigned)((cc + 255) / 256)), dim3(256), 0, stream,
                           dbg->cand_idx, dbg->cand_est, cc);
      } else {
        hipLaunchKernelGGL(pk::fill_empty_kernel, dim3((unsigned)((cc + 255) / 256)), dim3(256), 0, stream,
                           (int32_t*)nullptr, dbg->cand_est, cc);
      }
      if ((st = check_launch(ctx, "fill")) != PK_OK) return st;
    }
    if (dbg->cand_idx)
      PK_HIP(ctx, hipMemcpy2DAsync(dbg->cand_idx, (size_t)C_cap * 4, sc.cand_idx, (size_t)C * 4, (size_t)C * 4, Q,
                                   hipMemcpyDeviceToDevice, stream));
    if (dbg->cand_est)
      PK_HIP(ctx, hipMemcpy2DAsync(dbg->cand_est, (size_t)C_cap * 4, sc.cand_est, (size_t)C * 4, (size_t)C * 4, Q,
                                   hipMemcpyDeviceToDevice, stream));
  }
  return PK_OK;
}

pk_status attend_impl(const Plan& pl, const void* q, pk_dtype q_dtype, const void* k, const void* v,
                      pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows, const int32_t* topk_idx,
                      void* out, pk_dtype out_dtype, hipStream_t stream) {
  pk_context* ctx = pl.ctx;
  const pk_config& c = *pl.cfg;
  const int kk = c.top_k;
  const pk::AttendArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], n_rows, c.softmax_scale, out};
  Launch L(ctx, PK_KERNEL_ATTEND, stream);
#define PK_ATT(KT, QT, OT, R)                                                                                   \
  hipLaunchKernelGGL((pk::attend_kernel<KT, QT, OT, R>), dim3(pl.qheads), dim3(256), 0, stream, a, topk_idx, kk, \
                     c.n_q_heads, c.n_kv_heads, pl.group)
#define PK_ATT_R(KT, QT, OT) \
  do {                       \
    if (kk <= 128)           \
      PK_ATT(KT, QT, OT, 32); \
    else                     \
      PK_ATT(KT, QT, OT, 64); \
  } while (0)
#define PK_ATT_O(KT, QT)                           \
  do {                                             \
    if (out_dtype == PK_BF16)                      \
      PK_ATT_R(KT, QT, uint16_t);                  \
    else                                           \
      PK_ATT_R(KT, QT, float);                     \
  } while (0)
#define PK_ATT_Q(KT)                               \
  do {                                             \
    if (q_dtype == PK_BF16)                        \
      PK_ATT_O(KT, uint16_t);                      \
    else                                           \
      PK_ATT_O(KT, float);                         \
  } while (0)
  if (kv_dtype == PK_BF16)
    PK_ATT_Q(uint16_t);
  else
    PK_ATT_Q(float);
#undef PK_ATT_Q
#undef PK_ATT_O
#undef PK_ATT_R
#undef PK_ATT
  return check_launch(ctx, "attend");
}

// A retrieval with a context's scratch.
pk_status retrieve_ctx(pk_context* ctx, const void* q, pk_dtype q_dtype, const pk_summaries* s, int32_t* topk_idx,
                       float* topk_est, const pk_debug* dbg, hipStream_t stream, const pk::AttendArgs* att,
                       bool* attended, const PendingAppend* app = nullptr) {
  if (attended) *attended = false;
  const Plan pl = context_plan(ctx);
  if (s->n == 0) return retrieve_empty(pl, topk_idx, topk_est, dbg, stream);
  CallShape cs;
  pk_status st = call_shape(ctx, ctx->cfg, ctx->units, s->n, &cs);
  if (st != PK_OK) return st;
  if (cs.tiles > ctx->max_tiles)
    return fail(ctx, PK_ERR_CAPACITY, "internal tiling bound exceeded (%d > %lld)", cs.tiles,
                (long long)ctx->max_tiles);
  return retrieve_impl(pl, context_scratch(ctx), cs, q, q_dtype, s, topk_idx, topk_est, dbg, stream, att, attended,
                       app);
}

}  // namespace

extern "C" {

pk_status pk_retrieve(pk_context* ctx, const void* q, pk_dtype q_dtype, const pk_summaries* s,
                      int32_t* topk_idx, float* topk_est, const pk_debug* dbg, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  pk_status st = check_retrieve_args(ctx, ctx->cfg, q, q_dtype, s, topk_idx, topk_est);
  if (st != PK_OK) return st;
  return retrieve_ctx(ctx, q, q_dtype, s, topk_idx, topk_est, dbg, (hipStream_t)hip_stream, nullptr, nullptr);
}

pk_status pk_sparse_attend(pk_context* ctx, const void* q, pk_dtype q_dtype, const void* k, const void* v,
                           pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows,
                           const int32_t* topk_idx, void* out, pk_dtype out_dtype, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  pk_status st = check_attend_args(ctx, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype);
  if (st != PK_OK) return st;
  return attend_impl(context_plan(ctx), q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype,
                     (hipStream_t)hip_stream);
}

pk_status pk_sparse_dense_attend(pk_context* ctx, const void* q, pk_dtype q_dtype, const void* k, const void* v,
                                 pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows,
                                 const int32_t* topk_idx, const void* dense_k, const void* dense_v,
                                 const int64_t dense_strides[3], int64_t n_dense, void* out, pk_dtype out_dtype,
                                 void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  pk_status st = check_attend_args(ctx, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype);
  if (st != PK_OK) return st;
  if (n_dense < 0 || n_dense > PK_MAX_DENSE)
    return fail(ctx, PK_ERR_INVALID_ARG, "n_dense must be 0..%d (got %lld)", PK_MAX_DENSE, (long long)n_dense);
  if (n_dense > 0) {
    if ((st = check_strides(ctx, dense_k, kv_dtype, dense_strides, "dense_k")) != PK_OK) return st;
    if ((st = check_strides(ctx, dense_v, kv_dtype, dense_strides, "dense_v")) != PK_OK) return st;
  }
  hipStream_t stream = (hipStream_t)hip_stream;
  const pk_config& c = ctx->cfg;
  const int kk = c.top_k;
  const pk::AttendArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], n_rows, c.softmax_scale, out};
  const int64_t ds[3] = {n_dense > 0 ? dense_strides[0] : 0, n_dense > 0 ? dense_strides[1] : 0,
                         n_dense > 0 ? dense_strides[2] : 0};
  Launch L(ctx, PK_KERNEL_DENSE_ATTEND, stream);
#define PK_DA(KT, QT, OT)                                                                                      \
  hipLaunchKernelGGL((pk::dense_sparse_attend_kernel<KT, QT, OT>), dim3(ctx->qheads), dim3(pk::DA_THREADS), 0,  \
                     stream, a, topk_idx, kk, (const KT*)dense_k, (const KT*)dense_v, ds[0], ds[1], ds[2],          \
                     (int)n_dense, c.n_q_heads, c.n_kv_heads, ctx->group)
#define PK_DA_O(KT, QT)                 \
  do {                                  \
    if (out_dtype == PK_BF16)           \
      PK_DA(KT, QT, uint16_t);          \
    else                                \
      PK_DA(KT, QT, float);             \
  } while (0)
#define PK_DA_Q(KT)                     \
  do {                                  \
    if (q_dtype == PK_BF16)             \
      PK_DA_O(KT, uint16_t);            \
    else                                \
      PK_DA_O(KT, float);               \
  } while (0)
  if (kv_dtype == PK_BF16)
    PK_DA_Q(uint16_t);
  else
    PK_DA_Q(float);
#undef PK_DA_Q
#undef PK_DA_O
#undef PK_DA
  return check_launch(ctx, "dense_attend");
}

pk_status pk_retrieve_attend(pk_context* ctx, const void* q, pk_dtype q_dtype, const pk_summaries* s,
                             const void* k, const void* v, pk_dtype kv_dtype, const int64_t kv_strides[3],
                             int64_t n_rows, int32_t* topk_idx, float* topk_est, void* out, pk_dtype out_dtype,
                             const pk_debug* dbg, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  pk_status st = check_retrieve_args(ctx, ctx->cfg, q, q_dtype, s, topk_idx, topk_est);
  if (st != PK_OK) return st;
  st = check_attend_args(ctx, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype);
  if (st != PK_OK) return st;
  hipStream_t stream = (hipStream_t)hip_stream;
  const bool same_dtype = q_dtype == kv_dtype && kv_dtype == out_dtype;
  const pk::AttendArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], n_rows, ctx->cfg.softmax_scale, out};
  bool attended = false;
  st = retrieve_ctx(ctx, q, q_dtype, s, topk_idx, topk_est, dbg, stream, same_dtype ? &a : nullptr, &attended);
  if (st != PK_OK || attended) return st;
  return attend_impl(context_plan(ctx), q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype,
                     stream);
}

pk_status pk_append_retrieve_attend(pk_context* ctx, const void* new_keys, pk_dtype key_dtype,
                                    const int64_t key_strides[3], int64_t t, pk_summaries* inout, const void* q,
                                    pk_dtype q_dtype, const void* k, const void* v, pk_dtype kv_dtype,
                                    const int64_t kv_strides[3], int64_t n_rows, int32_t* topk_idx,
                                    float* topk_est, void* out, pk_dtype out_dtype, void* hip_stream) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  if (key_dtype != PK_F32 && key_dtype != PK_BF16)
    return fail(ctx, PK_ERR_UNSUPPORTED, "key dtype %d", (int)key_dtype);
  pk_status st = check_summaries(ctx, ctx->cfg, inout);
  if (st != PK_OK) return st;
  if (t < 0) return fail(ctx, PK_ERR_INVALID_ARG, "t < 0");
  if (inout->n + t > inout->n_capacity)
    return fail(ctx, PK_ERR_CAPACITY, "n + t (%lld) exceeds n_capacity (%lld)", (long long)(inout->n + t),
                (long long)inout->n_capacity);
  if (t > 0 && (st = check_strides(ctx, new_keys, key_dtype, key_strides, "new_keys")) != PK_OK) return st;
  pk_summaries after = *inout;
  after.n += t;
  if ((st = check_retrieve_args(ctx, ctx->cfg, q, q_dtype, &after, topk_idx, topk_est)) != PK_OK) return st;
  if ((st = check_attend_args(ctx, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype)) !=
      PK_OK)
    return st;
  hipStream_t stream = (hipStream_t)hip_stream;
  // rank tiers: qprep reads no centroid counts, so a few new rows per unit are
  // encoded by the first launch of the retrieval; otherwise by their own
  const bool fuse = t > 0 && t <= pk::ENC_DIRECT && ctx->cfg.tier_mode == PK_TIERS_RANK;
  if (t > 0 && !fuse &&
      (st = encode_rows(ctx, new_keys, key_dtype, key_strides, t, inout->n, inout, stream)) != PK_OK)
    return st;
  const PendingAppend app{new_keys, key_dtype, key_strides, t, inout->n};
  const bool same_dtype = q_dtype == kv_dtype && kv_dtype == out_dtype;
  const pk::AttendArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], n_rows, ctx->cfg.softmax_scale, out};
  bool attended = false;
  st = retrieve_ctx(ctx, q, q_dtype, &after, topk_idx, topk_est, nullptr, stream, same_dtype ? &a : nullptr,
                    &attended, fuse ? &app : nullptr);
  if (st == PK_OK && !attended)
    st = attend_impl(context_plan(ctx), q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype,
                     stream);
  if (st == PK_OK) inout->n = after.n;
  return st;
}

}  // extern "C"

// ---- retrieval without a context: scratch in a static device array ----------
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): it uses the per-device
// address from hipGetSymbolAddress, taken once per device on first use.
static __device__ __align__(256) unsigned char scratch[PK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};

pk_status device_scratch(int dev, unsigned char** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(nullptr, PK_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, PK_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return PK_OK;
}

// Carves the arrays of one call out of `base` (256-byte aligned each); with
// base NULL only the total is computed.
size_t carve_scratch(unsigned char* base, const pk_config& cfg, int units, int qheads, int64_t n,
                     const CallShape& cs, Scratch* sc) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    unsigned char* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  const size_t U = units, Q = qheads, MS = 4 * (size_t)cs.tiles, C = cs.C;
  const size_t bins = cs.pct ? pk::NBIN_MAX : pk::NBIN;       // suffix counts s = 1..bins + 1
  sc->lut = reinterpret_cast<uint32_t*>(take(U * 16 * 256 * 4));
  sc->rq = reinterpret_cast<float*>(take(Q * 128 * 4));
  sc->scores = reinterpret_cast<uint32_t*>(take(U * (size_t)n * 4));
  sc->score_stride = n;
  sc->tile_hist = reinterpret_cast<uint32_t*>(take(U * MS * pk::MAXG * (bins + 1) * 4));
  sc->max_subs = (int64_t)MS;
  sc->cand_idx = reinterpret_cast<int32_t*>(take(Q * C * 4));
  sc->cand_est = reinterpret_cast<float*>(take(Q * C * 4));
  sc->unit_tot = reinterpret_cast<uint32_t*>(take(U * pk::MAXG * bins * 4));
  sc->dev_err = nullptr;
  (void)cfg;
  return off;
}

}  // namespace

extern "C" {

pk_status pk_retrieve_attend_noalloc(const pk_config* cfg, const void* q, pk_dtype q_dtype, const pk_summaries* s,
                                     const void* k, const void* v, pk_dtype kv_dtype, const int64_t kv_strides[3],
                                     int64_t n_rows, int32_t* topk_idx, float* topk_est, void* out,
                                     pk_dtype out_dtype, void* hip_stream) {
  pk_status st = pk_validate_config(cfg);
  if (st != PK_OK) return st;
  if ((st = check_retrieve_args(nullptr, *cfg, q, q_dtype, s, topk_idx, topk_est)) != PK_OK) return st;
  if ((st = check_attend_args(nullptr, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype)) !=
      PK_OK)
    return st;
  Plan pl{cfg, cfg->n_q_heads / cfg->n_kv_heads, cfg->batch * cfg->n_kv_heads, cfg->batch * cfg->n_q_heads, {}, {},
          nullptr};
  kernel_tables(*cfg, &pl.tb, &pl.tiers);
  hipStream_t stream = (hipStream_t)hip_stream;
  const pk::AttendArgs a{q, k, v, kv_strides[0], kv_strides[1], kv_strides[2], n_rows, cfg->softmax_scale, out};
  const bool same_dtype = q_dtype == kv_dtype && kv_dtype == out_dtype;
  bool attended = false;
  if (s->n == 0) {
    st = retrieve_empty(pl, topk_idx, topk_est, nullptr, stream);
  } else {
    CallShape cs;
    if ((st = call_shape(nullptr, *cfg, pl.units, s->n, &cs)) != PK_OK) return st;
    Scratch sc;
    const size_t need = carve_scratch(nullptr, *cfg, pl.units, pl.qheads, s->n, cs, &sc);
    if (need > PK_NOALLOC_SCRATCH_BYTES)
      return fail(nullptr, PK_ERR_CAPACITY,
                  "this call needs %zu bytes of scratch; the static scratch of the no-allocation call holds %zu "
                  "(fewer keys, units or candidates per call fit)",
                  need, (size_t)PK_NOALLOC_SCRATCH_BYTES);
    int dev = 0;
    PK_HIP(nullptr, hipGetDevice(&dev));
    unsigned char* base = nullptr;
    if ((st = device_scratch(dev, &base)) != PK_OK) return st;
    carve_scratch(base, *cfg, pl.units, pl.qheads, s->n, cs, &sc);
    st = retrieve_impl(pl, sc, cs, q, q_dtype, s, topk_idx, topk_est, nullptr, stream, same_dtype ? &a : nullptr,
                       &attended);
  }
  if (st != PK_OK || attended) return st;
  return attend_impl(pl, q, q_dtype, k, v, kv_dtype, kv_strides, n_rows, topk_idx, out, out_dtype, stream);
}

pk_status pk_host_alloc_mapped(size_t bytes, void** host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr || bytes == 0) return fail(nullptr, PK_ERR_INVALID_ARG, "bad arguments");
  *host_ptr = *device_ptr = nullptr;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hipHostMallocMapped);
  if (e != hipSuccess || !h)
    return fail(nullptr, PK_ERR_OUT_OF_MEMORY, "hipHostMalloc(%zu, mapped) failed: %s", bytes, hipGetErrorString(e));
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return fail(nullptr, PK_ERR_HIP, "hipHostGetDevicePointer failed: %s", hipGetErrorString(e));
  }
  *host_ptr = h;
  *device_ptr = d;
  return PK_OK;
}

pk_status pk_offload_rows(const void* src, const int64_t src_strides[3], void* dst, const int64_t dst_strides[3],
                          pk_dtype dtype, int32_t batch, int32_t n_kv_heads, int64_t rows, void* hip_stream) {
  if (dtype != PK_F32 && dtype != PK_BF16) return fail(nullptr, PK_ERR_UNSUPPORTED, "dtype %d", (int)dtype);
  if (batch < 1 || n_kv_heads < 1 || rows < 0)
    return fail(nullptr, PK_ERR_INVALID_ARG, "batch and n_kv_heads must be >= 1 and rows >= 0");
  pk_status st = check_strides(nullptr, src, dtype, src_strides, "src");
  if (st != PK_OK) return st;
  if ((st = check_strides(nullptr, dst, dtype, dst_strides, "dst")) != PK_OK) return st;
  if (rows == 0) return PK_OK;
  const int64_t vec = dtype == PK_BF16 ? 8 : 4;   // elements per 16 bytes
  const int row_vec = (int)(PK_HEAD_DIM / vec);
  const int64_t total = (int64_t)batch * n_kv_heads * rows * row_vec;
  hipLaunchKernelGGL(pk::copy_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     (hipStream_t)hip_stream, reinterpret_cast<const uint4*>(src), src_strides[0] / vec,
                     src_strides[1] / vec, src_strides[2] / vec, reinterpret_cast<uint4*>(dst), dst_strides[0] / vec,
                     dst_strides[1] / vec, dst_strides[2] / vec, (int)n_kv_heads, rows, row_vec, total);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(nullptr, PK_ERR_HIP, "offload launch failed: %s", hipGetErrorString(e));
  return PK_OK;
}

pk_status pk_calibration_copy(void* dst, const void* src, size_t bytes, void* hip_stream) {
  if (!dst || !src || bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16))
    return fail(nullptr, PK_ERR_INVALID_ARG, "calibration copy needs non-NULL 16-byte aligned pointers and size");
  if (bytes == 0) return PK_OK;
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 8192);
  hipLaunchKernelGGL(pk::copy16_kernel, dim3(grid), dim3(256), 0, (hipStream_t)hip_stream,
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(nullptr, PK_ERR_HIP, "copy launch failed: %s", hipGetErrorString(e));
  return PK_OK;
}

pk_status pk_host_free(void* host_ptr) {
  if (!host_ptr) return PK_OK;
  hipError_t e = hipHostFree(host_ptr);
  if (e != hipSuccess) return fail(nullptr, PK_ERR_HIP, "hipHostFree failed: %s", hipGetErrorString(e));
  return PK_OK;
}

pk_status pk_device_errors(pk_context* ctx, uint32_t* flags, void* hip_stream) {
  static_assert(PK_DEVICE_ERR_SLOT == pk::PK_DEV_ERR_SLOT, "device error flags");
  if (!ctx || !flags) return fail(ctx, PK_ERR_INVALID_ARG, "NULL argument");
  hipStream_t stream = (hipStream_t)hip_stream;
  uint32_t v = 0;
  PK_HIP(ctx, hipMemcpyAsync(&v, ctx->dev_err, 4, hipMemcpyDeviceToHost, stream));
  PK_HIP(ctx, hipStreamSynchronize(stream));
  if (v) {
    hipLaunchKernelGGL(pk::fill_u32_kernel, dim3(1), dim3(256), 0, stream, ctx->dev_err, 0u, (int64_t)1);
    pk_status st = check_launch(ctx, "fill");
    if (st != PK_OK) return st;
    PK_HIP(ctx, hipStreamSynchronize(stream));
  }
  *flags = v;
  return PK_OK;
}

pk_status pk_timing_begin(pk_context* ctx, int32_t max_launches) {
  if (!ctx) return fail(nullptr, PK_ERR_INVALID_ARG, "context is NULL");
  if (max_launches < 1 || max_launches > 1000000) return fail(ctx, PK_ERR_INVALID_ARG, "max_launches out of range");
  for (int k = 0; k < PK_N_KERNELS; ++k) {
    for (hipEvent_t e : ctx->ev[k]) (void)hipEventDestroy(e);
    ctx->ev[k].assign(2 * (size_t)max_launches, nullptr);
    for (auto& e : ctx->ev[k]) PK_HIP(ctx, hipEventCreate(&e));
    ctx->ev_used[k] = 0;
  }
  ctx->timing_cap = max_launches;
  return PK_OK;
}

pk_status pk_timing_end(pk_context* ctx, pk_kernel_timing* out) {
  if (!ctx || !out) return fail(ctx, PK_ERR_INVALID_ARG, "NULL argument");
  for (int k = 0; k < PK_N_KERNELS; ++k) {
    out[k].launches = ctx->ev_used[k];
    out[k].total_ms = 0.0;
    for (int i = 0; i < ctx->ev_used[k]; ++i) {
      PK_HIP(ctx, hipEventSynchronize(ctx->ev[k][2 * i + 1]));
      float ms = 0.0f;
      PK_HIP(ctx, hipEventElapsedTime(&ms, ctx->ev[k][2 * i], ctx->ev[k][2 * i + 1]));
      out[k].total_ms += ms;
    }
  }
  ctx->timing_cap = 0;
  return PK_OK;
}

}  // extern "C"
