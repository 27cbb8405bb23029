/*
 * pariskv.h -- C ABI of the ParisKV decode-time KV-cache retrieval path for
 * AMD Instinct MI355X (gfx950).
 *
 * What the path computes (sources are the ParisKV pages, cited by title and
 * section / equation / frame):
 *   "README"  = ParisKV: Fast and Drift-Robust KV-Cache Retrieval for
 *               Long-Context LLMs, the authors' repository README;
 *   "Slides"  = ParisKV: Fast and Drift-Robust KV-Cache Retrieval, beamer
 *               slides of the ICML 2026 paper (frames cite paper Sec./Eq.).
 *
 * Per (sequence, KV head) "unit", keys are summarised once (pk_encode_keys,
 * pk_append_keys) and every decode step runs, per query head:
 *   1. SRHT normalise-rotate of the query and sign-pattern centroid scoring in
 *      each 8-dim subspace (Slides Eqs. (5)-(6); README "2. Decode");
 *   2. tier-weighted collision votes S_i over every key's 16 centroid IDs
 *      (Slides Eq. (15), Sec. 4.2.2), with centroid-rank tiers or the paper's
 *      six percentile tiers, and optionally the README's adaptive ratios;
 *   3. the C keys with the largest S_i, ties to the lower key index, found by
 *      histogram + prefix scan instead of a sort (Slides Sec. 4.2.2);
 *   4. the 4-bit inner-product estimate of each candidate (Slides Eqs. (7)-(10));
 *   5. the Top-k estimates, ties to the lower key index (Slides Sec. 4.2.3);
 *   6. softmax attention over the k retrieved full-precision K/V rows only,
 *      s_i = scale * <k_i, q>, o = sum softmax(s)_i v_i (Slides Sec. 3,
 *      Eqs. (1)-(3); README "3. Attention"); K/V may sit in pinned host memory
 *      read through a mapped device pointer (README "Key Insight"; Slides
 *      Fig. 5, Sec. 4.2.3).
 *
 * Conventions for every call:
 *   - All tensor arguments are raw pointers; "device" pointers are HIP device
 *     addresses (hipMalloc'd, or device views of mapped pinned host memory from
 *     pk_host_alloc_mapped).  The caller owns every tensor.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and the call returns a negative pk_status;
 *     pk_last_error() then describes it.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t, NULL for
 *     the default stream).  Outputs are valid after the stream synchronises;
 *     a device fault surfaces at that synchronisation.
 *   - A context owns scratch memory sized at pk_create; no call allocates
 *     device memory after that (pk_timing_begin allocates its events).  One
 *     context serves one stream at a time.  pk_retrieve_attend_noalloc needs
 *     no context and allocates nothing.
 *   - Outputs must not alias inputs.
 */
#ifndef PARISKV_H
#define PARISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PK_OK = 0,
  PK_ERR_INVALID_ARG = -1,   /* bad pointer, size, stride or config field     */
  PK_ERR_UNSUPPORTED = -2,   /* valid in principle, not supported by this library */
  PK_ERR_CAPACITY = -3,      /* keys would exceed the summaries' capacity      */
  PK_ERR_OUT_OF_MEMORY = -4, /* device or pinned host allocation failed        */
  PK_ERR_HIP = -5,           /* a HIP runtime call failed (no GPU, launch error) */
  /* never returned: they make every int32 value a valid pk_status, so that a
     caller's out-of-range value (e.g. to pk_status_str) is defined behaviour */
  PK_STATUS_MIN_ENUM_ = -0x7FFFFFFF - 1,
  PK_STATUS_MAX_ENUM_ = 0x7FFFFFFF
} pk_status;

typedef enum {
  PK_F32 = 0,
  PK_BF16 = 1,
  /* not dtypes: every int32 value is a pk_dtype, so that an invalid one is
     refused (PK_ERR_UNSUPPORTED) rather than undefined */
  PK_DTYPE_MIN_ENUM_ = -0x7FFFFFFF - 1,
  PK_DTYPE_MAX_ENUM_ = 0x7FFFFFFF
} pk_dtype;

/* Fixed geometry of this library. */
#define PK_HEAD_DIM 128      /* D */
#define PK_N_SUB 16          /* B subspaces (Slides, App. Table 4: B = 16, m = 8) */
#define PK_SUB_DIM 8         /* m: one byte of sign bits per subspace          */
#define PK_N_LEVELS 8        /* 3-bit magnitude index (README "Codebooks")     */
#define PK_RECORD_BYTES 128  /* 64 B of nibbles + 16 fp32 weights per key      */
#define PK_MAX_GROUP 4       /* query heads per KV head                        */
#define PK_MAX_TOPK 256
#define PK_MAX_CANDIDATES 16384
#define PK_MAX_DENSE 8192      /* dense rows per head in pk_sparse_dense_attend */

typedef struct {
  int32_t head_dim;          /* must be 128                                    */
  int32_t n_sub;             /* must be 16                                     */
  int32_t sub_dim;           /* must be 8                                      */
  uint64_t srht_seed;        /* Philox4x64-10 key for the SRHT sign vector     */
  int32_t n_tiers;           /* 1..4 */
  int32_t tier_top[4];       /* strictly increasing centroid-rank cut-offs, <= 256:
                                a key block whose centroid ranks r < tier_top[t]
                                (and >= tier_top[t-1]) for the query gets
                                tier_weight[t]; e.g. {1, 4, 16}               */
  int32_t tier_weight[4];    /* 0..4 each (n_sub * max weight must be <= 64)   */
  int32_t n_candidates;      /* C, 1..PK_MAX_CANDIDATES                        */
  int32_t top_k;             /* k, 1..min(C, PK_MAX_TOPK)                      */
  float softmax_scale;       /* s_i = scale * <k_i, q>                         */
  int32_t batch;             /* sequences                                      */
  int32_t n_kv_heads;        /* KV heads per sequence                          */
  int32_t n_q_heads;         /* query heads per sequence; query head h reads KV
                                head h / (n_q_heads / n_kv_heads); the ratio
                                must be an integer in 1..PK_MAX_GROUP          */
  int64_t n_capacity;        /* max keys per unit, 1..2^31-1                   */
  int32_t tier_mode;         /* PK_TIERS_RANK: the tier_top / tier_weight votes
                                above.  PK_TIERS_PERCENTILE (Slides Sec. 4.2.2,
                                Eq. (15)): in each block the keys are ordered by
                                their centroid's score for the query and the
                                first M = ceil(rho n) positions are split into
                                six equal percentile tiers with bonuses 6..1; a
                                centroid takes the tier of its first key's
                                position (needs pk_summaries.counts)          */
  int32_t collision_permille;/* percentile tiers: rho in 1/1000, 1..1000; unused
                                with adaptive_ratios                          */
  int32_t adaptive_ratios;   /* 1: the candidate ratio beta and the collision
                                ratio rho follow the retrieval-zone length n
                                (README "Parameters" table: n < 5K 0.5/0.5,
                                < 10K 0.25/0.3, < 30K 0.2/0.25, else 0.1/0.2);
                                C = ceil(beta n) must not exceed n_candidates,
                                which then only sizes the scratch            */
} pk_config;

#define PK_TIERS_RANK 0
#define PK_TIERS_PERCENTILE 1

typedef struct pk_context pk_context;   /* opaque */

/* Key summaries of every unit (unit = sequence * n_kv_heads + kv_head), device
 * memory owned by the caller and sized with pk_summary_bytes:
 *   codes   u8  [units][n_capacity][16]   centroid ID (sign pattern) per
 *                                         subspace (README "1. Prefill")
 *   records u8  [units][n_capacity][128]  bytes 0..63: 4-bit codes, nibble =
 *                                         (sign << 3) | magnitude index,
 *                                         coordinate 2p in the low nibble of
 *                                         byte p; bytes 64..127: 16 fp32
 *                                         per-subspace weights w_b (Slides
 *                                         Eq. (9))
 *   norms   f32 [units][n_capacity]       ||k|| of each key
 *   counts  u32 [units][16][256]          keys per (subspace, centroid) among
 *                                         the n valid keys; kept up to date by
 *                                         pk_encode_keys / pk_append_keys when
 *                                         non-NULL; needed by percentile tiers
 *                                         (NULL allowed with rank tiers)
 * codes rows must be 16-byte aligned and records 128-byte aligned (true for
 * hipMalloc'd bases).  `n` is the number of valid keys per unit. */
typedef struct {
  uint8_t* codes;
  uint8_t* records;
  float* norms;
  uint32_t* counts;
  int64_t n;
  int64_t n_capacity;
} pk_summaries;

/* Optional copies of intermediate results (device pointers, each nullable),
 * written by pk_retrieve after its kernels:
 *   rot_q    f32 [batch][n_q_heads][128]   R q * ||q||-scaled (= fl(H(s*q)/sqrt(D)))
 *   lut      u32 [units][16][256]          byte g = tier weight of that centroid
 *                                          for query head g of the unit
 *   scores   u32 [units][n]                byte g = collision score S of the key
 *                                          for query head g of the unit
 *   cand_idx i32 [batch][n_q_heads][C]     candidates, ascending key index;
 *   cand_est f32 [batch][n_q_heads][C]     their estimates (min(n, C) valid
 *                                          entries, the rest -1 / -inf)      */
typedef struct {
  float* rot_q;
  uint32_t* lut;
  uint32_t* scores;
  int32_t* cand_idx;
  float* cand_est;
} pk_debug;



/* Kernels whose launches pk_timing_* can bracket with HIP events. */
typedef enum {
  PK_KERNEL_ENCODE = 0,
  PK_KERNEL_QPREP = 1,
  PK_KERNEL_COLLIDE = 2,
  PK_KERNEL_THRESHOLD = 3,     /* reserved: no longer launched (every select
                                  workgroup derives the selection parameters) */
  PK_KERNEL_SELECT = 4,
  PK_KERNEL_RERANK = 5,        /* 4-bit rerank, several workgroups per head (few heads) */
  PK_KERNEL_TOPK = 6,          /* final top-k after PK_KERNEL_RERANK */
  PK_KERNEL_ATTEND = 7,
  PK_KERNEL_RERANK_TOPK = 8,   /* rerank and final top-k in one workgroup per head (many heads) */
  PK_KERNEL_DENSE_ATTEND = 9,  /* pk_sparse_dense_attend */
  PK_N_KERNELS = 10
} pk_kernel_id;

typedef struct {
  int32_t launches;          /* launches recorded                              */
  double total_ms;           /* summed event-to-event time                     */
} pk_kernel_timing;

/* ---- configuration and tables (host only, no GPU needed) ---------------- */

/* Check every field of `cfg`; PK_OK or PK_ERR_INVALID_ARG / _UNSUPPORTED. */
pk_status pk_validate_config(const pk_config* cfg);

/* Bytes of each summary array for `cfg` (units * n_capacity rows; counts:
 * units * 16 * 256 words).  Any output may be NULL. */
pk_status pk_summary_bytes(const pk_config* cfg, size_t* codes_bytes,
                           size_t* records_bytes, size_t* norms_bytes,
                           size_t* counts_bytes);

/* The constant tables a context uses, computed on the host:
 * signs[128]  +-1, sign j = +1 iff the top bit of the j-th 64-bit output of
 *             Philox4x64-10 with key (seed, 0) and counters 1, 2, ... is 0
 *             (the SRHT's random diagonal, Slides Eq. (5), Sec. 4.1.1);
 * levels[8], thresholds[7]  fp32 Lloyd-Max quantiser of |u_j| under the
 *             Beta(1/2, (m-1)/2) prior of u_j^2 (Slides Prop. 4.1, App. B.1;
 *             README "Codebooks"); index = #{thresholds <= |u_j|}. */
pk_status pk_tables(uint64_t seed, int8_t signs[128], float levels[8], float thresholds[7]);

/* ---- context ------------------------------------------------------------- */

/* Validate `cfg`, compute the tables, allocate the context's device scratch on
 * the current HIP device.  *out is NULL on error. */
pk_status pk_create(const pk_config* cfg, pk_context** out);
void pk_destroy(pk_context* ctx);

/* ---- summaries (Slides Eqs. (5)-(9); README "1. Prefill") ---------------- */

/* Encode keys [batch][n_kv_heads][n][128] (element strides `key_strides` =
 * {batch, head, token}; the last dimension is contiguous) into rows [0, n) of
 * every unit and set inout->n = n.  keys: device pointer, PK_F32 or PK_BF16.
 * When inout->counts is non-NULL it is recounted over the n keys.
 * What a row holds (README "1. Prefill": keys normalised, SRHT-rotated and
 * summarised twice): the 16 sign-pattern centroid IDs of the rotated key's
 * 8-dim blocks, one byte each (Slides Eqs. (5)-(6)); the 4-bit codes of its
 * coordinates, a sign bit and a 3-bit Lloyd-Max magnitude level (Slides frame
 * "The codebook is data-independent; the quantizer uses a prior"), with one
 * fp32 weight per block (Slides Eqs. (7)-(10)); and the key's norm. */
pk_status pk_encode_keys(pk_context* ctx, const void* keys, pk_dtype key_dtype,
                         const int64_t key_strides[3], int64_t n,
                         pk_summaries* inout, void* hip_stream);

/* Encode t new keys per unit ([batch][n_kv_heads][t][128], strides as above)
 * into rows [inout->n, inout->n + t) and advance inout->n by t.  New keys use
 * the same fixed analytic codebook, no retraining (Slides, frame "The codebook
 * is data-independent"); inout->counts (when non-NULL) gains their codes.
 * PK_ERR_CAPACITY if n + t > n_capacity. */
pk_status pk_append_keys(pk_context* ctx, const void* new_keys, pk_dtype key_dtype,
                         const int64_t key_strides[3], int64_t t,
                         pk_summaries* inout, void* hip_stream);

/* ---- decode step ------------------------------------------------------------ */

/* Retrieve the Top-k keys of every query head (README "2. Decode"): the query
 * is rotated and scored against each block's centroids (Slides Eqs. (5)-(6));
 * every key gets the tier-weighted collision vote S_i of Slides Eq. (15)
 * (Sec. 4.2.2, Stage I); the C keys with the largest S_i (ties to the lower
 * index) are reranked with the 4-bit inner-product estimate of Slides Eqs.
 * (7)-(10) (Stage II); the k largest estimates (ties to the lower index) are
 * returned (Slides Sec. 4.2.3).
 * q          device [batch][n_q_heads][128], PK_F32 or PK_BF16, contiguous;
 * sums       summaries with sums->n >= 0 valid keys per unit;
 * topk_idx   device i32 [batch][n_q_heads][k]: key indices sorted by
 *            (estimate desc, index asc); -1 pads when fewer than k keys exist;
 * topk_est   device f32 [batch][n_q_heads][k] estimates (nullable; -inf pads);
 * dbg        optional intermediate copies (nullable). */
pk_status pk_retrieve(pk_context* ctx, const void* q, pk_dtype q_dtype,
                      const pk_summaries* sums, int32_t* topk_idx, float* topk_est,
                      const pk_debug* dbg, void* hip_stream);

/* Sparse attention over the retrieved rows of every query head (Slides Sec. 3,
 * Eqs. (1)-(3); README "3. Attention"): s_i = softmax_scale * <k_i, q> over the
 * retrieved indices only, o = sum_i softmax(s)_i v_i, in fp32.  The rows may
 * sit in mapped host memory and are then read one by one over the host link
 * (README "Key Insight").
 * q          device [batch][n_q_heads][128], contiguous;
 * k, v       [batch][n_kv_heads][n][128] with element strides kv_strides =
 *            {batch, head, token} shared by K and V, last dim contiguous, rows
 *            16-byte aligned; device pointers or mapped host pointers;
 * n_rows     rows present per (sequence, KV head) in K and V;
 * topk_idx   device i32 [batch][n_q_heads][top_k]; entries < 0 or >= n_rows
 *            are skipped (never dereferenced);
 * out        device [batch][n_q_heads][128] in out_dtype; a head with no
 *            valid index gets zeros. */
pk_status pk_sparse_attend(pk_context* ctx, const void* q, pk_dtype q_dtype,
                           const void* k, const void* v, pk_dtype kv_dtype,
                           const int64_t kv_strides[3], int64_t n_rows,
                           const int32_t* topk_idx, void* out, pk_dtype out_dtype,
                           void* hip_stream);

/* Retrieval and sparse attention in one call (README "2. Decode" then
 * "3. Attention"; Slides Sec. 4.2.3 then Eqs. (1)-(3)): the same outputs as
 * pk_retrieve followed by pk_sparse_attend with these arguments on the same
 * stream.  When q, K/V and out share one dtype, the workgroup that selects a
 * head's Top-k also attends over that head's rows, so the retrieved indices
 * never leave the chip before they are used.  The output may then differ from
 * the separate attention call by fp32 summation order (the softmax and
 * weighted sum are split over 16 instead of 4 waves).
 * Arguments, layouts, ownership and errors as for the two calls. */
pk_status pk_retrieve_attend(pk_context* ctx, const void* q, pk_dtype q_dtype,
                             const pk_summaries* sums, const void* k, const void* v,
                             pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows,
                             int32_t* topk_idx, float* topk_est, void* out, pk_dtype out_dtype,
                             const pk_debug* dbg, void* hip_stream);

/* One decode step: the step's new keys join the summaries, then retrieval and
 * sparse attention over all n + t keys (README "2. Decode": new tokens are
 * encoded with the fixed codebook as they arrive, then the query retrieves;
 * Slides Sec. 4.2.3).  The results equal pk_append_keys(new_keys, t, inout)
 * followed by pk_retrieve_attend(q, inout, ...) on the same stream, and
 * inout->n advances by t when the call returns PK_OK.  With rank tiers and
 * t <= 64 the new rows are encoded by extra workgroups of the query-prep
 * launch, which saves a launch per step (percentile tiers need the new rows'
 * centroid counts before the query prep, so there the encode runs first).
 * new_keys, key_dtype, key_strides, t: as for pk_append_keys (the rows may be
 * rows n .. n + t - 1 of the k argument); the other arguments as for
 * pk_retrieve_attend, with no debug copies.  Errors as for the two calls; on
 * an error nothing is enqueued if it is an argument error, and inout->n is
 * unchanged in every case. */
pk_status pk_append_retrieve_attend(pk_context* ctx, const void* new_keys, pk_dtype key_dtype,
                                    const int64_t key_strides[3], int64_t t, pk_summaries* inout,
                                    const void* q, pk_dtype q_dtype, const void* k, const void* v,
                                    pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows,
                                    int32_t* topk_idx, float* topk_est, void* out, pk_dtype out_dtype,
                                    void* hip_stream);

/* pk_retrieve_attend without a context, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results, layouts and errors as
 * pk_retrieve_attend with a context created from *cfg (no debug copies, no
 * timings, no device error flags), except that nothing is allocated: the
 * call's scratch (tier LUT, rotated queries, packed scores, score bin
 * totals and sub-tile suffix counts, candidate lists) lives in a static device array of
 * PK_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends.  Its size per call is about 4 * units * n + 8 * (query heads)
 * * C + 16 KiB * units bytes; a call that needs more than the array returns
 * PK_ERR_CAPACITY (nothing enqueued).  The tables are computed on the host
 * at each call (no device work).  Every call on a GPU shares that GPU's array
 * and leaves its contents behind: calls that overlap on one GPU (on different
 * streams, or from several threads) race and must be serialised by the
 * caller.  No array needs clearing between calls. */
#define PK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pk_status pk_retrieve_attend_noalloc(const pk_config* cfg, const void* q, pk_dtype q_dtype,
                                     const pk_summaries* sums, const void* k, const void* v,
                                     pk_dtype kv_dtype, const int64_t kv_strides[3], int64_t n_rows,
                                     int32_t* topk_idx, float* topk_est, void* out, pk_dtype out_dtype,
                                     void* hip_stream);

/* Attention over the retrieved rows and a set of dense rows in one softmax
 * (README "3. Attention": sink, local and retrieved tokens; Slides Fig. 5,
 * Sec. 4.2.1-4.2.3: sink tokens and the recent local window with the update
 * buffer stay on the GPU for dense attention while the older retrieval zone
 * is searched through its summaries and read row by row).
 * q, k, v, kv_strides, n_rows, topk_idx as for pk_sparse_attend (k / v hold
 * the retrieval zone; indices are zone rows);
 * dense_k, dense_v  [batch][n_kv_heads][n_dense][128] in kv_dtype with
 *            element strides dense_strides = {batch, head, token}, last dim
 *            contiguous, rows 16-byte aligned: every row is attended (their
 *            order does not matter, so a ring buffer works);
 * n_dense    0..PK_MAX_DENSE;
 * out        device [batch][n_q_heads][128] in out_dtype; zeros when nothing
 *            is attended.  fp32 scores, softmax and sums. */
pk_status pk_sparse_dense_attend(pk_context* ctx, const void* q, pk_dtype q_dtype,
                                 const void* k, const void* v, pk_dtype kv_dtype,
                                 const int64_t kv_strides[3], int64_t n_rows,
                                 const int32_t* topk_idx, const void* dense_k, const void* dense_v,
                                 const int64_t dense_strides[3], int64_t n_dense,
                                 void* out, pk_dtype out_dtype, void* hip_stream);

/* ---- host-resident KV tier (README "Key Insight": UVA fetch) -------------- */

/* Pinned, mapped host memory: *host_ptr for the CPU, *device_ptr for kernels.
 * PK_ERR_OUT_OF_MEMORY if the allocation fails. */
pk_status pk_host_alloc_mapped(size_t bytes, void** host_ptr, void** device_ptr);
pk_status pk_host_free(void* host_ptr);

/* Offload of full-precision K or V rows into the host tier (README "1. Prefill":
 * K/V asynchronously offloaded to CPU memory; Slides Fig. 5, Sec. 4.2.1: a
 * full update buffer is encoded and its old local tokens are moved out):
 * copies rows [0, rows) of every (sequence, KV head) of src [batch][n_kv_heads]
 * [rows][128] to dst with the same shape.  src, dst: device pointers (dst
 * typically the device view of pk_host_alloc_mapped memory, at the zone row
 * where the rows belong), element strides {batch, head, token}, last dim
 * contiguous, rows 16-byte aligned; both of `dtype`.  Enqueued on hip_stream,
 * which may be a second stream beside the retrieval's: the caller orders any
 * attention that may read the rows after it (an event), and keeps src
 * unchanged until it completes.  PK_ERR_INVALID_ARG / _UNSUPPORTED on bad
 * arguments (nothing enqueued). */
pk_status pk_offload_rows(const void* src, const int64_t src_strides[3], void* dst,
                          const int64_t dst_strides[3], pk_dtype dtype, int32_t batch,
                          int32_t n_kv_heads, int64_t rows, void* hip_stream);

/* ---- measurement aids ------------------------------------------------------ */

/* Plain device-to-device copy of `bytes` (a multiple of 16; both pointers
 * 16-byte aligned, non-overlapping) in which every lane moves 16 bytes per
 * access, the access width of the collide and rerank kernels.  Used to
 * calibrate the HBM traffic counters (bytes read / written per counted KiB)
 * for that access pattern.  Asynchronous on `hip_stream`; PK_ERR_INVALID_ARG
 * on a NULL pointer, a misaligned pointer or size. */
pk_status pk_calibration_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

/* ---- timing --------------------------------------------------------------- */

/* Start bracketing each launch of every kernel with HIP events on the stream
 * it runs on, for at most `max_launches` launches per kernel (allocates the
 * events).  pk_timing_end synchronises them, fills timings[PK_N_KERNELS] and
 * stops recording. */
pk_status pk_timing_begin(pk_context* ctx, int32_t max_launches);
pk_status pk_timing_end(pk_context* ctx, pk_kernel_timing* timings);

/* ---- diagnostics ---------------------------------------------------------- */

/* Device-side consistency flags of `ctx`, accumulated over its launches since
 * the last call: PK_DEVICE_ERR_SLOT (a candidate's slot fell outside the list,
 * i.e. the selection parameters did not match the collision scores; the
 * candidate is dropped rather than written out of bounds).  Waits for
 * `hip_stream`, copies the flags to *flags and clears them.  PK_ERR_HIP if a
 * HIP call fails. */
#define PK_DEVICE_ERR_SLOT 1u
pk_status pk_device_errors(pk_context* ctx, uint32_t* flags, void* hip_stream);

const char* pk_status_str(pk_status status);
/* Last error message of `ctx`, or of the calling thread when ctx is NULL. */
const char* pk_last_error(const pk_context* ctx);

#ifdef __cplusplus
}
#endif
#endif /* PARISKV_H */
