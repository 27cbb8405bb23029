// HIP kernels of the ParisKV decode path for gfx950 (wave64, 160 KiB LDS/CU).
//
// Sources: "README" = ParisKV: Fast and Drift-Robust KV-Cache Retrieval for
// Long-Context LLMs (repository README); "Slides" = ParisKV: Fast and
// Drift-Robust KV-Cache Retrieval (ICML 2026 paper slides; frames cite the
// paper's Sec./Eq.).
//
// Floating-point operations that decide integers (sign codes, magnitude
// indices, centroid ranks) or produce the fp32 rerank estimates follow one
// fixed order, with no contraction into fused multiply-adds (the build passes
// -ffp-contract=off); division and square root are correctly rounded.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>

#define PK_SORT_N 256          // top-k sort slots (k <= 256)
#define PK_MAX_TOPK_ATT 256    // rows per attention head (k <= 256)
#define PK_MAX_DENSE 8192      // dense rows per head in dense + retrieved attention

namespace pk {

constexpr int D = 128;       // head dimension
constexpr int NSUB = 16;     // subspaces
constexpr int SUBD = 8;      // coordinates per subspace
constexpr int NLEV = 8;      // magnitude levels
constexpr int NBIN = 64;     // collision-score bins 1..64 with rank tiers (0 is derived)
constexpr int NBIN_MAX = 128; // bins with percentile tiers (S <= 16 * 6 = 96)
constexpr int MAXG = 4;      // query heads per KV head

// device-side error flags (one word of the context's scratch)
constexpr uint32_t PK_DEV_ERR_SLOT = 1u;   // a candidate slot fell outside the list

// Constant tables passed by value to every kernel that needs them.
struct Tables {
  uint32_t neg_bits[4];      // bit j of the 128-bit mask set <=> SRHT sign j is -1
  float levels[NLEV];        // Lloyd-Max magnitude levels
  float thresholds[NLEV - 1];
  float inv_sqrt_d;          // fl32(1 / sqrt(128))
};

struct TierSpec {
  int n_tiers;
  int top[4];
  int weight[4];
};

// Table entries picked by a per-lane index through selects over scalar
// registers: an indexed read of a kernel-argument array is a vector memory
// load, and waiting for it also waits for every load issued before it (the
// record gathers in the rerank, the key loads in the encoder).  The entries
// pass through readfirstlane so that the selects are not turned back into
// such a load.
__device__ __forceinline__ uint32_t sreg(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ float level_of(const Tables& tb, int i) {
  uint32_t lv[NLEV];
#pragma unroll
  for (int l = 0; l < NLEV; ++l) lv[l] = sreg(__float_as_uint(tb.levels[l]));
  uint32_t v = lv[0];
#pragma unroll
  for (int l = 1; l < NLEV; ++l) v = (i == l) ? lv[l] : v;
  return __uint_as_float(v);
}
// weight of the first tier whose top exceeds `rank` (0 past the last tier),
// by selects over the tiers in scalar registers: a loop that stops at a
// per-lane tier would index the argument array per lane (a vector load)
__device__ __forceinline__ uint32_t tier_weight_of(const TierSpec& tiers, int rank) {
  uint32_t wgt = 0;
#pragma unroll
  for (int tt = 3; tt >= 0; --tt)
    if (tt < tiers.n_tiers) wgt = rank < (int)sreg((uint32_t)tiers.top[tt]) ? sreg((uint32_t)tiers.weight[tt]) : wgt;
  return wgt;
}
__device__ __forceinline__ uint32_t neg_word(const Tables& tb, int i) {
  uint32_t nw[4];
#pragma unroll
  for (int l = 0; l < 4; ++l) nw[l] = sreg(tb.neg_bits[l]);
  uint32_t v = nw[0];
#pragma unroll
  for (int l = 1; l < 4; ++l) v = (i == l) ? nw[l] : v;
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// order-preserving map of a float to u32 (larger float -> larger key); -0 == +0
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Correctly rounded fp32 square root.  The hardware estimate s is within one
// ulp of sqrt(x); the rounded-to-nearest result is s - ulp, s or s + ulp.  For
// neighbours a < b the midpoint satisfies ((a + b) / 2)^2 = a*b + (b - a)^2 / 4,
// and x - a*b is an exact multiple of ulp(s)^2 (all three are multiples of it),
// so sqrt(x) lies below the midpoint iff x - a*b <= 0.  The single-rounding fma
// gives that sign exactly.
__device__ __forceinline__ float sqrt_rn(float x) {
  const float s = sqrtf(x);
  if (!(x > 0.0f) || !(x < __builtin_inff())) return s;
  const float sm = __uint_as_float(__float_as_uint(s) - 1u);
  const float sp = __uint_as_float(__float_as_uint(s) + 1u);
  const float rm = __builtin_fmaf(-sm, s, x);
  const float rp = __builtin_fmaf(-s, sp, x);
  float r = (rm <= 0.0f) ? sm : s;
  r = (rp > 0.0f) ? sp : r;
  return r;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---- cross-lane moves without LDS -------------------------------------------
// swap32_sum(a, b): lanes 32..63 of a trade places with lanes 0..31 of b
// (v_permlane32_swap), then the two are added, so lane l < 32 gets a + a of
// lane l + 32 and lane l >= 32 gets b + b of lane l - 32.  swap16_sum does the
// same between the odd 16-lane rows of a and the even rows of b (partner l ^ 16).
__device__ __forceinline__ uint32_t swap32_sum(uint32_t a, uint32_t b) {
  const auto t = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return t[0] + t[1];
}
__device__ __forceinline__ uint32_t swap16_sum(uint32_t a, uint32_t b) {
  const auto t = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  return t[0] + t[1];
}
// x of lane l ^ W for W = 1, 2, 4, 8 (DPP: quad permutations, half-row mirror, row rotate)
template <int W>
__device__ __forceinline__ uint32_t dpp_xor(uint32_t x) {
  if constexpr (W == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  else if constexpr (W == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  else if constexpr (W == 4) {
    const int m = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);   // row_half_mirror: l -> 7 - l
    return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);      // quad_perm 3,2,1,0
  } else {
    static_assert(W == 8, "W is 1, 2, 4 or 8");
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false);  // row_ror 8
  }
}
// inclusive prefix sum over the 64 lanes (lane l: lanes 0..l): shifts by 1, 2,
// 4, 8 inside each 16-lane row, then row totals carried upward
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr 1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr 2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr 4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr 8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast 15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast 31 -> rows 2, 3
  return x;
}
// x of lane l ^ W for W = 1 .. 32: DPP inside a 16-lane row, the lane-half
// swaps across rows (W = 16) and halves (W = 32).  Every lane must be active.
template <int W>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (W <= 8) {
    return dpp_xor<W>(x);
  } else if constexpr (W == 16) {
    const auto t = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? t[0] : t[1];
  } else {
    static_assert(W == 32, "W is a power of two up to 32");
    const auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? t[0] : t[1];
  }
}
template <int W>
__device__ __forceinline__ float lane_xor_f(float x, int lane) {
  return __uint_as_float(lane_xor<W>(__float_as_uint(x), lane));
}
// x = op(x, x of lane l ^ w) for w = 32, 16, 8, 4, 2, 1 in turn (the whole
// wave), or for w = 8, 4, 2, 1 (each 16-lane row); written out, since loops
// around these convergent moves are not unrolled
template <typename Op>
__device__ __forceinline__ float xor_butterfly16(float x, int lane, Op op) {
  x = op(x, lane_xor_f<8>(x, lane));
  x = op(x, lane_xor_f<4>(x, lane));
  x = op(x, lane_xor_f<2>(x, lane));
  return op(x, lane_xor_f<1>(x, lane));
}
template <typename Op>
__device__ __forceinline__ float xor_butterfly(float x, int lane, Op op) {
  x = op(x, lane_xor_f<32>(x, lane));
  x = op(x, lane_xor_f<16>(x, lane));
  return xor_butterfly16(x, lane, op);
}
template <typename Op>
__device__ __forceinline__ uint32_t xor_butterfly_u(uint32_t x, int lane, Op op) {
  x = op(x, lane_xor<32>(x, lane));
  x = op(x, lane_xor<16>(x, lane));
  x = op(x, lane_xor<8>(x, lane));
  x = op(x, lane_xor<4>(x, lane));
  x = op(x, lane_xor<2>(x, lane));
  return op(x, lane_xor<1>(x, lane));
}
// one stage of reduce_scatter64 below, width W <= 8 (DPP partner lane ^ W)
template <int W>
__device__ __forceinline__ void reduce_scatter_stage(uint32_t (&v)[64], int lane) {
  const bool up = (lane & W) != 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t send = up ? v[i] : v[i + W];
    const uint32_t keep = up ? v[i + W] : v[i];
    v[i] = keep + dpp_xor<W>(send);
  }
}

// Sum of entry l over the wave's 64 lanes, returned in lane l (v is consumed):
// after the stage of width w, v[i] (i < w) of lane l is the sum, over the
// 64 / w lanes that share l's bits below w, of entry i + (l & (64 - w));
// widths 32 and 16 trade register halves between lane halves / rows.
__device__ __forceinline__ uint32_t reduce_scatter64(uint32_t (&v)[64], int lane) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = swap32_sum(v[i], v[i + 32]);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = swap16_sum(v[i], v[i + 16]);
  reduce_scatter_stage<8>(v, lane);
  reduce_scatter_stage<4>(v, lane);
  reduce_scatter_stage<2>(v, lane);
  reduce_scatter_stage<1>(v, lane);
  return v[0];
}

struct AddF { __device__ float operator()(float a, float b) const { return a + b; } };
struct MaxF { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct MaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };
struct MinU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct AddU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };

// ===========================================================================
// encode: key summaries (Slides Eqs. (5)-(9); README "1. Prefill")
//
// 16 lanes per key, lane b owns coordinates 8b..8b+7 (subspace b).  The SRHT
// is s-flip then an unnormalised 128-point fast Walsh-Hadamard transform with
// butterfly stages h = 1, 2, 4 inside a lane and h = 8..64 across lanes; the
// 1/sqrt(128) and the key norm cancel in the codes and are folded into w:
//   y = H (s * k); rho_b = ||y_b||; bit j = [y_j > 0]; u = y / rho;
//   idx_j = #{tau_l <= |u_j|}; alpha = sum_j |u_j| L[idx_j];
//   w_b = rho_b fl(1/sqrt(128)) / alpha  (= ||k|| r_b / alpha_b, Eq. (9)).
// A workgroup encodes up to ENC_KEYS consecutive rows of one unit, 16 keys
// at a time, and counts its keys per (subspace, centroid) in LDS; the counts
// are added to the unit's totals once at the end.  A short append (at most
// ENC_DIRECT rows per unit) adds each key's counts directly instead.
// ===========================================================================
constexpr int ENC_KEYS = 1024;
constexpr int ENC_DIRECT = 64;

// lane b's 8 coordinates of one key, as fp32
template <typename KT>
__device__ __forceinline__ void load_key(const KT* __restrict__ src, float (&x)[SUBD]) {
  if constexpr (sizeof(KT) == 2) {
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  } else {
    const float4 v0 = *reinterpret_cast<const float4*>(src);
    const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
    x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
    x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
  }
}

// one cross-lane butterfly stage of a key's Walsh-Hadamard transform: the
// 16 lanes of a key form one DPP row; lanes b and b ^ M exchange coordinates,
// the lower one keeps the sums, the upper the differences
template <int M>
__device__ __forceinline__ void key_stage(float (&x)[SUBD], int b) {
  const bool upper = (b & M) != 0;
#pragma unroll
  for (int j = 0; j < SUBD; ++j) {
    const float p = __uint_as_float(dpp_xor<M>(__float_as_uint(x[j])));
    x[j] = upper ? (p - x[j]) : (x[j] + p);
  }
}

// code byte, nibbles, weight and partial squared norm of subspace b of one key
__device__ __forceinline__ void encode_key(float (&x)[SUBD], int b, const Tables& tb, uint32_t& code_out,
                                           uint32_t& nib_out, float& w_out, float& nsq_out) {
  float nsq = 0.0f;
#pragma unroll
  for (int j = 0; j < SUBD; ++j) nsq += x[j] * x[j];

  const uint32_t neg = (neg_word(tb, b >> 2) >> ((b & 3) * 8)) & 0xFFu;
#pragma unroll
  for (int j = 0; j < SUBD; ++j)
    x[j] = __uint_as_float(__float_as_uint(x[j]) ^ (((neg >> j) & 1u) << 31));

  // in-lane butterflies
#pragma unroll
  for (int h = 1; h < SUBD; h <<= 1) {
#pragma unroll
    for (int j = 0; j < SUBD; ++j) {
      if (!(j & h)) {
        const float a = x[j], c = x[j + h];
        x[j] = a + c;
        x[j + h] = a - c;
      }
    }
  }
  // cross-lane butterflies (partner lane b ^ m holds coordinate +- 8m)
  key_stage<1>(x, b);
  key_stage<2>(x, b);
  key_stage<4>(x, b);
  key_stage<8>(x, b);

  // per-subspace code, nibbles, weight
  float e = x[0] * x[0];
#pragma unroll
  for (int j = 1; j < SUBD; ++j) e = e + x[j] * x[j];
  const float rho = sqrt_rn(e);
  uint32_t code = 0, nib = 0;
#pragma unroll
  for (int j = 0; j < SUBD; ++j) {
    const uint32_t bit = x[j] > 0.0f ? 1u : 0u;
    code |= bit << j;
    nib |= (bit << 3) << (4 * j);
  }
  float w = 0.0f;
  if (rho > 0.0f) {
    float alpha = 0.0f;
#pragma unroll
    for (int j = 0; j < SUBD; ++j) {
      const float a = fabsf(__fdiv_rn(x[j], rho));
      uint32_t idx = 0;
      float lv = tb.levels[0];
#pragma unroll
      for (int l = 0; l < NLEV - 1; ++l) {
        const bool ge = a >= tb.thresholds[l];
        idx += ge ? 1u : 0u;
        lv = ge ? tb.levels[l + 1] : lv;
      }
      const float term = a * lv;
      alpha = (j == 0) ? term : alpha + term;
      nib |= idx << (4 * j);
    }
    w = __fdiv_rn(rho * tb.inv_sqrt_d, alpha);
  }

  code_out = code;
  nib_out = nib;
  w_out = w;
  nsq_out = nsq;
}

// Where the rows a launch encodes come from and go to.
template <typename KT>
struct EncodeArgs {
  const KT* keys;
  int64_t sb, sh, st;      // element strides of batch, KV head, token
  int n_kv_heads;
  int64_t t;               // rows per unit
  int chunks;              // workgroups per unit: ceil(t / ENC_KEYS)
  int64_t row0, n_cap;     // first row written, rows per unit of the summaries
  uint8_t* codes;
  uint8_t* records;
  float* norms;
  uint32_t* counts;        // nullable
};

// Workgroup `block` of NT threads (16 per key) encodes its rows.  DIRECT:
// every launch has t <= ENC_DIRECT, so the counts are added directly and no
// LDS counters are needed.
template <typename KT, int NT, bool DIRECT>
__device__ __forceinline__ void encode_body(const EncodeArgs<KT>& a, const Tables& tb, int block) {
  __shared__ uint32_t s_cnt[DIRECT ? 1 : NSUB * 256];
  const int64_t t = a.t, n_cap = a.n_cap, row0 = a.row0, st = a.st;
  const int64_t unit = block / a.chunks;
  const int64_t r0 = (int64_t)(block - unit * a.chunks) * ENC_KEYS;
  const int64_t r1 = (r0 + ENC_KEYS < t) ? r0 + ENC_KEYS : t;
  const int tid = threadIdx.x, b = tid & 15;
  const int64_t seq = unit / a.n_kv_heads, head = unit - seq * a.n_kv_heads;
  const KT* ubase = a.keys + seq * a.sb + head * a.sh + b * SUBD;
  const bool direct = DIRECT || t <= ENC_DIRECT;
  uint32_t* ucnt = a.counts ? a.counts + unit * NSUB * 256 : nullptr;
  uint8_t* codes = a.codes;
  uint8_t* records = a.records;
  float* norms = a.norms;
  if constexpr (!DIRECT) {
    if (ucnt && !direct) {
      for (int i = tid; i < NSUB * 256; i += NT) s_cnt[i] = 0;
      __syncthreads();
    }
  }

  // whole 16-lane groups; the next key's load is in flight while one is encoded
  constexpr int GROUPS = NT / 16;
  int64_t r = r0 + (tid >> 4);
  float xa[SUBD];
  if (r < r1) load_key<KT>(ubase + r * st, xa);
  for (; r < r1; r += GROUPS) {
    float xb[SUBD];
    if (r + GROUPS < r1) load_key<KT>(ubase + (r + GROUPS) * st, xb);
    uint32_t code, nib;
    float w, nsq;
    encode_key(xa, b, tb, code, nib, w, nsq);
#pragma unroll
    for (int j = 0; j < SUBD; ++j) xa[j] = xb[j];
    const int64_t row = unit * n_cap + row0 + r;
    codes[row * 16 + b] = (uint8_t)code;
    if (ucnt) {
      if (direct) atomicAdd(&ucnt[b * 256 + code], 1u);
      else if constexpr (!DIRECT) atomicAdd(&s_cnt[b * 256 + code], 1u);
    }
    uint32_t* rec = reinterpret_cast<uint32_t*>(records + row * 128);
    rec[b] = nib;
    reinterpret_cast<float*>(rec)[16 + b] = w;
    nsq += __uint_as_float(dpp_xor<8>(__float_as_uint(nsq)));
    nsq += __uint_as_float(dpp_xor<4>(__float_as_uint(nsq)));
    nsq += __uint_as_float(dpp_xor<2>(__float_as_uint(nsq)));
    nsq += __uint_as_float(dpp_xor<1>(__float_as_uint(nsq)));
    if (b == 0) norms[row] = sqrt_rn(nsq);
  }
  if constexpr (!DIRECT) {
    if (ucnt && !direct) {                  // keys per (subspace, centroid)
      __syncthreads();
      for (int i = tid; i < NSUB * 256; i += NT)
        if (s_cnt[i]) atomicAdd(&ucnt[i], s_cnt[i]);
    }
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
encode_kernel(EncodeArgs<KT> a, Tables tb) {
  encode_body<KT, 256, false>(a, tb, blockIdx.x);
}

// ===========================================================================
// qprep: query rotation and centroid activation (README "2. Decode";
// Slides Eqs. (5)-(6), Eq. (15) tiers).
//
// QP_WAVES waves per workgroup and NSUB / QP_WAVES workgroups per query head:
// wave 0 of each rotates the query (s-flip, then a 128-point fast
// Walsh-Hadamard transform with butterfly stages h = 1, 2, ..., 64), then each
// wave owns one subspace (one wave per SIMD, so the scalar ballot loops of the
// subspaces run side by side instead of sharing an issue slot).  Centroid c's score is
// sum_j (bit_j(c) ? +y_j : -y_j) in fp32, sequential in j.  The centroids
// ranking r < tier_top[last] by (score desc, c asc) are found with a bitwise
// threshold search over the order-preserving score keys, then ranked among
// themselves; each gets its tier weight, every other centroid 0.  The weight is
// written as byte g (query head g of the unit) of the unit's LUT; bytes of
// absent heads (g >= group) are written as 0.
// ===========================================================================
// Bitonic sort of one u32 per lane over the wave, descending (lane 0 ends
// with the largest): stage (K, J) compare-exchanges lanes l and l ^ J; blocks
// of K lanes with (l & K) == 0 keep the larger value at the lower lane.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic64_step(uint32_t v, int lane) {
  const uint32_t p = lane_xor<J>(v, lane);
  const bool keep_max = ((lane & K) == 0) == ((lane & J) == 0);
  const uint32_t hi = v > p ? v : p, lo = v > p ? p : v;
  return keep_max ? hi : lo;
}
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic64_j(uint32_t v, int lane) {
  v = bitonic64_step<K, J>(v, lane);
  if constexpr (J > 1) return bitonic64_j<K, J / 2>(v, lane);
  else return v;
}
template <int K>
__device__ __forceinline__ uint32_t bitonic64_k(uint32_t v, int lane) {
  v = bitonic64_j<K, K / 2>(v, lane);
  if constexpr (K < 64) return bitonic64_k<K * 2>(v, lane);
  else return v;
}

// Rank tiers of one subspace (one wave, centroid c = lane + 64 r holds score
// key key[r]) when the last tier ends at T <= 64: the T-th largest of the 64
// per-lane maxima is a lower bound of the T-th largest key (at least T keys
// reach it), so only keys at or above it can rank below T.  Those (typically
// a few dozen) are compacted as (score key << 32 | 255 - c), which orders by
// (score desc, c asc), and ranked among themselves; each centroid ranked
// below T gets its tier weight in lw[c].
__device__ __forceinline__ void rank_tiers_bound(const uint32_t (&key)[4], const TierSpec& tiers, uint64_t* sel,
                                                 uint8_t* lw, int lane) {
  const int T = tiers.top[tiers.n_tiers - 1];
  uint32_t m = key[0] > key[1] ? key[0] : key[1];
  m = m > key[2] ? m : key[2];
  m = m > key[3] ? m : key[3];
  const uint32_t sorted = bitonic64_k<2>(m, lane);
  const uint32_t bound = (uint32_t)__builtin_amdgcn_readlane((int)sorted, T - 1);   // T <= 64
  int cnt = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool take = key[r] >= bound;
    const uint64_t tm = __ballot(take);
    if (take) sel[cnt + (int)mbcnt(tm)] = ((uint64_t)key[r] << 32) | (uint64_t)(255 - (lane + 64 * r));
    cnt += __popcll(tm);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  for (int j = lane; j < cnt; j += 64) {
    const uint64_t e = sel[j];
    int rank = 0;
    for (int j2 = 0; j2 < cnt; ++j2) rank += (sel[j2] > e) ? 1 : 0;
    lw[255 - (int)(e & 0xFFu)] = (uint8_t)tier_weight_of(tiers, rank);   // rank >= T: weight 0, as the cleared entry
  }
}

// Rank tiers of one subspace (one wave, centroid c = lane + 64 r holds score
// key key[r]): the centroids ranked r < tiers.top[last] by (score desc, c asc)
// are found with a bitwise threshold search over the score keys, then ranked
// among themselves; each gets its tier weight in lw[c].  (rank_tiers_bound
// is used when the last tier ends within 64.)
__device__ __forceinline__ void rank_tiers(const uint32_t (&key)[4], const TierSpec& tiers, uint64_t* sel,
                                           uint8_t* lw, int lane) {
  const int T = tiers.top[tiers.n_tiers - 1];
  auto count_ge = [&](uint32_t x) {
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) cnt += __popcll(__ballot(key[r] >= x));
    return cnt;
  };
  // threshold key: the T-th largest score key among the 256 centroids, the
  // largest x with at least T keys >= x, built from the top bit down.  When
  // at least T keys share the sign and exponent bits of the largest key, the
  // threshold shares them too and the search starts below them.
  uint32_t kmax = key[0] > key[1] ? key[0] : key[1];
  kmax = kmax > key[2] ? kmax : key[2];
  kmax = kmax > key[3] ? kmax : key[3];
  kmax = xor_butterfly_u(kmax, lane, MaxU());
  const uint32_t top9 = (uint32_t)__builtin_amdgcn_readfirstlane((int)kmax) & 0xFF800000u;   // wave-uniform
  uint32_t thr = top9;
  if (count_ge(top9) < T) {
    thr = 0;
    for (int bit = 31; bit >= 23; --bit) {
      const uint32_t cand = thr | (1u << bit);
      if (count_ge(cand) >= T) thr = cand;
    }
  }
#pragma unroll
  for (int bit = 22; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    if (count_ge(cand) >= T) thr = cand;
  }
  int n_gt = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) n_gt += __popcll(__ballot(key[r] > thr));
  const int need_eq = T - n_gt;
  // compact the T selected centroids (ties at thr: lowest centroid index
  // first) as (score key << 32 | 255 - c): the larger value ranks first
  int eq_before = 0, sel_before = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t eqm = __ballot(key[r] == thr);
    const int eqrank = eq_before + (int)mbcnt(eqm);
    const bool sl = key[r] > thr || (key[r] == thr && eqrank < need_eq);
    const uint64_t sm = __ballot(sl);
    if (sl) sel[sel_before + (int)mbcnt(sm)] = ((uint64_t)key[r] << 32) | (uint64_t)(255 - (lane + 64 * r));
    eq_before += __popcll(eqm);
    sel_before += __popcll(sm);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // rank of each selected centroid = how many selected ones rank before it
  // (all packed values differ); tier weight by rank
  for (int j = lane; j < T; j += 64) {
    const uint64_t e = sel[j];
    int rank = 0;
#pragma unroll 16
    for (int j2 = 0; j2 < T; ++j2) rank += (sel[j2] > e) ? 1 : 0;
    lw[255 - (int)(e & 0xFFu)] = (uint8_t)tier_weight_of(tiers, rank);
  }
}

// Bitonic sort, descending, of 256 values over a wave: position x = 4 lane + r
// holds v[r].  Stage (K, J) compare-exchanges positions x and x ^ J (in the
// lane for J < 4, else with lane l ^ J / 4); blocks of K with (x & K) == 0
// keep the larger value at the lower position.
// Each value is kept or replaced by its partner: one compare and two selects
// per value across lanes, one compare and four selects per pair in a lane.
template <int K, int J>
__device__ __forceinline__ void bitonic_step(uint64_t (&v)[4], int lane) {
  if constexpr (J >= 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint64_t pv = ((uint64_t)lane_xor<J / 4>((uint32_t)(v[r] >> 32), lane) << 32) |
                          (uint64_t)lane_xor<J / 4>((uint32_t)v[r], lane);
      const int x = 4 * lane + r;
      const bool want_max = ((x & K) == 0) == ((x & J) == 0);
      v[r] = ((pv > v[r]) == want_max) ? pv : v[r];
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if ((a & J) == 0) {                          // the pair (a, a | J); a is the lower position
        const int b = a | J;
        const bool desc = ((4 * lane + a) & K) == 0;
        const uint64_t va = v[a], vb = v[b];
        const bool sw = desc ? (vb > va) : (va > vb);
        v[a] = sw ? vb : va;
        v[b] = sw ? va : vb;
      }
    }
  }
}
template <int K, int J>
__device__ __forceinline__ void bitonic_j(uint64_t (&v)[4], int lane) {
  bitonic_step<K, J>(v, lane);
  if constexpr (J > 1) bitonic_j<K, J / 2>(v, lane);
}
template <int K>
__device__ __forceinline__ void bitonic_k(uint64_t (&v)[4], int lane) {
  bitonic_j<K, K / 2>(v, lane);
  if constexpr (K < 256) bitonic_k<K * 2>(v, lane);
}

// Percentile tiers of one subspace (Slides Sec. 4.2.2, Eq. (15)): the 256
// centroids are sorted by (score desc, c asc) with a bitonic network over the
// wave (position x = 4 lane + r), their key counts are prefix-summed in that
// order, and a centroid whose first key sits at position P < keep_m gets the
// bonus 6 - floor(6 P / keep_m) (tiers 0..5 -> 6..1) in lw[c].  cnt holds
// the counts of centroids lane + 64 r, loaded before the scores were known;
// they go through the wave's LDS row s_cnt once the sort is done.
__device__ __forceinline__ void percentile_tiers(const uint32_t (&key)[4], const uint32_t (&cnt)[4],
                                                 uint32_t* s_cnt, uint32_t keep_m, uint8_t* lw, int lane) {
  uint64_t v[4];                                  // (score key, 255 - c): larger = earlier
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = ((uint64_t)key[r] << 8) | (uint64_t)(255u - (uint32_t)(lane + 64 * r));
  bitonic_k<2>(v, lane);
#pragma unroll
  for (int r = 0; r < 4; ++r) s_cnt[lane + 64 * r] = cnt[r];
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  uint32_t c[4], nk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    c[r] = 255u - (uint32_t)(v[r] & 0xFFu);
    nk[r] = s_cnt[c[r]];
  }
  const uint32_t tot = nk[0] + nk[1] + nk[2] + nk[3];
  const uint32_t incl = wave_incl_scan(tot);     // keys in this and lower lanes
  uint32_t first = incl - tot;                    // keys in better-ranked centroids
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (first < keep_m) lw[c[r]] = (uint8_t)(6u - (uint32_t)(((uint64_t)first * 6u) / keep_m));
    first += nk[r];
  }
}

// one butterfly stage of the query's Walsh-Hadamard transform: lanes l and
// l ^ H exchange; the lower one keeps the sum, the upper the difference
template <int H>
__device__ __forceinline__ void fwht_stage(float& v0, float& v1, int lane) {
  const bool upper = (lane & H) != 0;
  const float p0 = lane_xor_f<H>(v0, lane), p1 = lane_xor_f<H>(v1, lane);
  v0 = upper ? (p0 - v0) : (v0 + p0);
  v1 = upper ? (p1 - v1) : (v1 + p1);
}

// The unnormalised rotation y = H (s * q) of one query head by one wave: lane l
// ends with coordinates l (v0) and l + 64 (v1).  Butterflies h = 1..32 pair
// lanes l and l ^ h, h = 64 pairs the two registers.
template <typename QT>
__device__ __forceinline__ void rotate_query(const QT* __restrict__ qh, const Tables& tb, int lane, float& v0,
                                             float& v1) {
  if constexpr (sizeof(QT) == 2) {
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(qh);
    v0 = __uint_as_float((uint32_t)q16[lane] << 16);
    v1 = __uint_as_float((uint32_t)q16[lane + 64] << 16);
  } else {
    v0 = qh[lane];
    v1 = qh[lane + 64];
  }
  v0 = __uint_as_float(__float_as_uint(v0) ^ (((tb.neg_bits[lane >> 5] >> (lane & 31)) & 1u) << 31));
  v1 = __uint_as_float(__float_as_uint(v1) ^ (((tb.neg_bits[2 + (lane >> 5)] >> (lane & 31)) & 1u) << 31));
  fwht_stage<1>(v0, v1, lane);
  fwht_stage<2>(v0, v1, lane);
  fwht_stage<4>(v0, v1, lane);
  fwht_stage<8>(v0, v1, lane);
  fwht_stage<16>(v0, v1, lane);
  fwht_stage<32>(v0, v1, lane);
  const float a0 = v0, a1 = v1;
  v0 = a0 + a1;
  v1 = a0 - a1;
}

// Centroid score keys of subspace b (yb: its 8 rotated coordinates): centroid
// c = lane + 64 r scores sum_j (bit_j(c) ? +y_j : -y_j), sequential in j.
__device__ __forceinline__ void centroid_keys(const float (&yb)[SUBD], int lane, uint32_t (&key)[4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t c = lane + 64 * r;
    float sc = (c & 1u) ? yb[0] : -yb[0];
#pragma unroll
    for (int j = 1; j < SUBD; ++j) sc = sc + (((c >> j) & 1u) ? yb[j] : -yb[j]);
    key[r] = orderable(sc);
  }
}

constexpr int QP_WAVES = 2;
constexpr int QP_PARTS = NSUB / QP_WAVES;   // workgroups per query head

template <typename QT>
struct QprepArgs {
  const QT* q;
  int n_q_heads, n_kv_heads, group;
  float* rot_q;
  uint8_t* lut_bytes;
  const uint32_t* counts;  // percentile tiers
  uint32_t keep_m;         // percentile tiers: kept positions M (0: rank tiers)
  uint32_t* unit_tot;      // nullable: bin totals cleared for the collide kernel
};

template <typename QT>
__device__ __forceinline__ void qprep_body(const QprepArgs<QT>& a, const Tables& tb, const TierSpec& tiers,
                                           int block) {
  __shared__ float y[D];
  __shared__ uint64_t sel[QP_WAVES][256];   // (score key, 255 - centroid) of the selected centroids
  __shared__ uint8_t lw[QP_WAVES][256];     // tier weight per centroid
  __shared__ uint32_t s_cnt[QP_WAVES][256]; // percentile tiers: centroid key counts

  const QT* __restrict__ q = a.q;
  const int n_q_heads = a.n_q_heads, n_kv_heads = a.n_kv_heads, group = a.group;
  float* __restrict__ rot_q = a.rot_q;
  uint8_t* __restrict__ lut_bytes = a.lut_bytes;
  const uint32_t* __restrict__ counts = a.counts;
  const uint32_t keep_m = a.keep_m;
  uint32_t* __restrict__ unit_tot = a.unit_tot;
  const int head = block / QP_PARTS;        // sequence * n_q_heads + query head
  const int part = block - head * QP_PARTS;
  const int seq = head / n_q_heads, qh = head - seq * n_q_heads;
  const int unit = seq * n_kv_heads + qh / group, g = qh % group;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int b = part * QP_WAVES + w;        // subspace of this wave

  // percentile tiers: this subspace's centroid counts, requested first (they
  // do not depend on the query) and used after the centroid sort
  uint32_t cnt[4] = {0, 0, 0, 0};
  if (keep_m > 0) {
    const uint32_t* cr = counts + ((int64_t)unit * NSUB + b) * 256;
#pragma unroll
    for (int r = 0; r < 4; ++r) cnt[r] = cr[lane + 64 * r];
  }
  if (w == 0) {
    float v0, v1;
    rotate_query<QT>(q + (int64_t)head * D, tb, lane, v0, v1);
    y[lane] = v0;
    y[lane + 64] = v1;
    if (part == 0) {
      rot_q[(int64_t)head * D + lane] = v0 * tb.inv_sqrt_d;
      rot_q[(int64_t)head * D + lane + 64] = v1 * tb.inv_sqrt_d;
      // the collide kernel that follows adds this head's bin counts here
      if (unit_tot) {
        const int nb = keep_m > 0 ? NBIN_MAX : NBIN;
        unit_tot[((int64_t)unit * MAXG + g) * nb + lane] = 0u;
        if (keep_m > 0) unit_tot[((int64_t)unit * MAXG + g) * nb + 64 + lane] = 0u;
      }
    }
  }
  __syncthreads();

  float yb[SUBD];
#pragma unroll
  for (int j = 0; j < SUBD; ++j) yb[j] = y[b * SUBD + j];
  uint32_t key[4];
  centroid_keys(yb, lane, key);
#pragma unroll
  for (int r = 0; r < 4; ++r) lw[w][lane + 64 * r] = 0;

  if (keep_m > 0) {
    percentile_tiers(key, cnt, s_cnt[w], keep_m, lw[w], lane);
  } else if (tiers.top[tiers.n_tiers - 1] <= 64) {
    rank_tiers_bound(key, tiers, sel[w], lw[w], lane);
  } else {
    rank_tiers(key, tiers, sel[w], lw[w], lane);
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  // the last query head of a unit also clears the bytes of the absent heads
  // (g >= group), so the LUT needs no clearing between calls
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t c = lane + 64 * r;
    uint8_t* word = lut_bytes + (((int64_t)unit * NSUB + b) * 256 + c) * 4;
    word[g] = lw[w][c];
    if (g == group - 1)
      for (int g2 = group; g2 < MAXG; ++g2) word[g2] = 0;
  }
}

template <typename QT>
__global__ void __launch_bounds__(64 * QP_WAVES)
qprep_kernel(QprepArgs<QT> a, Tables tb, TierSpec tiers) {
  qprep_body<QT>(a, tb, tiers, blockIdx.x);
}

// One decode step's appended keys and the query preparation in one launch:
// workgroups [0, qprep_blocks) run qprep, the rest encode the new rows (at
// most ENC_DIRECT per unit).  The two touch disjoint data with rank tiers
// (qprep reads no centroid counts), so nothing orders them.
template <typename QT, typename KT>
__global__ void __launch_bounds__(64 * QP_WAVES)
append_qprep_kernel(QprepArgs<QT> qa, EncodeArgs<KT> ea, Tables tb, TierSpec tiers, int qprep_blocks) {
  if ((int)blockIdx.x < qprep_blocks) qprep_body<QT>(qa, tb, tiers, blockIdx.x);
  else encode_body<KT, 64 * QP_WAVES, true>(ea, tb, blockIdx.x - qprep_blocks);
}


// ===========================================================================
// collide: tier-weighted collision votes (Slides Eq. (15), Sec. 4.2.2;
// README "2. Decode"), per-sub-tile suffix counts of the scores and the
// unit's score histogram.
//
// Workgroup = (unit, tile of `tile` keys).  The unit's LUT (16 x 256 u32, byte
// g = weight for query head g) sits in LDS; a key's 16 code bytes index it
// and the 16 words are summed: four 8-bit lanes of at most 96 never carry, so
// one u32 add serves all query heads of the KV head.  S is stored packed.
// Wave w scores the w-th quarter ("sub-tile") of the tile.  Histogram bins
// 1..NB (64 with rank tiers, 128 with percentile tiers) are counted in LDS words of HIST_LANES per (head, bin): lanes l and
// l + 32 share a word, and byte w of it belongs to wave w (a byte counts at
// most 2 * keys per lane <= 128), which gives one histogram per sub-tile; bin
// 0 is implied by the sub-tile length.  Each lane keeps COLLIDE_UNROLL code
// loads in flight.
// ===========================================================================
constexpr int COLLIDE_UNROLL = 4;
constexpr int HIST_LANES = 32;

// (unit, tile) of workgroup i of a units x tiles grid.  Workgroups are dealt
// to the 8 XCDs in turn; when the units split evenly over them, all tiles of
// one unit run on one XCD (its LUT and histograms then share that L2).
__device__ __forceinline__ void xcd_unit_tile(int i, int units, int tiles, int& unit, int& tl) {
  if (units % 8 == 0) {
    const int slot = i / 8;
    unit = i % 8 + 8 * (slot / tiles);
    tl = slot % tiles;
  } else {
    unit = i / tiles;
    tl = i - unit * tiles;
  }
}

// word of the suffix count #{S >= s} (s = 1..NB + 1; s = NB + 1 is always 0)
// of head g in sub-tile `sub` of a unit: rows of max_subs sub-tiles, a unit
// holds MAXG * (NB + 1) rows
template <int NB>
__device__ __forceinline__ int64_t suf_index(int64_t unit, int max_subs, int g, int s, int sub) {
  return (((int64_t)unit * MAXG + g) * (NB + 1) + (s - 1)) * max_subs + sub;
}

template <int G, int NB>   // NB: histogram bins 1..NB
__global__ void __launch_bounds__(256)
collide_kernel(const uint4* __restrict__ codes, const uint32_t* __restrict__ lut,
               uint32_t* __restrict__ scores, uint32_t* __restrict__ tile_hist, uint32_t* __restrict__ unit_tot,
               int64_t n, int64_t n_cap, int64_t s_stride, int tiles, int max_subs, int tile) {
  constexpr int group = G;
  __shared__ uint32_t s_lut[NSUB * 256];
  __shared__ uint32_t s_hist[MAXG * NB * HIST_LANES];

  int unit, tl;
  xcd_unit_tile(blockIdx.x, gridDim.x / tiles, tiles, unit, tl);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wkeys = tile >> 2;                     // keys of this wave's sub-tile (multiple of 64)
  const int64_t w0 = (int64_t)tl * tile + (int64_t)wave * wkeys;
  const int64_t w1 = (w0 + wkeys < n) ? w0 + wkeys : n;
  const uint4* crow = codes + (int64_t)unit * n_cap;
  uint32_t* srow = scores + (int64_t)unit * s_stride;

  // Loads are issued unconditionally from a clamped index (lanes past the end
  // re-read the last key and discard it): conditional loads compile to
  // exec-masked blocks that serialise on the memory counter.
  const int64_t last = (w1 > w0) ? w1 - 1 : 0;
  // first batch of codes in flight while the tables are staged; the LUT is
  // requested all at once (a load-wait-store loop would wait once per part)
  uint4 c[COLLIDE_UNROLL];
#pragma unroll
  for (int u = 0; u < COLLIDE_UNROLL; ++u) {
    const int64_t i = w0 + (int64_t)u * 64 + lane;
    c[u] = crow[i < last ? i : last];
  }
  {
    constexpr int LUT_PER_THREAD = NSUB * 256 / 4 / 256;   // uint4 of the LUT per thread
    const uint4* src = reinterpret_cast<const uint4*>(lut + (int64_t)unit * NSUB * 256);
    uint4 lt[LUT_PER_THREAD];
#pragma unroll
    for (int k = 0; k < LUT_PER_THREAD; ++k) lt[k] = src[tid + 256 * k];
    uint4* h4 = reinterpret_cast<uint4*>(s_hist);
    for (int i = tid; i < group * NB * HIST_LANES / 4; i += 256) h4[i] = make_uint4(0, 0, 0, 0);
    uint4* dst = reinterpret_cast<uint4*>(s_lut);
#pragma unroll
    for (int k = 0; k < LUT_PER_THREAD; ++k) dst[tid + 256 * k] = lt[k];
  }
  __syncthreads();

  const uint32_t incr = 1u << (8 * wave);
  // bin s of head g lives at word (g * NB + s - 1) * HIST_LANES + lane % HIST_LANES
  const uint32_t hbase = (uint32_t)(lane & (HIST_LANES - 1)) * 4u - HIST_LANES * 4u;
  for (int64_t base = w0; base < w1; base += 64 * COLLIDE_UNROLL) {
    uint4 nx[COLLIDE_UNROLL];
    const int64_t nb = base + 64 * COLLIDE_UNROLL;
#pragma unroll
    for (int u = 0; u < COLLIDE_UNROLL; ++u) {
      const int64_t i = nb + (int64_t)u * 64 + lane;
      nx[u] = crow[i < last ? i : last];
    }
    // Every lane stores: a lane past the end holds the last key's codes, so it
    // rewrites that key's score with the same value.  Unconditional stores let
    // the wait for the next batch's loads leave this batch's stores in flight.
#pragma unroll
    for (int u = 0; u < COLLIDE_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * 64 + lane;
      const bool inb = i < w1;
      const uint32_t cw[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
      uint32_t acc = 0;
#pragma unroll
      for (int bb = 0; bb < NSUB; ++bb) acc += s_lut[bb * 256 + ((cw[bb >> 2] >> (8 * (bb & 3))) & 0xFFu)];
      srow[inb ? i : last] = acc;
      if (inb) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t sc = (acc >> (8 * g)) & 0xFFu;
          if (sc) atomicAdd(&s_hist[(g * NB * HIST_LANES * 4 + sc * HIST_LANES * 4 + hbase) >> 2], incr);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < COLLIDE_UNROLL; ++u) c[u] = nx[u];
  }
  __syncthreads();

  // Byte w of a counter word belongs to wave w.  Each sub-tile publishes its
  // suffix counts #{S >= s} (suf_index layout) and the bin counts are added to
  // the unit's totals, from which every select workgroup derives its
  // parameters.  Thread (g, s - 1) owns bin s of head g: a wave holds 64 bins
  // of one head, and with 128 bins the lower half adds the totals of the
  // upper half (the next wave).  The LUT's LDS words carry the upper halves'
  // totals (no lookup is left after the barrier above; a separate array
  // would take the 128-bin kernel past two workgroups per CU).
  uint32_t* s_upper = s_lut;
  for (int b0 = 0; b0 < group * NB; b0 += 256) {   // uniform; a wave is active or not as a whole
    const int gb = b0 + tid;
    const bool act = gb < group * NB;
    const int g = gb / NB, bin = gb % NB;
    uint32_t s01 = 0, s23 = 0, c = 0;
    if (act) {
      // the row's words four at a time, from a start rotated by thread
      // (neighbouring threads read neighbouring rows)
      const uint4* row = reinterpret_cast<const uint4*>(s_hist + (g * NB + bin) * HIST_LANES);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < HIST_LANES / 4; ++i) {
        const uint4 v = row[(i + tid) & (HIST_LANES / 4 - 1)];
        lo += (v.x & 0x00FF00FFu) + (v.y & 0x00FF00FFu) + (v.z & 0x00FF00FFu) + (v.w & 0x00FF00FFu);   // waves 0, 2
        hi += ((v.x >> 8) & 0x00FF00FFu) + ((v.y >> 8) & 0x00FF00FFu) + ((v.z >> 8) & 0x00FF00FFu) +
              ((v.w >> 8) & 0x00FF00FFu);                                                              // waves 1, 3
      }
      const uint32_t cnt[4] = {lo & 0xFFFFu, hi & 0xFFFFu, lo >> 16, hi >> 16};
      c = cnt[0] + cnt[1] + cnt[2] + cnt[3];
      // 16-bit fields: sub-tiles 0 and 1 in c01, 2 and 3 in c23 (counts <= tile / 4 < 2^16)
      const uint32_t c01 = cnt[0] | (cnt[1] << 16), c23 = cnt[2] | (cnt[3] << 16);
      const uint32_t i01 = wave_incl_scan(c01), i23 = wave_incl_scan(c23);
      const uint32_t t01 = (uint32_t)__builtin_amdgcn_readlane((int)i01, 63);
      const uint32_t t23 = (uint32_t)__builtin_amdgcn_readlane((int)i23, 63);
      s01 = t01 - i01 + c01;             // #{S >= bin + 1} among this wave's bins
      s23 = t23 - i23 + c23;
      if (NB > 64 && lane == 0) {
        s_upper[2 * wave] = t01;
        s_upper[2 * wave + 1] = t23;
      }
    }
    if constexpr (NB > 64) {
      static_assert(NB == 128, "64 or 128 bins");
      __syncthreads();
      if (act && bin < 64) {
        s01 += s_upper[2 * wave + 2];
        s23 += s_upper[2 * wave + 3];
      }
      __syncthreads();
    }
    if (act) {
      *reinterpret_cast<uint4*>(tile_hist + suf_index<NB>(unit, max_subs, g, bin + 1, 4 * tl)) =
          make_uint4(s01 & 0xFFFFu, s01 >> 16, s23 & 0xFFFFu, s23 >> 16);
      if (bin == 0)   // #{S >= NB + 1} = 0
        *reinterpret_cast<uint4*>(tile_hist + suf_index<NB>(unit, max_subs, g, NB + 1, 4 * tl)) = make_uint4(0, 0, 0, 0);
      if (c) atomicAdd(&unit_tot[((int64_t)unit * MAXG + g) * NB + bin], c);
    }
  }
}

// ===========================================================================
// streaming copy, 16 bytes per lane per access (traffic-counter calibration)
// ===========================================================================
__global__ void __launch_bounds__(256) copy16_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                     size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// ===========================================================================
// select: the candidate set of every query head (Slides Sec. 4.2.2: keep the
// top-beta keys by S_i, chosen by histogram + prefix scan instead of a sort;
// Sec. 4.3: C = ceil(beta n)).
//
// Workgroup = (unit, tile), same tiling as collide; wave w owns sub-tile w and
// starts from the counts of earlier keys above / at theta, which it derives
// from the unit's bin totals and the earlier sub-tiles' suffix counts (both
// written by collide).  A key is a candidate of head g iff S > theta, or S ==
// theta and fewer than need_eq keys with S == theta precede it; its slot is
// (#gt before) + min(#eq before, need_eq), which lists candidates in ascending
// key order.  Byte-parallel compares of the packed scores against all heads'
// theta find the keys at or above some head's theta; only those (about a
// tenth of the keys) are compacted, in key order, for the per-head ballots,
// since every other key leaves all counts unchanged.  A head whose need_eq
// keys at theta all lie before the sub-tile compares against theta + 1 there:
// its keys at theta can no longer be taken, and its slots only count keys
// above theta.
// ===========================================================================
constexpr int SEL_GRP = 16;             // score chunks per group
constexpr int SEL_MAXGRP = 4;           // groups of the largest sub-tile (64 chunks of 64 keys)
constexpr int SEL_QCAP = 2 * SEL_GRP * 64;    // compaction queue per wave (2 groups)

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// theta and need_eq of one query head from its bin totals (tot[h] at lane l:
// the count of keys with S = 64 h + l + 1 among the unit's n keys): theta =
// the highest score whose suffix count #{S >= theta} reaches C (0: every key
// is taken); need_eq = how many keys with S == theta are taken.
template <int NB>
__device__ __forceinline__ void theta_from_totals(const uint32_t (&tot)[NB / 64], int64_t n, int n_candidates,
                                                  int& theta, uint32_t& need_eq) {
  constexpr int H = NB / 64;
  uint32_t suf[H];                                   // suf[h] at lane l: #{S >= 64 h + l + 1}
  uint32_t above = 0;                                // keys in the higher halves
#pragma unroll
  for (int h = H - 1; h >= 0; --h) {
    const uint32_t incl = wave_incl_scan(tot[h]);
    const uint32_t all = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    suf[h] = all - incl + tot[h] + above;
    above += all;
  }
  theta = 0;
  uint32_t n_gt = above, eq_tot = (uint32_t)(n - above);   // theta 0: every key with S >= 1 is above
#pragma unroll
  for (int h = 0; h < H; ++h) {                      // a higher half overrides a lower one
    const uint64_t ge = __ballot(suf[h] >= (uint32_t)n_candidates);
    if (ge) {
      const int top = 63 - __builtin_clzll(ge);
      theta = 64 * h + top + 1;
      if (top < 63) n_gt = (uint32_t)__builtin_amdgcn_readlane((int)suf[h], top + 1);
      else n_gt = (h + 1 < H) ? (uint32_t)__builtin_amdgcn_readlane((int)suf[h + 1 < H ? h + 1 : h], 0) : 0u;
      eq_tot = (uint32_t)__builtin_amdgcn_readlane((int)tot[h], top);
    }
  }
  const uint32_t want = (uint32_t)n_candidates - n_gt;
  need_eq = want < eq_tot ? want : eq_tot;
}

// the bin totals of head g for theta_from_totals
template <int NB>
__device__ __forceinline__ void load_totals(const uint32_t* __restrict__ unit_tot, int unit, int g, int lane,
                                            uint32_t (&tot)[NB / 64]) {
#pragma unroll
  for (int h = 0; h < NB / 64; ++h) tot[h] = unit_tot[((int64_t)unit * MAXG + g) * NB + 64 * h + lane];
}

// chunks of 64 sub-tiles' suffix counts requested together when selection
// parameters need the counts of more than 64 earlier sub-tiles
constexpr int PFX_CH = 4;

// Selection parameters of query head g (wave g) for the sub-tiles 4 tl ..
// 4 tl + 3 of one select workgroup, from the unit's bin totals (tot at lane
// l: keys with S = l + 1) and the sub-tiles' suffix counts: theta / need_eq as
// theta_from_totals, then the keys above / at theta in every earlier
// sub-tile, 64 sub-tiles (one per lane) per chunk.  Results go to s_par[g] =
// (theta, need_eq) and s_base[w][g] = (#gt, #eq) before sub-tile 4 tl + w.
template <int NB>
__device__ __forceinline__ void select_params_suffix(const uint32_t (&tot)[NB / 64], const uint32_t* __restrict__ suf, int unit,
                                                     int max_subs, int sub_len, int64_t n, int tl, int g,
                                                     int n_candidates, int lane, int2* s_par,
                                                     int2 (*s_base)[MAXG]) {
  int theta;
  uint32_t need_eq;
  theta_from_totals<NB>(tot, n, n_candidates, theta, need_eq);
  const uint32_t* row_gt = suf + suf_index<NB>(unit, max_subs, g, theta + 1, 0);             // #{S > theta}
  const uint32_t* row_ge = suf + suf_index<NB>(unit, max_subs, g, theta > 0 ? theta : 1, 0);  // #{S >= theta}
  const int first = 4 * tl;
  int pre_gt = 0, pre_eq = 0;
  int in_gt[4] = {0, 0, 0, 0}, in_eq[4] = {0, 0, 0, 0};
  // chunks of 64 sub-tiles (one per lane), PFX_CH chunks requested together
  for (int c00 = 0; c00 < first + 4; c00 += 64 * PFX_CH) {   // uniform
    int gtv[PFX_CH], gev[PFX_CH];
#pragma unroll
    for (int c = 0; c < PFX_CH; ++c) {
      const int sub = c00 + 64 * c + lane;
      gtv[c] = 0;
      gev[c] = 0;
      if (sub < first + 4) {
        gtv[c] = (int)row_gt[sub];
        if (theta > 0) gev[c] = (int)row_ge[sub];
      }
    }
#pragma unroll
    for (int c = 0; c < PFX_CH; ++c) {
      const int c0 = c00 + 64 * c;
      if (c0 >= first + 4) break;                 // uniform
      const int sub = c0 + lane;
      int gt = 0, eq = 0;
      if (sub < first + 4) {
        gt = gtv[c];
        int ge;
        if (theta > 0) {
          ge = gev[c];
        } else {                                  // every key has S >= 0
          int64_t len = n - (int64_t)sub * sub_len;
          ge = (int)(len < 0 ? 0 : (len > sub_len ? sub_len : len));
        }
        eq = ge - gt;
      }
      const bool before = sub < first;
      pre_gt += (int)xor_butterfly_u(before ? (uint32_t)gt : 0u, lane, AddU());
      pre_eq += (int)xor_butterfly_u(before ? (uint32_t)eq : 0u, lane, AddU());
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int sw = first + w - c0;            // uniform
        if (sw >= 0 && sw < 64) {
          in_gt[w] = __builtin_amdgcn_readlane(gt, sw);
          in_eq[w] = __builtin_amdgcn_readlane(eq, sw);
        }
      }
    }
  }
  if (lane == 0) {
    s_par[g] = make_int2(theta, (int)need_eq);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s_base[w][g] = make_int2(pre_gt, pre_eq);
      pre_gt += in_gt[w];
      pre_eq += in_eq[w];
    }
  }
}

// Per-head selection state of one wave walking its keys in ascending order:
// theta, need_eq and the counts of keys above / at theta seen so far (the
// keys before the wave's first one included).  A key is a candidate of head g
// iff S > theta, or S == theta and fewer than need_eq keys with S == theta
// precede it; its slot is (#gt before) + min(#eq before, need_eq), so the list
// is in ascending key order.  Four heads' scores are the bytes of one u32 and
// are compared at once.
template <int G>
struct HeadSelect {
  int need[G], run_gt[G], run_eq[G];
  uint32_t th4 = 0x7F7F7F7Fu;     // absent heads: theta 127, never reached
  uint32_t thp4 = 0;              // theta + 1 per byte
  // compaction thresholds: theta, or theta + 1 for a head whose keys at theta
  // are all taken before the wave's keys (they can no longer be candidates)
  uint32_t thf4 = 0x7F7F7F7Fu;

  __device__ __forceinline__ void set(int g, int theta, int need_eq, int gt_before, int eq_before) {
    need[g] = need_eq;
    run_gt[g] = gt_before;
    run_eq[g] = eq_before;
    th4 = (th4 & ~(0xFFu << (8 * g))) | ((uint32_t)theta << (8 * g));
    thf4 = (thf4 & ~(0xFFu << (8 * g))) | ((uint32_t)(eq_before >= need_eq ? theta + 1 : theta) << (8 * g));
  }
  __device__ __forceinline__ void finish() { thp4 = th4 + 0x01010101u; }   // <= 128 per byte: no carry

  // nonzero iff some head may take a key with packed scores s
  __device__ __forceinline__ uint32_t interesting(uint32_t s) const { return ((s | 0x80808080u) - thf4) & 0x80808080u; }

  // the compacted keys e[0 .. cnt) of the wave, one per lane (cnt <= 64):
  // per-head ballots give each taken key its slot
  __device__ __forceinline__ void batch(uint2 e, bool valid, int32_t* __restrict__ cand_idx, int64_t qhead0,
                                        int n_candidates, uint32_t* err) {
    const uint32_t m = e.y | 0x80808080u;
    const uint32_t gt4 = (m - thp4) & 0x80808080u;
    const uint32_t eq4 = ((m - th4) & 0x80808080u) ^ gt4;
    bool over = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool isgt = valid && ((gt4 >> (8 * g + 7)) & 1u);
      const bool iseq = valid && ((eq4 >> (8 * g + 7)) & 1u);
      const uint64_t gtm = __ballot(isgt), eqm = __ballot(iseq);
      const int gt_before = run_gt[g] + (int)mbcnt(gtm);
      const int eq_before = run_eq[g] + (int)mbcnt(eqm);
      const bool sel = isgt || (iseq && eq_before < need[g]);
      const int pos = gt_before + (eq_before < need[g] ? eq_before : need[g]);
      if (sel && pos < n_candidates)              // pos < C whenever the parameters match S
        cand_idx[(qhead0 + g) * n_candidates + pos] = (int)e.x;
      over = over || (sel && pos >= n_candidates);
      run_gt[g] += __popcll(gtm);
      run_eq[g] += __popcll(eqm);
    }
    if (over && err) atomicOr(err, PK_DEV_ERR_SLOT);
  }
};

// Each workgroup derives the parameters itself from the unit's bin totals
// and the sub-tiles' suffix counts (select_params_suffix; NB: bins 1..NB).
// The tiles of one unit share an XCD where they can (xcd_unit_tile), so the
// unit's counts are fetched into its L2 once.
template <int G, int NB>
__global__ void __launch_bounds__(256)
select_kernel(const uint32_t* __restrict__ scores, int32_t* __restrict__ cand_idx, int64_t n, int64_t s_stride,
              int tiles, int max_subs, int tile, int n_q_heads, int n_kv_heads, int n_candidates,
              const uint32_t* __restrict__ unit_tot, const uint32_t* __restrict__ suf, uint32_t* __restrict__ err) {
  __shared__ uint2 s_ik[4][SEL_QCAP];             // compacted keys: (key, packed S)
  __shared__ int2 s_par[MAXG];
  __shared__ int2 s_base[4][MAXG];

  int unit, tl;
  xcd_unit_tile(blockIdx.x, gridDim.x / tiles, tiles, unit, tl);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seq = unit / n_kv_heads, kvh = unit - seq * n_kv_heads;
  const int64_t qhead0 = (int64_t)seq * n_q_heads + kvh * G;
  // key indices fit in 32 bits (n <= n_capacity < 2^31)
  const int k0 = tl * tile;
  const int k1 = ((int64_t)k0 + tile < n) ? k0 + tile : (int)n;
  const int wkeys = tile >> 2;                    // multiple of 64
  const int w0 = k0 + wave * wkeys;
  const int w1 = (w0 + wkeys < k1) ? w0 + wkeys : k1;
  const uint32_t* srow = scores + (int64_t)unit * s_stride;

  // the head's bin totals are requested before the scores, so that waiting
  // for them does not wait for the scores (the memory counter is in order)
  uint32_t tot[NB / 64] = {};
  if (wave < G) load_totals<NB>(unit_tot, unit, wave, lane, tot);

  // packed scores of keys w0 + r*64 + lane, in groups of SEL_GRP chunks
  // (clamped, unconditional loads; the next group is in flight while one is used)
  const int last = (w1 > w0) ? w1 - 1 : 0;
  uint32_t sp[SEL_GRP];
#pragma unroll
  for (int r = 0; r < SEL_GRP; ++r) {
    const int i = w0 + r * 64 + lane;
    sp[r] = srow[i < last ? i : last];
  }
  HeadSelect<G> hs;
  // per head: theta, need_eq, and the counts of keys above / at theta before
  // this wave's sub-tile
  auto setup = [&]() __attribute__((always_inline)) {
    if (wave < G)
      select_params_suffix<NB>(tot, suf, unit, max_subs, tile >> 2, n, tl, wave, n_candidates, lane, s_par, s_base);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int2 pr = s_par[g], sb2 = s_base[wave][g];
      hs.set(g, pr.x, pr.y, sb2.x, sb2.y);
    }
    hs.finish();
  };
  setup();        // behind the first group's loads; the other groups are requested after it
  uint2* ik = s_ik[wave];
  int nk = 0;

  auto select_batch = [&](int b0, int cnt) {
    const bool valid = lane < cnt;
    hs.batch(ik[b0 + (valid ? lane : 0)], valid, cand_idx, qhead0, n_candidates, err);
  };

  // Every group of the sub-tile is loaded before the first is compacted, and
  // no global store is issued until all of them have been compacted (a store
  // inside a loop would make the wave wait for every load in flight).  The
  // per-head ballots then run over the queued keys in batches of 64; a queue
  // that could overflow is drained between groups.
  auto load_group = [&](int grp, uint32_t (&dst)[SEL_GRP]) {
#pragma unroll
    for (int r = 0; r < SEL_GRP; ++r) {
      const int i = w0 + (grp * SEL_GRP + r) * 64 + lane;
      dst[r] = srow[i < last ? i : last];
    }
  };
  auto compact_group = [&](int grp, const uint32_t (&src)[SEL_GRP]) {
#pragma unroll
    for (int r = 0; r < SEL_GRP; ++r) {
      const int i = w0 + (grp * SEL_GRP + r) * 64 + lane;
      const bool valid = i < w1;                  // false for the whole wave past its keys
      const bool interesting = valid && hs.interesting(src[r]) != 0u;
      const uint64_t im = __ballot(interesting);
      if (interesting) ik[nk + (int)mbcnt(im)] = make_uint2((uint32_t)i, src[r]);
      nk += __popcll(im);
    }
  };
  auto drain = [&]() {                            // whole batches; the remainder (< 64) moves to the front
    wave_lds_sync();
    int b0 = 0;
    for (; b0 + 64 <= nk; b0 += 64) select_batch(b0, 64);
    if (b0 > 0) {
      const int rem = nk - b0;
      uint2 e = make_uint2(0u, 0u);
      if (lane < rem) e = ik[b0 + lane];
      wave_lds_sync();
      if (lane < rem) ik[lane] = e;
      nk = rem;
    }
    wave_lds_sync();
  };
  // NG groups are loaded unconditionally (clamped addresses; groups past the
  // sub-tile hold no valid key), which keeps the loads ahead of their use
  auto run = [&](auto ng_tag) {
    constexpr int NG = decltype(ng_tag)::value;
    uint32_t sg[NG > 1 ? NG - 1 : 1][SEL_GRP];
#pragma unroll
    for (int g = 1; g < NG; ++g) load_group(g, sg[g - 1]);
    compact_group(0, sp);
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      if (nk > SEL_QCAP - SEL_GRP * 64) drain();
      compact_group(g, sg[g - 1]);
    }
    drain();
  };
  const int ngrp = (wkeys / 64 + SEL_GRP - 1) / SEL_GRP;
  if (ngrp <= 1) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, SEL_MAXGRP>{});
  select_batch(0, nk);
}

// ===========================================================================
// select, one workgroup per sub-tile (the collide kernel's per-wave key
// range): the candidate set of every query head (Slides Sec. 4.2.2).
//
// The sub-tile's rows of 64 keys are split over the four waves (ROWS rows
// each at most).  The keys above / at theta before the sub-tile come from
// the unit's bin totals and the sub-tiles' suffix counts; the waves' own
// prefixes inside the sub-tile
// from byte-parallel counts of their registers.  Then each wave compacts its
// keys at or above some head's theta and gives them their slots
// (HeadSelect), as select_kernel does.  Four times as many workgroups as
// select_kernel keep more waves per compute unit to overlap the score loads
// with the slot ballots.
// ===========================================================================
constexpr int SS_DRAIN_ROWS = 8;                          // rows compacted between queue drains
constexpr int SS_QCAP = SS_DRAIN_ROWS * 64 + 64;          // queue entries per wave

// The selection parameters of head g (wave g) in two parts, so that the
// wave's score rows can be counted in between.  select_theta_sub: theta /
// need_eq from the unit's bin totals (to s_par[g]), and requests for the
// suffix counts of up to 64 earlier sub-tiles (they arrive behind the score
// rows).  select_prefix_sub: the keys above / at theta in the sub-tiles before
// `sub` (to s_sb[g]), 64 sub-tiles per step.
struct SubPrefix {
  int theta = 0, gt0 = 0, ge0 = 0;
};

__device__ __forceinline__ int keys_in_sub(int64_t n, int t, int sub_len) {
  const int64_t len = n - (int64_t)t * sub_len;
  return (int)(len < 0 ? 0 : (len > sub_len ? sub_len : len));
}

template <int NB>
__device__ __forceinline__ SubPrefix select_theta_sub(const uint32_t (&tot)[NB / 64], const uint32_t* __restrict__ suf, int unit,
                                                      int max_subs, int sub_len, int64_t n, int sub, int g,
                                                      int n_candidates, int lane, int2* s_par) {
  SubPrefix sp;
  uint32_t need_eq;
  theta_from_totals<NB>(tot, n, n_candidates, sp.theta, need_eq);
  if (lane < sub) {
    sp.gt0 = (int)suf[suf_index<NB>(unit, max_subs, g, sp.theta + 1, lane)];                        // #{S > theta}
    sp.ge0 = sp.theta > 0 ? (int)suf[suf_index<NB>(unit, max_subs, g, sp.theta, lane)]              // #{S >= theta}
                          : keys_in_sub(n, lane, sub_len);                                      // every key
  }
  if (lane == 0) s_par[g] = make_int2(sp.theta, (int)need_eq);
  return sp;
}

template <int NB>
__device__ __forceinline__ void select_prefix_sub(const SubPrefix& sp, const uint32_t* __restrict__ suf, int unit,
                                                  int max_subs, int sub_len, int64_t n, int sub, int g, int lane,
                                                  int2* s_sb) {
  int pre_gt = (int)xor_butterfly_u((uint32_t)sp.gt0, lane, AddU());
  int pre_eq = (int)xor_butterfly_u((uint32_t)(sp.ge0 - sp.gt0), lane, AddU());
  // the later chunks of 64 sub-tiles, PFX_CH chunks requested together
  for (int c0 = 64; c0 < sub; c0 += 64 * PFX_CH) {   // uniform
    int gt[PFX_CH], ge[PFX_CH];
#pragma unroll
    for (int c = 0; c < PFX_CH; ++c) {
      const int t = c0 + 64 * c + lane;
      gt[c] = 0;
      ge[c] = 0;
      if (t < sub) {
        gt[c] = (int)suf[suf_index<NB>(unit, max_subs, g, sp.theta + 1, t)];
        ge[c] = sp.theta > 0 ? (int)suf[suf_index<NB>(unit, max_subs, g, sp.theta, t)] : keys_in_sub(n, t, sub_len);
      }
    }
#pragma unroll
    for (int c = 0; c < PFX_CH; ++c) {
      if (c0 + 64 * c >= sub) break;                // uniform
      pre_gt += (int)xor_butterfly_u((uint32_t)gt[c], lane, AddU());
      pre_eq += (int)xor_butterfly_u((uint32_t)(ge[c] - gt[c]), lane, AddU());
    }
  }
  if (lane == 0) s_sb[g] = make_int2(pre_gt, pre_eq);
}

template <int G, int NB, int ROWS>
__global__ void __launch_bounds__(256)
select_sub_kernel(const uint32_t* __restrict__ scores, int32_t* __restrict__ cand_idx, int64_t n, int64_t s_stride,
                  int subs, int max_subs, int sub_len, int n_q_heads, int n_kv_heads, int n_candidates,
                  const uint32_t* __restrict__ unit_tot, const uint32_t* __restrict__ suf,
                  uint32_t* __restrict__ err) {
  __shared__ uint2 s_ik[4][SS_QCAP];               // compacted keys: (key, packed S)
  __shared__ int2 s_par[MAXG], s_sb[MAXG];
  __shared__ uint32_t s_wc[4][4];                  // per wave: #gt heads 0/2, 1/3, #eq heads 0/2, 1/3 (16-bit)

  int unit, sub;
  xcd_unit_tile(blockIdx.x, gridDim.x / subs, subs, unit, sub);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int seq = unit / n_kv_heads, kvh = unit - seq * n_kv_heads;
  const int64_t qhead0 = (int64_t)seq * n_q_heads + kvh * G;
  // key indices fit in 32 bits (n <= n_capacity < 2^31)
  const int rows_total = sub_len >> 6;
  const int rpw = (rows_total + 3) >> 2;           // rows per wave, <= ROWS
  const int r0 = wave * rpw;
  const int nrows = (r0 + rpw <= rows_total) ? rpw : (rows_total > r0 ? rows_total - r0 : 0);
  const int w0 = sub * sub_len + r0 * 64;
  const int wlen = (int)((int64_t)w0 + nrows * 64 <= n ? nrows * 64 : (n > w0 ? n - w0 : 0));
  const int jlast = wlen > 0 ? wlen - 1 : -w0;    // clamped loads re-read key w0 + jlast (>= 0)
  const uint32_t* srow = scores + (int64_t)unit * s_stride + w0;

  // the parameters' inputs are requested before the scores (the memory
  // counter is in order, so waiting for them does not wait for the scores)
  uint32_t tot[NB / 64] = {};
  if (wave < G) load_totals<NB>(unit_tot, unit, wave, lane, tot);
  uint32_t sp[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int j = r * 64 + lane;
    sp[r] = srow[j < jlast ? j : jlast];
  }
  SubPrefix pfx;
  if (wave < G) pfx = select_theta_sub<NB>(tot, suf, unit, max_subs, sub_len, n, sub, wave, n_candidates, lane, s_par);
  __syncthreads();
  // this wave's keys above / at each head's theta: byte g of the flag words
  // counts head g (at most ROWS <= 16 per lane), then 16-bit wave sums
  uint32_t th4 = 0x7F7F7F7Fu;
#pragma unroll
  for (int g = 0; g < G; ++g) th4 = (th4 & ~(0xFFu << (8 * g))) | ((uint32_t)s_par[g].x << (8 * g));
  const uint32_t thp4 = th4 + 0x01010101u;
  uint32_t cgt = 0, ceq = 0;
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r * 64 + lane < wlen) {
      const uint32_t m = sp[r] | 0x80808080u;
      const uint32_t gt4 = (m - thp4) & 0x80808080u;
      const uint32_t eq4 = ((m - th4) & 0x80808080u) ^ gt4;
      cgt += gt4 >> 7;
      ceq += eq4 >> 7;
    }
  }
  const uint32_t g02 = xor_butterfly_u(cgt & 0x00FF00FFu, lane, AddU());
  const uint32_t g13 = xor_butterfly_u((cgt >> 8) & 0x00FF00FFu, lane, AddU());
  const uint32_t e02 = xor_butterfly_u(ceq & 0x00FF00FFu, lane, AddU());
  const uint32_t e13 = xor_butterfly_u((ceq >> 8) & 0x00FF00FFu, lane, AddU());
  if (lane == 0) {
    s_wc[wave][0] = g02; s_wc[wave][1] = g13; s_wc[wave][2] = e02; s_wc[wave][3] = e13;
  }
  // the earlier sub-tiles' counts arrived behind the rows
  if (wave < G) select_prefix_sub<NB>(pfx, suf, unit, max_subs, sub_len, n, sub, wave, lane, s_sb);
  __syncthreads();
  HeadSelect<G> hs;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int word = g & 1, shift = 16 * (g >> 1);
    int bg = s_sb[g].x, be = s_sb[g].y;
    for (int w2 = 0; w2 < wave; ++w2) {
      bg += (int)((s_wc[w2][word] >> shift) & 0xFFFFu);
      be += (int)((s_wc[w2][2 + word] >> shift) & 0xFFFFu);
    }
    hs.set(g, s_par[g].x, s_par[g].y, bg, be);
  }
  hs.finish();

  uint2* ik = s_ik[wave];
  int nk = 0;
  auto drain = [&]() {                            // whole batches; the remainder (< 64) moves to the front
    wave_lds_sync();
    int b0 = 0;
    for (; b0 + 64 <= nk; b0 += 64) hs.batch(ik[b0 + lane], true, cand_idx, qhead0, n_candidates, err);
    if (b0 > 0) {
      const int rem = nk - b0;
      uint2 e = make_uint2(0u, 0u);
      if (lane < rem) e = ik[b0 + lane];
      wave_lds_sync();
      if (lane < rem) ik[lane] = e;
      nk = rem;
    }
    wave_lds_sync();
  };
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r % SS_DRAIN_ROWS == 0 && r > 0 && nk > SS_QCAP - SS_DRAIN_ROWS * 64) drain();   // uniform
    const bool take = r * 64 + lane < wlen && hs.interesting(sp[r]) != 0u;
    const uint64_t im = __ballot(take);
    if (take) ik[nk + (int)mbcnt(im)] = make_uint2((uint32_t)(w0 + r * 64 + lane), sp[r]);
    nk += __popcll(im);
  }
  drain();
  {
    const bool valid = lane < nk;
    hs.batch(ik[valid ? lane : 0], valid, cand_idx, qhead0, n_candidates, err);
  }
}

// ===========================================================================
// sparse attention over the retrieved rows (Slides Sec. 3, Eqs. (1)-(3);
// README "3. Attention"; UVA fetch of host-resident rows, Slides Sec. 4.2.3).
//
// NW waves per query head; wave w takes rows w, w+NW, ...; lane l holds dims
// 2l, 2l+1.  All K and V row loads of a wave are issued before any use, so
// host-memory latency overlaps.  fp32 scores and softmax.
// ===========================================================================
template <int NW>
struct AttShared {
  float score[PK_MAX_TOPK_ATT];
  float acc[NW][D];
};

template <typename KT, typename QT, typename OT, int MAXR, int NW>
__device__ void attend_block(const QT* __restrict__ qh_ptr, const KT* __restrict__ kb, const KT* __restrict__ vb,
                             int64_t st, int64_t n_rows, const int32_t* hidx, int k, float scale,
                             OT* __restrict__ out_head, AttShared<NW>& s, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  float q0, q1;
  if constexpr (sizeof(QT) == 2) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(qh_ptr)[lane];
    q0 = bf16_lo(w); q1 = bf16_hi(w);
  } else {
    const float2 w = reinterpret_cast<const float2*>(qh_ptr)[lane];
    q0 = w.x; q1 = w.y;
  }
  if (n_rows <= 0) {                            // no rows: nothing may be read
    if (tid < D) {
      if constexpr (sizeof(OT) == 2) reinterpret_cast<uint16_t*>(out_head)[tid] = 0;
      else out_head[tid] = 0.0f;
    }
    return;
  }
  // lane t holds the index of this wave's row wave + NW t (-1: padding / out of range)
  int myix = -1;
  {
    const int r = wave + NW * lane;
    const int v = hidx[r < k ? r : k - 1];
    myix = (lane < MAXR && r < k && v >= 0 && (int64_t)v < n_rows) ? v : -1;
  }
  // every row load is issued unconditionally (invalid rows read row 0 and are
  // masked below) so that all of them are in flight together
  float k0v[MAXR], k1v[MAXR], v0v[MAXR], v1v[MAXR];
  uint64_t okmask = 0;
#pragma unroll
  for (int t = 0; t < MAXR; ++t) {
    const int ix = __builtin_amdgcn_readlane(myix, t);
    okmask |= (ix >= 0 ? 1ull : 0ull) << t;
    const int64_t row = ix >= 0 ? ix : 0;
    if constexpr (sizeof(KT) == 2) {
      const uint32_t kw = reinterpret_cast<const uint32_t*>(kb + row * st)[lane];
      const uint32_t vw = reinterpret_cast<const uint32_t*>(vb + row * st)[lane];
      k0v[t] = bf16_lo(kw); k1v[t] = bf16_hi(kw); v0v[t] = bf16_lo(vw); v1v[t] = bf16_hi(vw);
    } else {
      const float2 kw = reinterpret_cast<const float2*>(kb + row * st)[lane];
      const float2 vw = reinterpret_cast<const float2*>(vb + row * st)[lane];
      k0v[t] = kw.x; k1v[t] = kw.y; v0v[t] = vw.x; v1v[t] = vw.y;
    }
  }
#pragma unroll
  for (int t = 0; t < MAXR; ++t) {
    const int r = wave + NW * t;
    float p = __builtin_fmaf(q0, k0v[t], q1 * k1v[t]);
    p = xor_butterfly(p, lane, AddF());
    if (lane == 0 && r < k) s.score[r] = ((okmask >> t) & 1ull) ? p * scale : -__builtin_inff();
  }
  __syncthreads();
  float m = -__builtin_inff();
  for (int r = lane; r < k; r += 64) m = fmaxf(m, s.score[r]);
  m = xor_butterfly(m, lane, MaxF());
  float ssum = 0.0f;
  for (int r = lane; r < k; r += 64) ssum += (s.score[r] == -__builtin_inff()) ? 0.0f : __expf(s.score[r] - m);
  ssum = xor_butterfly(ssum, lane, AddF());

  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int t = 0; t < MAXR; ++t) {
    const int r = wave + NW * t;
    const float pr = ((okmask >> t) & 1ull) ? __expf(s.score[r < k ? r : 0] - m) : 0.0f;
    a0 = __builtin_fmaf(pr, v0v[t], a0);
    a1 = __builtin_fmaf(pr, v1v[t], a1);
  }
  s.acc[wave][2 * lane] = a0;
  s.acc[wave][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < D) {
    float acc = s.acc[0][tid];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) acc += s.acc[w2][tid];
    const float o = (ssum > 0.0f) ? acc / ssum : 0.0f;
    if constexpr (sizeof(OT) == 2) {
      reinterpret_cast<uint16_t*>(out_head)[tid] = (uint16_t)f32_to_bf16_rne(o);
    } else {
      out_head[tid] = o;
    }
  }
}

// K / V of one query head and where its output goes
struct AttendArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t sb, sh, st;     // element strides: sequence, KV head, token
  int64_t n_rows;
  float scale;
  void* out;
};

template <typename KT, typename QT, typename OT, int MAXR>
__global__ void __launch_bounds__(256)
attend_kernel(AttendArgs a, const int32_t* __restrict__ idx, int k, int n_q_heads, int /*n_kv_heads*/, int group) {
  __shared__ AttShared<4> s_att;
  const int head = blockIdx.x;
  const int seq = head / n_q_heads, qh = head - seq * n_q_heads, kvh = qh / group;
  const KT* kb = reinterpret_cast<const KT*>(a.k) + seq * a.sb + kvh * a.sh;
  const KT* vb = reinterpret_cast<const KT*>(a.v) + seq * a.sb + kvh * a.sh;
  attend_block<KT, QT, OT, MAXR, 4>(reinterpret_cast<const QT*>(a.q) + (int64_t)head * D, kb, vb, a.st, a.n_rows,
                                    idx + (int64_t)head * k, k, a.scale,
                                    reinterpret_cast<OT*>(a.out) + (int64_t)head * D, s_att, threadIdx.x);
}

// ===========================================================================
// rerank (Slides Eqs. (7)-(10); README "2. Decode", fused 4-bit reranking) and
// top-k by (estimate desc, key index asc) (Slides Sec. 4.2.3: reranking
// returns the Top-100 indices).
//
// Rerank: one lane per candidate gathers the key's 128-byte record (nibble
// words, then the 16 weights) and evaluates
//   est = sum_b w_b * d_b,  d_b = sum_j T[8b+j][nib_j]   (sequential in j and b)
// with T[j][nib] = fl(v(nib) * Rq[j]), v(nib) = (nib & 8 ? +1 : -1) L[nib & 7],
// i.e. fl(v * Rq) of the estimator taken from an LDS table.
//
// Top-k: estimates map to order-preserving u32 keys; since the candidate list
// is in ascending key order, a lower slot breaks ties.  Leading bits shared by
// every candidate key are skipped; histograms of successive 12-bit digits
// below them narrow down the bin holding the k-th largest key until that bin
// holds at most TOPK_MAXB keys (or all its keys are equal): keys in higher bins
// are taken, and the remaining winners of the boundary bin are found by
// ranking its keys against each other (or, when all of its keys are equal, by
// lowest slot).  The k winners are finally placed by rank (count of winners
// ahead of each).
//
// With many query heads one workgroup of RT_THREADS does both for a head and
// keeps the estimates in LDS (rerank_topk_kernel); with few heads the rerank
// is spread over several workgroups per head (rerank_kernel) and a second
// launch selects (topk_kernel), so that every compute unit takes part.
// ===========================================================================
constexpr int TOPK_BINS = 4096;        // 12-bit digit
constexpr int TOPK_MAXB = 512;         // boundary-bin size handled by ranking

// (estimate key, key index): larger = better, so equal estimates go to the lower index
__device__ __forceinline__ uint64_t topk_item(uint32_t key, int32_t ix) {
  return ((uint64_t)key << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)ix);
}

// Wave priority for round r of `rounds` over which the waves of a workgroup
// gather records: a wave that is rounds behind the others issues first when
// both are ready, so that the waves finish their gathers close together (the
// workgroup's next step waits for the last one).  The last round, and a
// single round, run at the normal priority.
__device__ __forceinline__ void set_prio_behind(int r, int rounds) {
  const int left = rounds - 1 - r;          // rounds still to come after this one
  if (left >= 3) __builtin_amdgcn_s_setprio(3);
  else if (left == 2) __builtin_amdgcn_s_setprio(2);
  else if (left == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// LDS table T[j][nib] = fl(v(nib) * Rq[j]) of one query head; thread tid
// fills entries tid + k NT.  The Rq values are loaded first (rerank_rq_load),
// ahead of the record loads, so that building the table does not wait for
// the records.
template <int NT>
__device__ __forceinline__ void rerank_rq_load(const float* rq, int tid, float (&rqv)[D * 16 / NT]) {
#pragma unroll
  for (int k = 0; k < D * 16 / NT; ++k) rqv[k] = rq[(tid + k * NT) >> 4];
}

template <int NT>
__device__ __forceinline__ void rerank_table(float* s_T, const float (&rqv)[D * 16 / NT], const Tables& tb,
                                             int tid) {
#pragma unroll
  for (int k = 0; k < D * 16 / NT; ++k) {
    const int e = tid + k * NT, nb = e & 15;
    const float lv = level_of(tb, nb & 7);
    const float v = (nb & 8) ? lv : -lv;
    s_T[e] = v * rqv[k];
  }
}

__device__ __forceinline__ void rerank_load(uint4 (&buf)[8], const uint8_t* rbase, int key) {
  const uint4* rec = reinterpret_cast<const uint4*>(rbase + (int64_t)key * 128);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) buf[kk] = rec[kk];
}

__device__ __forceinline__ float rerank_eval(const uint4 (&buf)[8], const float* s_T) {
  const uint32_t* rw = reinterpret_cast<const uint32_t*>(buf);
  float est = 0.0f;
#pragma unroll
  for (int bb = 0; bb < NSUB; ++bb) {
    const uint32_t word = rw[bb];
    // byte k of lo / hi = 4 * nibble (2k) / (2k + 1), a byte offset into the table row
    uint32_t lo = (word << 2) & 0x3C3C3C3Cu, hi = (word >> 2) & 0x3C3C3C3Cu;
    asm volatile("" : "+v"(lo), "+v"(hi));
    const char* Tb = reinterpret_cast<const char*>(s_T) + bb * (SUBD * 16 * 4);
    float v[SUBD];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      v[2 * kk] = *reinterpret_cast<const float*>(Tb + (2 * kk) * 64 + ((lo >> (8 * kk)) & 0xFFu));
      v[2 * kk + 1] = *reinterpret_cast<const float*>(Tb + (2 * kk + 1) * 64 + ((hi >> (8 * kk)) & 0xFFu));
    }
    float d = v[0];
#pragma unroll
    for (int j = 1; j < SUBD; ++j) d = d + v[j];
    const float tprod = __uint_as_float(rw[16 + bb]) * d;
    est = (bb == 0) ? tprod : est + tprod;
    asm volatile("" : "+v"(est));     // keep the sum here, not sunk into a store's branch
  }
  return est;
}

template <int NT>
struct TopkShared {
  uint32_t h[TOPK_BINS];
  uint64_t b[TOPK_MAXB];
  uint64_t f[PK_SORT_N];
  int misc[8];
  uint32_t wsum[NT / 64];
  uint32_t stat[3][NT / 64];
};

// zeroes what topk_block expects zeroed on entry (a barrier must follow)
template <int NT>
__device__ __forceinline__ void topk_shared_init(TopkShared<NT>& s, int tid) {
  uint4* h4 = reinterpret_cast<uint4*>(s.h);
  for (int i = tid; i < TOPK_BINS / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  if (tid < 8) s.misc[tid] = 0;
}

// Range statistics of a thread's estimate keys (largest, smallest, smallest
// non-negative, count of non-negative), for topk_block.
constexpr uint32_t TOPK_POS = 0x80000000u;      // keys of estimates >= 0 have the top bit set

struct TopkStats {
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu, kminp = 0xFFFFFFFFu, npos = 0;
  __device__ __forceinline__ void add(uint32_t key) {
    kmax = key > kmax ? key : kmax;
    kmin = key < kmin ? key : kmin;
    if (key >= TOPK_POS) {
      kminp = key < kminp ? key : kminp;
      ++npos;
    }
  }
};

// reduces the statistics over the wave; lane 0 leaves them in s for
// topk_block (a barrier must come between)
template <int NT>
__device__ __forceinline__ void topk_stats_wave(TopkStats st, TopkShared<NT>& s, int lane, int wave) {
  st.kmax = xor_butterfly_u(st.kmax, lane, MaxU());
  st.kmin = xor_butterfly_u(st.kmin, lane, MinU());
  st.kminp = xor_butterfly_u(st.kminp, lane, MinU());
  st.npos = xor_butterfly_u(st.npos, lane, AddU());
  if (lane == 0) { s.wsum[wave] = st.kmax; s.stat[0][wave] = st.kmin; s.stat[1][wave] = st.kminp; s.stat[2][wave] = st.npos; }
}

// Top-k of one head's n_sel candidates; thread tid holds slots r * NT + tid
// as order-preserving estimate keys key[r] and the slots' key indices kix[r].
// Slots are in ascending key order, so slot order breaks ties as the key index
// does.  s.misc and s.h must be zero on entry (topk_shared_init).  With PRE
// the caller has already left
// the waves' range statistics in s (topk_stats_wave, then a barrier).
template <int R, int NT, bool PRE = false>
__device__ void topk_block(const uint32_t (&key)[R], const int32_t (&kix)[R], int n_sel, int k, int32_t* out_idx,
                           float* out_est, TopkShared<NT>& s, int tid, int32_t* lds_idx = nullptr) {
  constexpr int NW = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const int keff = k < n_sel ? k : n_sel;
  // the common leading bits of all candidate keys need no histogram: digits
  // start at the highest bit where the largest and smallest keys differ.
  // When at least k estimates are >= 0 (keys with the top bit set), the
  // negative ones cannot win and the range starts at the smallest such key.
  if constexpr (!PRE) {
    TopkStats st;
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r * NT + tid < n_sel) st.add(key[r]);
    topk_stats_wave<NT>(st, s, lane, wave);
    __syncthreads();
  }
  uint32_t kmax = 0, kmin = 0xFFFFFFFFu, kminp = 0xFFFFFFFFu, npos = 0;
  for (int w2 = 0; w2 < NW; ++w2) {
    kmax = s.wsum[w2] > kmax ? s.wsum[w2] : kmax;
    kmin = s.stat[0][w2] < kmin ? s.stat[0][w2] : kmin;
    kminp = s.stat[1][w2] < kminp ? s.stat[1][w2] : kminp;
    npos += s.stat[2][w2];
  }
  int m = n_sel;
  if (kmin < TOPK_POS && npos >= (uint32_t)keff && keff > 0) {   // uniform
    kmin = kminp;
    m = (int)npos;
  }
  const uint32_t diff = kmax ^ kmin;
  int top = diff ? 31 - __builtin_clz(diff) : -1;        // highest undecided bit
  uint32_t pmask = top >= 0 ? ~((2u << top) - 1u) : 0xFFFFFFFFu;
  if (top == 31) pmask = 0;
  uint32_t prefix = kmax & pmask;                       // the keys in [kmin, kmax] share it
  int n_above = 0, need = keff;
  constexpr int per = TOPK_BINS / NT;                   // bins per thread
  while (keff > 0 && top >= 0 && m > TOPK_MAXB) {        // uniform
    const int shift = top >= 11 ? top - 11 : 0;
    const uint32_t dmask = (top - shift == 31) ? 0xFFFFFFFFu : ((2u << (top - shift)) - 1u);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r * NT + tid < n_sel && (key[r] & pmask) == prefix) atomicAdd(&s.h[(key[r] >> shift) & dmask], 1u);
    __syncthreads();
    // thread t owns bins [per*t, per*t + per); suffix counts from the top bin
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) mine += s.h[per * tid + i];
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t suf = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63) - incl + mine;   // lanes >= this one
    if (lane == 0) s.wsum[wave] = suf;
    __syncthreads();
    uint32_t above = suf - mine;
    for (int w2 = wave + 1; w2 < NW; ++w2) above += s.wsum[w2];
    if (above < (uint32_t)need && above + mine >= (uint32_t)need) {
      uint32_t run = above;
      for (int i = per - 1; i >= 0; --i) {
        const uint32_t c = s.h[per * tid + i];
        if (run + c >= (uint32_t)need) {
          s.misc[0] = per * tid + i;       // boundary digit
          s.misc[1] = (int)run;            // keys above it within the current range
          s.misc[2] = (int)c;              // keys with this digit
          break;
        }
        run += c;
      }
    }
    __syncthreads();
    n_above += s.misc[1];
    need -= s.misc[1];
    m = s.misc[2];
    prefix |= (uint32_t)s.misc[0] << shift;
    pmask |= dmask << shift;
    top = shift - 1;
    if (keff > 0 && top >= 0 && m > TOPK_MAXB) {  // another pass: a zeroed histogram
      uint4* h4 = reinterpret_cast<uint4*>(s.h);
      for (int i = tid; i < TOPK_BINS / 4; i += NT) h4[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
    }
  }
  __syncthreads();

  if (keff > 0) {
    // winners strictly above the boundary range, and the boundary range itself
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int p = r * NT + tid;
      if (p < n_sel) {
        const uint32_t mk = key[r] & pmask;
        if (mk > prefix) s.f[atomicAdd(&s.misc[3], 1)] = topk_item(key[r], kix[r]);
        else if (mk == prefix && m <= TOPK_MAXB) s.b[atomicAdd(&s.misc[4], 1)] = topk_item(key[r], kix[r]);
      }
    }
    __syncthreads();
    if (m <= TOPK_MAXB) {
      for (int j = tid; j < m; j += NT) {
        const uint64_t e = s.b[j];
        int rank = 0;
        for (int j2 = 0; j2 < m; ++j2) rank += (s.b[j2] > e) ? 1 : 0;
        if (rank < need) s.f[n_above + rank] = e;
      }
    } else {
      // every key of the boundary range is equal: the lowest slots win
      int eq_run = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int p = r * NT + tid;
        const bool eq = p < n_sel && (key[r] & pmask) == prefix;
        const uint64_t em = __ballot(eq);
        if (lane == 0) s.wsum[wave] = (uint32_t)__popcll(em);
        __syncthreads();
        int before = eq_run + (int)mbcnt(em), tot = 0;
        for (int w2 = 0; w2 < NW; ++w2) {
          if (w2 < wave) before += (int)s.wsum[w2];
          tot += (int)s.wsum[w2];
        }
        if (eq && before < need) s.f[n_above + before] = topk_item(key[r], kix[r]);
        eq_run += tot;
        __syncthreads();
      }
    }
  }
  __syncthreads();
  // place the keff winners by rank; PARTS neighbouring lanes count the
  // winners above winner j, each over every PARTS-th entry
  constexpr int PARTS = NT >= 1024 ? 8 : (NT >= 512 ? 4 : 2);
  for (int jb = 0; jb < keff; jb += NT / PARTS) {      // uniform
    const int j = jb + tid / PARTS, part = tid % PARTS;
    const bool act = j < keff;
    const uint64_t e = s.f[act ? j : 0];
    int rank = 0;
#pragma unroll 4
    for (int j2 = part; j2 < keff; j2 += PARTS) rank += (s.f[j2] > e) ? 1 : 0;
    if constexpr (PARTS >= 2) rank += (int)lane_xor<1>((uint32_t)rank, lane);
    if constexpr (PARTS >= 4) rank += (int)lane_xor<2>((uint32_t)rank, lane);
    if constexpr (PARTS >= 8) rank += (int)lane_xor<4>((uint32_t)rank, lane);
    if (act && part == 0) {
      const int32_t key_index = (int32_t)(0xFFFFFFFFu - (uint32_t)e);
      out_idx[rank] = key_index;
      if (lds_idx) lds_idx[rank] = key_index;
      if (out_est) out_est[rank] = from_orderable((uint32_t)(e >> 32));
    }
  }
  for (int r = keff + tid; r < k; r += NT) {
    out_idx[r] = -1;
    if (lds_idx) lds_idx[r] = -1;
    if (out_est) out_est[r] = -__builtin_inff();
  }
}

// lane part's 8 of a row's 128 coordinates, as fp32
template <typename KT>
__device__ __forceinline__ void load8(const KT* __restrict__ row, int part, float (&x)[8]) {
  if constexpr (sizeof(KT) == 2) {
    const uint4 v = reinterpret_cast<const uint4*>(row)[part];
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  } else {
    const float4 a = reinterpret_cast<const float4*>(row)[2 * part];
    const float4 b = reinterpret_cast<const float4*>(row)[2 * part + 1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// One thread's 8 dimensions of q, as loaded (bf16: one 16-byte word; fp32:
// two): requested at the start of a kernel that attends at its end, and
// converted only there, so that no wait for q sits in front of the rows'
// requests.
struct QRaw {
  uint4 a, b;
};
template <typename T>
__device__ __forceinline__ QRaw q_raw_load(const T* __restrict__ qh, int part) {
  QRaw r;
  if constexpr (sizeof(T) == 2) {
    r.a = reinterpret_cast<const uint4*>(qh)[part];
    r.b = make_uint4(0u, 0u, 0u, 0u);
  } else {
    r.a = reinterpret_cast<const uint4*>(qh)[2 * part];
    r.b = reinterpret_cast<const uint4*>(qh)[2 * part + 1];
  }
  return r;
}
template <typename T>
__device__ __forceinline__ void q_raw_cvt(const QRaw& r, float (&x)[8]) {
  if constexpr (sizeof(T) == 2) {
    x[0] = bf16_lo(r.a.x); x[1] = bf16_hi(r.a.x); x[2] = bf16_lo(r.a.y); x[3] = bf16_hi(r.a.y);
    x[4] = bf16_lo(r.a.z); x[5] = bf16_hi(r.a.z); x[6] = bf16_lo(r.a.w); x[7] = bf16_hi(r.a.w);
  } else {
    x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y); x[2] = __uint_as_float(r.a.z);
    x[3] = __uint_as_float(r.a.w); x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
    x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
  }
}

// ---- many heads: rerank and top-k of one head in one workgroup -------------
constexpr int RT_THREADS = 1024;

// Attention of one query head over its k <= 64 P retrieved rows with
// RT_THREADS threads: sixteen threads share a row, each holding 8 of its 128
// dimensions, so 64 rows are covered per pass; the K and V rows of all P
// passes are loaded before any is used.  Scores: 16-lane partial dot
// products; one max and one sum over the workgroup; the value rows are
// weighted in registers, summed over the four rows of a wave by lane swaps and
// over the waves in LDS.  fp32; indices < 0 or >= n_rows are skipped.
template <int NW>
struct AttRowsShared {
  float red[NW];
  float acc[NW][D];
};

template <typename T, int P>
__device__ void attend_rows16(const QRaw& qraw, const T* __restrict__ kb, const T* __restrict__ vb,
                              int64_t st, int64_t n_rows, const int32_t* hidx, int k, float scale,
                              T* __restrict__ out_head, AttRowsShared<RT_THREADS / 64>& s, int tid) {
  constexpr int NW = RT_THREADS / 64, RG = RT_THREADS / 16;
  const int lane = tid & 63, wave = tid >> 6, part = tid & 15, rg = tid >> 4;
  if (n_rows <= 0) {                              // no rows: nothing may be read
    if (tid < D) {
      if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t*>(out_head)[tid] = 0;
      else out_head[tid] = 0.0f;
    }
    return;
  }
  float kx[P][8], vx[P][8];
  bool ok[P];
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const int r = rg + RG * pp;
    const int v = hidx[r < k ? r : k - 1];
    ok[pp] = r < k && v >= 0 && (int64_t)v < n_rows;
    const int64_t row = ok[pp] ? v : 0;          // skipped rows read row 0 and are masked
    load8(kb + row * st, part, kx[pp]);
    load8(vb + row * st, part, vx[pp]);
  }
  float qv[8];
  q_raw_cvt<T>(qraw, qv);
  float sc[P];
  float m = -__builtin_inff();
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    float d = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qv[e], kx[pp][e], d);
    d = xor_butterfly16(d, lane, AddF());
    sc[pp] = ok[pp] ? d * scale : -__builtin_inff();
    m = fmaxf(m, sc[pp]);
  }
  m = fmaxf(m, lane_xor_f<32>(m, lane));
  m = fmaxf(m, lane_xor_f<16>(m, lane));
  if (lane == 0) s.red[wave] = m;
  __syncthreads();
  m = s.red[0];
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) m = fmaxf(m, s.red[w2]);
  __syncthreads();                               // s.red is reused for the sums
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float ssum = 0.0f;
#pragma unroll
  for (int pp = 0; pp < P; ++pp) {
    const float pr = ok[pp] ? __expf(sc[pp] - m) : 0.0f;
    ssum += pr;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(pr, vx[pp][e], acc[e]);
  }
  // the four row groups of the wave: every lane of a group holds the group's sum
  ssum += lane_xor_f<16>(ssum, lane);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += lane_xor_f<16>(acc[e], lane);
  ssum += lane_xor_f<32>(ssum, lane);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] += lane_xor_f<32>(acc[e], lane);
  if (lane == 0) s.red[wave] = ssum;
  if (lane < 16) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s.acc[wave][8 * part + e] = acc[e];
  }
  __syncthreads();
  if (tid < D) {
    float o = s.acc[0][tid], tot = s.red[0];
#pragma unroll
    for (int w2 = 1; w2 < NW; ++w2) { o += s.acc[w2][tid]; tot += s.red[w2]; }
    const float res = (tot > 0.0f) ? o / tot : 0.0f;
    if constexpr (sizeof(T) == 2) reinterpret_cast<uint16_t*>(out_head)[tid] = (uint16_t)f32_to_bf16_rne(res);
    else out_head[tid] = res;
  }
}

// T, MAXR, ATT: with ATT the workgroup goes on to attend over its head's k
// rows (q, K, V and the output all of type T; MAXR rows per wave).
template <int R, typename T, int P, bool ATT>   // candidate slots per thread: n_sel <= R * RT_THREADS
__global__ void __launch_bounds__(RT_THREADS)
rerank_topk_kernel(const uint8_t* __restrict__ records, const float* __restrict__ rot_q,
                   int32_t* __restrict__ cand_idx, float* __restrict__ cand_est_out, int64_t n_cap, int n_sel,
                   int n_candidates, int n_q_heads, int n_kv_heads, int group, Tables tb, int k,
                   int32_t* __restrict__ out_idx, float* __restrict__ out_est, AttendArgs att) {
  __shared__ float s_T[D * 16];
  __shared__ float s_est[R * RT_THREADS];
  __shared__ TopkShared<RT_THREADS> s_tk;
  __shared__ int32_t s_idx[ATT ? PK_MAX_TOPK_ATT : 1];
  __shared__ AttRowsShared<ATT ? RT_THREADS / 64 : 1> s_att;

  // the query heads of one KV head on one XCD (their common records meet in its L2)
  int unit_x, g_x;
  xcd_unit_tile(blockIdx.x, gridDim.x / group, group, unit_x, g_x);
  const int head = unit_x * group + g_x, tid = threadIdx.x;
  QRaw qraw{};
  if constexpr (ATT) qraw = q_raw_load<T>(reinterpret_cast<const T*>(att.q) + (int64_t)head * D, tid & 15);
  const int seq = head / n_q_heads, qh = head - seq * n_q_heads;
  const int unit = seq * n_kv_heads + qh / group;
  const uint8_t* rbase = records + (int64_t)unit * n_cap * 128;
  int32_t* ci = cand_idx + (int64_t)head * n_candidates;
  float* ce = cand_est_out ? cand_est_out + (int64_t)head * n_candidates : nullptr;
  const int plast = n_sel > 0 ? n_sel - 1 : 0;
  const int rounds = (n_sel + RT_THREADS - 1) / RT_THREADS;

  // the key index of the next round is loaded one round ahead, so each
  // round waits for one memory trip (its records), not two
  float rqv[D * 16 / RT_THREADS];
  rerank_rq_load<RT_THREADS>(rot_q + (int64_t)head * D, tid, rqv);
  // unconditional (clamped) loads: a branch around them would make the
  // table below wait for the records as well
  uint4 ra[8];
  rerank_load(ra, rbase, ci[tid < plast ? tid : plast]);
  int ixn = ci[RT_THREADS + tid < plast ? RT_THREADS + tid : plast];
  rerank_table<RT_THREADS>(s_T, rqv, tb, tid);
  topk_shared_init<RT_THREADS>(s_tk, tid);
  for (int p = n_sel + tid; p < n_candidates; p += RT_THREADS) {   // invalid tail slots (n < C)
    ci[p] = -1;
    if (ce) ce[p] = -__builtin_inff();
  }
  __syncthreads();
  TopkStats st;
#pragma unroll 1
  for (int r = 0; r < rounds; ++r) {
    const int p = r * RT_THREADS + tid;
    if (r) {
      rerank_load(ra, rbase, ixn);
      ixn = ci[p + RT_THREADS < plast ? p + RT_THREADS : plast];
    }
    set_prio_behind(r, rounds);     // the top-k waits for the last wave
    const float est = rerank_eval(ra, s_T);
    s_est[p] = est;
    if (p < n_sel) st.add(orderable(est));
    if (ce && p < n_sel) ce[p] = est;
  }
  __builtin_amdgcn_s_setprio(0);
  int32_t kix[R];                   // the slots' key indices (L2), in flight during the first top-k steps
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int p = r * RT_THREADS + tid;
    kix[r] = ci[p < plast ? p : plast];
  }
  topk_stats_wave<RT_THREADS>(st, s_tk, tid & 63, tid >> 6);
  __syncthreads();
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int p = r * RT_THREADS + tid;
    key[r] = orderable(s_est[p < plast ? p : plast]);
  }
  topk_block<R, RT_THREADS, true>(key, kix, n_sel, k, out_idx + (int64_t)head * k, out_est ? out_est + (int64_t)head * k : nullptr,
                            s_tk, tid, ATT ? s_idx : nullptr);
  if constexpr (ATT) {
    __syncthreads();
    const int kvh = qh / group;
    const T* kb = reinterpret_cast<const T*>(att.k) + seq * att.sb + kvh * att.sh;
    const T* vb = reinterpret_cast<const T*>(att.v) + seq * att.sb + kvh * att.sh;
    attend_rows16<T, P>(qraw, kb, vb, att.st, att.n_rows, s_idx,
                        k, att.scale, reinterpret_cast<T*>(att.out) + (int64_t)head * D, s_att, tid);
  }
}

// ---- few heads: rerank spread over workgroups of 256 x RR candidates --------
// RR: candidates per lane (rounds of 256 per workgroup)
template <int RR>
__global__ void __launch_bounds__(256)
rerank_kernel(const uint8_t* __restrict__ records, const float* __restrict__ rot_q,
              int32_t* __restrict__ cand_idx, float* __restrict__ cand_est, int64_t n_cap,
              int n_sel, int n_candidates, int chunks, int n_q_heads, int n_kv_heads, int group, Tables tb) {
  __shared__ float s_T[D * 16];
  const int head = blockIdx.x / chunks, ch = blockIdx.x - head * chunks;
  const int tid = threadIdx.x;
  const int seq = head / n_q_heads, qh = head - seq * n_q_heads;
  const int unit = seq * n_kv_heads + qh / group;
  const uint8_t* rbase = records + (int64_t)unit * n_cap * 128;
  int32_t* ci = cand_idx + (int64_t)head * n_candidates;
  float* ce = cand_est + (int64_t)head * n_candidates;
  const int p0 = ch * 256 * RR;
  const int plast = n_sel - 1;

  float rqv[D * 16 / 256];
  rerank_rq_load<256>(rot_q + (int64_t)head * D, tid, rqv);
  uint4 ra[8];
  rerank_load(ra, rbase, ci[p0 + tid < plast ? p0 + tid : plast]);
  int ixn = ci[p0 + 256 + tid < plast ? p0 + 256 + tid : plast];   // next round's key index
  rerank_table<256>(s_T, rqv, tb, tid);
  __syncthreads();
  // nothing that reads the records is scheduled above the table build (it
  // would make the table wait for the record loads)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
  for (int r = 0; r < RR; ++r) {
    const int p = p0 + r * 256 + tid;
    if (r) {
      rerank_load(ra, rbase, ixn);
      ixn = ci[p + 256 < plast ? p + 256 : plast];
    }
    const float est = rerank_eval(ra, s_T);
    // every lane stores: past the end a lane holds the last slot's record and
    // rewrites that slot's estimate with the same value (an unconditional
    // store keeps the wait for the next key index from covering it)
    ce[p < n_sel ? p : plast] = est;
  }
}

constexpr int TK_THREADS = RT_THREADS;   // top-k workgroup (few heads, many candidates)

// T, P, ATT: with ATT the workgroup goes on to attend over its head's k rows
// (q, K, V and the output all of type T; P passes of 64 rows), as
// rerank_topk_kernel does.
template <int R, typename T, int P, bool ATT>
__global__ void __launch_bounds__(TK_THREADS)
topk_kernel(int32_t* __restrict__ cand_idx, float* __restrict__ cand_est, int n_sel,
            int n_candidates, int k, int32_t* __restrict__ out_idx, float* __restrict__ out_est,
            int n_q_heads, int group, AttendArgs att) {
  __shared__ TopkShared<TK_THREADS> s_tk;
  __shared__ int32_t s_idx[ATT ? PK_MAX_TOPK_ATT : 1];
  __shared__ AttRowsShared<ATT ? TK_THREADS / 64 : 1> s_att;
  const int head = blockIdx.x, tid = threadIdx.x;
  QRaw qraw{};
  if constexpr (ATT) qraw = q_raw_load<T>(reinterpret_cast<const T*>(att.q) + (int64_t)head * D, tid & 15);
  int32_t* ci = cand_idx + (int64_t)head * n_candidates;
  float* ce = cand_est + (int64_t)head * n_candidates;
  // candidate estimates: clamped unconditional loads, all in flight together
  float ev[R];
  int32_t kix[R];
  const int plast = n_sel > 0 ? n_sel - 1 : 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int p = r * TK_THREADS + tid;
    ev[r] = ce[p < plast ? p : plast];
    kix[r] = ci[p < plast ? p : plast];
  }
  topk_shared_init<TK_THREADS>(s_tk, tid);
  for (int p = n_sel + tid; p < n_candidates; p += TK_THREADS) {   // invalid tail slots (n < C)
    ci[p] = -1;
    ce[p] = -__builtin_inff();
  }
  uint32_t key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) key[r] = orderable(ev[r]);
  topk_block<R, TK_THREADS>(key, kix, n_sel, k, out_idx + (int64_t)head * k, out_est ? out_est + (int64_t)head * k : nullptr,
                     s_tk, tid, ATT ? s_idx : nullptr);
  if constexpr (ATT) {
    __syncthreads();
    const int seq = head / n_q_heads, qh = head - seq * n_q_heads, kvh = qh / group;
    const T* kb = reinterpret_cast<const T*>(att.k) + seq * att.sb + kvh * att.sh;
    const T* vb = reinterpret_cast<const T*>(att.v) + seq * att.sb + kvh * att.sh;
    attend_rows16<T, P>(qraw, kb, vb, att.st, att.n_rows, s_idx,
                        k, att.scale, reinterpret_cast<T*>(att.out) + (int64_t)head * D, s_att, tid);
  }
}

// ===========================================================================
// attention over the retrieved rows and the dense rows together (README
// "3. Attention": sink, local and retrieved tokens; Slides Fig. 5,
// Sec. 4.2.1-4.2.3: sink and recent local tokens, with the update buffer,
// stay on the GPU for dense attention).
//
// One workgroup per query head.  Sixteen threads share a row, each holding 8
// of its 128 dimensions (one 16-byte load of bf16, two of fp32), so a
// workgroup covers DA_THREADS / 16 rows per pass with coalesced loads.  Rows
// are the k retrieved rows, then the n_dense dense rows; a row's K and V are
// loaded together.  Each row group keeps a running softmax over its rows
// (max, sum, and its 8 dimensions of the weighted value sum); the groups are
// rescaled to the workgroup max and added in LDS.  fp32.
// ===========================================================================
constexpr int DA_THREADS = 1024;
constexpr int DA_GROUPS = DA_THREADS / 16;     // rows per pass
constexpr int DA_UNROLL = 4;                   // passes whose rows are loaded together


template <typename KT, typename QT, typename OT>
__global__ void __launch_bounds__(DA_THREADS)
dense_sparse_attend_kernel(AttendArgs a, const int32_t* __restrict__ idx, int k, const KT* __restrict__ dk,
                           const KT* __restrict__ dv, int64_t dsb, int64_t dsh, int64_t dst, int n_dense,
                           int n_q_heads, int /*n_kv_heads*/, int group) {
  __shared__ int32_t s_ix[PK_MAX_TOPK_ATT];                // retrieved rows (-1: skipped)
  __shared__ float s_red[DA_THREADS / 64];
  __shared__ float s_acc[DA_GROUPS][D + 4];

  const int head = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = tid & 15, rg = tid >> 4;           // dimensions 8 part .. 8 part + 7; row group
  const int seq = head / n_q_heads, qh = head - seq * n_q_heads, kvh = qh / group;
  const KT* kb = reinterpret_cast<const KT*>(a.k) + seq * a.sb + kvh * a.sh;
  const KT* vb = reinterpret_cast<const KT*>(a.v) + seq * a.sb + kvh * a.sh;
  const KT* dkb = dk + seq * dsb + kvh * dsh;
  const KT* dvb = dv + seq * dsb + kvh * dsh;
  float qv[8];
  if constexpr (sizeof(QT) == 2) {
    const uint4 v = reinterpret_cast<const uint4*>(a.q)[(int64_t)head * (D / 8) + part];
    qv[0] = bf16_lo(v.x); qv[1] = bf16_hi(v.x); qv[2] = bf16_lo(v.y); qv[3] = bf16_hi(v.y);
    qv[4] = bf16_lo(v.z); qv[5] = bf16_hi(v.z); qv[6] = bf16_lo(v.w); qv[7] = bf16_hi(v.w);
  } else {
    const float4 x = reinterpret_cast<const float4*>(a.q)[(int64_t)head * (D / 4) + 2 * part];
    const float4 y = reinterpret_cast<const float4*>(a.q)[(int64_t)head * (D / 4) + 2 * part + 1];
    qv[0] = x.x; qv[1] = x.y; qv[2] = x.z; qv[3] = x.w; qv[4] = y.x; qv[5] = y.y; qv[6] = y.z; qv[7] = y.w;
  }
  // with no zone rows the retrieved indices are all skipped and nothing of
  // the zone is read
  const int kz = a.n_rows > 0 ? k : 0;
  for (int r = tid; r < kz; r += DA_THREADS) {
    const int v = idx[(int64_t)head * k + r];
    s_ix[r] = (v >= 0 && (int64_t)v < a.n_rows) ? v : -1;
  }
  __syncthreads();
  const int total = kz + n_dense;
  if (total == 0) {
    if (tid < D) {
      if constexpr (sizeof(OT) == 2) reinterpret_cast<uint16_t*>(a.out)[(int64_t)head * D + tid] = 0;
      else reinterpret_cast<float*>(a.out)[(int64_t)head * D + tid] = 0.0f;
    }
    return;
  }

  // one pass over the rows: each row group keeps a running max, sum and
  // weighted value sum of its rows (invalid retrieved rows and rows past the
  // end are skipped; they re-read a valid row)
  float m = -__builtin_inff(), l = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const int passes = (total + DA_UNROLL * DA_GROUPS - 1) / (DA_UNROLL * DA_GROUPS);
  for (int r0 = 0; r0 < total; r0 += DA_UNROLL * DA_GROUPS) {   // uniform
    set_prio_behind(r0 / (DA_UNROLL * DA_GROUPS), passes);       // the merge waits for the last wave
    float x[DA_UNROLL][8], y[DA_UNROLL][8];
    bool ok[DA_UNROLL];
#pragma unroll
    for (int u = 0; u < DA_UNROLL; ++u) {         // every row's K and V in flight first
      const int r = r0 + u * DA_GROUPS + rg;
      const int rr = r < total ? r : total - 1;
      ok[u] = r < total;
      const KT* krow;
      const KT* vrow;
      if (rr < kz) {
        const int ix = s_ix[rr];
        ok[u] = ok[u] && ix >= 0;
        krow = kb + (int64_t)(ix >= 0 ? ix : 0) * a.st;
        vrow = vb + (int64_t)(ix >= 0 ? ix : 0) * a.st;
      } else {
        krow = dkb + (int64_t)(rr - kz) * dst;
        vrow = dvb + (int64_t)(rr - kz) * dst;
      }
      load8(krow, part, x[u]);
      load8(vrow, part, y[u]);
    }
#pragma unroll
    for (int u = 0; u < DA_UNROLL; ++u) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = __builtin_fmaf(qv[e], x[u][e], d);
      d = xor_butterfly16(d, lane, AddF());
      if (ok[u]) {                                // uniform over the row group
        const float sc = d * a.scale;
        const float mn = fmaxf(m, sc);
        const float f = __expf(m - mn);           // m = -inf: 0
        const float pr = __expf(sc - mn);
        l = l * f + pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(pr, y[u][e], acc[e] * f);
        m = mn;
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  // workgroup max of the group maxima, then rescale each group's sums to it
  float mw = m;
  mw = fmaxf(mw, lane_xor_f<32>(mw, lane));
  mw = fmaxf(mw, lane_xor_f<16>(mw, lane));
  if (lane == 0) s_red[wave] = mw;
  __syncthreads();
  float M = s_red[0];
#pragma unroll
  for (int w2 = 1; w2 < DA_THREADS / 64; ++w2) M = fmaxf(M, s_red[w2]);
  __syncthreads();                                // s_red is reused for the sums
  const float f = (m == -__builtin_inff()) ? 0.0f : __expf(m - M);
  float ssum = (part == 0) ? l * f : 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= f;
  ssum = xor_butterfly(ssum, lane, AddF());
  if (lane == 0) s_red[wave] = ssum;
  __syncthreads();
  ssum = 0.0f;
#pragma unroll
  for (int w2 = 0; w2 < DA_THREADS / 64; ++w2) ssum += s_red[w2];

#pragma unroll
  for (int e = 0; e < 8; ++e) s_acc[rg][8 * part + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float o = s_acc[0][tid];
    for (int g2 = 1; g2 < DA_GROUPS; ++g2) o += s_acc[g2][tid];
    const float res = (ssum > 0.0f) ? o / ssum : 0.0f;
    if constexpr (sizeof(OT) == 2) {
      reinterpret_cast<uint16_t*>(a.out)[(int64_t)head * D + tid] = (uint16_t)f32_to_bf16_rne(res);
    } else {
      reinterpret_cast<float*>(a.out)[(int64_t)head * D + tid] = res;
    }
  }
}

// rows [0, rows) of every (sequence, KV head) from src to dst, 16 bytes per
// lane (row_vec 16-byte pieces per row); dst may be the device view of mapped
// host memory, so the stores cross the host link
__global__ void __launch_bounds__(256) copy_rows_kernel(const uint4* __restrict__ src, int64_t ssb, int64_t ssh,
                                                      int64_t sst, uint4* __restrict__ dst, int64_t dsb,
                                                      int64_t dsh, int64_t dst_, int n_kv_heads, int64_t rows,
                                                      int row_vec, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t v = i % row_vec, r = (i / row_vec) % rows, uh = i / (row_vec * rows);
  const int64_t b = uh / n_kv_heads, h = uh - b * n_kv_heads;
  dst[b * dsb + h * dsh + r * dst_ + v] = src[b * ssb + h * ssh + r * sst + v];
}

// set `count` words to `value`
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t value, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < count) p[i] = value;
}

// fill top-k outputs for an empty key set
__global__ void fill_empty_kernel(int32_t* __restrict__ idx, float* __restrict__ est, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    if (idx) idx[i] = -1;
    if (est) est[i] = -__builtin_inff();
  }
}

}  // namespace pk
