// Constant tables of the ParisKV path (host side).
#pragma once
#include <cstdint>

namespace pk {

constexpr int kHeadDim = 128;   // D
constexpr int kNSub = 16;       // B
constexpr int kSubDim = 8;      // m = D / B
constexpr int kLevels = 8;      // 3-bit magnitude index

// SRHT random diagonal: sign j = +1 iff the top bit of the j-th 64-bit output
// of Philox4x64-10 with key (seed, 0), counters 1, 2, ..., is clear.
void srht_signs(uint64_t seed, int8_t signs[kHeadDim]);

// fp64 Lloyd-Max levels / thresholds of |u_j| for u uniform on S^{m-1}.
void lloyd_max(int n_levels, int m, double* levels, double* thresholds);

// The fp32 tables encode and rerank consume (m = 8, 8 levels).
void magnitude_tables(float levels[kLevels], float thresholds[kLevels - 1]);

}  // namespace pk
