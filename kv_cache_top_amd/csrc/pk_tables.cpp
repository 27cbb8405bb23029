// Host-side constant tables of the ParisKV path: the SRHT sign vector and the
// 3-bit magnitude quantiser.  Pure C++ (no HIP), computed once per context.
#include "pk_tables.hpp"

#include <cmath>
#include <cstring>

namespace pk {

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11): per round two 64x64->128-bit products with the constants
// below; the key is bumped by the Weyl increments between rounds.
// ---------------------------------------------------------------------------
static void philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
  uint64_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint64_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B97F4A7C15ull;
      k1 += 0xBB67AE8584CAA73Bull;
    }
    const unsigned __int128 p0 = (unsigned __int128)0xD2E7470EE14C6C93ull * c[0];
    const unsigned __int128 p1 = (unsigned __int128)0xCA5A826395121157ull * c[2];
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0;
    const uint64_t hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n1 = lo1, n2 = hi0 ^ c[3] ^ k1, n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
  std::memcpy(out, c, sizeof(c));
}

void srht_signs(uint64_t seed, int8_t signs[kHeadDim]) {
  // Stream of 64-bit words for key (seed, 0): counter 1, 2, ... each giving four
  // words in order.  Sign j is +1 when the top bit of word j is clear.
  const uint64_t key[2] = {seed, 0};
  for (int blk = 0; blk < kHeadDim / 4; ++blk) {
    const uint64_t ctr[4] = {(uint64_t)blk + 1, 0, 0, 0};
    uint64_t w[4];
    philox4x64_10(ctr, key, w);
    for (int i = 0; i < 4; ++i) signs[blk * 4 + i] = (w[i] >> 63) ? -1 : 1;
  }
}

// ---------------------------------------------------------------------------
// Lloyd-Max quantiser of a = |u_j|, u uniform on the unit sphere of R^m.
// u_j^2 ~ Beta(1/2, (m-1)/2), so a has density proportional to
// (1 - a^2)^((m-3)/2) on [0, 1].  Cell masses and first moments are integrated
// with composite Gauss-Legendre quadrature; the normalising constant cancels
// in the conditional means.
// ---------------------------------------------------------------------------
namespace {

constexpr int kGL = 24;        // nodes per panel
constexpr int kPanels = 32;    // panels per cell

struct GaussLegendre {
  double x[kGL], w[kGL];
  GaussLegendre() {
    // roots of P_n by Newton's method from the Chebyshev-like initial guess
    const int n = kGL;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          const double p2 = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = p2;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        const double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-17) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre& gl() {
  static const GaussLegendre g;
  return g;
}

// mass and first moment of (1 - a^2)^e over [lo, hi]
void cell_moments(double lo, double hi, double e, double* mass, double* mom) {
  const GaussLegendre& q = gl();
  double m0 = 0.0, m1 = 0.0;
  const double h = (hi - lo) / kPanels;
  for (int p = 0; p < kPanels; ++p) {
    const double a = lo + p * h, mid = a + 0.5 * h, half = 0.5 * h;
    for (int i = 0; i < kGL; ++i) {
      const double t = mid + half * q.x[i];
      const double f = std::pow(std::fmax(0.0, 1.0 - t * t), e) * q.w[i] * half;
      m0 += f;
      m1 += t * f;
    }
  }
  *mass = m0;
  *mom = m1;
}

}  // namespace

void lloyd_max(int n_levels, int m, double* levels, double* thresholds) {
  const double e = 0.5 * (m - 3);
  for (int l = 0; l < n_levels; ++l) levels[l] = (l + 0.5) / n_levels;   // uniform start
  for (int it = 0; it < 100000; ++it) {
    double change = 0.0;
    double lo = 0.0;
    double next[64];
    for (int l = 0; l < n_levels; ++l) {
      const double hi = (l + 1 < n_levels) ? 0.5 * (levels[l] + levels[l + 1]) : 1.0;
      double mass, mom;
      cell_moments(lo, hi, e, &mass, &mom);
      next[l] = mom / mass;
      lo = hi;
    }
    for (int l = 0; l < n_levels; ++l) {
      change = std::fmax(change, std::fabs(next[l] - levels[l]));
      levels[l] = next[l];
    }
    if (change < 1e-15) break;
  }
  for (int l = 0; l + 1 < n_levels; ++l) thresholds[l] = 0.5 * (levels[l] + levels[l + 1]);
}

void magnitude_tables(float levels[kLevels], float thresholds[kLevels - 1]) {
  double L[kLevels], T[kLevels - 1];
  lloyd_max(kLevels, kSubDim, L, T);
  for (int l = 0; l < kLevels; ++l) levels[l] = (float)L[l];
  for (int l = 0; l + 1 < kLevels; ++l) thresholds[l] = (float)T[l];
}

}  // namespace pk
