"""Pins of the oracle's constant tables against things other than the oracle:
the Philox4x64-10 definition and its known-answer vector, and the closed-form
Beta prior of the magnitude quantiser (independent numerical integration,
Monte Carlo)."""
import json
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.special

from oracle import pariskv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
M64 = (1 << 64) - 1


def _philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds, written from its published definition
    (Salmon, Moraes, Dror, Shaw, 'Parallel random numbers: as easy as 1, 2, 3',
    SC'11): two 64x64->128 multiplies per round, Weyl key schedule."""
    c = list(ctr)
    k = list(key)
    for r in range(10):
        if r:
            k[0] = (k[0] + 0x9E3779B97F4A7C15) & M64
            k[1] = (k[1] + 0xBB67AE8584CAA73B) & M64
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [((p1 >> 64) ^ c[1] ^ k[0]) & M64, p1 & M64,
             ((p0 >> 64) ^ c[3] ^ k[1]) & M64, p0 & M64]
    return c


def test_philox_known_answer():
    # Random123 known-answer vector for philox4x64-10, zero counter and key.
    assert _philox4x64_10([0, 0, 0, 0], [0, 0]) == [
        0x16554D9ECA36314C, 0xDB20FE9D672D0FDC, 0xD7E772CEE186176B, 0x7E68B68AEC7BA23B]


@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_srht_signs_follow_philox_definition(seed):
    words = []
    for ctr in range(1, 33):
        words += _philox4x64_10([ctr, 0, 0, 0], [seed, 0])
    expect = np.array([1 if (w >> 63) == 0 else -1 for w in words[:128]], dtype=np.int8)
    got = O.srht_signs(seed)
    assert got.dtype == np.int8 and got.shape == (128,)
    np.testing.assert_array_equal(got, expect)


def test_srht_signs_differ_by_seed_and_are_balanced():
    s0, s1 = O.srht_signs(0), O.srht_signs(1)
    assert (s0 != s1).any()
    assert 40 < int((s0 > 0).sum()) < 88


# ---------------------------------------------------------------------------
# Magnitude prior and Lloyd-Max table
# ---------------------------------------------------------------------------
def _density(a, m=8):
    # |u_j| density for u uniform on S^{m-1}: derivative of I_{a^2}(1/2, (m-1)/2)
    return 2.0 * (1.0 - a * a) ** ((m - 3) / 2.0) / scipy.special.beta(0.5, (m - 1) / 2.0)


def test_golden_structural_constants():
    g = json.load(open(GOLDEN))
    assert O.N_LEVELS == g["magnitude_levels"]["value"]
    assert O.SUB_DIM == g["sub_dim_m"]["value"]
    assert O.N_SUB == g["n_sub_B"]["value"]
    assert O.D == O.N_SUB * O.SUB_DIM
    assert 2 ** g["nibble_bits"]["magnitude"] == O.N_LEVELS
    assert g["nibble_bits"]["sign"] + g["nibble_bits"]["magnitude"] == 4
    assert O.N_CENTROIDS == 2 ** O.SUB_DIM


@pytest.mark.filterwarnings("ignore::scipy.integrate.IntegrationWarning")
@pytest.mark.parametrize("m", [8, 4, 16])
def test_prior_cdf_matches_independent_integration(m):
    for a in [0.05, 0.2, 0.37, 0.5, 0.81, 0.99]:
        ref, _ = scipy.integrate.quad(_density, 0.0, a, args=(m,), epsabs=1e-14)
        assert abs(O.magnitude_cdf(a, m) - ref) < 1e-11
        ref1, _ = scipy.integrate.quad(lambda x: x * _density(x, m), 0.0, a, epsabs=1e-14)
        assert abs(O.magnitude_partial_mean(a, m) - ref1) < 1e-11
    total, _ = scipy.integrate.quad(_density, 0.0, 1.0, args=(m,), epsabs=1e-14, epsrel=1e-14, limit=200)
    assert abs(total - 1.0) < 1e-12
    # E[u_j^2] = mean of Beta(1/2, (m-1)/2) = 1/m
    m2, _ = scipy.integrate.quad(lambda x: x * x * _density(x, m), 0.0, 1.0, epsabs=1e-14, epsrel=1e-14, limit=200)
    assert abs(m2 - 1.0 / m) < 1e-12


def test_prior_cdf_matches_sphere_monte_carlo():
    rng = np.random.default_rng(7)
    g = rng.standard_normal((200000, 8))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    a = np.sort(np.abs(u[:, 0]))
    emp = np.arange(1, a.size + 1) / a.size
    ks = np.max(np.abs(emp - O.magnitude_cdf(a, 8)))
    assert ks < 0.006


def test_lloyd_max_fixed_point_by_quadrature():
    L, tau = O.lloyd_max_levels()
    assert L.shape == (8,) and tau.shape == (7,)
    assert np.all(np.diff(L) > 0) and 0 < L[0] and L[-1] < 1
    np.testing.assert_allclose(tau, 0.5 * (L[:-1] + L[1:]), rtol=0, atol=1e-15)
    edges = np.concatenate([[0.0], tau, [1.0]])
    for l in range(8):
        mass, _ = scipy.integrate.quad(_density, edges[l], edges[l + 1], epsabs=1e-15)
        mom, _ = scipy.integrate.quad(lambda x: x * _density(x), edges[l], edges[l + 1], epsabs=1e-15)
        assert abs(mom / mass - L[l]) < 1e-10


def _mse(L):
    tau = 0.5 * (L[:-1] + L[1:])
    edges = np.concatenate([[0.0], tau, [1.0]])
    tot = 0.0
    for l in range(len(L)):
        v, _ = scipy.integrate.quad(lambda x: (x - L[l]) ** 2 * _density(x), edges[l], edges[l + 1])
        tot += v
    return tot


def test_lloyd_max_is_locally_optimal():
    L, _ = O.lloyd_max_levels()
    base = _mse(L)
    for l in range(8):
        for d in (-1e-3, 1e-3):
            Lp = L.copy()
            Lp[l] += d
            assert _mse(Lp) > base


def test_lloyd_max_agrees_with_sample_based_lloyd():
    # the repository regenerates its levels from samples (README 'Codebooks');
    # a 1-D Lloyd run on sphere samples lands on the same levels
    rng = np.random.default_rng(3)
    g = rng.standard_normal((400000, 8))
    a = np.abs((g / np.linalg.norm(g, axis=1, keepdims=True)).ravel())
    L = np.quantile(a, (np.arange(8) + 0.5) / 8)
    for _ in range(200):
        tau = 0.5 * (L[:-1] + L[1:])
        cell = np.searchsorted(tau, a, side="right")
        L = np.bincount(cell, weights=a, minlength=8) / np.bincount(cell, minlength=8)
    L_ref, _ = O.lloyd_max_levels()
    np.testing.assert_allclose(L, L_ref, atol=1.5e-3)


def test_f32_tables_are_rounded_fp64():
    L, tau = O.lloyd_max_levels()
    L32, tau32 = O.magnitude_tables_f32()
    assert L32.dtype == np.float32 and tau32.dtype == np.float32
    np.testing.assert_array_equal(L32, L.astype(np.float32))
    np.testing.assert_array_equal(tau32, tau.astype(np.float32))
