"""Pins of the oracle's rotation and key encoding: the Hadamard closed form,
orthogonality and inner-product preservation of R, brute-force centroid
assignment over all 256 sign patterns, nearest-level quantisation, the Beta
prior moments of the rotated blocks, and agreement of the fp32 order with the
literal fp64 formulas."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S

SIGNS = O.srht_signs(0)
L32, TAU32 = O.magnitude_tables_f32()
L64, TAU64 = O.lloyd_max_levels()


def _popcount_hadamard(n):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_hadamard_closed_form():
    np.testing.assert_array_equal(O.hadamard(128), _popcount_hadamard(128))


def test_fwht_equals_dense_hadamard_fp64():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128))
    H = _popcount_hadamard(128)
    np.testing.assert_allclose(O.fwht(x), x @ H.T, rtol=0, atol=1e-11)


def test_fwht_f32_exact_on_small_integers():
    rng = np.random.default_rng(1)
    x = rng.integers(-50, 50, size=(64, 128))
    H = _popcount_hadamard(128).astype(np.int64)
    got = O.fwht(x.astype(np.float32))
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got.astype(np.int64), x @ H.T)


def test_rotation_orthogonal_and_preserves_inner_products():
    R = O.rotation_matrix(SIGNS)
    np.testing.assert_allclose(R @ R.T, np.eye(128), atol=1e-12)
    # R e_j = s_j H[:, j] / sqrt(D)
    H = _popcount_hadamard(128)
    np.testing.assert_allclose(R[:, 5], SIGNS[5] * H[:, 5] / np.sqrt(128), atol=1e-15)
    # fp32 path: <Rx, Ry> = <x, y> within 1e-5 relative
    rng = np.random.default_rng(2)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    y = rng.standard_normal((200, 128)).astype(np.float32)
    c = np.float32(1 / np.sqrt(128))
    rx = O.fwht(x * SIGNS.astype(np.float32)) * c
    ry = O.fwht(y * SIGNS.astype(np.float32)) * c
    lhs = np.sum(rx.astype(np.float64) * ry, axis=1)
    rhs = np.sum(x.astype(np.float64) * y, axis=1)
    scale = np.linalg.norm(x, axis=1) * np.linalg.norm(y, axis=1)
    assert np.max(np.abs(lhs - rhs) / scale) < 1e-5


def _keys(n=3000, seed=5):
    w = S.custom("tiny4k", n=n)
    return S.as_f32(S.unit_keys(w, 0, 0))


def test_codes_are_brute_force_argmax_over_256_centres():
    k = _keys(2000)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    lit = O.encode_literal(k, SIGNS, L64, TAU64)
    # brute force, independently of the oracle: all 256 inner products
    R = O.rotation_matrix(SIGNS)
    kt = (k.astype(np.float64) / np.linalg.norm(k, axis=1, keepdims=True)) @ R.T
    u = kt.reshape(-1, 16, 8)
    u = u / np.linalg.norm(u, axis=2, keepdims=True)
    best = np.zeros(u.shape[:2], dtype=np.int64)
    bestv = np.full(u.shape[:2], -np.inf)
    for c in range(256):
        om = np.array([1.0 if (c >> j) & 1 else -1.0 for j in range(8)]) / np.sqrt(8)
        v = u @ om
        better = v > bestv
        best[better] = c
        bestv[better] = v[better]
    clear = np.min(np.abs(u), axis=2) > 1e-6
    assert clear.mean() > 0.99
    np.testing.assert_array_equal(enc["codes"][clear], best[clear])
    np.testing.assert_array_equal(lit["codes"][clear], best[clear])


def _key_with_rotated(yprime):
    """Integer key k = s * (H y') so that the fp32 rotation gives y = 128 y' exactly."""
    H = _popcount_hadamard(128).astype(np.int64)
    return (SIGNS.astype(np.int64) * (H @ np.asarray(yprime, dtype=np.int64))).astype(np.float32)


def test_zero_coordinate_takes_bit_zero():
    yp = np.ones(128, dtype=np.int64)
    yp[0] = 0
    yp[3] = -2
    k = _key_with_rotated(yp)
    enc = O.encode_f32(k[None], SIGNS, L32, TAU32)
    np.testing.assert_array_equal(enc["y"][0], 128.0 * yp)
    lit = O.encode_literal(k[None], SIGNS, L64, TAU64)
    # y_0 = 0 -> bit 0 clear; y_3 < 0 -> bit 3 clear; the rest positive
    assert enc["codes"][0, 0] == 0b11110110
    # the fp64 dense rotation leaves a rounding residue at u_0, so the literal
    # path sees a near-tie: either maximiser is acceptable there
    assert lit["codes"][0, 0] in (0b11110110, 0b11110111)
    assert abs(lit["u"][0, 0, 0]) < 1e-12
    nib = O.unpack_nibbles(enc["nibbles"])[0]
    assert nib[0] == 0                          # sign bit 0, magnitude index 0


def test_magnitude_index_is_nearest_level():
    k = _keys(2000)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    nib = O.unpack_nibbles(enc["nibbles"])
    a = np.abs(enc["y"].reshape(-1, 16, 8).astype(np.float64))
    a = a / np.linalg.norm(a, axis=2, keepdims=True)
    a = a.reshape(-1, 128)
    nearest = np.argmin(np.abs(a[..., None] - L64[None, None, :]), axis=2)
    far = np.min(np.abs(a[..., None] - TAU64[None, None, :]), axis=2) > 1e-6
    np.testing.assert_array_equal((nib & 7)[far], nearest[far])
    # sign bit of the nibble is the code bit of that coordinate
    bits = np.stack([(enc["codes"] >> j) & 1 for j in range(8)], axis=2).reshape(-1, 128)
    np.testing.assert_array_equal(nib >> 3, bits)


def test_f32_order_agrees_with_literal_formulas():
    k = _keys(3000)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    lit = O.encode_literal(k, SIGNS, L32.astype(np.float64), TAU32.astype(np.float64))
    u = lit["u"].reshape(-1, 128)
    near0 = np.abs(u) < 1e-6
    neart = np.min(np.abs(np.abs(u)[..., None] - TAU32.astype(np.float64)), axis=2) < 1e-6
    ok = ~(near0 | neart)
    nib = O.unpack_nibbles(enc["nibbles"])
    np.testing.assert_array_equal((nib & 7)[ok], lit["mag_idx"][ok])
    np.testing.assert_allclose(enc["weights"], lit["weights"], rtol=1e-5)
    np.testing.assert_allclose(enc["norms"], lit["norms"], rtol=1e-6)


def test_rotated_blocks_follow_beta_prior():
    # isotropic keys are uniform on the sphere after any rotation, so the
    # Beta laws of Proposition 4.1 hold exactly: r_b^2 ~ Beta(m/2, (D-m)/2),
    # (u_b)_j^2 ~ Beta(1/2, (m-1)/2)
    rng = np.random.default_rng(11)
    k = rng.standard_normal((20000, 128))
    lit = O.encode_literal(k, SIGNS, L64, TAU64)
    kt = (k / np.linalg.norm(k, axis=1, keepdims=True)) @ O.rotation_matrix(SIGNS).T
    r2 = np.sum(kt.reshape(-1, 16, 8) ** 2, axis=2)
    np.testing.assert_allclose(r2.sum(axis=1), 1.0, atol=1e-12)
    a, b = 4.0, 60.0
    assert abs(r2.mean() - a / (a + b)) < 5e-4
    assert abs(r2.var() - a * b / ((a + b) ** 2 * (a + b + 1))) < 5e-5
    u2 = lit["u"] ** 2
    assert abs(u2.mean() - 1 / 8) < 2e-3


def test_zero_key_and_zero_block():
    yp = np.zeros(128, dtype=np.int64)
    yp[8:] = np.arange(1, 121) % 7 - 3
    yp[8] = 5                                   # every block but block 0 is non-zero
    for b in range(1, 16):
        if not yp[8 * b:8 * b + 8].any():
            yp[8 * b] = 1
    k = np.stack([np.zeros(128, np.float32), _key_with_rotated(yp)])
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    assert (enc["weights"][0] == 0).all() and (enc["codes"][0] == 0).all()
    assert enc["norms"][0] == 0
    assert (O.unpack_nibbles(enc["nibbles"])[0] == 0).all()
    assert (enc["y"][1, :8] == 0).all()
    assert enc["weights"][1, 0] == 0 and enc["codes"][1, 0] == 0
    assert (enc["weights"][1, 1:] > 0).all()
