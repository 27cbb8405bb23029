"""Pins of the percentile-tier votes and the adaptive ratios (oracle only).

Slides, frame "Stage I uses multi-tier collision votes to prune keys"
(Sec. 4.2.2, Eq. (15)): per block, keep the top-rho fraction of keys by their
centroid score, split it into six percentile tiers with bonuses 6..1.
README "Parameters": candidate / collision ratios by retrieval-zone length."""
import json
import os

import numpy as np
import pytest

from oracle import pariskv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def test_bonuses_and_table_match_the_pages():
    g = json.load(open(GOLDEN))
    assert list(O.PERCENTILE_BONUSES) == g["percentile_tier_bonuses"]["value"]
    rows = g["adaptive_ratios"]["rows"]
    assert len(rows) == len(O.ADAPTIVE_RATIOS_PERMILLE)
    for row, (limit, beta, rho) in zip(rows, O.ADAPTIVE_RATIOS_PERMILLE):
        assert row["zone_len_below"] == limit
        assert round(row["candidate_ratio"] * 1000) == beta
        assert round(row["collision_ratio"] * 1000) == rho


@pytest.mark.parametrize("n,expect", [(1, (500, 500)), (4999, (500, 500)), (5000, (250, 300)),
                                      (9999, (250, 300)), (10000, (200, 250)), (29999, (200, 250)),
                                      (30000, (100, 200)), (1 << 20, (100, 200))])
def test_adaptive_ratio_boundaries(n, expect):
    assert O.adaptive_ratios_permille(n) == expect


def test_ratio_count_is_exact_ceiling():
    from fractions import Fraction
    for permille in (100, 200, 250, 300, 500, 1000, 7):
        for n in (1, 3, 999, 1000, 1001, 131072, 1048576, 32768):
            want = -(-Fraction(permille, 1000) * n // 1)
            assert O.ratio_count(permille, n) == int(want)
    assert O.ratio_count(100, 131072) == 13108


def _brute_weights(scores, codes, M, bonuses=O.PERCENTILE_BONUSES):
    """Rank every key of every block explicitly: by centroid score desc, then
    centroid index, then key index; a centroid's bonus comes from the position
    of its first key (R13).  Returns [16, 256] (0 for centroids without keys
    past the kept range or with no key)."""
    n = codes.shape[0]
    w = np.zeros((O.N_SUB, O.N_CENTROIDS), dtype=np.int64)
    for b in range(O.N_SUB):
        keyed = sorted(range(n), key=lambda i: (-float(scores[b, codes[i, b]]), int(codes[i, b]), i))
        first_pos = {}
        for pos, i in enumerate(keyed):
            first_pos.setdefault(int(codes[i, b]), pos)
        for c, pos in first_pos.items():
            if pos < M:
                w[b, c] = bonuses[(len(bonuses) * pos) // M]
    return w


@pytest.mark.parametrize("n,M", [(300, 60), (300, 300), (97, 13), (500, 1), (64, 64)])
def test_percentile_tiers_brute_force(n, M):
    rng = np.random.default_rng(n * 7 + M)
    # few distinct scores so that centroids tie, and clustered codes so that
    # centroids hold many keys and straddle tier boundaries
    scores = rng.integers(-4, 5, size=(O.N_SUB, O.N_CENTROIDS)).astype(np.float32)
    codes = rng.integers(0, 12, size=(n, O.N_SUB)).astype(np.uint8) * 17
    counts = O.centroid_occupancy(codes)
    got = O.percentile_tier_weights(O.centroid_ranks(scores), counts, M)
    want = _brute_weights(scores, codes, M)
    # centroids holding no key may carry any bonus: they never vote
    present = counts > 0
    np.testing.assert_array_equal(got[present], want[present])
    # every kept key position gets exactly one tier; the kept keys are the first M or more
    S = O.collision_scores(codes, got)
    assert S.max() <= 6 * O.N_SUB


def test_percentile_single_centroid_and_uniform_cases():
    n = 256 * 6
    # one centroid per block holds every key: first position 0, bonus 6 everywhere
    codes = np.full((n, O.N_SUB), 5, dtype=np.uint8)
    scores = np.zeros((O.N_SUB, O.N_CENTROIDS), dtype=np.float32)
    w = O.percentile_tier_weights(O.centroid_ranks(scores), O.centroid_occupancy(codes), M=n // 10)
    assert (O.collision_scores(codes, w) == 6 * O.N_SUB).all()
    # every centroid holds 6 keys, scores decreasing with the centroid index:
    # with M = 6 * 60 the kept centroids are 0..59, ten per tier
    codes = np.tile(np.repeat(np.arange(256, dtype=np.uint8), 6)[:, None], (1, O.N_SUB))
    scores = np.tile(-np.arange(256, dtype=np.float32), (O.N_SUB, 1))
    w = O.percentile_tier_weights(O.centroid_ranks(scores), O.centroid_occupancy(codes), M=360)
    for b in range(O.N_SUB):
        np.testing.assert_array_equal(w[b, :60], np.repeat([6, 5, 4, 3, 2, 1], 10))
        assert (w[b, 60:] == 0).all()


def test_percentile_votes_keep_about_rho_of_each_block():
    rng = np.random.default_rng(3)
    n = 5000
    codes = rng.integers(0, 256, size=(n, O.N_SUB)).astype(np.uint8)
    scores = rng.standard_normal((O.N_SUB, O.N_CENTROIDS)).astype(np.float32)
    counts = O.centroid_occupancy(codes)
    M = O.ratio_count(200, n)
    w = O.percentile_tier_weights(O.centroid_ranks(scores), counts, M)
    for b in range(O.N_SUB):
        kept = int(counts[b][w[b] > 0].sum())
        # the kept keys cover the first M positions and at most one more centroid
        assert M <= kept <= M + counts[b].max()
