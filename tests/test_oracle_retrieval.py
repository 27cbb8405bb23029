"""Pins of the oracle's decode side: centroid scoring against dense inner
products, the estimator's closed form (exact when q is parallel to k), its
invariances, collision scores by exhaustive loops, candidate / Top-k selection
by brute-force sorting, and attention reducing to dense softmax attention."""
import numpy as np
import pytest
import torch

from oracle import pariskv_oracle as O
from workloads import synthetic as S

SIGNS = O.srht_signs(0)
L32, TAU32 = O.magnitude_tables_f32()
L64, TAU64 = O.lloyd_max_levels()
TOP, WT = (1, 4, 16), (4, 2, 1)


def _unit(n=4096, wl="tiny4k"):
    w = S.custom(wl, n=n)
    k = S.as_f32(S.unit_keys(w, 0, 0))
    v = S.as_f32(S.unit_values(w, 0, 0))
    q = S.as_f32(S.query(w, 0, 0, S.unit_keys(w, 0, 0)))
    return w, k, v, q


# ---------------------------------------------------------------------------
# query side
# ---------------------------------------------------------------------------
def test_centroid_scores_are_dense_inner_products():
    _, _, _, q = _unit()
    Rq, y, sc = O.qprep_f32(q, SIGNS)
    # dense: <q~_b, omega_c> * sqrt(m) * ||q|| * sqrt(D) = sum_j omega_j y_j (bit 1 -> +)
    R = O.rotation_matrix(SIGNS)
    yq = (R @ q.astype(np.float64)) * np.sqrt(128)
    for b in (0, 7, 15):
        for c in (0, 1, 0x80, 0xA5, 255):
            om = np.array([1.0 if (c >> j) & 1 else -1.0 for j in range(8)])
            ref = om @ yq[8 * b:8 * b + 8]
            assert abs(sc[b, c] - ref) <= 1e-5 * np.abs(yq[8 * b:8 * b + 8]).sum()
    np.testing.assert_allclose(Rq, R @ q.astype(np.float64), rtol=1e-5, atol=1e-5 * np.abs(q).max())
    # the best centroid of each block is the query's own sign pattern
    ranks = O.centroid_ranks(sc)
    for b in range(16):
        own = sum(1 << j for j in range(8) if y[8 * b + j] > 0)
        assert ranks[b, own] == 0


def test_centroid_ranks_brute_force_and_tiers():
    rng = np.random.default_rng(4)
    sc = rng.integers(-3, 4, size=(16, 256)).astype(np.float32)   # many ties
    ranks = O.centroid_ranks(sc)
    for b in (0, 3, 15):
        order = sorted(range(256), key=lambda c: (-float(sc[b, c]), c))
        for r, c in enumerate(order):
            assert ranks[b, c] == r
    wt = O.tier_weights(ranks, TOP, WT)
    assert (wt[ranks == 0] == 4).all()
    assert (wt[(ranks >= 1) & (ranks < 4)] == 2).all()
    assert (wt[(ranks >= 4) & (ranks < 16)] == 1).all()
    assert (wt[ranks >= 16] == 0).all()
    assert (np.sort(wt, axis=1)[:, ::-1][:, :16].sum(axis=1) == 4 + 3 * 2 + 12).all()


def test_collision_scores_by_exhaustive_loops():
    _, k, _, q = _unit(700)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    _, _, sc = O.qprep_f32(q, SIGNS)
    S_or = O.collision_scores(enc["codes"], O.tier_weights(O.centroid_ranks(sc), TOP, WT))
    for i in range(0, 700, 7):
        tot = 0
        for b in range(16):
            c = int(enc["codes"][i, b])
            rank = sum(1 for c2 in range(256)
                       if sc[b, c2] > sc[b, c] or (sc[b, c2] == sc[b, c] and c2 < c))
            tot += 4 if rank < 1 else 2 if rank < 4 else 1 if rank < 16 else 0
        assert S_or[i] == tot
    assert S_or.min() >= 0 and S_or.max() <= 64


# ---------------------------------------------------------------------------
# candidates and Top-k
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,C", [(1000, 100), (1000, 999), (1000, 1000), (50, 100), (0, 10)])
def test_select_candidates_brute_force(n, C):
    rng = np.random.default_rng(n + C)
    S_ = rng.integers(0, 9, size=n)                 # heavy ties
    got = O.select_candidates(S_, C)
    ref = sorted(sorted(range(n), key=lambda i: (-int(S_[i]), i))[:min(n, C)])
    assert list(got) == ref
    if 0 < C < n:
        theta = S_[got].min()
        rest = np.setdiff1d(np.arange(n), got)
        assert (S_[rest] <= theta).all()
        tied_out = rest[S_[rest] == theta]
        tied_in = got[S_[got] == theta]
        if tied_out.size and tied_in.size:
            assert tied_out.min() > tied_in.max()


def test_top_k_brute_force():
    rng = np.random.default_rng(9)
    cand = np.sort(rng.choice(5000, 700, replace=False))
    est = rng.integers(-20, 20, size=700).astype(np.float32)   # ties
    ti, te = O.top_k(est, cand, 100)
    ref = sorted(range(700), key=lambda p: (-float(est[p]), int(cand[p])))[:100]
    assert list(ti) == [int(cand[p]) for p in ref]
    assert list(te) == [float(est[p]) for p in ref]
    ti, _ = O.top_k(est[:30], cand[:30], 100)
    assert len(ti) == 30


def test_exact_topk_brute_force():
    _, k, _, q = _unit(1500)
    got = O.exact_topk(k, q, 100)
    s = k.astype(np.float64) @ q.astype(np.float64)
    ref = sorted(range(1500), key=lambda i: (-s[i], i))[:100]
    assert list(got) == ref


# ---------------------------------------------------------------------------
# estimator (Eq. (10))
# ---------------------------------------------------------------------------
def test_estimator_exact_for_parallel_query():
    _, k, _, _ = _unit(300)
    lit = O.encode_literal(k, SIGNS, L64, TAU64)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    for i in (0, 17, 299):
        for c in (1.0, 4.0, -0.25):          # powers of two: q is exactly parallel in fp32 too
            q = c * k[i].astype(np.float64)
            true = float(k[i].astype(np.float64) @ q)
            e_lit = O.estimate_literal({key: v[i:i + 1] for key, v in lit.items()}, q, SIGNS, L64)[0]
            assert abs(e_lit - true) < 1e-10 * abs(true)
            Rq, _, _ = O.qprep_f32(q.astype(np.float32), SIGNS)
            e32 = O.rerank_f32(enc["nibbles"][i:i + 1], enc["weights"][i:i + 1], Rq, L32)[0]
            e64 = O.rerank_f64(enc["nibbles"][i:i + 1], enc["weights"][i:i + 1], Rq, L32)[0]
            assert abs(e64 - true) < 2e-5 * abs(true)
            assert abs(e32 - true) < 2e-5 * abs(true)


def test_estimator_invariances():
    _, k, _, q = _unit(500)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    Rq, _, _ = O.qprep_f32(q, SIGNS)
    base = O.rerank_f32(enc["nibbles"], enc["weights"], Rq, L32)
    # doubling every level doubles alpha and v: w halves, the estimate is bit-identical
    enc2 = O.encode_f32(k, SIGNS, 2 * L32, TAU32)
    np.testing.assert_array_equal(enc2["codes"], enc["codes"])
    np.testing.assert_array_equal(enc2["nibbles"], enc["nibbles"])
    np.testing.assert_array_equal(enc2["weights"], enc["weights"] / 2)
    np.testing.assert_array_equal(O.rerank_f32(enc2["nibbles"], enc2["weights"], Rq, 2 * L32), base)
    # linear in q (fp64 evaluation)
    rng = np.random.default_rng(1)
    q2 = rng.standard_normal(128).astype(np.float32)
    lit = O.encode_literal(k, SIGNS, L64, TAU64)
    e1 = O.estimate_literal(lit, q.astype(np.float64), SIGNS, L64)
    e2 = O.estimate_literal(lit, q2.astype(np.float64), SIGNS, L64)
    e12 = O.estimate_literal(lit, q.astype(np.float64) + q2, SIGNS, L64)
    np.testing.assert_allclose(e12, e1 + e2, rtol=1e-9, atol=1e-9 * np.abs(e1).max())


def test_estimator_tracks_true_scores_and_f32_within_tolerance():
    _, k, _, q = _unit(4096)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    Rq, _, _ = O.qprep_f32(q, SIGNS)
    e32 = O.rerank_f32(enc["nibbles"], enc["weights"], Rq, L32)
    e64 = O.rerank_f64(enc["nibbles"], enc["weights"], Rq, L32)
    scale = O.rerank_abs_scale(enc["nibbles"], enc["weights"], Rq, L32)
    assert np.all(np.abs(e32 - e64) <= 1e-5 * scale)
    true = k.astype(np.float64) @ q.astype(np.float64)
    assert np.corrcoef(e64, true)[0, 1] > 0.98
    # fp32 path agrees with the literal Eq. (10) pipeline
    lit = O.encode_literal(k, SIGNS, L64, TAU64)
    e_lit = O.estimate_literal(lit, q.astype(np.float64), SIGNS, L64)
    assert np.corrcoef(e_lit, e64)[0, 1] > 0.9999


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def test_attention_with_all_keys_is_dense_attention():
    _, k, v, q = _unit(512)
    scale = 1 / np.sqrt(128)
    o = O.sparse_attention(q, k, v, np.arange(512), scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64))[None, None, None],
        torch.from_numpy(k.astype(np.float64))[None, None],
        torch.from_numpy(v.astype(np.float64))[None, None], scale=scale)[0, 0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_attention_edge_cases():
    _, k, v, _ = _unit(300)
    q0 = np.zeros(128, np.float32)
    idx = np.array([3, 9, 200, -1, -1])
    np.testing.assert_allclose(O.sparse_attention(q0, k, v, idx, 0.1),
                               v[[3, 9, 200]].astype(np.float64).mean(axis=0), rtol=1e-12)
    assert (O.sparse_attention(q0, k, v, np.array([-1, -1]), 0.1) == 0).all()


def test_pipeline_recall_on_planted_query():
    w, k, v, q = _unit(4096)
    enc = O.encode_f32(k, SIGNS, L32, TAU32)
    r = O.decode_unit(q[None], k, v, enc, SIGNS, L32, TOP, WT, w.n_candidates, 100,
                      w.softmax_scale)[0]
    assert len(r["cand"]) == 512 and len(r["top_idx"]) == 100
    exact = O.exact_topk(k, q, 100)
    recall = len(set(r["top_idx"]) & set(exact)) / 100
    assert recall > 0.5
    # the planted keys dominate the true scores and are retrieved
    assert np.all(np.abs(r["est32"] - r["est64"]) <= 1e-5 * r["abs_scale"])


def test_layout_attention_special_cases():
    """Dense + retrieved attention: no dense rows is the sparse attention; no
    retrieved rows is plain softmax attention (torch's CPU routine); the dense
    rows' order does not matter; one dominant row returns its value."""
    import torch
    rng = np.random.default_rng(11)
    K = rng.standard_normal((300, O.D)).astype(np.float32)
    V = rng.standard_normal((300, O.D)).astype(np.float32)
    Kd = rng.standard_normal((70, O.D)).astype(np.float32)
    Vd = rng.standard_normal((70, O.D)).astype(np.float32)
    q = rng.standard_normal(O.D).astype(np.float32)
    idx = np.array([5, 17, -1, 250, 3])
    scale = 1 / np.sqrt(O.D)
    np.testing.assert_allclose(O.layout_attention(q, K, V, idx, Kd[:0], Vd[:0], scale),
                               O.sparse_attention(q, K, V, idx, scale), rtol=1e-12, atol=1e-12)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[None, None, None].astype(np.float64)), torch.from_numpy(Kd[None, None].astype(np.float64)),
        torch.from_numpy(Vd[None, None].astype(np.float64)), scale=scale)[0, 0, 0].numpy()
    np.testing.assert_allclose(O.layout_attention(q, K, V, np.array([-1]), Kd, Vd, scale), ref, rtol=1e-10, atol=1e-12)
    perm = rng.permutation(70)
    np.testing.assert_allclose(O.layout_attention(q, K, V, idx, Kd, Vd, scale),
                               O.layout_attention(q, K, V, idx, Kd[perm], Vd[perm], scale), rtol=1e-12, atol=1e-12)
    Kd2 = Kd.copy()
    Kd2[7] = 100.0 * q                                 # dominates every other score
    np.testing.assert_allclose(O.layout_attention(q, K, V, idx, Kd2, Vd, scale), Vd[7], atol=1e-9)
    assert not O.layout_attention(q, K, V, np.array([-1]), Kd[:0], Vd[:0], scale).any()
