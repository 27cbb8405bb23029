"""CPU checks of the recall-study helpers (kv_cache_top_amd/studies.py) against
the oracle: the exact Top-k is the definition (fp64 inner products, ties to
the lower key index), Stage-I Top-k ranks by (S desc, index asc), and the
per-head recalls are the set overlaps of those lists with the oracle's
candidates and Top-k."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S

torch = pytest.importorskip("torch")
studies = pytest.importorskip("kv_cache_top_amd.studies")


def test_exact_topk_matches_oracle_including_ties():
    rng = np.random.default_rng(7)
    K = rng.standard_normal((3000, 128)).astype(np.float32)
    K[100] = K[2000]          # exact ties: the lower index must win
    K[5] = K[2999]
    Q = rng.standard_normal((4, 128)).astype(np.float32)
    Q[1] = K[2000]            # the tied rows are the best match of head 1
    Q[2] = K[2999]
    got = studies.exact_topk_fp64(torch.from_numpy(K), torch.from_numpy(Q), 100)
    for g in range(4):
        np.testing.assert_array_equal(got[g], O.exact_topk(K, Q[g], 100))
    assert got[1][0] == 100 and got[2][0] == 5


def test_exact_topk_bf16_keys_and_short_lists():
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=2, n=50, n_candidates=32, wid=1600)
    K = S.all_keys(w)
    Q = S.all_queries(w, K)
    kt = torch.from_numpy(K[0, 0].view(np.int16)).view(torch.bfloat16)
    qt = torch.from_numpy(Q[0].view(np.int16)).view(torch.bfloat16)
    got = studies.exact_topk_fp64(kt, qt, 100)          # k > n: every key, ranked
    for g in range(2):
        np.testing.assert_array_equal(got[g], O.exact_topk(S.as_f32(K[0, 0]), S.as_f32(Q[0, g]), 100))


def test_stage1_topk_brute_force():
    rng = np.random.default_rng(3)
    Sx = rng.integers(0, 6, size=500)
    got = studies.stage1_topk(Sx, 40)
    ref = sorted(range(500), key=lambda i: (-int(Sx[i]), i))[:40]
    np.testing.assert_array_equal(got, ref)


def test_head_recalls_from_oracle_decode():
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=4, n=4000, n_candidates=400, wid=1601)
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    kf, vf, qs = S.as_f32(K[0, 0]), S.as_f32(V[0, 0]), S.as_f32(Q[0])
    signs = O.srht_signs(0)
    L32, T32 = O.magnitude_tables_f32()
    enc = O.encode_f32(kf, signs, L32, T32)
    res = O.decode_unit(qs, kf, vf, enc, signs, L32, w.tier_top, w.tier_weight, w.n_candidates, w.top_k,
                        w.softmax_scale)
    for g in range(4):
        ex = O.exact_topk(kf, qs[g], w.top_k)
        st, c, f = studies.head_recalls(ex, res[g]["S"], res[g]["cand"], res[g]["top_idx"])
        e = set(ex.tolist())
        by_s = sorted(range(w.n), key=lambda i: (-int(res[g]["S"][i]), i))[:w.top_k]
        assert st == len(e & set(by_s)) / 100
        assert c == len(e & set(res[g]["cand"].tolist())) / 100
        assert f == len(e & set(res[g]["top_idx"].tolist())) / 100
        assert f <= c                              # the final Top-k comes from the candidates
