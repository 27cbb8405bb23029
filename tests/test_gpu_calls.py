"""GPU parity across calls and at the method's degenerate sizes: back-to-back
calls of different sizes on one context, many repeated calls (identical
results), one key, fewer keys than one wave's share of a tile, and n <= C
(every key a candidate).  Every result is compared with the oracle bit for
bit, and the device-side consistency flags stay clear."""
import numpy as np
import pytest

from workloads import synthetic as S
from tests.parity_util import HipRun, check_encode_unit, check_retrieve_unit, oracle_encode, say

pytestmark = pytest.mark.gpu


def _inputs(w, n=None):
    K = S.all_keys(w, n)
    V = S.all_values(w, n)
    Q = S.all_queries(w, K)
    return K, V, Q


@pytest.mark.parametrize("case", ["one_key", "partial_wave", "all_taken"])
def test_degenerate_sizes(case):
    if case == "one_key":
        w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=1, n_candidates=16, top_k=4, wid=1403)
    elif case == "partial_wave":   # fewer keys than one wave's share of a tile
        w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=4, n=70, n_candidates=32, top_k=8, wid=1404)
    else:                          # n <= C: theta = 0, every key is a candidate
        w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=900, n_candidates=1024, wid=1402)
    say(f"case {case} units={w.units} n={w.n} C={w.n_candidates}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve_attend()
    for u in range(w.units):
        b, h = divmod(u, w.n_kv_heads)
        kf, vf = S.as_f32(K[b, h]), S.as_f32(V[b, h])
        check_retrieve_unit(run, b, h, kf, vf, check_encode_unit(run, u, kf))
    assert run.device_errors() == 0
    run.close()


def test_back_to_back_calls_of_different_sizes():
    """One context, n shrinking and growing between calls (the tiling and the
    selection parameters change with n): every call matches the oracle."""
    w = S.custom("llama32k", batch=2, n_kv_heads=4, n_q_heads=16, n=9000, n_candidates=512, wid=1410)
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q, n=9000)
    for n in (9000, 2049, 9000, 64, 5000):
        say(f"case back-to-back n={n}")
        run.sums.s.n = n
        run.retrieve()
        for u in (0, 5):
            b, h = divmod(u, w.n_kv_heads)
            kf = S.as_f32(K[b, h, :n])
            vf = S.as_f32(V[b, h, :n])
            # the summaries hold all 9000 keys; a call reads the first n
            check_retrieve_unit(run, b, h, kf, vf, oracle_encode(kf), check_attention=False)
    assert run.device_errors() == 0
    run.close()


def test_repeated_calls_identical():
    """Fifty calls on one context give identical candidates, estimates and Top-k."""
    import torch
    w = S.custom("llama32k", batch=2, n_kv_heads=8, n_q_heads=32, n=20000, n_candidates=1024, wid=1411)
    say(f"case repeated units={w.units} n={w.n}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve()
    ref = [t.clone() for t in (run.cand_idx, run.cand_est, run.topk_idx, run.topk_est)]
    for _ in range(50):
        run.retrieve()
        for a, b in zip((run.cand_idx, run.cand_est, run.topk_idx, run.topk_est), ref):
            assert torch.equal(a, b)
    assert run.device_errors() == 0
    run.close()


def test_two_launch_geometries_same_results():
    """Units (0, 0) and (0, 1) alone (2 units, 8 query heads: small tiles, the
    rerank spread over workgroups, then a top-k kernel) and inside a batch of
    64 units (256 query heads: large tiles, rerank and top-k in one workgroup
    per head) see the same keys and queries: candidates, estimates and Top-k
    are bit-identical, attention within the fp32 summation-order tolerance."""
    import torch
    from tests.parity_util import attention_ok
    small = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=20000, n_candidates=1024, wid=1420)
    big = S.custom("llama32k", batch=8, n_kv_heads=8, n_q_heads=32, n=20000, n_candidates=1024, wid=1420)
    runs = []
    for w in (small, big):
        say(f"case geometry units={w.units}")
        K = S.all_keys(w)
        V = S.all_values(w)
        Q = S.all_queries(w, K)
        runs.append(HipRun(w, K, V, Q).retrieve_attend())
    a, b = runs
    np.testing.assert_array_equal(a.Q[0, :8], b.Q[0, :8])          # same inputs for these heads
    for t_a, t_b in ((a.cand_idx, b.cand_idx), (a.cand_est, b.cand_est)):
        assert torch.equal(t_a[:8], t_b[:8])
    assert torch.equal(a.topk_idx[0, :8], b.topk_idx[0, :8])
    assert torch.equal(a.topk_est[0, :8], b.topk_est[0, :8])
    for qh in range(8):
        assert attention_ok(a.out[0, qh].float().cpu().numpy(), b.out[0, qh].float().cpu().numpy())
    for r in runs:
        assert r.device_errors() == 0
        r.close()


def test_many_short_sub_tiles():
    """One unit of 300,000 keys: short tiles (768 keys at one unit), about
    1,560 sub-tiles, so a select workgroup near the end sums the suffix counts
    of 25 chunks of 64 earlier sub-tiles, requested four chunks at a time;
    every intermediate and the Top-k match the oracle bit for bit."""
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=4, n=300000, n_candidates=4096, wid=1430)
    say(f"case many sub-tiles units={w.units} n={w.n} C={w.n_candidates}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve_attend()
    kf, vf = S.as_f32(K[0, 0]), S.as_f32(V[0, 0])
    check_retrieve_unit(run, 0, 0, kf, vf, check_encode_unit(run, 0, kf))
    assert run.device_errors() == 0
    run.close()
