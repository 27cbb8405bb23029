"""GPU parity of the pages' own Stage I: six percentile tiers of the top
rho fraction of each block's keys (Slides Sec. 4.2.2, Eq. (15)) and the
README's adaptive candidate / collision ratios, against the oracle: centroid
counts, tier LUTs, collision scores, candidates, estimates and Top-k bit for
bit, attention within 2e-2."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S
from tests.parity_util import HipRun, check_encode_unit, check_retrieve_unit, say, to_torch

pytestmark = pytest.mark.gpu


def _run(w, units, n=None, fused=False):
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q, n=n)
    run = run.retrieve_attend() if fused else run.retrieve().attend()
    for u in units:
        b, h = divmod(u, w.n_kv_heads)
        kf = S.as_f32(K[b, h, :run.n])
        vf = S.as_f32(V[b, h, :run.n])
        enc = check_encode_unit(run, u, kf)
        check_retrieve_unit(run, b, h, kf, vf, enc)
    return run


@pytest.mark.parametrize("n,C,rho", [(3001, 512, 200), (1000, 300, 1000), (777, 256, 1)])
def test_percentile_fixed_ratio(n, C, rho):
    w = S.custom("llama32k", batch=2, n_kv_heads=2, n_q_heads=8, n=n, n_candidates=C, tier_mode="percentile",
                 collision_permille=rho, wid=600 + rho)
    say(f"case percentile n={n} C={C} rho={rho / 1000}")
    _run(w, [0, 3]).close()


@pytest.mark.parametrize("n", [4000, 9000, 20000, 40000])
def test_percentile_adaptive(n):
    """Each zone-length band of the table: C = ceil(beta n), M = ceil(rho n)."""
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=n, n_candidates=4096, tier_mode="percentile",
                 adaptive=True, wid=610 + n % 97)
    say(f"case percentile adaptive n={n}")
    _run(w, [1]).close()


def test_rank_tiers_adaptive_candidates():
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=9000, n_candidates=4096, adaptive=True, wid=620)
    say("case rank tiers, adaptive candidates n=9000")
    _run(w, [0]).close()


def test_percentile_many_heads_fused_call():
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=3000, n_candidates=1600, tier_mode="percentile",
                 adaptive=True, wid=630)
    say("case percentile adaptive, 128 heads, fused call")
    _run(w, [0, 31], fused=True).close()


def test_adaptive_candidates_over_capacity_is_an_error():
    from kv_cache_top_amd import pariskv as P
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=4000, n_candidates=1000, adaptive=True, wid=640)
    say("case adaptive C over capacity")
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q)
    with pytest.raises(P.PkError) as e:
        run.retrieve()                              # ceil(0.5 * 4000) = 2000 > 1000
    assert e.value.status == P.PK_ERR_CAPACITY
    run.close()


def test_percentile_counts_follow_appends():
    """Counts recounted on encode and advanced on append; retrieval after appends."""
    from kv_cache_top_amd import pariskv as P
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=2600, n_candidates=600, tier_mode="percentile",
                 collision_permille=250, wid=650)
    say("case percentile with appends")
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q, n=2000, capacity=2600)
    for t0 in range(2000, 2600, 150):
        P.pk_append_keys(run.ctx.h, to_torch(K[:, :, t0:t0 + 150]), run.sums.s)
    assert run.n == 2600
    run.retrieve().attend()
    for u in range(w.units):
        b, h = divmod(u, w.n_kv_heads)
        kf = S.as_f32(K[b, h])
        enc = check_encode_unit(run, u, kf)
        check_retrieve_unit(run, b, h, kf, S.as_f32(V[b, h]), enc)
    # re-encoding from scratch recounts
    P.pk_encode_keys(run.ctx.h, run.Kt[:, :, :500], run.sums.s)
    import torch
    torch.cuda.synchronize()
    c = run.sums.counts_view().cpu().numpy()
    assert (c.sum(axis=2) == 500).all()
    run.close()
