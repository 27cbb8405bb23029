"""GPU check of the recall studies (kv_cache_top_amd/studies.py): a small
drift stream (8192 prefill keys plus 64 appended keys per KV head, 2 KV heads
of 4 query heads) run through the library gives, at every measured step, the
same Stage-I-only, candidate and final recall@100 as the oracle's decode of the
same keys and queries against the oracle's exact Top-k (fp64, ties to the
lower index).  Recall itself is a property of the synthetic data (parity
unpinned); what is checked is that the studies compute it from results equal
to the oracle's."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S
from tests.parity_util import oracle_encode, say, tables

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["rank", "percentile"])
def test_drift_study_recalls_equal_oracle(mode):
    from kv_cache_top_amd import studies
    kw = dict(batch=1, n_kv_heads=2, n_q_heads=8, n=8192, n_candidates=512, append_steps=64, wid=1700)
    if mode == "percentile":
        kw.update(tier_mode="percentile", adaptive=True, n_candidates=2100)
    w = S.custom("drift128k", **kw)
    say(f"case drift study {mode} n={w.n}+{w.append_steps}")
    rows, Kall = studies.drift_stream(w, every=16)
    assert [r["step"] for r in rows] == [0, 16, 32, 48, 64]
    signs, L32, _ = tables()
    encs = [oracle_encode(S.as_f32(Kall[0, h])) for h in range(w.n_kv_heads)]
    for r in rows:
        n_t, Q = r["n"], r["_Q"]
        C = O.ratio_count(O.adaptive_ratios_permille(n_t)[0], n_t) if w.adaptive else w.n_candidates
        M = O.ratio_count(O.adaptive_ratios_permille(n_t)[1], n_t) if mode == "percentile" else None
        st, cr, fr = [], [], []
        for h in range(w.n_kv_heads):
            kf = S.as_f32(Kall[0, h, :n_t])
            qs = S.as_f32(Q[0, h * w.group:(h + 1) * w.group])
            res = O.decode_unit(qs, kf, np.zeros_like(kf), encs[h], signs, L32, w.tier_top, w.tier_weight, C,
                                w.top_k, w.softmax_scale, n=n_t, percentile_M=M)
            for g in range(w.group):
                ex = O.exact_topk(kf, qs[g], w.top_k)
                a, b, c = studies.head_recalls(ex, res[g]["S"], res[g]["cand"], res[g]["top_idx"])
                st.append(a)
                cr.append(b)
                fr.append(c)
        assert r["stage1_top_k_recall"] == round(float(np.mean(st)), 4), r
        assert r["candidate_recall"] == round(float(np.mean(cr)), 4), r
        assert r["final_recall"] == round(float(np.mean(fr)), 4), r
