"""pk_append_retrieve_attend, one decode step in one call (README "2. Decode":
new keys are encoded as they arrive, then the query retrieves): over several
steps it gives the same summaries, Top-k, estimates and attention output, bit
for bit, as pk_append_keys followed by pk_retrieve_attend, on every path (new
rows encoded inside the query-prep launch with rank tiers and t <= 64, by
their own launch otherwise), and the last step's Top-k and attention match
the oracle."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S
from tests.parity_util import attention_ok, call_sizes, oracle_encode, say, tables, to_torch

pytestmark = pytest.mark.gpu

# (label, base, overrides, prefill rows n0, steps, rows per step t)
CASES = [
    ("g4_bf16_t1", "llama32k", dict(batch=1, n_kv_heads=2, n_q_heads=8, n_candidates=512, wid=1801), 5000, 3, 1),
    ("g1_f32_t3", "tiny4k", dict(batch=2, n_kv_heads=1, n_q_heads=1, n_candidates=256, top_k=32, wid=1802),
     3000, 3, 3),
    ("g2_t64", "llama32k", dict(batch=1, n_kv_heads=2, n_q_heads=4, n_candidates=300, wid=1803), 4000, 2, 64),
    ("g4_t65_own_launch", "llama32k", dict(batch=1, n_kv_heads=2, n_q_heads=8, n_candidates=300, wid=1804),
     4000, 2, 65),
    ("g3_from_empty", "llama32k", dict(batch=1, n_kv_heads=2, n_q_heads=6, n_candidates=64, top_k=16, wid=1805),
     0, 3, 2),
    ("no_new_rows", "llama32k", dict(batch=1, n_kv_heads=2, n_q_heads=8, n_candidates=256, wid=1806), 3000, 2, 0),
    ("percentile", "batched128k_pct", dict(batch=1, n_kv_heads=2, n_q_heads=8, n_candidates=4000, wid=1807),
     6000, 2, 1),
]


@pytest.mark.parametrize("label,base,kw,n0,steps,t", CASES, ids=[c[0] for c in CASES])
def test_decode_step_equals_separate_calls(label, base, kw, n0, steps, t):
    import torch
    from kv_cache_top_amd import pariskv as P
    cap = n0 + steps * t
    w = S.custom(base, n=cap, **kw)
    say(f"case {label}: n0={n0} steps={steps} t={t}")
    K = S.all_keys(w)
    V = S.all_values(w)
    cfg = P.make_config(w.batch, w.n_kv_heads, w.n_q_heads, max(cap, 1), w.n_candidates, w.top_k,
                        w.softmax_scale, w.srht_seed, w.tier_top, w.tier_weight,
                        P.PK_TIERS_PERCENTILE if w.tier_mode == "percentile" else P.PK_TIERS_RANK,
                        w.collision_permille, w.adaptive)
    Kt, Vt = to_torch(K), to_torch(V)
    ctx = [P.Context(cfg), P.Context(cfg)]
    sums = [P.Summaries(cfg), P.Summaries(cfg)]
    for c, s in zip(ctx, sums):
        if n0:
            P.pk_encode_keys(c.h, Kt[:, :, :n0], s.s)
    odt = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float32
    res = [None, None]
    n = n0
    for step in range(steps):
        n += t
        Q = S.all_queries(w, K[:, :, :n], step=step)
        q = to_torch(Q)
        new = Kt[:, :, n - t:n]
        for j in range(2):
            idx = torch.full((w.batch, w.n_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
            est = torch.zeros((w.batch, w.n_q_heads, w.top_k), dtype=torch.float32, device="cuda")
            out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=odt, device="cuda")
            if j == 0:
                if t:
                    P.pk_append_keys(ctx[0].h, new, sums[0].s)
                P.pk_retrieve_attend(ctx[0].h, q, sums[0].s, Kt, Vt, idx, out, est)
            else:
                P.pk_append_retrieve_attend(ctx[1].h, new, q, sums[1].s, Kt, Vt, idx, out, est)
            res[j] = (idx, est, out)
        torch.cuda.synchronize()
        assert sums[0].n == sums[1].n == n
        for a, b in zip(res[0], res[1]):
            assert torch.equal(a, b), f"{label} step {step}"
    for view in ("codes_view", "records_view", "norms_view", "counts_view"):
        assert torch.equal(getattr(sums[0], view)()[:, :n] if view != "counts_view" else sums[0].counts_view(),
                           getattr(sums[1], view)()[:, :n] if view != "counts_view" else sums[1].counts_view())
    for c in ctx:
        assert P.pk_device_errors(c.h) == 0
    # the last step against the oracle
    if n:
        signs, L32, _ = tables()
        idx, est, out = (r.cpu() for r in res[1])
        C, M = call_sizes(w, n)
        for u in range(w.units):
            b, h = divmod(u, w.n_kv_heads)
            kf, vf = S.as_f32(K[b, h, :n]), S.as_f32(V[b, h, :n])
            qs = S.as_f32(Q[b, h * w.group:(h + 1) * w.group])
            ref = O.decode_unit(qs, kf, vf, oracle_encode(kf), signs, L32, w.tier_top, w.tier_weight, C, w.top_k,
                                w.softmax_scale, n=n, percentile_M=M)
            keff = min(w.top_k, n, C)
            for g in range(w.group):
                qh = h * w.group + g
                np.testing.assert_array_equal(idx[b, qh, :keff].numpy(), ref[g]["top_idx"])
                np.testing.assert_array_equal(est[b, qh, :keff].numpy(), ref[g]["top_est"])
                assert attention_ok(out[b, qh].float().numpy(), ref[g]["out"])
    for c in ctx:
        c.close()
