"""GPU check of pk_retrieve_attend_noalloc (the entry point for callers that
cannot allocate device memory) through the C ABI: on two calls in a row, the
second over fewer keys, it gives exactly what pk_retrieve_attend gives with a
context on the same inputs (indices, estimates and attention outputs bit for
bit, and Top-k equal to the oracle's); a call whose scratch would exceed the
static array is refused before anything is enqueued."""
import pytest

from workloads import synthetic as S
from tests.parity_util import HipRun, check_retrieve_unit, oracle_encode, say

pytestmark = pytest.mark.gpu


def test_noalloc_matches_context_call_twice():
    import torch
    from kv_cache_top_amd import pariskv as P
    w = S.custom("llama32k", batch=2, n_kv_heads=4, n_q_heads=16, n=9000, n_candidates=1024, wid=1500)
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q, debug=False)
    for n in (9000, 3001):                       # the second call over fewer keys
        say(f"case noalloc n={n}")
        run.sums.s.n = n
        run.retrieve_attend()                    # the context call
        ref = [t.clone() for t in (run.topk_idx, run.topk_est, run.out)]
        idx = torch.full_like(run.topk_idx, -7)
        est = torch.zeros_like(run.topk_est)
        out = torch.zeros_like(run.out)
        P.pk_retrieve_attend_noalloc(run.cfg, run.Qt, run.sums.s, run.Kt, run.Vt, idx, out, est)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]), f"top-k indices differ at n={n}"
        assert torch.equal(est, ref[1]), f"top-k estimates differ at n={n}"
        assert torch.equal(out, ref[2]), f"attention outputs differ at n={n}"
        # and the oracle's Top-k on two units
        run.topk_idx, run.topk_est = idx, est
        for u in (0, w.units - 1):
            b, h = divmod(u, w.n_kv_heads)
            kf, vf = S.as_f32(K[b, h, :n]), S.as_f32(V[b, h, :n])
            check_retrieve_unit(run, b, h, kf, vf, oracle_encode(kf), check_attention=False)
    run.close()


def test_noalloc_refuses_oversized_call():
    import torch
    from kv_cache_top_amd import pariskv as P
    cfg = P.make_config(8, 8, 32, 1 << 20, 8192)     # 64 units x 2^20 keys: 256 MiB of scores
    sums = P.pk_summaries(1 << 10, 1 << 10, 1 << 10, 0, 1 << 20, 1 << 20)
    q = torch.zeros((8, 32, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((8, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((8, 32, 100), dtype=torch.int32, device="cuda")
    out = torch.zeros((8, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(P.PkError) as ei:
        P.pk_retrieve_attend_noalloc(cfg, q, sums, kv, kv, idx, out)
    assert ei.value.status == P.PK_ERR_CAPACITY
    assert "static scratch" in str(ei.value)
    assert int(idx.abs().sum()) == 0                 # nothing was enqueued
