"""Retrieval + attention captured in a HIP graph (through torch.cuda.graph, on
the capturing stream): pk_retrieve_attend with a context and
pk_retrieve_attend_noalloc allocate nothing per call and enqueue only kernel
launches (no memset or copy nodes), so the captured call can be replayed.
Each replay, with new query contents written into the captured input between
replays and eager work and synchronisations in between, gives bit for bit the
eager call's indices, estimates and attention outputs."""
import pytest

from workloads import synthetic as S
from tests.parity_util import HipRun, say, to_torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("entry", ["context", "noalloc"])
def test_captured_retrieval_replays_equal_eager(entry):
    import torch
    from kv_cache_top_amd import pariskv as P
    w = S.custom("llama32k", batch=1, n_kv_heads=4, n_q_heads=16, n=12000, n_candidates=1024, wid=1900)
    K = S.all_keys(w)
    V = S.all_values(w)
    Qs = [S.all_queries(w, K, step=s) for s in range(3)]
    run = HipRun(w, K, V, Qs[0], debug=False)
    q = to_torch(Qs[0]).contiguous()
    idx = torch.full((w.batch, w.n_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
    est = torch.zeros((w.batch, w.n_q_heads, w.top_k), dtype=torch.float32, device="cuda")
    out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")

    def call():
        if entry == "context":
            P.pk_retrieve_attend(run.ctx.h, q, run.sums.s, run.Kt, run.Vt, idx, out, est)
        else:
            P.pk_retrieve_attend_noalloc(run.cfg, q, run.sums.s, run.Kt, run.Vt, idx, out, est)

    # eager references, one per query set
    refs = []
    for Q in Qs:
        q.copy_(to_torch(Q))
        call()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in (idx, est, out)])
    say(f"case graph {entry}: capturing")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(6):
        s = rep % 3
        q.copy_(to_torch(Qs[s]))
        for t in (idx, est, out):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((idx, est, out), refs[s]):
            assert torch.equal(a, b), f"replay {rep} ({entry}) differs from the eager call"
        call()                                   # eager work between replays
        torch.cuda.synchronize()
    assert run.device_errors() == 0
    run.close()
