"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on small
and ragged shapes and the edge cases of the method.  Codes, nibbles, weights,
rotated queries, tier tables, collision scores, candidates, fp32 estimates and
Top-k are compared bit for bit; estimates also within 1e-5 of the fp64
estimator (relative to sum |w_b v_j Rq_j|); attention within 2e-2 of fp64."""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S
from tests.parity_util import HipRun, check_encode_unit, check_retrieve_unit, oracle_encode, say, tables

pytestmark = pytest.mark.gpu


def _inputs(w, n=None):
    K = S.all_keys(w, n)
    V = S.all_values(w, n)
    Q = S.all_queries(w, K)
    return K, V, Q


def _check_all_units(run, K, V, units=None):
    w = run.w
    for u in (range(w.units) if units is None else units):
        b, h = divmod(u, w.n_kv_heads)
        kf = S.as_f32(K[b, h, :run.n])
        vf = S.as_f32(V[b, h, :run.n])
        enc = check_encode_unit(run, u, kf)
        check_retrieve_unit(run, b, h, kf, vf, enc)


def test_tiny_single_head_fp32():
    w = S.WORKLOADS["tiny4k"]
    say("case tiny4k fp32 n=4096 C=512")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


@pytest.mark.parametrize("n", [3001, 4096, 777])
def test_gqa_ragged_bf16(n):
    w = S.custom("llama32k", batch=2, n_kv_heads=2, n_q_heads=8, n=n, n_candidates=256, wid=100 + n)
    say(f"case gqa bf16 n={n}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


@pytest.mark.parametrize("group", [1, 2, 3])
def test_group_sizes(group):
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=2 * group, n=2500, n_candidates=300,
                 wid=200 + group)
    say(f"case group={group}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


@pytest.mark.parametrize("n,C", [(3001, 256), (2500, 1800)])
def test_many_heads_one_workgroup_topk(n, C):
    """128 query heads: rerank and top-k run in one workgroup per head."""
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=n, n_candidates=C, wid=260 + C)
    say(f"case 128 heads n={n} C={C}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V, units=[0, 13, 31])
    run.close()


@pytest.mark.parametrize("batch,n_kv,n_q,n", [(1, 1, 4, 20000), (4, 8, 32, 17000)])
def test_maximum_candidates_and_top_k(batch, n_kv, n_q, n):
    """C = 16384 and k = 256, the largest the ABI takes, with 4 and with 128
    query heads: the rerank spread over 1024-candidate workgroups, then one
    top-k workgroup per head over sixteen slots per thread."""
    from kv_cache_top_amd import pariskv as P
    C, k = P.PK_MAX_CANDIDATES, P.PK_MAX_TOPK
    w = S.custom("llama32k", batch=batch, n_kv_heads=n_kv, n_q_heads=n_q, n=n, n_candidates=C, top_k=k,
                 wid=270 + n_q)
    say(f"case maximum C={C} k={k} heads={batch * n_q} n={n}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V, units=None if w.units == 1 else [0, 31])
    run.close()


def test_many_subtiles_single_unit():
    """One KV head with a long ragged key range: the selection's per-sub-tile
    prefix counts span several 256-sub-tile chunks."""
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=4, n=70001, n_candidates=1024, wid=250)
    say("case single unit n=70001 C=1024")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


@pytest.mark.parametrize("n,C,k", [(200, 256, 100), (50, 256, 100), (1, 16, 8), (513, 512, 100), (100, 100, 100)])
def test_small_n_edges(n, C, k):
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=4, n=n, n_candidates=C, top_k=k, wid=300 + n)
    say(f"case small n={n} C={C} k={k}")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


def test_empty_key_set():
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=4, n=16, n_candidates=64, top_k=10, wid=400)
    say("case empty")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q, n=0).retrieve().attend()
    assert run.n == 0
    assert (run.topk_idx.cpu().numpy() == -1).all()
    assert np.isneginf(run.topk_est.cpu().numpy()).all()
    assert (run.out.float().cpu().numpy() == 0).all()
    run.close()


def test_zero_keys_and_zero_query():
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=2, n=1000, n_candidates=128, wid=500)
    say("case zero keys / zero query")
    K, V, Q = _inputs(w)
    K[0, 0, 10:20] = 0          # bf16 +0
    Q[0, 1] = 0                 # a zero query: all centroid scores tie
    run = HipRun(w, K, V, Q).retrieve().attend()
    _check_all_units(run, K, V)
    run.close()


def test_deterministic_repeat():
    w = S.custom("llama32k", batch=2, n_kv_heads=2, n_q_heads=8, n=5000, n_candidates=400, wid=600)
    say("case determinism")
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q).retrieve().attend()
    a = [t.cpu().numpy().copy() for t in (run.topk_idx, run.topk_est, run.cand_idx, run.cand_est, run.out.float())]
    run.retrieve().attend()
    b = [t.cpu().numpy() for t in (run.topk_idx, run.topk_est, run.cand_idx, run.cand_est, run.out.float())]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    run.close()


def test_append_equals_full_encode():
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=3000, n_candidates=256, wid=700)
    say("case append")
    K, V, Q = _inputs(w)
    full = HipRun(w, K, V, Q)
    # encode the first 2000 rows; attention later reads all 3000 rows of K / V
    part = HipRun(w, K, V, Q, n=2000, capacity=3000)
    from kv_cache_top_amd import pariskv as P
    from tests.parity_util import to_torch
    P.pk_append_keys(part.ctx.h, to_torch(K[:, :, 2000:2990]), part.sums.s)
    for t in range(2990, 3000, 4):          # several small appends, ragged last one
        P.pk_append_keys(part.ctx.h, to_torch(K[:, :, t:min(t + 4, 3000)]), part.sums.s)
    import torch
    torch.cuda.synchronize()
    assert part.n == 3000
    for u in range(w.units):
        np.testing.assert_array_equal(part.sums.codes_view()[u, :3000].cpu().numpy(),
                                      full.sums.codes_view()[u, :3000].cpu().numpy())
        np.testing.assert_array_equal(part.sums.records_view()[u, :3000].cpu().numpy(),
                                      full.sums.records_view()[u, :3000].cpu().numpy())
    # centroid counts: workgroup-aggregated (long encodes) and per-key (short appends) agree
    np.testing.assert_array_equal(part.sums.counts_view().cpu().numpy(), full.sums.counts_view().cpu().numpy())
    assert int(full.sums.counts_view()[0].sum()) == 16 * 3000
    part.retrieve().attend()
    _check_all_units(part, K, V)
    full.close()
    part.close()


def test_capacity_and_argument_errors():
    from kv_cache_top_amd import pariskv as P
    w = S.custom("llama32k", batch=1, n_kv_heads=1, n_q_heads=1, n=64, n_candidates=32, top_k=8, wid=800)
    K, V, Q = _inputs(w)
    run = HipRun(w, K, V, Q)
    from tests.parity_util import to_torch
    with pytest.raises(P.PkError) as ei:
        P.pk_append_keys(run.ctx.h, to_torch(K[:, :, :1]), run.sums.s)
    assert ei.value.status == P.PK_ERR_CAPACITY
    assert run.n == 64
    import torch
    out = torch.zeros((1, 1, 8), dtype=torch.int32, device="cuda")
    strided_q = torch.zeros((1, 1, 256), dtype=torch.bfloat16, device="cuda")[:, :, ::2]
    with pytest.raises(ValueError):
        P.pk_retrieve(run.ctx.h, strided_q, run.sums.s, out)
    # a NULL output is rejected by the library before anything is enqueued
    import ctypes
    st = P._lib.pk_retrieve(run.ctx.h, ctypes.c_void_p(run.Qt.data_ptr()), P.PK_BF16, ctypes.byref(run.sums.s),
                            None, None, None, None)
    assert st == P.PK_ERR_INVALID_ARG
    # q is read with 16-byte vector loads: a q that is only 8-byte aligned is refused
    qbuf = torch.zeros(128 + 8, dtype=torch.bfloat16, device="cuda")
    for call in (lambda qp: P._lib.pk_retrieve(run.ctx.h, qp, P.PK_BF16, ctypes.byref(run.sums.s),
                                               ctypes.c_void_p(out.data_ptr()), None, None, None),
                 lambda qp: P._lib.pk_sparse_attend(run.ctx.h, qp, P.PK_BF16, ctypes.c_void_p(run.Kt.data_ptr()),
                                                    ctypes.c_void_p(run.Vt.data_ptr()), P.PK_BF16,
                                                    P._strides4(run.Kt), run.Kt.shape[2],
                                                    ctypes.c_void_p(out.data_ptr()),
                                                    ctypes.c_void_p(qbuf.data_ptr()), P.PK_BF16, None)):
        assert call(ctypes.c_void_p(qbuf.data_ptr() + 8)) == P.PK_ERR_INVALID_ARG
        assert "16-byte" in P.pk_last_error(run.ctx.h)
    assert run.device_errors() == 0
    run.close()
