"""GPU parity of the single retrieve + attend call (pk_retrieve_attend) against
the oracle, on the paths it can take: the fused rerank + top-k + attention
workgroup (at most 4096 candidates per head with 128 or more heads, at most
1024 otherwise), the rerank spread over workgroups followed by one top-k +
attention workgroup per head (more candidates), the attention kernel after
either (mixed dtypes), mapped host K/V and the empty key set."""
import numpy as np
import pytest

from workloads import synthetic as S
from tests.parity_util import HipRun, check_encode_unit, check_retrieve_unit, say

pytestmark = pytest.mark.gpu


def _run(w, units, kv_host=False, out_dtype="match", n=None):
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q, kv_host=kv_host, n=n).retrieve_attend(out_dtype=out_dtype)
    for u in units:
        b, h = divmod(u, w.n_kv_heads)
        kf = S.as_f32(K[b, h, :run.n])
        vf = S.as_f32(V[b, h, :run.n])
        enc = check_encode_unit(run, u, kf)
        check_retrieve_unit(run, b, h, kf, vf, enc)
    return run


def test_fused_tiny_fp32():
    say("case fused tiny4k fp32")
    _run(S.WORKLOADS["tiny4k"], [0]).close()


@pytest.mark.parametrize("n,C,k", [(3001, 256, 100), (2500, 1800, 100), (2500, 1800, 200)])
def test_fused_many_heads(n, C, k):
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=n, n_candidates=C, top_k=k, wid=500 + C + k)
    say(f"case fused 128 heads n={n} C={C} k={k}")
    _run(w, [0, 17, 31]).close()


def test_split_path_then_attention():
    """Few heads and many candidates: the rerank spread over workgroups, then
    the top-k workgroup of each head attends over its rows."""
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=9000, n_candidates=4096, wid=520)
    say("case split path n=9000 C=4096")
    _run(w, [0, 1]).close()


def test_mixed_dtype_output():
    """bf16 K/V with an fp32 output: retrieval fused, attention as its own kernel."""
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=1500, n_candidates=300, wid=530)
    say("case fused retrieval, fp32 output")
    _run(w, [5], out_dtype="f32").close()


def test_fused_mapped_host_kv():
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=2000, n_candidates=512, wid=540)
    say("case fused, K/V in mapped host memory")
    _run(w, [0, 30], kv_host=True).close()


def test_fused_empty():
    w = S.custom("llama32k", batch=4, n_kv_heads=8, n_q_heads=32, n=16, n_candidates=64, top_k=10, wid=550)
    say("case fused, empty key set")
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    run = HipRun(w, K, V, Q, n=0).retrieve_attend()
    assert (run.topk_idx.cpu().numpy() == -1).all()
    assert (run.out.float().cpu().numpy() == 0).all()
    run.close()


@pytest.mark.parametrize("batch,n_kv,n_q,n,C", [(1, 2, 8, 3000, 1024), (1, 2, 8, 3000, 1025),
                                                 (4, 8, 32, 5000, 4096), (4, 8, 32, 5000, 4097)])
def test_path_boundaries(batch, n_kv, n_q, n, C):
    """Candidate counts on both sides of the switch between the fused workgroup
    and the spread rerank, with few (8) and many (128) query heads."""
    w = S.custom("llama32k", batch=batch, n_kv_heads=n_kv, n_q_heads=n_q, n=n, n_candidates=C, wid=560 + C % 97)
    say(f"case path boundary heads={batch * n_q} C={C}")
    _run(w, [0, 1] if w.units <= 2 else [0, 13, 31]).close()


@pytest.mark.parametrize("k", [1, 256])
def test_spread_path_top_k_extremes(k):
    """k = 1 and k = 256 on the spread rerank with attention in the top-k workgroup."""
    w = S.custom("llama32k", batch=1, n_kv_heads=2, n_q_heads=8, n=4000, n_candidates=2000, top_k=k, wid=570 + k)
    say(f"case spread path k={k}")
    _run(w, [0, 1]).close()


def test_spread_path_fp32():
    """fp32 q / K / V / output on the spread rerank with attention in the top-k workgroup."""
    w = S.custom("tiny4k", n=3000, n_candidates=1500, wid=580)
    say("case spread path fp32")
    _run(w, [0]).close()
