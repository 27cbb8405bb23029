"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one pk_retrieve_attend call per step): the whole workload
runs on the GPU; the oracle recomputes sampled units (every intermediate bit
for bit, attention within 2e-2).

  llama32k     1 x 8 KV / 32 q heads, n = 32768, C = 2048; 4 of 8 units checked
  batched128k  8 x 8 KV / 32 q heads, n = 131072, C = 4096; 8 of 64 units checked
  offload1m    1 x 8 KV / 32 q heads, n = 1048576, C = 8192, K/V in pinned
               host memory read through mapped device pointers; 4 of 8 units
  drift128k    n = 131072 prefill + 1024 decode steps appending one key per KV
               head with a drifting mean; 8 steps over the run checked on 2
               units, recall reported
  batched128k_pct  batched128k with the pages' percentile tiers and adaptive
               ratios (C = 13108)
  drift128k_layout the sink / local / update-buffer layout over the drift stream
"""
import numpy as np
import pytest

from oracle import pariskv_oracle as O
from workloads import synthetic as S
from tests.parity_util import HipRun, check_encode_unit, check_retrieve_unit, oracle_encode, say, tables, to_torch

pytestmark = pytest.mark.gpu


def _run_full(name, units, kv_host=False):
    w = S.WORKLOADS[name]
    say(f"case {name}: generating")
    K = S.all_keys(w)
    V = S.all_values(w)
    Q = S.all_queries(w, K)
    say(f"case {name}: GPU run")
    run = HipRun(w, K, V, Q, kv_host=kv_host).retrieve_attend()
    stats = {}
    for u in units:
        b, h = divmod(u, w.n_kv_heads)
        say(f"case {name}: oracle unit {u}")
        kf = S.as_f32(K[b, h])
        vf = S.as_f32(V[b, h])
        enc = check_encode_unit(run, u, kf)
        check_retrieve_unit(run, b, h, kf, vf, enc, stats=stats)
    # every head of every unit: Top-k indices valid, sorted, in range
    ti = run.topk_idx.cpu().numpy()
    te = run.topk_est.cpu().numpy()
    assert (ti >= 0).all() and (ti < w.n).all()
    assert (np.diff(te, axis=-1) <= 0).all()
    for row in ti.reshape(-1, w.top_k):
        assert len(np.unique(row)) == w.top_k
    run.close()
    say(f"case {name}: recall@{w.top_k} of sampled heads {np.mean(stats['recall']):.3f}")
    return stats


def test_full_llama32k():
    _run_full("llama32k", units=[0, 3, 5, 7])


def test_full_batched128k():
    """One unit in every eighth: 0, 9, ..., 63 (units 8 apart run on one XCD)."""
    _run_full("batched128k", units=[0, 9, 18, 27, 36, 45, 54, 63])


def test_full_batched128k_percentile_adaptive():
    """The pages' Stage I at full size: percentile tiers, C = ceil(0.1 n) = 13108."""
    _run_full("batched128k_pct", units=[0, 63])


def test_full_offload1m_mapped_host_kv():
    _run_full("offload1m", units=[0, 2, 5, 7], kv_host=True)


def test_full_drift_stream():
    """1024 decode steps, each one pk_append_retrieve_attend call (the call the
    benchmark times): append one drifting key per KV head, retrieve, attend.
    At the checked steps the same retrieval also runs with debug copies, its
    intermediates are compared with the oracle, and the decode-step call's
    Top-k, estimates and output must equal it bit for bit."""
    import torch
    from kv_cache_top_amd import pariskv as P
    w = S.WORKLOADS["drift128k"]
    T = w.append_steps
    say("case drift128k: generating")
    K0 = S.all_keys(w)
    V0 = S.all_values(w)
    ak = np.stack([np.stack([np.stack([S.appended_key(w, b, h, t) for t in range(T)])
                             for h in range(w.n_kv_heads)]) for b in range(w.batch)])
    av = np.stack([np.stack([np.stack([S.appended_value(w, b, h, t) for t in range(T)])
                             for h in range(w.n_kv_heads)]) for b in range(w.batch)])
    Kall = np.concatenate([K0, ak], axis=2)
    Vall = np.concatenate([V0, av], axis=2)
    Q0 = S.all_queries(w, K0)
    run = HipRun(w, Kall, Vall, Q0, n=w.n, capacity=w.n + T)
    check_steps = {0, 1, 127, 255, 511, 767, 895, T - 1}
    units = (3, 6)
    ref = {}
    for unit in units:
        b, h = divmod(unit, w.n_kv_heads)
        kf_all = S.as_f32(Kall[b, h])
        ref[unit] = (kf_all, S.as_f32(Vall[b, h]), oracle_encode(kf_all))
    recalls = []
    idx = torch.empty((w.batch, w.n_q_heads, w.top_k), dtype=torch.int32, device="cuda")
    est = torch.empty((w.batch, w.n_q_heads, w.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    for t in range(T):
        n_t = w.n + t + 1
        Qt = S.all_queries(w, lambda bb, hh, J: Kall[bb, hh, J], step=t, n_t=n_t)
        run.Q = Qt
        run.Qt = to_torch(Qt)
        P.pk_append_retrieve_attend(run.ctx.h, run.Kt[:, :, n_t - 1:n_t], run.Qt, run.sums.s, run.Kt, run.Vt, idx,
                                    out, est)
        if t in check_steps:
            run.debug = True
            run.retrieve_attend()
            for a, r in zip((idx, est, out), (run.topk_idx, run.topk_est, run.out)):
                assert torch.equal(a, r), f"decode-step call differs from the retrieval at step {t}"
            for unit in units:
                say(f"case drift128k: step {t}, oracle unit {unit}")
                b, h = divmod(unit, w.n_kv_heads)
                kf_all, vf_all, enc_all = ref[unit]
                enc = {k: v[:n_t] for k, v in enc_all.items()}
                check_encode_unit(run, unit, kf_all[:n_t], enc=enc, rows=slice(w.n - 8, n_t))
                st = {}
                check_retrieve_unit(run, b, h, kf_all[:n_t], vf_all[:n_t], enc, stats=st)
                recalls += st["recall"]
    assert run.n == w.n + T
    run.close()
    say(f"case drift128k: recall@100 at checked steps {np.round(recalls, 3).tolist()}")


def test_full_layout_stream():
    """drift128k_layout as the benchmark runs it: 64 sink tokens and a window of
    512 + up to 256 new tokens attended densely, the rest of the 128K prefill as
    the retrieval zone; 300 steps with one update-buffer flush; the last step is
    checked against the oracle on one unit."""
    import torch
    from kv_cache_top_amd import pariskv as P
    w = S.WORKLOADS["drift128k_layout"]
    sink, local, upd, steps = w.sink_tokens, w.local_tokens, w.update_tokens, 300
    say("case drift128k_layout: generating")
    K = S.all_keys(w)
    V = S.all_values(w)
    T = local + steps
    ak = np.stack([np.stack([np.stack([S.appended_key(w, b, h, t) for t in range(T)])
                             for h in range(w.n_kv_heads)]) for b in range(w.batch)])
    av = np.stack([np.stack([np.stack([S.appended_value(w, b, h, t) for t in range(T)])
                             for h in range(w.n_kv_heads)]) for b in range(w.batch)])
    zone0 = w.n - sink
    Kz = np.concatenate([K[:, :, sink:], ak], axis=2)
    Vz = np.concatenate([V[:, :, sink:], av], axis=2)
    Q = S.all_queries(w, K)
    run = HipRun(w, Kz, Vz, Q, n=zone0, capacity=Kz.shape[2])
    window = local                                     # stream tokens 0..local-1 are in the window
    for t in range(steps):
        window += 1                                   # token local + t joins the window
        if window == local + upd:
            P.pk_append_keys(run.ctx.h, run.Kt[:, :, run.n:run.n + upd], run.sums.s)
            window = local
    torch.cuda.synchronize()
    n_zone = run.n
    assert n_zone == zone0 + upd
    run.retrieve()
    lo = n_zone                                        # first window row in the zone tensor
    Kd = np.concatenate([K[:, :, :sink], Kz[:, :, lo:lo + window]], axis=2)
    Vd = np.concatenate([V[:, :, :sink], Vz[:, :, lo:lo + window]], axis=2)
    out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    P.pk_sparse_dense_attend(run.ctx.h, run.Qt, run.Kt, run.Vt, run.topk_idx, to_torch(Kd), to_torch(Vd), out)
    torch.cuda.synchronize()
    u = 3
    b, h = divmod(u, w.n_kv_heads)
    kf = S.as_f32(Kz[b, h, :n_zone])
    vf = S.as_f32(Vz[b, h, :n_zone])
    enc = oracle_encode(kf)
    check_encode_unit(run, u, kf, enc=enc, rows=slice(zone0 - 8, n_zone))
    check_retrieve_unit(run, b, h, kf, vf, enc, check_attention=False)
    ti = run.topk_idx.cpu().numpy()
    from tests.parity_util import attention_ok
    for g in range(w.group):
        qh = h * w.group + g
        ref = O.layout_attention(S.as_f32(Q[b, qh]), kf, vf, ti[b, qh], S.as_f32(Kd[b, h]), S.as_f32(Vd[b, h]),
                                 w.softmax_scale)
        o = out[b, qh].float().cpu().numpy()
        assert attention_ok(o, ref), f"layout attention g={g}: {np.abs(o - ref).max()}"
    run.close()
