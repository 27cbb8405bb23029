"""Recall studies on seeded synthetic keys, run through the library on the GPU.

Analogues, without a model, of the pages' retrieval-quality figures (Slides:
Fig. 1 and Fig. 10, recall over long decoding, coarse Stage I against the
final two-stage result; Fig. 9, recall against the candidate ratio):

* ``drift``: the drift stream (one key per KV head appended per step with a
  mean that drifts from +0.5 to -0.5); at every ``--every``-th step the
  queries are planted on the current keys and recall@k is measured for the k
  keys with the largest collision score (Stage I alone), for the candidate set
  (how many of the exact Top-k it holds) and for the final Top-k.
* ``ratio``: recall against the candidate ratio beta = C / n at several n.
* ``union``: how many distinct keys the G query heads of one KV head select
  together, i.e. the tighter Stage II byte count 128 B x |union of the G
  candidate sets| per unit, against the per-head sum 128 B x G x C.

The exact Top-k is the definition: <k_i, q> in fp64 over all current keys,
ties to the lower key index (torch, on the device that holds the keys).
Each result is printed as one JSON line, then a markdown table.

    python -m kv_cache_top_amd.studies drift [--every 64]
    python -m kv_cache_top_amd.studies ratio
    python -m kv_cache_top_amd.studies union
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _torch(a, dev):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _config(P, w, cap):
    return P.make_config(w.batch, w.n_kv_heads, w.n_q_heads, cap, w.n_candidates, w.top_k, w.softmax_scale,
                         w.srht_seed, w.tier_top, w.tier_weight,
                         P.PK_TIERS_PERCENTILE if w.tier_mode == "percentile" else P.PK_TIERS_RANK,
                         w.collision_permille, w.adaptive)


def exact_topk_fp64(K, Q, k: int) -> np.ndarray:
    """Exact Top-k of <k_i, q> for each row q of Q: fp64 inner products over
    the keys K [n, 128] (torch tensors, any dtype and device), ordered by
    (score desc, key index asc).  Returns numpy [G, min(k, n)]."""
    import torch
    sc = K.double() @ Q.double().T                                  # [n, G]
    order = torch.sort(-sc, dim=0, stable=True).indices             # equal scores keep ascending index
    return order[:min(k, K.shape[0])].T.cpu().numpy()


def stage1_topk(S: np.ndarray, k: int) -> np.ndarray:
    """The k keys with the largest collision score S, ties to the lower index."""
    return np.lexsort((np.arange(S.shape[0]), -S.astype(np.int64)))[:k]


def head_recalls(exact, S, cand, top):
    """Recall of one query head's exact Top-k by (Stage I alone: the k keys
    with the largest S; the candidate set; the final Top-k)."""
    ex = set(np.asarray(exact).tolist())
    k = len(ex)
    by_s = stage1_topk(np.asarray(S), k)
    c = np.asarray(cand)
    t = np.asarray(top)
    return (len(ex & set(by_s.tolist())) / k, len(ex & set(c[c >= 0].tolist())) / k,
            len(ex & set(t[t >= 0].tolist())) / k)


def _recalls(Kt, q, cand, top, scores, n, G, k):
    """Mean recall@k over the query heads of one retrieval, of: the k keys with
    the largest collision score S (Stage I alone, ties to the lower index), the
    candidate set (an upper bound for the final result) and the final Top-k."""
    s_top, coarse, final = [], [], []
    B, Hq, Hkv = q.shape[0], q.shape[1], Kt.shape[1]
    for b in range(B):
        for h in range(Hkv):
            ex = exact_topk_fp64(Kt[b, h, :n], q[b, h * G:(h + 1) * G], k)
            packed = scores[b * Hkv + h, :n]
            for g in range(G):
                hid = b * Hq + h * G + g
                S = (packed >> np.uint32(8 * g)) & np.uint32(0xFF)
                r = head_recalls(ex[g], S, cand[hid], top[b, h * G + g])
                s_top.append(r[0])
                coarse.append(r[1])
                final.append(r[2])
    return float(np.mean(s_top)), float(np.mean(coarse)), float(np.mean(final))


def _retrieve(P, ctx, sums, q, w, cfg_c, dev):
    import torch
    H = w.batch * w.n_q_heads
    idx = torch.empty((w.batch, w.n_q_heads, w.top_k), dtype=torch.int32, device=dev)
    cand = torch.full((H, cfg_c), -1, dtype=torch.int32, device=dev)
    scores = torch.zeros((w.units, sums.n), dtype=torch.int32, device=dev)
    dbg = P.pk_debug(0, 0, scores.data_ptr(), cand.data_ptr(), 0)
    P.pk_retrieve(ctx.h, q, sums.s, idx, None, dbg)
    torch.cuda.synchronize()
    return cand.cpu().numpy(), idx.cpu().numpy(), scores.cpu().numpy().view(np.uint32)


def drift_stream(w, every: int, T: int | None = None, dev=None):
    """Recall rows of one drift stream: encode the w.n prefill keys, then
    append T keys per KV head one step at a time; every `every`-th step (and
    the last) retrieve with queries planted on the current keys."""
    import torch

    from kv_cache_top_amd import pariskv as P
    from workloads import synthetic as S
    dev = dev or torch.device("cuda")
    T = w.append_steps if T is None else T
    K = S.all_keys(w)
    ak = np.stack([np.stack([np.stack([S.appended_key(w, b, h, t) for t in range(T)])
                             for h in range(w.n_kv_heads)]) for b in range(w.batch)])
    Kall = np.concatenate([K, ak], axis=2)
    Kt = _torch(Kall, dev)
    cfg = _config(P, w, w.n + T)
    ctx = P.Context(cfg)
    sums = P.Summaries(cfg)
    P.pk_encode_keys(ctx.h, Kt[:, :, :w.n], sums.s)
    rows = []
    for t in range(T + 1):
        if t % every == 0 or t == T:
            n_t = w.n + t
            Q = S.all_queries(w, lambda bb, hh, J: Kall[bb, hh, J], step=t, n_t=n_t)
            cand, top, scores = _retrieve(P, ctx, sums, _torch(Q, dev), w, cfg.n_candidates, dev)
            st, c, f = _recalls(Kt, _torch(Q, dev), cand, top, scores, n_t, w.group, w.top_k)
            rows.append({"study": "drift", "tiers": w.tier_mode, "step": t, "n": n_t,
                         "stage1_top_k_recall": round(st, 4), "candidate_recall": round(c, 4),
                         "final_recall": round(f, 4), "_Q": Q})
        if t < T:
            P.pk_append_keys(ctx.h, Kt[:, :, w.n + t:w.n + t + 1], sums.s)
    ctx.close()
    return rows, Kall


def drift(every: int, modes):
    from workloads import synthetic as S
    rows = []
    for mode in modes:
        base = S.WORKLOADS["drift128k"]
        # adaptive candidates: C = ceil(0.1 n) grows with the stream up to n + T keys
        w = base if mode == "rank" else S.custom("drift128k", tier_mode="percentile", adaptive=True,
                                                  n_candidates=(100 * (base.n + base.append_steps) + 999) // 1000)
        for row in drift_stream(w, every)[0]:
            row.pop("_Q")
            print(json.dumps(row), flush=True)
            rows.append(row)
    return rows


def ratio(n_list, permilles, modes):
    import torch

    from kv_cache_top_amd import pariskv as P
    from workloads import synthetic as S
    dev = torch.device("cuda")
    rows = []
    for n in n_list:
        for mode in modes:
            for pm in permilles:
                C = (pm * n + 999) // 1000
                if C > P.PK_MAX_CANDIDATES:
                    continue
                kw = dict(n=n, n_candidates=C, wid=900 + n % 1000)
                if mode == "percentile":
                    kw.update(tier_mode="percentile", collision_permille=max(200, pm))
                w = S.custom("llama32k", **kw)
                K = S.all_keys(w)
                Kt = _torch(K, dev)
                cfg = _config(P, w, n)
                ctx = P.Context(cfg)
                sums = P.Summaries(cfg)
                P.pk_encode_keys(ctx.h, Kt, sums.s)
                ss, cs, fs = [], [], []
                for step in range(4):
                    Q = S.all_queries(w, K, step=step)
                    cand, top, scores = _retrieve(P, ctx, sums, _torch(Q, dev), w, C, dev)
                    st, c, f = _recalls(Kt, _torch(Q, dev), cand, top, scores, n, w.group, w.top_k)
                    ss.append(st)
                    cs.append(c)
                    fs.append(f)
                row = {"study": "ratio", "tiers": mode, "n": n, "candidate_ratio": pm / 1000, "C": C,
                       "stage1_top_k_recall": round(float(np.mean(ss)), 4),
                       "candidate_recall": round(float(np.mean(cs)), 4), "final_recall": round(float(np.mean(fs)), 4)}
                print(json.dumps(row), flush=True)
                rows.append(row)
                ctx.close()
    return rows


def union(names):
    import torch

    from kv_cache_top_amd import pariskv as P
    from workloads import synthetic as S
    dev = torch.device("cuda")
    rows = []
    for name in names:
        w = S.WORKLOADS[name]
        K = S.all_keys(w)
        Kt = _torch(K, dev)
        cfg = _config(P, w, w.n)
        ctx = P.Context(cfg)
        sums = P.Summaries(cfg)
        P.pk_encode_keys(ctx.h, Kt, sums.s)
        del Kt
        sizes = []
        C = w.n_candidates
        for step in range(2):
            Q = S.all_queries(w, K, step=step)
            cand, _, _ = _retrieve(P, ctx, sums, _torch(Q, dev), w, C, dev)
            cand = cand.reshape(w.batch, w.n_q_heads, -1)
            for b in range(w.batch):
                for h in range(w.n_kv_heads):
                    ids = cand[b, h * w.group:(h + 1) * w.group].reshape(-1)
                    sizes.append(int(np.unique(ids[ids >= 0]).size))
        c_used = int((cand >= 0).sum(axis=-1).max())
        u = float(np.mean(sizes))
        row = {"study": "union", "workload": name, "G": w.group, "C": c_used, "mean_union": round(u, 1),
               "union_over_GC": round(u / (w.group * c_used), 4),
               "stage2_bytes_per_head_sum": 128 * w.group * c_used * w.units,
               "stage2_bytes_union": int(round(128 * u * w.units))}
        print(json.dumps(row), flush=True)
        rows.append(row)
        ctx.close()
    return rows


def table(rows):
    if not rows:
        return ""
    keys = [k for k in rows[0] if k != "study"]
    out = ["| " + " | ".join(keys) + " |", "|" + "---|" * len(keys)]
    out += ["| " + " | ".join(str(r[k]) for k in keys) + " |" for r in rows]
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("study", choices=["drift", "ratio", "union"])
    ap.add_argument("--every", type=int, default=128)
    ap.add_argument("--modes", default="rank,percentile")
    args = ap.parse_args()
    modes = args.modes.split(",")
    if args.study == "drift":
        rows = drift(args.every, modes)
    elif args.study == "union":
        rows = union(("llama32k", "batched128k", "batched128k_pct"))
    else:
        rows = ratio((32768, 131072), (10, 20, 50, 100, 200, 400), modes)
    print(table(rows), flush=True)


if __name__ == "__main__":
    main()
