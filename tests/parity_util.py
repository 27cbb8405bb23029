"""Shared machinery of the GPU parity tests: run the HIP path through the C ABI
on seeded synthetic inputs, run the oracle on the same inputs, compare."""
from __future__ import annotations

import ctypes
import sys

import numpy as np

from oracle import pariskv_oracle as O
from workloads import synthetic as S

SIGNS = None
L32 = TAU32 = None


def tables():
    global SIGNS, L32, TAU32
    if SIGNS is None:
        SIGNS = O.srht_signs(0)
        L32, TAU32 = O.magnitude_tables_f32()
    return SIGNS, L32, TAU32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_torch(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def oracle_encode(keys_f32: np.ndarray, chunk: int = 65536):
    """oracle.encode_f32 in chunks (bounded memory at 1M keys)."""
    signs, L32_, TAU32_ = tables()
    parts = [O.encode_f32(keys_f32[i:i + chunk], signs, L32_, TAU32_) for i in range(0, keys_f32.shape[0], chunk)]
    if not parts:
        return dict(codes=np.zeros((0, 16), np.uint8), nibbles=np.zeros((0, 64), np.uint8),
                    weights=np.zeros((0, 16), np.float32), norms=np.zeros(0, np.float32))
    return {k: np.concatenate([p[k] for p in parts]) for k in ("codes", "nibbles", "weights", "norms")}


class HipRun:
    """One workload run through the library: encode, retrieve (with debug copies), attend."""

    def __init__(self, w: S.Workload, K: np.ndarray, V: np.ndarray, Q: np.ndarray, n: int | None = None,
                 kv_host: bool = False, debug: bool = True, append: np.ndarray | None = None,
                 capacity: int | None = None):
        import torch
        from kv_cache_top_amd import pariskv as P
        self.P = P
        self.w = w
        n = K.shape[2] if n is None else n
        cap = n + (append.shape[2] if append is not None else 0) if capacity is None else capacity
        self.cfg = P.make_config(w.batch, w.n_kv_heads, w.n_q_heads, max(cap, 1), w.n_candidates, w.top_k,
                                 w.softmax_scale, w.srht_seed, w.tier_top, w.tier_weight,
                                 P.PK_TIERS_PERCENTILE if w.tier_mode == "percentile" else P.PK_TIERS_RANK,
                                 w.collision_permille, w.adaptive)
        self.ctx = P.Context(self.cfg)
        self.sums = P.Summaries(self.cfg)
        self.host_bufs = []
        if kv_host:
            self.Kd, self.kv_strides, kptr = self._mapped(K)
            self.Vd, _, vptr = self._mapped(V)
            self.kptr, self.vptr = kptr, vptr
        else:
            self.Kt = to_torch(K)
            self.Vt = to_torch(V)
        self.kv_host = kv_host
        dt = P.PK_BF16 if K.dtype == np.uint16 else P.PK_F32
        self.kv_dtype = dt
        # encode rows [0, n)
        if kv_host:
            st = (ctypes.c_int64 * 3)(*self.kv_strides)
            P._check(P._lib.pk_encode_keys(self.ctx.h, ctypes.c_void_p(self.kptr), dt, st, n,
                                           ctypes.byref(self.sums.s), P._stream(None)), self.ctx.h)
        else:
            P.pk_encode_keys(self.ctx.h, self.Kt[:, :, :n], self.sums.s)
        if append is not None:
            At = to_torch(append)
            P.pk_append_keys(self.ctx.h, At, self.sums.s)
        torch.cuda.synchronize()
        self.Q = Q
        self.Qt = to_torch(Q)
        self.debug = debug

    @property
    def n(self) -> int:
        return self.sums.n

    def _mapped(self, A: np.ndarray):
        P = self.P
        h, d = P.pk_host_alloc_mapped(A.nbytes)
        self.host_bufs.append(h)
        view = np.ctypeslib.as_array((ctypes.c_uint8 * A.nbytes).from_address(h)).view(A.dtype).reshape(A.shape)
        view[...] = A
        strides = (A.shape[1] * A.shape[2] * A.shape[3], A.shape[2] * A.shape[3], A.shape[3])
        return view, strides, d

    def _outputs(self, Q):
        import torch
        P = self.P
        w, cfg = self.w, self.cfg
        H = w.batch * w.n_q_heads
        self.topk_idx = torch.full((w.batch, w.n_q_heads, w.top_k), -7, dtype=torch.int32, device="cuda")
        self.topk_est = torch.zeros((w.batch, w.n_q_heads, w.top_k), dtype=torch.float32, device="cuda")
        dbg = None
        if self.debug:
            self.rot_q = torch.zeros((H, 128), dtype=torch.float32, device="cuda")
            self.lut = torch.zeros((w.units, 16, 256), dtype=torch.int32, device="cuda")
            self.scores = torch.zeros((w.units, max(self.n, 1)), dtype=torch.int32, device="cuda")
            self.cand_idx = torch.zeros((H, cfg.n_candidates), dtype=torch.int32, device="cuda")
            self.cand_est = torch.zeros((H, cfg.n_candidates), dtype=torch.float32, device="cuda")
            dbg = P.pk_debug(self.rot_q.data_ptr(), self.lut.data_ptr(), self.scores.data_ptr(),
                             self.cand_idx.data_ptr(), self.cand_est.data_ptr())
        return (self.Qt if Q is None else to_torch(Q)), dbg

    def retrieve(self, Q: np.ndarray | None = None):
        import torch
        Qt, dbg = self._outputs(Q)
        self.P.pk_retrieve(self.ctx.h, Qt, self.sums.s, self.topk_idx, self.topk_est, dbg)
        torch.cuda.synchronize()
        return self

    def retrieve_attend(self, out_dtype="match"):
        """Retrieval and attention through the single fused call."""
        import torch
        P = self.P
        w = self.w
        Qt, dbg = self._outputs(None)
        odt = torch.float32 if (self.kv_dtype == P.PK_F32 or out_dtype == "f32") else torch.bfloat16
        self.out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=odt, device="cuda")
        if self.kv_host:
            P.pk_retrieve_attend_raw(self.ctx.h, Qt, self.sums.s, self.kptr, self.vptr, self.kv_dtype,
                                     self.kv_strides, self.Kd.shape[2], self.topk_idx, self.out, self.topk_est, dbg)
        else:
            P.pk_retrieve_attend(self.ctx.h, Qt, self.sums.s, self.Kt, self.Vt, self.topk_idx, self.out,
                                 self.topk_est, dbg)
        torch.cuda.synchronize()
        return self

    def attend(self, out_dtype="match"):
        import torch
        P = self.P
        w = self.w
        odt = torch.float32 if (self.kv_dtype == P.PK_F32 or out_dtype == "f32") else torch.bfloat16
        self.out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=odt, device="cuda")
        if self.kv_host:
            P.pk_sparse_attend_raw(self.ctx.h, self.Qt, self.kptr, self.vptr, self.kv_dtype, self.kv_strides,
                                   self.Kd.shape[2], self.topk_idx, self.out)
        else:
            P.pk_sparse_attend(self.ctx.h, self.Qt, self.Kt, self.Vt, self.topk_idx, self.out)
        torch.cuda.synchronize()
        return self

    def device_errors(self) -> int:
        return self.P.pk_device_errors(self.ctx.h)

    def close(self):
        self.ctx.close()
        for h in self.host_bufs:
            self.P.pk_host_free(h)
        self.host_bufs = []


# ---------------------------------------------------------------------------
# comparisons
# ---------------------------------------------------------------------------
def check_encode_unit(run: HipRun, u: int, keys_f32: np.ndarray, enc=None, rows=None):
    """Codes, nibbles and weights bit-exact, norms to 1e-6 relative, for unit u."""
    enc = oracle_encode(keys_f32) if enc is None else enc
    n = keys_f32.shape[0]
    sl = slice(0, n) if rows is None else rows
    codes = run.sums.codes_view()[u, :n].cpu().numpy()
    rec = run.sums.records_view()[u, :n].cpu().numpy()
    norms = run.sums.norms_view()[u, :n].cpu().numpy()
    np.testing.assert_array_equal(codes[sl], enc["codes"][sl], err_msg=f"codes unit {u}")
    np.testing.assert_array_equal(rec[sl, :64], enc["nibbles"][sl], err_msg=f"nibbles unit {u}")
    wg = np.ascontiguousarray(rec[sl, 64:]).view(np.float32)
    np.testing.assert_array_equal(wg, enc["weights"][sl], err_msg=f"weights unit {u}")
    np.testing.assert_allclose(norms[sl], enc["norms"][sl], rtol=1e-6, err_msg=f"norms unit {u}")
    counts = run.sums.counts_view()[u].cpu().numpy()
    np.testing.assert_array_equal(counts, O.centroid_occupancy(enc["codes"][:n]), err_msg=f"centroid counts unit {u}")
    return enc


def call_sizes(w: S.Workload, n: int):
    """(C, M) of a retrieval over n keys: candidates, and kept positions per block
    with percentile tiers (None with rank tiers)."""
    if w.adaptive:
        beta, rho = O.adaptive_ratios_permille(n)
        C = O.ratio_count(beta, n)
    else:
        C, rho = w.n_candidates, w.collision_permille
    M = O.ratio_count(rho, n) if w.tier_mode == "percentile" else None
    return C, M


def attention_ok(o_gpu: np.ndarray, o_ref: np.ndarray, rel: float = 2e-2) -> bool:
    o_ref = np.asarray(o_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(o_ref ** 2))
    return bool(np.all(np.abs(o_gpu.astype(np.float64) - o_ref) <= rel * (np.abs(o_ref) + rms)))


def check_retrieve_unit(run: HipRun, b: int, h: int, keys_f32, values_f32, enc, heads=None,
                        check_attention=True, stats=None):
    """Every intermediate of the unit's query heads against the oracle."""
    signs, L32_, _ = tables()
    w = run.w
    G = w.group
    u = b * w.n_kv_heads + h
    n = run.n
    qs = S.as_f32(run.Q[b, h * G:(h + 1) * G])
    C, M = call_sizes(w, n)
    res = O.decode_unit(qs, keys_f32, values_f32, enc, signs, L32_, w.tier_top, w.tier_weight,
                        C, w.top_k, w.softmax_scale, n=n, percentile_M=M)
    lut = run.lut[u].cpu().numpy().view(np.uint32) if run.debug else None
    sc = run.scores[u, :n].cpu().numpy().view(np.uint32) if run.debug else None
    n_sel = min(n, C)
    for g in (range(G) if heads is None else heads):
        qh = h * G + g
        hid = b * w.n_q_heads + qh
        r = res[g]
        tag = f"(b={b}, kv={h}, g={g})"
        if run.debug:
            np.testing.assert_array_equal(run.rot_q[hid].cpu().numpy(), r["Rq"], err_msg=f"rot_q {tag}")
            np.testing.assert_array_equal((lut >> (8 * g)) & 0xFF, r["weights"], err_msg=f"lut {tag}")
            np.testing.assert_array_equal((sc >> (8 * g)) & 0xFF, r["S"], err_msg=f"S {tag}")
            ci = run.cand_idx[hid].cpu().numpy()
            ce = run.cand_est[hid].cpu().numpy()
            np.testing.assert_array_equal(ci[:n_sel], r["cand"], err_msg=f"candidates {tag}")
            assert (ci[n_sel:] == -1).all()
            np.testing.assert_array_equal(ce[:n_sel], r["est32"], err_msg=f"fp32 estimates {tag}")
            assert np.all(np.abs(ce[:n_sel].astype(np.float64) - r["est64"]) <= 1e-5 * r["abs_scale"]), \
                f"estimates vs fp64 {tag}"
        ti = run.topk_idx[b, qh].cpu().numpy()
        te = run.topk_est[b, qh].cpu().numpy()
        keff = min(w.top_k, n_sel)
        np.testing.assert_array_equal(ti[:keff], r["top_idx"], err_msg=f"top-k {tag}")
        np.testing.assert_array_equal(te[:keff], r["top_est"], err_msg=f"top-k est {tag}")
        assert (ti[keff:] == -1).all()
        if check_attention and hasattr(run, "out"):
            o = run.out[b, qh].float().cpu().numpy()
            assert attention_ok(o, r["out"]), f"attention {tag}: max err {np.abs(o - r['out']).max()}"
        if stats is not None:
            exact = O.exact_topk(keys_f32[:n], qs[g], w.top_k)
            stats.setdefault("recall", []).append(len(set(ti[:keff]) & set(exact)) / max(1, len(exact)))
    return res
