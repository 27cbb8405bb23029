"""Thin ctypes binding of libpariskv.so (include/pariskv.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.  The
functions keep the C names; tensors are passed as torch tensors and converted
to raw pointers here.  Importing fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch first: its HIP runtime must be the one in the process before the
# library's own dependency on libamdhip64 is resolved, or torch later finds
# the device taken by a second runtime.
import torch  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
# PARISKV_LIB selects another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("PARISKV_LIB") or os.path.join(PKG, "libpariskv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_top_amd.build` "
                      "(there is no CPU fallback)")
_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------------------
# ABI types
# ---------------------------------------------------------------------------
PK_OK, PK_ERR_INVALID_ARG, PK_ERR_UNSUPPORTED, PK_ERR_CAPACITY, PK_ERR_OUT_OF_MEMORY, PK_ERR_HIP = \
    0, -1, -2, -3, -4, -5
PK_F32, PK_BF16 = 0, 1
PK_TIERS_RANK, PK_TIERS_PERCENTILE = 0, 1
PK_MAX_CANDIDATES, PK_MAX_TOPK, PK_MAX_DENSE = 16384, 256, 8192
PK_NOALLOC_SCRATCH_BYTES = 64 << 20
KERNELS = ["encode", "qprep", "collide", "threshold", "select", "rerank", "topk", "attend", "rerank_topk",
           "dense_attend"]
PK_DEVICE_ERR_SLOT = 1
PK_N_KERNELS = len(KERNELS)


class pk_config(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("n_sub", ctypes.c_int32), ("sub_dim", ctypes.c_int32),
        ("srht_seed", ctypes.c_uint64),
        ("n_tiers", ctypes.c_int32), ("tier_top", ctypes.c_int32 * 4), ("tier_weight", ctypes.c_int32 * 4),
        ("n_candidates", ctypes.c_int32), ("top_k", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_capacity", ctypes.c_int64),
        ("tier_mode", ctypes.c_int32), ("collision_permille", ctypes.c_int32), ("adaptive_ratios", ctypes.c_int32),
    ]


class pk_summaries(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("records", ctypes.c_void_p), ("norms", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("n", ctypes.c_int64), ("n_capacity", ctypes.c_int64)]


class pk_debug(ctypes.Structure):
    _fields_ = [("rot_q", ctypes.c_void_p), ("lut", ctypes.c_void_p), ("scores", ctypes.c_void_p),
                ("cand_idx", ctypes.c_void_p), ("cand_est", ctypes.c_void_p)]


class pk_kernel_timing(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I64x3 = ctypes.c_int64 * 3
_SIGS = {
    "pk_validate_config": ([ctypes.POINTER(pk_config)], ctypes.c_int),
    "pk_summary_bytes": ([ctypes.POINTER(pk_config), ctypes.POINTER(ctypes.c_size_t),
                          ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                          ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "pk_tables": ([ctypes.c_uint64, _P, _P, _P], ctypes.c_int),
    "pk_create": ([ctypes.POINTER(pk_config), ctypes.POINTER(_P)], ctypes.c_int),
    "pk_destroy": ([_P], None),
    "pk_encode_keys": ([_P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, ctypes.POINTER(pk_summaries), _P],
                       ctypes.c_int),
    "pk_append_keys": ([_P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, ctypes.POINTER(pk_summaries), _P],
                       ctypes.c_int),
    "pk_retrieve": ([_P, _P, ctypes.c_int, ctypes.POINTER(pk_summaries), _P, _P, ctypes.POINTER(pk_debug), _P],
                    ctypes.c_int),
    "pk_sparse_attend": ([_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, _P, _P,
                          ctypes.c_int, _P],
                         ctypes.c_int),
    "pk_retrieve_attend": ([_P, _P, ctypes.c_int, ctypes.POINTER(pk_summaries), _P, _P, ctypes.c_int, _I64x3,
                            ctypes.c_int64, _P, _P, _P, ctypes.c_int, ctypes.POINTER(pk_debug), _P], ctypes.c_int),
    "pk_append_retrieve_attend": ([_P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, ctypes.POINTER(pk_summaries), _P,
                                   ctypes.c_int, _P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, _P, _P, _P,
                                   ctypes.c_int, _P], ctypes.c_int),
    "pk_retrieve_attend_noalloc": ([ctypes.POINTER(pk_config), _P, ctypes.c_int, ctypes.POINTER(pk_summaries), _P,
                                    _P, ctypes.c_int, _I64x3, ctypes.c_int64, _P, _P, _P, ctypes.c_int, _P],
                                   ctypes.c_int),
    "pk_sparse_dense_attend": ([_P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _I64x3, ctypes.c_int64, _P, _P, _P,
                                _I64x3, ctypes.c_int64, _P, ctypes.c_int, _P], ctypes.c_int),
    "pk_host_alloc_mapped": ([ctypes.c_size_t, ctypes.POINTER(_P), ctypes.POINTER(_P)], ctypes.c_int),
    "pk_host_free": ([_P], ctypes.c_int),
    "pk_offload_rows": ([_P, _I64x3, _P, _I64x3, ctypes.c_int, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, _P],
                        ctypes.c_int),
    "pk_calibration_copy": ([_P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "pk_device_errors": ([_P, ctypes.POINTER(ctypes.c_uint32), _P], ctypes.c_int),
    "pk_timing_begin": ([_P, ctypes.c_int32], ctypes.c_int),
    "pk_timing_end": ([_P, ctypes.POINTER(pk_kernel_timing)], ctypes.c_int),
    "pk_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "pk_last_error": ([_P], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class PkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_lib.pk_status_str(status).decode()}: {msg}")
        self.status = status


def _check(status: int, ctx=None):
    if status != PK_OK:
        raise PkError(status, (_lib.pk_last_error(ctx) or b"").decode())


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PK_BF16
    if t.dtype == torch.float32:
        return PK_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _strides4(t):
    """[batch, heads, tokens, 128] tensor -> element strides (batch, head, token)."""
    if t.dim() != 4 or t.shape[-1] != 128 or t.stride(-1) != 1:
        raise ValueError("expected a [batch, heads, tokens, 128] tensor with a contiguous last dim")
    return _I64x3(t.stride(0), t.stride(1), t.stride(2))


# configuration of every live context, by handle value: the C ABI sees raw
# pointers only, so shapes, dtypes and devices are checked here before a call
_CONFIGS: dict = {}


def _handle_value(ctx) -> int:
    return ctx.value if isinstance(ctx, ctypes.c_void_p) else int(ctx)


def _cfg_of(ctx) -> "pk_config":
    cfg = _CONFIGS.get(_handle_value(ctx) if ctx else 0)
    if cfg is None:
        raise ValueError("unknown or destroyed context")
    return cfg


def _need(t, name: str, shape, dtypes, contiguous: bool = True):
    """Shape, dtype, layout and then device of one tensor argument."""
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    del torch


def _need_rows(t, name: str, cfg, dtypes):
    """[>= batch, >= n_kv_heads, rows, 128] K/V-like tensor on the GPU."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dim() != 4 or t.shape[0] < cfg.batch or t.shape[1] < cfg.n_kv_heads or t.shape[3] != 128:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected [>= {cfg.batch}, >= {cfg.n_kv_heads}, rows, 128]")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")


def _float_types():
    import torch
    return (torch.float32, torch.bfloat16)


def _check_q(cfg, q):
    _need(q, "q", (cfg.batch, cfg.n_q_heads, 128), _float_types())


def _check_topk(cfg, topk_idx, topk_est):
    import torch
    _need(topk_idx, "topk_idx", (cfg.batch, cfg.n_q_heads, cfg.top_k), (torch.int32,))
    if topk_est is not None:
        _need(topk_est, "topk_est", (cfg.batch, cfg.n_q_heads, cfg.top_k), (torch.float32,))


def _check_out(cfg, out):
    _need(out, "out", (cfg.batch, cfg.n_q_heads, 128), _float_types())


def _check_kv(cfg, k, v):
    _need_rows(k, "k", cfg, _float_types())
    _need_rows(v, "v", cfg, _float_types())
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("K and V must share shape, dtype and strides")


def make_config(batch, n_kv_heads, n_q_heads, n_capacity, n_candidates, top_k=100, softmax_scale=None,
                srht_seed=0, tier_top=(1, 4, 16), tier_weight=(4, 2, 1), tier_mode=PK_TIERS_RANK,
                collision_permille=0, adaptive_ratios=False) -> pk_config:
    c = pk_config()
    c.head_dim, c.n_sub, c.sub_dim = 128, 16, 8
    c.srht_seed = srht_seed
    c.n_tiers = len(tier_top)
    for i, (t, w) in enumerate(zip(tier_top, tier_weight)):
        c.tier_top[i], c.tier_weight[i] = t, w
    c.n_candidates, c.top_k = n_candidates, top_k
    c.softmax_scale = (1.0 / 128 ** 0.5) if softmax_scale is None else softmax_scale
    c.batch, c.n_kv_heads, c.n_q_heads, c.n_capacity = batch, n_kv_heads, n_q_heads, n_capacity
    c.tier_mode, c.collision_permille, c.adaptive_ratios = tier_mode, collision_permille, int(bool(adaptive_ratios))
    return c


# ---------------------------------------------------------------------------
# C-named entry points
# ---------------------------------------------------------------------------
def pk_validate_config(cfg: pk_config) -> int:
    return _lib.pk_validate_config(ctypes.byref(cfg))


def pk_summary_bytes(cfg: pk_config):
    a, b, c, d = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.pk_summary_bytes(ctypes.byref(cfg), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                 ctypes.byref(d)))
    return a.value, b.value, c.value, d.value


def pk_tables(seed: int):
    import numpy as np
    s = np.zeros(128, np.int8)
    L = np.zeros(8, np.float32)
    T = np.zeros(7, np.float32)
    _check(_lib.pk_tables(seed, s.ctypes.data, L.ctypes.data, T.ctypes.data))
    return s, L, T


def pk_create(cfg: pk_config):
    h = ctypes.c_void_p()
    _check(_lib.pk_create(ctypes.byref(cfg), ctypes.byref(h)))
    keep = pk_config()
    ctypes.pointer(keep)[0] = cfg
    _CONFIGS[h.value] = keep
    return h


def pk_destroy(ctx) -> None:
    _CONFIGS.pop(_handle_value(ctx) if ctx else 0, None)
    _lib.pk_destroy(ctx)


def pk_encode_keys(ctx, keys, sums: pk_summaries, stream=None):
    cfg = _cfg_of(ctx)
    _need_rows(keys, "keys", cfg, _float_types())
    _check(_lib.pk_encode_keys(ctx, _ptr(keys), _dtype(keys), _strides4(keys), keys.shape[2],
                               ctypes.byref(sums), _stream(stream)), ctx)


def pk_append_keys(ctx, new_keys, sums: pk_summaries, stream=None):
    cfg = _cfg_of(ctx)
    _need_rows(new_keys, "new_keys", cfg, _float_types())
    _check(_lib.pk_append_keys(ctx, _ptr(new_keys), _dtype(new_keys), _strides4(new_keys), new_keys.shape[2],
                               ctypes.byref(sums), _stream(stream)), ctx)


def pk_retrieve(ctx, q, sums: pk_summaries, topk_idx, topk_est=None, debug: pk_debug | None = None,
                stream=None):
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_topk(cfg, topk_idx, topk_est)
    _check(_lib.pk_retrieve(ctx, _ptr(q), _dtype(q), ctypes.byref(sums), _ptr(topk_idx), _ptr(topk_est),
                            ctypes.byref(debug) if debug is not None else None, _stream(stream)), ctx)


def pk_sparse_attend(ctx, q, k, v, topk_idx, out, stream=None):
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_kv(cfg, k, v)
    _check_topk(cfg, topk_idx, None)
    _check_out(cfg, out)
    _check(_lib.pk_sparse_attend(ctx, _ptr(q), _dtype(q), _ptr(k), _ptr(v), _dtype(k), _strides4(k),
                                 k.shape[2], _ptr(topk_idx), _ptr(out), _dtype(out), _stream(stream)), ctx)


def pk_sparse_attend_raw(ctx, q, k_ptr: int, v_ptr: int, kv_dtype: int, kv_strides, n_rows: int, topk_idx, out,
                         stream=None):
    """Variant for K/V that are not torch tensors (e.g. mapped host memory)."""
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_topk(cfg, topk_idx, None)
    _check_out(cfg, out)
    _check(_lib.pk_sparse_attend(ctx, _ptr(q), _dtype(q), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
                                 kv_dtype, _I64x3(*kv_strides), n_rows, _ptr(topk_idx), _ptr(out), _dtype(out),
                                 _stream(stream)), ctx)


def pk_retrieve_attend(ctx, q, sums: pk_summaries, k, v, topk_idx, out, topk_est=None,
                       debug: pk_debug | None = None, stream=None):
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_kv(cfg, k, v)
    _check_topk(cfg, topk_idx, topk_est)
    _check_out(cfg, out)
    _check(_lib.pk_retrieve_attend(ctx, _ptr(q), _dtype(q), ctypes.byref(sums), _ptr(k), _ptr(v), _dtype(k),
                                   _strides4(k), k.shape[2], _ptr(topk_idx), _ptr(topk_est), _ptr(out), _dtype(out),
                                   ctypes.byref(debug) if debug is not None else None, _stream(stream)), ctx)


def pk_append_retrieve_attend(ctx, new_keys, q, sums: pk_summaries, k, v, topk_idx, out, topk_est=None,
                              stream=None):
    """One decode step: new_keys [batch][n_kv_heads][t][128] join the summaries,
    then retrieval + attention over all keys (k, v hold every row)."""
    cfg = _cfg_of(ctx)
    _need_rows(new_keys, "new_keys", cfg, _float_types())
    _check_q(cfg, q)
    _check_kv(cfg, k, v)
    _check_topk(cfg, topk_idx, topk_est)
    _check_out(cfg, out)
    _check(_lib.pk_append_retrieve_attend(ctx, _ptr(new_keys), _dtype(new_keys), _strides4(new_keys),
                                          new_keys.shape[2], ctypes.byref(sums), _ptr(q), _dtype(q), _ptr(k),
                                          _ptr(v), _dtype(k), _strides4(k), k.shape[2], _ptr(topk_idx),
                                          _ptr(topk_est), _ptr(out), _dtype(out), _stream(stream)), ctx)


def pk_retrieve_attend_raw(ctx, q, sums: pk_summaries, k_ptr: int, v_ptr: int, kv_dtype: int, kv_strides,
                           n_rows: int, topk_idx, out, topk_est=None, debug: pk_debug | None = None, stream=None):
    """Variant for K/V that are not torch tensors (e.g. mapped host memory)."""
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_topk(cfg, topk_idx, topk_est)
    _check_out(cfg, out)
    _check(_lib.pk_retrieve_attend(ctx, _ptr(q), _dtype(q), ctypes.byref(sums), ctypes.c_void_p(k_ptr),
                                   ctypes.c_void_p(v_ptr), kv_dtype, _I64x3(*kv_strides), n_rows, _ptr(topk_idx),
                                   _ptr(topk_est), _ptr(out), _dtype(out),
                                   ctypes.byref(debug) if debug is not None else None, _stream(stream)), ctx)


def pk_retrieve_attend_noalloc(cfg: pk_config, q, sums: pk_summaries, k, v, topk_idx, out, topk_est=None,
                               stream=None):
    """pk_retrieve_attend with no context: the scratch is the library's static device array."""
    _check_q(cfg, q)
    _check_kv(cfg, k, v)
    _check_topk(cfg, topk_idx, topk_est)
    _check_out(cfg, out)
    _check(_lib.pk_retrieve_attend_noalloc(ctypes.byref(cfg), _ptr(q), _dtype(q), ctypes.byref(sums), _ptr(k),
                                           _ptr(v), _dtype(k), _strides4(k), k.shape[2], _ptr(topk_idx),
                                           _ptr(topk_est), _ptr(out), _dtype(out), _stream(stream)))


def pk_sparse_dense_attend(ctx, q, k, v, topk_idx, dense_k, dense_v, out, stream=None):
    """Attention over the retrieved rows of k / v and every row of dense_k / dense_v."""
    cfg = _cfg_of(ctx)
    _check_q(cfg, q)
    _check_kv(cfg, k, v)
    _check_kv(cfg, dense_k, dense_v)
    if dense_k.dtype != k.dtype:
        raise ValueError("dense rows must have the dtype of K / V")
    _check_topk(cfg, topk_idx, None)
    _check_out(cfg, out)
    _check(_lib.pk_sparse_dense_attend(ctx, _ptr(q), _dtype(q), _ptr(k), _ptr(v), _dtype(k), _strides4(k),
                                       k.shape[2], _ptr(topk_idx), _ptr(dense_k), _ptr(dense_v),
                                       _strides4(dense_k), dense_k.shape[2], _ptr(out), _dtype(out),
                                       _stream(stream)), ctx)


def pk_host_alloc_mapped(nbytes: int):
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    _check(_lib.pk_host_alloc_mapped(nbytes, ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def pk_host_free(host_ptr: int) -> None:
    _check(_lib.pk_host_free(ctypes.c_void_p(host_ptr)))


def pk_offload_rows(src, dst_ptr: int, dst_strides, stream=None) -> None:
    """Copy every row of src [batch, heads, rows, 128] (a GPU tensor) to the
    device pointer dst_ptr (e.g. the device view of mapped host memory, at the
    first destination row) with element strides dst_strides."""
    if src.device.type != "cuda":
        raise ValueError("src must be a GPU tensor")
    _check(_lib.pk_offload_rows(_ptr(src), _strides4(src), ctypes.c_void_p(dst_ptr), _I64x3(*dst_strides),
                                _dtype(src), src.shape[0], src.shape[1], src.shape[2], _stream(stream)))


def pk_calibration_copy(dst, src, stream=None) -> None:
    """Copy the bytes of device tensor `src` into `dst` (same size) with 16-byte lane accesses."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("dst and src differ in size")
    _check(_lib.pk_calibration_copy(_ptr(dst), _ptr(src), n, _stream(stream)))


def pk_device_errors(ctx, stream=None) -> int:
    """Device-side consistency flags since the last call (waits for the stream, then clears them)."""
    v = ctypes.c_uint32()
    _check(_lib.pk_device_errors(ctx, ctypes.byref(v), _stream(stream)), ctx)
    return v.value


def pk_timing_begin(ctx, max_launches: int) -> None:
    _check(_lib.pk_timing_begin(ctx, max_launches), ctx)


def pk_timing_end(ctx) -> dict:
    arr = (pk_kernel_timing * PK_N_KERNELS)()
    _check(_lib.pk_timing_end(ctx, arr), ctx)
    return {name: (arr[i].launches, arr[i].total_ms) for i, name in enumerate(KERNELS)}


def pk_status_str(status: int) -> str:
    return _lib.pk_status_str(status).decode()


def pk_last_error(ctx=None) -> str:
    return (_lib.pk_last_error(ctx) or b"").decode()


# ---------------------------------------------------------------------------
# convenience wrappers used by tests and the benchmark
# ---------------------------------------------------------------------------
class Summaries:
    """Device arrays of the key summaries (torch-owned) plus the ABI struct."""

    def __init__(self, cfg: pk_config, device="cuda"):
        import torch
        cb, rb, nb, kb = pk_summary_bytes(cfg)
        units = cfg.batch * cfg.n_kv_heads
        self.codes = torch.empty(cb, dtype=torch.uint8, device=device)
        self.records = torch.empty(rb, dtype=torch.uint8, device=device)
        self.norms = torch.empty(nb // 4, dtype=torch.float32, device=device)
        self.counts = torch.zeros(kb // 4, dtype=torch.int32, device=device)
        self.units, self.n_capacity = units, cfg.n_capacity
        self.s = pk_summaries(self.codes.data_ptr(), self.records.data_ptr(), self.norms.data_ptr(),
                              self.counts.data_ptr(), 0, cfg.n_capacity)

    @property
    def n(self) -> int:
        return self.s.n

    def codes_view(self):
        return self.codes.view(self.units, self.n_capacity, 16)

    def records_view(self):
        return self.records.view(self.units, self.n_capacity, 128)

    def norms_view(self):
        return self.norms.view(self.units, self.n_capacity)

    def counts_view(self):
        return self.counts.view(self.units, 16, 256)

    def clone(self, cfg: pk_config) -> "Summaries":
        other = Summaries.__new__(Summaries)
        other.codes, other.records, other.norms = self.codes.clone(), self.records.clone(), self.norms.clone()
        other.counts = self.counts.clone()
        other.units, other.n_capacity = self.units, self.n_capacity
        other.s = pk_summaries(other.codes.data_ptr(), other.records.data_ptr(), other.norms.data_ptr(),
                               other.counts.data_ptr(), self.s.n, self.s.n_capacity)
        return other


class Context:
    """Owns a pk_context (destroyed on close / garbage collection)."""

    def __init__(self, cfg: pk_config):
        self.cfg = cfg
        self.h = pk_create(cfg)

    def close(self):
        if self.h:
            pk_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
