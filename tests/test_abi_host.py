"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/pariskv.h declares, rejects bad configurations and
arguments with the documented status codes before touching a device, and its
host-computed tables equal the oracle's bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import pariskv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pariskv.h")

P = pytest.importorskip("kv_cache_top_amd.pariskv", reason="libpariskv.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(pk_\w+)\s*\(", text, flags=re.M)))


def test_header_parses():
    fns = header_functions()
    assert "pk_retrieve" in fns and "pk_sparse_attend" in fns and len(fns) >= 15


def test_every_declared_function_is_exported():
    lib = ctypes.CDLL(P.LIB_PATH)
    missing = [f for f in header_functions() if not hasattr(lib, f)]
    assert not missing, missing
    # the binding wraps exactly the declared functions
    assert sorted(P.EXPORTED) == header_functions()


def test_exported_symbols_are_unmangled_c():
    out = os.popen(f"nm -D --defined-only {P.LIB_PATH}").read()
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for f in header_functions():
        assert f in syms


def test_status_strings():
    names = {s: P._lib.pk_status_str(s).decode() for s in (0, -1, -2, -3, -4, -5)}
    assert names[0] == "PK_OK" and len(set(names.values())) == 6
    assert P._lib.pk_status_str(-99).decode() == "PK_ERR_UNKNOWN"


def good_config(**kw):
    base = dict(batch=2, n_kv_heads=8, n_q_heads=32, n_capacity=4096, n_candidates=512, top_k=100)
    base.update(kw)
    return P.make_config(**base)


def status(cfg):
    return P._lib.pk_validate_config(ctypes.byref(cfg))


def test_validate_accepts_workload_configs():
    from workloads import synthetic as S
    for w in S.WORKLOADS.values():
        cfg = P.make_config(w.batch, w.n_kv_heads, w.n_q_heads, w.n + w.append_steps, w.n_candidates, w.top_k)
        assert status(cfg) == P.PK_OK, (w.name, P._lib.pk_last_error(None))


@pytest.mark.parametrize("field,value,expect", [
    ("head_dim", 64, P.PK_ERR_UNSUPPORTED),
    ("n_sub", 8, P.PK_ERR_UNSUPPORTED),
    ("sub_dim", 16, P.PK_ERR_UNSUPPORTED),
    ("n_tiers", 0, P.PK_ERR_INVALID_ARG),
    ("n_tiers", 5, P.PK_ERR_INVALID_ARG),
    ("n_candidates", 0, P.PK_ERR_INVALID_ARG),
    ("n_candidates", 16385, P.PK_ERR_INVALID_ARG),
    ("top_k", 0, P.PK_ERR_INVALID_ARG),
    ("top_k", 257, P.PK_ERR_INVALID_ARG),
    ("top_k", 513, P.PK_ERR_INVALID_ARG),          # > n_candidates
    ("softmax_scale", float("inf"), P.PK_ERR_INVALID_ARG),
    ("softmax_scale", float("nan"), P.PK_ERR_INVALID_ARG),
    ("batch", 0, P.PK_ERR_INVALID_ARG),
    ("n_kv_heads", 0, P.PK_ERR_INVALID_ARG),
    ("n_q_heads", 30, P.PK_ERR_INVALID_ARG),       # not a multiple of 8
    ("n_q_heads", 40, P.PK_ERR_UNSUPPORTED),       # group of 5
    ("n_capacity", 0, P.PK_ERR_INVALID_ARG),
    ("n_capacity", 1 << 31, P.PK_ERR_INVALID_ARG),
])
def test_validate_rejects(field, value, expect):
    cfg = good_config()
    setattr(cfg, field, value)
    assert status(cfg) == expect
    assert P._lib.pk_last_error(None)             # a message is left behind


def test_validate_tiers():
    cfg = good_config()
    cfg.tier_top[1] = cfg.tier_top[0]              # not strictly increasing
    assert status(cfg) == P.PK_ERR_INVALID_ARG
    cfg = good_config()
    cfg.tier_weight[0] = 5                         # 16 subspaces x 5 > 64: S would not fit a byte lane
    assert status(cfg) == P.PK_ERR_UNSUPPORTED
    cfg = good_config()
    cfg.tier_weight[2] = -1
    assert status(cfg) == P.PK_ERR_INVALID_ARG
    assert P._lib.pk_validate_config(None) == P.PK_ERR_INVALID_ARG


def test_summary_bytes():
    cfg = good_config(batch=3, n_kv_heads=2, n_q_heads=4, n_capacity=1000)
    c, r, n, k = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert P._lib.pk_summary_bytes(ctypes.byref(cfg), ctypes.byref(c), ctypes.byref(r), ctypes.byref(n),
                                   ctypes.byref(k)) == 0
    rows = 3 * 2 * 1000
    assert (c.value, r.value, n.value, k.value) == (16 * rows, 128 * rows, 4 * rows, 6 * 16 * 256 * 4)
    cfg.head_dim = 64
    assert P._lib.pk_summary_bytes(ctypes.byref(cfg), None, None, None, None) == P.PK_ERR_UNSUPPORTED


def test_validate_tier_modes():
    cfg = good_config(tier_mode=P.PK_TIERS_PERCENTILE, collision_permille=200)
    cfg.tier_weight[0] = 200                       # rank-tier fields are not used with percentile tiers
    assert status(cfg) == P.PK_OK
    cfg.collision_permille = 0
    assert status(cfg) == P.PK_ERR_INVALID_ARG
    cfg.adaptive_ratios = 1                        # the ratio then comes from the zone-length table
    assert status(cfg) == P.PK_OK
    cfg.adaptive_ratios = 2
    assert status(cfg) == P.PK_ERR_INVALID_ARG
    cfg = good_config(tier_mode=7)
    assert status(cfg) == P.PK_ERR_INVALID_ARG
    cfg = good_config(tier_mode=P.PK_TIERS_PERCENTILE, collision_permille=1001)
    assert status(cfg) == P.PK_ERR_INVALID_ARG


def test_create_rejects_before_touching_a_device():
    out = ctypes.c_void_p()
    cfg = good_config(n_candidates=0)
    assert P._lib.pk_create(ctypes.byref(cfg), ctypes.byref(out)) == P.PK_ERR_INVALID_ARG
    assert out.value is None
    assert P._lib.pk_create(ctypes.byref(good_config()), None) == P.PK_ERR_INVALID_ARG
    P._lib.pk_destroy(None)                        # no-op


def test_host_alloc_rejects_bad_arguments():
    h, d = ctypes.c_void_p(), ctypes.c_void_p()
    assert P._lib.pk_host_alloc_mapped(0, ctypes.byref(h), ctypes.byref(d)) == P.PK_ERR_INVALID_ARG
    assert P._lib.pk_host_alloc_mapped(64, None, ctypes.byref(d)) == P.PK_ERR_INVALID_ARG


def test_calls_with_null_context_fail_cleanly():
    assert P._lib.pk_timing_begin(None, 8) == P.PK_ERR_INVALID_ARG
    assert P._lib.pk_timing_end(None, None) == P.PK_ERR_INVALID_ARG
    assert P._lib.pk_retrieve(None, None, 0, None, None, None, None, None) == P.PK_ERR_INVALID_ARG
    assert P._lib.pk_encode_keys(None, None, 0, P._I64x3(0, 0, 128), 0, None, None) == P.PK_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", [0, 1, 12345, 2**63 + 7])
def test_tables_equal_oracle(seed):
    signs = (ctypes.c_int8 * 128)()
    levels = (ctypes.c_float * 8)()
    thr = (ctypes.c_float * 7)()
    assert P._lib.pk_tables(ctypes.c_uint64(seed), signs, levels, thr) == 0
    np.testing.assert_array_equal(np.frombuffer(signs, np.int8), O.srht_signs(seed).astype(np.int8))
    L32, T32 = O.magnitude_tables_f32()
    assert np.frombuffer(levels, np.float32).tobytes() == L32.astype(np.float32).tobytes()
    assert np.frombuffer(thr, np.float32).tobytes() == T32.astype(np.float32).tobytes()
    assert P._lib.pk_tables(0, None, levels, thr) == P.PK_ERR_INVALID_ARG


@pytest.fixture
def fake_ctx():
    """A registered configuration under a handle that is never passed to the
    library: the binding's checks run, and each case below must raise before
    any call reaches it."""
    import torch  # noqa: F401
    cfg = good_config(batch=2, n_kv_heads=2, n_q_heads=8, top_k=16)
    h = ctypes.c_void_p(0x5EED0)
    P._CONFIGS[h.value] = cfg
    yield h, cfg
    P._CONFIGS.pop(h.value, None)


def test_binding_refuses_misshaped_tensors(fake_ctx):
    import torch
    h, cfg = fake_ctx
    B, Hq, Hk, k = cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.top_k
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16)
    idx = torch.zeros((B, Hq, k), dtype=torch.int32)
    out = torch.zeros((B, Hq, 128), dtype=torch.bfloat16)
    kv = torch.zeros((B, Hk, 64, 128), dtype=torch.bfloat16)
    sums = P.pk_summaries()
    cases = {
        "q heads": lambda: P.pk_retrieve(h, torch.zeros((B, Hq - 1, 128), dtype=torch.bfloat16), sums, idx),
        "q dim": lambda: P.pk_retrieve(h, torch.zeros((B, Hq, 64), dtype=torch.bfloat16), sums, idx),
        "q dtype": lambda: P.pk_retrieve(h, q.half(), sums, idx),
        "q strided": lambda: P.pk_retrieve(h, torch.zeros((B, Hq, 256), dtype=torch.bfloat16)[:, :, ::2], sums, idx),
        "topk_idx int64": lambda: P.pk_retrieve(h, q, sums, idx.long()),
        "topk_idx short": lambda: P.pk_retrieve(h, q, sums, idx[:, :, :k - 1]),
        "topk_est shape": lambda: P.pk_retrieve(h, q, sums, idx, torch.zeros((B, Hq, k + 1))),
        "out too small": lambda: P.pk_sparse_attend(h, q, kv, kv, idx, out[:, :Hq - 1]),
        "kv too few heads": lambda: P.pk_sparse_attend(h, q, kv[:, :Hk - 1], kv[:, :Hk - 1], idx, out),
        "kv too few sequences": lambda: P.pk_retrieve_attend(h, q, sums, kv[:B - 1], kv[:B - 1], idx, out),
        "k / v differ": lambda: P.pk_sparse_attend(h, q, kv, kv[:, :, :32], idx, out),
        "dense too few heads": lambda: P.pk_sparse_dense_attend(h, q, kv, kv, idx, kv[:, :1], kv[:, :1], out),
        "keys too few heads": lambda: P.pk_encode_keys(h, kv[:, :1], sums),
    }
    for name, call in cases.items():
        with pytest.raises(ValueError):
            call()
        assert name  # every case raised


def test_binding_refuses_host_tensors(fake_ctx):
    import torch
    h, cfg = fake_ctx
    q = torch.zeros((cfg.batch, cfg.n_q_heads, 128), dtype=torch.bfloat16)
    idx = torch.zeros((cfg.batch, cfg.n_q_heads, cfg.top_k), dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        P.pk_retrieve(h, q, P.pk_summaries(), idx)


def test_binding_refuses_unknown_context():
    import torch
    with pytest.raises(ValueError, match="context"):
        P.pk_retrieve(ctypes.c_void_p(0x5EED1), torch.zeros((1, 1, 128)), P.pk_summaries(),
                      torch.zeros((1, 1, 1), dtype=torch.int32))



def test_invalid_enum_values_are_refused():
    """Out-of-range dtypes and statuses from a caller are defined behaviour:
    refused or named unknown (the host-sanitized build checks that no
    undefined enum load happens)."""
    src = ctypes.create_string_buffer(4096 + 16)
    base = (ctypes.addressof(src) + 15) // 16 * 16
    st3 = P._I64x3(128, 128, 128)
    for bad in (7, -1, 2 ** 31 - 1, -2 ** 31):
        assert P._lib.pk_offload_rows(ctypes.c_void_p(base), st3, ctypes.c_void_p(base), st3, bad, 1, 1, 1,
                                      None) == P.PK_ERR_UNSUPPORTED
    for bad in (1, -6, -99, 2 ** 31 - 1, -2 ** 31):
        assert P._lib.pk_status_str(bad).decode() == "PK_ERR_UNKNOWN"


def test_offload_rows_rejects_before_launch():
    st3 = P._I64x3(128, 128, 128)
    assert P._lib.pk_offload_rows(None, st3, ctypes.c_void_p(256), st3, P.PK_BF16, 1, 1, 1, None) == \
        P.PK_ERR_INVALID_ARG
    assert P._lib.pk_offload_rows(ctypes.c_void_p(256), st3, ctypes.c_void_p(264), st3, P.PK_BF16, 1, 1, 1,
                                  None) == P.PK_ERR_INVALID_ARG          # misaligned destination
    assert P._lib.pk_offload_rows(ctypes.c_void_p(256), st3, ctypes.c_void_p(512), st3, P.PK_BF16, 0, 1, 1,
                                  None) == P.PK_ERR_INVALID_ARG          # no sequences
    # zero rows: valid, nothing to copy, no device touched
    assert P._lib.pk_offload_rows(ctypes.c_void_p(256), st3, ctypes.c_void_p(512), st3, P.PK_BF16, 1, 1, 0,
                                  None) == P.PK_OK
