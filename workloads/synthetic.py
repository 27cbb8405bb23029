"""Seeded synthetic inputs for the ParisKV decode path.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic; both the CPU oracle (``oracle/``)
and the GPU side (tests, bench) take their inputs from here.

Workload shapes follow the Llama-3.1-8B-shaped decode settings used for the
efficiency study in the ParisKV slides (frame "Evaluation spans long generation
and long input": Llama3.1-8B / Qwen3-8B, 64K-1024K contexts, batch and
single-request analyses; frame "At 1024K, on-demand KV access cuts decode
latency": 1024K context, batch 1, Top-100).  The real KV tensors of those models
and the evaluation datasets are not available, so these seeded tensors stand in
for them:

* keys    z ~ N(0, 1) per coordinate (float32 draws), four outlier channels per
          (sequence, KV head) scaled by 8, then a shared +0.5 offset on every
          channel, rounded to the storage dtype (bf16 RNE, or kept fp32);
* values  N(0, 1), same dtype;
* queries 0.7 * (sum of `planted` distinct keys of the head's KV head, drawn
          uniformly without replacement) + N(0, I) noise, rounded to the dtype;
* drift   appended key t (t = 0..steps-1) uses offset 0.5 - t/(steps-1) with
          the head's outlier channels.

Seeds are tuples ``(workload id, stream, ...)`` fed to numpy's PCG64 through
``default_rng``; every (sequence, head) is generated independently so a test can
regenerate one unit without the rest.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
N_OUTLIER = 4
OUTLIER_SCALE = 8.0
MEAN_OFFSET = 0.5
PLANT_WEIGHT = 0.7

# stream ids inside a workload's seed tuple
_S_KEYS, _S_VALUES, _S_QUERY, _S_APPEND_K, _S_APPEND_V = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace
    batch: int
    n_kv_heads: int
    n_q_heads: int
    n: int                   # prefill keys per (sequence, KV head)
    kv_dtype: str            # "f32" or "bf16"
    n_candidates: int        # C
    top_k: int = 100
    planted: int = 64
    kv_home: str = "hbm"     # "hbm" or "host" (pinned, read through a mapped pointer)
    append_steps: int = 0    # drift stream: one appended key per KV head per step
    # method constants (fixed by the workload table)
    srht_seed: int = 0
    tier_top: tuple = (1, 4, 16)
    tier_weight: tuple = (4, 2, 1)
    # vote tiers: "rank" (the tiers above) or "percentile" (six percentile tiers
    # of the top collision_permille / 1000 keys per block); with adaptive the
    # candidate and collision ratios follow the retrieval-zone length and
    # n_candidates is the largest candidate count the run may need
    tier_mode: str = "rank"
    collision_permille: int = 0
    adaptive: bool = False
    # sink / local / update-buffer layout: the first sink_tokens prefill rows
    # and a window of the newest tokens are attended densely; the window holds
    # local_tokens plus up to update_tokens new ones, after which the oldest
    # update_tokens of it move into the summarised retrieval zone
    sink_tokens: int = 0
    local_tokens: int = 0
    update_tokens: int = 0
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def units(self) -> int:
        return self.batch * self.n_kv_heads

    @property
    def n_capacity(self) -> int:
        return self.n + self.append_steps

    @property
    def softmax_scale(self) -> float:
        return 1.0 / np.sqrt(HEAD_DIM)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny4k", 1, 1, 1, 1, 4096, "f32", 512, planted=20),
        Workload("llama32k", 2, 1, 8, 32, 32768, "bf16", 2048),
        Workload("batched128k", 3, 8, 8, 32, 131072, "bf16", 4096),
        Workload("offload1m", 4, 1, 8, 32, 1048576, "bf16", 8192, kv_home="host"),
        Workload("drift128k", 5, 1, 8, 32, 131072, "bf16", 4096, append_steps=1024),
        # the pages' own Stage I: percentile tiers with adaptive ratios
        # (at n = 131072: beta = 0.1 -> C = 13108, rho = 0.2)
        Workload("batched128k_pct", 6, 8, 8, 32, 131072, "bf16", 13108, tier_mode="percentile", adaptive=True),
        # decode stream with the pages' memory layout: 64 sink tokens, a
        # 512-token local window and a 256-token update buffer stay dense;
        # the zone (the rest of the 128K prefill) is retrieved from
        Workload("drift128k_layout", 7, 1, 8, 32, 131072, "bf16", 4096, append_steps=1024, sink_tokens=64,
                 local_tokens=512, update_tokens=256),
        # the same with the zone's K/V in pinned host memory: flushed rows are
        # offloaded there and read back through mapped pointers
        Workload("drift128k_layout_host", 7, 1, 8, 32, 131072, "bf16", 4096, append_steps=1024, sink_tokens=64,
                 local_tokens=512, update_tokens=256, kv_home="host"),
    ]
}


def custom(base: str, **kw) -> Workload:
    """A workload with the recipe of `base` but other sizes (ragged / edge cases)."""
    w = WORKLOADS[base]
    d = {f: getattr(w, f) for f in w.__dataclass_fields__ if f != "extra"}
    d.update(kw)
    return Workload(**d)


# ----------------------------------------------------------------------------
# dtype helpers (storage rounding only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rnd = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rnd) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(dtype)


def as_f32(x: np.ndarray) -> np.ndarray:
    """Storage array (uint16 bf16 bits or float32) -> exact float32 values."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def _rng(*seed: int) -> np.random.Generator:
    return np.random.default_rng([int(s) for s in seed])


# ----------------------------------------------------------------------------
# per-unit generators
# ----------------------------------------------------------------------------
def outlier_channels(w: Workload, b: int, h: int) -> np.ndarray:
    return _rng(w.wid, _S_KEYS, b, h).choice(HEAD_DIM, N_OUTLIER, replace=False)


def unit_keys(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    """Prefill keys of (sequence b, KV head h): storage dtype, shape [n, 128]."""
    n = w.n if n is None else n
    rng = _rng(w.wid, _S_KEYS, b, h)
    ch = rng.choice(HEAD_DIM, N_OUTLIER, replace=False)
    z = rng.standard_normal((n, HEAD_DIM), dtype=np.float32)
    z[:, ch] *= np.float32(OUTLIER_SCALE)
    z += np.float32(MEAN_OFFSET)
    return to_storage(z, w.kv_dtype)


def unit_values(w: Workload, b: int, h: int, n: int | None = None) -> np.ndarray:
    n = w.n if n is None else n
    z = _rng(w.wid, _S_VALUES, b, h).standard_normal((n, HEAD_DIM), dtype=np.float32)
    return to_storage(z, w.kv_dtype)


def drift_offset(w: Workload, t: int) -> float:
    if w.append_steps <= 1:
        return MEAN_OFFSET
    return MEAN_OFFSET - t / (w.append_steps - 1)


def appended_key(w: Workload, b: int, h: int, t: int) -> np.ndarray:
    """Key appended at decode step t to (b, h): storage dtype, shape [128]."""
    ch = outlier_channels(w, b, h)
    z = _rng(w.wid, _S_APPEND_K, t, b, h).standard_normal(HEAD_DIM, dtype=np.float32)
    z[ch] *= np.float32(OUTLIER_SCALE)
    z += np.float32(drift_offset(w, t))
    return to_storage(z, w.kv_dtype)


def appended_value(w: Workload, b: int, h: int, t: int) -> np.ndarray:
    z = _rng(w.wid, _S_APPEND_V, t, b, h).standard_normal(HEAD_DIM, dtype=np.float32)
    return to_storage(z, w.kv_dtype)


def query(w: Workload, b: int, qh: int, keys, step: int = 0, n_t: int | None = None) -> np.ndarray:
    """Planted query for (sequence b, q head qh) against the first `n_t` current
    keys of its KV head.  `keys` is that head's storage array [>=n_t, 128] or a
    callable mapping a row-index array to storage rows.  Returns the storage
    dtype, shape [128]."""
    rng = _rng(w.wid, _S_QUERY, step, b, qh)
    if n_t is None:
        n_t = keys.shape[0]
    m = min(w.planted, n_t)
    J = np.sort(rng.choice(n_t, m, replace=False))
    eps = rng.standard_normal(HEAD_DIM)
    rows = keys(J) if callable(keys) else keys[J]
    q = PLANT_WEIGHT * as_f32(rows).astype(np.float64).sum(axis=0) + eps
    return to_storage(q.astype(np.float32), w.kv_dtype)


# ----------------------------------------------------------------------------
# whole-workload generators (threaded; each unit is independent)
# ----------------------------------------------------------------------------
def _pool_size() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def all_units(w: Workload, fn, n: int | None = None) -> np.ndarray:
    """[batch, n_kv_heads, n, 128] storage array built unit by unit with `fn`."""
    n = w.n if n is None else n
    dt = np.uint16 if w.kv_dtype == "bf16" else np.float32
    out = np.empty((w.batch, w.n_kv_heads, n, HEAD_DIM), dtype=dt)

    def one(u):
        b, h = divmod(u, w.n_kv_heads)
        out[b, h] = fn(w, b, h, n)

    with ThreadPoolExecutor(_pool_size()) as ex:
        list(ex.map(one, range(w.units)))
    return out


def all_keys(w: Workload, n: int | None = None) -> np.ndarray:
    return all_units(w, unit_keys, n)


def all_values(w: Workload, n: int | None = None) -> np.ndarray:
    return all_units(w, unit_values, n)


def all_queries(w: Workload, keys, step: int = 0, n_t: int | None = None) -> np.ndarray:
    """[batch, n_q_heads, 128] queries.  `keys` is the storage array
    [batch, n_kv_heads, >=n_t, 128] of current keys, or a callable
    (b, h, J) -> storage rows."""
    dt = np.uint16 if w.kv_dtype == "bf16" else np.float32
    out = np.empty((w.batch, w.n_q_heads, HEAD_DIM), dtype=dt)
    if n_t is None:
        n_t = keys.shape[2]
    for b in range(w.batch):
        for qh in range(w.n_q_heads):
            h = qh // w.group
            src = (lambda J, b=b, h=h: keys(b, h, J)) if callable(keys) else keys[b, h]
            out[b, qh] = query(w, b, qh, src, step, n_t)
    return out
