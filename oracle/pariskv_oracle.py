"""ParisKV decode-path ORACLE.  Test infrastructure only.

A plain, slow CPU implementation (numpy / scipy, no GPU code) of what the ParisKV
decode path computes.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does, and this file imports nothing from the product.

Sources (cited by page title and the section / equation / frame on it):
  * README  -- "ParisKV: Fast and Drift-Robust KV-Cache Retrieval for
    Long-Context LLMs", the authors' repository README (sections "Key Insight",
    "1. Prefill", "2. Decode", "3. Attention", "Parameters", "Codebooks").
  * Slides  -- "ParisKV: Fast and Drift-Robust KV-Cache Retrieval", beamer
    slides of the ICML 2026 paper; each frame names the paper Sec./Eq./Table/Fig.

Two precisions are kept apart:
  * ``*_literal`` functions follow the pages' formulas in fp64;
  * ``*_f32`` functions fix the single-precision operation order that decides
    integer outputs (sign codes, 3-bit magnitude indices, centroid ranks) and
    the fp32 rerank estimate, so that a GPU implementation taking the same
    decisions in the same precision can be compared bit for bit.

Readings taken where the pages are silent:
  R1  SRHT: R = (1/sqrt(D)) * H * diag(s), H the Sylvester-ordered Hadamard
      matrix, s a vector of +-1 drawn from Philox4x64-10 with key (seed, 0):
      sign j = +1 iff the top bit of the j-th 64-bit output is 0, counters
      1, 2, ... (numpy's Philox stream).  No permutation / subsampling.
  R2  FWHT in fp32: butterfly stages h = 1, 2, ..., 64; the pair (j, j+h), j
      with bit h clear, becomes (a + b, a - b).
  R3  Sign code: bit j of the block code is 1 iff the rotated coordinate is
      > 0 (a zero coordinate takes bit 0 = the lower-index maximiser).
  R4  Magnitude quantiser: 8-level Lloyd-Max (MSE) quantiser of |u_j| under the
      exact marginal density of a coordinate of a uniform unit vector in R^m
      (u_j^2 ~ Beta(1/2, (m-1)/2)); index = #{thresholds <= |u_j|}.
  R5  Nibble = (sign bit << 3) | magnitude index; coordinate 2p in the low
      nibble of byte p.  A block with zero energy gets magnitude indices 0 and
      weight 0.
  R6  fp32 encode order: e = sum_j y_j*y_j sequentially (no fused multiply-add),
      rho = sqrt(e), u = y/rho, alpha = sum_j |u_j| * L[idx_j] sequentially,
      w = (rho * fl32(1/sqrt(D))) / alpha  (= ||k|| r_b / alpha_b of Eq. (9)).
  R7  Query centroid score of pattern c in block b: sum over j of
      (bit_j(c) ? +y_j : -y_j) in fp32, sequential in j, started from the
      j = 0 term; ranked by (score desc, centroid index asc); -0 == +0.
  R8  Tiers (workload table): the query's top-1 / top-4 / top-16 centroids per
      block carry weights 4 / 2 / 1, disjoint (innermost weight applies).
  R9  Candidates: the C largest collision scores, ties by ascending key index;
      returned in ascending index order; all keys when n <= C.
  R10 fp32 rerank order: p_j = v_j * Rq_j, d_b = sum_j p_j sequentially, t_b =
      w_b * d_b, est = sum_b t_b sequentially (no fused multiply-add).
  R11 Final Top-k by (estimate desc, key index asc).
  R12 Attention softmax over the retrieved rows only, scores scale * <k_i, q>.
  R13 Percentile tiers (Slides, frame "Stage I uses multi-tier collision
      votes to prune keys", Sec. 4.2.2, Eq. (15)): in block b every key is
      scored by its centroid, so the key order within a block is the centroid
      order of R7 with a centroid's keys side by side.  A centroid whose first
      key sits at position P (the number of keys in better-ranked centroids)
      is kept iff P < M = ceil(rho n), and lies in tier floor(6 P / M) of the
      six equal percentile slices of the kept positions; tiers 0..5 add the
      bonuses 6..1.  A centroid that straddles a slice boundary takes the tier
      of its first key.
  R14 Ratios are fractions of the retrieval zone rounded up: C = ceil(beta n),
      M = ceil(rho n), with beta and rho from the README's zone-length table
      when they adapt; they are kept as per-mille integers so that the count is
      exact.
"""
from __future__ import annotations

import numpy as np
import scipy.linalg
import scipy.special

D = 128          # head dimension
N_SUB = 16       # B, subspaces per key
SUB_DIM = 8      # m = D / B
N_CENTROIDS = 1 << SUB_DIM   # |Omega| = 2^m
N_LEVELS = 8     # 3-bit magnitude index
RECORD_NIBBLE_BYTES = D // 2

F32 = np.float32
INV_SQRT_D_F32 = np.float32(1.0 / np.sqrt(float(D)))


# =============================================================================
# Tables
# =============================================================================
def srht_signs(seed: int) -> np.ndarray:
    """SRHT sign vector s (int8, +-1), reading R1.

    Slides, frame "Normalization and rotation enable a fixed codebook"
    (Sec. 4.1.1, Eq. (5)): R is one shared orthogonal transform implemented
    with an SRHT.  The random signs come from the Philox4x64-10 counter-based
    generator (Salmon et al., SC'11) as numpy implements it."""
    raw = np.random.Philox(key=int(seed)).random_raw(D)
    top = (raw >> np.uint64(63)).astype(np.int8)
    return (1 - 2 * top).astype(np.int8)


def hadamard(n: int = D) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix (+-1 entries), fp64."""
    return scipy.linalg.hadamard(n).astype(np.float64)


def rotation_matrix(signs: np.ndarray) -> np.ndarray:
    """R = H diag(s) / sqrt(D) in fp64 (reading R1)."""
    return hadamard(D) * signs.astype(np.float64)[None, :] / np.sqrt(D)


def magnitude_cdf(a, m: int = SUB_DIM):
    """P(|u_j| <= a) for u uniform on the unit sphere of R^m.

    Slides, frame "The codebook is data-independent; the quantizer uses a
    prior" (Prop. 4.1) and backup frame "why the rotation prior is Beta"
    (App. B.1.1-B.1.2): (u_b)_j^2 ~ Beta(1/2, (m-1)/2)."""
    a = np.asarray(a, dtype=np.float64)
    return scipy.special.betainc(0.5, (m - 1) / 2.0, np.clip(a, 0.0, 1.0) ** 2)


def magnitude_partial_mean(a, m: int = SUB_DIM):
    """E[|u_j| ; |u_j| <= a] under the same prior.

    With Y = u_j^2 ~ Beta(1/2, b), b = (m-1)/2:  E[sqrt(Y); Y <= a^2]
    = B(1, b) I_{a^2}(1, b) / B(1/2, b)."""
    a = np.asarray(a, dtype=np.float64)
    b = (m - 1) / 2.0
    return (scipy.special.betainc(1.0, b, np.clip(a, 0.0, 1.0) ** 2)
            * scipy.special.beta(1.0, b) / scipy.special.beta(0.5, b))


def lloyd_max_levels(n_levels: int = N_LEVELS, m: int = SUB_DIM,
                     tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd-Max (MSE-optimal) scalar quantiser of |u_j| (reading R4), fp64.

    README "Codebooks": the 3-bit magnitude codebook has 8 levels for m = 8.
    Slides, frame "The codebook is data-independent; the quantizer uses a
    prior" (App. B.1): shared 3-bit levels from offline Lloyd-Max quantisation
    of the Beta prior; a fourth bit stores the sign.

    Alternates the two optimality conditions (thresholds at midpoints of
    adjacent levels, levels at conditional means of their cells) until the
    levels move less than `tol`.  Returns (levels[n_levels], thresholds[n_levels-1])."""
    # start from the prior's quantiles
    probs = (np.arange(n_levels) + 0.5) / n_levels
    grid = np.linspace(0.0, 1.0, 200001)
    cdf = magnitude_cdf(grid, m)
    L = np.interp(probs, cdf, grid)
    for _ in range(max_iter):
        tau = 0.5 * (L[:-1] + L[1:])
        edges = np.concatenate([[0.0], tau, [1.0]])
        Fm = magnitude_cdf(edges, m)
        Gm = magnitude_partial_mean(edges, m)
        L_new = (Gm[1:] - Gm[:-1]) / (Fm[1:] - Fm[:-1])
        done = np.max(np.abs(L_new - L)) < tol
        L = L_new
        if done:
            break
    tau = 0.5 * (L[:-1] + L[1:])
    return L, tau


def magnitude_tables_f32(m: int = SUB_DIM):
    """The fp32 level / threshold tables both encode and rerank consume."""
    L, tau = lloyd_max_levels(N_LEVELS, m)
    return L.astype(F32), tau.astype(F32)


def sign_patterns() -> np.ndarray:
    """Omega without the 1/sqrt(m) factor: [256, 8] of +-1, bit j of c -> coord j,
    bit value 1 -> +1 (Slides, Eq. (6): Omega = {+-1/sqrt(m)}^m)."""
    c = np.arange(N_CENTROIDS)[:, None]
    bits = (c >> np.arange(SUB_DIM)[None, :]) & 1
    return (2 * bits - 1).astype(np.int8)


# =============================================================================
# Fast Walsh-Hadamard transform
# =============================================================================
def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform over the last axis (length 128),
    butterfly stages h = 1, 2, ..., 64 (reading R2), in the dtype of `x`.
    Equals H @ x exactly in real arithmetic."""
    y = np.array(x, copy=True)
    lead = y.shape[:-1]
    h = 1
    while h < D:
        y = y.reshape(*lead, D // (2 * h), 2, h)
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)
        h *= 2
    return y.reshape(*lead, D)


# =============================================================================
# Key encoding (prefill summaries; README "1. Prefill"; Slides Eqs. (5)-(9))
# =============================================================================
def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[n, 128] nibbles -> [n, 64] bytes, coordinate 2p in the low nibble (R5)."""
    nib = nib.astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], D), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def encode_f32(keys: np.ndarray, signs: np.ndarray, L32: np.ndarray, tau32: np.ndarray):
    """Encode keys (float32 [n, 128]) in the fp32 order of reading R6.

    Slides, frame "Normalization and rotation enable a fixed codebook"
    (Eqs. (5)-(6)): normalise, rotate with the shared R, split into B blocks of
    m coordinates, assign each block its sign-pattern centroid.  Frame "Stage II
    estimates the raw attention score from 4-bit codes" (Eqs. (7)-(9)):
    r = ||k~_b||, u = k~_b / r, alpha = <v, u>, w = ||k|| r / alpha.
    README "1. Prefill": two summaries -- centroid IDs, and 4-bit direction
    codes plus per-subspace weights.

    Normalisation cancels in w and in the codes, so the fp32 path rotates the
    raw key: y = H (s * k), rho_b = ||y_b||, w_b = rho_b * fl32(1/sqrt(D)) / alpha_b.

    Returns dict(codes u8 [n,16], nibbles u8 [n,64], weights f32 [n,16],
    norms f32 [n], y f32 [n,128])."""
    k = np.asarray(keys, dtype=F32)
    n = k.shape[0]
    x = k * signs.astype(F32)[None, :]
    y = fwht(x)
    yb = y.reshape(n, N_SUB, SUB_DIM)
    e = yb[..., 0] * yb[..., 0]
    for j in range(1, SUB_DIM):
        e = e + yb[..., j] * yb[..., j]
    rho = np.sqrt(e)
    bits = (yb > 0)
    codes = np.zeros((n, N_SUB), dtype=np.uint8)
    for j in range(SUB_DIM):
        codes |= (bits[..., j].astype(np.uint8) << j)
    nz = rho > 0
    safe_rho = np.where(nz, rho, F32(1.0))
    u = yb / safe_rho[..., None]
    a = np.abs(u)
    idx = np.zeros(a.shape, dtype=np.uint8)
    for t in tau32:
        idx += (a >= t).astype(np.uint8)
    idx = np.where(nz[..., None], idx, 0).astype(np.uint8)
    La = L32[idx]
    alpha = a[..., 0] * La[..., 0]
    for j in range(1, SUB_DIM):
        alpha = alpha + a[..., j] * La[..., j]
    safe_alpha = np.where(nz, alpha, F32(1.0))
    w = np.where(nz, (rho * INV_SQRT_D_F32) / safe_alpha, F32(0.0)).astype(F32)
    nib = ((bits.astype(np.uint8) << 3) | idx).reshape(n, D)
    norms = np.sqrt(np.sum(k.astype(np.float64) ** 2, axis=1)).astype(F32)
    return dict(codes=codes, nibbles=pack_nibbles(nib), weights=w, norms=norms, y=y)


def encode_literal(keys: np.ndarray, signs: np.ndarray, L: np.ndarray, tau: np.ndarray):
    """The pages' encoding in fp64, formula by formula (Slides Eqs. (5)-(9)).

    k^ = k/||k||, k~ = R k^; per block r_b = ||k~_b||, u_b = k~_b / r_b,
    c_b = argmax over Omega of u_b . omega (brute force over 256 centres),
    v_b = sign-of-centre * L[index], alpha_b = <v_b, u_b>, w_b = ||k|| r_b / alpha_b.
    Returns dict(codes, mag_idx [n,128], weights f64, norms f64, u f64)."""
    k = np.asarray(keys, dtype=np.float64)
    n = k.shape[0]
    R = rotation_matrix(signs)
    norm = np.sqrt(np.sum(k * k, axis=1))
    khat = k / np.where(norm > 0, norm, 1.0)[:, None]
    kt = khat @ R.T
    kb = kt.reshape(n, N_SUB, SUB_DIM)
    r = np.sqrt(np.sum(kb * kb, axis=2))
    u = kb / np.where(r > 0, r, 1.0)[..., None]
    omega = sign_patterns().astype(np.float64) / np.sqrt(SUB_DIM)      # [256, 8]
    ip = np.einsum("nbj,cj->nbc", u, omega)
    codes = np.argmax(ip, axis=2).astype(np.uint8)                        # lowest index on ties
    a = np.abs(u)
    mag = np.zeros(a.shape, dtype=np.int64)
    for t in np.asarray(tau, dtype=np.float64):
        mag += (a >= t)
    sgn = sign_patterns()[codes.astype(np.int64)].astype(np.float64)     # [n,16,8]
    v = sgn * np.asarray(L, dtype=np.float64)[mag]
    alpha = np.sum(v * u, axis=2)
    w = np.where(r > 0, norm[:, None] * r / np.where(alpha != 0, alpha, 1.0), 0.0)
    return dict(codes=codes, mag_idx=mag.reshape(n, D), weights=w, norms=norm, u=u)


# =============================================================================
# Query side: rotation, centroid activation, tier table
# =============================================================================
def qprep_f32(q: np.ndarray, signs: np.ndarray):
    """Rotate one query and score every centroid of every block (R7).

    README "2. Decode": each query activates the nearest direction centroids in
    every subspace.  Slides, Eq. (5): q~ = R q^.  The rerank needs
    ||q|| q~_b = (R q)_b, kept as Rq = fl32(y * fl32(1/sqrt(D))).

    Returns (Rq f32 [128], y f32 [128], scores f32 [16, 256])."""
    x = np.asarray(q, dtype=F32) * signs.astype(F32)
    y = fwht(x)
    Rq = (y * INV_SQRT_D_F32).astype(F32)
    pats = sign_patterns().astype(F32)                                     # [256, 8]
    yb = y.reshape(N_SUB, SUB_DIM)
    scores = np.empty((N_SUB, N_CENTROIDS), dtype=F32)
    for b in range(N_SUB):
        terms = pats * yb[b][None, :]                                      # exact sign flips
        s = terms[:, 0]
        for j in range(1, SUB_DIM):
            s = s + terms[:, j]
        scores[b] = s
    return Rq, y, scores


def centroid_ranks(scores: np.ndarray) -> np.ndarray:
    """Rank of each centroid within its block by (score desc, index asc)."""
    ranks = np.empty(scores.shape, dtype=np.int64)
    cidx = np.arange(scores.shape[1])
    for b in range(scores.shape[0]):
        order = np.lexsort((cidx, -scores[b].astype(np.float64)))
        ranks[b, order] = np.arange(scores.shape[1])
    return ranks


def tier_weights(ranks: np.ndarray, tier_top, tier_weight) -> np.ndarray:
    """Per-(block, centroid) vote weight from the centroid's rank (R8).

    Slides, frame "Stage I uses multi-tier collision votes to prune keys"
    (Eq. (15)): each (key, block) falls in at most one tier l(i, b) and adds
    that tier's weight."""
    w = np.zeros(ranks.shape, dtype=np.int64)
    assigned = np.zeros(ranks.shape, dtype=bool)
    for top, wt in zip(tier_top, tier_weight):
        hit = (ranks < top) & ~assigned
        w[hit] = wt
        assigned |= hit
    return w


# =============================================================================
# Stage I: collision votes and candidate selection
# =============================================================================
def collision_scores(codes: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """S_i = sum_b weight_b(code_{i,b})  (Slides Eq. (15)); int64 [n]."""
    codes = np.asarray(codes, dtype=np.int64)
    return weights[np.arange(N_SUB)[None, :], codes].sum(axis=1)


# -----------------------------------------------------------------------------
# Percentile tiers and adaptive ratios
# -----------------------------------------------------------------------------
PERCENTILE_BONUSES = (6, 5, 4, 3, 2, 1)
# README "Parameters": (zone length below, candidate ratio, collision ratio), per mille
ADAPTIVE_RATIOS_PERMILLE = ((5000, 500, 500), (10000, 250, 300), (30000, 200, 250), (None, 100, 200))


def adaptive_ratios_permille(zone_len: int):
    """(beta, rho) in 1/1000 for a retrieval zone of zone_len keys (R14)."""
    for limit, beta, rho in ADAPTIVE_RATIOS_PERMILLE:
        if limit is None or zone_len < limit:
            return beta, rho
    raise AssertionError("unreachable")


def ratio_count(permille: int, n: int) -> int:
    """ceil(permille / 1000 * n), exact (R14)."""
    return (permille * n + 999) // 1000


def centroid_occupancy(codes: np.ndarray) -> np.ndarray:
    """Keys per (block, centroid): int64 [16, 256]."""
    codes = np.asarray(codes, dtype=np.int64).reshape(-1, N_SUB)
    counts = np.zeros((N_SUB, N_CENTROIDS), dtype=np.int64)
    for b in range(N_SUB):
        counts[b] = np.bincount(codes[:, b], minlength=N_CENTROIDS)
    return counts


def percentile_tier_weights(ranks: np.ndarray, counts: np.ndarray, M: int,
                            bonuses=PERCENTILE_BONUSES) -> np.ndarray:
    """Per-(block, centroid) bonus of the six percentile tiers of the top M
    keys of each block (R13; Slides Sec. 4.2.2, Eq. (15))."""
    nt = len(bonuses)
    w = np.zeros(ranks.shape, dtype=np.int64)
    for b in range(ranks.shape[0]):
        first = 0                                   # keys in better-ranked centroids
        for c in np.argsort(ranks[b], kind="stable"):
            if first >= M:
                break
            w[b, c] = bonuses[(nt * first) // M]
            first += int(counts[b, c])
    return w


def select_candidates(S: np.ndarray, C: int) -> np.ndarray:
    """Indices of the C largest S, ties by ascending index, returned ascending (R9).

    Slides, frame "Stage I ..." (Sec. 4.2.2): keep the top-beta keys by S_i;
    frame "Fewer transferred bytes ..." (Sec. 4.3): C = ceil(beta n)."""
    S = np.asarray(S)
    n = S.shape[0]
    idx = np.arange(n)
    order = np.lexsort((idx, -S))
    return np.sort(order[:min(C, n)])


# =============================================================================
# Stage II: 4-bit rerank, final Top-k
# =============================================================================
def nibble_values(nibbles_packed: np.ndarray, L32: np.ndarray) -> np.ndarray:
    """v_{i,b,j} = (sign bit ? +1 : -1) * L[magnitude index], fp32 [n, 128]."""
    nib = unpack_nibbles(nibbles_packed)
    mag = L32[nib & 7]
    return np.where((nib & 8) != 0, mag, -mag).astype(F32)


def rerank_f32(nibbles_packed, weights, Rq, L32) -> np.ndarray:
    """fp32 estimate of <k_i, q> in the order of reading R10.

    Slides, frame "Stage II estimates the raw attention score from 4-bit codes"
    (Eq. (10)): <k, q> ~= ||q|| sum_b w_b <v_b, q~_b> = sum_b w_b <v_b, Rq_b>."""
    v = nibble_values(nibbles_packed, L32)
    n = v.shape[0]
    p = (v * np.asarray(Rq, dtype=F32)[None, :]).reshape(n, N_SUB, SUB_DIM)
    d = p[..., 0]
    for j in range(1, SUB_DIM):
        d = d + p[..., j]
    t = np.asarray(weights, dtype=F32) * d
    est = t[:, 0]
    for b in range(1, N_SUB):
        est = est + t[:, b]
    return est.astype(F32)


def rerank_f64(nibbles_packed, weights, Rq, L32) -> np.ndarray:
    """The same estimator evaluated in fp64 from the fp32 inputs."""
    v = nibble_values(nibbles_packed, L32).astype(np.float64)
    n = v.shape[0]
    vb = v.reshape(n, N_SUB, SUB_DIM)
    qb = np.asarray(Rq, dtype=np.float64).reshape(N_SUB, SUB_DIM)
    return np.einsum("nb,nb->n", np.asarray(weights, dtype=np.float64),
                     np.einsum("nbj,bj->nb", vb, qb))


def rerank_abs_scale(nibbles_packed, weights, Rq, L32) -> np.ndarray:
    """sum_b |w_b| sum_j |v_j Rq_j|: the scale the 1e-5 rerank tolerance is relative to."""
    v = np.abs(nibble_values(nibbles_packed, L32).astype(np.float64))
    n = v.shape[0]
    qb = np.abs(np.asarray(Rq, dtype=np.float64)).reshape(N_SUB, SUB_DIM)
    return np.einsum("nb,nb->n", np.abs(np.asarray(weights, dtype=np.float64)),
                     np.einsum("nbj,bj->nb", v.reshape(n, N_SUB, SUB_DIM), qb))


def estimate_literal(enc_lit: dict, q: np.ndarray, signs: np.ndarray, L: np.ndarray) -> np.ndarray:
    """Eq. (10) in fp64 from the literal encoding: ||q|| sum_b w_b <v_b, q~_b>."""
    q = np.asarray(q, dtype=np.float64)
    qn = np.sqrt(q @ q)
    qt = rotation_matrix(signs) @ (q / qn)
    sgn = sign_patterns()[enc_lit["codes"].astype(np.int64)].astype(np.float64)
    n = sgn.shape[0]
    v = sgn * np.asarray(L, dtype=np.float64)[enc_lit["mag_idx"].reshape(n, N_SUB, SUB_DIM)]
    ip = np.einsum("nbj,bj->nb", v, qt.reshape(N_SUB, SUB_DIM))
    return qn * np.sum(enc_lit["weights"] * ip, axis=1)


def top_k(est: np.ndarray, cand: np.ndarray, k: int):
    """Top-k of the candidates by (estimate desc, index asc) (R11).

    Slides, frame "The memory layout amortizes updates and fetches Top-k"
    (Sec. 4.2.3): reranking returns the Top-100 indices."""
    est = np.asarray(est)
    cand = np.asarray(cand)
    order = np.lexsort((cand, -est.astype(np.float64)))[:min(k, cand.shape[0])]
    return cand[order], est[order]


# =============================================================================
# Sparse attention over the retrieved rows
# =============================================================================
def sparse_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
                     scale: float) -> np.ndarray:
    """o = sum_i softmax(s)_i v_i over the retrieved rows only, s_i = scale <k_i, q>.

    Slides, frame "The target is high-score KV indices at each decode step"
    (Sec. 3, Eqs. (1)-(3)): recompute softmax and value aggregation on the
    selected full-precision KV.  README "3. Attention".  fp64; indices < 0
    are padding and skipped; an empty set gives a zero output."""
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    if idx.size == 0:
        return np.zeros(D, dtype=np.float64)
    k = np.asarray(K, dtype=np.float64)[idx]
    v = np.asarray(V, dtype=np.float64)[idx]
    s = scale * (k @ np.asarray(q, dtype=np.float64))
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ v


def layout_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
                     K_dense: np.ndarray, V_dense: np.ndarray, scale: float) -> np.ndarray:
    """One softmax over the retrieved rows K[idx] and every dense row.

    README "3. Attention": attention runs over the sink tokens, the local
    tokens and the retrieved tokens; Slides, frame "The memory layout
    amortizes updates and fetches Top-k" (Fig. 5, Sec. 4.2.1-4.2.3): sink and
    recent local tokens (with the update buffer) stay on the GPU for dense
    attention.  K_dense / V_dense hold those rows; fp64, padding indices < 0
    skipped, zero output when nothing is attended."""
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    k = np.concatenate([np.asarray(K, dtype=np.float64)[idx], np.asarray(K_dense, dtype=np.float64).reshape(-1, D)])
    v = np.concatenate([np.asarray(V, dtype=np.float64)[idx], np.asarray(V_dense, dtype=np.float64).reshape(-1, D)])
    if k.shape[0] == 0:
        return np.zeros(D, dtype=np.float64)
    s = scale * (k @ np.asarray(q, dtype=np.float64))
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ v


def exact_topk(K: np.ndarray, q: np.ndarray, k: int) -> np.ndarray:
    """Exact Top-k of <k_i, q> over all keys (fp64), ties by ascending index."""
    s = np.asarray(K, dtype=np.float64) @ np.asarray(q, dtype=np.float64)
    idx = np.arange(s.shape[0])
    return np.lexsort((idx, -s))[:min(k, s.shape[0])]


# =============================================================================
# One decode step for one (sequence, KV head) unit
# =============================================================================
def decode_unit(qs, keys_f32, values, enc, signs, L32, tier_top, tier_weight,
                C: int, k: int, scale: float, n: int | None = None, percentile_M: int | None = None):
    """Retrieve and attend for the G query heads of one unit.

    qs: float32 [G, 128]; keys_f32 / values: [>= n, 128]; enc: encode_f32 output
    (or the same fields from elsewhere) covering >= n keys.
    Returns a list (one per head) of dicts with Rq, scores, weights, S, cand,
    est32, est64, scale64, top_idx, top_est, out.
    With percentile_M the votes use the percentile tiers of the top
    percentile_M keys per block (R13) instead of the rank tiers."""
    n = enc["codes"].shape[0] if n is None else n
    codes = enc["codes"][:n]
    counts = centroid_occupancy(codes) if percentile_M is not None else None
    nib = enc["nibbles"][:n]
    w = enc["weights"][:n]
    out = []
    for q in np.asarray(qs, dtype=F32):
        Rq, _, sc = qprep_f32(q, signs)
        if percentile_M is None:
            wt = tier_weights(centroid_ranks(sc), tier_top, tier_weight)
        else:
            wt = percentile_tier_weights(centroid_ranks(sc), counts, percentile_M)
        S = collision_scores(codes, wt)
        cand = select_candidates(S, C)
        est32 = rerank_f32(nib[cand], w[cand], Rq, L32)
        est64 = rerank_f64(nib[cand], w[cand], Rq, L32)
        absc = rerank_abs_scale(nib[cand], w[cand], Rq, L32)
        ti, te = top_k(est32, cand, k)
        o = sparse_attention(q, keys_f32[:n], values[:n], ti, scale)
        out.append(dict(Rq=Rq, scores=sc, weights=wt, S=S, cand=cand, est32=est32,
                        est64=est64, abs_scale=absc, top_idx=ti, top_est=te, out=o))
    return out
