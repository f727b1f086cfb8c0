"""Plain fp64 CPU oracle of one SparsePR attention call.

TEST INFRASTRUCTURE ONLY: only the test suite, the smoke check and the bench's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

Sources (cited by page title and section; no code is copied from any page):
  [PR]   "Partition the Support, Reconstruct the Residual: Training-Free Sparse
         Attention for Video Generation and World Models" (gist.science summary),
         technical summary section 2 (A response-coupled partitioning, B probe-fitted
         residual reconstruction, C sparse execution).
  [SVOO] "Attention Sparsity is Input-Stable: ... Online QK Co-Clustering"
         (papernotes.org), key-design item "block selection + sparse attention
         assembly" (centroid-logit top-k, softmax over the kept logits).
  [BLOG] "SparsePR稀疏注意力：无训练加速视频生成与世界模型推理" (framerc.cn),
         section 1.2 (the attention formula) and section 7.3 (per-head selection).
  [BAIDU] cloud.baidu.com sparse-attention explainer, the masked-score pseudocode
         paragraph (mask first, then softmax over the allowed positions).

Where the pages leave a step open, the reading taken is stated in the function's
docstring. Every function works on one head; heads are independent ([BLOG] 7.3).
All floating point is fp64.

Parity status: every function below is pinned by tests that do not re-derive it
from itself (brute force, closed forms, second formulations, invariants).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

GOLDEN_32 = 0x9E3779B9   # floor(2^32 / golden ratio)


# ---------------------------------------------------------------- sampling ---
def weyl_multiplier(n: int) -> int:
    """Multiplier a of the golden-ratio (Weyl) index sequence over n items.

    Reading: the pages do not say how the sampled queries Q_s [PR 2A] (or the
    k-means seeds) are picked. We use idx_j = (j * a) mod n with
    a = floor(n * GOLDEN_32 / 2^32), bumped up until gcd(a, n) = 1 so that the
    first n indices are a permutation. No random numbers are involved.
    """
    a = (n * GOLDEN_32) >> 32
    while math.gcd(a, n) != 1:
        a += 1
    return a


def weyl_indices(n: int, m: int) -> np.ndarray:
    """First m indices of the Weyl sequence over n items (distinct when m <= n)."""
    a = weyl_multiplier(n)
    j = np.arange(m, dtype=np.int64)
    return (j * a) % n


# --------------------------------------------------------------- partition ---
def key_metric(q: np.ndarray, n_sample: int) -> np.ndarray:
    """M_K = Q_s^T Q_s / M_s over the sampled queries [PR 2A, key-response coordinates]."""
    qs = np.asarray(q, np.float64)[weyl_indices(q.shape[0], n_sample)]
    return qs.T @ qs / n_sample


def key_projection(m_k: np.ndarray, key_rank: int):
    """Leading eigenvectors of M_K, scaled so that distances are metric distances.

    [PR 2A] clusters keys by k-means on the eigenvectors of M_K. Reading: keep the
    r_K largest eigenpairs and use W = U_r diag(sqrt(lambda_r)), so that
    |k1 W - k2 W|^2 = (k1-k2)^T M_r (k1-k2), the response-profile distance
    restricted to the leading directions. Eigenvalues are clamped at 0 (M_K is
    positive semi-definite; tiny negative values are rounding).
    Returns (W [d, r_K], eigenvalues in descending order).
    """
    lam, u = np.linalg.eigh(np.asarray(m_k, np.float64))
    lam = lam[::-1]
    u = u[:, ::-1]
    w = u[:, :key_rank] * np.sqrt(np.maximum(lam[:key_rank], 0.0))[None, :]
    return w, lam


def squared_distances(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """|x_n - c_g|^2 for all n, g (expanded with one matrix product)."""
    x = np.asarray(x, np.float64)
    c = np.asarray(c, np.float64)
    return (np.sum(x * x, axis=1)[:, None] - 2.0 * (x @ c.T)
            + np.sum(c * c, axis=1)[None, :])


def assign(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Nearest centroid of every point; ties go to the lowest centroid index."""
    return np.argmin(squared_distances(x, c), axis=1).astype(np.int32)


def update_centroids(x: np.ndarray, labels: np.ndarray, prev: np.ndarray) -> np.ndarray:
    """Mean of each group's members; an empty group keeps its previous centroid."""
    c = np.array(prev, np.float64, copy=True)
    for g in np.unique(labels):
        c[g] = np.asarray(x, np.float64)[labels == g].mean(axis=0)
    return c


def lloyd(x: np.ndarray, groups: int, iters: int):
    """Lloyd's k-means, deterministic.

    Reading ([PR 2A] names k-means but not its details): seeds are the points at
    the first `groups` Weyl indices; each of the `iters` rounds assigns every
    point to its nearest centroid (lowest index on ties) and then moves each
    non-empty centroid to its members' mean. The labels are the last assignment.
    Returns (labels [N] int32, centroids after the last update [G, D]).
    """
    x = np.asarray(x, np.float64)
    c = x[weyl_indices(x.shape[0], groups)].copy()
    labels = np.zeros(x.shape[0], np.int32)
    for _ in range(iters):
        labels = assign(x, c)
        c = update_centroids(x, labels, c)
    return labels, c


def group_means(x: np.ndarray, labels: np.ndarray, groups: int) -> np.ndarray:
    """Raw-space group means; an empty group gets the zero vector."""
    x = np.asarray(x, np.float64)
    out = np.zeros((groups, x.shape[1]))
    for g in np.unique(labels):
        out[g] = x[labels == g].mean(axis=0)
    return out


def query_profiles(q: np.ndarray, key_centroids: np.ndarray) -> np.ndarray:
    """Pre-softmax logit profile of each query against the K/V group centroids,
    p(q)_g = q . c^K_g / sqrt(d) [PR 2A, query-response coordinates]."""
    d = q.shape[1]
    return np.asarray(q, np.float64) @ np.asarray(key_centroids, np.float64).T / math.sqrt(d)


@dataclass
class Partition:
    key_labels: np.ndarray
    q_labels: np.ndarray
    key_centroids: np.ndarray      # raw d-dim means [G_k, d]
    q_centroids: np.ndarray        # raw d-dim means [G_q, d]
    metric_eigenvalues: np.ndarray


def partition(q: np.ndarray, k: np.ndarray, n_sample: int, key_rank: int,
              kv_groups: int, q_groups: int, iters: int) -> Partition:
    """Response-coupled partition, one asymmetric pass [PR 2A]:
    keys by k-means in M_K eigen-coordinates, then queries by k-means of their
    logit profiles against the raw key-group centroids. Nothing is refined
    afterwards (no alternation)."""
    m_k = key_metric(q, n_sample)
    w, lam = key_projection(m_k, key_rank)
    z = np.asarray(k, np.float64) @ w
    key_labels, _ = lloyd(z, kv_groups, iters)
    ck = group_means(k, key_labels, kv_groups)
    prof = query_profiles(q, ck)
    q_labels, _ = lloyd(prof, q_groups, iters)
    cq = group_means(q, q_labels, q_groups)
    return Partition(key_labels, q_labels, ck, cq, lam)


def raw_partition(q: np.ndarray, k: np.ndarray, kv_groups: int, q_groups: int,
                  iters: int) -> Partition:
    """Comparison partitioner, not the method: keys and queries each clustered by
    plain Euclidean k-means of their raw rows, independently of each other (the
    clustering that [SVOO]'s design-motivation item attributes to cluster-based
    sparse attention such as SVG2, and that [PR 2A]'s response coupling replaces).
    Reading: the same Lloyd (seeds, rounds, ties) as the method's partition, so that
    the two differ only in the space each side is clustered in."""
    key_labels, _ = lloyd(k, kv_groups, iters)
    q_labels, _ = lloyd(q, q_groups, iters)
    ck = group_means(k, key_labels, kv_groups)
    cq = group_means(q, q_labels, q_groups)
    return Partition(key_labels, q_labels, ck, cq, np.zeros(0))


def svoo_partition(q: np.ndarray, k: np.ndarray, kv_groups: int, q_groups: int,
                   iters: int) -> Partition:
    """Comparison partitioner, not the method: the online bidirectional co-clustering of
    [SVOO] (its online co-clustering item). Each round has two steps. Step A takes the
    current query centroids as anchors: every key gets its affinity vector against them
    (p(k)_i = k . c^Q_i / sqrt(d)) and joins the key block whose centre, the mean affinity
    vector of the block's current members under the same anchors, is nearest. The raw key
    centroids are then updated. Step B does the same for the queries against the updated
    key centroids.
    Readings (the item gives neither seeds nor round count, nor what an empty block holds):
    the seeds of both sides are the rows at the first G Weyl indices (as the method's
    Lloyd), `iters` rounds, ties to the lowest index, and an empty block's raw centroid is
    the zero vector (as the method's key centroids for the query profiles). By linearity the
    mean affinity of a block's members is the affinity of their raw mean."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    n = q.shape[0]
    cq = q[weyl_indices(n, q_groups)].copy()
    ck = k[weyl_indices(n, kv_groups)].copy()
    key_labels = np.zeros(n, np.int32)
    q_labels = np.zeros(n, np.int32)
    for _ in range(iters):
        key_labels = assign(query_profiles(k, cq), query_profiles(ck, cq))     # step A
        ck = group_means(k, key_labels, kv_groups)
        q_labels = assign(query_profiles(q, ck), query_profiles(cq, ck))       # step B
        cq = group_means(q, q_labels, q_groups)
    return Partition(key_labels, q_labels, ck, cq, np.zeros(0))


# ------------------------------------------------------------------ layout ---
def group_major(labels: np.ndarray, groups: int):
    """Contiguous group-major layout [PR 2C]: a stable sort of token indices by
    label (ascending original index inside a group).
    Returns (perm with perm[new] = old, offsets [groups + 1])."""
    perm = np.argsort(labels, kind="stable").astype(np.int32)
    counts = np.bincount(labels, minlength=groups)
    off = np.zeros(groups + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return perm, off


# ----------------------------------------------------------------- routing ---
def routed_count(density: float, kv_groups: int) -> int:
    """k = ceil(rho * G_k) key groups per query group ([SVOO] keeps
    ceil((1 - s) K_k) blocks; here 1 - s is the density rho), clamped to [1, G_k].
    The 1e-9 guards products that are integers in exact arithmetic."""
    k = math.ceil(density * kv_groups - 1e-9)
    return int(min(max(k, 1), kv_groups))


def route(q_centroids: np.ndarray, key_centroids: np.ndarray, key_counts: np.ndarray,
          k: int) -> np.ndarray:
    """Centroid-logit top-k block selection [SVOO, block selection].

    S_ij = c^Q_i . c^K_j / sqrt(d) (fp64). Each query group keeps the k key
    groups of largest S_ij among the non-empty key groups (all of them if fewer
    than k are non-empty); equal scores go to the lower index. Returned in
    ascending key-group order, padded with -1 to k columns.
    """
    d = q_centroids.shape[1]
    s = np.asarray(q_centroids, np.float64) @ np.asarray(key_centroids, np.float64).T / math.sqrt(d)
    nonempty = np.nonzero(np.asarray(key_counts) > 0)[0]
    out = np.full((s.shape[0], k), -1, np.int32)
    for i in range(s.shape[0]):
        order = np.lexsort((nonempty, -s[i, nonempty]))
        pick = np.sort(nonempty[order[:k]])
        out[i, :len(pick)] = pick
    return out


def probe_positions(q_counts: np.ndarray, probes: int) -> np.ndarray:
    """Stratified probe rows across query groups [PR 2B, probe selection].

    Reading (allocation and placement are not stated): proportional allocation
    m_i = floor(P n_i / N); the P - sum(m_i) left over go one each to the groups
    with the largest remainders P n_i mod N (lower index first on ties). Inside
    group i the probes are the members at ranks floor((2t + 1) n_i / (2 m_i)),
    t < m_i (centred ranks). Returned as group-major positions, ascending.
    """
    n_i = np.asarray(q_counts, np.int64)
    n = int(n_i.sum())
    if probes == 0:
        return np.zeros(0, np.int32)
    m = (probes * n_i) // n
    rem = (probes * n_i) % n
    left = probes - int(m.sum())
    order = np.lexsort((np.arange(len(n_i)), -rem))
    m[order[:left]] += 1
    off = np.concatenate([[0], np.cumsum(n_i)])
    pos = []
    for i in range(len(n_i)):
        for t in range(int(m[i])):
            pos.append(off[i] + ((2 * t + 1) * n_i[i]) // (2 * m[i]))
    return np.asarray(pos, np.int32)


# --------------------------------------------------------------- attention ---
def softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits - np.max(logits, axis=1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=1, keepdims=True)


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(Q K^T / sqrt(d)) V  [BLOG 1.2]."""
    d = q.shape[1]
    q = np.asarray(q, np.float64)
    out = np.empty((q.shape[0], v.shape[1]))
    step = max(1, (1 << 24) // max(1, k.shape[0]))
    for s0 in range(0, q.shape[0], step):
        p = softmax_rows(q[s0:s0 + step] @ np.asarray(k, np.float64).T / math.sqrt(d))
        out[s0:s0 + step] = p @ np.asarray(v, np.float64)
    return out


def routed_keys(key_off: np.ndarray, blocks_row: np.ndarray) -> np.ndarray:
    """Group-major key positions of the union U_i of the routed key groups."""
    parts = [np.arange(key_off[j], key_off[j + 1]) for j in blocks_row if j >= 0]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def sparse_attention(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, q_off: np.ndarray,
                     key_off: np.ndarray, blocks: np.ndarray,
                     rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Variable-block-sparse attention in group-major order [PR 2C; SVOO block
    selection; BAIDU masked score]: row q of query group i attends only to the
    keys of its routed groups U_i, and the softmax is normalised over U_i alone
    (every other logit is -inf). With `rows` given, only those group-major rows
    are computed (returned in the order given)."""
    d = qp.shape[1]
    n_q = qp.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    group_of = np.searchsorted(q_off, rows, side="right") - 1
    out = np.empty((len(rows), vp.shape[1]))
    for i in np.unique(group_of):
        sel = np.nonzero(group_of == i)[0]
        u = routed_keys(key_off, blocks[i])
        logits = np.asarray(qp[rows[sel]], np.float64) @ np.asarray(kp[u], np.float64).T / math.sqrt(d)
        out[sel] = softmax_rows(logits) @ np.asarray(vp[u], np.float64)
    return out


# ------------------------------------------------- fp8 logits (an experiment) ---
# Not the method: [BLOG] section 8.4 names quantization as an extension to combine with the
# sparse attention. The experiment computes the sparse logits Q K^T from Q and K rounded to
# the OCP FP8 E4M3 format after a per-head power-of-two scale; everything else is unchanged.

def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest FP8 E4M3 value (OCP 8-bit floating point: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; below 2^-6 the subnormals share the spacing 2^-9; the largest
    finite magnitude is 448 and there is no infinity), ties to the even mantissa. Larger
    magnitudes (which the per-head scale never produces) saturate to 448."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                        # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.float64) - 1.0, -6.0)   # binade [2^e, 2^(e+1)), floored at 2^-6
    ulp = np.exp2(e - 3.0)                     # three mantissa bits
    r = np.round(a / ulp) * ulp                # a / ulp is the integer significand; ties to even
    return np.copysign(np.minimum(r, 448.0), x)


def f8_scale_exp(absmax: float) -> int:
    """The per-head scale exponent: the largest e with absmax 2^e <= 448 (the largest E4M3
    magnitude), kept within [-120, 120]; 0 for an all-zero tensor."""
    if not absmax > 0.0:
        return 0
    f, ex = math.frexp(float(absmax))           # absmax = (2 f) 2^(ex - 1), 2 f in [1, 2)
    e = 8 - (ex - 1) if 2.0 * f <= 1.75 else 7 - (ex - 1)   # 448 = 1.75 * 2^8
    return max(-120, min(120, e))


def fp8_dequantized(x: np.ndarray, e: int) -> np.ndarray:
    """x scaled by 2^e, rounded to E4M3, scaled back: the values the fp8 products see."""
    return e4m3_round(np.asarray(x, np.float64) * 2.0 ** e) * 2.0 ** (-e)


# ------------------------------------------------------ probe-fitted residual ---
def ridge_affine(x: np.ndarray, y: np.ndarray, lam: float):
    """Ridge-regularised affine fit y ~ b + x B [PR 2B, affine calibration].

    Reading: the intercept is not penalised (columns are centred first) and
    lambda is used as given (not scaled by P):
      B = (Xc^T Xc + lambda I)^-1 Xc^T Yc,  b = mean(y) - mean(x) B.
    lambda = 0 means the minimum-norm least-squares solution.
    """
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    xm = x.mean(axis=0)
    ym = y.mean(axis=0)
    xc = x - xm
    yc = y - ym
    if lam > 0:
        b_mat = np.linalg.solve(xc.T @ xc + lam * np.eye(x.shape[1]), xc.T @ yc)
    else:
        b_mat = np.linalg.pinv(xc) @ yc
    return b_mat, ym - xm @ b_mat


def residual_projector(y: np.ndarray, rank: int):
    """Projector onto the leading right singular vectors of the probe residuals
    [PR 2B, subspace restriction].

    Reading: the SVD is of the uncentred residual matrix (so the intercept lies
    in the subspace); the kept rank is min(r, #{sigma_i > sigma_1 max(P, d) 2^-52}).
    Returns (Pi [d, d], singular values).
    """
    y = np.asarray(y, np.float64)
    d = y.shape[1]
    if y.shape[0] == 0:
        return np.zeros((d, d)), np.zeros(0)
    _, s, vt = np.linalg.svd(y, full_matrices=False)
    thr = s[0] * max(y.shape) * 2.0 ** -52
    r_eff = min(rank, int(np.sum(s > thr))) if s[0] > 0 else 0
    v = vt[:r_eff].T
    return v @ v.T, s


def probe_fit(x: np.ndarray, y: np.ndarray, lam: float, rank: int):
    """Fitted map restricted to the residual subspace: B' = B Pi, b' = b Pi.
    With no probes there is nothing to fit and the map is zero."""
    d = np.shape(x)[1]
    if np.shape(x)[0] == 0:
        return np.zeros((d, d)), np.zeros(d)
    b_mat, b_vec = ridge_affine(x, y, lam)
    pi, _ = residual_projector(y, rank)
    return b_mat @ pi, b_vec @ pi


def correct(o_sparse: np.ndarray, probe_pos: np.ndarray, o_dense_probe: np.ndarray,
            b_mat: np.ndarray, b_vec: np.ndarray) -> np.ndarray:
    """Add the fitted residual to the unprobed rows [PR 2B, correction]:
    O = O_s + b' + O_s B'. Reading: probe rows output their exact dense value."""
    o = np.asarray(o_sparse, np.float64)
    out = o + b_vec[None, :] + o @ b_mat
    if len(probe_pos):
        out[probe_pos] = o_dense_probe
    return out


# --------------------------------------------------------------- full call ---
@dataclass
class HeadResult:
    key_labels: np.ndarray
    q_labels: np.ndarray
    key_perm: np.ndarray
    q_perm: np.ndarray
    key_off: np.ndarray
    q_off: np.ndarray
    blocks: np.ndarray
    probe_pos: np.ndarray          # group-major positions
    probe_orig: np.ndarray         # original token indices
    o_sparse: np.ndarray           # [N, d], group-major
    x: np.ndarray                  # O_s at the probes
    y: np.ndarray                  # O_dense - O_s at the probes
    b_mat: np.ndarray              # B' = B Pi
    b_vec: np.ndarray              # b' = b Pi
    o: np.ndarray                  # [N, d], original order
    extra: Dict[str, object] = field(default_factory=dict)


def oracle_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, n_sample: int, key_rank: int,
                kv_groups: int, q_groups: int, kmeans_iters: int, density: float, probes: int,
                ridge_lambda: float, corr_rank: int,
                part: Optional[Partition] = None, raw_kmeans: bool = False,
                svoo: bool = False, reuse: Optional["HeadResult"] = None,
                fp8_qk: bool = False) -> HeadResult:
    """One head of one SparsePR call, stage by stage:
    partition -> group-major layout -> routing + probes -> sparse attention and
    exact probe rows -> probe fit -> correction -> original order.
    `part` injects a partition (labels) instead of computing it; `raw_kmeans` and `svoo`
    use a comparison partitioner (raw_partition, svoo_partition) instead of the method's.
    `reuse` (an experiment, not the method: [PR 2B] uses no temporal reuse, [BLOG]'s
    mask_update_stride refreshes the mask only every few steps) keeps an earlier call's
    labels, block lists and probe rows for these new inputs; everything after the routing
    is computed from the new q, k, v.
    `fp8_qk` (an experiment, see e4m3_round) takes the sparse attention's logits from Q and K
    rounded to FP8 E4M3 after their per-head power-of-two scales (the largest magnitude of
    each tensor over the head sets the scale); the probe rows, their fit and the dense rows
    stay in the inputs' precision, and the correction is applied to that sparse output."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if reuse is not None:
        part = Partition(reuse.key_labels, reuse.q_labels, None, None, np.zeros(0))
    if part is None and raw_kmeans:
        part = raw_partition(q, k, kv_groups, q_groups, kmeans_iters)
    elif part is None and svoo:
        part = svoo_partition(q, k, kv_groups, q_groups, kmeans_iters)
    elif part is None:
        part = partition(q, k, n_sample, key_rank, kv_groups, q_groups, kmeans_iters)
    ck = group_means(k, part.key_labels, kv_groups)
    cq = group_means(q, part.q_labels, q_groups)
    kperm, koff = group_major(part.key_labels, kv_groups)
    qperm, qoff = group_major(part.q_labels, q_groups)
    kk = routed_count(density, kv_groups)
    if reuse is not None:
        blocks, ppos = reuse.blocks, reuse.probe_pos
    else:
        blocks = route(cq, ck, np.diff(koff), kk)
        ppos = probe_positions(np.diff(qoff), probes)
    qp, kp, vp = q[qperm], k[kperm], v[kperm]
    o_s = sparse_attention(qp, kp, vp, qoff, koff, blocks)
    o_d = dense_attention(qp[ppos], kp, vp) if len(ppos) else np.zeros((0, v.shape[1]))
    x = o_s[ppos]
    y = o_d - x
    b_mat, b_vec = probe_fit(x, y, ridge_lambda, corr_rank)
    if fp8_qk:
        eq = f8_scale_exp(float(np.max(np.abs(q))) if q.size else 0.0)
        ek = f8_scale_exp(float(np.max(np.abs(k))) if k.size else 0.0)
        o_s = sparse_attention(fp8_dequantized(qp, eq), fp8_dequantized(kp, ek), vp, qoff, koff, blocks)
    o_perm = correct(o_s, ppos, o_d, b_mat, b_vec)
    o = np.empty_like(o_perm)
    o[qperm] = o_perm
    return HeadResult(part.key_labels, part.q_labels, kperm, qperm, koff, qoff, blocks, ppos,
                      qperm[ppos], o_s, x, y, b_mat, b_vec, o,
                      extra={"metric_eigenvalues": part.metric_eigenvalues})


def oracle_call(q: np.ndarray, k: np.ndarray, v: np.ndarray, settings,
                heads: Optional[Sequence[int]] = None, raw_kmeans: bool = False,
                svoo: bool = False, fp8_qk: bool = False) -> List[HeadResult]:
    """All heads of one call; `settings` carries the SparsePR parameters by name."""
    kw = dict(n_sample=settings.n_sample, key_rank=settings.key_rank,
              kv_groups=settings.kv_groups, q_groups=settings.q_groups,
              kmeans_iters=settings.kmeans_iters, density=settings.density,
              probes=settings.probes, ridge_lambda=settings.ridge_lambda,
              corr_rank=settings.corr_rank, raw_kmeans=raw_kmeans, svoo=svoo, fp8_qk=fp8_qk)
    hs = range(q.shape[0]) if heads is None else heads
    return [oracle_head(q[h], k[h], v[h], **kw) for h in hs]
