"""Pins of the fp64 oracle against things other than itself: pure-Python brute
force on tiny inputs, closed forms, second formulations and invariants.
All CPU, no GPU."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from oracle import brute
from synthetic import bf16_round, get_config, make_inputs, token_grid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _tolist(a):
    return np.asarray(a, np.float64).tolist()


# ----------------------------------------------------------- inputs / grid ---
def test_token_grid_matches_page_example():
    g = json.load(open(os.path.join(GOLDEN, "token_grid.json")))
    t, y, x = token_grid(g["frames"], g["patch_rows"], g["patch_cols"])
    assert len(t) == g["tokens"]
    assert int(np.sum(t == 0)) == g["tokens_per_frame"]
    n = (t * g["patch_rows"] + y) * g["patch_cols"] + x
    assert np.array_equal(n, np.arange(g["tokens"]))


def test_generator_is_deterministic_and_bf16():
    cfg = get_config("C1")
    q1, k1, v1 = make_inputs(cfg)
    q2, k2, v2 = make_inputs(cfg)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(bf16_round(q1), q1)
    logits = q1[0] @ k1[0].T / math.sqrt(cfg.d)
    assert 2.0 < logits.std() < 4.0


# ------------------------------------------------------------------- Weyl ---
@pytest.mark.parametrize("n", [1, 2, 7, 64, 2048, 32760, 75600, 118800])
def test_weyl_sequence_is_a_permutation(n):
    a = orc.weyl_multiplier(n)
    assert math.gcd(a, n) == 1
    idx = orc.weyl_indices(n, n)
    assert np.array_equal(np.sort(idx), np.arange(n))


@pytest.mark.parametrize("n", [2048, 32760, 75600, 118800])
def test_weyl_multiplier_is_golden_fraction(n):
    # independent arithmetic: floor(n / phi) in 50-digit decimals, then the
    # smallest value >= it that is coprime to n
    getcontext().prec = 50
    phi = (1 + Decimal(5).sqrt()) / 2
    a = int((Decimal(n) / phi).to_integral_value(rounding="ROUND_FLOOR"))
    while math.gcd(a, n) != 1:
        a += 1
    assert orc.weyl_multiplier(n) == a


# ------------------------------------------------------------- key metric ---
def test_key_metric_is_sample_second_moment():
    q = _rand((50, 6), 1)
    m = orc.key_metric(q, 10)
    idx = orc.weyl_indices(50, 10)
    for i in range(6):
        for j in range(6):
            ref = sum(q[s, i] * q[s, j] for s in idx) / 10
            assert abs(m[i, j] - ref) < 1e-13
    assert np.allclose(m, m.T)
    assert np.min(np.linalg.eigvalsh(m)) > -1e-12
    assert abs(np.trace(m) - np.mean(np.sum(q[idx] ** 2, axis=1))) < 1e-12


def test_key_projection_full_rank_equals_response_profiles():
    """With r_K = d, k-means on Z = K W must give the labels of k-means on the
    raw response profiles Q_s k / sqrt(M_s) (a second formulation of the metric)."""
    rng = np.random.default_rng(3)
    d, n, ms = 8, 300, 40
    centres = rng.standard_normal((6, d)) * 3
    k = centres[rng.integers(6, size=n)] + rng.standard_normal((n, d))
    q = rng.standard_normal((n, d))
    w, lam = orc.key_projection(orc.key_metric(q, ms), d)
    lab_z, _ = orc.lloyd(k @ w, 6, 5)
    qs = q[orc.weyl_indices(n, ms)]
    prof = k @ qs.T / math.sqrt(ms)
    lab_p, _ = orc.lloyd(prof, 6, 5)
    assert np.array_equal(lab_z, lab_p)
    assert np.all(np.diff(lam) <= 0)


def test_key_projection_distances_are_truncated_metric():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((100, 10))
    m = orc.key_metric(q, 30)
    w, _ = orc.key_projection(m, 4)
    lam, u = np.linalg.eigh(m)
    mr = u[:, -4:] @ np.diag(lam[-4:]) @ u[:, -4:].T
    a, b = rng.standard_normal(10), rng.standard_normal(10)
    assert abs(np.sum(((a - b) @ w) ** 2) - (a - b) @ mr @ (a - b)) < 1e-10


def test_partition_labels_invariant_to_power_of_two_scaling():
    cfg = get_config("C1")
    q, k, _ = make_inputs(cfg)
    st = cfg.settings
    args = (st.n_sample, st.key_rank, st.kv_groups, st.q_groups, st.kmeans_iters)
    p1 = orc.partition(q[0], k[0], *args)
    p2 = orc.partition(2 * q[0], 2 * k[0], *args)
    assert np.array_equal(p1.key_labels, p2.key_labels)
    assert np.array_equal(p1.q_labels, p2.q_labels)


# ----------------------------------------------------------------- k-means ---
@pytest.mark.parametrize("seed", range(6))
def test_lloyd_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n, dim, g = int(rng.integers(8, 64)), int(rng.integers(1, 5)), int(rng.integers(1, 8))
    x = rng.standard_normal((n, dim)).round(1)          # coarse values: many exact ties
    if seed % 2:
        x[n // 2:] = x[: n - n // 2]                    # duplicated points
    lab, _ = orc.lloyd(x, g, 4)
    ref = brute.lloyd(_tolist(x), orc.weyl_indices(n, g).tolist(), 4)
    assert lab.tolist() == ref


def test_lloyd_degenerate_group_counts():
    x = _rand((40, 3), 7)
    lab, _ = orc.lloyd(x, 1, 5)
    assert np.all(lab == 0)
    lab, _ = orc.lloyd(x, 40, 5)                        # every point seeds itself
    seeds = orc.weyl_indices(40, 40)
    expect = np.empty(40, np.int64)
    expect[seeds] = np.arange(40)
    assert np.array_equal(lab, expect)


def test_lloyd_all_equal_points_go_to_group_zero():
    lab, _ = orc.lloyd(np.ones((30, 4)), 5, 5)
    assert np.all(lab == 0)


@pytest.mark.parametrize("seed", range(3))
def test_raw_partition_is_brute_force_lloyd_of_each_side(seed):
    """The comparison partitioner clusters raw keys and raw queries independently."""
    rng = np.random.default_rng(300 + seed)
    n, dim = int(rng.integers(10, 40)), int(rng.integers(2, 5))
    q = rng.standard_normal((n, dim)).round(1)
    k = rng.standard_normal((n, dim)).round(1)
    gk, gq = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    part = orc.raw_partition(q, k, gk, gq, 3)
    assert part.key_labels.tolist() == brute.lloyd(_tolist(k), orc.weyl_indices(n, gk).tolist(), 3)
    assert part.q_labels.tolist() == brute.lloyd(_tolist(q), orc.weyl_indices(n, gq).tolist(), 3)
    assert np.allclose(part.key_centroids, orc.group_means(k, part.key_labels, gk))


def test_raw_partition_recovers_planted_blobs():
    """Well-separated blobs whose seed points (the first Weyl indices) lie in distinct
    blobs come back exactly as the groups, labelled in seed order."""
    rng = np.random.default_rng(9)
    n, g, dim = 300, 6, 8
    centers = rng.standard_normal((g, dim)) * 50
    blob = rng.integers(0, g, n)
    seeds = orc.weyl_indices(n, g)
    blob[seeds] = np.arange(g)
    k = centers[blob] + rng.standard_normal((n, dim))
    q = centers[(blob + 1) % g] + rng.standard_normal((n, dim))
    part = orc.raw_partition(q, k, g, g, 5)
    assert np.array_equal(part.key_labels, blob)
    # the query seed at index seeds[j] sits in blob (j + 1) % g, so label j is that blob
    expect_q = np.empty(g, np.int64)
    expect_q[(np.arange(g) + 1) % g] = np.arange(g)
    assert np.array_equal(part.q_labels, expect_q[(blob + 1) % g])


def test_query_profile_kmeans_equals_cholesky_coordinates():
    """Profile-space distances equal |(q - c) L|^2 with L L^T = C_K^T C_K / d, so
    k-means in either space must give identical labels."""
    rng = np.random.default_rng(5)
    d, n, gk = 6, 400, 12
    ck = rng.standard_normal((gk, d))
    q = rng.standard_normal((n, d)) * 2
    lab_p, _ = orc.lloyd(orc.query_profiles(q, ck), 9, 5)
    low = np.linalg.cholesky(ck.T @ ck / d)
    lab_c, _ = orc.lloyd(q @ low, 9, 5)
    assert np.array_equal(lab_p, lab_c)


def test_query_centroid_profile_is_profile_mean():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((50, 5))
    ck = rng.standard_normal((7, 5))
    lab = rng.integers(4, size=50)
    cq = orc.group_means(q, lab, 4)
    prof = orc.query_profiles(q, ck)
    for g in range(4):
        assert np.allclose(orc.query_profiles(cq[g:g + 1], ck)[0], prof[lab == g].mean(0))


# ------------------------------------------------------------------ layout ---
def test_group_major_is_stable_permutation_and_round_trips():
    rng = np.random.default_rng(8)
    lab = rng.integers(0, 9, size=500).astype(np.int32)
    lab[lab == 4] = 5                                   # an empty group
    perm, off = orc.group_major(lab, 9)
    assert np.array_equal(np.sort(perm), np.arange(500))
    assert off[0] == 0 and off[-1] == 500 and np.all(np.diff(off) >= 0)
    assert off[5] == off[4]
    for g in range(9):
        seg = perm[off[g]:off[g + 1]]
        assert np.all(lab[seg] == g) and np.all(np.diff(seg) > 0)
    # permute: row i of the group-major copy is token perm[i]; unpermute with an inverse
    # built by an explicit loop (inv[perm[i]] = i), independent of numpy fancy assignment
    x = rng.standard_normal((500, 3))
    xp = x[perm]
    inv = [0] * 500
    for i, old in enumerate(perm.tolist()):
        inv[old] = i
    assert sorted(inv) == list(range(500))
    back = np.array([xp[inv[t]] for t in range(500)])
    assert np.array_equal(back, x)
    for i in (0, 17, 499):                              # the layout definition, row by row
        assert np.array_equal(xp[i], x[perm[i]]) and lab[perm[i]] == np.searchsorted(off, i, "right") - 1


# ----------------------------------------------------------------- routing ---
def test_routed_count_rule():
    assert orc.routed_count(0.25, 16) == 4
    assert orc.routed_count(0.26, 256) == 67
    assert orc.routed_count(0.22, 256) == 57
    assert orc.routed_count(0.15, 256) == 39
    assert orc.routed_count(0.35, 256) == 90
    assert orc.routed_count(0.24, 384) == 93
    assert orc.routed_count(1.0, 256) == 256
    assert orc.routed_count(1e-6, 256) == 1


def test_route_matches_sorted_tuples():
    rng = np.random.default_rng(9)
    cq = rng.standard_normal((11, 4)).round(0)           # integer centroids: many ties
    ck = rng.standard_normal((13, 4)).round(0)
    counts = rng.integers(0, 3, size=13)
    k = 5
    blocks = orc.route(cq, ck, counts, k)
    for i in range(11):
        cand = [(-float(np.dot(cq[i], ck[j])), j) for j in range(13) if counts[j] > 0]
        pick = sorted(j for _, j in sorted(cand)[:k])
        assert blocks[i].tolist() == pick + [-1] * (k - len(pick))


def test_route_density_one_and_argmax():
    rng = np.random.default_rng(10)
    cq, ck = rng.standard_normal((6, 3)), rng.standard_normal((8, 3))
    counts = np.array([3, 0, 1, 2, 5, 0, 1, 1])
    full = orc.route(cq, ck, counts, 8)
    for row in full:
        assert row.tolist() == [0, 2, 3, 4, 6, 7, -1, -1]
    one = orc.route(cq, ck, counts, 1)
    s = cq @ ck.T
    s[:, counts == 0] = -np.inf
    assert np.array_equal(one[:, 0], np.argmax(s, axis=1))


# ------------------------------------------------------------------ probes ---
def _hamilton(counts, probes):
    n = sum(counts)
    quota = [Fraction(probes * c, n) for c in counts]
    m = [int(math.floor(x)) for x in quota]
    left = probes - sum(m)
    order = sorted(range(len(counts)), key=lambda i: (-(quota[i] - m[i]), i))
    for i in order[:left]:
        m[i] += 1
    return m


@pytest.mark.parametrize("seed", range(5))
def test_probe_allocation_is_largest_remainder(seed):
    rng = np.random.default_rng(200 + seed)
    counts = rng.integers(0, 40, size=int(rng.integers(1, 20)))
    counts[0] += 1
    n = int(counts.sum())
    for p in {0, 1, n // 3, n - 1, n}:
        pos = orc.probe_positions(counts, p)
        assert len(pos) == p and len(set(pos.tolist())) == p
        off = np.concatenate([[0], np.cumsum(counts)])
        got = [int(np.sum((pos >= off[i]) & (pos < off[i + 1]))) for i in range(len(counts))]
        assert got == _hamilton(counts.tolist(), p)
        if p == n:
            assert np.array_equal(pos, np.arange(n))


def test_probe_ranks_are_centred():
    pos = orc.probe_positions(np.array([10, 20]), 3)    # m = (1, 2)
    assert pos.tolist() == [5, 10 + 5, 10 + 15]


# --------------------------------------------------------------- attention ---
def test_dense_matches_brute_force():
    q, k, v = _rand((9, 5), 11), _rand((13, 5), 12), _rand((13, 3), 13)
    ref = brute.attention(_tolist(q), _tolist(k), _tolist(v))
    assert np.allclose(orc.dense_attention(q, k, v), ref, atol=1e-13)


def test_dense_closed_forms():
    q, v = _rand((7, 4), 14), _rand((10, 3), 15)
    k = np.tile(_rand((1, 4), 16), (10, 1))             # identical keys: uniform weights
    assert np.allclose(orc.dense_attention(q, k, v), np.tile(v.mean(0), (7, 1)), atol=1e-13)
    vc = np.tile(_rand((1, 3), 17), (10, 1))            # constant values
    assert np.allclose(orc.dense_attention(q, _rand((10, 4), 18), vc), vc[:7], atol=1e-13)


def test_sparse_matches_brute_force_masked_softmax():
    rng = np.random.default_rng(19)
    n, d = 40, 4
    qlab = rng.integers(0, 4, size=n)
    klab = rng.integers(0, 5, size=n)
    qlab[:4] = np.arange(4)
    klab[:5] = np.arange(5)
    q, k, v = _rand((n, d), 20), _rand((n, d), 21), _rand((n, 3), 22)
    qperm, qoff = orc.group_major(qlab, 4)
    kperm, koff = orc.group_major(klab, 5)
    blocks = np.array([[0, 2], [1, -1], [3, 4], [0, 4]])
    o = orc.sparse_attention(q[qperm], k[kperm], v[kperm], qoff, koff, blocks)
    allowed = [[int(klab[kperm[j]]) in blocks[int(qlab[qperm[i]])].tolist() for j in range(n)]
               for i in range(n)]
    ref = brute.attention(_tolist(q[qperm]), _tolist(k[kperm]), _tolist(v[kperm]), allowed)
    assert np.allclose(o, ref, atol=1e-13)
    sub = orc.sparse_attention(q[qperm], k[kperm], v[kperm], qoff, koff, blocks,
                               rows=np.array([7, 3, 30]))
    assert np.allclose(sub, o[[7, 3, 30]], atol=1e-14)


def test_sparse_with_all_groups_is_dense_and_key_order_free():
    rng = np.random.default_rng(23)
    n = 50
    lab = rng.integers(0, 6, size=n)
    lab[:6] = np.arange(6)
    q, k, v = _rand((n, 4), 24), _rand((n, 4), 25), _rand((n, 2), 26)
    perm, off = orc.group_major(lab, 6)
    blocks = np.tile(np.arange(6), (6, 1))
    o = orc.sparse_attention(q[perm], k[perm], v[perm], off, off, blocks)
    assert np.allclose(o, orc.dense_attention(q[perm], k, v), atol=1e-13)
    o_rev = orc.sparse_attention(q[perm], k[perm], v[perm], off, off, blocks[:, ::-1].copy())
    assert np.allclose(o, o_rev, atol=1e-14)


# -------------------------------------------------------------------- fit ---
def test_ridge_matches_brute_normal_equations():
    x, y = _rand((12, 3), 27), _rand((12, 2), 28)
    b_mat, b_vec = orc.ridge_affine(x, y, 0.3)
    rb_mat, rb_vec = brute.ridge_affine(_tolist(x), _tolist(y), 0.3)
    assert np.allclose(b_mat, rb_mat, atol=1e-12) and np.allclose(b_vec, rb_vec, atol=1e-12)


def test_ridge_recovers_exact_affine_map():
    x = _rand((40, 5), 29)
    b_true, c_true = _rand((5, 5), 30), _rand((5,), 31)
    y = c_true + x @ b_true
    for lam in (0.0, 1e-12):
        b_mat, b_vec = orc.ridge_affine(x, y, lam)
        assert np.allclose(b_mat, b_true, atol=1e-8) and np.allclose(b_vec, c_true, atol=1e-8)


def test_ridge_limits():
    x, y = _rand((20, 4), 32), _rand((20, 4), 33)
    b_mat, b_vec = orc.ridge_affine(x, y, 1e14)
    assert np.abs(b_mat).max() < 1e-10 and np.allclose(b_vec, y.mean(0), atol=1e-9)
    b_mat, b_vec = orc.ridge_affine(x[:1], y[:1], 1e-3)
    assert np.all(b_mat == 0) and np.allclose(b_vec, y[0])


def test_projector_closed_forms():
    rng = np.random.default_rng(34)
    y = rng.standard_normal((30, 3)) @ rng.standard_normal((3, 8))        # rank 3
    pi, _ = orc.residual_projector(y, 5)
    assert np.allclose(pi @ y.T, y.T, atol=1e-10)
    assert abs(np.trace(pi) - 3) < 1e-9
    assert np.allclose(pi, pi.T) and np.allclose(pi @ pi, pi, atol=1e-12)
    full = rng.standard_normal((30, 8))
    assert np.allclose(orc.residual_projector(full, 8)[0], np.eye(8), atol=1e-12)
    assert np.all(orc.residual_projector(np.zeros((30, 8)), 4)[0] == 0)
    pi2, s = orc.residual_projector(full, 2)
    _, _, vt = np.linalg.svd(full)
    top = vt[:2].T
    assert np.allclose(pi2, top @ top.T, atol=1e-12)
    assert np.allclose(pi2 @ (full.T @ full) @ top, full.T @ full @ top, atol=1e-9)


def test_projector_on_right_singular_space():
    """Pi acts on the output (column) side: it fixes the rows of Y, not its columns."""
    rng = np.random.default_rng(35)
    y = rng.standard_normal((6, 2)) @ rng.standard_normal((2, 9))        # P < d
    pi, _ = orc.residual_projector(y, 2)
    assert pi.shape == (9, 9)
    assert np.allclose(y @ pi, y, atol=1e-12)


def test_probe_fit_single_probe():
    x, y = _rand((1, 4), 36), _rand((1, 4), 37)
    b_mat, b_vec = orc.probe_fit(x, y, 1e-3, 2)
    assert np.all(b_mat == 0) and np.allclose(b_vec, y[0], atol=1e-14)



# ------------------------------------------------------ fit composition pins ---
def _planted_residual(seed, p=60, d=10, r=3):
    """Y = b* + X B* with B* = B0 V V^T and b* in span(V): a residual that is exactly
    affine in X and lies in the r-dimensional subspace span(V)."""
    rng = np.random.default_rng(seed)
    v, _ = np.linalg.qr(rng.standard_normal((d, r)))
    b_star = rng.standard_normal((d, d)) @ v @ v.T
    b_vec = rng.standard_normal(r) @ v.T
    x = rng.standard_normal((p, d))
    return x, b_vec + x @ b_star, b_star, b_vec, v


def test_probe_fit_recovers_planted_residual_map():
    """[PR 2B] With Y = b* + X B*, B* = B0 V V^T, b* in span(V), lambda -> 0 and rank
    r = rank(V), the residual subspace is span(V) and the fit must return (B*, b*).
    A projector applied on the wrong side (Pi B) or a transposed map fails here."""
    x, y, b_star, b_vec, v = _planted_residual(40)
    for lam in (0.0, 1e-13):
        bm, bv = orc.probe_fit(x, y, lam, 3)
        assert np.allclose(bm, b_star, atol=1e-9) and np.allclose(bv, b_vec, atol=1e-9)
    pi = v @ v.T                                   # the wrong compositions differ here
    assert np.abs(pi @ b_star - b_star).max() > 0.1
    assert np.abs(b_star.T - b_star).max() > 0.1


def test_probe_fit_map_lies_in_the_residual_subspace():
    """[PR 2B, subspace restriction] B' and b' have no component outside the leading
    right singular subspace of the residuals. That subspace is found here by orthogonal
    iteration on Y^T Y, not by the SVD the oracle uses; a dropped projector fails."""
    rng = np.random.default_rng(42)
    p, d, r = 50, 8, 2
    x = rng.standard_normal((p, d))
    y = (rng.standard_normal((p, r)) * [5.0, 3.0]) @ np.linalg.qr(rng.standard_normal((d, r)))[0].T
    y += 0.1 * rng.standard_normal((p, d))
    bm, bv = orc.probe_fit(x, y, 1e-3, r)
    g = y.T @ y
    basis = np.linalg.qr(rng.standard_normal((d, r)))[0]
    for _ in range(400):
        basis = np.linalg.qr(g @ basis)[0]
    pi = basis @ basis.T
    assert np.abs(bm - bm @ pi).max() < 1e-9 and np.abs(bv - bv @ pi).max() < 1e-9
    b_raw, v_raw = orc.ridge_affine(x, y, 1e-3)    # without the projection: outside it
    assert np.abs(b_raw - b_raw @ pi).max() > 1e-3


def test_correct_applies_the_map_on_the_right_row_by_row():
    """[PR 2B, correction] An unprobed row gets O_s[q] + b' + O_s[q] B' (the row vector
    times B', as in R ~ b + x B); a probe row gets its exact dense value. Explicit loops."""
    rng = np.random.default_rng(41)
    n, d = 9, 4
    o = rng.standard_normal((n, d))
    bm, bv = rng.standard_normal((d, d)), rng.standard_normal(d)
    probes, od = [2, 7], rng.standard_normal((2, d))
    out = orc.correct(o, np.array(probes), od, bm, bv)
    for i in range(n):
        for c in range(d):
            if i in probes:
                ref = od[probes.index(i)][c]
            else:
                ref = o[i][c] + bv[c] + sum(o[i][j] * bm[j][c] for j in range(d))
            assert abs(out[i][c] - ref) < 1e-12


def test_call_residuals_are_dense_minus_sparse_at_the_probes():
    """[PR 2B] The fit's inputs: X is the routed (sparse) output at the probe rows and
    Y = O_dense - X there, with O_dense the plain dense attention of those queries over all
    keys in token order (independent of the group-major layout)."""
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    st = cfg.settings
    r = orc.oracle_head(q[0], k[0], v[0], n_sample=st.n_sample, key_rank=st.key_rank,
                        kv_groups=st.kv_groups, q_groups=st.q_groups,
                        kmeans_iters=st.kmeans_iters, density=st.density, probes=st.probes,
                        ridge_lambda=st.ridge_lambda, corr_rank=st.corr_rank)
    dense = orc.dense_attention(q[0][r.probe_orig], k[0], v[0])
    assert np.allclose(r.x + r.y, dense, atol=1e-12)
    assert np.array_equal(r.x, r.o_sparse[r.probe_pos])
    assert np.array_equal(r.q_perm[r.probe_pos], r.probe_orig)


# ------------------------------------------------- partition composition pin ---
def _brute_partition(q, k, ms, rk, gk, gq, iters):
    """[PR 2A] recomputed with loops: M_K from the Weyl sample, W from numpy's eigh (a library
    step), pure-Python Lloyd on K W, raw key-group means, logit profiles against those raw
    means, pure-Python Lloyd on the profiles."""
    n, d = len(q), len(q[0])
    idx = orc.weyl_indices(n, ms).tolist()
    m = [[sum(q[s][i] * q[s][j] for s in idx) / ms for j in range(d)] for i in range(d)]
    lam, u = np.linalg.eigh(np.array(m))
    order = np.argsort(-lam, kind="stable")[:rk]
    w = [[u[c][e] * math.sqrt(max(lam[e], 0.0)) for e in order] for c in range(d)]
    z = [[sum(k[t][c] * w[c][j] for c in range(d)) for j in range(rk)] for t in range(n)]
    klab = brute.lloyd(z, orc.weyl_indices(n, gk).tolist(), iters)
    ck = []
    for g in range(gk):
        mem = [k[t] for t in range(n) if klab[t] == g]
        ck.append([sum(r[c] for r in mem) / len(mem) for c in range(d)] if mem else [0.0] * d)
    prof = [[sum(q[t][c] * ck[g][c] for c in range(d)) / math.sqrt(d) for g in range(gk)]
            for t in range(n)]
    qlab = brute.lloyd(prof, orc.weyl_indices(n, gq).tolist(), iters)
    return klab, qlab, z, w


@pytest.mark.parametrize("seed", range(3))
def test_partition_is_the_brute_force_composition(seed):
    rng = np.random.default_rng(500 + seed)
    n, d, ms, rk, gk, gq = 48, 6, 12, 2, 5, 4
    q = rng.standard_normal((n, d)).round(2)                       # diffuse queries
    k = (rng.standard_normal((6, d))[rng.integers(0, 6, size=n)] * 2
         + 0.5 * rng.standard_normal((n, d))).round(2)               # clustered keys
    part = orc.partition(q, k, ms, rk, gk, gq, 3)
    klab, qlab, z, w = _brute_partition(_tolist(q), _tolist(k), ms, rk, gk, gq, 3)
    assert part.key_labels.tolist() == klab
    assert part.q_labels.tolist() == qlab
    # profiles of the projected queries against the projected key centroids, instead of the
    # raw ones, give other query labels on these inputs (the pin separates the two)
    zc = np.array([np.mean(np.array(z)[np.array(klab) == g], axis=0) for g in range(gk)])
    wrong = (q @ np.array(w)) @ zc.T / math.sqrt(d)
    lab_wrong = brute.lloyd(_tolist(wrong), orc.weyl_indices(n, gq).tolist(), 3)
    assert lab_wrong != qlab

def _brute_svoo(q, k, gk, gq, iters):
    """[SVOO] online co-clustering recomputed with loops, in the pages' terms: affinity
    vectors against the other side's centroids, each block centre the mean affinity vector of
    its current members (before the first round, the seed row alone), nearest centre with the
    lowest index on ties; keys first, then queries against the updated key centroids."""
    n, d = len(q), len(q[0])
    rd = math.sqrt(d)

    def aff(x, anchors):
        return [sum(x[c] * a[c] for c in range(d)) / rd for a in anchors]

    def mean(rows):
        return [sum(r[c] for r in rows) / len(rows) for c in range(d)] if rows else [0.0] * d

    def nearest(p, centres):
        best, bi = None, 0
        for g, ctr in enumerate(centres):
            dist = sum((p[i] - ctr[i]) ** 2 for i in range(len(p)))
            if best is None or dist < best:
                best, bi = dist, g
        return bi

    kmem = [[k[i]] for i in orc.weyl_indices(n, gk).tolist()]     # members of each key block
    qmem = [[q[i]] for i in orc.weyl_indices(n, gq).tolist()]
    cq = [mean(m) for m in qmem]
    klab = qlab = None
    for _ in range(iters):
        centres = [[sum(col) / len(m) for col in zip(*[aff(r, cq) for r in m])] if m else [0.0] * gq
                   for m in kmem]
        klab = [nearest(aff(k[t], cq), centres) for t in range(n)]
        kmem = [[k[t] for t in range(n) if klab[t] == g] for g in range(gk)]
        ck = [mean(m) for m in kmem]
        centres = [[sum(col) / len(m) for col in zip(*[aff(r, ck) for r in m])] if m else [0.0] * gk
                   for m in qmem]
        qlab = [nearest(aff(q[t], ck), centres) for t in range(n)]
        qmem = [[q[t] for t in range(n) if qlab[t] == g] for g in range(gq)]
        cq = [mean(m) for m in qmem]
    return klab, qlab


@pytest.mark.parametrize("seed", range(3))
def test_svoo_partition_is_the_brute_force_co_clustering(seed):
    """svoo_partition against the loop form of [SVOO]'s alternating steps. The inputs are
    chosen so that independent raw k-means (raw_partition) and the method's partition both
    give other labels, and so does running the query step first."""
    rng = np.random.default_rng(700 + seed)
    n, d, gk, gq, iters = 48, 6, 5, 4, 3
    base = rng.standard_normal((6, d))
    q = (base[rng.integers(0, 6, size=n)] + 0.8 * rng.standard_normal((n, d))).round(2)
    k = (base[rng.integers(0, 6, size=n)] * 1.5 + 0.6 * rng.standard_normal((n, d))).round(2)
    part = orc.svoo_partition(q, k, gk, gq, iters)
    klab, qlab = _brute_svoo(_tolist(q), _tolist(k), gk, gq, iters)
    assert part.key_labels.tolist() == klab
    assert part.q_labels.tolist() == qlab
    assert np.array_equal(part.key_centroids, orc.group_means(k, part.key_labels, gk))
    raw = orc.raw_partition(q, k, gk, gq, iters)
    assert (raw.key_labels.tolist(), raw.q_labels.tolist()) != (klab, qlab)
    meth = orc.partition(q, k, 12, 2, gk, gq, iters)
    assert (meth.key_labels.tolist(), meth.q_labels.tolist()) != (klab, qlab)
    # queries first (step B before step A) gives other labels too
    swapped = orc.svoo_partition(k, q, gq, gk, iters)
    assert (swapped.q_labels.tolist(), swapped.key_labels.tolist()) != (klab, qlab)


def test_svoo_partition_round_is_the_metric_form():
    """One step A is nearest-centroid assignment of raw keys under the metric
    C_Q^T C_Q / d (the form the library's kernels use): |(k - c) C_Q^T|^2 / d."""
    rng = np.random.default_rng(77)
    n, d, gk, gq = 64, 8, 6, 5
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d)) * 2
    part = orc.svoo_partition(q, k, gk, gq, 1)
    cq = q[orc.weyl_indices(n, gq)]
    ck = k[orc.weyl_indices(n, gk)]
    m = cq.T @ cq / d
    dist = np.array([[(k[t] - ck[g]) @ m @ (k[t] - ck[g]) for g in range(gk)] for t in range(n)])
    assert np.array_equal(part.key_labels, np.argmin(dist, axis=1))


# -------------------------------------------------------------- full call ---
def _c1(**kw):
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    st = cfg.settings
    args = dict(n_sample=st.n_sample, key_rank=st.key_rank, kv_groups=st.kv_groups,
                q_groups=st.q_groups, kmeans_iters=st.kmeans_iters, density=st.density,
                probes=st.probes, ridge_lambda=st.ridge_lambda, corr_rank=st.corr_rank)
    args.update(kw)
    return q[0], k[0], v[0], args


def test_call_with_no_probes_is_plain_sparse_output():
    q, k, v, a = _c1(probes=0)
    r = orc.oracle_head(q, k, v, **a)
    back = np.empty_like(r.o_sparse)
    back[r.q_perm] = r.o_sparse
    assert np.array_equal(r.o, back)


def test_call_with_every_row_probed_is_dense():
    q, k, v, a = _c1(probes=2048)
    r = orc.oracle_head(q, k, v, **a)
    assert np.allclose(r.o, orc.dense_attention(q, k, v), atol=1e-12)


def test_call_at_full_density_is_dense():
    q, k, v, a = _c1(density=1.0)
    r = orc.oracle_head(q, k, v, **a)
    assert np.all(r.blocks >= 0) or np.all((r.blocks >= 0).sum(1) == (np.diff(r.key_off) > 0).sum())
    assert np.abs(r.y).max() < 1e-12
    assert np.allclose(r.o, orc.dense_attention(q, k, v), atol=1e-11)


def test_call_c1_structure():
    q, k, v, a = _c1()
    r = orc.oracle_head(q, k, v, **a)
    assert np.array_equal(np.sort(r.q_perm), np.arange(2048))
    assert r.blocks.shape == (16, 4) and len(r.probe_pos) == 64
    assert np.all(np.isfinite(r.o))
    # the unprobed rows get exactly O_s + b' + O_s B', in original order
    o_perm = r.o_sparse + r.b_vec + r.o_sparse @ r.b_mat
    unprobed = np.setdiff1d(np.arange(2048), r.probe_pos)
    assert np.allclose(r.o[r.q_perm[unprobed]], o_perm[unprobed], atol=1e-13)
    # probe rows output their exact dense value
    dense = orc.dense_attention(q, k, v)
    assert np.allclose(r.o[r.probe_orig], dense[r.probe_orig], atol=1e-12)


# ------------------------------------------------------------ reuse experiment ---
def test_reuse_on_the_same_inputs_is_the_same_call():
    """oracle_head(reuse=r) on the inputs that produced r reproduces r field by field."""
    q, k, v, a = _c1()
    r = orc.oracle_head(q, k, v, **a)
    again = orc.oracle_head(q, k, v, reuse=r, **a)
    for f in ("key_labels", "q_labels", "key_perm", "q_perm", "key_off", "q_off", "blocks",
              "probe_pos", "probe_orig", "o_sparse", "x", "y", "b_mat", "b_vec", "o"):
        assert np.array_equal(getattr(again, f), getattr(r, f)), f


def test_reuse_keeps_the_layout_but_attends_with_the_new_inputs():
    """With every block pair kept (rho = 1) the sparse output of a reused call is plain dense
    attention of the NEW inputs, whatever partition was kept; the kept labels, blocks and
    probe rows are the earlier call's."""
    q, k, v, a = _c1(density=1.0)
    r0 = orc.oracle_head(q, k, v, **a)
    rng = np.random.default_rng(91)
    q1 = q + 0.5 * rng.standard_normal(q.shape)
    k1 = k + 0.5 * rng.standard_normal(k.shape)
    v1 = v[rng.permutation(v.shape[0])]
    r1 = orc.oracle_head(q1, k1, v1, reuse=r0, **a)
    assert np.array_equal(r1.key_labels, r0.key_labels) and np.array_equal(r1.blocks, r0.blocks)
    assert np.array_equal(r1.probe_orig, r0.probe_orig)
    dense = orc.dense_attention(q1, k1, v1)
    back = np.empty_like(r1.o_sparse)
    back[r1.q_perm] = r1.o_sparse
    assert np.allclose(back, dense, rtol=0, atol=1e-12)
    # and the new partition of these inputs differs from the kept one (the test separates them)
    assert not np.array_equal(orc.oracle_head(q1, k1, v1, **a).key_labels, r0.key_labels)


# ------------------------------------------------------- fp8 logits (an experiment) ---
def test_e4m3_round_matches_the_decoded_code_table():
    """e4m3_round against a search over every decoded E4M3 code: random magnitudes over
    the whole range, every midpoint between neighbouring values (the ties) and the values
    themselves."""
    vals = brute.e4m3_values()
    rng = np.random.default_rng(8)
    xs = list(np.exp2(rng.uniform(-12, 9.2, 400)) * rng.choice([-1, 1], 400))
    xs += [0.5 * (a + b) for a, b in zip(vals[:-1], vals[1:])]
    xs += vals + [-v for v in vals[1:]] + [0.0, 448.0, 460.0, -1e-6]
    got = orc.e4m3_round(np.array(xs))
    want = np.array([brute.e4m3_nearest(float(x)) for x in xs])
    assert np.array_equal(got, want)


def test_e4m3_known_values():
    """Closed cases of the format: the extremes, the subnormal spacing and ties to even."""
    r = orc.e4m3_round
    assert r(np.array([448.0]))[0] == 448.0                    # largest finite
    assert r(np.array([2.0 ** -6]))[0] == 2.0 ** -6            # smallest normal
    assert r(np.array([2.0 ** -9]))[0] == 2.0 ** -9            # smallest subnormal
    assert r(np.array([2.0 ** -10]))[0] == 0.0                 # tie between 0 and 2^-9: even
    assert r(np.array([1.0625]))[0] == 1.0                     # tie 1.0 / 1.125: even mantissa 0
    assert r(np.array([1.1875]))[0] == 1.25                    # tie 1.125 / 1.25: even mantissa 2
    assert r(np.array([-2.5]))[0] == -2.5
    assert r(np.array([3.3]))[0] == 3.25                       # spacing 0.25 in [2, 4)


def test_f8_scale_exp_is_the_largest_exponent_that_fits():
    rng = np.random.default_rng(9)
    for a in list(np.exp2(rng.uniform(-30, 30, 300))) + [448.0, 1.75, 1.7500001, 224.0, 1.0]:
        e = orc.f8_scale_exp(float(a))
        assert a * 2.0 ** e <= 448.0 < a * 2.0 ** (e + 1)
    assert orc.f8_scale_exp(0.0) == 0


def _tiny_call_inputs(seed, n=48, d=16):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(n, d)), rng.normal(size=(n, d)), rng.normal(size=(n, d)))


def test_fp8_logits_are_exact_for_e4m3_representable_inputs():
    """When every scaled q and k is already an E4M3 value, the fp8 call is the plain call
    (so the scales are applied and undone exactly)."""
    vals = np.array(brute.e4m3_values())
    rng = np.random.default_rng(10)
    n, d = 48, 16
    q = rng.choice(vals, size=(n, d)) * rng.choice([-1.0, 1.0], size=(n, d))
    k = rng.choice(vals, size=(n, d)) * rng.choice([-1.0, 1.0], size=(n, d))
    q[0, 0], k[0, 0] = 448.0, -448.0                      # scales 2^0 after the 2^-3 below
    q, k = q * 2.0 ** -3, k * 2.0 ** -5
    v = rng.normal(size=(n, d))
    kw = dict(n_sample=8, key_rank=4, kv_groups=4, q_groups=3, kmeans_iters=2, density=0.5,
              probes=6, ridge_lambda=1e-3, corr_rank=2)
    plain = orc.oracle_head(q, k, v, **kw)
    f8 = orc.oracle_head(q, k, v, fp8_qk=True, **kw)
    assert np.array_equal(plain.o_sparse, f8.o_sparse)
    assert np.array_equal(plain.o, f8.o)


def test_fp8_logits_quantize_q_and_k_per_tensor_and_leave_the_rest():
    """The fp8 sparse output is the masked softmax of brute-quantized Q and K (each scaled by
    its own power of two, V untouched), and the probe data and fit are the plain call's."""
    q, k, v = _tiny_call_inputs(11)
    kw = dict(n_sample=8, key_rank=4, kv_groups=4, q_groups=3, kmeans_iters=2, density=0.5,
              probes=6, ridge_lambda=1e-3, corr_rank=2)
    plain = orc.oracle_head(q, k, v, **kw)
    f8 = orc.oracle_head(q, k, v, fp8_qk=True, **kw)
    eq, ek = orc.f8_scale_exp(np.abs(q).max()), orc.f8_scale_exp(np.abs(k).max())
    qq = [[brute.e4m3_nearest(x * 2.0 ** eq) * 2.0 ** -eq for x in row] for row in q[plain.q_perm]]
    kq = [[brute.e4m3_nearest(x * 2.0 ** ek) * 2.0 ** -ek for x in row] for row in k[plain.key_perm]]
    vp = v[plain.key_perm].tolist()
    for i in range(len(plain.q_off) - 1):
        allowed_keys = set(orc.routed_keys(plain.key_off, plain.blocks[i]).tolist())
        rows = range(plain.q_off[i], plain.q_off[i + 1])
        mask = [[j in allowed_keys for j in range(len(kq))] for _ in rows]
        want = brute.attention([qq[r] for r in rows], kq, vp, mask)
        assert np.allclose(f8.o_sparse[list(rows)], np.array(want), rtol=1e-12, atol=1e-12)
    assert np.array_equal(plain.x, f8.x) and np.array_equal(plain.y, f8.y)
    assert np.array_equal(plain.b_mat, f8.b_mat)
    assert not np.array_equal(plain.o_sparse, f8.o_sparse)
