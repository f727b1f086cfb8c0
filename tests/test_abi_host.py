"""CPU tests of the C ABI: exported symbols, parameter validation, and the host-side
fp64 solves (checked against numpy and the oracle). No GPU calls."""
import ctypes
import os
import re

import numpy as np
import pytest

import free_block_sparse_eigen_amd as spr
import oracle as orc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "sparsepr.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparsepr_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared()
    assert len(names) >= 20
    for n in names:
        assert hasattr(spr.lib, n), n
    assert sorted(spr.EXPORTS) == names


def _params(**kw):
    base = dict(heads=2, n=2048, d=64, dtype=spr.F32, kv_groups=16, q_groups=16, density=0.25,
                probes=64, corr_rank=8)
    base.update(kw)
    return spr.make_params(**base)


def test_validation_accepts_configs_and_rejects_bad_values():
    assert spr.sparsepr_validate(_params()) == 0
    assert spr.sparsepr_workspace_bytes(_params()) > 0
    bad = [dict(d=96), dict(n=0), dict(heads=0), dict(kv_groups=0), dict(kv_groups=2049),
           dict(q_groups=1025, n=4096), dict(density=0.0), dict(density=1.5), dict(probes=-1),
           dict(probes=4097, n=8192), dict(corr_rank=65), dict(ridge_lambda=-1.0),
           dict(ridge_lambda=float("nan")), dict(kmeans_iters=0), dict(key_rank=0),
           dict(key_rank=65), dict(n_sample=0), dict(dtype=7), dict(flags=1 << 20)]
    for kw in bad:
        p = _params(**kw)
        if "n_sample" in kw:
            p.n_sample = kw["n_sample"]
        assert spr.sparsepr_validate(p) != 0, kw
        assert spr.sparsepr_workspace_bytes(p) == 0, kw


def test_status_strings():
    for s in range(7):
        assert spr.lib.sparsepr_status_str(s).decode()
    assert spr.lib.sparsepr_last_error(None).decode() == ""


def test_null_context_is_rejected_without_gpu():
    assert spr.lib.sparsepr_sparse_attn(None, None) == 1
    assert spr.lib.sparsepr_probe_fit(None, None) == 1
    s = spr.Stats()
    assert spr.lib.sparsepr_get_stats(None, ctypes.byref(s)) == 1


# --------------------------------------------------------------- host solves ---
@pytest.mark.parametrize("n,r,seed", [(1, 1, 0), (2, 2, 1), (7, 3, 2), (64, 16, 3),
                                      (128, 32, 4), (128, 128, 5)])
def test_sym_eig_top_matches_numpy(n, r, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((n, n))
    a = a @ a.T / n
    lam, vec = spr.sparsepr_host_sym_eig_top(a, r)
    ref = np.linalg.eigvalsh(a)[::-1][:r]
    assert np.allclose(lam, ref, rtol=1e-12, atol=1e-13 * abs(ref[0]))
    assert np.allclose(a @ vec, vec * lam, atol=1e-10 * abs(ref[0]))
    assert np.allclose(vec.T @ vec, np.eye(r), atol=1e-10)


def test_sym_eig_top_clustered_and_deficient():
    rng = np.random.default_rng(7)
    u, _ = np.linalg.qr(rng.standard_normal((40, 40)))
    lam = np.concatenate([[5.0, 5.0, 5.0, 3.0, 3.0 + 1e-12], np.zeros(35)])
    a = u @ np.diag(lam) @ u.T
    got, vec = spr.sparsepr_host_sym_eig_top(a, 5)
    assert np.allclose(got, lam[:5], atol=1e-12)
    assert np.allclose(vec.T @ vec, np.eye(5), atol=1e-9)
    proj = vec[:, :3] @ vec[:, :3].T
    assert np.allclose(proj, u[:, :3] @ u[:, :3].T, atol=1e-9)


def test_sym_eig_top_zero_matrix():
    lam, vec = spr.sparsepr_host_sym_eig_top(np.zeros((5, 5)), 2)
    assert np.all(lam == 0) and np.allclose(vec.T @ vec, np.eye(2))


def test_key_projection_matches_oracle_metric_distances():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((300, 64))
    mk = orc.key_metric(q, 128)
    w = spr.sparsepr_host_key_projection(mk, 16)
    w_ref, _ = orc.key_projection(mk, 16)
    # columns may differ by sign; W W^T is unique
    assert np.allclose(w @ w.T, w_ref @ w_ref.T, atol=1e-11)


@pytest.mark.parametrize("p,d,lam,r", [(64, 64, 1e-3, 8), (256, 128, 1e-3, 16), (300, 32, 0.5, 4),
                                       (1, 16, 1e-3, 4), (10, 16, 1e-3, 16)])
def test_probe_fit_matches_oracle(p, d, lam, r):
    rng = np.random.default_rng(11 + p)
    x = rng.standard_normal((p, d))
    y = 0.1 * rng.standard_normal((p, d)) + 0.05 * x @ rng.standard_normal((d, d))
    bm, bv = spr.sparsepr_host_probe_fit(x, y, lam, r)
    rbm, rbv = orc.probe_fit(x, y, lam, r)
    scale = max(1.0, np.abs(rbm).max())
    assert np.allclose(bm, rbm, atol=1e-9 * scale) and np.allclose(bv, rbv, atol=1e-9 * scale)


def test_probe_fit_zero_residual_and_no_probes():
    x = np.random.default_rng(12).standard_normal((50, 8))
    bm, bv = spr.sparsepr_host_probe_fit(x, np.zeros((50, 8)), 1e-3, 4)
    assert np.all(bm == 0) and np.all(bv == 0)
    bm, bv = spr.sparsepr_host_probe_fit(np.zeros((0, 8)), np.zeros((0, 8)), 1e-3, 4)
    assert np.all(bm == 0) and np.all(bv == 0)


def test_probe_fit_exact_low_rank_residual():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((80, 12))
    y = rng.standard_normal((80, 3)) @ rng.standard_normal((3, 12))
    bm, bv = spr.sparsepr_host_probe_fit(x, y, 1e-6, 8)
    rbm, rbv = orc.probe_fit(x, y, 1e-6, 8)
    assert np.allclose(bm, rbm, atol=1e-8) and np.allclose(bv, rbv, atol=1e-8)


def test_probe_fit_min_norm_least_squares():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((40, 6))
    y = rng.standard_normal((40, 6))
    bm, bv = spr.sparsepr_host_probe_fit(x, y, 0.0, 6)
    rbm, rbv = orc.probe_fit(x, y, 0.0, 6)
    assert np.allclose(bm, rbm, atol=1e-9) and np.allclose(bv, rbv, atol=1e-9)


def test_single_hip_runtime_in_process():
    """Importing the binding alone (before anything else loads torch) leaves exactly one
    HIP runtime mapped: the library must bind to torch's, never load a second copy."""
    import subprocess
    import sys
    code = ("import free_block_sparse_eigen_amd, re\n"
            "paths = set()\n"
            "for line in open('/proc/self/maps'):\n"
            "    f = line.split()[-1]\n"
            "    if re.search(r'libamdhip64\\.so', f): paths.add(f)\n"
            "print(len(paths)); print(sorted(paths))\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split("\n")[0] == "1", r.stdout


def test_diagnostics_support_statistics_on_a_constructed_case():
    """Each query attends (to machine precision) to one key: row supports are 1, a group's
    aggregate support is the number of distinct keys its rows attend to, and the routed
    mass is the share of its rows whose key lies in the routed key groups."""
    from free_block_sparse_eigen_amd import diagnostics as dg
    d = 4
    k = (np.eye(d) * 10.0)[None]                      # key j along axis j
    attend = np.array([0, 0, 1, 2, 0])                # query row -> attended key
    q = (np.eye(d)[attend] * 10.0)[None]              # logits 50 on the attended key, 0 elsewhere
    part = {"q_perm": np.array([[0, 1, 2, 3, 4]]), "q_off": np.array([[0, 3, 5]]),
            "key_perm": np.array([[0, 1, 2, 3]]), "key_off": np.array([[0, 2, 4]])}
    rout = {"blocks": np.array([[[0], [1]]])}         # q group 0 -> keys {0,1}, group 1 -> {2,3}
    res = dg._support_stats(q, k, part, rout, groups=2, tau=0.9, d=d)
    assert [r["group"] for r in res] == [0, 1]
    g0, g1 = res
    assert g0["rows"] == 3 and g0["mean_row_support"] == 1.0 and g0["aggregate_support"] == 2
    assert g0["expansion"] == 2.0 and g0["routed_keys"] == 2 and abs(g0["routed_mass"] - 1.0) < 1e-12
    assert g1["rows"] == 2 and g1["aggregate_support"] == 2 and abs(g1["routed_mass"] - 0.5) < 1e-12


def test_validate_accepts_the_comparison_partitioner_flag():
    p = spr.make_params(1, 4096, 64, spr.F32, n_sample=128, key_rank=16, kv_groups=16,
                        q_groups=16, density=0.25, probes=64, corr_rank=8, flags=spr.F_RAW_KMEANS)
    assert spr.lib.sparsepr_validate(ctypes.byref(p)) == 0
    p.flags = spr.F_RAW_KMEANS | spr.F_STAGE_TIMING
    assert spr.lib.sparsepr_validate(ctypes.byref(p)) == 0
    p.flags = spr.F_RAW_KMEANS | spr.F_CHECK_FINITE
    assert spr.lib.sparsepr_validate(ctypes.byref(p)) == 0
    p.flags = 1 << 20
    assert spr.lib.sparsepr_validate(ctypes.byref(p)) == 1        # SPARSEPR_ERR_INVALID_ARG
    # the comparison partitioner needs d-wide fp64 key centroids: the workspace grows
    # (against the method with its eigensolve on the host, which has no device eigen scratch,
    # at a key rank of 8, which has no split key coordinates for the screen)
    p.key_rank = 8
    p.flags = spr.F_HOST_SOLVE
    base = spr.lib.sparsepr_workspace_bytes(ctypes.byref(p))
    p.flags = 0
    assert spr.lib.sparsepr_workspace_bytes(ctypes.byref(p)) > base      # device eigen scratch
    p.flags = spr.F_RAW_KMEANS
    assert spr.lib.sparsepr_workspace_bytes(ctypes.byref(p)) > base



@pytest.mark.parametrize("gk,rho", [(16, 0.25), (128, 0.25), (256, 0.15), (256, 0.22), (256, 0.26),
                                    (256, 0.35), (256, 1.0), (384, 0.24), (256, 1e-6), (7, 0.5)])
def test_routed_count_comes_from_the_library(gk, rho):
    """The block-list width k is the library's (the binding computes nothing of the method);
    it follows the oracle's rule k = ceil(rho G_k - 1e-9) clamped to [1, G_k]."""
    p = _params(n=4096, kv_groups=gk, density=rho)
    assert spr.sparsepr_routed_count(p) == orc.routed_count(rho, gk)
    p.density = 0.0
    assert spr.lib.sparsepr_routed_count(ctypes.byref(p)) < 0


def test_validate_limits_one_heads_rows_to_32_bit_offsets():
    """The kernels address one head's bf16 rows with 32-bit buffer offsets: n d 2 < 2^31."""
    for d, n_max in ((128, (1 << 23) - 1), (64, (1 << 24) - 1)):
        ok = _params(heads=1, n=n_max, d=d, key_rank=d // 4, corr_rank=8)
        assert spr.sparsepr_validate(ok) == 0, (d, n_max)
        big = _params(heads=1, n=n_max + 1, d=d, key_rank=d // 4, corr_rank=8)
        assert spr.sparsepr_validate(big) == 2, (d, n_max + 1)          # SPARSEPR_ERR_SHAPE


def test_sym_eig_top_resolves_eigenvalues_far_below_the_norm():
    """Eigenvalues spanning 1e-10 of the largest (a Gram of residuals whose singular values
    span 1e-5): each must come out to high relative accuracy, in order, with orthonormal
    vectors (shifts kept apart relative to each eigenvalue, not to |A|)."""
    rng = np.random.default_rng(12)
    n, r = 64, 20
    u, _ = np.linalg.qr(rng.standard_normal((n, n)))
    ev = np.sort(np.concatenate([np.logspace(0, -10, 30), np.zeros(n - 30)]))[::-1]
    a = (u * ev) @ u.T
    lam, vec = spr.sparsepr_host_sym_eig_top(a, r)
    assert np.all(np.abs(lam / ev[:r] - 1) < 1e-5)
    assert np.all(np.diff(lam) < 0)
    assert np.abs(vec.T @ vec - np.eye(r)).max() < 1e-12
    assert np.abs(a @ vec - vec * lam).max() < 1e-13


def test_probe_fit_with_a_wide_residual_spectrum_matches_oracle():
    """Residual singular values spanning 1e-5 (as at the 720p shape with rho = 0.35): the
    Gram-route fit must still give the oracle's (SVD-route) B' and b'."""
    rng = np.random.default_rng(13)
    p, d, r = 256, 128, 16
    x = rng.standard_normal((p, d))
    sv = np.logspace(0, -5.5, d)
    uy, _ = np.linalg.qr(rng.standard_normal((p, d)))
    vy, _ = np.linalg.qr(rng.standard_normal((d, d)))
    y = (uy * sv) @ vy.T
    bm, bv = spr.sparsepr_host_probe_fit(x, y, 1e-3, r)
    rbm, rbv = orc.probe_fit(x, y, 1e-3, r)
    scale = max(1.0, np.abs(rbm).max())
    assert np.abs(bm - rbm).max() < 1e-10 * scale and np.abs(bv - rbv).max() < 1e-10 * scale


def test_noalloc_dense_rejects_shapes_and_pointers_before_any_device_use():
    """The no-allocation dense entry point checks its limits (d, the static scratch's 8192
    work units of 256 rows, heads * n) and its pointers on the host, before it touches a
    device, and reports why through sparsepr_last_error(NULL)."""
    lib = spr.lib
    f = lib.sparsepr_dense_attn_noalloc
    assert f(1, 2097153, 64, None, None, None, None, None) == 2
    assert b"8192" in lib.sparsepr_last_error(None)
    assert f(1, 1000, 96, None, None, None, None, None) == 2
    assert f(0, 1000, 64, None, None, None, None, None) == 2
    assert f(1100, 2000000, 128, None, None, None, None, None) == 2      # heads * n >= 2^31
    assert f(1, 2097152, 64, None, None, None, None, None) == 1          # largest n: pointers
    assert b"null or misaligned" in lib.sparsepr_last_error(None)


def test_svoo_and_raw_kmeans_flags_are_exclusive():
    """The two comparison partitioners cannot be combined; each alone is accepted."""
    kw = dict(kv_groups=16, q_groups=16, density=0.25, probes=8, corr_rank=4)
    both = spr.make_params(1, 1024, 64, spr.BF16, flags=spr.F_SVOO | spr.F_RAW_KMEANS, **kw)
    assert spr.sparsepr_validate(both) == 1
    for f in (spr.F_SVOO, spr.F_RAW_KMEANS):
        assert spr.sparsepr_validate(spr.make_params(1, 1024, 64, spr.BF16, flags=f, **kw)) == 0
    # the co-clustering context has no M_K eigensolve but the same workspace otherwise
    assert spr.sparsepr_workspace_bytes(spr.make_params(1, 1024, 64, spr.BF16, flags=spr.F_SVOO, **kw)) > 0


def test_serial_partition_flag_is_accepted_alone_and_combined():
    """SPARSEPR_F_SERIAL_PARTITION only changes which streams the partition runs on."""
    kw = dict(kv_groups=16, q_groups=16, density=0.25, probes=8, corr_rank=4)
    for f in (spr.F_SERIAL_PARTITION, spr.F_SERIAL_PARTITION | spr.F_STAGE_TIMING,
              spr.F_SERIAL_PARTITION | spr.F_HOST_SOLVE | spr.F_CHECK_FINITE):
        assert spr.sparsepr_validate(spr.make_params(2, 1024, 64, spr.BF16, flags=f, **kw)) == 0
    assert spr.sparsepr_validate(spr.make_params(2, 1024, 64, spr.BF16, flags=512, **kw)) == 1


def test_uniform_units_flag_is_accepted_and_keeps_the_workspace():
    """SPARSEPR_F_UNIFORM_UNITS only changes how the sparse kernel's work is cut: it is valid
    alone and with the other flags, and the workspace (which always holds both unit lists)
    is the same with and without it."""
    kw = dict(kv_groups=16, q_groups=16, density=0.25, probes=8, corr_rank=4)
    assert spr.F_UNIFORM_UNITS == 256
    for f in (spr.F_UNIFORM_UNITS, spr.F_UNIFORM_UNITS | spr.F_STAGE_TIMING | spr.F_SERIAL_PARTITION,
              spr.F_UNIFORM_UNITS | spr.F_FP8_QK):
        assert spr.sparsepr_validate(spr.make_params(2, 1024, 64, spr.BF16, flags=f, **kw)) == 0
    ws = [spr.sparsepr_workspace_bytes(spr.make_params(2, 75600, 128, spr.BF16, flags=f, **kw))
          for f in (0, spr.F_UNIFORM_UNITS)]
    assert ws[0] == ws[1] > 0


def test_raw_key_screen_flag_drops_the_split_key_coordinates():
    """By default the key screen runs on the split coordinates x W (bf16 hi + lo, [H][N][2][r_K])
    and a bound coefficient per key (fp32 [H][N]); SPARSEPR_F_RAW_KEY_SCREEN screens raw keys
    and needs neither. Key ranks without a coordinate kernel (8) never take them; key groups
    whose raw screen streams its centroids (384 at d = 128) still do, since their split
    coordinates fit in LDS (their candidate lists are then screened in the coordinates too)."""
    kw = dict(q_groups=16, density=0.25, probes=8, corr_rank=4)
    ws = lambda f, rk, gk, d=64: spr.sparsepr_workspace_bytes(
        spr.make_params(2, 1024, d, spr.BF16, flags=f, key_rank=rk, kv_groups=gk, **kw))
    assert ws(0, 16, 16) - ws(spr.F_RAW_KEY_SCREEN, 16, 16) == 2 * 1024 * 2 * 16 * 2 + 2 * 1024 * 4
    assert ws(0, 32, 16) - ws(spr.F_RAW_KEY_SCREEN, 32, 16) == 2 * 1024 * 2 * 32 * 2 + 2 * 1024 * 4
    assert ws(0, 8, 16) == ws(spr.F_RAW_KEY_SCREEN, 8, 16)
    assert ws(0, 32, 384, 128) - ws(spr.F_RAW_KEY_SCREEN, 32, 384, 128) == 2 * 1024 * 2 * 32 * 2 + 2 * 1024 * 4
    assert spr.sparsepr_validate(spr.make_params(2, 1024, 64, spr.BF16, flags=spr.F_RAW_KEY_SCREEN,
                                                 kv_groups=16, **kw)) == 0


def test_fp8_logit_flag_grows_the_workspace_by_one_byte_per_key_element():
    kw = dict(kv_groups=16, q_groups=16, density=0.25, probes=8, corr_rank=4)
    base = spr.sparsepr_workspace_bytes(spr.make_params(2, 1024, 64, spr.BF16, **kw))
    f8 = spr.sparsepr_workspace_bytes(spr.make_params(2, 1024, 64, spr.BF16, flags=spr.F_FP8_QK, **kw))
    assert 2 * 1024 * 64 <= f8 - base <= 2 * 1024 * 64 + 3 * 256
