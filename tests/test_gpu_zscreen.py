"""GPU parity of the key screen in the key coordinates.

With the key centroids resident in LDS and r_K = 16 or 32, the key side of the k-means
screens each key through its coordinates z = x W (formed once per call on MFMA and split
into bf16 hi + lo) against the centroids' split coordinates. Each key carries a bound
coefficient that covers the coordinates' own error, the splits' residuals and the fp32 sum;
keys whose margin it does not certify go to the fp64 recheck. The partition must therefore
be bit-identical to the one SPARSEPR_F_RAW_KEY_SCREEN gives (raw keys against W c), and
bit-exact against the oracle wherever the oracle's own rounding does not decide a tie.
These inputs put many keys on or near the boundary between centroids: keys drawn from a
few distinct rows (exact duplicates, equal seeds and so exact ties), the same keys scaled
far from 1, and clusters of nearly equal keys.
"""
import numpy as np
import pytest

import oracle as orc
from synthetic import bf16_round
from tests.gpu_common import check_close, run_gpu_call, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _inputs(kind, n, d, seed):
    rng = np.random.default_rng(seed)
    q = bf16_round(rng.standard_normal((1, n, d)) * 1.5)
    v = bf16_round(rng.standard_normal((1, n, d)))
    if kind == "duplicates":
        # 40 distinct rows on a half-integer lattice (exact in bf16), each repeated
        base = rng.integers(-2, 3, size=(40, d)) * 0.5
        k = base[rng.integers(0, 40, size=n)][None]
    else:
        # 60 cluster centres, each key its centre plus a perturbation of 1 % (bf16-rounded)
        base = rng.standard_normal((60, d))
        k = base[rng.integers(0, 60, size=n)] + 0.01 * rng.standard_normal((n, d))
        k = bf16_round(k[None])
    return q, k, v


CASES = [("duplicates", 64, 16, 1.0), ("duplicates", 64, 16, 2.0 ** 12), ("duplicates", 64, 16, 2.0 ** -12),
         ("duplicates", 128, 32, 1.0), ("near", 64, 16, 1.0), ("near", 128, 32, 1.0),
         ("near", 128, 16, 1.0), ("near", 64, 32, 1.0)]
IDS = ["dup-d64", "dup-d64-x4096", "dup-d64-x2^-12", "dup-d128", "near-d64", "near-d128", "near-d128-r16",
       "near-d64-r32"]


def _run(spr, q, k, v, kw, flags):
    n, d = q.shape[1], q.shape[2]
    ctx = spr.SparsePR(spr.make_params(1, n, d, spr.BF16, flags=flags, **kw))
    g = run_gpu_call(ctx, q, k, v, "bf16")
    ctx.close()
    return g


@pytest.mark.timeout(300)
@pytest.mark.parametrize("kind,d,rk,scale", CASES, ids=IDS)
def test_key_screen_in_coordinates_keeps_labels_exact(spr, kind, d, rk, scale):
    """Both screens certify against the same exact scores of the same fp64 centroids and leave
    the rest to the same fp64 recheck, so the partition must be bit-identical between them on
    any input. Against the oracle only without exact duplicates: with them, groups seeded
    from equal keys tie exactly, and the oracle's centroids (means of its fp64 coordinates,
    rounded) break those ties by their last bits while the device's (coordinates of exact
    raw means) keep them tied for the lowest index; both are nearest-centroid labels."""
    n = 3000
    say(f"key screen in the coordinates: {kind}, d={d}, r_K={rk}, keys x {scale}")
    q, k, v = _inputs(kind, n, d, seed=11 + d + rk)
    k = k * scale                                   # a power of two: exact in bf16
    kw = dict(n_sample=64, key_rank=rk, kv_groups=64, q_groups=16, kmeans_iters=3, density=0.5,
              probes=20, ridge_lambda=1e-3, corr_rank=4)
    gz = _run(spr, q, k, v, kw, 0)
    gr = _run(spr, q, k, v, kw, spr.F_RAW_KEY_SCREEN)
    say(f"recheck points per call: {gz['stats']['recheck_points']} (coordinates), "
        f"{gr['stats']['recheck_points']} (raw keys)")
    assert np.array_equal(gz["key_labels"], gr["key_labels"]), "key labels, coordinates against raw"
    assert np.array_equal(gz["key_centroids"], gr["key_centroids"]), "key centroids"
    assert np.array_equal(gz["q_labels"], gr["q_labels"]), "query labels"
    assert np.array_equal(gz["blocks"], gr["blocks"]), "blocks"
    assert np.array_equal(gz["o"], gr["o"]), "output"
    assert np.all(np.isfinite(gz["o"]))
    if kind == "duplicates":
        assert gz["stats"]["recheck_points"] > 0   # equal seeds tie exactly: the recheck ran
        return
    ref = orc.oracle_head(q[0], k[0], v[0], **kw)
    assert np.array_equal(gz["key_labels"][0], ref.key_labels), "key labels"
    assert np.array_equal(gz["q_labels"][0], ref.q_labels), "query labels"
    assert np.array_equal(gz["blocks"][0], ref.blocks), "blocks"
    check_close(gz["o"][0], ref.o, f"O {kind} d={d}", out_rel=2.0 ** -24)


@pytest.mark.timeout(300)
def test_key_screen_modes_agree_on_three_heads(spr):
    """Three heads (an uneven split into two head groups on two streams), N = 2,500 (not a
    multiple of 64), r_K = 32: both screens bit-identical, and the oracle per head."""
    n, d, heads = 2500, 128, 3
    qs, ks, vs = zip(*(_inputs("near", n, d, seed=40 + i) for i in range(heads)))
    q, k, v = (np.concatenate(a, axis=0) for a in (qs, ks, vs))
    kw = dict(n_sample=64, key_rank=32, kv_groups=48, q_groups=24, kmeans_iters=3, density=0.4,
              probes=16, ridge_lambda=1e-3, corr_rank=4)
    out = []
    for flags in (0, spr.F_RAW_KEY_SCREEN):
        ctx = spr.SparsePR(spr.make_params(heads, n, d, spr.BF16, flags=flags, **kw))
        out.append(run_gpu_call(ctx, q, k, v, "bf16"))
        ctx.close()
    for key in ("key_labels", "key_centroids", "q_labels", "blocks", "o"):
        assert np.array_equal(out[0][key], out[1][key]), key
    for i in range(heads):
        ref = orc.oracle_head(q[i], k[i], v[i], **kw)
        assert np.array_equal(out[0]["key_labels"][i], ref.key_labels), f"h{i} key labels"
        assert np.array_equal(out[0]["q_labels"][i], ref.q_labels), f"h{i} query labels"


@pytest.mark.timeout(600)
def test_key_screen_modes_agree_on_c2(spr):
    """Both screens on two C2 heads (r_K = 32, 128 key groups, N = 32,760), split over two
    streams: bit-identical partitions."""
    from synthetic import get_config, make_inputs
    cfg = get_config("C2")
    heads = [1, 6]
    q, k, v = make_inputs(cfg, heads=heads)
    out = []
    for flags in (0, spr.F_RAW_KEY_SCREEN):
        ctx = spr.SparsePR.from_settings(len(heads), cfg.n, cfg.d, spr.BF16, cfg.settings, flags=flags)
        out.append(run_gpu_call(ctx, q, k, v, cfg.dtype))
        ctx.close()
    say(f"C2 recheck points: {out[0]['stats']['recheck_points']} (coordinates), "
        f"{out[1]['stats']['recheck_points']} (raw keys)")
    for key in ("key_labels", "key_centroids", "q_labels", "blocks", "o"):
        assert np.array_equal(out[0][key], out[1][key]), key


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", ["near", "duplicates"])
def test_key_screen_modes_agree_with_candidate_lists(spr, kind):
    """384 key groups at d = 128: the raw screen streams its centroids and the keys it does not
    certify get candidate lists before the fp64 check; in the coordinates the screen stays
    resident and the lists are screened in the coordinates too. Clustered keys (and exact
    duplicates) leave many keys near a boundary, so the lists are long and some overflow to
    the full recheck. Both screens bit-identical, on two heads over two streams; the oracle
    as well for the clustered keys."""
    n, d, heads = 12000, 128, 2
    qs, ks, vs = zip(*(_inputs(kind, n, d, seed=70 + i) for i in range(heads)))
    q, k, v = (np.concatenate(a, axis=0) for a in (qs, ks, vs))
    kw = dict(n_sample=64, key_rank=32, kv_groups=384, q_groups=24, kmeans_iters=3, density=0.3,
              probes=16, ridge_lambda=1e-3, corr_rank=4)
    out = []
    for flags in (0, spr.F_RAW_KEY_SCREEN):
        ctx = spr.SparsePR(spr.make_params(heads, n, d, spr.BF16, flags=flags, **kw))
        out.append(run_gpu_call(ctx, q, k, v, "bf16"))
        ctx.close()
    say(f"384 groups, {kind}: recheck points {out[0]['stats']['recheck_points']} (coordinates), "
        f"{out[1]['stats']['recheck_points']} (raw keys)")
    assert out[0]["stats"]["recheck_points"] > 0
    for key in ("key_labels", "key_centroids", "q_labels", "blocks", "o"):
        assert np.array_equal(out[0][key], out[1][key]), key
    if kind == "duplicates":
        return
    for i in range(heads):
        ref = orc.oracle_head(q[i], k[i], v[i], **kw)
        assert np.array_equal(out[0]["key_labels"][i], ref.key_labels), f"h{i} key labels"
        assert np.array_equal(out[0]["q_labels"][i], ref.q_labels), f"h{i} query labels"
