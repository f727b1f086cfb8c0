"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Integer results (labels, permutations, offsets, block lists, probe rows) must be
bit-exact; floating-point outputs must be within 5e-3 relative Frobenius and 2e-2
max-abs of the oracle, on the same bf16-rounded inputs."""
import math

import numpy as np
import pytest

import oracle as orc
from synthetic import bf16_round, get_config, make_inputs
from tests.gpu_common import (check_close, from_dev, max_abs, oracle_given_partition, rel_fro,
                              run_gpu_call, say, settings_kw, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import free_block_sparse_eigen_amd as mod
    return mod


def _random_qkv(h, n, d, seed, logit_std=3.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((h, n, d))
    k = rng.standard_normal((h, n, d))
    v = rng.standard_normal((h, n, d))
    s = math.sqrt(logit_std)
    return bf16_round(q * s), bf16_round(k * s), bf16_round(v)


# ------------------------------------------------------------------ dense ---
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 300, 1000])
def test_dense_attention_matches_oracle(spr, d, dtype, n):
    say(f"dense d={d} dtype={dtype} n={n}")
    import torch
    q, k, v = _random_qkv(2, n, d, seed=n + d)
    ctx = spr.SparsePR(spr.make_params(2, n, d, spr.BF16 if dtype == "bf16" else spr.F32,
                                       kv_groups=1, q_groups=1, density=1.0, probes=0,
                                       corr_rank=0))
    o = from_dev(ctx.sparsepr_dense_attn(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)))
    torch.cuda.synchronize()
    for h in range(2):
        check_close(o[h], orc.dense_attention(q[h], k[h], v[h]), f"dense head {h}",
                    out_rel=2.0 ** -8 if dtype == "bf16" else 2.0 ** -24)


# ------------------------------------------------------------- tiny config ---
@pytest.fixture(scope="module")
def c1_run(spr):
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    say("C1 full call")
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings)
    g = run_gpu_call(ctx, q, k, v, "f32")
    ref = orc.oracle_call(q, k, v, cfg.settings)[0]
    return cfg, (q, k, v), g, ref


def test_c1_partition_bit_exact(c1_run):
    _, _, g, ref = c1_run
    assert np.array_equal(g["key_labels"][0], ref.key_labels)
    assert np.array_equal(g["q_labels"][0], ref.q_labels)
    assert np.array_equal(g["key_perm"][0], ref.key_perm)
    assert np.array_equal(g["q_perm"][0], ref.q_perm)
    assert np.array_equal(g["key_off"][0], ref.key_off)
    assert np.array_equal(g["q_off"][0], ref.q_off)


def test_c1_routing_and_probes_bit_exact(c1_run):
    _, _, g, ref = c1_run
    assert np.array_equal(g["blocks"][0], ref.blocks)
    assert np.array_equal(g["probe_pos"][0], ref.probe_pos)
    assert np.array_equal(g["probe_orig"][0], ref.probe_orig)


def test_c1_centroids(c1_run):
    _, (q, k, _), g, ref = c1_run
    ck = orc.group_means(k[0], ref.key_labels, 16)
    cq = orc.group_means(q[0], ref.q_labels, 16)
    assert np.allclose(g["key_centroids"][0], ck, rtol=0, atol=1e-12)
    assert np.allclose(g["q_centroids"][0], cq, rtol=0, atol=1e-12)


def test_c1_sparse_output(c1_run):
    _, _, g, ref = c1_run
    check_close(g["o_sparse"][0], ref.o_sparse, "O_s", rel=3e-3, out_rel=2.0 ** -24)


def test_c1_probe_rows(c1_run):
    _, _, g, ref = c1_run
    assert rel_fro(g["x"][0], ref.x) < 1e-4
    assert max_abs(g["y"][0], ref.y) < 1e-4 * max(1.0, np.abs(ref.x).max())


def test_c1_fit_given_gpu_probes(c1_run):
    cfg, _, g, _ = c1_run
    st = cfg.settings
    bm, bv = orc.probe_fit(g["x"][0].astype(np.float64), g["y"][0].astype(np.float64),
                           st.ridge_lambda, st.corr_rank)
    assert max_abs(g["b_mat"][0], bm) < 1e-9 * max(1.0, np.abs(bm).max())
    assert max_abs(g["b_vec"][0], bv) < 1e-9 * max(1.0, np.abs(bv).max())


def test_c1_final_output(c1_run):
    _, _, g, ref = c1_run
    check_close(g["o"][0], ref.o, "O", out_rel=2.0 ** -24)
    st = g["stats"]
    say(f"C1 stats {st}")
    assert st["routed_pairs"] == sum(
        int(np.diff(ref.q_off)[i]) * int(sum(np.diff(ref.key_off)[j] for j in ref.blocks[i] if j >= 0))
        for i in range(16))


def test_c1_deterministic(spr, c1_run):
    cfg, (q, k, v), g, _ = c1_run
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings)
    g2 = run_gpu_call(ctx, q, k, v, "f32")
    for key in ("key_labels", "q_labels", "blocks", "probe_pos", "o_sparse", "x", "y", "o"):
        assert np.array_equal(g[key], g2[key]), key


def test_c1_dense_between_partition_and_route(spr, c1_run):
    """An fp32 context's dense entry point rewrites the bf16 copies of its inputs; called
    between the partition and the route stage it must wait for the partition's K permute
    (side stream), so the call's results stay bit-identical to the plain sequence."""
    import torch
    cfg, (q, k, v), g, _ = c1_run
    say("C1 dense call between partition and route (fp32 context)")
    q2, k2, v2 = _random_qkv(1, cfg.n, cfg.d, seed=7)
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    od = torch.empty_like(qd)
    ctx.sparsepr_partition(qd, kd)
    o_dense = from_dev(ctx.sparsepr_dense_attn(to_dev(q2, "f32"), to_dev(k2, "f32"),
                                               to_dev(v2, "f32")))
    ctx.sparsepr_route(qd, kd, vd)
    ctx.sparsepr_sparse_attn()
    ctx.sparsepr_probe_fit()
    ctx.sparsepr_correct(od)
    torch.cuda.synchronize()
    assert np.array_equal(ctx.sparsepr_get_sparse_out().astype(np.float64), g["o_sparse"])
    assert np.array_equal(from_dev(od), g["o"])
    check_close(o_dense[0], orc.dense_attention(q2[0], k2[0], v2[0]), "dense in between",
                out_rel=2.0 ** -24)


# ---------------------------------------------------------------- invariants ---
def _c1_variant(spr, **over):
    cfg = get_config("C1")
    q, k, v = make_inputs(cfg)
    ctx = spr.SparsePR.from_settings(1, cfg.n, cfg.d, spr.F32, cfg.settings, **over)
    return cfg, (q, k, v), run_gpu_call(ctx, q, k, v, "f32")


def test_no_probes_means_no_correction(spr):
    say("C1 P=0")
    cfg, _, g = _c1_variant(spr, probes=0)
    perm = g["q_perm"][0]
    o_s = np.empty_like(g["o_sparse"][0])
    o_s[perm] = g["o_sparse"][0]
    assert np.array_equal(g["o"][0].astype(np.float32), o_s.astype(np.float32))


def test_full_density_is_dense(spr):
    say("C1 rho=1")
    cfg, (q, k, v), g = _c1_variant(spr, density=1.0)
    assert np.all(g["blocks"][0] >= 0) or g["blocks"].shape[-1] == 16
    dense = orc.dense_attention(q[0], k[0], v[0])
    check_close(g["o"][0], dense, "O at rho=1", out_rel=2.0 ** -24)
    assert np.abs(g["y"][0]).max() == 0.0
    assert np.all(g["b_mat"][0] == 0) and np.all(g["b_vec"][0] == 0)


def test_all_rows_probed_is_dense(spr):
    say("C1 P=N")
    cfg, (q, k, v), g = _c1_variant(spr, probes=2048)
    dense = orc.dense_attention(q[0], k[0], v[0])
    check_close(g["o"][0], dense, "O at P=N", rel=1e-4, mabs=1e-3, out_rel=2.0 ** -24)


# ------------------------------------------------------------ degenerate data ---
def test_degenerate_inputs_stay_finite_and_match(spr):
    say("degenerate inputs")
    rng = np.random.default_rng(5)
    n, d = 500, 64
    q = bf16_round(rng.standard_normal((1, n, d)))
    k = np.repeat(bf16_round(rng.standard_normal((1, 1, d))), n, axis=1)   # all keys equal
    v = bf16_round(rng.standard_normal((1, n, d)))
    q[0, 250:] = q[0, :250]                                               # duplicated queries
    kw = dict(n_sample=64, key_rank=8, kv_groups=8, q_groups=10, kmeans_iters=3, density=0.5,
              probes=20, ridge_lambda=1e-3, corr_rank=4)
    ctx = spr.SparsePR(spr.make_params(1, n, d, spr.F32, **kw))
    g = run_gpu_call(ctx, q, k, v, "f32")
    ref = orc.oracle_head(q[0], k[0], v[0], **kw)
    assert np.all(np.isfinite(g["o"]))
    assert np.array_equal(g["key_labels"][0], ref.key_labels)
    assert np.array_equal(g["q_labels"][0], ref.q_labels)
    assert np.array_equal(g["blocks"][0], ref.blocks)
    check_close(g["o"][0], ref.o, "O degenerate", out_rel=2.0 ** -24)


def test_single_group_each_side(spr):
    say("G=1")
    q, k, v = _random_qkv(1, 700, 128, seed=3)
    kw = dict(n_sample=100, key_rank=32, kv_groups=1, q_groups=1, kmeans_iters=2, density=1.0,
              probes=7, ridge_lambda=1e-3, corr_rank=2)
    ctx = spr.SparsePR(spr.make_params(1, 700, 128, spr.BF16, **kw))
    g = run_gpu_call(ctx, q, k, v, "bf16")
    assert np.all(g["key_labels"] == 0) and np.all(g["q_labels"] == 0)
    check_close(g["o"][0], orc.dense_attention(q[0], k[0], v[0]), "O G=1")


# ------------------------------------------------------------ ABI on device ---
def test_stage_order_and_bad_pointers(spr):
    import torch
    q, k, v = _random_qkv(1, 256, 64, seed=9)
    ctx = spr.SparsePR(spr.make_params(1, 256, 64, spr.BF16, kv_groups=4, q_groups=4,
                                       density=0.5, probes=8, corr_rank=2))
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    with pytest.raises(spr.SparsePRError) as e:
        ctx.sparsepr_route(qd, kd, vd)
    assert e.value.status == 5
    with pytest.raises(spr.SparsePRError) as e:
        ctx.sparsepr_sparse_attn()
    assert e.value.status == 5
    st = torch.cuda.current_stream().cuda_stream
    assert spr.lib.sparsepr_partition(ctx._ctx, qd.data_ptr() + 2, kd.data_ptr(), st) == 1
    assert spr.lib.sparsepr_partition(ctx._ctx, None, kd.data_ptr(), st) == 1
    ctx.sparsepr_partition(qd, kd)
    ctx.sparsepr_route(qd, kd, vd)
    ctx.sparsepr_sparse_attn()
    ctx.sparsepr_probe_fit()
    od = torch.empty_like(qd)
    ctx.sparsepr_correct(od)
    torch.cuda.synchronize()
    assert torch.isfinite(od.float()).all()
