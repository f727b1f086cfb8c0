"""sparsepr_dense_attn_noalloc: dense attention with no device allocation (its work-unit
metadata in the library's static scratch), called through the C ABI. It launches the same
kernel as sparsepr_dense_attn on a bf16 context, so the two outputs must be identical bit for
bit; both are also checked on sampled rows against the plain fp64 softmax(QK^T/sqrt(d))V.
Two calls in a row, the second smaller (fewer heads, shorter, d = 64), so the second call
runs on scratch the first one left behind."""
import math

import numpy as np
import pytest

import oracle as orc
from synthetic import bf16_round
from tests.gpu_common import check_close, from_dev, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _qkv(h, n, d, seed):
    rng = np.random.default_rng(seed)
    q = bf16_round(rng.standard_normal((h, n, d)) * math.sqrt(3.0))
    k = bf16_round(rng.standard_normal((h, n, d)) * math.sqrt(3.0))
    v = bf16_round(rng.standard_normal((h, n, d)))
    return q, k, v


def test_noalloc_dense_matches_the_context_dense_twice(spr):
    import torch
    # second call smaller: fewer heads, a ragged length (not a multiple of 256), d = 64
    for h, n, d, seed in ((3, 9000, 128, 61), (2, 1337, 64, 62)):
        say(f"no-alloc dense: heads={h} n={n} d={d}")
        q, k, v = _qkv(h, n, d, seed)
        qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
        o_na = torch.full_like(qd, float("nan"))
        spr.sparsepr_dense_attn_noalloc(qd, kd, vd, o_na)
        ctx = spr.SparsePR(spr.make_params(h, n, d, spr.BF16, kv_groups=1, q_groups=1, density=1.0,
                                           probes=0, corr_rank=0, n_sample=min(128, n),
                                           key_rank=min(32, d)))
        o_ctx = ctx.sparsepr_dense_attn(qd, kd, vd)
        torch.cuda.synchronize()
        assert torch.equal(o_na.view(torch.int16), o_ctx.view(torch.int16)), "not bit-identical"
        got = from_dev(o_na)
        rows = np.unique(np.concatenate([np.arange(0, n, 53), [n - 1]]))
        for i in range(h):
            ref = orc.dense_attention(q[i][rows], k[i], v[i])
            check_close(got[i][rows], ref, f"no-alloc dense h{i} n={n} d={d}")
        ctx.close()

