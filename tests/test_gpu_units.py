"""Work units of the sparse kernel: 256-row chunks first, then 128-row units.

By default the sparse stage runs every whole 256-row chunk of a query group, and a rest of
more than 128 rows, as one unit of an 8-wave block, and a shorter rest as a 128-row unit of
a 4-wave block in a second launch beside the first; SPARSEPR_F_UNIFORM_UNITS cuts every
group into 128-row units. A wave's 32 rows start at the
same offset inside their group either way and walk the same 64-key tiles of the group's
routed union, so the two must agree bit for bit, in the sparse output and in the corrected
output. The default path is also checked against the oracle's sparse attention on the
library's own partition (the same routing, block lists and group-major rows), at d = 64 and
d = 128, with query groups large enough that several whole chunks and a ragged rest occur.
"""
import numpy as np
import pytest

import oracle as orc
from synthetic import get_config, make_inputs
from tests.gpu_common import check_close, run_gpu_call, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spr():
    import torch
    assert torch.cuda.is_available()
    import free_block_sparse_eigen_amd as mod
    return mod


def _oracle_sparse(q, k, v, out, h, settings):
    """The oracle's sparse attention of head h over the library's partition and routing, in
    group-major row order (the order of the library's sparse output)."""
    kl, ql = out["key_labels"][h], out["q_labels"][h]
    kperm, koff = orc.group_major(kl, settings.kv_groups)
    qperm, qoff = orc.group_major(ql, settings.q_groups)
    assert np.array_equal(kperm, out["key_perm"][h]) and np.array_equal(qperm, out["q_perm"][h])
    qh, kh, vh = (np.asarray(x, np.float64) for x in (q[h], k[h], v[h]))
    return orc.sparse_attention(qh[qperm], kh[kperm], vh[kperm], qoff, koff, out["blocks"][h]), qoff


CASES = [
    # C1-shaped (fp32, d = 64) with 5 query groups (groups of about 400 rows) and 64 heads:
    # 2^17 query rows, the smallest call that takes 256-row units
    ("C1", 64, dict(q_groups=5)),
    # C2 (bf16, d = 128): 128 groups of about 256 rows, five of its heads (163,800 rows)
    ("C2", [0, 3, 5, 7, 11], {}),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,heads,over", CASES, ids=[c[0] for c in CASES])
def test_big_units_match_uniform_units_and_the_oracle(spr, name, heads, over):
    cfg = get_config(name)
    if over:
        cfg = cfg.with_settings(**over)
    if isinstance(heads, int):
        cfg = cfg.with_heads(heads)
        heads = None
    st = cfg.settings
    q, k, v = make_inputs(cfg, heads=heads)
    H = q.shape[0]
    dt = spr.BF16 if cfg.dtype == "bf16" else spr.F32
    say(f"[units] {name} H={H} N={cfg.n} d={cfg.d} Gq={st.q_groups}: default units")
    ctx = spr.SparsePR.from_settings(H, cfg.n, cfg.d, dt, st)
    a = run_gpu_call(ctx, q, k, v, cfg.dtype)
    ctx.close()
    say(f"[units] {name}: uniform 128-row units")
    ctx = spr.SparsePR.from_settings(H, cfg.n, cfg.d, dt, st, flags=spr.F_UNIFORM_UNITS)
    b = run_gpu_call(ctx, q, k, v, cfg.dtype)
    ctx.close()
    for key in ("key_labels", "q_labels", "blocks", "probe_orig"):
        assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), f"{name}: {key} differs"
    assert np.array_equal(a["o_sparse"], b["o_sparse"]), f"{name}: sparse output differs"
    assert np.array_equal(a["o"], b["o"]), f"{name}: corrected output differs"
    sizes = np.concatenate([np.diff(a["q_off"][h]) for h in range(H)])
    rest = sizes % 256
    assert (sizes >= 256).any() and (rest > 128).any() and ((rest > 0) & (rest <= 128)).any(), \
        f"{name}: the groups do not cover whole chunks and both kinds of rest"
    for h in range(min(H, 2)):
        ref, qoff = _oracle_sparse(q, k, v, a, h, st)
        assert np.array_equal(qoff, a["q_off"][h])
        check_close(a["o_sparse"][h], ref, f"{name} head {h} sparse output", rel=3e-3,
                    out_rel=2.0 ** -24)
    say(f"[units] {name}: bit-identical to uniform units, oracle ok on the first heads "
        f"(largest group {sizes.max()} rows)")
