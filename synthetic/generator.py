"""Seeded spatio-temporal Gaussian-mixture Q/K/V, shaped like one video-DiT
self-attention call.

Recipe (every head independent, drawn from its own child stream):
  * tokens sit on a raster grid n = (t*Hp + y)*Wp + x;
  * a smooth field f(t,y,x) (four random sinusoids) is rank-transformed and cut
    at cumulative component weights, so every component is one smooth
    space-time region whose size is exactly its mixture weight (equal weights,
    or a Zipf law for heavy-tailed region sizes);
  * queries and keys of a token are its component mean plus N(0, 0.3^2) noise
    (the mean is shared by Q and K, so tokens attend to their own region); values
    use separate means; optional temporal drift of the means across frames;
  * one Haar rotation is applied to Q and K (logits unchanged), another to V;
  * Q and K are scaled so that q.k/sqrt(d) has the requested standard deviation;
  * values are rounded to bf16 (round-to-nearest-even) and returned as float32.

Nothing here implements any step of the attention method itself.
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .configs import WorkloadConfig

SEED_BASE = 20260820
STEP_SEED_BASE = 20261203        # the second noise draw of make_step_inputs
NOISE_STD = 0.3
DRIFT_STD = 0.05
N_SCALE_PAIRS = 4096


def token_grid(frames: int, rows: int, cols: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(t, y, x) of every token in raster order; N = frames * rows * cols."""
    n = np.arange(frames * rows * cols, dtype=np.int64)
    x = n % cols
    y = (n // cols) % rows
    t = n // (cols * rows)
    return t, y, x


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even); returned as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def _haar_rotation(rng: np.random.Generator, d: int) -> np.ndarray:
    a = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    return qm * np.sign(np.diag(rm))[None, :]


def _component_map(rng: np.random.Generator, cfg: WorkloadConfig) -> np.ndarray:
    t, y, x = token_grid(cfg.frames, cfg.patch_rows, cfg.patch_cols)
    grid = np.stack([t / cfg.frames, y / cfg.patch_rows, x / cfg.patch_cols], axis=1)
    freqs = np.array([(a, b, c) for a in range(3) for b in range(3) for c in range(3)
                      if (a, b, c) != (0, 0, 0)], dtype=np.float64)
    f = np.zeros(cfg.n)
    for _ in range(4):
        u = freqs[rng.integers(len(freqs))]
        amp = rng.uniform(0.5, 1.0)
        phase = rng.uniform(0.0, 2.0 * np.pi)
        f += amp * np.sin(2.0 * np.pi * (grid @ u) + phase)
    order = np.argsort(f, kind="stable")          # ties broken by token index
    rank = np.empty(cfg.n, dtype=np.int64)
    rank[order] = np.arange(cfg.n)
    c = np.arange(cfg.components, dtype=np.float64)
    w = np.ones(cfg.components) if cfg.zipf is None else (c + 1.0) ** (-cfg.zipf)
    bounds = np.floor(cfg.n * np.cumsum(w) / w.sum()).astype(np.int64)
    bounds[-1] = cfg.n
    return np.searchsorted(bounds, rank, side="right")


def make_head(cfg: WorkloadConfig, rng: np.random.Generator,
              logit_std: float, step_mix=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One head's (q, k, v), each [N, d] float32 holding bf16-representable values.
    step_mix = (alt_rng, c, s): every token's noise becomes c n + s n' with n' drawn from
    alt_rng (the same structure with the fine detail turned by an angle; c = 1, s = 0 is
    the plain head)."""
    d, n = cfg.d, cfg.n

    def noise():
        z = rng.standard_normal((n, d))
        if step_mix is not None:
            alt, c, s_ = step_mix
            z = c * z + s_ * alt.standard_normal((n, d))
        return NOISE_STD * z

    comp = _component_map(rng, cfg)
    mu = rng.standard_normal((cfg.components, d))
    nu = rng.standard_normal((cfg.components, d))
    if cfg.drift:
        delta = DRIFT_STD * rng.standard_normal((cfg.components, d))
        t, _, _ = token_grid(cfg.frames, cfg.patch_rows, cfg.patch_cols)
        mean_qk = mu[comp] + t[:, None] * delta[comp]
    else:
        mean_qk = mu[comp]
    q = mean_qk + noise()
    k = mean_qk + noise()
    del mean_qk
    v = nu[comp] + noise()
    rot_qk = _haar_rotation(rng, d)
    rot_v = _haar_rotation(rng, d)
    q = q @ rot_qk
    k = k @ rot_qk
    v = v @ rot_v
    i = rng.integers(n, size=N_SCALE_PAIRS)
    j = rng.integers(n, size=N_SCALE_PAIRS)
    sigma_hat = np.std(np.sum(q[i] * k[j], axis=1) / np.sqrt(d))
    scale = np.sqrt(logit_std / sigma_hat)
    return bf16_round(q * scale), bf16_round(k * scale), bf16_round(v)


def make_step_inputs(cfg: WorkloadConfig, step: int, theta: float = 0.1,
                     heads: Optional[Iterable[int]] = None
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Inputs of successive calls of one layer (a stand-in for successive denoising steps):
    the same components, means, rotations and layout as make_inputs, with each token's noise
    turned by theta * step radians towards an independent draw. Step 0 is make_inputs."""
    root = np.random.Generator(np.random.PCG64(SEED_BASE + cfg.index))
    alt_root = np.random.Generator(np.random.PCG64(STEP_SEED_BASE + cfg.index))
    children = root.spawn(cfg.heads)
    alts = alt_root.spawn(cfg.heads)
    c, s = float(np.cos(theta * step)), float(np.sin(theta * step))
    sel = list(range(cfg.heads)) if heads is None else list(heads)
    shape = (len(sel), cfg.n, cfg.d)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for out_h, h in enumerate(sel):
        q[out_h], k[out_h], v[out_h] = make_head(cfg, children[h], cfg.head_logit_std(h),
                                                 step_mix=(alts[h], c, s))
    return q, k, v


def make_inputs(cfg: WorkloadConfig, heads: Optional[Iterable[int]] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(q, k, v) as [H_sel, N, d] float32 arrays of bf16-representable values.

    Head h always comes from child stream h of the workload's seed, so any subset
    of heads can be generated on its own and matches the full call's heads.
    """
    root = np.random.Generator(np.random.PCG64(SEED_BASE + cfg.index))
    children = root.spawn(cfg.heads)
    sel = list(range(cfg.heads)) if heads is None else list(heads)
    shape = (len(sel), cfg.n, cfg.d)
    q = np.empty(shape, np.float32)
    k = np.empty(shape, np.float32)
    v = np.empty(shape, np.float32)
    for out_h, h in enumerate(sel):
        q[out_h], k[out_h], v[out_h] = make_head(cfg, children[h], cfg.head_logit_std(h))
    return q, k, v
