"""The five workload shapes and their SparsePR settings.

Shapes follow the video-DiT token grids (frames x patch rows x patch columns,
raster order), as in the token-count arithmetic of the framerc.cn post
"SparsePR稀疏注意力：无训练加速视频生成与世界模型推理", section 1.1.
Where a setting is given only for the tiny workload, the others inherit it.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class SparsePRSettings:
    n_sample: int          # M_s, sampled queries for the key metric
    key_rank: int          # r_K, leading metric eigenvectors kept
    kv_groups: int         # G_k
    q_groups: int          # G_q
    density: float         # rho, fraction of key groups routed per query group
    probes: int            # P, exact probe rows per head
    ridge_lambda: float    # lambda
    corr_rank: int         # r, rank of the residual subspace
    kmeans_iters: int = 5  # T


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    index: int                      # 1..5, also selects the seed
    heads: int
    frames: int
    patch_rows: int
    patch_cols: int
    d: int
    dtype: str                      # "f32" (bf16-representable values) or "bf16"
    components: int                 # mixture components
    drift: bool                     # temporal drift of component means
    zipf: Optional[float]           # component-size law exponent, None = equal sizes
    logit_std: Tuple[float, ...]    # per-head target logit std (one value = all heads)
    settings: SparsePRSettings = field(default=None)
    densities: Tuple[float, ...] = ()  # density sweep (bench); settings.density is the default

    @property
    def n(self) -> int:
        return self.frames * self.patch_rows * self.patch_cols

    def head_logit_std(self, h: int) -> float:
        if len(self.logit_std) == 1:
            return self.logit_std[0]
        return self.logit_std[h]

    def with_settings(self, **kw) -> "WorkloadConfig":
        return replace(self, settings=replace(self.settings, **kw))

    def with_heads(self, heads: int) -> "WorkloadConfig":
        return replace(self, heads=heads)


CONFIGS = {
    "C1": WorkloadConfig(
        name="tiny-fp32", index=1, heads=1, frames=8, patch_rows=16, patch_cols=16, d=64,
        dtype="f32", components=16, drift=False, zipf=None, logit_std=(3.0,),
        settings=SparsePRSettings(n_sample=128, key_rank=16, kv_groups=16, q_groups=16,
                                  density=0.25, probes=64, ridge_lambda=1e-3, corr_rank=8)),
    "C2": WorkloadConfig(
        name="wan2.1-1.3b-480p", index=2, heads=12, frames=21, patch_rows=30, patch_cols=52,
        d=128, dtype="bf16", components=256, drift=False, zipf=None, logit_std=(3.0,),
        settings=SparsePRSettings(n_sample=128, key_rank=32, kv_groups=128, q_groups=128,
                                  density=0.25, probes=128, ridge_lambda=1e-3, corr_rank=16)),
    "C3": WorkloadConfig(
        name="wan2.1-1.3b-720p", index=3, heads=12, frames=21, patch_rows=45, patch_cols=80,
        d=128, dtype="bf16", components=400, drift=True, zipf=None, logit_std=(3.0,),
        settings=SparsePRSettings(n_sample=128, key_rank=32, kv_groups=256, q_groups=256,
                                  density=0.26, probes=256, ridge_lambda=1e-3, corr_rank=16),
        densities=(0.15, 0.22, 0.26, 0.35, 1.0)),
    "C4": WorkloadConfig(
        name="wan2.1-14b-720p", index=4, heads=40, frames=21, patch_rows=45, patch_cols=80,
        d=128, dtype="bf16", components=400, drift=True, zipf=None,
        logit_std=tuple([5.0] * 20 + [1.5] * 20),
        settings=SparsePRSettings(n_sample=128, key_rank=32, kv_groups=256, q_groups=256,
                                  density=0.22, probes=256, ridge_lambda=1e-3, corr_rank=16)),
    "C5": WorkloadConfig(
        name="hunyuanvideo-13b-720p", index=5, heads=24, frames=33, patch_rows=45, patch_cols=80,
        d=128, dtype="bf16", components=512, drift=False, zipf=1.2, logit_std=(3.0,),
        settings=SparsePRSettings(n_sample=128, key_rank=32, kv_groups=384, q_groups=384,
                                  density=0.24, probes=384, ridge_lambda=1e-3, corr_rank=32)),
}


def get_config(name: str) -> WorkloadConfig:
    return CONFIGS[name]
