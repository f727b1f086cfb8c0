"""Python binding of libsparsepr.so, the SparsePR attention-call hot path on MI355X.

Argument marshalling only: every step runs in the HIP library. Tensors are torch
tensors on the GPU (device pointers); streams are torch's current stream. Each
C entry point sparsepr_<name> has a wrapper of the same name here; `SparsePR`
bundles a context with typed getters.

The library is built in-tree by `free_block_sparse_eigen_amd.build`; importing
this package when it is missing raises immediately (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparsepr.so")

BF16, F32 = 0, 1
F_STAGE_TIMING = 1
F_RAW_KMEANS = 2      # comparison partitioner: independent Euclidean k-means of raw Q and K
F_CHECK_FINITE = 4    # count non-finite inputs and outputs on the device (sparsepr_get_stats)
F_HOST_SOLVE = 8      # M_K eigensolve on the host instead of the device
F_SVOO = 16           # comparison partitioner: alternating Q/K co-clustering (not the method)
F_SERIAL_PARTITION = 32  # all heads of the partition on the caller's stream (default: two halves, two streams)
F_FP8_QK = 64         # experiment: the sparse kernel's logits from FP8 E4M3 Q and K (per-head scales)
F_RAW_KEY_SCREEN = 128  # the key k-means screens raw keys against W c, not their coordinates (same labels)
F_UNIFORM_UNITS = 256  # the sparse kernel in 128-row units only (default: 256-row units for whole chunks and rests over 128 rows)

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "out of memory",
          4: "HIP error", 5: "stage order", 6: "numerical failure"}

EXPORTS = [
    "sparsepr_validate", "sparsepr_workspace_bytes", "sparsepr_create", "sparsepr_destroy",
    "sparsepr_status_str", "sparsepr_last_error", "sparsepr_partition", "sparsepr_route",
    "sparsepr_sparse_attn", "sparsepr_probe_fit", "sparsepr_correct", "sparsepr_attention",
    "sparsepr_dense_attn", "sparsepr_get_partition", "sparsepr_get_routing",
    "sparsepr_get_centroids", "sparsepr_get_sparse_out", "sparsepr_get_probes",
    "sparsepr_get_fit", "sparsepr_get_stats", "sparsepr_set_partition", "sparsepr_routed_count",
    "sparsepr_get_gaps", "sparsepr_get_metric", "sparsepr_dense_attn_noalloc",
    "sparsepr_reuse_route", "sparsepr_attention_reuse",
    "sparsepr_host_sym_eig_top", "sparsepr_host_key_projection",
    "sparsepr_host_probe_fit",
]


class SparsePRError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        super().__init__(f"{STATUS.get(status, status)}: {detail}" if detail else STATUS.get(status, str(status)))
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("n", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("n_sample", ctypes.c_int32),
                ("key_rank", ctypes.c_int32), ("kv_groups", ctypes.c_int32),
                ("q_groups", ctypes.c_int32), ("kmeans_iters", ctypes.c_int32),
                ("probes", ctypes.c_int32), ("corr_rank", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("density", ctypes.c_double),
                ("ridge_lambda", ctypes.c_double)]


class Stats(ctypes.Structure):
    _fields_ = [("routed_pairs", ctypes.c_int64), ("probe_pairs", ctypes.c_int64),
                ("exec_density", ctypes.c_double), ("recheck_points", ctypes.c_int64),
                ("routed_k", ctypes.c_int32), ("query_dims", ctypes.c_int32),
                ("stage_ms", ctypes.c_float * 6), ("timed_calls", ctypes.c_int32),
                ("nonfinite_inputs", ctypes.c_int64), ("nonfinite_outputs", ctypes.c_int64),
                ("metric_gap_min", ctypes.c_double), ("resid_gap_min", ctypes.c_double)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python free_block_sparse_eigen_amd/build.py`")
# torch first: its bundled HIP runtime has the same soname as the system one, so the
# library then binds to that runtime. Loaded the other way round, the process would hold
# two HIP runtimes, and torch's device pointers and streams would be foreign to ours.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int32
_ctx = ctypes.c_void_p
_sigs = {
    "sparsepr_validate": (_I, [ctypes.POINTER(Params)]),
    "sparsepr_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "sparsepr_create": (_I, [ctypes.POINTER(Params), ctypes.POINTER(_ctx)]),
    "sparsepr_destroy": (None, [_ctx]),
    "sparsepr_status_str": (ctypes.c_char_p, [_I]),
    "sparsepr_last_error": (ctypes.c_char_p, [_ctx]),
    "sparsepr_partition": (_I, [_ctx, _P, _P, _P]),
    "sparsepr_route": (_I, [_ctx, _P, _P, _P, _P]),
    "sparsepr_sparse_attn": (_I, [_ctx, _P]),
    "sparsepr_probe_fit": (_I, [_ctx, _P]),
    "sparsepr_correct": (_I, [_ctx, _P, _P]),
    "sparsepr_attention": (_I, [_ctx, _P, _P, _P, _P, _P]),
    "sparsepr_dense_attn": (_I, [_ctx, _P, _P, _P, _P, _P]),
    "sparsepr_get_partition": (_I, [_ctx, _P, _P, _P, _P, _P, _P, _I, _P]),
    "sparsepr_get_routing": (_I, [_ctx, _P, _P, _P, _I, _P]),
    "sparsepr_get_centroids": (_I, [_ctx, _P, _P, _I, _P]),
    "sparsepr_get_sparse_out": (_I, [_ctx, _P, _I, _P]),
    "sparsepr_get_probes": (_I, [_ctx, _P, _P, _I, _P]),
    "sparsepr_get_fit": (_I, [_ctx, _P, _P, _I, _P]),
    "sparsepr_get_stats": (_I, [_ctx, ctypes.POINTER(Stats)]),
    "sparsepr_set_partition": (_I, [_ctx, _P, _P, _P, _P, _I, _P]),
    "sparsepr_routed_count": (_I, [ctypes.POINTER(Params)]),
    "sparsepr_get_gaps": (_I, [_ctx, _P, _P, _I, _P]),
    "sparsepr_get_metric": (_I, [_ctx, _P, _P, _I, _P]),
    "sparsepr_dense_attn_noalloc": (_I, [_I, _I, _I, _P, _P, _P, _P, _P]),
    "sparsepr_reuse_route": (_I, [_ctx, _P, _P, _P, _P]),
    "sparsepr_attention_reuse": (_I, [_ctx, _P, _P, _P, _P, _P]),
    "sparsepr_host_sym_eig_top": (_I, [_I, _P, _I, _P, _P]),
    "sparsepr_host_key_projection": (_I, [_I, _P, _I, _P]),
    "sparsepr_host_probe_fit": (_I, [_I, _I, _P, _P, ctypes.c_double, _I, _P, _P]),
}
for _name, (_res, _args) in _sigs.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _check(status: int, ctx=None) -> None:
    if status != 0:
        detail = lib.sparsepr_last_error(ctx).decode()   # ctx None: why create failed
        raise SparsePRError(status, detail)


def _np_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def make_params(heads: int, n: int, d: int, dtype: int = BF16, *, n_sample: int = 128,
                key_rank: Optional[int] = None, kv_groups: int, q_groups: int,
                kmeans_iters: int = 5, density: float, probes: int, ridge_lambda: float = 1e-3,
                corr_rank: int, flags: int = 0) -> Params:
    return Params(heads=heads, n=n, d=d, dtype=dtype, n_sample=min(n_sample, n),
                  key_rank=key_rank if key_rank is not None else d // 4, kv_groups=kv_groups,
                  q_groups=q_groups, kmeans_iters=kmeans_iters, probes=probes,
                  corr_rank=corr_rank, flags=flags, density=density, ridge_lambda=ridge_lambda)


# ---------------------------------------------------------------- host solves ---
def sparsepr_validate(p: Params) -> int:
    return lib.sparsepr_validate(ctypes.byref(p))


def sparsepr_workspace_bytes(p: Params) -> int:
    return lib.sparsepr_workspace_bytes(ctypes.byref(p))


def sparsepr_routed_count(p: Params) -> int:
    k = lib.sparsepr_routed_count(ctypes.byref(p))
    if k < 0:
        raise SparsePRError(-k, "invalid parameters")
    return k


def sparsepr_host_sym_eig_top(a: np.ndarray, r: int):
    a = np.ascontiguousarray(a, np.float64)
    n = a.shape[0]
    lam = np.zeros(max(r, 1))
    vec = np.zeros((n, max(r, 1)))
    _check(lib.sparsepr_host_sym_eig_top(n, _np_ptr(a), r, _np_ptr(lam), _np_ptr(vec)))
    return lam[:r], vec[:, :r]


def sparsepr_host_key_projection(m_k: np.ndarray, r: int) -> np.ndarray:
    m_k = np.ascontiguousarray(m_k, np.float64)
    w = np.zeros((m_k.shape[0], r))
    _check(lib.sparsepr_host_key_projection(m_k.shape[0], _np_ptr(m_k), r, _np_ptr(w)))
    return w


def sparsepr_host_probe_fit(x: np.ndarray, y: np.ndarray, lam: float, rank: int):
    x = np.ascontiguousarray(x, np.float64)
    y = np.ascontiguousarray(y, np.float64)
    p, d = x.shape
    bm = np.zeros((d, d))
    bv = np.zeros(d)
    _check(lib.sparsepr_host_probe_fit(p, d, _np_ptr(x) if p else None, _np_ptr(y) if p else None,
                                       float(lam), rank, _np_ptr(bm), _np_ptr(bv)))
    return bm, bv


# ------------------------------------------------------------ device context ---
def _stream_ptr(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _tptr(t) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous GPU tensor")
    return t.data_ptr()


def sparsepr_dense_attn_noalloc(q, k, v, o, stream=None):
    """Dense attention of bf16 q, k, v [H][n][d] into the caller's o with no device
    allocation (no context; the library's static scratch)."""
    import torch
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16 or t.dim() != 3 or tuple(t.shape) != tuple(q.shape):
            raise ValueError("q, k, v and o must be bf16 [H][n][d] of one shape")
    h, n, d = q.shape
    _check(lib.sparsepr_dense_attn_noalloc(h, n, d, _tptr(q), _tptr(k), _tptr(v), _tptr(o),
                                           _stream_ptr(stream)))
    return o


class SparsePR:
    """One library context (workspace for fixed shapes and settings)."""

    def __init__(self, params: Params):
        self.params = params
        self._ctx = _ctx()
        _check(lib.sparsepr_create(ctypes.byref(params), ctypes.byref(self._ctx)))
        self.k = sparsepr_routed_count(params)

    @classmethod
    def from_settings(cls, heads: int, n: int, d: int, dtype: int, settings, flags: int = 0,
                      **overrides) -> "SparsePR":
        kw = dict(n_sample=settings.n_sample, key_rank=settings.key_rank,
                  kv_groups=settings.kv_groups, q_groups=settings.q_groups,
                  kmeans_iters=settings.kmeans_iters, density=settings.density,
                  probes=settings.probes, ridge_lambda=settings.ridge_lambda,
                  corr_rank=settings.corr_rank, flags=flags)
        kw.update(overrides)
        return cls(make_params(heads, n, d, dtype, **kw))

    def close(self) -> None:
        if self._ctx:
            lib.sparsepr_destroy(self._ctx)
            self._ctx = _ctx()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _c(self, status: int) -> None:
        _check(status, self._ctx)

    # the five stages
    def sparsepr_partition(self, q, k, stream=None):
        self._c(lib.sparsepr_partition(self._ctx, _tptr(q), _tptr(k), _stream_ptr(stream)))

    def sparsepr_route(self, q, k, v, stream=None):
        self._c(lib.sparsepr_route(self._ctx, _tptr(q), _tptr(k), _tptr(v), _stream_ptr(stream)))

    def sparsepr_sparse_attn(self, stream=None):
        self._c(lib.sparsepr_sparse_attn(self._ctx, _stream_ptr(stream)))

    def sparsepr_probe_fit(self, stream=None):
        self._c(lib.sparsepr_probe_fit(self._ctx, _stream_ptr(stream)))

    def sparsepr_correct(self, o, stream=None):
        self._c(lib.sparsepr_correct(self._ctx, _tptr(o), _stream_ptr(stream)))

    def sparsepr_attention(self, q, k, v, o=None, stream=None):
        import torch
        o = torch.empty_like(q) if o is None else o
        self._c(lib.sparsepr_attention(self._ctx, _tptr(q), _tptr(k), _tptr(v), _tptr(o),
                                       _stream_ptr(stream)))
        return o

    def sparsepr_reuse_route(self, q, k, v, stream=None):
        self._c(lib.sparsepr_reuse_route(self._ctx, _tptr(q), _tptr(k), _tptr(v), _stream_ptr(stream)))

    def sparsepr_attention_reuse(self, q, k, v, o=None, stream=None):
        import torch
        o = torch.empty_like(q) if o is None else o
        self._c(lib.sparsepr_attention_reuse(self._ctx, _tptr(q), _tptr(k), _tptr(v), _tptr(o),
                                             _stream_ptr(stream)))
        return o

    def sparsepr_dense_attn(self, q, k, v, o=None, stream=None):
        import torch
        o = torch.empty_like(q) if o is None else o
        self._c(lib.sparsepr_dense_attn(self._ctx, _tptr(q), _tptr(k), _tptr(v), _tptr(o),
                                        _stream_ptr(stream)))
        return o

    def sparsepr_set_partition(self, q, k, key_labels: np.ndarray, q_labels: np.ndarray,
                               stream=None):
        kl = np.ascontiguousarray(key_labels, np.int32)
        ql = np.ascontiguousarray(q_labels, np.int32)
        self._c(lib.sparsepr_set_partition(self._ctx, _tptr(q), _tptr(k), _np_ptr(kl), _np_ptr(ql),
                                           1, _stream_ptr(stream)))

    # inspection (host copies as numpy arrays)
    def sparsepr_get_partition(self, stream=None):
        p = self.params
        hn = (p.heads, p.n)
        out = {name: np.empty(hn, np.int32) for name in ("key_labels", "q_labels", "key_perm", "q_perm")}
        out["key_off"] = np.empty((p.heads, p.kv_groups + 1), np.int32)
        out["q_off"] = np.empty((p.heads, p.q_groups + 1), np.int32)
        self._c(lib.sparsepr_get_partition(
            self._ctx, *[_np_ptr(out[n]) for n in ("key_labels", "q_labels", "key_perm", "q_perm",
                                                   "key_off", "q_off")], 1, _stream_ptr(stream)))
        return out

    def sparsepr_get_routing(self, stream=None):
        p = self.params
        blocks = np.empty((p.heads, p.q_groups, self.k), np.int32)
        po = np.empty((p.heads, max(p.probes, 1)), np.int32)
        pp = np.empty((p.heads, max(p.probes, 1)), np.int32)
        self._c(lib.sparsepr_get_routing(self._ctx, _np_ptr(blocks), _np_ptr(po), _np_ptr(pp), 1,
                                         _stream_ptr(stream)))
        return {"blocks": blocks, "probe_orig": po[:, :p.probes], "probe_pos": pp[:, :p.probes]}

    def sparsepr_get_metric(self, stream=None):
        p = self.params
        mk = np.empty((p.heads, p.d, p.d))
        w = np.empty((p.heads, p.d, p.key_rank))
        self._c(lib.sparsepr_get_metric(self._ctx, _np_ptr(mk), _np_ptr(w), 1, _stream_ptr(stream)))
        return mk, w

    def sparsepr_get_centroids(self, stream=None):
        p = self.params
        ck = np.empty((p.heads, p.kv_groups, p.d))
        cq = np.empty((p.heads, p.q_groups, p.d))
        self._c(lib.sparsepr_get_centroids(self._ctx, _np_ptr(ck), _np_ptr(cq), 1, _stream_ptr(stream)))
        return ck, cq

    def sparsepr_get_sparse_out(self, stream=None):
        p = self.params
        o = np.empty((p.heads, p.n, p.d), np.float32)
        self._c(lib.sparsepr_get_sparse_out(self._ctx, _np_ptr(o), 1, _stream_ptr(stream)))
        return o

    def sparsepr_get_probes(self, stream=None):
        p = self.params
        x = np.zeros((p.heads, p.probes, p.d), np.float32)
        y = np.zeros((p.heads, p.probes, p.d), np.float32)
        self._c(lib.sparsepr_get_probes(self._ctx, _np_ptr(x), _np_ptr(y), 1, _stream_ptr(stream)))
        return x, y

    def sparsepr_get_fit(self, stream=None):
        p = self.params
        bm = np.empty((p.heads, p.d, p.d))
        bv = np.empty((p.heads, p.d))
        self._c(lib.sparsepr_get_fit(self._ctx, _np_ptr(bm), _np_ptr(bv), 1, _stream_ptr(stream)))
        return bm, bv

    def sparsepr_get_gaps(self, stream=None):
        h = self.params.heads
        mg, rg = np.empty(h), np.empty(h)
        self._c(lib.sparsepr_get_gaps(self._ctx, _np_ptr(mg), _np_ptr(rg), 1, _stream_ptr(stream)))
        return mg, rg

    def sparsepr_get_stats(self) -> dict:
        s = Stats()
        self._c(lib.sparsepr_get_stats(self._ctx, ctypes.byref(s)))
        return {"routed_pairs": s.routed_pairs, "probe_pairs": s.probe_pairs,
                "exec_density": s.exec_density, "recheck_points": s.recheck_points,
                "routed_k": s.routed_k, "query_dims": s.query_dims,
                "stage_ms": list(s.stage_ms), "timed_calls": s.timed_calls,
                "nonfinite_inputs": s.nonfinite_inputs, "nonfinite_outputs": s.nonfinite_outputs,
                "metric_gap_min": s.metric_gap_min, "resid_gap_min": s.resid_gap_min}
