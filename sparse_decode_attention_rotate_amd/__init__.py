"""Loki sparse decode attention on AMD MI355X -- thin Python binding.

Every call below marshals torch tensors (device memory) and the current HIP
stream into the C ABI of include/loki.h, exported by the in-tree HIP library
libloki.so; all the work runs in its gfx950 kernels.  There is no CPU path:
importing this package fails if the library has not been built
(python sparse_decode_attention_rotate_amd/build.py).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libloki.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libloki.so not found at {LIB_PATH}; build it with "
        "`python sparse_decode_attention_rotate_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

F32, F16, BF16 = 0, 1, 2
FLAG_SEPARATE_KERNELS = 1
FLAG_NO_HELPERS = 2
FLAG_NO_SHARED_STREAM = 4
FLAG_SHARED_NO_WAIT = 8
FLAG_PER_HEAD_KERNEL = 16
NOALLOC_SCRATCH_BYTES = 64 << 20  # LOKI_NOALLOC_SCRATCH_BYTES of include/loki.h
DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
TORCH_DTYPE = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}
NAME_CODE = {"f32": F32, "f16": F16, "bf16": BF16}

STATUS = {0: "LOKI_OK", -1: "LOKI_EINVAL", -2: "LOKI_EUNSUPPORTED", -3: "LOKI_EWORKSPACE",
          -4: "LOKI_EHIP"}

# every symbol declared in include/loki.h
EXPORTS = ["loki_strerror", "loki_last_error", "loki_kcache_elems", "loki_workspace_bytes",
           "loki_pack_kcache", "loki_unpack_kcache", "loki_append", "loki_rotate_query",
           "loki_score", "loki_topk", "loki_attend", "loki_decode", "loki_decode_append",
           "loki_decode_plan", "loki_full_attention", "loki_prefill", "loki_pca_attention",
           "loki_calibrate_workspace_bytes", "loki_calibrate", "loki_decode_noalloc"]


class _CDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("seq_capacity", ctypes.c_int32),
                ("panel_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_uint32),
                ("out_dtype", ctypes.c_int32)]


_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_D = ctypes.POINTER(_CDesc)
_SIG = {
    "loki_strerror": ([_i], ctypes.c_char_p),
    "loki_last_error": ([], ctypes.c_char_p),
    "loki_kcache_elems": ([_D, ctypes.POINTER(_sz)], _i),
    "loki_workspace_bytes": ([_D, _i, _i, ctypes.POINTER(_sz)], _i),
    "loki_pack_kcache": ([_vp, ctypes.c_int32, _vp, _D, _vp], _i),
    "loki_unpack_kcache": ([_vp, ctypes.c_int32, _vp, _D, _vp], _i),
    "loki_append": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _D, _vp], _i),
    "loki_rotate_query": ([_vp, _vp, _vp, _D, _vp], _i),
    "loki_score": ([_vp, _vp, _i, _vp, _D, _vp], _i),
    "loki_topk": ([_vp, _i, _vp, _vp, _D, _vp], _i),
    "loki_attend": ([_vp, _vp, _vp, _vp, _vp, _i, _vp, _D, _vp, _sz, _vp], _i),
    "loki_decode": ([_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _D, _vp, _sz, _vp], _i),
    "loki_decode_append": ([_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _D, _vp, _sz,
                            _vp], _i),
    "loki_decode_plan": ([_D, _i, _i, _i, ctypes.POINTER(_i)], _i),
    "loki_full_attention": ([_vp, _vp, _vp, _vp, _vp, _D, _vp, _sz, _vp], _i),
    "loki_pca_attention": ([_vp, _vp, _vp, _vp, _i, _vp, _D, _vp, _sz, _vp], _i),
    "loki_calibrate_workspace_bytes": ([_D, ctypes.c_int32, ctypes.POINTER(_sz)], _i),
    "loki_calibrate": ([_vp, ctypes.c_int32, _vp, _vp, _D, _vp, _sz, _vp], _i),
    "loki_prefill": ([_vp, _vp, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp, _D, _vp], _i),
    "loki_decode_noalloc": ([_vp, _vp, _vp, _vp, _i, _i, _vp, _vp, _vp, _D, _vp], _i),
}
for _name, (_args, _res) in _SIG.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class LokiError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        detail = _lib.loki_last_error().decode()
        super().__init__(f"{where}: {STATUS.get(code, code)} ({detail})")


@dataclasses.dataclass(frozen=True)
class Desc:
    """Problem description (mirrors loki_desc)."""
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int
    seq_capacity: int
    panel_dim: int
    dtype: int
    softmax_scale: float = 0.0
    flags: int = 0
    out_dtype: int = F32

    def c(self) -> _CDesc:
        return _CDesc(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.seq_len,
                      self.seq_capacity, self.panel_dim, self.dtype, self.softmax_scale,
                      self.flags, self.out_dtype)

    def with_flags(self, flags: int) -> "Desc":
        return dataclasses.replace(self, flags=flags)

    def with_out_dtype(self, out_dtype: int) -> "Desc":
        return dataclasses.replace(self, out_dtype=out_dtype)

    def with_seq_len(self, s: int) -> "Desc":
        return dataclasses.replace(self, seq_len=s)

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPE[self.dtype]

    @property
    def torch_out_dtype(self) -> torch.dtype:
        return TORCH_DTYPE[self.out_dtype]


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise LokiError(rc, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be in device memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _out(desc: "Desc", out, device):
    """The attention output [B, Hq, D] in desc's output dtype (allocated if None)."""
    shp = (desc.batch, desc.n_q_heads, desc.head_dim)
    if out is None:
        return torch.empty(shp, dtype=desc.torch_out_dtype, device=device)
    _expect(out, shp, desc.torch_out_dtype, "out")
    return out


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _expect(t: torch.Tensor, shape, dtype, name: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")


def kcache_elems(desc: Desc) -> int:
    n = ctypes.c_size_t()
    _check(_lib.loki_kcache_elems(ctypes.byref(desc.c()), ctypes.byref(n)), "loki_kcache_elems")
    return n.value


def workspace_bytes(desc: Desc, d: int, k: int) -> int:
    n = ctypes.c_size_t()
    _check(_lib.loki_workspace_bytes(ctypes.byref(desc.c()), d, k, ctypes.byref(n)),
           "loki_workspace_bytes")
    return n.value


def decode_kernel(desc: Desc, d: int, k: int, append: bool = False) -> int:
    """Launch plan code of loki_decode_plan: 0 separate launches, 1 one
    workgroup per (b, kv) unit, 2 one workgroup per query head."""
    one = ctypes.c_int()
    _check(_lib.loki_decode_plan(ctypes.byref(desc.c()), d, k, int(append), ctypes.byref(one)),
           "loki_decode_plan")
    return one.value


def decode_plan(desc: Desc, d: int, k: int, append: bool = False) -> bool:
    """True when the decode step runs as one kernel launch."""
    return decode_kernel(desc, d, k, append) != 0


def empty_kcache(desc: Desc, device="cuda") -> torch.Tensor:
    return torch.zeros(kcache_elems(desc), dtype=desc.torch_dtype, device=device)


def empty_vcache(desc: Desc, device="cuda") -> torch.Tensor:
    return torch.zeros((desc.batch, desc.n_kv_heads, desc.seq_capacity, desc.head_dim),
                       dtype=desc.torch_dtype, device=device)


def empty_workspace(desc: Desc, d: int, k: int, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_bytes(desc, d, k), dtype=torch.uint8, device=device)


def pack_kcache(krot_rows: torch.Tensor, kcache: torch.Tensor, desc: Desc, stream=None):
    n = krot_rows.shape[2]
    _expect(krot_rows, (desc.batch, desc.n_kv_heads, n, desc.head_dim), desc.torch_dtype,
            "krot_rows")
    _check(_lib.loki_pack_kcache(_ptr(krot_rows), n, _ptr(kcache), ctypes.byref(desc.c()),
                                 _stream(stream)), "loki_pack_kcache")
    return kcache


def unpack_kcache(kcache: torch.Tensor, n_tokens: int, desc: Desc, out=None, stream=None):
    if out is None:
        out = torch.empty((desc.batch, desc.n_kv_heads, n_tokens, desc.head_dim),
                          dtype=desc.torch_dtype, device=kcache.device)
    _check(_lib.loki_unpack_kcache(_ptr(kcache), n_tokens, _ptr(out), ctypes.byref(desc.c()),
                                   _stream(stream)), "loki_unpack_kcache")
    return out


def append(k_new, v_new, P, kcache, vcache, pos: int, desc: Desc, stream=None):
    shp = (desc.batch, desc.n_kv_heads, desc.head_dim)
    _expect(k_new, shp, desc.torch_dtype, "k_new")
    _expect(v_new, shp, desc.torch_dtype, "v_new")
    _expect(P, (desc.n_kv_heads, desc.head_dim, desc.head_dim), torch.float32, "P")
    _check(_lib.loki_append(_ptr(k_new), _ptr(v_new), _ptr(P), _ptr(kcache), _ptr(vcache), pos,
                            ctypes.byref(desc.c()), _stream(stream)), "loki_append")


def prefill(k_rows, P, kcache, desc: Desc, v_rows=None, vcache=None, pos: int = 0,
            stream=None):
    """Project a run of unrotated keys [B, Hkv, n, D] by P into K cache rows
    [pos, pos + n); with v_rows, copy them into the same rows of vcache."""
    n = k_rows.shape[2] if k_rows.dim() == 4 else -1
    shp = (desc.batch, desc.n_kv_heads, n, desc.head_dim)
    _expect(k_rows, shp, desc.torch_dtype, "k_rows")
    if v_rows is not None:
        _expect(v_rows, shp, desc.torch_dtype, "v_rows")
    _expect(P, (desc.n_kv_heads, desc.head_dim, desc.head_dim), torch.float32, "P")
    _check(_lib.loki_prefill(_ptr(k_rows), _ptr(v_rows), n, pos, _ptr(P), _ptr(kcache),
                             _ptr(vcache), ctypes.byref(desc.c()), _stream(stream)),
           "loki_prefill")
    return kcache


def rotate_query(q, P, desc: Desc, qr=None, stream=None):
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    if qr is None:
        qr = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    _check(_lib.loki_rotate_query(_ptr(q), _ptr(P), _ptr(qr), ctypes.byref(desc.c()),
                                  _stream(stream)), "loki_rotate_query")
    return qr


def score(qr, kcache, d: int, desc: Desc, scores=None, stream=None):
    if scores is None:
        scores = torch.empty((desc.batch, desc.n_q_heads, desc.seq_len), dtype=torch.float32,
                             device=qr.device)
    _check(_lib.loki_score(_ptr(qr), _ptr(kcache), d, _ptr(scores), ctypes.byref(desc.c()),
                           _stream(stream)), "loki_score")
    return scores


def topk(scores, k: int, desc: Desc, idx=None, sel_out=None, stream=None):
    """Top-k indices [B, Hq, k] (ascending); sel_out, if given, gets their scores."""
    _expect(scores, (desc.batch, desc.n_q_heads, desc.seq_len), torch.float32, "scores")
    if idx is None:
        idx = torch.empty((desc.batch, desc.n_q_heads, k), dtype=torch.int32,
                          device=scores.device)
    _check(_lib.loki_topk(_ptr(scores), k, _ptr(idx), _ptr(sel_out), ctypes.byref(desc.c()),
                          _stream(stream)), "loki_topk")
    return idx


def attend(qr, kcache, vcache, idx, desc: Desc, out=None, workspace=None, sel_scores=None,
           stream=None):
    """Exact attention over idx; with sel_scores (partial logits over the leading
    panel_dim coordinates) only the remaining key coordinates are read."""
    k = idx.shape[-1]
    _expect(idx, (desc.batch, desc.n_q_heads, k), torch.int32, "idx")
    out = _out(desc, out, qr.device)
    if workspace is None:
        workspace = empty_workspace(desc, desc.head_dim, k, qr.device)
    _check(_lib.loki_attend(_ptr(qr), _ptr(kcache), _ptr(vcache), _ptr(idx), _ptr(sel_scores), k,
                            _ptr(out),
                            ctypes.byref(desc.c()), _ptr(workspace), workspace.numel(),
                            _stream(stream)), "loki_attend")
    return out


def _check_decode_outputs(desc: Desc, k: int, idx_out, scores_out):
    if idx_out is not None:
        _expect(idx_out, (desc.batch, desc.n_q_heads, k), torch.int32, "idx_out")
    if scores_out is not None:
        _expect(scores_out, (desc.batch, desc.n_q_heads, desc.seq_len), torch.float32,
                "scores_out")


def decode(q, kcache, vcache, P, d: int, k: int, desc: Desc, out=None, idx_out=None,
           workspace=None, stream=None, scores_out=None):
    """One Loki decode step; returns out [B, Hq, D] in desc's output dtype (and
    fills idx_out [B, Hq, k] and scores_out [B, Hq, S] fp32 if given)."""
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    _check_decode_outputs(desc, k, idx_out, scores_out)
    out = _out(desc, out, q.device)
    if workspace is None:
        workspace = empty_workspace(desc, d, k, q.device)
    _check(_lib.loki_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(P), d, k, _ptr(out),
                            _ptr(idx_out), _ptr(scores_out), ctypes.byref(desc.c()),
                            _ptr(workspace), workspace.numel(), _stream(stream)), "loki_decode")
    return out


def decode_noalloc(q, kcache, vcache, P, d: int, k: int, desc: Desc, out=None, idx_out=None,
                   stream=None, scores_out=None):
    """loki_decode_noalloc: one decode step whose workspace is the library's
    fixed per-GPU scratch (NOALLOC_SCRATCH_BYTES); nothing is allocated
    beyond `out` when it is not given."""
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    _check_decode_outputs(desc, k, idx_out, scores_out)
    out = _out(desc, out, q.device)
    _check(_lib.loki_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(P), d, k,
                                    _ptr(out), _ptr(idx_out), _ptr(scores_out),
                                    ctypes.byref(desc.c()), _stream(stream)),
           "loki_decode_noalloc")
    return out


def decode_append(q, k_new, v_new, kcache, vcache, P, d: int, k: int, desc: Desc, out=None,
                  idx_out=None, workspace=None, stream=None, scores_out=None):
    """Append (k_new, v_new) at row seq_len-1, then one decode step over seq_len tokens."""
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    shp = (desc.batch, desc.n_kv_heads, desc.head_dim)
    _expect(k_new, shp, desc.torch_dtype, "k_new")
    _expect(v_new, shp, desc.torch_dtype, "v_new")
    _check_decode_outputs(desc, k, idx_out, scores_out)
    out = _out(desc, out, q.device)
    if workspace is None:
        workspace = empty_workspace(desc, d, k, q.device)
    _check(_lib.loki_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kcache), _ptr(vcache),
                                   _ptr(P), d, k, _ptr(out), _ptr(idx_out), _ptr(scores_out),
                                   ctypes.byref(desc.c()), _ptr(workspace), workspace.numel(),
                                   _stream(stream)),
           "loki_decode_append")
    return out


def full_attention(q, kcache, vcache, P, desc: Desc, out=None, workspace=None, stream=None):
    """Dense decode attention over all seq_len cached tokens (the baseline of
    the Loki step); returns out [B, Hq, D] in desc's output dtype."""
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    out = _out(desc, out, q.device)
    if workspace is None:
        workspace = empty_workspace(desc, desc.head_dim, desc.seq_len, q.device)
    _check(_lib.loki_full_attention(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(P), _ptr(out),
                                    ctypes.byref(desc.c()), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "loki_full_attention")
    return out


def pca_attention(q, kcache, vcache, P, d: int, desc: Desc, out=None, workspace=None,
                  stream=None):
    """PCAAttn: softmax over all seq_len tokens of the scaled scores from the
    leading d rotated coordinates, weighted sum of all V rows; returns out
    [B, Hq, D] in desc's output dtype."""
    _expect(q, (desc.batch, desc.n_q_heads, desc.head_dim), desc.torch_dtype, "q")
    out = _out(desc, out, q.device)
    if workspace is None:
        workspace = empty_workspace(desc, desc.head_dim, desc.seq_len, q.device)
    _check(_lib.loki_pca_attention(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(P), d, _ptr(out),
                                   ctypes.byref(desc.c()), _ptr(workspace), workspace.numel(),
                                   _stream(stream)), "loki_pca_attention")
    return out


def calibrate(keys, desc: Desc, P=None, variances=None, workspace=None, stream=None):
    """PCA of calibration keys [Hkv, n, D] (storage dtype) on the GPU; returns
    (P [Hkv, D, D] fp32, variances [Hkv, D] fp32)."""
    Hkv, D = desc.n_kv_heads, desc.head_dim
    n = keys.shape[1] if keys.dim() == 3 else -1
    _expect(keys, (Hkv, n, D), desc.torch_dtype, "keys")
    if P is None:
        P = torch.empty((Hkv, D, D), dtype=torch.float32, device=keys.device)
    if variances is None:
        variances = torch.empty((Hkv, D), dtype=torch.float32, device=keys.device)
    if workspace is None:
        nb = ctypes.c_size_t()
        _check(_lib.loki_calibrate_workspace_bytes(ctypes.byref(desc.c()), n, ctypes.byref(nb)),
               "loki_calibrate_workspace_bytes")
        workspace = torch.empty(nb.value, dtype=torch.uint8, device=keys.device)
    _check(_lib.loki_calibrate(_ptr(keys), n, _ptr(P), _ptr(variances), ctypes.byref(desc.c()),
                               _ptr(workspace), workspace.numel(), _stream(stream)),
           "loki_calibrate")
    return P, variances


def strerror(code: int) -> str:
    return _lib.loki_strerror(code).decode()


def last_error() -> str:
    return _lib.loki_last_error().decode()


def c_desc(desc: Desc) -> _CDesc:
    """The ctypes loki_desc of a Desc (for callers that drive the C ABI directly)."""
    return desc.c()


lib = _lib
