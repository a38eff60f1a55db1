"""ctypes binding of libcgqa_fa.so (argument marshalling only).

The names match the C ABI in ``include/fa.h``: ``fa_fwd``, ``fa_bwd_delta``,
``fa_bwd``, ``fa_bwd_dq``, ``fa_bwd_dkv`` and their ``*_block_sparse`` forms.  Each takes torch tensors that live on the GPU (torch is used
for device memory and streams only), checks dtype/contiguity/device, derives
the sizes from the shapes and calls the library on the current stream.  Every
step of the computation runs in the HIP kernels; there is no other path.  If
the library is missing or a call returns a non-zero status, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_NAME, PKG_DIR

NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_NOALLOC_SCRATCH_BYTES

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_ALIGN", 3: "FA_ERR_SHAPE",
    4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_GQA", 6: "FA_ERR_CAUSAL_LQ_GT_LK",
    7: "FA_ERR_SCALE", 8: "FA_ERR_LAUNCH", 9: "FA_ERR_STRIDE", 10: "FA_ERR_DTYPE",
    11: "FA_ERR_WORKSPACE",
}

_c_int, _c_float, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p


class FaTensor(ctypes.Structure):
    """fa_tensor: a strided [B, H, L, D] view (element strides; D contiguous)."""
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_l", ctypes.c_int64)]


_T = FaTensor
FA_BF16, FA_F16 = 0, 1
FA_GRAD_DQ, FA_GRAD_DKV = 1, 2

_SIGS = {
    "fa_fwd": [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 6 + [_c_float, _c_int, _vp],
    "fa_bwd_delta": [_vp, _vp, _vp] + [_c_int] * 4 + [_vp],
    "fa_bwd": [_vp] * 10 + [_c_int] * 6 + [_c_float, _c_int, _vp],
    "fa_bwd_dq": [_vp] * 7 + [_c_int] * 6 + [_c_float, _c_int, _vp],
    "fa_bwd_dkv": [_vp] * 8 + [_c_int] * 6 + [_c_float, _c_int, _vp],
    "fa_fwd_ex": [_T] * 4 + [_vp] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _vp, _vp],
    "fa_bwd_delta_ex": [_T, _T, _vp] + [_c_int] * 4 + [_c_int, _vp],
    "fa_bwd_ex": [_T] * 3 + [_vp, _vp] + [_T] * 4 + [_c_int] * 6
                 + [_c_float, _c_int, _c_int, _vp, ctypes.c_uint, _vp],
    "fa_short_workspace_bytes": [_c_int] * 6,
    "fa_bwd_workspace_bytes": [_c_int] * 7,
    "fa_bwd_ws": [_T] * 3 + [_vp, _vp] + [_T] * 4 + [_c_int] * 6
                 + [_c_float, _c_int, _c_int, _vp, ctypes.c_uint, _vp, ctypes.c_size_t, _vp],
    "fa_fwd_short": [_T] * 4 + [_vp] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _vp, ctypes.c_size_t, _vp],
    "fa_fwd_short_noalloc": [_T] * 4 + [_vp] + [_c_int] * 6 + [_c_float, _c_int, _c_int, _vp],
    "fa_bwd_short": [_T] * 3 + [_vp, _vp] + [_T] * 4 + [_c_int] * 6
                    + [_c_float, _c_int, _c_int, ctypes.c_uint, _vp, ctypes.c_size_t, _vp],
    "fa_fwd_block_sparse": [_vp] * 5 + [_c_int] * 6 + [_c_float, _c_int, _vp, _vp],
    "fa_bwd_block_sparse": [_vp] * 10 + [_c_int] * 6 + [_c_float, _c_int, _vp, _vp],
    "fa_bwd_dq_block_sparse": [_vp] * 7 + [_c_int] * 6 + [_c_float, _c_int, _vp, _vp],
    "fa_bwd_dkv_block_sparse": [_vp] * 8 + [_c_int] * 6 + [_c_float, _c_int, _vp, _vp],
    "fa_status_str": [_c_int],
    "fa_version": [],
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


def lib_path() -> str:
    """The in-tree library built by ``build.build_library()``."""
    return os.path.join(PKG_DIR, LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library (raises if it was not built)."""
    global _lib
    if _lib is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(p)
        for name, argtypes in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = (ctypes.c_char_p if name in ("fa_status_str", "fa_version")
                          else ctypes.c_size_t if name.endswith("_workspace_bytes") else ctypes.c_int)
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def version() -> str:
    return load_library().fa_version().decode()


def _check(status: int, call: str) -> None:
    if status != FA_OK:
        raise FAError(status, call)


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _require(t, name, dtype, ndim):
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


MASK_BLOCK = 64  # block-sparse mask granularity (FA_MASK_BLOCK)


def _require_mask(m, Lq, Lk):
    shape = (-(-Lq // MASK_BLOCK), -(-Lk // MASK_BLOCK))
    if m.dtype not in (torch.uint8, torch.bool):
        raise TypeError(f"block_mask must be uint8 or bool, got {m.dtype}")
    if tuple(m.shape) != shape:
        raise ValueError(f"block_mask must be {shape} for Lq={Lq}, Lk={Lk}, got {tuple(m.shape)}")
    if not m.is_cuda:
        raise ValueError("block_mask must be a GPU tensor")
    if not m.is_contiguous():
        raise ValueError("block_mask must be contiguous")


def fa_fwd(q, k, v, o=None, lse=None, *, scale: float, causal: bool, stream=None):
    """O, LSE = attention(q, k, v).  q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D] bf16."""
    return _fwd(q, k, v, None, o, lse, scale, causal, stream)


def fa_fwd_block_sparse(q, k, v, block_mask, o=None, lse=None, *, scale: float, causal: bool,
                        stream=None):
    """fa_fwd restricted to the 64 x 64 blocks where block_mask [ceil(Lq/64), ceil(Lk/64)]
    is nonzero.  Rows that see no key get O = 0 and lse = -inf."""
    return _fwd(q, k, v, block_mask, o, lse, scale, causal, stream)


def _fwd(q, k, v, mask, o, lse, scale, causal, stream):
    _require(q, "q", torch.bfloat16, 4)
    _require(k, "k", torch.bfloat16, 4)
    _require(v, "v", torch.bfloat16, 4)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require(o, "o", torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("output shapes do not match q")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)))
    lib = load_library()
    if mask is None:
        st, name = lib.fa_fwd(*args, _stream_ptr(stream)), "fa_fwd"
    else:
        _require_mask(mask, Lq, Lk)
        st = lib.fa_fwd_block_sparse(*args, _ptr(mask), _stream_ptr(stream))
        name = "fa_fwd_block_sparse"
    _check(st, name)
    return o, lse


def fa_bwd_delta(o, do, delta=None, *, stream=None):
    """delta[b,h,i] = sum_d dO*O in fp32.  o, do [B,H,Lq,D] bf16."""
    _require(o, "o", torch.bfloat16, 4)
    _require(do, "do", torch.bfloat16, 4)
    if tuple(do.shape) != tuple(o.shape):
        raise ValueError("do must have the shape of o")
    B, H, Lq, D = o.shape
    if delta is None:
        delta = torch.empty((B, H, Lq), dtype=torch.float32, device=o.device)
    _require(delta, "delta", torch.float32, 3)
    if tuple(delta.shape) != (B, H, Lq):
        raise ValueError("delta must be [B, H, Lq]")
    st = load_library().fa_bwd_delta(_ptr(o), _ptr(do), _ptr(delta), B, H, Lq, D, _stream_ptr(stream))
    _check(st, "fa_bwd_delta")
    return delta


def fa_bwd(q, k, v, o, lse, delta, do, dq=None, dk=None, dv=None, *, scale: float, causal: bool,
           stream=None):
    """dQ, dK, dV of attention given the saved lse, the precomputed delta and dO."""
    return _bwd(q, k, v, o, lse, delta, do, None, dq, dk, dv, scale, causal, stream)


def fa_bwd_block_sparse(q, k, v, o, lse, delta, do, block_mask, dq=None, dk=None, dv=None, *,
                        scale: float, causal: bool, stream=None):
    """fa_bwd under the block mask the forward used."""
    return _bwd(q, k, v, o, lse, delta, do, block_mask, dq, dk, dv, scale, causal, stream)


def _bwd(q, k, v, o, lse, delta, do, mask, dq, dk, dv, scale, causal, stream):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
        _require(t, n, torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    _require(delta, "delta", torch.float32, 3)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if tuple(lse.shape) != (B, Hq, Lq) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("lse/delta must be [B, Hq, Lq]")
    if o is not None:
        _require(o, "o", torch.bfloat16, 4)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _require(t, n, torch.bfloat16, 4)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{n} has the wrong shape")
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(delta), _ptr(do),
            _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)))
    lib = load_library()
    if mask is None:
        st, name = lib.fa_bwd(*args, _stream_ptr(stream)), "fa_bwd"
    else:
        _require_mask(mask, Lq, Lk)
        st = lib.fa_bwd_block_sparse(*args, _ptr(mask), _stream_ptr(stream))
        name = "fa_bwd_block_sparse"
    _check(st, name)
    return dq, dk, dv


def _bwd_half(which, q, k, v, lse, delta, do, outs, scale, causal, stream, mask=None):
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
        _require(t, n, torch.bfloat16, 4)
    _require(lse, "lse", torch.float32, 3)
    _require(delta, "delta", torch.float32, 3)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or tuple(do.shape) != tuple(q.shape):
        raise ValueError("shape mismatch")
    if tuple(lse.shape) != (B, Hq, Lq) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("lse/delta must be [B, Hq, Lq]")
    lib = load_library()
    tail = (B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)))
    suffix = ""
    if mask is not None:
        _require_mask(mask, Lq, Lk)
        tail += (_ptr(mask),)
        suffix = "_block_sparse"
    tail += (_stream_ptr(stream),)
    fn = getattr(lib, "fa_bwd_" + which + suffix)
    if which == "dq":
        (dq,) = outs
        _require(dq, "dq", torch.bfloat16, 4)
        if tuple(dq.shape) != tuple(q.shape):
            raise ValueError("dq has the wrong shape")
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(delta), _ptr(do), _ptr(dq), *tail)
    else:
        dk, dv = outs
        for t, n in ((dk, "dk"), (dv, "dv")):
            _require(t, n, torch.bfloat16, 4)
            if tuple(t.shape) != tuple(k.shape):
                raise ValueError(f"{n} has the wrong shape")
        st = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(delta), _ptr(do),
                _ptr(dk), _ptr(dv), *tail)
    _check(st, "fa_bwd_" + which + suffix)
    return outs


def fa_bwd_dq(q, k, v, lse, delta, do, dq=None, *, scale: float, causal: bool, stream=None):
    """dQ only (the query-block kernel of fa_bwd)."""
    dq = torch.empty_like(q) if dq is None else dq
    return _bwd_half("dq", q, k, v, lse, delta, do, (dq,), scale, causal, stream)[0]


def fa_bwd_dkv(q, k, v, lse, delta, do, dk=None, dv=None, *, scale: float, causal: bool, stream=None):
    """dK and dV only (the key-block kernel of fa_bwd)."""
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    return _bwd_half("dkv", q, k, v, lse, delta, do, (dk, dv), scale, causal, stream)


def fa_bwd_dq_block_sparse(q, k, v, lse, delta, do, block_mask, dq=None, *, scale: float,
                           causal: bool, stream=None):
    """fa_bwd_dq under a block mask."""
    dq = torch.empty_like(q) if dq is None else dq
    return _bwd_half("dq", q, k, v, lse, delta, do, (dq,), scale, causal, stream, block_mask)[0]


def fa_bwd_dkv_block_sparse(q, k, v, lse, delta, do, block_mask, dk=None, dv=None, *,
                            scale: float, causal: bool, stream=None):
    """fa_bwd_dkv under a block mask."""
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    return _bwd_half("dkv", q, k, v, lse, delta, do, (dk, dv), scale, causal, stream, block_mask)


# ---------------------------------------------------------------- general calls
# fp16 or bf16, any strided [B, H, L, D] views whose last dimension is
# contiguous (for instance [B, L, H, D] buffers seen through .transpose(1, 2),
# or the first Lk rows of a longer K/V cache).

_DTYPES = {torch.bfloat16: FA_BF16, torch.float16: FA_F16}


def _view(t, name, dtype=None):
    if t.dtype not in _DTYPES:
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have the dtype of q ({dtype}), got {t.dtype}")
    if t.dim() != 4:
        raise ValueError(f"{name} must have 4 dims [B, H, L, D], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous (stride 1)")
    return FaTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _null_view():
    return FaTensor(None, 0, 0, 0)


def _out_like(ref, shape=None):
    """A new output for `ref`'s [B, H, L, D] view: the same layout when ref is
    a permutation of a dense buffer, else contiguous."""
    return torch.empty_like(ref) if shape is None else torch.empty(shape, dtype=ref.dtype, device=ref.device)


def fa_fwd_ex(q, k, v, o=None, lse=None, *, scale: float, causal: bool, block_mask=None, stream=None):
    """fa_fwd for bf16 or fp16 strided views (and an optional block mask)."""
    qt = _view(q, "q")
    kt, vt = _view(k, "k", q.dtype), _view(v, "v", q.dtype)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    o = _out_like(q) if o is None else o
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have the shape of q")
    ot = _view(o, "o", q.dtype)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be [B, Hq, Lq]")
    mask = 0
    if block_mask is not None:
        _require_mask(block_mask, Lq, Lk)
        mask = _ptr(block_mask)
    st = load_library().fa_fwd_ex(qt, kt, vt, ot, _ptr(lse), B, Hq, Hkv, Lq, Lk, D, float(scale),
                                  int(bool(causal)), _DTYPES[q.dtype], mask, _stream_ptr(stream))
    _check(st, "fa_fwd_ex")
    return o, lse


def fa_bwd_delta_ex(o, do, delta=None, *, stream=None):
    """fa_bwd_delta for bf16 or fp16 strided views."""
    ot = _view(o, "o")
    dt = _view(do, "do", o.dtype)
    if tuple(do.shape) != tuple(o.shape):
        raise ValueError("do must have the shape of o")
    B, H, Lq, D = o.shape
    if delta is None:
        delta = torch.empty((B, H, Lq), dtype=torch.float32, device=o.device)
    _require(delta, "delta", torch.float32, 3)
    if tuple(delta.shape) != (B, H, Lq):
        raise ValueError("delta must be [B, H, Lq]")
    st = load_library().fa_bwd_delta_ex(ot, dt, _ptr(delta), B, H, Lq, D, _DTYPES[o.dtype],
                                        _stream_ptr(stream))
    _check(st, "fa_bwd_delta_ex")
    return delta


def fa_bwd_ex(q, k, v, lse, delta, do, dq=None, dk=None, dv=None, *, scale: float, causal: bool,
              block_mask=None, grads: str = "all", stream=None, workspace=False):
    """fa_bwd for bf16 or fp16 strided views.  grads: "all", "dq" or "dkv";
    returns (dq, dk, dv) with None for what was not asked for.  `workspace`:
    False for fa_bwd_ex; a GPU byte tensor (at least fa_bwd_workspace_bytes)
    or True (allocated here through torch) for fa_bwd_ws, whose dK/dV kernel
    splits long query lists over several workgroups."""
    want = {"all": FA_GRAD_DQ | FA_GRAD_DKV, "dq": FA_GRAD_DQ, "dkv": FA_GRAD_DKV}[grads]
    qt = _view(q, "q")
    kt, vt, dot = _view(k, "k", q.dtype), _view(v, "v", q.dtype), _view(do, "do", q.dtype)
    _require(lse, "lse", torch.float32, 3)
    _require(delta, "delta", torch.float32, 3)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or tuple(do.shape) != tuple(q.shape) or k.shape[0] != B \
            or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if tuple(lse.shape) != (B, Hq, Lq) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("lse/delta must be [B, Hq, Lq]")
    dqt = dkt = dvt = _null_view()
    if want & FA_GRAD_DQ:
        dq = _out_like(q) if dq is None else dq
        if tuple(dq.shape) != tuple(q.shape):
            raise ValueError("dq has the wrong shape")
        dqt = _view(dq, "dq", q.dtype)
    if want & FA_GRAD_DKV:
        dk = _out_like(k) if dk is None else dk
        dv = _out_like(v) if dv is None else dv
        for t, n in ((dk, "dk"), (dv, "dv")):
            if tuple(t.shape) != tuple(k.shape):
                raise ValueError(f"{n} has the wrong shape")
        dkt, dvt = _view(dk, "dk", q.dtype), _view(dv, "dv", q.dtype)
    mask = 0
    if block_mask is not None:
        _require_mask(block_mask, Lq, Lk)
        mask = _ptr(block_mask)
    if workspace is False:
        st = load_library().fa_bwd_ex(qt, kt, vt, _ptr(lse), _ptr(delta), dot, dqt, dkt, dvt,
                                      B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)),
                                      _DTYPES[q.dtype], mask, want, _stream_ptr(stream))
        _check(st, "fa_bwd_ex")
    else:
        nbytes = fa_bwd_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, block_mask is not None)
        ws = _workspace(None if workspace is True else workspace, nbytes, q.device) if nbytes else None
        st = load_library().fa_bwd_ws(qt, kt, vt, _ptr(lse), _ptr(delta), dot, dqt, dkt, dvt,
                                      B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)),
                                      _DTYPES[q.dtype], mask, want, _ptr(ws), 0 if ws is None else ws.numel(),
                                      _stream_ptr(stream))
        _check(st, "fa_bwd_ws")
    return (dq if want & FA_GRAD_DQ else None,
            dk if want & FA_GRAD_DKV else None,
            dv if want & FA_GRAD_DKV else None)


def fa_bwd_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, masked=False) -> int:
    """Workspace bytes of fa_bwd_ws for this shape (0: no split planned)."""
    return int(load_library().fa_bwd_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, int(bool(masked))))


# ---------------------------------------------------------------- short queries

SHORT_MAX_LQ = 8


def fa_short_workspace_bytes(B: int, Hq: int, Hkv: int, Lq: int, Lk: int, D: int) -> int:
    """Bytes of device workspace fa_fwd_short / fa_bwd_short need (0: sizes refused)."""
    return int(load_library().fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D))


def _workspace(ws, nbytes, device):
    if ws is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws


def fa_fwd_short(q, k, v, o=None, lse=None, *, scale: float, causal: bool, workspace=None, stream=None):
    """Forward for Lq <= 8 (bf16 or fp16 strided views).  `workspace`: a GPU
    byte tensor of at least fa_short_workspace_bytes(...) bytes, allocated
    here through torch when not given."""
    qt = _view(q, "q")
    kt, vt = _view(k, "k", q.dtype), _view(v, "v", q.dtype)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    o = _out_like(q) if o is None else o
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have the shape of q")
    ot = _view(o, "o", q.dtype)
    if lse is None:
        lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device=q.device)
    _require(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be [B, Hq, Lq]")
    nbytes = fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D)
    ws = _workspace(workspace, nbytes, q.device)
    st = load_library().fa_fwd_short(qt, kt, vt, ot, _ptr(lse), B, Hq, Hkv, Lq, Lk, D, float(scale),
                                     int(bool(causal)), _DTYPES[q.dtype], _ptr(ws), ws.numel(),
                                     _stream_ptr(stream))
    _check(st, "fa_fwd_short")
    return o, lse


def fa_fwd_short_noalloc(q, k, v, o, lse, *, scale: float, causal: bool, stream=None):
    """fa_fwd_short with the library's static per-device scratch instead of a
    workspace: o and lse must be given (nothing is allocated, here or in the
    library).  Calls that may overlap on one GPU race on that scratch."""
    qt = _view(q, "q")
    kt, vt = _view(k, "k", q.dtype), _view(v, "v", q.dtype)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k/v shapes do not match q")
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have the shape of q")
    ot = _view(o, "o", q.dtype)
    _require(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, Hq, Lq):
        raise ValueError("lse must be [B, Hq, Lq]")
    st = load_library().fa_fwd_short_noalloc(qt, kt, vt, ot, _ptr(lse), B, Hq, Hkv, Lq, Lk, D, float(scale),
                                             int(bool(causal)), _DTYPES[q.dtype], _stream_ptr(stream))
    _check(st, "fa_fwd_short_noalloc")
    return o, lse


def fa_bwd_short(q, k, v, lse, delta, do, dq=None, dk=None, dv=None, *, scale: float, causal: bool,
                 grads: str = "all", workspace=None, stream=None):
    """Backward for Lq <= 8; grads "all", "dq" or "dkv" (see fa_bwd_ex)."""
    want = {"all": FA_GRAD_DQ | FA_GRAD_DKV, "dq": FA_GRAD_DQ, "dkv": FA_GRAD_DKV}[grads]
    qt = _view(q, "q")
    kt, vt, dot = _view(k, "k", q.dtype), _view(v, "v", q.dtype), _view(do, "do", q.dtype)
    _require(lse, "lse", torch.float32, 3)
    _require(delta, "delta", torch.float32, 3)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    if tuple(v.shape) != tuple(k.shape) or tuple(do.shape) != tuple(q.shape) or k.shape[0] != B \
            or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if tuple(lse.shape) != (B, Hq, Lq) or tuple(delta.shape) != (B, Hq, Lq):
        raise ValueError("lse/delta must be [B, Hq, Lq]")
    dqt = dkt = dvt = _null_view()
    ws_ptr, ws_len = None, 0
    if want & FA_GRAD_DQ:
        dq = _out_like(q) if dq is None else dq
        if tuple(dq.shape) != tuple(q.shape):
            raise ValueError("dq has the wrong shape")
        dqt = _view(dq, "dq", q.dtype)
        ws = _workspace(workspace, fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D), q.device)
        ws_ptr, ws_len = _ptr(ws), ws.numel()
    if want & FA_GRAD_DKV:
        dk = _out_like(k) if dk is None else dk
        dv = _out_like(v) if dv is None else dv
        for t, n in ((dk, "dk"), (dv, "dv")):
            if tuple(t.shape) != tuple(k.shape):
                raise ValueError(f"{n} has the wrong shape")
        dkt, dvt = _view(dk, "dk", q.dtype), _view(dv, "dv", q.dtype)
    st = load_library().fa_bwd_short(qt, kt, vt, _ptr(lse), _ptr(delta), dot, dqt, dkt, dvt,
                                     B, Hq, Hkv, Lq, Lk, D, float(scale), int(bool(causal)),
                                     _DTYPES[q.dtype], want, ws_ptr, ws_len, _stream_ptr(stream))
    _check(st, "fa_bwd_short")
    return (dq if want & FA_GRAD_DQ else None,
            dk if want & FA_GRAD_DKV else None,
            dv if want & FA_GRAD_DKV else None)
