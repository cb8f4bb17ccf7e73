"""Python binding for libtca.so: causal GQA tiled attention on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/tca.h. PyTorch provides device
memory and the current stream. There is no CPU fallback: if the library is
not built, every call raises.

    o, lse = attn_fwd(q, k, v, causal=True)             # q [B,Hq,N,d], k/v [B,Hkv,N,d]
    dq, dk, dv = attn_bwd(q, k, v, o, lse, dO, causal=True)

Inputs are float32 or bfloat16 CUDA tensors, contiguous. Outputs o, dq, dk, dv
are float32 by default or bfloat16 (attn_fwd(..., out_dtype=torch.bfloat16);
the backward follows o's dtype); lse is always float32.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtca.so")

ATTN_F32, ATTN_BF16 = 0, 1
ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP, ATTN_ESCRATCH = 0, 1, 2, 3, 4
DECODE_SCRATCH_BYTES = 16 << 20   # the fixed array behind attn_decode_noalloc (ATTN_DECODE_SCRATCH_BYTES)
ABI_VERSION = 4                   # the interface these argument lists follow (attn_abi_version)

_lib = None


class AttnLayout(ctypes.Structure):
    """Element strides (batch, head, row) of a [B, H, N, d] tensor with contiguous d."""
    _fields_ = [("stride_b", ctypes.c_longlong), ("stride_h", ctypes.c_longlong), ("stride_n", ctypes.c_longlong)]


class AttnError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libtca.so with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python tiled_causal_attention_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, i, f, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_abi_version.argtypes, L.attn_abi_version.restype = [], i
    if L.attn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} implements interface version {L.attn_abi_version()}, this binding "
                           f"version {ABI_VERSION}: rebuild the library")
    L.attn_status_str.argtypes, L.attn_status_str.restype = [i], ctypes.c_char_p
    L.attn_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_fwd_workspace_bytes.restype = sz
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_fwd.argtypes = [i, i, vp, vp, vp, vp, fp, vp, sz, i, i, i, i, i, i, f, vp]
    L.attn_fwd.restype = i
    bwd_args = [i, i, vp, vp, vp, vp, fp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, vp]
    for name in ("attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv"):
        getattr(L, name).argtypes = bwd_args
        getattr(L, name).restype = i
    lp = ctypes.POINTER(AttnLayout)
    for nm in ("attn_fwd_rope_workspace_bytes", "attn_bwd_rope_workspace_bytes"):
        getattr(L, nm).argtypes = [i, i, i, i, i, i, i]
        getattr(L, nm).restype = sz
    L.attn_fwd_rope.argtypes = [i, i, vp, lp, vp, lp, vp, lp, fp, fp, vp, vp, fp, vp, sz, i, i, i, i, i, i, f, vp]
    L.attn_fwd_rope.restype = i
    L.attn_bwd_rope.argtypes = [i, i, vp, lp, vp, lp, vp, lp, fp, fp, vp, vp, fp, vp, vp, lp, vp, lp, vp, lp, vp,
                                sz, i, i, i, i, i, i, f, vp]
    L.attn_bwd_rope.restype = i
    L.attn_fwd_naive_workspace_bytes.argtypes = [i, i, i]
    L.attn_fwd_naive_workspace_bytes.restype = sz
    L.attn_fwd_naive.argtypes = [i, i, vp, vp, vp, vp, fp, vp, sz, i, i, i, i, i, i, f, vp]
    L.attn_fwd_naive.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [i, i, vp, vp, vp, vp, fp, vp, sz, i, i, i, i, i, i, i, f, vp]
    L.attn_decode.restype = i
    L.attn_decode_noalloc.argtypes = [i, i, vp, vp, vp, vp, fp, i, i, i, i, i, i, i, f, vp]
    L.attn_decode_noalloc.restype = i
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().attn_status_str(int(status)).decode()


def _check(status: int):
    if status != ATTN_OK:
        raise AttnError(status, status_str(status))


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return ATTN_F32
    if dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {dtype}; use float32 or bfloat16")


def _dtype_code(t: torch.Tensor) -> int:
    return _code(t.dtype)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dims(q: torch.Tensor, k: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    return B, Hq, k.shape[1], N, d


# Every tensor is checked against q's and k's sizes before a pointer reaches the
# C ABI: the kernels size their buffer walks from (B, Hq, Hkv, N, d) alone, so a
# short tensor would otherwise be read or written past its end.
def _expect(t: torch.Tensor, name: str, shape, dtypes=None):
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} is {t.dtype}, expected one of {tuple(dtypes)}")


def _same_device(ref: torch.Tensor, **named):
    for name, t in named.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, q on {ref.device}: all tensors must share one device")


_IN_DTYPES = (torch.float32, torch.bfloat16)


def _check_qkv(q, k, v, kv_rows=None):
    """(B, Hq, Hkv, Nq, d) after checking that k and v are [B, Hkv, Nk, d] with q's
    dtype (Nk = kv_rows, or q's N when None)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, N, d]")
    B, Hq, N, d = q.shape
    _expect(q, "q", q.shape, _IN_DTYPES)
    Nk = N if kv_rows is None else kv_rows
    _expect(k, "k", (B, k.shape[1], Nk, d), (q.dtype,))
    _expect(v, "v", k.shape, (q.dtype,))
    _same_device(q, k=k, v=v)
    return B, Hq, k.shape[1], N, d


def _check_outputs(q, o, lse, B, Hq, N, d):
    _expect(o, "o", (B, Hq, N, d), _IN_DTYPES)
    _expect(lse, "lse", (B, Hq, N), (torch.float32,))
    _same_device(q, o=o, lse=lse)


def _check_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws):
    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    _check_outputs(q, o, lse, B, Hq, N, d)
    _expect(dO, "dO", q.shape, (q.dtype,))
    _expect(dq, "dq", q.shape, (o.dtype,))
    _expect(dk, "dk", k.shape, (o.dtype,))
    _expect(dv, "dv", k.shape, (o.dtype,))
    _same_device(q, dO=dO, dq=dq, dk=dk, dv=dv, workspace=ws)
    return B, Hq, Hkv, N, d


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
             scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
             out_dtype: Optional[torch.dtype] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward: returns (o [B,Hq,N,d] in out_dtype (float32 unless given, or
    the dtype of out[0]), lse float32 [B,Hq,N])."""
    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    if out is None:
        o = torch.empty((B, Hq, N, d), dtype=out_dtype or torch.float32, device=q.device)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if out_dtype is not None and o.dtype != out_dtype:
            raise TypeError(f"out[0] is {o.dtype}, out_dtype is {out_dtype}")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check_outputs(q, o, lse, B, Hq, N, d)
    L = lib()
    ws_bytes = L.attn_fwd_workspace_bytes(dt, B, Hq, Hkv, N, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    _check(L.attn_fwd(dt, _code(o.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(ws), ws_bytes,
                      B, Hq, Hkv, N, d, int(bool(causal)), scale, _stream(q.device)))
    return o, lse


def bwd_workspace(q: torch.Tensor, k: torch.Tensor) -> torch.Tensor:
    B, Hq, Hkv, N, d = _dims(q, k)
    n = lib().attn_bwd_workspace_bytes(_dtype_code(q), B, Hq, Hkv, N, d)
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=q.device)


def _bwd_call(name, q, k, v, o, lse, dO, dq, dk, dv, ws, causal, scale):
    for t in (dq, dk, dv):
        if t is not None and o is not None and t.dtype != o.dtype:
            raise TypeError(f"dq, dk, dv must have o's dtype {o.dtype}, got {t.dtype}")
    if lse is not None and lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    B, Hq, Hkv, N, d = _check_bwd(q, k, v, o, lse, dO, dq, dk, dv, ws)
    scale = default_scale(d) if scale is None else float(scale)
    _check(getattr(lib(), name)(_dtype_code(q), _code(o.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), _nbytes(ws),
                                B, Hq, Hkv, N, d, int(bool(causal)), scale, _stream(q.device)))


def attn_bwd(q, k, v, o, lse, dO, causal: bool = True, scale: Optional[float] = None,
             out=None, workspace: Optional[torch.Tensor] = None):
    """Backward: returns (dq [B,Hq,N,d], dk, dv [B,Hkv,N,d]) in o's dtype."""
    if out is None:
        dq = torch.empty(q.shape, dtype=o.dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=o.dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=o.dtype, device=q.device)
    else:
        dq, dk, dv = out
    ws = bwd_workspace(q, k) if workspace is None else workspace
    _bwd_call("attn_bwd", q, k, v, o, lse, dO, dq, dk, dv, ws, causal, scale)
    return dq, dk, dv


def attn_bwd_dq(q, k, v, o, lse, dO, dq, dk, dv, workspace, causal=True, scale=None):
    """First backward phase (D = rowsum(dO o O) into the workspace, then dq)."""
    _bwd_call("attn_bwd_dq", q, k, v, o, lse, dO, dq, dk, dv, workspace, causal, scale)


def attn_bwd_dkdv(q, k, v, o, lse, dO, dq, dk, dv, workspace, causal=True, scale=None):
    """Second backward phase (dk, dv; reads D from the workspace)."""
    _bwd_call("attn_bwd_dkdv", q, k, v, o, lse, dO, dq, dk, dv, workspace, causal, scale)


def decode_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace of `nbytes` (attn_decode_workspace_bytes) for attn_decode."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def attn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Few-query attention over a cache: q [B,Hq,Nq,d] are the last Nq positions of
    the sequence whose keys/values k, v [B,Hkv,Nk,d] hold. Returns (o [B,Hq,Nq,d]
    in out_dtype (float32 unless given, or out[0]'s dtype), lse float32 [B,Hq,Nq])."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d]")
    B, Hq, Hkv, Nq, d = _check_qkv(q, k, v, kv_rows=k.shape[2])
    Nk = k.shape[2]
    scale = default_scale(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    if out is None:
        o = torch.empty((B, Hq, Nq, d), dtype=out_dtype or torch.float32, device=q.device)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if out_dtype is not None and o.dtype != out_dtype:
            raise TypeError(f"out[0] is {o.dtype}, out_dtype is {out_dtype}")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    _check_outputs(q, o, lse, B, Hq, Nq, d)
    L = lib()
    ws_bytes = int(L.attn_decode_workspace_bytes(dt, B, Hq, Hkv, Nq, Nk, d))
    if workspace is None and ws_bytes:
        workspace = decode_workspace(ws_bytes, q.device)
    _same_device(q, workspace=workspace)
    wsn = _nbytes(workspace)
    _check(L.attn_decode(dt, _code(o.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                         _ptr(workspace), wsn, B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
                         _stream(q.device)))
    return o, lse


def attn_decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                        scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                        out_dtype: Optional[torch.dtype] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_decode without a workspace: the library's fixed device array holds the
    split partials (calls that overlap on one GPU race on it). With `out` given the
    call allocates nothing. Raises AttnError (ATTN_ESCRATCH) when the sizes need more
    than DECODE_SCRATCH_BYTES of partials."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d]")
    B, Hq, Hkv, Nq, d = _check_qkv(q, k, v, kv_rows=k.shape[2])
    Nk = k.shape[2]
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        o = torch.empty((B, Hq, Nq, d), dtype=out_dtype or torch.float32, device=q.device)
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if out_dtype is not None and o.dtype != out_dtype:
            raise TypeError(f"out[0] is {o.dtype}, out_dtype is {out_dtype}")
    _check_outputs(q, o, lse, B, Hq, Nq, d)
    _check(lib().attn_decode_noalloc(_dtype_code(q), _code(o.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                     _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), scale,
                                     _stream(q.device)))
    return o, lse


def attn_fwd_naive(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
                   scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
                   out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Unoptimised forward through the materialised score matrix (B*Hq*N*N floats
    of workspace): same results as attn_fwd, for teaching and comparison."""
    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    if out is None:
        o = torch.empty((B, Hq, N, d), dtype=out_dtype or torch.float32, device=q.device)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    _check_outputs(q, o, lse, B, Hq, N, d)
    L = lib()
    ws_bytes = int(L.attn_fwd_naive_workspace_bytes(B, Hq, N))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _same_device(q, workspace=workspace)
    _check(L.attn_fwd_naive(_dtype_code(q), _code(o.dtype), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                            _ptr(workspace), _nbytes(workspace), B, Hq, Hkv, N, d, int(bool(causal)), scale,
                            _stream(q.device)))
    return o, lse


def _layout(t: torch.Tensor) -> AttnLayout:
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError("tensors must be [B, H, N, d] views with a contiguous head dimension")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return AttnLayout(t.stride(0), t.stride(1), t.stride(2))


def _sptr(t: torch.Tensor) -> Optional[int]:
    return t.data_ptr() if t.numel() else None


def _tables(cos, sin, N, d):
    if cos is None and sin is None:
        return None, None
    for t in (cos, sin):
        if t is None or t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != (N, d // 2) \
                or not t.is_contiguous():
            raise ValueError(f"rope tables must be contiguous float32 CUDA tensors of shape {(N, d // 2)}")
    return cos.data_ptr(), sin.data_ptr()


def _check_k_rot(k_rot, q, B, Hkv, N, d):
    """k_rot: None or a contiguous [B, Hkv, N, d] tensor on q's device with q's element
    size (bfloat16 or float16 storage for bfloat16 inputs, float32 for float32). The
    library keeps the rotated keys there in its own precision (fp16 on the
    matrix-core path), for attn_bwd_rope."""
    if k_rot is None:
        return None
    _expect(k_rot, "k_rot", (B, Hkv, N, d), (q.dtype, torch.float16) if q.dtype == torch.bfloat16 else (q.dtype,))
    _same_device(q, k_rot=k_rot)
    return _ptr(k_rot)


def attn_fwd_rope(q, k, v, cos=None, sin=None, causal: bool = True, scale: Optional[float] = None, out=None,
                  out_dtype: Optional[torch.dtype] = None, workspace: Optional[torch.Tensor] = None,
                  k_rot: Optional[torch.Tensor] = None):
    """Forward with rotary position embedding of q and k (rotate-half pairing; cos,
    sin: [N, d/2] float32 tables, or both None) on [B, H, N, d] views with any
    strides (e.g. slices of one fused QKV projection). Returns (o, lse) like attn_fwd.
    k_rot: optional contiguous [B, Hkv, N, d] tensor with q's element size that receives
    the rotated keys (fp16 on the matrix-core path), to be passed to attn_bwd_rope
    (which then does not rotate k again)."""
    B, Hq, Hkv, N, d = _check_qkv(q, k, v)
    kr = _check_k_rot(k_rot, q, B, Hkv, N, d)
    scale = default_scale(d) if scale is None else float(scale)
    dt = _dtype_code(q)
    if out is None:
        o = torch.empty((B, Hq, N, d), dtype=out_dtype or torch.float32, device=q.device)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
    _check_outputs(q, o, lse, B, Hq, N, d)
    L = lib()
    cs, sn = _tables(cos, sin, N, d)
    n = int(L.attn_fwd_rope_workspace_bytes(dt, _code(o.dtype), B, Hq, Hkv, N, d))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    _same_device(q, workspace=workspace)
    ql, kl, vl = _layout(q), _layout(k), _layout(v)
    _check(L.attn_fwd_rope(dt, _code(o.dtype), _sptr(q), ctypes.byref(ql), _sptr(k), ctypes.byref(kl), _sptr(v),
                           ctypes.byref(vl), cs, sn, kr, _ptr(o), _ptr(lse), _ptr(workspace), _nbytes(workspace),
                           B, Hq, Hkv, N, d, int(bool(causal)), scale, _stream(q.device)))
    return o, lse


def attn_bwd_rope(q, k, v, o, lse, dO, cos=None, sin=None, causal: bool = True, scale: Optional[float] = None,
                  out=None, workspace: Optional[torch.Tensor] = None, k_rot: Optional[torch.Tensor] = None):
    """Backward of attn_fwd_rope: gradients of the unrotated q, k and of v, in o's
    dtype, written into `out` = (dq, dk, dv) views (any strides) or new contiguous tensors.
    k_rot: the tensor attn_fwd_rope filled for the same k and tables, unchanged since
    (the rotated keys are then read from it, not recomputed), or None."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or o.dim() != 4:
        raise ValueError("q, k, v, o must be 4-D [B, H, N, d]")
    dt = _dtype_code(q)
    if out is None:
        dq = torch.empty(q.shape, dtype=o.dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=o.dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=o.dtype, device=q.device)
    else:
        dq, dk, dv = out
    for t in (dq, dk, dv):
        if t.dtype != o.dtype:
            raise TypeError("dq, dk, dv must have o's dtype")
    B, Hq, Hkv, N, d = _check_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace)
    kr = _check_k_rot(k_rot, q, B, Hkv, N, d)
    scale = default_scale(d) if scale is None else float(scale)
    L = lib()
    cs, sn = _tables(cos, sin, N, d)
    n = int(L.attn_bwd_rope_workspace_bytes(dt, _code(o.dtype), B, Hq, Hkv, N, d))
    if workspace is None:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    ls = [_layout(t) for t in (q, k, v, dq, dk, dv)]
    _check(L.attn_bwd_rope(dt, _code(o.dtype), _sptr(q), ctypes.byref(ls[0]), _sptr(k), ctypes.byref(ls[1]),
                           _sptr(v), ctypes.byref(ls[2]), cs, sn, kr, _ptr(o), _ptr(lse), _ptr(dO),
                           _sptr(dq), ctypes.byref(ls[3]), _sptr(dk), ctypes.byref(ls[4]), _sptr(dv),
                           ctypes.byref(ls[5]), _ptr(workspace), _nbytes(workspace), B, Hq, Hkv, N, d,
                           int(bool(causal)), scale, _stream(q.device)))
    return dq, dk, dv

