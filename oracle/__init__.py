"""CPU oracle for causal GQA attention (float64, plain C + OpenMP).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline may import this package; the product path (the HIP library and its
Python binding) never does. The oracle and the HIP path share no code.

The arithmetic lives in ``oracle.c``; this module compiles it with gcc when the
shared library is missing and marshals float64 numpy arrays through ctypes.
Scale: the caller's float (normally the float32 value of 1/sqrt(d)), widened to
float64 exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# Plain float64 semantics: no fast-math, no FMA contraction.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into ``out`` (always recompiles)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str = _LIB):
    """Load a compiled oracle library (building the default one if absent)."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if path == _LIB and not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, ctypes.c_double]
    lib.oracle_attn_fwd.restype = None
    lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, ctypes.c_double]
    lib.oracle_attn_bwd.restype = None
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_attn_sampled.argtypes = [dp, dp, dp, dp, i, i, i, i, ctypes.c_double,
                                        i, ip, ip, dp, dp, dp, i, ip, dp, dp]
    lib.oracle_attn_sampled.restype = None
    lib.oracle_attn_decode.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i, i, ctypes.c_double]
    lib.oracle_attn_decode.restype = None
    lib.oracle_attn_fwd_rope.argtypes = [dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, ctypes.c_double]
    lib.oracle_attn_fwd_rope.restype = None
    lib.oracle_attn_bwd_rope.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, i, i, i, i, i, i, ctypes.c_double]
    lib.oracle_attn_bwd_rope.restype = None
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q, k):
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (B, N, d) != (Bk, Nk, dk) or Hkv < 1 or Hq % Hkv:
        raise ValueError(f"bad shapes q{q.shape} k{k.shape}")
    return B, Hq, Hkv, N, d


def attn_fwd(q, k, v, causal: int = 1, scale: float | None = None, lib=None
             ) -> Tuple[np.ndarray, np.ndarray]:
    """Return (o [B,Hq,N,d], lse [B,Hq,N]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    (lib or load()).oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    B, Hq, Hkv, N, d, int(causal), float(scale))
    return o, lse


def attn_decode(q, k, v, causal: int = 1, scale: float | None = None, lib=None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Few-query attention over a cache: q [B,Hq,Nq,d] are the last Nq positions of
    the Nk-token sequence whose keys and values k, v [B,Hkv,Nk,d] hold (Nq <= Nk).
    Return (o [B,Hq,Nq,d], lse [B,Hq,Nq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (B, d) != (Bk, dk) or v.shape != k.shape or Hkv < 1 or Hq % Hkv or Nq > Nk:
        raise ValueError(f"bad shapes q{q.shape} k{k.shape} v{v.shape}")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.zeros((B, Hq, Nq, d))
    lse = np.zeros((B, Hq, Nq))
    (lib or load()).oracle_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                       B, Hq, Hkv, Nq, Nk, d, int(causal), float(scale))
    return o, lse


def attn_bwd(q, k, v, dout, causal: int = 1, scale: float | None = None, lib=None
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Return (dq [B,Hq,N,d], dk [B,Hkv,N,d], dv [B,Hkv,N,d]) in float64."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Hkv, N, d = _dims(q, k)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    (lib or load()).oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                    _ptr(dq), _ptr(dk), _ptr(dv),
                                    B, Hq, Hkv, N, d, int(causal), float(scale))
    return dq, dk, dv


def attn_sampled(q, k, v, dout, b: int, hkv: int, rows, keys, causal: int = 1,
                 scale: float | None = None, lib=None):
    """Sampled outputs of the (b, hkv) unit, for shapes too large for the full oracle.

    rows: list of (g, i) with g the query head's index inside the group
    (query head hq = hkv * group + g) and i the query row; keys: list of key rows.
    Returns dict with o [R,d], lse [R], dq [R,d], dk [K,d], dv [K,d] (float64).
    Only the unit's slices are widened to float64.
    """
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qs = _f64(q[b, hkv * G:(hkv + 1) * G])
    dos = _f64(dout[b, hkv * G:(hkv + 1) * G])
    ks, vs = _f64(k[b, hkv]), _f64(v[b, hkv])
    N, d = ks.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rg = np.ascontiguousarray([g for g, _ in rows], dtype=np.int32)
    ri = np.ascontiguousarray([i for _, i in rows], dtype=np.int32)
    kj = np.ascontiguousarray(list(keys), dtype=np.int32)
    R, K = len(rg), len(kj)
    out = dict(o=np.zeros((R, d)), lse=np.zeros(R), dq=np.zeros((R, d)),
               dk=np.zeros((K, d)), dv=np.zeros((K, d)))
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    (lib or load()).oracle_attn_sampled(
        _ptr(qs), _ptr(ks), _ptr(vs), _ptr(dos), G, N, d, int(causal), float(scale),
        R, ip(rg), ip(ri), _ptr(out["o"]), _ptr(out["lse"]), _ptr(out["dq"]),
        K, ip(kj), _ptr(out["dk"]), _ptr(out["dv"]))
    return out


def threads(lib=None) -> int:
    """OpenMP threads the oracle will use (before capping by work units)."""
    return int((lib or load()).oracle_threads())


def _tables(cos, sin, N, d):
    cs, sn = _f64(cos), _f64(sin)
    if cs.shape != (N, d // 2) or sn.shape != (N, d // 2) or d % 2:
        raise ValueError(f"rope tables must be [N, d/2] = {(N, d // 2)}")
    return cs, sn


def attn_fwd_rope(q, k, v, cos, sin, causal: int = 1, scale: float | None = None, lib=None):
    """Forward with rotary position embedding (rotate-half pairing) of q and k;
    cos, sin: [N, d/2] tables. Returns (o, lse) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Hkv, N, d = _dims(q, k)
    cs, sn = _tables(cos, sin, N, d)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    (lib or load()).oracle_attn_fwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(cs), _ptr(sn), _ptr(o), _ptr(lse),
                                         B, Hq, Hkv, N, d, int(causal), float(scale))
    return o, lse


def attn_bwd_rope(q, k, v, dout, cos, sin, causal: int = 1, scale: float | None = None, lib=None):
    """Gradients of the unrotated q, k and of v for the rotary forward above."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Hkv, N, d = _dims(q, k)
    cs, sn = _tables(cos, sin, N, d)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    dq = np.zeros((B, Hq, N, d))
    dk = np.zeros((B, Hkv, N, d))
    dv = np.zeros((B, Hkv, N, d))
    (lib or load()).oracle_attn_bwd_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(cs), _ptr(sn),
                                         _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d, int(causal), float(scale))
    return dq, dk, dv
