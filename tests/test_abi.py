"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects every invalid argument before touching the GPU.

Validation happens on the host before any HIP call, so these calls use host
addresses (or made-up aligned addresses) and never launch anything.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import tiled_causal_attention_amd as tca
from tiled_causal_attention_amd import build as tca_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tca.h")

F32, BF16 = tca.ATTN_F32, tca.ATTN_BF16
OK, EINVAL, EUNSUP = tca.ATTN_OK, tca.ATTN_EINVAL, tca.ATTN_EUNSUPPORTED


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tca.LIB_PATH):
        tca_build.build()
    return tca.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("attn_fwd", "attn_bwd", "attn_bwd_workspace_bytes", "attn_status_str",
                     "attn_bwd_dq", "attn_bwd_dkdv", "attn_fwd_workspace_bytes",
                     "attn_abi_version", "attn_decode", "attn_decode_workspace_bytes",
                     "attn_fwd_naive", "attn_fwd_naive_workspace_bytes", "attn_fwd_rope", "attn_bwd_rope",
                     "attn_fwd_rope_workspace_bytes", "attn_bwd_rope_workspace_bytes", "attn_decode_noalloc"):
        assert required in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_exports_are_c_symbols():
    out = os.popen(f"nm -D --defined-only {tca.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(L):
    assert L.attn_abi_version() == 4 == tca.ABI_VERSION
    for s in (OK, EINVAL, EUNSUP, tca.ATTN_EHIP, tca.ATTN_ESCRATCH):
        assert L.attn_status_str(s)
    assert b"unknown" in L.attn_status_str(99)


def test_workspace_sizes(L):
    assert L.attn_fwd_workspace_bytes(BF16, 8, 12, 4, 1024, 64) == 0
    rows = 8 * 12 * 1024
    # matrix-core path: D and base-2 lse (float32 per row), fp16 copies of q and dO
    n = L.attn_bwd_workspace_bytes(BF16, 8, 12, 4, 1024, 64)
    assert n == 2 * rows * 4 + 2 * rows * 64 * 2 and n % 256 == 0
    # float32 path (and bf16 with small d): D only, rounded up to 256 bytes
    assert L.attn_bwd_workspace_bytes(F32, 1, 2, 1, 3, 16) == 256
    assert L.attn_bwd_workspace_bytes(BF16, 1, 2, 1, 3, 32) == 256
    assert L.attn_bwd_workspace_bytes(BF16, 1, 2, 1, 3, 128) == 256 + 256 + 2 * (6 * 128 * 2)


# A made-up, 16-byte-aligned address: never dereferenced because every call
# below fails validation (or is a no-op) before any HIP call.
FAKE = 0x10000


def fwd(L, dtype=BF16, out_dtype=F32, B=2, Hq=4, Hkv=2, N=64, d=64, causal=1, scale=0.125,
        q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=None, wsb=0):
    return L.attn_fwd(dtype, out_dtype, q, k, v, o, lse, ws, wsb, B, Hq, Hkv, N, d, causal, scale, None)


def bwd(L, name="attn_bwd", dtype=BF16, out_dtype=F32, B=2, Hq=4, Hkv=2, N=64, d=64, causal=1,
        scale=0.125, ptrs=None, ws=FAKE, wsb=1 << 20):
    p = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dO=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
    p.update(ptrs or {})
    return getattr(L, name)(dtype, out_dtype, p["q"], p["k"], p["v"], p["o"], p["lse"], p["dO"], p["dq"],
                            p["dk"], p["dv"], ws, wsb, B, Hq, Hkv, N, d, causal, scale, None)


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=7), EINVAL),
    (dict(out_dtype=2), EINVAL),
    (dict(out_dtype=-1), EINVAL),
    (dict(out_dtype=BF16, o=FAKE + 8), EINVAL),   # bf16 o: still 16-byte aligned
    (dict(B=-1), EINVAL),
    (dict(N=-5), EINVAL),
    (dict(Hq=0), EINVAL),
    (dict(Hkv=0), EINVAL),
    (dict(Hq=12, Hkv=5), EINVAL),
    (dict(Hq=2, Hkv=4), EINVAL),
    (dict(causal=2), EINVAL),
    (dict(causal=-1), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL),
    (dict(N=1 << 25, d=64), EINVAL),           # N*d overflows int32
    (dict(N=(1 << 25) - 64, d=64), EINVAL),    # the tail tile's rows would pass 2^31 elements
    (dict(B=1 << 20, Hq=4096, Hkv=4096, N=1024, d=16), EINVAL),   # B*Hq*N overflows
    (dict(d=48), EUNSUP),
    (dict(d=256), EUNSUP),
    (dict(d=8), EUNSUP),
    (dict(q=None), EINVAL),
    (dict(k=None), EINVAL),
    (dict(v=None), EINVAL),
    (dict(o=None), EINVAL),
    (dict(lse=None), EINVAL),
    (dict(q=FAKE + 8), EINVAL),              # not 16-byte aligned
    (dict(o=FAKE + 4), EINVAL),
    (dict(lse=FAKE + 2), EINVAL),
])
def test_fwd_rejects(L, kw, want):
    assert fwd(L, **kw) == want


@pytest.mark.parametrize("name", ["attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv"])
@pytest.mark.parametrize("kw,want", [
    (dict(dtype=3), EINVAL),
    (dict(out_dtype=5), EINVAL),
    (dict(out_dtype=BF16, ptrs=dict(dq=FAKE + 2)), EINVAL),
    (dict(Hq=6, Hkv=4), EINVAL),
    (dict(causal=5), EINVAL),
    (dict(d=96), EUNSUP),
    (dict(ws=None), EINVAL),
    (dict(ws=FAKE + 8), EINVAL),
    (dict(wsb=100), EINVAL),                  # smaller than attn_bwd_workspace_bytes
    (dict(ptrs=dict(dO=None)), EINVAL),
    (dict(ptrs=dict(dq=None)), EINVAL),
    (dict(ptrs=dict(dk=FAKE + 4)), EINVAL),
    (dict(ptrs=dict(dv=None)), EINVAL),
    (dict(ptrs=dict(o=None)), EINVAL),
    (dict(ptrs=dict(lse=FAKE + 12)), EINVAL),
])
def test_bwd_rejects(L, name, kw, want):
    assert bwd(L, name, **kw) == want


def test_empty_inputs_are_noops(L):
    # B*N == 0: OK without touching (or needing) any pointer
    assert fwd(L, B=0, q=None, k=None, v=None, o=None, lse=None) == OK
    assert fwd(L, N=0, q=None, k=None, v=None, o=None, lse=None) == OK
    nul = dict(q=None, k=None, v=None, o=None, lse=None, dO=None, dq=None, dk=None, dv=None)
    for name in ("attn_bwd", "attn_bwd_dq", "attn_bwd_dkdv"):
        assert bwd(L, name, B=0, ptrs=nul, ws=None, wsb=0) == OK
        assert bwd(L, name, N=0, ptrs=nul, ws=None, wsb=0) == OK
    # but an empty call with an invalid flag or dtype is still rejected
    assert fwd(L, B=0, causal=3) == EINVAL
    assert fwd(L, B=0, out_dtype=9) == EINVAL


def test_outputs_untouched_on_error(L):
    # host buffers passed as pointers: validation fails, so nothing is written
    o = np.full(4 * 64 * 64, 7.0, dtype=np.float32)
    lse = np.full(4 * 64, 7.0, dtype=np.float32)
    st = fwd(L, B=1, Hq=4, Hkv=3, N=64, d=64, o=o.ctypes.data, lse=lse.ctypes.data)
    assert st == EINVAL
    assert (o == 7.0).all() and (lse == 7.0).all()


def test_python_binding_checks_output_dtypes():
    import torch
    q = torch.zeros(1, 2, 8, 16)
    with pytest.raises(TypeError):
        tca._code(torch.float16)
    o32, obf = torch.zeros(1, 2, 8, 16), torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    # out tensors that disagree with out_dtype, or a non-float32 lse, are refused before any call
    with pytest.raises(TypeError):
        tca.attn_fwd(q, q, q, out=(o32, lse), out_dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tca.attn_fwd(q, q, q, out=(obf, lse.bfloat16()))
    with pytest.raises(TypeError):
        tca.attn_bwd(q, q, q, obf, lse, q, out=(obf, o32, obf), workspace=torch.zeros(1))


def test_python_binding_checks_every_shape():
    """Each tensor is checked against q's and k's sizes before any pointer reaches the
    C ABI (the kernels size their walks from B, Hq, Hkv, N, d alone). The checks come
    before the device check, so they are visible here on CPU tensors."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(2, 6, 40, 64, dtype=bf)
    k = torch.zeros(2, 2, 40, 64, dtype=bf)
    o, lse = torch.zeros(2, 6, 40, 64), torch.zeros(2, 6, 40)
    dq, dk = torch.zeros(2, 6, 40, 64), torch.zeros(2, 2, 40, 64)
    ws = torch.zeros(16, dtype=torch.uint8)
    cases = [
        (lambda: tca.attn_fwd(q, k[:, :, :39], k), "k has shape"),
        (lambda: tca.attn_fwd(q, k, k[:, :, :39]), "v has shape"),
        (lambda: tca.attn_fwd(q, k[:1], k[:1]), "k has shape"),
        (lambda: tca.attn_fwd(q, k[..., :32], k[..., :32]), "k has shape"),
        (lambda: tca.attn_fwd(q, k, k, out=(o[:, :, :39], lse)), "o has shape"),
        (lambda: tca.attn_fwd(q, k, k, out=(o, lse[:1])), "lse has shape"),
        (lambda: tca.attn_bwd(q, k, k, o, lse, q[:, :, :20], workspace=ws), "dO has shape"),
        (lambda: tca.attn_bwd(q, k, k, o[:1], lse, q, workspace=ws), "o has shape"),
        (lambda: tca.attn_bwd(q, k, k, o, lse, q, out=(dq[:, :3], dk, dk), workspace=ws), "dq has shape"),
        (lambda: tca.attn_bwd(q, k, k, o, lse, q, out=(dq, dk[:, :1], dk), workspace=ws), "dk has shape"),
        (lambda: tca.attn_bwd(q, k, k, o, lse, q, out=(dq, dk, dk[:, :, :8]), workspace=ws), "dv has shape"),
        (lambda: tca.attn_decode(q[:, :, :1], k, k[:, :, :20]), "v has shape"),
        (lambda: tca.attn_decode(q[:, :, :1], k, k, out=(o[:, :, :2], lse[:, :, :1])), "o has shape"),
        (lambda: tca.attn_fwd_naive(q, k, k[:, :1]), "v has shape"),
        (lambda: tca.attn_fwd_rope(q, k, k[:, :, :5]), "v has shape"),
        (lambda: tca.attn_bwd_rope(q, k, k, o, lse, q, out=(dq, dk, dk[:1]), workspace=ws), "dv has shape"),
    ]
    for fn, msg in cases:
        with pytest.raises(ValueError, match=msg):
            fn()
    with pytest.raises(TypeError, match="k is"):
        tca.attn_fwd(q, k.float(), k.float())
    with pytest.raises(TypeError, match="dO is"):
        tca.attn_bwd(q, k, k, o, lse, q.float(), workspace=ws)
    with pytest.raises(TypeError, match="dq, dk, dv"):
        tca.attn_bwd(q, k, k, o, lse, q, out=(dq.bfloat16(), dk, dk), workspace=ws)


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 16)
    with pytest.raises(ValueError):
        tca.attn_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous())


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tca, "_lib", None)
    monkeypatch.setattr(tca, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        tca.lib()


def dec(L, dtype=BF16, out_dtype=F32, B=2, Hq=4, Hkv=2, Nq=1, Nk=64, d=64, causal=1, scale=0.125,
        q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 20):
    return L.attn_decode(dtype, out_dtype, q, k, v, o, lse, ws, wsb, B, Hq, Hkv, Nq, Nk, d, causal, scale, None)


@pytest.mark.parametrize("kw,want", [
    (dict(dtype=4), EINVAL),
    (dict(out_dtype=3), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(Nq=-1), EINVAL),
    (dict(Nq=65, Nk=64), EINVAL),              # more queries than cached positions
    (dict(Hq=6, Hkv=4), EINVAL),
    (dict(causal=2), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(Nk=1 << 22, d=128), EINVAL),         # K/V byte offsets of a head pass 2^31
    (dict(d=80), EUNSUP),
    (dict(q=None), EINVAL),
    (dict(k=FAKE + 8), EINVAL),
    (dict(o=None), EINVAL),
    (dict(lse=FAKE + 4), EINVAL),
    (dict(Nk=4096, ws=None), EINVAL),          # split keys need the workspace
    (dict(Nk=4096, wsb=64), EINVAL),
    (dict(Nk=4096, ws=FAKE + 8), EINVAL),
])
def test_decode_rejects(L, kw, want):
    assert dec(L, **kw) == want


def test_decode_noalloc_validation(L):
    """The allocation-free decode checks its arguments like attn_decode and refuses,
    before any HIP call, sizes whose split partials exceed its fixed array."""
    def nd(dtype=BF16, out_dtype=F32, B=2, Hq=4, Hkv=2, Nq=1, Nk=64, d=64, causal=1, scale=0.125,
           q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE):
        return L.attn_decode_noalloc(dtype, out_dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale,
                                     None)
    assert nd(dtype=4) == EINVAL and nd(Nq=65) == EINVAL and nd(Hq=6, Hkv=4) == EINVAL
    assert nd(causal=2) == EINVAL and nd(scale=float("inf")) == EINVAL and nd(d=80) == EUNSUP
    assert nd(q=None) == EINVAL and nd(k=FAKE + 8) == EINVAL
    nul = dict(q=None, k=None, v=None, o=None, lse=None)
    assert nd(B=0, **nul) == OK and nd(Nq=0, **nul) == OK
    big = dict(B=1, Hq=16, Hkv=2, Nq=8, Nk=16384, d=128)
    need = L.attn_decode_workspace_bytes(BF16, *big.values())
    assert need > tca.DECODE_SCRATCH_BYTES
    assert nd(**big) == tca.ATTN_ESCRATCH
    assert b"ESCRATCH" in L.attn_status_str(tca.ATTN_ESCRATCH)
    header = open(HEADER).read()
    assert re.search(r"#define ATTN_DECODE_SCRATCH_BYTES \(16u << 20\)", header)


def test_decode_noops_and_workspace(L):
    nul = dict(q=None, k=None, v=None, o=None, lse=None, ws=None, wsb=0)
    assert dec(L, B=0, **nul) == OK
    assert dec(L, Nq=0, **nul) == OK
    assert dec(L, B=0, causal=3, **nul) == EINVAL
    # one split: no workspace; more: partial outputs and LSEs, 256-byte parts, unless
    # the call has >= 256 row groups of <= 16 splits each, merged inside one workgroup
    # (bf16 calls at d = 64 or 128 with 3+ rows per KV head merge in the matrix-core
    # form from 128 chunks of 32 rows; with fewer chunks, 8+ rows at d = 128 take the
    # matrix-core split instead, when its partials fit the no-allocation scratch)
    assert L.attn_decode_workspace_bytes(BF16, 1, 2, 1, 1, 64, 64) == 0
    n = L.attn_decode_workspace_bytes(BF16, 8, 12, 4, 1, 1024, 64)              # 32 groups of 16 splits
    rows = 8 * 12
    assert n > 0 and n % 256 == 0
    nsplit = round(n / (rows * 64 * 4 + rows * 4))
    assert nsplit == 16
    assert n == ((nsplit * rows * 64 * 4 + 255) // 256 + (nsplit * rows * 4 + 255) // 256) * 256
    assert L.attn_decode_workspace_bytes(BF16, 64, 12, 4, 1, 1024, 64) == 0     # 256 groups of 16 splits
    # float32 queries of 4 rows: at most 8 splits per workgroup
    assert L.attn_decode_workspace_bytes(F32, 128, 8, 2, 1, 400, 64) == 0        # 7 splits
    assert L.attn_decode_workspace_bytes(F32, 128, 8, 2, 1, 600, 64) > 0         # 10 splits
    assert L.attn_decode_workspace_bytes(BF16, 128, 8, 2, 1, 600, 64) == 0    # 4 rows: merged
    assert L.attn_decode_workspace_bytes(BF16, 256, 8, 1, 1, 512, 64) == 0    # 8 rows at d = 64: merged
    assert L.attn_decode_workspace_bytes(BF16, 256, 8, 1, 1, 512, 128) == 0   # 8 rows at d = 128: merged
    assert L.attn_decode_workspace_bytes(F32, 256, 8, 1, 1, 512, 128) == 0    # float32: merged
    assert L.attn_decode_workspace_bytes(BF16, 32, 12, 4, 1, 1024, 64) == 0  # 128 chunks: merged
    assert L.attn_decode_workspace_bytes(BF16, 16, 12, 4, 1, 1024, 64) > 0   # 64 chunks: split
    n = L.attn_decode_workspace_bytes(BF16, 64, 32, 1, 1, 512, 128)   # 256 8-row chunks, 64 of 32 rows
    rows, nsplit = 64 * 32, 8                                          # -> the matrix-core split
    assert n == ((nsplit * rows * 128 * 4 + 255) // 256 + (nsplit * rows * 4 + 255) // 256) * 256
    assert L.attn_decode_workspace_bytes(BF16, 8, 12, 4, 2, 1, 64) == 0   # invalid: Nq > Nk


def test_naive_validation(L):
    assert L.attn_fwd_naive_workspace_bytes(8, 12, 1024) == 8 * 12 * 1024 * 1024 * 4
    assert L.attn_fwd_naive_workspace_bytes(-1, 12, 1024) == 0
    args = lambda **kw: dict(dict(dtype=BF16, out=F32, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, ws=FAKE,
                                  wsb=1 << 30, B=2, Hq=4, Hkv=2, N=64, d=64, causal=1, scale=0.125), **kw)
    call = lambda a: L.attn_fwd_naive(a["dtype"], a["out"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"],
                                      a["wsb"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                                      a["scale"], None)
    assert call(args(ws=None)) == EINVAL
    assert call(args(wsb=2 * 4 * 64 * 64 * 4 - 1)) == EINVAL       # one byte short of the score matrix
    assert call(args(Hq=6, Hkv=4)) == EINVAL
    assert call(args(out=7)) == EINVAL
    assert call(args(d=48)) == EUNSUP
    assert call(args(B=0, q=None, ws=None, wsb=0)) == OK
    assert call(args(B=64, Hq=64, Hkv=64, N=16384, d=16, wsb=0)) == EINVAL   # B*Hq*N*N >= 2^39


def test_rope_validation(L):
    import ctypes
    lay = lambda sb, sh, sn: ctypes.byref(tca.AttnLayout(sb, sh, sn))
    nq, nk = 2 * 4 * 64 * 64, 2 * 2 * 64 * 64
    rnd = lambda n: (n + 255) // 256 * 256
    # forward: q, k, v copies; backward adds float32 gradients (and a float32 o for bf16 outputs)
    # and attn_bwd's own workspace
    assert L.attn_fwd_rope_workspace_bytes(BF16, F32, 2, 4, 2, 64, 64) == rnd(nq * 2) + 2 * rnd(nk * 2)
    bwd = L.attn_bwd_rope_workspace_bytes(BF16, BF16, 2, 4, 2, 64, 64)
    assert bwd == (rnd(nq * 2) + 2 * rnd(nk * 2) + rnd(nq * 4) + rnd(nq * 4) + 2 * rnd(nk * 4)
                   + L.attn_bwd_workspace_bytes(BF16, 2, 4, 2, 64, 64))

    def fwd_rope(cos=FAKE, sin=FAKE, ql=None, q=FAKE, d=64, ws=FAKE, wsb=1 << 30, kr=None, **kw):
        a = dict(dtype=BF16, out=F32, B=2, Hq=4, Hkv=2, N=64, causal=1, scale=0.125)
        a.update(kw)
        return L.attn_fwd_rope(a["dtype"], a["out"], q, ql, FAKE, None, FAKE, None, cos, sin, kr, FAKE, FAKE, ws,
                               wsb, a["B"], a["Hq"], a["Hkv"], a["N"], d, a["causal"], a["scale"], None)

    def bwd_rope(kr=None, dq=FAKE, ws=FAKE, wsb=1 << 30, **kw):
        a = dict(dtype=BF16, out=F32, B=2, Hq=4, Hkv=2, N=64, d=64, causal=1, scale=0.125)
        a.update(kw)
        return L.attn_bwd_rope(a["dtype"], a["out"], FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, kr, FAKE, FAKE,
                               FAKE, dq, None, FAKE, None, FAKE, None, ws, wsb, a["B"], a["Hq"], a["Hkv"], a["N"],
                               a["d"], a["causal"], a["scale"], None)
    assert fwd_rope(kr=FAKE + 8) == EINVAL              # the rotated-key buffer is 16-byte aligned
    assert bwd_rope(kr=FAKE + 8) == EINVAL
    assert bwd_rope(kr=FAKE, wsb=100) == EINVAL         # the workspace size does not shrink with k_rot
    assert bwd_rope(kr=FAKE, dq=FAKE + 2) == EINVAL     # float32 gradients need 4-byte alignment
    assert bwd_rope(kr=FAKE, B=0, ws=None, wsb=0) == OK
    assert fwd_rope(cos=None) == EINVAL                 # one table without the other
    assert fwd_rope(cos=FAKE + 4) == EINVAL             # tables 16-byte aligned
    assert fwd_rope(ql=lay(-1, 64, 64)) == EINVAL       # negative stride
    assert fwd_rope(q=FAKE + 1) == EINVAL               # bf16 needs 2-byte alignment
    assert fwd_rope(wsb=100) == EINVAL
    assert fwd_rope(ws=None) == EINVAL
    assert fwd_rope(d=80) == EUNSUP
    assert fwd_rope(B=0, q=None, ws=None, wsb=0) == OK
    assert fwd_rope(causal=4) == EINVAL
