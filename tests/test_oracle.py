"""Pins for the float64 CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * a library routine: torch's float64 CPU scaled_dot_product_attention
    (is_causal, enable_gqa) and autograd through it;
  * the gradient check the NanoEuler pages describe (FAQ, "How does gradient
    checking work"): central finite differences with epsilon 1e-5, relative
    error below 1e-4;
  * closed forms (scale 0, V = ones, N = 1, query row 0);
  * invariants of the mathematics (softmax shift invariance, sum of dV, the
    Q/K rescaling identity, GQA equals MHA with repeated K/V);
  * hand-worked examples under tests/golden/;
  * rotary position embedding: torch autograd through the rotation and SDPA, a
    hand-worked direction example, position-shift invariance, identity tables;
  * few-query (decode) attention over a cache: torch's SDPA with an explicit
    bottom-right causal mask, the last rows of a full-sequence forward, and
    closed forms;
  * planted mistakes: mutated copies of oracle.c must fail at least one pin.
"""
import json
import math
import os
import re
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(B, Hq, Hkv, N, d, seed=0, std=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float64) * std
    k = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float64) * std
    v = torch.randn(B, Hkv, N, d, generator=g, dtype=torch.float64)
    do = torch.randn(B, Hq, N, d, generator=g, dtype=torch.float64)
    return q, k, v, do


def _torch_fwd(q, k, v, causal, scale):
    return F.scaled_dot_product_attention(q, k, v, is_causal=bool(causal), scale=scale,
                                          enable_gqa=True)


def _torch_lse(q, k, causal, scale):
    g = q.shape[1] // k.shape[1]
    kr = k.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(q, kr.transpose(-1, -2).contiguous())
    if causal:
        N = q.shape[2]
        mask = torch.ones(N, N, dtype=torch.bool).triu(1)
        s = s.masked_fill(mask, float("-inf"))
    return torch.logsumexp(s, dim=-1)


def _torch_bwd(q, k, v, do, causal, scale):
    q, k, v = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = _torch_fwd(q, k, v, causal, scale)
    o.backward(do)
    return q.grad, k.grad, v.grad


SHAPES = [
    # B, Hq, Hkv, N, d
    (1, 2, 1, 64, 16),
    (2, 4, 2, 17, 8),
    (1, 3, 1, 33, 5),
    (2, 6, 2, 40, 12),
    (1, 4, 4, 9, 7),
    (1, 12, 4, 31, 4),
    (1, 2, 1, 1, 3),
]


def _pin_failures(lib=None, shapes=SHAPES, atol=1e-10):
    """Run the library and hand-example pins; return a list of failure strings."""
    fails = []
    for (B, Hq, Hkv, N, d) in shapes:
        for causal in (1, 0):
            q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=N * 7 + d)
            scale = 1.0 / math.sqrt(d)
            o, lse = oracle.attn_fwd(q, k, v, causal, scale, lib=lib)
            ro = _torch_fwd(q, k, v, causal, scale).numpy()
            rl = _torch_lse(q, k, causal, scale).numpy()
            if not np.allclose(o, ro, atol=atol, rtol=0):
                fails.append(f"O vs sdpa {B,Hq,Hkv,N,d,causal}: {np.nanmax(np.abs(o - ro))}")
            if not np.allclose(lse, rl, atol=atol, rtol=0):
                fails.append(f"LSE vs logsumexp {B,Hq,Hkv,N,d,causal}: {np.nanmax(np.abs(lse - rl))}")
            dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale, lib=lib)
            tq, tk, tv = (t.numpy() for t in _torch_bwd(q, k, v, do, causal, scale))
            for nm, a, b in (("dQ", dq, tq), ("dK", dk, tk), ("dV", dv, tv)):
                if not np.allclose(a, b, atol=atol, rtol=0):
                    fails.append(f"{nm} vs autograd {B,Hq,Hkv,N,d,causal}: {np.nanmax(np.abs(a - b))}")
    fails += _sampled_failures(lib, atol)
    fails += _decode_failures(lib, atol)
    fails += _rope_failures(lib, atol)
    for fname in sorted(os.listdir(GOLDEN)):
        if not fname.endswith(".json"):
            continue
        ex = json.load(open(os.path.join(GOLDEN, fname)))
        if "cos" in ex:   # the rotary example, checked by _rope_failures
            continue
        arr = {kk: np.array(ex[kk], dtype=np.float64) for kk in ("q", "k", "v", "dO", "o", "lse", "dq", "dk", "dv")}
        o, lse = oracle.attn_fwd(arr["q"], arr["k"], arr["v"], ex["causal"], ex["scale"], lib=lib)
        dq, dk, dv = oracle.attn_bwd(arr["q"], arr["k"], arr["v"], arr["dO"], ex["causal"], ex["scale"], lib=lib)
        for nm, a in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            if not np.allclose(a, arr[nm], atol=1e-12, rtol=0):
                fails.append(f"golden {fname} {nm}: got {a.ravel()} want {arr[nm].ravel()}")
    return fails


DECODE_SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 2, 1, 1, 1, 4),
    (2, 6, 2, 1, 37, 8),
    (1, 4, 1, 3, 20, 5),
    (2, 4, 4, 7, 7, 6),
    (1, 12, 4, 5, 64, 16),
]


def _bottom_right_mask(Nq, Nk):
    """Query row i (sequence position Nk - Nq + i) sees keys j <= Nk - Nq + i."""
    return torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)


def _decode_failures(lib=None, atol=1e-10):
    """Few-query attention over a cache against torch's float64 CPU
    scaled_dot_product_attention with an explicit bottom-right causal mask, and
    LSE against torch.logsumexp of the same masked scores."""
    fails = []
    for (B, Hq, Hkv, Nq, Nk, d) in DECODE_SHAPES:
        G = Hq // Hkv
        for causal in (1, 0):
            gen = torch.Generator("cpu").manual_seed(Nq * 131 + Nk + causal)
            q = torch.randn(B, Hq, Nq, d, generator=gen, dtype=torch.float64)
            k = torch.randn(B, Hkv, Nk, d, generator=gen, dtype=torch.float64)
            v = torch.randn(B, Hkv, Nk, d, generator=gen, dtype=torch.float64)
            scale = 1.0 / math.sqrt(d)
            o, lse = oracle.attn_decode(q, k, v, causal, scale, lib=lib)
            kr, vr = k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1)
            mask = _bottom_right_mask(Nq, Nk) if causal else torch.ones(Nq, Nk, dtype=torch.bool)
            ro = F.scaled_dot_product_attention(q, kr, vr, attn_mask=mask, scale=scale).numpy()
            sc = (scale * torch.matmul(q, kr.transpose(-1, -2).contiguous())).masked_fill(~mask, float("-inf"))
            rl = torch.logsumexp(sc, dim=-1).numpy()
            if not np.allclose(o, ro, atol=atol, rtol=0):
                fails.append(f"decode O vs sdpa {B,Hq,Hkv,Nq,Nk,d,causal}: {np.nanmax(np.abs(o - ro))}")
            if not np.allclose(lse, rl, atol=atol, rtol=0):
                fails.append(f"decode LSE vs logsumexp {B,Hq,Hkv,Nq,Nk,d,causal}: {np.nanmax(np.abs(lse - rl))}")
    return fails


def test_decode_matches_library():
    assert _decode_failures() == []


@pytest.mark.parametrize("causal", [1, 0])
def test_decode_rows_equal_last_rows_of_full_sequence(causal):
    # the last Nq rows of attention over the whole sequence do not depend on the
    # earlier query rows: a full-length query block whose tail is the decode
    # queries gives the decode result in its last Nq rows
    B, Hq, Hkv, Nq, Nk, d = 2, 6, 2, 4, 45, 8
    g = torch.Generator("cpu").manual_seed(77)
    qf = torch.randn(B, Hq, Nk, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    of, lf = oracle.attn_fwd(qf, k, v, causal, 0.4)
    od, ld = oracle.attn_decode(qf[:, :, Nk - Nq:].contiguous(), k, v, causal, 0.4)
    assert np.allclose(od, of[:, :, Nk - Nq:], atol=1e-13, rtol=0)
    assert np.allclose(ld, lf[:, :, Nk - Nq:], atol=1e-13, rtol=0)


def test_decode_closed_forms():
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 5, 12, 3
    g = torch.Generator("cpu").manual_seed(5)
    q = torch.randn(B, Hq, Nq, d, generator=g, dtype=torch.float64)
    k = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    v = torch.randn(B, Hkv, Nk, d, generator=g, dtype=torch.float64)
    # scale 0: uniform weights over the visible prefix of each query's position
    o, lse = oracle.attn_decode(q, k, v, 1, 0.0)
    vn = v.numpy()
    for hq in range(Hq):
        for i in range(Nq):
            p = Nk - Nq + i
            assert np.allclose(o[0, hq, i], vn[0, hq // 2, :p + 1].mean(0), atol=1e-14)
            assert abs(lse[0, hq, i] - math.log(p + 1)) < 1e-14
    o, lse = oracle.attn_decode(q, k, v, 0, 0.0)
    assert np.allclose(o[0, 0, 0], vn[0, 0].mean(0), atol=1e-14) and np.allclose(lse, math.log(Nk))
    # V = ones: O = 1
    o, _ = oracle.attn_decode(q, k, torch.ones_like(v), 1, 0.7)
    assert np.allclose(o, 1.0, atol=1e-14)
    # a single cached key: O = V_0, LSE = scale <q, k_0>
    o, lse = oracle.attn_decode(q[:, :, :1].contiguous(), k[:, :, :1].contiguous(), v[:, :, :1].contiguous(), 1, 0.7)
    assert np.allclose(o[0, :, 0], vn[0, [0, 0, 1, 1], 0], atol=1e-14)
    kq = (q[0, :, 0].numpy() * k[0, [0, 0, 1, 1], 0].numpy()).sum(-1)
    assert np.allclose(lse[0, :, 0], 0.7 * kq, atol=1e-14)


def rope_tables(N, d, base=10000.0, offset=0):
    """cos/sin [N, d/2] of (n + offset) * base^(-2i/d), float64."""
    n = torch.arange(N, dtype=torch.float64)[:, None] + offset
    inv = base ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = n * inv[None, :]
    return torch.cos(ang), torch.sin(ang)


def _torch_rotate(x, cos, sin):
    # rotate-half pairing written with torch ops (x1, x2 the two halves of the head dimension)
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def _rope_failures(lib=None, atol=1e-10):
    """Rotary forward/backward against torch float64: the rotation in torch ops, SDPA,
    autograd through both (so the backward's transpose rotation is pinned by autograd);
    plus the hand-worked direction example in tests/golden."""
    fails = []
    for (B, Hq, Hkv, N, d) in [(1, 2, 1, 9, 4), (2, 6, 2, 17, 8), (1, 4, 4, 12, 6)]:
        for causal in (1, 0):
            q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=N + d + causal)
            cos, sin = rope_tables(N, d, base=100.0)
            scale = 1.0 / math.sqrt(d)
            o, lse = oracle.attn_fwd_rope(q, k, v, cos, sin, causal, scale, lib=lib)
            dq, dk, dv = oracle.attn_bwd_rope(q, k, v, do, cos, sin, causal, scale, lib=lib)
            qt, kt, vt = (t.clone().requires_grad_(True) for t in (q, k, v))
            qr, kr = _torch_rotate(qt, cos, sin), _torch_rotate(kt, cos, sin)
            ot = _torch_fwd(qr, kr, vt, causal, scale)
            ot.backward(do)
            rl = _torch_lse(qr.detach(), kr.detach(), causal, scale).numpy()
            for nm, a, b in (("o", o, ot.detach().numpy()), ("lse", lse, rl), ("dq", dq, qt.grad.numpy()),
                             ("dk", dk, kt.grad.numpy()), ("dv", dv, vt.grad.numpy())):
                if not np.allclose(a, b, atol=atol, rtol=0):
                    fails.append(f"rope {nm} vs torch {B,Hq,Hkv,N,d,causal}: {np.nanmax(np.abs(a - b))}")
    ex = json.load(open(os.path.join(GOLDEN, "rope_direction_n2_d2.json")))
    arr = {kk: np.array(ex[kk], dtype=np.float64) for kk in ("q", "k", "v", "cos", "sin", "o", "lse")}
    o, lse = oracle.attn_fwd_rope(arr["q"], arr["k"], arr["v"], arr["cos"], arr["sin"], ex["causal"], ex["scale"],
                                  lib=lib)
    if not (np.allclose(o, arr["o"], atol=1e-12) and np.allclose(lse, arr["lse"], atol=1e-12)):
        fails.append(f"rope golden: o {o.ravel()} lse {lse.ravel()}")
    return fails


def test_rope_matches_torch_and_golden():
    assert _rope_failures() == []


@pytest.mark.parametrize("causal", [1, 0])
def test_rope_depends_on_relative_position_only(causal):
    # shifting every position by the same amount rotates q and k alike: scores,
    # hence O and LSE, are unchanged, and so are the gradients
    B, Hq, Hkv, N, d = 2, 4, 2, 20, 8
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=8)
    c0, s0 = rope_tables(N, d)
    c1, s1 = rope_tables(N, d, offset=37)
    o0, l0 = oracle.attn_fwd_rope(q, k, v, c0, s0, causal, 0.3)
    o1, l1 = oracle.attn_fwd_rope(q, k, v, c1, s1, causal, 0.3)
    assert np.allclose(o0, o1, atol=1e-12) and np.allclose(l0, l1, atol=1e-12)
    # and a real rotation does change the result against no rotation
    o2, _ = oracle.attn_fwd(q, k, v, causal, 0.3)
    assert np.abs(o2 - o0).max() > 1e-3


def test_rope_identity_tables_equal_plain_attention():
    B, Hq, Hkv, N, d = 1, 6, 3, 15, 4
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=10)
    one, zero = torch.ones(N, d // 2, dtype=torch.float64), torch.zeros(N, d // 2, dtype=torch.float64)
    for causal in (1, 0):
        a = oracle.attn_fwd_rope(q, k, v, one, zero, causal, 0.5) + oracle.attn_bwd_rope(q, k, v, do, one, zero, causal, 0.5)
        b = oracle.attn_fwd(q, k, v, causal, 0.5) + oracle.attn_bwd(q, k, v, do, causal, 0.5)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def _sampled_failures(lib=None, atol=1e-10):
    """The sampled-output entry against torch autograd on small shapes."""
    fails = []
    for (B, Hq, Hkv, N, d) in [(2, 6, 2, 37, 8), (1, 4, 1, 20, 16)]:
        G = Hq // Hkv
        for causal in (1, 0):
            q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=N + 100 * causal)
            scale = 1.0 / math.sqrt(d)
            ro = _torch_fwd(q, k, v, causal, scale).numpy()
            rl = _torch_lse(q, k, causal, scale).numpy()
            tq, tk, tv = (t.numpy() for t in _torch_bwd(q, k, v, do, causal, scale))
            b, hkv = B - 1, Hkv - 1
            rows = [(g, i) for g in range(G) for i in (0, 1, N // 2, N - 1)]
            keys = [0, 1, N // 3, N - 2, N - 1]
            got = oracle.attn_sampled(q, k, v, do, b, hkv, rows, keys, causal, scale, lib=lib)
            for r, (g, i) in enumerate(rows):
                hq = hkv * G + g
                for nm, a, want in (("o", got["o"][r], ro[b, hq, i]), ("lse", got["lse"][r], rl[b, hq, i]),
                                    ("dq", got["dq"][r], tq[b, hq, i])):
                    if not np.allclose(a, want, atol=atol, rtol=0):
                        fails.append(f"sampled {nm} row {(g, i)} of {B,Hq,Hkv,N,d,causal}")
            for t, j in enumerate(keys):
                for nm, a, want in (("dk", got["dk"][t], tk[b, hkv, j]), ("dv", got["dv"][t], tv[b, hkv, j])):
                    if not np.allclose(a, want, atol=atol, rtol=0):
                        fails.append(f"sampled {nm} key {j} of {B,Hq,Hkv,N,d,causal}")
    return fails


def test_sampled_entry_matches_full_oracle():
    B, Hq, Hkv, N, d = 2, 6, 3, 45, 8
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=77, std=2.0)
    o, lse = oracle.attn_fwd(q, k, v, 1)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 1)
    rows = [(g, i) for g in range(2) for i in range(N)]
    got = oracle.attn_sampled(q, k, v, do, 1, 2, rows, list(range(N)), 1)
    assert np.allclose(got["o"].reshape(2, N, d), o[1, 4:6], atol=1e-13)
    assert np.allclose(got["lse"].reshape(2, N), lse[1, 4:6], atol=1e-13)
    assert np.allclose(got["dq"].reshape(2, N, d), dq[1, 4:6], atol=1e-13)
    assert np.allclose(got["dk"], dk[1, 2], atol=1e-13)
    assert np.allclose(got["dv"], dv[1, 2], atol=1e-13)


def test_library_and_golden_pins():
    assert _pin_failures() == []


def test_headline_shape_slice_vs_sdpa():
    # one (b, kv-head) slice of the GPT-2-small GQA shape: group 3, d=64, bf16-rounded inputs
    s = workloads.make_shape(1, 3, 1, 256, 64, seed=5)
    q, k, v, _ = (t.double() for t in workloads.make_inputs(s))
    o, lse = oracle.attn_fwd(q, k, v, 1, s.scale)
    assert np.allclose(o, _torch_fwd(q, k, v, 1, s.scale).numpy(), atol=1e-12, rtol=0)
    assert np.allclose(lse, _torch_lse(q, k, 1, s.scale).numpy(), atol=1e-12, rtol=0)


def _torch_explicit(q, k, v, causal, scale):
    # softmax(scale Q K^T, masked keys at -inf after scaling) V, built from plain torch ops
    # (torch's fused causal attention masks before it scales, which a negative scale breaks)
    g = q.shape[1] // k.shape[1]
    kr, vr = k.repeat_interleave(g, dim=1), v.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(q, kr.transpose(-1, -2).contiguous())
    if causal:
        N = q.shape[2]
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    return torch.matmul(torch.softmax(s, dim=-1), vr), torch.logsumexp(s, dim=-1)


@pytest.mark.parametrize("causal", [1, 0])
def test_negative_scale_vs_explicit_softmax(causal):
    # a negative scale flips which keys dominate; the definition holds for any finite scale
    for (B, Hq, Hkv, N, d), scale in (((2, 6, 2, 40, 12), -0.7), ((1, 4, 1, 33, 5), -2.0)):
        q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=N + 11)
        o, lse = oracle.attn_fwd(q, k, v, causal, scale)
        qq, kk, vv = (t.clone().requires_grad_(True) for t in (q, k, v))
        ro, rl = _torch_explicit(qq, kk, vv, causal, scale)
        assert np.allclose(o, ro.detach().numpy(), atol=1e-10, rtol=0)
        assert np.allclose(lse, rl.detach().numpy(), atol=1e-10, rtol=0)
        ro.backward(do)
        dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal, scale)
        for a, t in zip((dq, dk, dv), (qq, kk, vv)):
            assert np.allclose(a, t.grad.numpy(), atol=1e-10, rtol=0)


# ---------------------------------------------------------------- finite differences
def _fd_grads(q, k, v, G, causal, scale, eps=1e-5):
    """Central differences of L = sum(O * G) with respect to every input element."""
    out = []
    for which in range(3):
        base = [q.copy(), k.copy(), v.copy()]
        x = base[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = np.sum(oracle.attn_fwd(*base, causal, scale)[0] * G)
            x[idx] = orig - eps
            lm = np.sum(oracle.attn_fwd(*base, causal, scale)[0] * G)
            x[idx] = orig
            g[idx] = (lp - lm) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize("B,Hq,Hkv,N,d", [(1, 2, 1, 1, 3), (1, 2, 1, 5, 4), (1, 2, 1, 8, 3), (2, 4, 2, 7, 4)])
@pytest.mark.parametrize("causal", [1, 0])
def test_finite_difference_gradient_check(B, Hq, Hkv, N, d, causal):
    q, k, v, G = (t.numpy() for t in _inputs(B, Hq, Hkv, N, d, seed=3 + N))
    scale = 1.0 / math.sqrt(d)
    an = oracle.attn_bwd(q, k, v, G, causal, scale)
    fd = _fd_grads(q, k, v, G, causal, scale)
    for a, b in zip(an, fd):
        rel = np.abs(a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-3)
        assert rel.max() < 1e-4, rel.max()


# ---------------------------------------------------------------- closed forms
def test_scale_zero_closed_form():
    B, Hq, Hkv, N, d = 2, 4, 2, 23, 6
    q, k, v, do = (t.numpy() for t in _inputs(B, Hq, Hkv, N, d))
    vr = np.repeat(v, 2, axis=1)
    o, lse = oracle.attn_fwd(q, k, v, 1, 0.0)
    cnt = np.arange(1, N + 1, dtype=np.float64)
    assert np.allclose(o, np.cumsum(vr, axis=2) / cnt[:, None], atol=1e-12)
    assert np.allclose(lse, np.broadcast_to(np.log(cnt), lse.shape), atol=1e-12)
    o, lse = oracle.attn_fwd(q, k, v, 0, 0.0)
    assert np.allclose(o, np.broadcast_to(vr.mean(axis=2, keepdims=True), o.shape), atol=1e-12)
    assert np.allclose(lse, math.log(N), atol=1e-12)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 1, 0.0)
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    # dV_j = sum over the group and over i >= j of dO_i / (i + 1)
    w = do / cnt[None, None, :, None]
    tail = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    want = tail.reshape(B, Hkv, 2, N, d).sum(axis=2)
    assert np.allclose(dv, want, atol=1e-12)


def test_v_ones_closed_form():
    B, Hq, Hkv, N, d = 1, 6, 2, 19, 5
    q, k, _, do = (t.numpy() for t in _inputs(B, Hq, Hkv, N, d, std=2.0))
    v = np.ones((B, Hkv, N, d))
    for causal in (1, 0):
        o, _ = oracle.attn_fwd(q, k, v, causal)
        assert np.allclose(o, 1.0, atol=1e-13)
        dq, dk, _ = oracle.attn_bwd(q, k, v, do, causal)
        assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


def test_single_key_and_row_zero():
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, k, v, do = (t.numpy() for t in _inputs(B, Hq, Hkv, 1, d))
    o, lse = oracle.attn_fwd(q, k, v, 1)
    vr, kr = np.repeat(v, 2, axis=1), np.repeat(k, 2, axis=1)
    assert np.allclose(o, vr, atol=1e-14)
    assert np.allclose(lse, np.sum(q * kr, axis=-1)[..., 0:1] / math.sqrt(d), atol=1e-13)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 1)
    assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
    assert np.allclose(dv, do.reshape(B, Hkv, 2, 1, d).sum(axis=2), atol=1e-14)
    # causal row 0 of a longer sequence sees only key 0
    q, k, v, _ = (t.numpy() for t in _inputs(B, Hq, Hkv, 13, d))
    o, lse = oracle.attn_fwd(q, k, v, 1)
    vr, kr = np.repeat(v, 2, axis=1), np.repeat(k, 2, axis=1)
    assert np.allclose(o[:, :, 0], vr[:, :, 0], atol=1e-14)
    assert np.allclose(lse[:, :, 0], np.sum(q[:, :, 0] * kr[:, :, 0], axis=-1) / math.sqrt(d), atol=1e-13)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [1, 0])
def test_gradient_invariants(causal):
    B, Hq, Hkv, N, d = 2, 6, 2, 29, 7
    g = Hq // Hkv
    q, k, v, do = (t.numpy() for t in _inputs(B, Hq, Hkv, N, d, seed=11, std=1.5))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, causal)
    # softmax is invariant to adding one vector to every key: sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # rows of P sum to one: sum_j dV_j = sum over the group of sum_i dO_i
    assert np.allclose(dv.sum(axis=2), do.reshape(B, Hkv, g, N, d).sum(axis=(2, 3)), atol=1e-12)
    # S is unchanged by Q -> tQ, K -> K/t: <Q,dQ> = <K,dK> per (b, group)
    lhs = (q * dq).reshape(B, Hkv, g * N * d).sum(-1)
    rhs = (k * dk).reshape(B, Hkv, N * d).sum(-1)
    assert np.allclose(lhs, rhs, atol=1e-11)


def test_probability_rows_sum_to_one_via_lse():
    # sum_j exp(s_ij - LSE_i) = 1, with the scores built independently here
    B, Hq, Hkv, N, d = 1, 4, 1, 37, 9
    q, k, v, _ = _inputs(B, Hq, Hkv, N, d, seed=2, std=3.0)
    scale = 1.0 / math.sqrt(d)
    _, lse = oracle.attn_fwd(q, k, v, 1, scale)
    s = scale * np.einsum("bhid,bjd->bhij", q.numpy(), k[:, 0].numpy())
    p = np.exp(s - lse[..., None]) * np.tril(np.ones((N, N)))
    assert np.allclose(p.sum(-1), 1.0, atol=1e-13)


@pytest.mark.parametrize("g", [1, 2, 3, 4, 6])
def test_gqa_equals_mha_with_repeated_kv(g):
    B, Hkv, N, d = 2, 2, 21, 8
    Hq = Hkv * g
    q, k, v, do = (t.numpy() for t in _inputs(B, Hq, Hkv, N, d, seed=g))
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    o1, l1 = oracle.attn_fwd(q, k, v, 1)
    o2, l2 = oracle.attn_fwd(q, kr, vr, 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    dq1, dk1, dv1 = oracle.attn_bwd(q, k, v, do, 1)
    dq2, dk2, dv2 = oracle.attn_bwd(q, kr, vr, do, 1)
    assert np.array_equal(dq1, dq2)
    assert np.allclose(dk1, dk2.reshape(B, Hkv, g, N, d).sum(2), atol=1e-13)
    assert np.allclose(dv1, dv2.reshape(B, Hkv, g, N, d).sum(2), atol=1e-13)


def test_thread_count_does_not_change_bits():
    B, Hq, Hkv, N, d = 2, 4, 2, 50, 16
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed=9)
    code = (
        "import sys, numpy as np, torch; sys.path.insert(0, %r); import oracle\n"
        "g = torch.Generator('cpu').manual_seed(9)\n"
        "t = [torch.randn(*s, generator=g, dtype=torch.float64) for s in %r]\n"
        "r = oracle.attn_fwd(t[0], t[1], t[2], 1) + oracle.attn_bwd(t[0], t[1], t[2], t[3], 1)\n"
        "np.save(sys.argv[1], np.concatenate([x.ravel() for x in r]))\n"
    ) % (os.path.dirname(GOLDEN).rsplit("/tests", 1)[0],
         [(B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d), (B, Hq, N, d)])
    outs = []
    with tempfile.TemporaryDirectory() as td:
        for nt in ("1", "3"):
            f = os.path.join(td, f"r{nt}.npy")
            env = dict(os.environ, OMP_NUM_THREADS=nt)
            subprocess.run(["python", "-c", code, f], check=True, env=env)
            outs.append(np.load(f))
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------- planted mistakes
MUTANTS = [
    ("dropped scale in dQ", "dqi[c] += scale * ds *", "dqi[c] += ds *"),
    ("wrong sign of D in dS", "p * (dp[j] - D)", "p * (dp[j] + D)"),
    ("dropped D term", "p * (dp[j] - D)", "p * (dp[j])"),
    ("strided GQA head map", "const int hq = hkv * group + g;", "const int hq = g * Hkv + hkv;"),
    ("causal mask off by one", "return causal ? (j <= i) : 1;", "return causal ? (j <= i + 1 && j < 1000000) : 1;"),
    ("LSE without the max", "return m + log(l);", "return log(l);"),
    ("dK uses dO instead of Q", "dkh[(size_t)j * d + c] += scale * ds * qi[c];",
     "dkh[(size_t)j * d + c] += scale * ds * doi[c];"),
    ("dV uses P without dO", "dvh[(size_t)j * d + c] += p * doi[c];", "dvh[(size_t)j * d + c] += p * qi[c];"),
    ("sampled: dropped scale in dK", "dkj[c] += scale * ds * qi[c];", "dkj[c] += ds * qi[c];"),
    ("sampled: D without P", "D += exp(s[j] - L) * acc;", "D += acc;"),
    ("sampled: O row uses K", "oi[c] += s[j] * v[(size_t)j * d + c];", "oi[c] += s[j] * k[(size_t)j * d + c];"),
    ("decode: queries aligned to the start", "const int pos = Nk - Nq + i;", "const int pos = i;"),
    ("decode: position off by one", "const int pos = Nk - Nq + i;", "const int pos = Nk - Nq + i - 1;"),
    ("rope: opposite rotation direction", "row[i] = a * c - b * s;\n                row[i + h] = b * c + a * s;",
     "row[i] = a * c + b * s;\n                row[i + h] = b * c - a * s;"),
    ("rope: gradient rotated forward, not back", "rope_apply(dq, cs, sn, (size_t)B * Hq, N, d, 1);",
     "rope_apply(dq, cs, sn, (size_t)B * Hq, N, d, 0);"),
    ("rope: adjacent pairs", "const double a = row[i], b = row[i + h];", "const double a = row[2 * (i % (h / 2 > 0 ? h / 2 : 1))], b = row[i + h];"),
    ("transposed V index", "acc += doi[c] * vh[(size_t)j * d + c];", "acc += doi[c] * vh[(size_t)c * d + j % d];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = src.replace(old, new)
    csrc = tmp_path / "mutant.c"
    csrc.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(csrc), so)
    lib = oracle.load(so)
    shapes = [(1, 2, 1, 9, 4), (2, 4, 2, 12, 3)]
    with np.errstate(all="ignore"):
        fails = _pin_failures(lib, shapes=shapes)
    assert fails, f"mutant '{name}' passed every pin"
