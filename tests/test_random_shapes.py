"""GPU parity on seeded random shapes: fwd + bwd, rotary fwd + bwd and decode
against the float64 oracle, through the C ABI.

The cases are drawn once from a fixed seed, over everything the entry points
accept and the kernels branch on: batch, GQA group (1 to 6 query heads per KV
head), sequence lengths on and off the 32- and 64-row tile boundaries, every
supported head size, bfloat16 and float32 inputs, causal or not, and a float32
scale that is usually not 1/sqrt(d) (a few negative). Tolerances as in
test_parity.py: float32 inputs max |x - ref| <= 1e-4; bfloat16 inputs 2e-2 max
abs and 1e-2 relative RMS, per output tensor.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_causal_attention_amd as tca
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, None), "bf16": (2e-2, 1e-2)}
_N_EDGE = [1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191, 255, 256, 257]


def _scale(rng, d):
    u = rng.random()
    if u < 0.4:
        s = 1.0 / math.sqrt(d)
    elif u < 0.9:
        s = rng.uniform(0.02, 0.3)
    else:
        s = -rng.uniform(0.05, 0.3)
    return float(np.float32(s))


def _fwd_cases(n=40, seed=20260):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128], p=[0.15, 0.15, 0.4, 0.3]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 6]))
        B = int(rng.integers(1, 4))
        N = int(rng.choice(_N_EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 600))
        causal = int(rng.random() < 0.7)
        out.append((i, B, G * Hkv, Hkv, N, d, dtype, causal, _scale(rng, d), 5000 + i))
    return out


def _decode_cases(n=20, seed=20261):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.integers(1, 5))
        Nq = int(rng.integers(1, 9))
        Nk = int(rng.integers(Nq, 3000))
        causal = int(rng.random() < 0.8)
        out.append((i, B, G * Hkv, Hkv, Nq, Nk, d, dtype, causal, _scale(rng, d), 6000 + i))
    return out


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tca.lib()
    yield


def _check(name, got, ref, dtype, ctx):
    g = got.float().cpu().double().numpy()
    assert np.isfinite(g).all(), f"{ctx} {name}: non-finite"
    if g.size == 0:
        return
    max_abs, rel_bound = TOL[dtype]
    diff = np.abs(g - ref)
    assert diff.max() <= max_abs, f"{ctx} {name}: max abs {diff.max():.3e}"
    if rel_bound is not None:
        den = float(np.linalg.norm(ref))
        rel = float(np.linalg.norm(g - ref)) / den if den > 0 else float(np.linalg.norm(g - ref))
        assert rel <= rel_bound, f"{ctx} {name}: rel rms {rel:.3e}"


@pytest.mark.parametrize("case", _fwd_cases(), ids=lambda c: f"fb{c[0]}")
def test_random_fwd_bwd(case):
    i, B, Hq, Hkv, N, d, dtype, causal, scale, seed = case
    ctx = f"case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} causal={causal} scale={scale:.4f}"
    print(f"[random fwd+bwd] {ctx}", flush=True)
    s = workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=seed, causal=causal)
    q, k, v, do = workloads.make_inputs(s)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = tca.attn_fwd(qd, kd, vd, causal=bool(causal), scale=scale)
    dq, dk, dv = tca.attn_bwd(qd, kd, vd, o, lse, dod, causal=bool(causal), scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(q, k, v, causal, scale)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, causal, scale)
    for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check(name, got, ref, dtype, ctx)


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda c: f"dec{c[0]}")
def test_random_decode(case):
    i, B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale, seed = case
    ctx = f"case {i}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} scale={scale:.4f}"
    print(f"[random decode] {ctx}", flush=True)
    s = workloads.make_decode_shape(B, Hq, Hkv, Nq, Nk, d, dtype=dtype, seed=seed, causal=causal)
    q, k, v = workloads.make_decode_inputs(s)
    o, lse = tca.attn_decode(q.cuda(), k.cuda(), v.cuda(), causal=bool(causal), scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_decode(q, k, v, causal, scale)
    for name, got, ref in (("o", o, ro), ("lse", lse, rl)):
        _check(name, got, ref, dtype, ctx)


def _rope_cases(n=12, seed=20262):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128], p=[0.15, 0.15, 0.4, 0.3]))
        dtype = "f32" if rng.random() < 0.25 else "bf16"
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 3, 4]))
        B = int(rng.integers(1, 3))
        N = int(rng.choice(_N_EDGE)) if rng.random() < 0.5 else int(rng.integers(1, 400))
        layout = str(rng.choice(["fused", "odd"]))
        keep_k = bool(rng.random() < 0.5)
        causal = int(rng.random() < 0.7)
        scale = _scale(rng, d)
        if dtype == "bf16" and d not in (64, 128):
            # the staged path (bfloat16 inputs at d = 16, 32) rounds the rotated q, k to
            # bfloat16, an input-sized rounding whose effect grows with the scores:
            # scales up to 1/sqrt(d)
            scale = float(np.float32(math.copysign(min(abs(scale), 1.0 / math.sqrt(d)), scale)))
        out.append((i, B, G * Hkv, Hkv, N, d, dtype, causal, scale, layout, keep_k, 7000 + i))
    return out


@pytest.mark.parametrize("case", _rope_cases(), ids=lambda c: f"rope{c[0]}")
def test_random_rope(case):
    # rotary q/k on views of one fused projection buffer (16-byte aligned rows) or on
    # rows d + 1 elements apart starting one element in (read through contiguous
    # copies), with or without the forward's rotated keys kept for the backward
    i, B, Hq, Hkv, N, d, dtype, causal, scale, layout, keep_k, seed = case
    ctx = f"case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} causal={causal} scale={scale:.4f} {layout} k_rot={keep_k}"
    print(f"[random rope] {ctx}", flush=True)
    s = workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=seed, causal=causal)
    q, k, v, do = workloads.make_inputs(s)
    cos, sin = workloads.rope_tables(N, d, base=500.0)
    if layout == "fused":
        buf = torch.empty((B, N, Hq + 2 * Hkv, d), dtype=q.dtype, device="cuda")
        views = [buf[:, :, :Hq], buf[:, :, Hq:Hq + Hkv], buf[:, :, Hq + Hkv:]]
        qv, kv, vv = (x.permute(0, 2, 1, 3) for x in views)
        qv.copy_(q), kv.copy_(k), vv.copy_(v)
    else:
        def odd(t):
            b = torch.zeros(t.shape[:3] + (d + 1,), dtype=t.dtype, device="cuda")
            b[..., 1:].copy_(t.cuda())
            return b[..., 1:]
        qv, kv, vv = odd(q), odd(k), odd(v)
    kr = torch.empty((B, Hkv, N, d), dtype=q.dtype, device="cuda") if keep_k else None
    cd, sd = cos.cuda(), sin.cuda()
    o, lse = tca.attn_fwd_rope(qv, kv, vv, cd, sd, causal=bool(causal), scale=scale, k_rot=kr)
    dq, dk, dv = tca.attn_bwd_rope(qv, kv, vv, o, lse, do.cuda(), cd, sd, causal=bool(causal), scale=scale, k_rot=kr)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_rope(q, k, v, cos, sin, causal, scale)
    rq, rk, rv = oracle.attn_bwd_rope(q, k, v, do, cos, sin, causal, scale)
    for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        _check(name, got, ref, dtype, ctx)


@pytest.mark.parametrize("case", _fwd_cases()[:20], ids=lambda c: f"bo{c[0]}")
def test_random_bf16_outputs_are_rounded(case):
    # bfloat16 outputs are the float32 results rounded once: o and lse of the forward,
    # and dq, dk, dv of a backward that takes the bfloat16 o against a float32-output
    # backward given that o widened; bit for bit on every path
    i, B, Hq, Hkv, N, d, dtype, causal, scale, seed = case
    print(f"[random bf16 out] case {i}: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} {dtype} causal={causal}", flush=True)
    s = workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=seed, causal=causal)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(s))
    o16, l16 = tca.attn_fwd(q, k, v, causal=bool(causal), scale=scale, out_dtype=torch.bfloat16)
    o32, l32 = tca.attn_fwd(q, k, v, causal=bool(causal), scale=scale)
    g16 = tca.attn_bwd(q, k, v, o16, l16, do, causal=bool(causal), scale=scale)
    g32 = tca.attn_bwd(q, k, v, o16.float(), l16, do, causal=bool(causal), scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(l16, l32), i
    assert torch.equal(o16, o32.to(torch.bfloat16)), i
    for name, a, b in zip(("dq", "dk", "dv"), g16, g32):
        assert a.dtype == torch.bfloat16 and torch.equal(a, b.to(torch.bfloat16)), f"case {i} {name}"


@pytest.mark.parametrize("case", _decode_cases()[:10], ids=lambda c: f"dbo{c[0]}")
def test_random_decode_bf16_outputs_are_rounded(case):
    i, B, Hq, Hkv, Nq, Nk, d, dtype, causal, scale, seed = case
    s = workloads.make_decode_shape(B, Hq, Hkv, Nq, Nk, d, dtype=dtype, seed=seed, causal=causal)
    q, k, v = (t.cuda() for t in workloads.make_decode_inputs(s))
    o16, l16 = tca.attn_decode(q, k, v, causal=bool(causal), scale=scale, out_dtype=torch.bfloat16)
    o32, l32 = tca.attn_decode(q, k, v, causal=bool(causal), scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(l16, l32) and torch.equal(o16, o32.to(torch.bfloat16)), i
