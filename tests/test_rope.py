"""GPU parity of the rotary / strided-input path (attn_fwd_rope, attn_bwd_rope)
against the float64 oracle's rotary attention, through the C ABI.

q, k, v are read through arbitrary [B, H, N, d] strides (contiguous, or views of
one fused projection buffer [B, N, Hq + 2 Hkv, d]); q and k are rotated
(rotate-half pairing, float32 tables from workloads.rope_tables, the same
values the oracle widens); gradients are of the unrotated q, k. Tolerances per
output tensor: float32 inputs max abs 1e-4; bfloat16 inputs 2e-2 max abs and
1e-2 rel RMS (the rotated q, k are rounded before the products: to fp16 on the
matrix-core path, to bfloat16 on the staged one, one more rounding of the size
of the inputs' own); bfloat16 outputs add half a bfloat16 ulp (<= 2^-8 |x|).
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_causal_attention_amd as tca
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tca.lib()
    yield


def check(name, got, ref, dtype, out_bf16, ctx):
    g = got.float().cpu().double().numpy()
    assert np.isfinite(g).all(), f"{ctx} {name}"
    diff = np.abs(g - ref)
    base = 1e-4 if dtype == "f32" and not out_bf16 else 2e-2
    bound = base + (2.0 ** -8 * np.maximum(np.abs(g), np.abs(ref)) if out_bf16 else 0.0)
    assert (diff <= bound).all(), f"{ctx} {name}: max abs {diff.max():.3e}"
    if dtype == "bf16" or out_bf16:
        rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
        assert rel <= 1e-2, f"{ctx} {name}: rel rms {rel:.3e}"


def fused_views(q, k, v):
    """q, k, v [B, H, N, d] copied into one fused buffer [B, N, Hq + 2 Hkv, d]; returns the views."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    buf = torch.empty((B, N, Hq + 2 * Hkv, d), dtype=q.dtype, device="cuda")
    qv = buf[:, :, :Hq].permute(0, 2, 1, 3)
    kv = buf[:, :, Hq:Hq + Hkv].permute(0, 2, 1, 3)
    vv = buf[:, :, Hq + Hkv:].permute(0, 2, 1, 3)
    qv.copy_(q)
    kv.copy_(k)
    vv.copy_(v)
    return buf, qv, kv, vv


def run_parity(s, layout="contiguous", out_dtype=torch.float32, rope=True):
    q, k, v, do = workloads.make_inputs(s)
    cos, sin = workloads.rope_tables(s.N, s.d, base=500.0)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    cd, sd = (cos.cuda(), sin.cuda()) if rope else (None, None)
    if layout == "fused":
        _, qd, kd, vd = fused_views(qd, kd, vd)
        gbuf = torch.full((s.B, s.N, s.Hq + 2 * s.Hkv, s.d), float("nan"), dtype=out_dtype, device="cuda")
        out = (gbuf[:, :, :s.Hq].permute(0, 2, 1, 3), gbuf[:, :, s.Hq:s.Hq + s.Hkv].permute(0, 2, 1, 3),
               gbuf[:, :, s.Hq + s.Hkv:].permute(0, 2, 1, 3))
    else:
        out = None
    o, lse = tca.attn_fwd_rope(qd, kd, vd, cd, sd, causal=bool(s.causal), scale=s.scale, out_dtype=out_dtype)
    dq, dk, dv = tca.attn_bwd_rope(qd, kd, vd, o, lse, dod, cd, sd, causal=bool(s.causal), scale=s.scale, out=out)
    torch.cuda.synchronize()
    if rope:
        ro, rl = oracle.attn_fwd_rope(q, k, v, cos, sin, s.causal, s.scale)
        rq, rk, rv = oracle.attn_bwd_rope(q, k, v, do, cos, sin, s.causal, s.scale)
    else:
        ro, rl = oracle.attn_fwd(q, k, v, s.causal, s.scale)
        rq, rk, rv = oracle.attn_bwd(q, k, v, do, s.causal, s.scale)
    ctx = f"rope={rope} {layout} {s.B,s.Hq,s.Hkv,s.N,s.d} {s.dtype} causal={s.causal} out={out_dtype}"
    ob = out_dtype == torch.bfloat16
    # bf16 outputs: D is formed from bf16(O); on these N(0, 1) inputs that moves dQ, dK by far
    # less than the bound (the bf16-output tests cover the exact contract)
    for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref, s.dtype, ob and name != "lse", ctx)


SHAPES = [
    (2, 6, 2, 200, 64, "bf16"),
    (1, 4, 4, 129, 64, "bf16"),
    (2, 4, 2, 161, 128, "bf16"),
    (1, 6, 3, 77, 32, "bf16"),
    (2, 4, 2, 37, 16, "f32"),
    (1, 3, 1, 100, 64, "f32"),
]


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype", SHAPES)
@pytest.mark.parametrize("causal", [1, 0])
def test_rope_contiguous(B, Hq, Hkv, N, d, dtype, causal):
    run_parity(workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=600 + N + d, causal=causal))


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype", SHAPES[:3] + SHAPES[4:5])
def test_rope_fused_qkv_layout(B, Hq, Hkv, N, d, dtype):
    run_parity(workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=650 + N), layout="fused")


def test_rope_bf16_outputs_fused_layout():
    run_parity(workloads.make_shape(2, 6, 2, 200, 64, seed=77), layout="fused", out_dtype=torch.bfloat16)


def test_strided_without_rope_fused_layout():
    run_parity(workloads.make_shape(2, 12, 4, 300, 64, seed=78), layout="fused", rope=False)


def test_rope_dkdv_split_form():
    # d = 64 with 384 dK/dV workgroups: the pass runs split by tensor, and its epilogue
    # turns dK back and stores dK, dV through the fused layout
    run_parity(workloads.make_shape(2, 12, 12, 1024, 64, seed=79, causal=0), layout="fused")


def test_rope_headline_shape():
    print("[rope parity] gpt2_gqa", flush=True)
    run_parity(workloads.CONFIGS["gpt2_gqa"], layout="fused")


def test_strided_copies_are_exact():
    # no rotation: staging is an exact copy, so the strided path runs the same kernels on the
    # same values as attn_fwd / attn_bwd on contiguous tensors: bitwise equal results
    s = workloads.make_shape(2, 12, 4, 333, 64, seed=79)
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(s))
    _, qv, kv, vv = fused_views(q, k, v)
    o1, l1 = tca.attn_fwd(q, k, v, scale=s.scale)
    g1 = tca.attn_bwd(q, k, v, o1, l1, do, scale=s.scale)
    o2, l2 = tca.attn_fwd_rope(qv, kv, vv, scale=s.scale)
    g2 = tca.attn_bwd_rope(qv, kv, vv, o2, l2, do, scale=s.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_rope_unaligned_views():
    # rows d+1 elements apart, starting one element in: no 16-byte alignment, so the
    # copies take their element-wise path
    s = workloads.make_shape(2, 6, 2, 150, 64, dtype="bf16", seed=81)
    q, k, v, do = workloads.make_inputs(s)
    cos, sin = workloads.rope_tables(s.N, s.d, base=500.0)

    def odd_view(t):
        B, H, N, d = t.shape
        buf = torch.zeros((B, H, N, d + 1), dtype=t.dtype, device="cuda")
        view = buf[..., 1:]
        view.copy_(t.cuda())
        return view

    qv, kv, vv = odd_view(q), odd_view(k), odd_view(v)
    assert qv.data_ptr() % 16 != 0
    cd, sd = cos.cuda(), sin.cuda()
    outs = tuple(odd_view(torch.zeros(t.shape)) for t in (q, k, v))
    o, lse = tca.attn_fwd_rope(qv, kv, vv, cd, sd, scale=s.scale)
    dq, dk, dv = tca.attn_bwd_rope(qv, kv, vv, o, lse, do.cuda(), cd, sd, scale=s.scale, out=outs)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd_rope(q, k, v, cos, sin, 1, s.scale)
    rq, rk, rv = oracle.attn_bwd_rope(q, k, v, do, cos, sin, 1, s.scale)
    for name, got, ref in (("o", o, ro), ("lse", lse, rl), ("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(name, got, ref, "bf16", False, "unaligned views")


@pytest.mark.parametrize("case", ["fused_d64", "fused_d128", "f32_staged", "unaligned_copies"])
def test_saved_rotated_keys(case):
    # attn_fwd_rope's k_rot receives the rotated keys; attn_bwd_rope given them reads them
    # back instead of rotating k: every output bitwise equal to the calls without k_rot
    B, Hq, Hkv, N, d, dtype = {"fused_d64": (2, 6, 2, 200, 64, "bf16"), "fused_d128": (1, 4, 2, 161, 128, "bf16"),
                               "f32_staged": (1, 3, 1, 100, 64, "f32"),
                               "unaligned_copies": (2, 6, 2, 150, 64, "bf16")}[case]
    print(f"[rope k_rot] {case}", flush=True)
    s = workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=90 + N)
    q, k, v, do = workloads.make_inputs(s)
    cos, sin = workloads.rope_tables(s.N, s.d, base=500.0)
    if case == "unaligned_copies":
        def view(t):
            buf = torch.zeros(t.shape[:3] + (d + 1,), dtype=t.dtype, device="cuda")
            buf[..., 1:].copy_(t.cuda())
            return buf[..., 1:]
        qv, kv, vv = view(q), view(k), view(v)
    else:
        _, qv, kv, vv = fused_views(q.cuda(), k.cuda(), v.cuda())
    cd, sd, dod = cos.cuda(), sin.cuda(), do.cuda()
    o1, l1 = tca.attn_fwd_rope(qv, kv, vv, cd, sd, scale=s.scale)
    g1 = tca.attn_bwd_rope(qv, kv, vv, o1, l1, dod, cd, sd, scale=s.scale)
    kr = torch.full((B, Hkv, N, d), float("nan"), dtype=q.dtype, device="cuda")
    o2, l2 = tca.attn_fwd_rope(qv, kv, vv, cd, sd, scale=s.scale, k_rot=kr)
    g2 = tca.attn_bwd_rope(qv, kv, vv, o2, l2, dod, cd, sd, scale=s.scale, k_rot=kr)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), case
    for name, a, b in zip(("dq", "dk", "dv"), g1, g2):
        assert torch.equal(a, b), f"{case} {name}"
    # the saved keys: k rotated pairwise (i, i + d/2) by the table's angle, one rounding:
    # to fp16 on the matrix-core path (bf16 inputs, d in {64, 128}; unaligned views go
    # through contiguous copies), else to the input type
    kf = k.double().numpy()
    c, sn = cos.double().numpy()[None, None], sin.double().numpy()[None, None]
    x1, x2 = kf[..., :d // 2], kf[..., d // 2:]
    ref = np.concatenate([x1 * c - x2 * sn, x2 * c + x1 * sn], axis=-1)
    fused = dtype == "bf16" and d in (64, 128)
    got = (kr.view(torch.float16) if fused else kr).float().cpu().double().numpy()
    ulp = 2.0 ** -11 if fused else (2.0 ** -8 if dtype == "bf16" else 2.0 ** -23)
    assert (np.abs(got - ref) <= ulp * np.abs(ref) + 1e-6).all(), case
