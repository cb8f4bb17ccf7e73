"""GPU parity of the unoptimised materialised-score forward (attn_fwd_naive)
against the float64 oracle, through the C ABI. It computes in float32 from
exactly widened inputs, so the float32 bound (max abs 1e-4) is used for float32
inputs and outputs, the bfloat16 bound (2e-2 max abs, 1e-2 rel RMS) otherwise,
plus half a bfloat16 ulp (<= 2^-8 |x|) for bfloat16 outputs."""
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


def check(name, got, ref, tight, out_bf16, ctx):
    g = got.float().cpu().double().numpy()
    assert np.isfinite(g).all(), f"{ctx} {name}"
    diff = np.abs(g - ref)
    bound = (1e-4 if tight else 2e-2) + (2.0 ** -8 * np.maximum(np.abs(g), np.abs(ref)) if out_bf16 else 0.0)
    assert (diff <= bound).all(), f"{ctx} {name}: max abs {diff.max():.3e}"
    if not tight:
        rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
        assert rel <= 1e-2, f"{ctx} {name}: rel rms {rel:.3e}"


@pytest.mark.parametrize("B,Hq,Hkv,N,d,dtype,causal,out", [
    (1, 2, 1, 1, 16, "f32", 1, "f32"),
    (2, 4, 2, 37, 16, "f32", 1, "f32"),
    (1, 3, 1, 100, 32, "f32", 0, "f32"),
    (2, 6, 2, 200, 64, "bf16", 1, "f32"),
    (1, 4, 4, 129, 128, "bf16", 0, "f32"),
    (1, 6, 3, 77, 64, "bf16", 1, "bf16"),
    (8, 12, 4, 1024, 64, "bf16", 1, "f32"),   # the GPT-2-small GQA shape
])
def test_naive_matches_oracle(B, Hq, Hkv, N, d, dtype, causal, out):
    s = workloads.make_shape(B, Hq, Hkv, N, d, dtype=dtype, seed=400 + N + d, causal=causal)
    q, k, v, _ = workloads.make_inputs(s)
    out_dt = torch.bfloat16 if out == "bf16" else torch.float32
    o, lse = tca.attn_fwd_naive(q.cuda(), k.cuda(), v.cuda(), causal=bool(causal), scale=s.scale, out_dtype=out_dt)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(q, k, v, causal, s.scale)
    tight = dtype == "f32" and out == "f32"
    ctx = f"naive {B,Hq,Hkv,N,d} {dtype} causal={causal} out={out}"
    check("o", o, ro, tight, out == "bf16", ctx)
    check("lse", lse, rl, tight, False, ctx)


def test_naive_and_tiled_agree():
    s = workloads.make_shape(2, 12, 4, 300, 64, dtype="bf16", seed=3)
    q, k, v, _ = (t.cuda() for t in workloads.make_inputs(s))
    o1, l1 = tca.attn_fwd_naive(q, k, v, scale=s.scale)
    o2, l2 = tca.attn_fwd(q, k, v, scale=s.scale)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 2e-2 and (l1 - l2).abs().max().item() <= 1e-3
