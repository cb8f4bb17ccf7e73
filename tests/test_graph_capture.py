"""The library's calls captured in a HIP graph (they launch kernels only: no
memsets, no allocation, no host synchronisation) and replayed several times, with
eager work and synchronisations between the replays; every replay must equal the
eager result bit for bit (the same kernels on the same inputs)."""
import pytest
import torch

import tiled_causal_attention_amd as tca
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tca.lib()
    yield


def capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", ["gpt2_gqa", "tiny_f32"])
def test_fwd_bwd_graph_replays_match_eager(name):
    s = workloads.CONFIGS[name]
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(s))
    o = torch.empty((s.B, s.Hq, s.N, s.d), device="cuda")
    lse = torch.empty((s.B, s.Hq, s.N), device="cuda")
    dq, dk, dv = (torch.empty(t.shape, device="cuda") for t in (q, k, v))
    ws = tca.bwd_workspace(q, k)

    def step():
        tca.attn_fwd(q, k, v, True, s.scale, out=(o, lse))
        tca.attn_bwd(q, k, v, o, lse, do, True, s.scale, out=(dq, dk, dv), workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, dq, dk, dv)]
    g = capture(step)
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((o, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {rep}"
        step()   # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["decode_wide_d128", "decode_gpt2_gqa", "decode_gpt2_gqa_b64"])
def test_decode_graph_replays_match_eager(name):
    # wide: 128 key splits per row (column-block merge); GPT-2-small: 16 (whole-row merge);
    # batch 64: 256 row groups, each group's 16 splits merged inside its workgroup
    s = workloads.DECODE_CONFIGS[name]
    q, k, v = (t.cuda() for t in workloads.make_decode_inputs(s))
    o = torch.empty((s.B, s.Hq, s.Nq, s.d), device="cuda")
    lse = torch.empty((s.B, s.Hq, s.Nq), device="cuda")
    n = int(tca.lib().attn_decode_workspace_bytes(tca.ATTN_BF16, s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.d))
    ws = tca.decode_workspace(n, "cuda")
    call = lambda: tca.attn_decode(q, k, v, True, s.scale, out=(o, lse), workspace=ws)
    call()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    g = capture(call)
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep}"
        call()
        torch.cuda.synchronize()


def test_rope_fused_qkv_graph_replays_match_eager():
    # rotary fwd + bwd on fused-QKV views, the forward's rotated keys kept for the backward:
    # one K rotation launch and the six matrix-core kernels, no allocation or memset
    s = workloads.CONFIGS["gpt2_gqa"]
    q, k, v, do = (t.cuda() for t in workloads.make_inputs(s))
    cos, sin = (t.cuda() for t in workloads.rope_tables(s.N, s.d))
    H = s.Hq + 2 * s.Hkv
    buf = torch.empty((s.B, s.N, H, s.d), dtype=q.dtype, device="cuda")
    gbuf = torch.empty((s.B, s.N, H, s.d), device="cuda")
    views = lambda b: (b[:, :, :s.Hq].permute(0, 2, 1, 3), b[:, :, s.Hq:s.Hq + s.Hkv].permute(0, 2, 1, 3),
                       b[:, :, s.Hq + s.Hkv:].permute(0, 2, 1, 3))
    qv, kv, vv = views(buf)
    qv.copy_(q), kv.copy_(k), vv.copy_(v)
    grads = views(gbuf)
    o = torch.empty((s.B, s.Hq, s.N, s.d), device="cuda")
    lse = torch.empty((s.B, s.Hq, s.N), device="cuda")
    kr = torch.empty((s.B, s.Hkv, s.N, s.d), dtype=q.dtype, device="cuda")
    L = tca.lib()
    wsf = torch.empty(int(L.attn_fwd_rope_workspace_bytes(tca.ATTN_BF16, tca.ATTN_F32, s.B, s.Hq, s.Hkv, s.N, s.d)),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.empty(int(L.attn_bwd_rope_workspace_bytes(tca.ATTN_BF16, tca.ATTN_F32, s.B, s.Hq, s.Hkv, s.N, s.d)),
                      dtype=torch.uint8, device="cuda")

    def step():
        tca.attn_fwd_rope(qv, kv, vv, cos, sin, True, s.scale, out=(o, lse), workspace=wsf, k_rot=kr)
        tca.attn_bwd_rope(qv, kv, vv, o, lse, do, cos, sin, True, s.scale, out=grads, workspace=wsb, k_rot=kr)

    step()
    torch.cuda.synchronize()
    outs = (o, lse, kr, gbuf)
    ref = [t.clone() for t in outs]
    g = capture(step)
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {rep}"
        step()
        torch.cuda.synchronize()
