"""The allocation-free decode entry point (attn_decode_noalloc) against attn_decode.

attn_decode_noalloc keeps its split partials in the library's fixed device array
instead of a caller workspace. Through the C ABI it must give attn_decode's
results bit for bit; two calls in a row, the second with a smaller input, check
that the array's leftover contents from the first call do not leak into the
second.
"""
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


def _pair(s, seed, scratch=True):
    q, k, v = (t.cuda() for t in workloads.make_decode_inputs(s, seed))
    ws_bytes = int(tca.lib().attn_decode_workspace_bytes(tca.ATTN_BF16, s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.d))
    if scratch:
        assert 0 < ws_bytes <= tca.DECODE_SCRATCH_BYTES, ws_bytes
    else:
        assert ws_bytes == 0, ws_bytes
    o_ref, l_ref = tca.attn_decode(q, k, v, causal=bool(s.causal), scale=s.scale)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    tca.attn_decode_noalloc(q, k, v, causal=bool(s.causal), scale=s.scale, out=(o, lse))
    torch.cuda.synchronize()
    return (o, lse), (o_ref, l_ref)


def test_noalloc_matches_workspace_decode_twice():
    wide = workloads.DECODE_CONFIGS["decode_wide_d128"]       # 128 splits of 64 keys, d = 128: 4.2 MB
    big_first = workloads.make_decode_shape(wide.B, wide.Hq, wide.Hkv, 2, wide.Nk, wide.d)   # 8 MiB of partials
    small = workloads.DECODE_CONFIGS["decode_gpt2_gqa"]       # fewer rows, splits and columns
    merged = workloads.make_decode_shape(64, 12, 4, 1, 1024, 64)   # splits merged in workgroups: no scratch
    for s, seed, scratch in ((big_first, 31, True), (small, 32, True), (merged, 33, False)):
        print(f"[no-alloc] {s.B, s.Hq, s.Hkv, s.Nq, s.Nk, s.d}", flush=True)
        (o, lse), (o_ref, l_ref) = _pair(s, seed, scratch)
        assert torch.equal(o, o_ref), s
        assert torch.equal(lse, l_ref), s
