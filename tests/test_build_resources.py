"""Compiler resource report of every kernel in the library (CPU only: hipcc
cross-compiles the gfx950 device code here).

A kernel change that makes the compiler spill registers to scratch memory, or
that drops a matrix-core kernel below the occupancy its tiling is built for,
costs time on every shape that kernel serves and is invisible to the parity
tests. The report (hipcc -Rpass-analysis=kernel-resource-usage) catches both
at build time:
  - no kernel spills vector registers or uses scratch memory;
  - the matrix-core kernels keep their waves per SIMD: forward 4 at d = 64 and
    2 at d = 128, dQ pass 3 and 2, dK/dV pass 2 at both (3 for the d = 64
    form split by tensor), matrix-core decode split 3 and 2.
"""
import pytest

from tiled_causal_attention_amd import build


def _have_hipcc():
    try:
        build.hipcc()
        return True
    except RuntimeError:
        return False


pytestmark = pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")

# mangled-name fragment -> minimum waves per SIMD
MIN_OCCUPANCY = {
    "fwd_mfma_kernelILi64E": 4,
    "fwd_mfma_kernelILi128E": 2,
    "bwd_dq_kernelILi64E": 3,
    "bwd_dq_kernelILi128E": 2,
    "bwd_dkdv_kernelILi64E": 2,
    "bwd_dkdv_kernelILi128E": 2,
    # d = 64 split by tensor (last template argument true), float and bf16 outputs
    "bwd_dkdv_kernelILi64EfLb0ELb1E": 3,
    "bwd_dkdv_kernelILi64EfLb1ELb1E": 3,
    "bwd_dkdv_kernelILi64EtLb0ELb1E": 3,
    "bwd_dkdv_kernelILi64EtLb1ELb1E": 3,
    "decode_mfma_kernelIfLi64E": 3,
    "decode_mfma_kernelIfLi128E": 2,
}


@pytest.fixture(scope="module")
def report():
    rows = build.resource_usage()
    assert len(rows) > 100, "the report lists every kernel instantiation"
    return rows


def test_no_kernel_spills_or_uses_scratch(report):
    bad = [(r["kernel"], r.get("VGPRs Spill"), r.get("ScratchSize [bytes/lane]"))
           for r in report if r.get("VGPRs Spill") != "0" or r.get("ScratchSize [bytes/lane]") != "0"]
    assert not bad, f"kernels spilling vector registers or using scratch: {bad}"


@pytest.mark.parametrize("fragment,waves", sorted(MIN_OCCUPANCY.items()))
def test_matrix_core_kernels_keep_their_occupancy(report, fragment, waves):
    hits = [r for r in report if fragment in r["kernel"]]
    assert hits, f"no kernel matches {fragment}"
    low = [(r["kernel"], r.get("Occupancy [waves/SIMD]")) for r in hits
           if int(r.get("Occupancy [waves/SIMD]", "0")) < waves]
    assert not low, f"below {waves} waves per SIMD: {low}"
