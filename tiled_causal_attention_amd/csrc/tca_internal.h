// tca_internal.h -- host-side plumbing shared by the library's translation
// units: the validated argument bundle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/tca.h"
#include "tca_device.h"

namespace tca {

struct AttnArgs {
    attn_dtype dtype;
    const void* q;
    const void* k;
    const void* v;
    float* o;            // forward output; backward input
    float* lse;          // forward output; backward input
    const void* dout;
    float* dq;
    float* dk;
    float* dv;
    void* workspace;
    size_t workspace_bytes;
    int B, Hq, Hkv, N, d, causal;
    float scale;
};

// float32-arithmetic path (any supported d, either dtype). The backward's
// first phase writes D = rowsum(dO o O) into the workspace and dq; the second
// reads D and writes dk, dv.
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_generic_dq(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_generic_dkdv(const AttnArgs& a, hipStream_t st);

// matrix-core path: bf16 inputs, d in {64, 128}; same two backward phases
bool mfma_path(const AttnArgs& a);
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma_dq(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma_dkdv(const AttnArgs& a, hipStream_t st);

}  // namespace tca
