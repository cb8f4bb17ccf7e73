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

// float32-arithmetic path (any supported d, either dtype)
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_generic(const AttnArgs& a, hipStream_t st);
// backward preprocess shared by both paths: delta into the workspace, and
// clearing of dq (clear_dq) and dk/dv (clear_dkdv)
hipError_t launch_bwd_preprocess(const AttnArgs& a, bool clear_dq, bool clear_dkdv, hipStream_t st);

// matrix-core path: bf16 inputs, d in {64, 128}
bool mfma_path(const AttnArgs& a);
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t st);
// which outputs the matrix-core backward accumulates atomically
bool bwd_mfma_atomic_dkdv(const AttnArgs& a);

}  // namespace tca
