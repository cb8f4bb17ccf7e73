// tca_internal.h -- host-side plumbing shared by the library's translation
// units: the validated argument bundle and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "../../include/tca.h"
#include "tca_device.h"

namespace tca {

struct AttnArgs {
    attn_dtype dtype;      // q, k, v, dO
    attn_dtype out_dtype;  // o, dq, dk, dv
    const void* q;
    const void* k;
    const void* v;
    void* o;             // forward output; backward input
    float* lse;          // forward output; backward input
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    void* workspace;
    size_t workspace_bytes;
    int B, Hq, Hkv, N, d, causal;
    float scale;
    // matrix-core path only: Q read through these strides and rotated in registers
    // (k, v hold the rotated keys and the values); the dQ pass stores dQ turned back
    // by the transpose rotation through rope->dq's strides. nullptr: plain layout.
    const QRope* rope = nullptr;
    // matrix-core dK/dV pass only: V read through these strides (k holds the rotated
    // keys), dK turned back by the transpose rotation, dK and dV stored through these
    // strides. nullptr: plain layout.
    const KVRope* kvrope = nullptr;
};

// True when the matrix-core kernels serve these inputs: bf16, d in {64, 128}.
inline bool mfma_shape(attn_dtype dtype, int d) { return dtype == ATTN_BF16 && (d == 64 || d == 128); }

// Backward workspace, each section starting on a 256-byte boundary:
//   delta  D = rowsum(dO o O), float32 [B, Hq, N]           (both paths; the matrix-core
//          path stores -D, the dK/dV pass's starting dP accumulator)
//   l2     lse * log2(e), float32 [B, Hq, N]                (matrix-core path)
//   q16    q converted to fp16, [B, Hq, N, d]               (matrix-core path)
//   do16   dO converted to fp16, [B, Hq, N, d]              (matrix-core path)
// The dQ phase writes all of them; the dK/dV phase reads them.
struct BwdWorkspace {
    float* delta;
    float* l2;
    _Float16* q16;
    _Float16* do16;
};
inline size_t ws_round(size_t n) { return (n + 255) & ~(size_t)255; }
inline size_t bwd_workspace_size(attn_dtype dtype, int B, int Hq, int N, int d) {
    const size_t rows = (size_t)B * Hq * N;
    size_t n = ws_round(rows * sizeof(float));
    if (mfma_shape(dtype, d)) n += ws_round(rows * sizeof(float)) + 2 * ws_round(rows * d * 2);
    return n;
}
inline BwdWorkspace bwd_workspace_layout(void* ws, attn_dtype dtype, int B, int Hq, int N, int d) {
    const size_t rows = (size_t)B * Hq * N;
    char* p = static_cast<char*>(ws);
    BwdWorkspace w = {reinterpret_cast<float*>(p), nullptr, nullptr, nullptr};
    if (mfma_shape(dtype, d)) {
        p += ws_round(rows * sizeof(float));
        w.l2 = reinterpret_cast<float*>(p);
        p += ws_round(rows * sizeof(float));
        w.q16 = reinterpret_cast<_Float16*>(p);
        p += ws_round(rows * d * 2);
        w.do16 = reinterpret_cast<_Float16*>(p);
    }
    return w;
}

// float32-arithmetic path (any supported d, either dtype). The backward's
// first phase writes D = rowsum(dO o O) into the workspace and dq; the second
// reads D and writes dk, dv.
hipError_t launch_fwd_generic(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_generic_dq(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_generic_dkdv(const AttnArgs& a, hipStream_t st);

// Few-query attention over a cache (decode): q, o [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d].
struct DecodeArgs {
    attn_dtype dtype, out_dtype;
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    void* workspace;
    int B, Hq, Hkv, Nq, Nk, d, causal;
    float scale;
};
// Launch shape of the decode kernels, a function of the sizes only: RM rows per
// wave (1, 2, 4 or 8; 32 on the matrix-core split), nrc row chunks of a GQA
// group's G * Nq rows, nsplit key splits of split_len keys (a multiple of 64).
struct DecodePlan {
    int rm, nrc, nsplit, split_len;
    bool fused;   // the splits of a row chunk are the waves of one workgroup, merged in LDS
    bool mfma;    // bf16 inputs, d 64 or 128: the matrix-core kernels' 32-row chunks (fused: merged form)
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, bool in32);
size_t decode_workspace_size(bool in32, int B, int Hq, int Hkv, int Nq, int Nk, int d);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// Size of the fixed device array behind attn_decode_noalloc, and its address on
// the current device (looked up on the first call per device, then cached).
constexpr size_t kDecodeScratchBytes = (size_t)ATTN_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(void** out);

// Strided copies of [B, H, N, d] tensors (head dimension contiguous) with an
// optional rotary rotation of the (i, i + d/2) pairs at each row's position:
// rot 0 none, 1 forward, 2 transpose; cs, sn [N][d/2]. Up to three copies of
// the same element types run in one launch.
struct CopyJob {
    const void* src;
    void* dst;
    long long sb, sh, sn, db, dh, dn;   // element strides (batch, head, row) of source and destination
    int H, rot;
    long long count, begin;             // threads of this job (one per 8 pairs of a row) and its first thread
};
struct CopyJobs {
    CopyJob j[3];
    int n;
};
CopyJob copy_job(const void* src, const attn_layout& sl, void* dst, const attn_layout& dl, int B, int H, int N, int d,
                 int rot);
hipError_t layout_copy(attn_dtype ti, attn_dtype to, const CopyJobs& jobs, const float* cs, const float* sn, int N,
                       int d, hipStream_t st);
// The same from bfloat16 into fp16 (the rotated keys of the matrix-core rotary path).
hipError_t layout_copy_to_f16(const CopyJobs& jobs, const float* cs, const float* sn, int N, int d, hipStream_t st);

// Unoptimised forward through a materialised score matrix (B*Hq*N*N floats of workspace).
size_t naive_workspace_size(int B, int Hq, int N);
hipError_t launch_fwd_naive(const AttnArgs& a, hipStream_t st);

// matrix-core path: bf16 inputs, d in {64, 128}; same two backward phases
bool mfma_path(const AttnArgs& a);
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma_dq(const AttnArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma_dkdv(const AttnArgs& a, hipStream_t st);

}  // namespace tca
