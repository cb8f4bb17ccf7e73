// tca_api.hip -- the extern "C" entry points declared in include/tca.h:
// argument validation (host only, before any HIP call) and dispatch to the
// matrix-core or float32-arithmetic kernels.
#include <math.h>
#include <stdint.h>

#include "tca_internal.h"

using tca::AttnArgs;

namespace {

constexpr int kAbiVersion = 4;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Shape, flag and scalar checks shared by every entry point.
bool known_dtype(attn_dtype t) { return t == ATTN_F32 || t == ATTN_BF16; }

attn_status check_sizes(attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d, int causal,
                        float scale) {
    if (!known_dtype(dtype) || !known_dtype(out_dtype)) return ATTN_EINVAL;
    if (B < 0 || N < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_EINVAL;
    if (Hq % Hkv != 0) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    if ((int64_t)(N + 64) * d >= ((int64_t)1 << 31)) return ATTN_EINVAL;   // row offsets of a head, tail tile included, fit 32-bit byte offsets
    if ((int64_t)B * Hq * N >= ((int64_t)1 << 31)) return ATTN_EINVAL;
    if (!supported_d(d)) return ATTN_EUNSUPPORTED;
    return ATTN_OK;
}

attn_status check_ptrs(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p == nullptr || !aligned16(p)) return ATTN_EINVAL;
    return ATTN_OK;
}


attn_status check_bwd(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                      void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                      float scale, bool* noop) {
    attn_status s = check_sizes(dtype, out_dtype, B, Hq, Hkv, N, d, causal, scale);
    if (s != ATTN_OK) return s;
    *noop = ((int64_t)B * N == 0);
    if (*noop) return ATTN_OK;
    s = check_ptrs({q, k, v, o, lse, dO, dq, dk, dv, ws});
    if (s != ATTN_OK) return s;
    if (ws_bytes < tca::bwd_workspace_size(dtype, B, Hq, N, d)) return ATTN_EINVAL;
    return ATTN_OK;
}

AttnArgs make_args(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv, void* ws,
                   size_t ws_bytes, int B, int Hq, int Hkv, int N, int d, int causal, float scale) {
    AttnArgs a;
    a.dtype = dtype;
    a.out_dtype = out_dtype;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = const_cast<void*>(o);
    a.lse = const_cast<float*>(lse);
    a.dout = dO;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.workspace = ws;
    a.workspace_bytes = ws_bytes;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.causal = causal;
    a.scale = scale;
    return a;
}

attn_status from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EHIP; }

// ---- rotary / strided path: workspace carving
size_t elsize(attn_dtype t) { return t == ATTN_F32 ? 4 : 2; }
attn_layout contiguous_layout(int H, int N, int d) {
    attn_layout l;
    l.stride_b = (long long)H * N * d;
    l.stride_h = (long long)N * d;
    l.stride_n = d;
    return l;
}
struct RopeWs {
    char* q;
    char* k;
    char* v;
    float* o32;
    float* dq;
    float* dk;
    float* dv;
    char* bwd;
    size_t bwd_bytes;
    size_t total;
};
RopeWs rope_ws(void* base, bool bwd, attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d) {
    RopeWs w = {};
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* r = p ? p + off : nullptr;
        off += tca::ws_round(bytes);
        return r;
    };
    const size_t nq = (size_t)B * Hq * N * d, nk = (size_t)B * Hkv * N * d;
    w.q = take(nq * elsize(dtype));
    w.k = take(nk * elsize(dtype));
    w.v = take(nk * elsize(dtype));
    if (bwd) {
        if (out_dtype == ATTN_BF16) w.o32 = reinterpret_cast<float*>(take(nq * 4));
        w.dq = reinterpret_cast<float*>(take(nq * 4));
        w.dk = reinterpret_cast<float*>(take(nk * 4));
        w.dv = reinterpret_cast<float*>(take(nk * 4));
        w.bwd_bytes = tca::bwd_workspace_size(dtype, B, Hq, N, d);
        w.bwd = take(w.bwd_bytes);
    }
    w.total = off;
    return w;
}

bool layout_ok(const attn_layout* l) {
    return l == nullptr || (l->stride_b >= 0 && l->stride_h >= 0 && l->stride_n >= 0);
}
bool elem_aligned(const void* p, attn_dtype t) { return p != nullptr && ((uintptr_t)p % elsize(t)) == 0; }

attn_status check_rope(attn_dtype dtype, attn_dtype out_dtype, const void* q, const attn_layout* ql, const void* k,
                       const attn_layout* kl, const void* v, const attn_layout* vl, const float* cs, const float* sn,
                       int d) {
    if ((cs == nullptr) != (sn == nullptr)) return ATTN_EINVAL;
    if (cs != nullptr && (d % 2 != 0 || !aligned16(cs) || !aligned16(sn))) return ATTN_EINVAL;
    if (!layout_ok(ql) || !layout_ok(kl) || !layout_ok(vl)) return ATTN_EINVAL;
    if (!elem_aligned(q, dtype) || !elem_aligned(k, dtype) || !elem_aligned(v, dtype)) return ATTN_EINVAL;
    (void)out_dtype;
    return ATTN_OK;
}

// q, k (rotated; unless the rotated keys are already there) and v into the
// contiguous staging copies, one launch
hipError_t stage_qkv(const RopeWs& w, attn_dtype dtype, const void* q, const attn_layout* ql, const void* k,
                     const attn_layout* kl, const void* v, const attn_layout* vl, const float* cs, const float* sn,
                     int B, int Hq, int Hkv, int N, int d, bool with_k, hipStream_t st) {
    const int rot = cs ? 1 : 0;
    const attn_layout cq = contiguous_layout(Hq, N, d), ck = contiguous_layout(Hkv, N, d);
    tca::CopyJobs jobs;
    jobs.n = 0;
    jobs.j[jobs.n++] = tca::copy_job(q, ql ? *ql : cq, w.q, cq, B, Hq, N, d, rot);
    if (with_k) jobs.j[jobs.n++] = tca::copy_job(k, kl ? *kl : ck, w.k, ck, B, Hkv, N, d, rot);
    jobs.j[jobs.n++] = tca::copy_job(v, vl ? *vl : ck, w.v, ck, B, Hkv, N, d, 0);
    return tca::layout_copy(dtype, dtype, jobs, cs, sn, N, d, st);
}

// Q (and dQ) read / written in place by the matrix-core kernels: rows 16-byte aligned
bool rows_aligned16(const void* p, const attn_layout* l, size_t es) {
    if (p == nullptr || (uintptr_t)p % 16 != 0) return false;
    if (l == nullptr) return true;
    return ((size_t)l->stride_b * es) % 16 == 0 && ((size_t)l->stride_h * es) % 16 == 0 &&
           ((size_t)l->stride_n * es) % 16 == 0;
}

// k (bfloat16), rotated, into its contiguous fp16 staging copy, one launch (on the
// fused path q is rotated into fp16 in the kernels' registers and v is read in place)
hipError_t stage_k(const RopeWs& w, const void* k, const attn_layout* kl, const float* cs, const float* sn, int B,
                   int Hkv, int N, int d, hipStream_t st) {
    const attn_layout ck = contiguous_layout(Hkv, N, d);
    tca::CopyJobs jobs;
    jobs.n = 1;
    jobs.j[0] = tca::copy_job(k, kl ? *kl : ck, w.k, ck, B, Hkv, N, d, 1);
    return tca::layout_copy_to_f16(jobs, cs, sn, N, d, st);
}

// V read in place by the matrix-core kernels: 16-byte aligned rows at least d apart, and
// every byte offset within a head's rows (past the last row included) fits 32 bits
bool v_in_place(const void* v, const attn_layout* vl, int Hkv, int N, int d) {
    if (!rows_aligned16(v, vl, 2)) return false;
    const attn_layout l = vl ? *vl : contiguous_layout(Hkv, N, d);
    return l.stride_n >= d && (int64_t)(N + 64) * l.stride_n * 2 < ((int64_t)1 << 32);
}

// q and v as the matrix-core rotary kernels read them: in place when their rows allow it
// (q: 16-byte aligned rows; v: as v_in_place), else through exact contiguous copies
// in the workspace (one launch for both). qv/vv and ql/vl receive what to read.
hipError_t fused_inputs(const RopeWs& w, const void* q, const attn_layout* q_layout, const void* v,
                        const attn_layout* v_layout, int B, int Hq, int Hkv, int N, int d, const void** qv,
                        const attn_layout** ql, const void** vv, const attn_layout** vl, hipStream_t st) {
    const attn_layout cq = contiguous_layout(Hq, N, d), ck = contiguous_layout(Hkv, N, d);
    *qv = q;
    *ql = q_layout;
    *vv = v;
    *vl = v_layout;
    tca::CopyJobs jobs;
    jobs.n = 0;
    if (!rows_aligned16(q, q_layout, 2)) {
        jobs.j[jobs.n++] = tca::copy_job(q, q_layout ? *q_layout : cq, w.q, cq, B, Hq, N, d, 0);
        *qv = w.q;
        *ql = nullptr;
    }
    if (!v_in_place(v, v_layout, Hkv, N, d)) {
        jobs.j[jobs.n++] = tca::copy_job(v, v_layout ? *v_layout : ck, w.v, ck, B, Hkv, N, d, 0);
        *vv = w.v;
        *vl = nullptr;
    }
    return jobs.n ? tca::layout_copy(ATTN_BF16, ATTN_BF16, jobs, nullptr, nullptr, N, d, st) : hipSuccess;
}

// The matrix-core rotary kernels take every bfloat16 call with tables and d in {64, 128}
// whose contiguous copies they could read (a contiguous V head's byte offsets fit 32 bits)
bool fused_rope(attn_dtype dtype, const float* cs, int N, int d) {
    return cs != nullptr && tca::mfma_shape(dtype, d) && (int64_t)(N + 64) * d * 2 < ((int64_t)1 << 32);
}

tca::QRope make_qrope(const void* q, const attn_layout* ql, const float* cs, const float* sn, void* dq,
                      const attn_layout* gl, const void* v, const attn_layout* vl, int Hq, int Hkv, int N, int d) {
    const attn_layout cq = contiguous_layout(Hq, N, d);
    const attn_layout a = ql ? *ql : cq, g = gl ? *gl : cq;
    const attn_layout vv = vl ? *vl : contiguous_layout(Hkv, N, d);
    tca::QRope r;
    r.q = static_cast<const tca::bf16_t*>(q);
    r.qb = a.stride_b;
    r.qh = a.stride_h;
    r.qn = a.stride_n;
    r.dq = dq;
    r.gb = g.stride_b;
    r.gh = g.stride_h;
    r.gn = g.stride_n;
    r.cs = cs;
    r.sn = sn;
    r.v = static_cast<const tca::bf16_t*>(v);
    r.vb = vv.stride_b;
    r.vh = vv.stride_h;
    r.vn = vv.stride_n;
    return r;
}

tca::KVRope make_kvrope(const void* v, const attn_layout* vl, void* dk, const attn_layout* kl, void* dv,
                        const attn_layout* dl, const float* cs, const float* sn, int Hkv, int N, int d) {
    const attn_layout ck = contiguous_layout(Hkv, N, d);
    const attn_layout vv = vl ? *vl : ck, gk = kl ? *kl : ck, gv = dl ? *dl : ck;
    tca::KVRope r;
    r.v = static_cast<const tca::bf16_t*>(v);
    r.vb = vv.stride_b;
    r.vh = vv.stride_h;
    r.vn = vv.stride_n;
    r.dk = dk;
    r.kb = gk.stride_b;
    r.kh = gk.stride_h;
    r.kn = gk.stride_n;
    r.dv = dv;
    r.db = gv.stride_b;
    r.dh = gv.stride_h;
    r.dn = gv.stride_n;
    r.cs = cs;
    r.sn = sn;
    return r;
}

attn_status run_dq(const AttnArgs& a, hipStream_t st) {
    return from_hip(tca::mfma_path(a) ? tca::launch_bwd_mfma_dq(a, st) : tca::launch_bwd_generic_dq(a, st));
}

attn_status run_dkdv(const AttnArgs& a, hipStream_t st) {
    return from_hip(tca::mfma_path(a) ? tca::launch_bwd_mfma_dkdv(a, st) : tca::launch_bwd_generic_dkdv(a, st));
}

// Size, flag and pointer checks of the decode entry points (not the workspace)
attn_status check_decode(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                         void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
                         float scale, bool* noop) {
    *noop = false;
    if (!known_dtype(dtype) || !known_dtype(out_dtype)) return ATTN_EINVAL;
    if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || d < 1) return ATTN_EINVAL;
    if (Hq % Hkv != 0 || Nq > Nk) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale)) return ATTN_EINVAL;
    if ((int64_t)(Nk + 256) * d * 4 >= ((int64_t)1 << 31)) return ATTN_EINVAL;   // byte offsets in a head's K/V
    if ((int64_t)B * Hq * Nq >= ((int64_t)1 << 31)) return ATTN_EINVAL;
    if ((int64_t)B * Hkv * Hq * Nq >= ((int64_t)1 << 31)) return ATTN_EINVAL;   // work items
    if (!supported_d(d)) return ATTN_EUNSUPPORTED;
    if ((int64_t)B * Nq == 0) {
        *noop = true;
        return ATTN_OK;
    }
    return check_ptrs({q, k, v, o, lse});
}

tca::DecodeArgs decode_args(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                            void* o, float* lse, void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                            int causal, float scale) {
    tca::DecodeArgs a;
    a.dtype = dtype;
    a.out_dtype = out_dtype;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.workspace = workspace;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.Nq = Nq;
    a.Nk = Nk;
    a.d = d;
    a.causal = causal;
    a.scale = scale;
    return a;
}
}  // namespace


extern "C" {

int attn_abi_version(void) { return kAbiVersion; }

const char* attn_status_str(attn_status s) {
    switch (s) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_EINVAL: return "ATTN_EINVAL: invalid argument";
        case ATTN_EUNSUPPORTED: return "ATTN_EUNSUPPORTED: unsupported head dimension";
        case ATTN_EHIP: return "ATTN_EHIP: HIP runtime error while enqueueing";
        case ATTN_ESCRATCH:
            return "ATTN_ESCRATCH: the decode needs more split-partial memory than the fixed scratch array holds";
        default: return "unknown attn_status";
    }
}

size_t attn_fwd_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int N, int d) {
    (void)dtype; (void)B; (void)Hq; (void)Hkv; (void)N; (void)d;
    return 0;
}

attn_status attn_fwd(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                     void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                     int N, int d, int causal, float scale, void* stream) {
    attn_status s = check_sizes(dtype, out_dtype, B, Hq, Hkv, N, d, causal, scale);
    if (s != ATTN_OK) return s;
    if ((int64_t)B * N == 0) return ATTN_OK;
    s = check_ptrs({q, k, v, o, lse});
    if (s != ATTN_OK) return s;
    if (workspace_bytes < attn_fwd_workspace_bytes(dtype, B, Hq, Hkv, N, d)) return ATTN_EINVAL;
    const AttnArgs a = make_args(dtype, out_dtype, q, k, v, o, lse, nullptr, nullptr, nullptr, nullptr,
                                 workspace, workspace_bytes, B, Hq, Hkv, N, d, causal, scale);
    hipStream_t st = (hipStream_t)stream;
    return from_hip(tca::mfma_path(a) ? tca::launch_fwd_mfma(a, st) : tca::launch_fwd_generic(a, st));
}

size_t attn_bwd_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int N, int d) {
    (void)Hkv;
    if (B < 0 || Hq < 0 || N < 0) return 0;
    return tca::bwd_workspace_size(dtype, B, Hq, N, d);
}

attn_status attn_bwd_dq(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                        int causal, float scale, void* stream) {
    bool noop = false;
    attn_status s = check_bwd(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B,
                              Hq, Hkv, N, d, causal, scale, &noop);
    if (s != ATTN_OK || noop) return s;
    const AttnArgs a = make_args(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes,
                                 B, Hq, Hkv, N, d, causal, scale);
    return run_dq(a, (hipStream_t)stream);
}

attn_status attn_bwd_dkdv(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                          int causal, float scale, void* stream) {
    bool noop = false;
    attn_status s = check_bwd(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B,
                              Hq, Hkv, N, d, causal, scale, &noop);
    if (s != ATTN_OK || noop) return s;
    const AttnArgs a = make_args(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes,
                                 B, Hq, Hkv, N, d, causal, scale);
    return run_dkdv(a, (hipStream_t)stream);
}

attn_status attn_bwd(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dO, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                     int causal, float scale, void* stream) {
    bool noop = false;
    attn_status s = check_bwd(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B,
                              Hq, Hkv, N, d, causal, scale, &noop);
    if (s != ATTN_OK || noop) return s;
    const AttnArgs a = make_args(dtype, out_dtype, q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes,
                                 B, Hq, Hkv, N, d, causal, scale);
    hipStream_t st = (hipStream_t)stream;
    s = run_dq(a, st);
    if (s != ATTN_OK) return s;
    return run_dkdv(a, st);
}

size_t attn_fwd_rope_workspace_bytes(attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d) {
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0) return 0;
    return rope_ws(nullptr, false, dtype, out_dtype, B, Hq, Hkv, N, d).total;
}
size_t attn_bwd_rope_workspace_bytes(attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d) {
    if (B < 0 || Hq < 0 || Hkv < 0 || N < 0 || d < 0) return 0;
    return rope_ws(nullptr, true, dtype, out_dtype, B, Hq, Hkv, N, d).total;
}

attn_status attn_fwd_rope(attn_dtype dtype, attn_dtype out_dtype, const void* q, const attn_layout* q_layout,
                          const void* k, const attn_layout* k_layout, const void* v, const attn_layout* v_layout,
                          const float* rope_cos, const float* rope_sin, void* k_rot, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal,
                          float scale, void* stream) {
    attn_status s = check_sizes(dtype, out_dtype, B, Hq, Hkv, N, d, causal, scale);
    if (s != ATTN_OK) return s;
    if ((int64_t)B * N == 0) return ATTN_OK;
    s = check_rope(dtype, out_dtype, q, q_layout, k, k_layout, v, v_layout, rope_cos, rope_sin, d);
    if (s != ATTN_OK) return s;
    s = check_ptrs({o, lse, workspace});
    if (s != ATTN_OK) return s;
    if (k_rot != nullptr && !aligned16(k_rot)) return ATTN_EINVAL;
    RopeWs w = rope_ws(workspace, false, dtype, out_dtype, B, Hq, Hkv, N, d);
    if (workspace_bytes < w.total) return ATTN_EINVAL;
    if (k_rot != nullptr) w.k = static_cast<char*>(k_rot);   // the rotated keys go to the caller's buffer
    hipStream_t st = (hipStream_t)stream;
    if (fused_rope(dtype, rope_cos, N, d)) {
        // fused: the forward reads q through its strides and rotates it into fp16 in
        // registers, and reads v in place (both through contiguous copies where their
        // rows do not allow it); only k is staged (rotated into fp16 once, read by every
        // query tile)
        const void *qv, *vv;
        const attn_layout *ql, *vl;
        if (fused_inputs(w, q, q_layout, v, v_layout, B, Hq, Hkv, N, d, &qv, &ql, &vv, &vl, st) != hipSuccess)
            return ATTN_EHIP;
        if (stage_k(w, k, k_layout, rope_cos, rope_sin, B, Hkv, N, d, st) != hipSuccess) return ATTN_EHIP;
        const tca::QRope rq = make_qrope(qv, ql, rope_cos, rope_sin, nullptr, nullptr, vv, vl, Hq, Hkv, N, d);
        AttnArgs a = make_args(dtype, out_dtype, qv, w.k, vv, o, lse, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                               B, Hq, Hkv, N, d, causal, scale);
        a.rope = &rq;
        return from_hip(tca::launch_fwd_mfma(a, st));
    }
    hipError_t e =
        stage_qkv(w, dtype, q, q_layout, k, k_layout, v, v_layout, rope_cos, rope_sin, B, Hq, Hkv, N, d, true, st);
    if (e != hipSuccess) return ATTN_EHIP;
    const AttnArgs a = make_args(dtype, out_dtype, w.q, w.k, w.v, o, lse, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, 0, B, Hq, Hkv, N, d, causal, scale);
    return from_hip(tca::mfma_path(a) ? tca::launch_fwd_mfma(a, st) : tca::launch_fwd_generic(a, st));
}

attn_status attn_bwd_rope(attn_dtype dtype, attn_dtype out_dtype, const void* q, const attn_layout* q_layout,
                          const void* k, const attn_layout* k_layout, const void* v, const attn_layout* v_layout,
                          const float* rope_cos, const float* rope_sin, const void* k_rot, const void* o,
                          const float* lse, const void* dO, void* dq, const attn_layout* dq_layout, void* dk,
                          const attn_layout* dk_layout, void* dv, const attn_layout* dv_layout, void* workspace,
                          size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                          void* stream) {
    attn_status s = check_sizes(dtype, out_dtype, B, Hq, Hkv, N, d, causal, scale);
    if (s != ATTN_OK) return s;
    if ((int64_t)B * N == 0) return ATTN_OK;
    s = check_rope(dtype, out_dtype, q, q_layout, k, k_layout, v, v_layout, rope_cos, rope_sin, d);
    if (s != ATTN_OK) return s;
    if (!layout_ok(dq_layout) || !layout_ok(dk_layout) || !layout_ok(dv_layout)) return ATTN_EINVAL;
    if (!elem_aligned(dq, out_dtype) || !elem_aligned(dk, out_dtype) || !elem_aligned(dv, out_dtype))
        return ATTN_EINVAL;
    s = check_ptrs({o, lse, dO, workspace});
    if (s != ATTN_OK) return s;
    if (k_rot != nullptr && !aligned16(k_rot)) return ATTN_EINVAL;
    RopeWs w = rope_ws(workspace, true, dtype, out_dtype, B, Hq, Hkv, N, d);
    if (workspace_bytes < w.total) return ATTN_EINVAL;
    const bool rotate_k = k_rot == nullptr;   // else the forward's rotated keys are read back
    if (!rotate_k) w.k = static_cast<char*>(const_cast<void*>(k_rot));
    hipStream_t st = (hipStream_t)stream;
    if (fused_rope(dtype, rope_cos, N, d)) {
        // fused: only k is staged (rotated into fp16), unless the forward's copy is given.
        // The dQ pass reads q through its strides, rotates it into fp16 in registers (its
        // fp16 copy for the dK/dV pass is rotated too), reads v in place and stores dq
        // turned back through dq's strides; the dK/dV pass reads v in place and stores dk
        // turned back, and dv, through their strides. q and v go through contiguous copies
        // where their rows do not allow reading them in place, and dq, whose rows are
        // stored 16 or 8 bytes at a time, through a contiguous copy scattered afterwards
        // where its rows are not 16-byte aligned.
        const void *qv, *vv;
        const attn_layout *ql, *vl;
        if (fused_inputs(w, q, q_layout, v, v_layout, B, Hq, Hkv, N, d, &qv, &ql, &vv, &vl, st) != hipSuccess)
            return ATTN_EHIP;
        if (rotate_k && stage_k(w, k, k_layout, rope_cos, rope_sin, B, Hkv, N, d, st) != hipSuccess)
            return ATTN_EHIP;
        const bool dq_direct = rows_aligned16(dq, dq_layout, elsize(out_dtype));
        void* dqt = dq_direct ? dq : static_cast<void*>(w.dq);
        const attn_layout* dql = dq_direct ? dq_layout : nullptr;
        const tca::QRope rq = make_qrope(qv, ql, rope_cos, rope_sin, dqt, dql, vv, vl, Hq, Hkv, N, d);
        const tca::KVRope rv = make_kvrope(vv, vl, dk, dk_layout, dv, dv_layout, rope_cos, rope_sin, Hkv, N, d);
        AttnArgs a = make_args(dtype, out_dtype, qv, w.k, vv, o, lse, dO, dqt, dk, dv, w.bwd, w.bwd_bytes, B, Hq, Hkv,
                               N, d, causal, scale);
        a.rope = &rq;
        s = run_dq(a, st);
        if (s != ATTN_OK) return s;
        AttnArgs a2 = a;
        a2.rope = nullptr;
        a2.kvrope = &rv;
        s = run_dkdv(a2, st);
        if (s != ATTN_OK || dq_direct) return s;
        const attn_layout cq = contiguous_layout(Hq, N, d);
        tca::CopyJobs jobs;
        jobs.n = 1;
        jobs.j[0] = tca::copy_job(w.dq, cq, dq, dq_layout ? *dq_layout : cq, B, Hq, N, d, 0);
        return from_hip(tca::layout_copy(out_dtype, out_dtype, jobs, nullptr, nullptr, N, d, st));
    }
    hipError_t e =
        stage_qkv(w, dtype, q, q_layout, k, k_layout, v, v_layout, rope_cos, rope_sin, B, Hq, Hkv, N, d, rotate_k, st);
    if (e != hipSuccess) return ATTN_EHIP;
    const attn_layout cq = contiguous_layout(Hq, N, d), ck = contiguous_layout(Hkv, N, d);
    const void* o_in = o;
    if (out_dtype == ATTN_BF16) {   // the backward runs with float32 outputs: widen o exactly
        tca::CopyJobs jobs;
        jobs.n = 1;
        jobs.j[0] = tca::copy_job(o, cq, w.o32, cq, B, Hq, N, d, 0);
        e = tca::layout_copy(ATTN_BF16, ATTN_F32, jobs, nullptr, nullptr, N, d, st);
        if (e != hipSuccess) return ATTN_EHIP;
        o_in = w.o32;
    }
    const AttnArgs a = make_args(dtype, ATTN_F32, w.q, w.k, w.v, o_in, lse, dO, w.dq, w.dk, w.dv, w.bwd, w.bwd_bytes,
                                 B, Hq, Hkv, N, d, causal, scale);
    s = run_dq(a, st);
    if (s != ATTN_OK) return s;
    s = run_dkdv(a, st);
    if (s != ATTN_OK) return s;
    // dq, dk turned back by the transpose rotation, dv copied; one launch
    const int rot = rope_cos ? 2 : 0;
    tca::CopyJobs jobs;
    jobs.n = 3;
    jobs.j[0] = tca::copy_job(w.dq, cq, dq, dq_layout ? *dq_layout : cq, B, Hq, N, d, rot);
    jobs.j[1] = tca::copy_job(w.dk, ck, dk, dk_layout ? *dk_layout : ck, B, Hkv, N, d, rot);
    jobs.j[2] = tca::copy_job(w.dv, ck, dv, dv_layout ? *dv_layout : ck, B, Hkv, N, d, 0);
    return from_hip(tca::layout_copy(ATTN_F32, out_dtype, jobs, rope_cos, rope_sin, N, d, st));
}

size_t attn_fwd_naive_workspace_bytes(int B, int Hq, int N) {
    if (B < 0 || Hq < 0 || N < 0) return 0;
    return tca::naive_workspace_size(B, Hq, N);
}

attn_status attn_fwd_naive(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                           void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                           int N, int d, int causal, float scale, void* stream) {
    attn_status s = check_sizes(dtype, out_dtype, B, Hq, Hkv, N, d, causal, scale);
    if (s != ATTN_OK) return s;
    if ((int64_t)B * N == 0) return ATTN_OK;
    if ((int64_t)B * Hq * N * N >= ((int64_t)1 << 39)) return ATTN_EINVAL;   // score count: grid and workspace
    s = check_ptrs({q, k, v, o, lse, workspace});
    if (s != ATTN_OK) return s;
    if (workspace_bytes < tca::naive_workspace_size(B, Hq, N)) return ATTN_EINVAL;
    const AttnArgs a = make_args(dtype, out_dtype, q, k, v, o, lse, nullptr, nullptr, nullptr, nullptr,
                                 workspace, workspace_bytes, B, Hq, Hkv, N, d, causal, scale);
    return from_hip(tca::launch_fwd_naive(a, (hipStream_t)stream));
}

size_t attn_decode_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (!known_dtype(dtype)) return 0;
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Nq < 1 || Nk < Nq || !supported_d(d)) return 0;
    return tca::decode_workspace_size(dtype == ATTN_F32, B, Hq, Hkv, Nq, Nk, d);
}

attn_status attn_decode(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                        int Nq, int Nk, int d, int causal, float scale, void* stream) {
    bool noop = false;
    attn_status s = check_decode(dtype, out_dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, &noop);
    if (s != ATTN_OK || noop) return s;
    const size_t need = tca::decode_workspace_size(dtype == ATTN_F32, B, Hq, Hkv, Nq, Nk, d);
    if (need > 0 && (workspace_bytes < need || workspace == nullptr || !aligned16(workspace))) return ATTN_EINVAL;
    const tca::DecodeArgs a =
        decode_args(dtype, out_dtype, q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, causal, scale);
    return from_hip(tca::launch_decode(a, (hipStream_t)stream));
}

attn_status attn_decode_noalloc(attn_dtype dtype, attn_dtype out_dtype, const void* q, const void* k,
                                const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                                int causal, float scale, void* stream) {
    bool noop = false;
    attn_status s = check_decode(dtype, out_dtype, q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, scale, &noop);
    if (s != ATTN_OK || noop) return s;
    const size_t need = tca::decode_workspace_size(dtype == ATTN_F32, B, Hq, Hkv, Nq, Nk, d);
    if (need > tca::kDecodeScratchBytes) return ATTN_ESCRATCH;
    void* ws = nullptr;
    if (need > 0 && tca::decode_scratch(&ws) != hipSuccess) return ATTN_EHIP;
    const tca::DecodeArgs a = decode_args(dtype, out_dtype, q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, causal, scale);
    return from_hip(tca::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
