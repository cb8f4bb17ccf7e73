// attn_decode.hip -- few-query attention over a key/value cache (decode).
//
// Inference (the NanoEuler blog page's FAQ: inference works, on 8 GB cards)
// runs the same attention with a handful of new query rows against every
// cached key: Nq rows that are the last Nq positions of an Nk-token sequence.
// Query row i sits at position Nk - Nq + i and, causally, sees keys
// j <= Nk - Nq + i. Definitions as in the forward (natural-log LSE saved).
//
// With few rows the work is a stream over the K/V cache: a GQA group of G
// query heads and Nq rows does 4 d G Nq flops per key against 4 d bytes of
// bf16 K and V, a few flops per byte, so HBM bandwidth bounds it. There are two
// split kernels. decode_mfma_kernel (bf16 inputs, d = 64 or 128, at least 3 rows
// per KV head, or 2 at d = 64) runs the forward's tile step on the matrix cores
// with the group's rows as the 32 columns of the products: columns that are
// mostly empty still cost less than the VALU dot products, whose per-key work
// otherwise outlasts the loads (details at the kernel). decode_split_kernel
// serves every other case on the VALU and is built around the loads:
//
//  * The G * Nq rows that share a KV head are processed together (RM rows per
//    wave, RM in {1, 2, 4, 8}; 32 on the matrix cores), so each K/V row is read
//    once per group.
//  * Split-K: the keys are cut into splits; one wave owns one (batch, KV head,
//    row chunk, split) item and the splits run in parallel. Each writes a
//    normalised partial output and its LSE; a second kernel merges the splits
//    through the LSEs: LSE = log sum_s e^LSE_s, O = sum_s e^(LSE_s - LSE) O_s.
//    A single split writes the result directly. With enough (batch, KV head,
//    row chunk) groups the splits of a group are instead the waves of one
//    workgroup, which merge through LDS: one launch and no workspace
//    (decode_fused_kernel from 256 groups, at most 16 splits, 8 for 8-row waves;
//    decode_mfma_fused_kernel from 128 chunks of 32 rows, 8 waves taking the
//    64-key tiles in turn). With fewer groups the CUs would not all be
//    streaming, so the splits stay spread over the chip.
//  * Lane layout: lane = CPR * slot + c, CPR = d / 8. A slot is one key, c is an
//    8-element chunk of its row, so one load instruction covers 64/CPR
//    consecutive whole K (or V) rows: 1 KB of contiguous bf16 per wave. Each
//    lane keeps its query chunks in registers, the partial dot products of a
//    slot are summed across its CPR lanes with DPP, and every slot runs its own
//    online softmax (running max with lazy rescaling, sum, and its 8 output
//    columns), so no cross-slot exchange happens inside the key loop. The
//    slots are merged once, at the end, with lane shuffles.
//  * kUnroll keys per slot are loaded ahead of their math (128 bytes per lane
//    in flight for bf16), enough outstanding loads to cover HBM latency at
//    2-4 waves per SIMD.
#include <mutex>
#include <type_traits>

#include "tca_internal.h"

namespace tca {

namespace dec {
constexpr int kWaves = 1;        // waves per workgroup (each wave runs its own work item)
constexpr int kUnroll = 2;       // keys per slot per batch (two batches in flight)
constexpr float kTau = 8.f;      // lazy-rescale threshold, log2 units
constexpr int kTargetWaves = 4096;   // work items aimed for (4 per SIMD)
constexpr int kMinSplitKeys = 64;    // keys per split at least
// splits merged inside one workgroup at most (its waves): 16 waves of at most 128
// registers share a CU; waves with more registers (8 rows; 4 rows of float32
// queries) go 8 to a workgroup
template <typename T, int RM>
constexpr int kFusedWaves = (RM == 8 || (RM == 4 && std::is_same<T, float>::value)) ? 8 : 16;
inline int fused_waves(int rm, bool in32) { return (rm == 8 || (rm == 4 && in32)) ? 8 : 16; }
constexpr long long kFusedMinGroups = 256;   // workgroups a merged-in-LDS launch needs at least (one per CU)
}  // namespace dec

// DPP lane moves within rows of 16 lanes (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7 - i within 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15 - i within 16 lanes

// Sum over the CPR consecutive lanes of a key slot (CPR in {2, 4, 8, 16}):
// after the quad steps each quad holds its sum; the mirrors pair lanes of
// different quads (8 lanes), then of different half-rows (16 lanes).
template <int CPR>
__device__ __forceinline__ float slot_sum(float x) {
    x += dpp<kQuadSwap1>(x);
    if constexpr (CPR >= 4) x += dpp<kQuadSwap2>(x);
    if constexpr (CPR >= 8) x += dpp<kRowHalfMirror>(x);
    if constexpr (CPR >= 16) x += dpp<kRowMirror>(x);
    return x;
}

// a.lo * b.lo + a.hi * b.hi + acc over packed bf16 pairs, in float32 (v_dot2_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}

// One 8-element chunk of a K or V row as raw bits (bf16: 16 bytes; float: 32).
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
    u32x4 w;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) { w = buf_load16(rs, off); }
    __device__ __forceinline__ void unpack(float (&x)[8]) const {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
};
template <> struct Chunk<float> {
    u32x4 a, b;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
        a = buf_load16(rs, off);
        b = buf_load16(rs, off + 16);
    }
    __device__ __forceinline__ void unpack(float (&x)[8]) const {
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y); x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y); x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    }
};

// One wave's split: keys [split * split_len, min(Nk, (split + 1) * split_len)) of
// unit = b * Hkv + hkv for rows rho = rc * RM + r < G * Nq (query head hkv * G +
// rho / Nq, query row rho % Nq). On return the lanes of slot 0 hold, per row, the
// running max m (log2 units), the sum l and the unnormalised output columns acc
// (lane c: columns 8c .. 8c + 7); grow is the row's global index (b, hq, i) and ok
// whether the row exists.
template <int RM>
struct SplitState {
    float m[RM], l[RM], acc[RM][8];
    size_t grow[RM];
    bool ok[RM];
};

template <typename T, int D, int RM>
__device__ __forceinline__ void decode_split_wave(SplitState<RM>& out, const T* __restrict__ q,
                                                  const T* __restrict__ k, const T* __restrict__ v, int Hq, int Hkv,
                                                  int Nq, int Nk, int causal, float scale, int unit, int rc, int split,
                                                  int split_len) {
    using namespace dec;
    constexpr int CPR = D / 8;        // lanes per key row
    constexpr int KS = 64 / CPR;      // key slots per wave
    const int lane = threadIdx.x & 63;
    const int b = unit / Hkv, hkv = unit % Hkv;
    const int G = Hq / Hkv, R = G * Nq;
    const int slot = lane / CPR, c = lane % CPR;
    const float sl2 = scale * kLog2e;

    const size_t kvoff = (size_t)unit * Nk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kvoff, (uint32_t)((size_t)Nk * D * sizeof(T)));
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + kvoff, (uint32_t)((size_t)Nk * D * sizeof(T)));
    // one batch: kUnroll keys per slot, i.e. KS * kUnroll consecutive keys
    constexpr int STEP = KS * kUnroll;
    auto load_batch = [&](Chunk<T> (&kc)[kUnroll], Chunk<T> (&vc)[kUnroll], int base) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            // rows past Nk read as zero through the buffer resource; they are masked below
            const uint32_t off = (uint32_t)(((base + u * KS + slot) * D + 8 * c) * (int)sizeof(T));
            kc[u].load(krs, off);
            vc[u].load(vrs, off);
        }
    };
    // the split's first batch goes out before the query rows are read (every key
    // of it lies below Nk + STEP, inside the buffer or reading zero past it)
    const int k0 = split * split_len;
    const int k1 = min(Nk, k0 + split_len);
    Chunk<T> ka[kUnroll], va[kUnroll], kb[kUnroll], vb[kUnroll];
    load_batch(ka, va, k0);

    // this lane's chunk of every row's query: bf16 inputs keep the raw pairs for
    // v_dot2_f32_bf16 (the score is scaled to log2 units after the slot sum);
    // float inputs keep floats pre-scaled to log2 units
    constexpr bool kBf16 = std::is_same<T, bf16_t>::value;
    float qr[RM][8];
    u32x4 qp2[RM];
    int lim[RM];          // keys j < lim[r] are visible to row r in this split
    size_t (&grow)[RM] = out.grow;   // global row index (b, hq, i) of row r
    bool (&ok)[RM] = out.ok;
    int kend = k0;        // keys this wave must visit
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        const int rho = rc * RM + r;
        ok[r] = rho < R;
        const int g = ok[r] ? rho / Nq : 0, i = ok[r] ? rho % Nq : 0;
        grow[r] = ((size_t)b * Hq + hkv * G + g) * Nq + i;
        const int pos = Nk - Nq + i;
        lim[r] = !ok[r] ? k0 : (causal ? min(k1, pos + 1) : k1);
        kend = max(kend, lim[r]);
        Chunk<T> qc;   // 8 consecutive elements: one (bf16) or two (float) 16-byte loads
        qc.load(make_rsrc(q + grow[r] * D, (uint32_t)(D * sizeof(T))), (uint32_t)(8 * c * (int)sizeof(T)));
        if constexpr (kBf16) {
            qp2[r] = ok[r] ? qc.w : u32x4{0u, 0u, 0u, 0u};
        } else {
            float x[8];
            qc.unpack(x);
#pragma unroll
            for (int t = 0; t < 8; ++t) qr[r][t] = ok[r] ? x[t] * sl2 : 0.f;
        }
    }

    float (&m)[RM] = out.m;
    float (&l)[RM] = out.l;
    float (&acc)[RM][8] = out.acc;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        m[r] = -0x1p100f;   // finite and far below any score: the first rescale factor is 0
        l[r] = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[r][t] = 0.f;
    }

    // a batch's scores first (independent products), then one rescale check per
    // batch, then the probabilities and the output columns
    auto compute_batch = [&](const Chunk<T> (&kc)[kUnroll], const Chunk<T> (&vc)[kUnroll], int base) {
        float sc[kUnroll][RM];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int j = base + u * KS + slot;
            if constexpr (kBf16) {
                const u32x4 kw = kc[u].w;
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    float part = dot2_bf16(qp2[r].x, kw.x, 0.f);
                    part = dot2_bf16(qp2[r].y, kw.y, part);
                    part = dot2_bf16(qp2[r].z, kw.z, part);
                    part = dot2_bf16(qp2[r].w, kw.w, part);
                    const float s = slot_sum<CPR>(part) * sl2;
                    sc[u][r] = (j < lim[r]) ? s : -INFINITY;
                }
            } else {
                float kf[8];
                kc[u].unpack(kf);
#pragma unroll
                for (int r = 0; r < RM; ++r) {
                    float part = 0.f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) part = fmaf(qr[r][t], kf[t], part);
                    const float s = slot_sum<CPR>(part);
                    sc[u][r] = (j < lim[r]) ? s : -INFINITY;
                }
            }
        }
        bool grow_max = false;
        float mb[RM];
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            mb[r] = sc[0][r];
#pragma unroll
            for (int u = 1; u < kUnroll; ++u) mb[r] = vmax(mb[r], sc[u][r]);
            grow_max |= mb[r] > m[r] + kTau;
        }
        if (__any(grow_max)) {
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const float mn = vmax(m[r], mb[r]);
                const float alpha = fast_exp2(m[r] - mn);   // 1 where the max did not move
                l[r] *= alpha;
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[r][t] *= alpha;
                m[r] = mn;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float vf[8];
            vc[u].unpack(vf);
#pragma unroll
            for (int r = 0; r < RM; ++r) {
                const float p = fast_exp2(sc[u][r] - m[r]);
                l[r] += p;
#pragma unroll
                for (int t = 0; t < 8; ++t) acc[r][t] = fmaf(p, vf[t], acc[r][t]);
            }
        }
    };
    // two register batches in turn: the loads of batch n + 1 are in flight while
    // batch n is computed (the wait for batch n leaves the younger loads pending)
    for (int base = k0; base < kend;) {
        if (base + STEP < kend) load_batch(kb, vb, base + STEP);
        compute_batch(ka, va, base);
        base += STEP;
        if (base >= kend) break;
        if (base + STEP < kend) load_batch(ka, va, base + STEP);
        compute_batch(kb, vb, base);
        base += STEP;
    }

    // merge the KS slots of the wave (lanes c, c + CPR, c + 2 CPR, ... hold the same
    // columns of different keys): log2(KS) rounds of pairwise merges across lanes
#pragma unroll
    for (int st = CPR; st < 64; st <<= 1) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const float mo = __shfl_xor(m[r], st, 64), lo = __shfl_xor(l[r], st, 64);
            const float mn = vmax(m[r], mo);
            const float a = fast_exp2(m[r] - mn), bb = fast_exp2(mo - mn);
            l[r] = a * l[r] + bb * lo;
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[r][t] = a * acc[r][t] + bb * __shfl_xor(acc[r][t], st, 64);
            m[r] = mn;
        }
    }
}

// Work item (one wave): item = ((unit * nrc) + rc) * nsplit + split, unit = b * Hkv + hkv.
// nsplit == 1: o and lse are written; otherwise opart [nsplit][B Hq Nq][D] (O_s,
// normalised) and lpart [nsplit][B Hq Nq] (LSE_s in log2 units, -inf when the
// split holds no visible key of the row).
template <typename T, typename OT, int D, int RM>
__global__ void __launch_bounds__(64 * dec::kWaves)
decode_split_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    OT* __restrict__ o, float* __restrict__ lse, float* __restrict__ opart,
                    float* __restrict__ lpart, int Hq, int Hkv, int Nq, int Nk, int causal, float scale,
                    int nrc, int nsplit, int split_len, int nitems, int nrows) {
    using namespace dec;
    constexpr int CPR = D / 8;
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (item >= nitems) return;       // whole waves only; the kernel has no barrier
    const int split = item % nsplit, rest = item / nsplit;
    const int rc = rest % nrc, unit = rest / nrc;
    SplitState<RM> st;
    decode_split_wave<T, D, RM>(st, q, k, v, Hq, Hkv, Nq, Nk, causal, scale, unit, rc, split, split_len);
    const int slot = lane / CPR, c = lane % CPR;
    const float (&m)[RM] = st.m;
    const float (&l)[RM] = st.l;
    const float (&acc)[RM][8] = st.acc;
    const size_t (&grow)[RM] = st.grow;
    const bool (&ok)[RM] = st.ok;
    if (slot != 0) return;
#pragma unroll
    for (int r = 0; r < RM; ++r) {
        if (!ok[r]) continue;
        const bool any = l[r] > 0.f;
        const float inv = any ? 1.f / l[r] : 0.f;
        const f32x4 lo4 = {acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv};
        const f32x4 hi4 = {acc[r][4] * inv, acc[r][5] * inv, acc[r][6] * inv, acc[r][7] * inv};
        const float l2 = any ? m[r] + __log2f(l[r]) : -INFINITY;
        if (nsplit == 1) {
            OT* orow = o + grow[r] * D + 8 * c;
            store_out4(orow, lo4);
            store_out4(orow + 4, hi4);
            if (c == 0) lse[grow[r]] = l2 * kLn2;
        } else {
            const size_t prow = (size_t)split * nrows + grow[r];
            *reinterpret_cast<f32x4*>(opart + prow * D + 8 * c) = lo4;
            *reinterpret_cast<f32x4*>(opart + prow * D + 8 * c + 4) = hi4;
            if (c == 0) lpart[prow] = l2;
        }
    }
}

// All nsplit splits of one (batch, KV head, row chunk) in one workgroup, wave w
// taking split w: each wave leaves its rows' normalised partial output and LSE
// (log2 units) in LDS, then the workgroup merges them as the merge kernel does,
// thread t taking column t % D of row t / D: LSE = log2 sum_w 2^LSE_w,
// O = sum_w 2^(LSE_w - LSE) O_w, with the splits added in order. Split 0 holds key
// 0, visible to every row, so the maximum is finite. Launched with 64 * nsplit
// threads, nsplit <= kFusedWaves<T, RM>.
template <typename T, typename OT, int D, int RM>
__global__ void __launch_bounds__((64 * dec::kFusedWaves<T, RM>))
decode_fused_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    OT* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk, int causal,
                    float scale, int nrc, int nsplit, int split_len) {
    using namespace dec;
    constexpr int MW = kFusedWaves<T, RM>;
    constexpr int CPR = D / 8;
    __shared__ __attribute__((aligned(16))) float po[MW][RM][D];
    __shared__ float pl[MW][RM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rc = blockIdx.x % nrc, unit = blockIdx.x / nrc;
    SplitState<RM> st;
    decode_split_wave<T, D, RM>(st, q, k, v, Hq, Hkv, Nq, Nk, causal, scale, unit, rc, w, split_len);
    const int slot = lane / CPR, c = lane % CPR;
    if (slot == 0) {
#pragma unroll
        for (int r = 0; r < RM; ++r) {
            const bool any = st.l[r] > 0.f;
            const float inv = any ? 1.f / st.l[r] : 0.f;
            *reinterpret_cast<f32x4*>(&po[w][r][8 * c]) =
                f32x4{st.acc[r][0] * inv, st.acc[r][1] * inv, st.acc[r][2] * inv, st.acc[r][3] * inv};
            *reinterpret_cast<f32x4*>(&po[w][r][8 * c + 4]) =
                f32x4{st.acc[r][4] * inv, st.acc[r][5] * inv, st.acc[r][6] * inv, st.acc[r][7] * inv};
            if (c == 0) pl[w][r] = any ? st.m[r] + __log2f(st.l[r]) : -INFINITY;
        }
    }
    __syncthreads();
    const int G = Hq / Hkv, R = G * Nq;
    const int b = unit / Hkv, hkv = unit % Hkv;
    for (int t = threadIdx.x; t < RM * D; t += 64 * nsplit) {
        const int r = t / D, col = t % D;
        const int rho = rc * RM + r;
        if (rho >= R) continue;
        const size_t grow = ((size_t)b * Hq + hkv * G + rho / Nq) * Nq + rho % Nq;
        float mx = pl[0][r];
        for (int sidx = 1; sidx < nsplit; ++sidx) mx = vmax(mx, pl[sidx][r]);
        float sum = 0.f, a = 0.f;
        for (int sidx = 0; sidx < nsplit; ++sidx) {
            const float wgt = fast_exp2(pl[sidx][r] - mx);
            sum += wgt;
            a = fmaf(wgt, po[sidx][r][col], a);
        }
        store_out1(o + grow * D + col, a * (1.f / sum));
        if (col == 0) lse[grow] = (mx + __log2f(sum)) * kLn2;
    }
}

// ---------------------------------------------------------------- matrix cores
// The matrix-core decode (bf16 inputs, d = 64 or 128): a chunk of 32 rows of a
// KV head's GQA group is the column set of 32x32x16 products, and each 64-key
// tile of the cache takes the forward's step (mfma_dec_tile). Two kernels use
// it: a split kernel (one wave per key split, merged by decode_merge_kernel) and
// a workgroup-merged form for calls with many chunks.
namespace decm {
constexpr int BC = 64;           // keys per tile
constexpr int kFusedWaves = 8;   // waves of the workgroup-merged form
// K reaches the A operands through LDS too (direct copies of whole rows) at d = 64:
// 1-10% faster there than each lane's 32-byte global loads; at d = 128 the second
// 16 KB tile per wave costs occupancy (the wide decode 19.8 -> 22.0 us), so K stays
// in registers
template <int D> constexpr bool kKLds = (D == 64);
// 32-row chunks from which the workgroup-merged form serves a call: measured
// faster than split kernel + merge kernel from 128 chunks on (caches of 1-4K keys),
// equal or slower below
constexpr long long kFusedMinChunks = 128;
using dec::kTau;
}

// One wave's running state over the tiles it has seen: the unnormalised O^T
// accumulator (lane (h, r): dims 32x + 8(e/4) + 4h + e%4 of row r), the running
// max in log2 units, and this lane's half of the sum of the fp16-rounded
// probabilities.
template <int D>
struct MfmaDecState {
    f32x16 oacc[D / 32];
    float m_s, l_run;
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int x = 0; x < D / 32; ++x) oacc[x] = f32x16{};
        m_s = -0x1p100f;   // finite, far below any score: the first rescale factor is 0
        l_run = 0.f;
    }
};

// This lane's row (column r of the products) of a (batch, KV head, 32-row chunk):
// its global index (b, hq, i), whether it exists, and its sequence position.
struct MfmaDecRow {
    size_t grow;
    bool ok;
    int pos;
    __device__ __forceinline__ MfmaDecRow(int b, int hkv, int rc, int r, int Hq, int Hkv, int Nq, int Nk) {
        const int G = Hq / Hkv, R = G * Nq;
        const int rho = rc * 32 + r;
        ok = rho < R;
        const int rv = ok ? rho : R - 1;
        const int g = rv / Nq, i = rv % Nq;
        grow = ((size_t)b * Hq + hkv * G + g) * Nq + i;
        pos = Nk - Nq + i;
    }
};

// The row's query chunks as loaded (a row past the chunk's rows reads the last
// one; its operand is zeroed when the first tile forms the operands): no use of
// the loaded values here, so the first tile's K and V requests go out behind
// these loads instead of after their arrival.
template <int D>
__device__ __forceinline__ void mfma_dec_load_q(u32x4 (&qraw)[D / 16], const bf16_t* q, const MfmaDecRow& row,
                                                int h) {
    const bf16_t* qrow = q + row.grow * D + 8 * h;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qraw[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
}

// Keys [t0, t0 + 64) of the unit, keys below `lim` visible to this lane's row. The
// V tile is copied into this wave's LDS buffer Vs (swizzled rows, bf16 bits), and
// the K tile into Ks (kKLds) or the K rows straight into registers as A operands;
// the wave waits for both (one round trip),
// then S^T = K Q^T, the online softmax down each column and O^T += V^T P^T with P
// rounded to fp16 and V^T read transposed (converted to fp16 at the read). Only
// this wave touches Vs: the fences keep its LDS reads of the previous tile ahead
// of the copies and its reads of this tile behind their arrival.
//
// The query's B operands (bf16, the scale's sign folded in, zero for a row past the
// chunk's rows) are formed from its loaded chunks in the first tile (`first`, wave
// uniform), after the wait that covers the query loads too.
template <int D>
__device__ __forceinline__ void mfma_dec_tile(MfmaDecState<D>& st, bf16x8 (&qb)[D / 16], const u32x4 (&qraw)[D / 16],
                                              bool first, bool qok, const ScoreScale& sc,
                                              __amdgpu_buffer_rsrc_t krs, const bf16_t* kunit, const bf16_t* vunit,
                                              int Nk, int t0, int lim, _Float16* Vs, _Float16* Ks, float sl2,
                                              int lane) {
    using namespace decm;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int NCOPY = BC * D * 2 / 1024;   // 1 KB direct copies per V tile
    const int h = lane >> 5, r = lane & 31;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    {
        const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vunit + (size_t)t0 * D, (uint32_t)((Nk - t0) * D * 2));
#pragma unroll
        for (int u = 0; u < NCOPY; ++u) lds_copy16(vrs, Vs + u * 512, tile_copy_src<D>(u, lane));
        if constexpr (kKLds<D>) {
            const __amdgpu_buffer_rsrc_t ks = make_rsrc(kunit + (size_t)t0 * D, (uint32_t)((Nk - t0) * D * 2));
#pragma unroll
            for (int u = 0; u < NCOPY; ++u) lds_copy16(ks, Ks + u * 512, tile_copy_src<D>(u, lane));
        }
    }
    const int krow_a = perm32(r);
    u32x4 ka[2][DC];
    if constexpr (!kKLds<D>) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < DC; ++c)
                ka[kb][c] = buf_load16(krs, (uint32_t)(((t0 + 32 * kb + krow_a) * D + 16 * c + 8 * h) * 2));
    }
    wait_vmem_all();   // the copies are in LDS
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (first) {
#pragma unroll
        for (int c = 0; c < DC; ++c) qb[c] = qok ? __builtin_bit_cast(bf16x8, apply_qsign(qraw[c], sc)) : bf16x8{};
    }
    // ---- S^T = K Q^T; accumulator e of block kb: key t0 + 32 kb + 16(e/8) + 8h + e%8
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const bf16x8 a = kKLds<D> ? *reinterpret_cast<const bf16x8*>(Ks + tile_off<D>(32 * kb + krow_a, 16 * c + 8 * h))
                                      : __builtin_bit_cast(bf16x8, ka[kb][c]);
            s[kb] = mfma_bf16(a, qb[c], s[kb]);
        }
        const int lm = lim - t0 - 32 * kb - 8 * h;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = (16 * (e >> 3) + (e & 7) < lm) ? s[kb][e] : -INFINITY;
    }
    // ---- online softmax down each column, lazy rescale (log2 units)
    const float mt = max_halves(vmax(max16(s[0]), max16(s[1]))) * sl2;
    if (__any(mt > st.m_s + kTau)) {
        const float m_new = vmax(st.m_s, mt);
        const float alpha = fast_exp2(st.m_s - m_new);
        st.l_run *= alpha;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.oacc[x][e] *= alpha;
        st.m_s = m_new;
    }
    // ---- O^T += V^T P^T, P in fp16 (its rounded values are the ones summed)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            uint32_t pk[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                pk[t] = pack_f16(fast_exp2(fmaf(s[kb][8 * c2 + 2 * t], sl2, -st.m_s)),
                                 fast_exp2(fmaf(s[kb][8 * c2 + 2 * t + 1], sl2, -st.m_s)));
                st.l_run = add_f16_pair(pk[t], st.l_run);
            }
            const f16x8 pb = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
            for (int x = 0; x < DB; ++x) {
                const f16x8 vt = tile_tr_operand<D>(Vs, 32 * kb + 16 * c2, 32 * x, h, r);   // bf16 bits
                const f16x8 a = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(__builtin_bit_cast(u32x4, vt)));
                st.oacc[x] = mfma_f16(a, pb, st.oacc[x]);
            }
        }
}

// Matrix-core split for bf16 inputs at d = 64 and 128. One wave per (batch, KV
// head, row chunk, key split) item, as decode_split_kernel, but the chunk holds
// 32 rows of the GQA group -- the columns of 32x32x16 products -- and each
// 64-key tile is the forward's step with the roles kept (mfma_dec_tile): K rows
// as the A operand straight from global memory (rows past Nk read as zero), the
// chunk's queries as the B operand, V through LDS. Rows past the chunk's G * Nq
// rows carry zero queries and are not stored. The scale's sign is folded into Q
// (ScoreScale), so the exponent's multiplier is positive and masked keys stay at
// -inf. Output as the split kernel's: o, lse when nsplit == 1, else the
// normalised partial and its LSE (log2 units) per split for the merge kernel.
template <typename OT, int D>
__global__ void __launch_bounds__(64, (D == 64) ? 3 : 2)   // waves per SIMD at least
decode_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                   OT* __restrict__ o, float* __restrict__ lse, float* __restrict__ opart,
                   float* __restrict__ lpart, int Hq, int Hkv, int Nq, int Nk, int causal, ScoreScale sc,
                   int nrc, int nsplit, int split_len, int nrows) {
    using namespace decm;
    constexpr int DB = D / 32;
    __shared__ __attribute__((aligned(16))) _Float16 Vs[BC * D];
    __shared__ __attribute__((aligned(16))) _Float16 Ks[kKLds<D> ? BC * D : 8];
    const int lane = threadIdx.x, h = lane >> 5, r = lane & 31;
    const int item = blockIdx.x;
    const int split = item % nsplit, rest = item / nsplit;
    const int rc = rest % nrc, unit = rest / nrc;
    const int b = unit / Hkv, hkv = unit % Hkv;
    const MfmaDecRow row(b, hkv, rc, r, Hq, Hkv, Nq, Nk);
    const int k0 = split * split_len, k1 = min(Nk, k0 + split_len);
    const int lim = !row.ok ? k0 : (causal ? min(k1, row.pos + 1) : k1);   // keys below lim are visible

    u32x4 qraw[D / 16];
    bf16x8 qb[D / 16];
    mfma_dec_load_q<D>(qraw, q, row, h);
    const size_t kvoff = (size_t)unit * Nk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kvoff, (uint32_t)((size_t)Nk * D * 2));
    MfmaDecState<D> st;
    st.init();
    for (int t0 = k0; t0 < k1; t0 += BC)
        mfma_dec_tile<D>(st, qb, qraw, t0 == k0, row.ok, sc, krs, k + kvoff, v + kvoff, Nk, t0, lim, Vs, Ks, sc.sl2,
                         lane);

    // ---- this split's normalised output and LSE
    const float l_tot = sum_halves(st.l_run);
    if (!row.ok) return;
    const bool any = l_tot > 0.f;
    const float inv = any ? 1.f / l_tot : 0.f;
    const float l2 = any ? st.m_s + __log2f(l_tot) : -INFINITY;
    if (nsplit == 1) {
        OT* orow = o + row.grow * D;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
                store_out4(orow + 32 * x + 8 * a4 + 4 * h,
                           f32x4{st.oacc[x][4 * a4] * inv, st.oacc[x][4 * a4 + 1] * inv,
                                 st.oacc[x][4 * a4 + 2] * inv, st.oacc[x][4 * a4 + 3] * inv});
        if (h == 0) lse[row.grow] = l2 * kLn2;
    } else {
        const size_t prow = (size_t)split * nrows + row.grow;
        float* orow = opart + prow * D;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
                *reinterpret_cast<f32x4*>(orow + 32 * x + 8 * a4 + 4 * h) =
                    f32x4{st.oacc[x][4 * a4] * inv, st.oacc[x][4 * a4 + 1] * inv, st.oacc[x][4 * a4 + 2] * inv,
                          st.oacc[x][4 * a4 + 3] * inv};
        if (h == 0) lpart[prow] = l2;
    }
}

// The workgroup-merged form of the matrix-core split: one workgroup of 8 waves per
// (batch, KV head, 32-row chunk); wave w takes the 64-key tiles w, w + 8, ... of
// the whole cache with one running state, leaves its unnormalised output (over
// its V buffer, [32 rows][D] floats at merge_off positions) and its rows' max and
// sum in LDS, and after one barrier the workgroup merges the 8 states in wave
// order: M = max_w m_w, L = sum_w 2^(m_w - M) l_w, O = sum_w 2^(m_w - M) O_w / L.
// One launch, no workspace. The wave holding key 0 gives every row a finite max.
template <typename OT, int D>
__global__ void __launch_bounds__(64 * decm::kFusedWaves)
decode_mfma_fused_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                         OT* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int Nq, int Nk, int causal,
                         ScoreScale sc, int nrc) {
    using namespace decm;
    constexpr int W = kFusedWaves, DB = D / 32;
    static_assert(32 * D * 4 == BC * D * 2, "a wave's partial output fills its V buffer");
    __shared__ __attribute__((aligned(16))) _Float16 Vs[W][BC * D];
    __shared__ __attribute__((aligned(16))) _Float16 Ks[kKLds<D> ? W : 1][kKLds<D> ? BC * D : 8];
    __shared__ float ml[W][2][32];
    const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rc = blockIdx.x % nrc, unit = blockIdx.x / nrc;
    const int b = unit / Hkv, hkv = unit % Hkv;
    const MfmaDecRow row(b, hkv, rc, r, Hq, Hkv, Nq, Nk);
    const int lim = !row.ok ? 0 : (causal ? min(Nk, row.pos + 1) : Nk);

    u32x4 qraw[D / 16];
    bf16x8 qb[D / 16];
    mfma_dec_load_q<D>(qraw, q, row, h);
    const size_t kvoff = (size_t)unit * Nk * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kvoff, (uint32_t)((size_t)Nk * D * 2));
    MfmaDecState<D> st;
    st.init();
    const int ntiles = (Nk + BC - 1) / BC;
    for (int t = w; t < ntiles; t += W)
        mfma_dec_tile<D>(st, qb, qraw, t == w, row.ok, sc, krs, k + kvoff, v + kvoff, Nk, t * BC, lim, Vs[w],
                         Ks[kKLds<D> ? w : 0], sc.sl2, lane);

    // ---- this wave's state into LDS (its V buffer, whose reads are done)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    float* po = reinterpret_cast<float*>(Vs[w]);
#pragma unroll
    for (int x = 0; x < DB; ++x)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
            *reinterpret_cast<f32x4*>(po + merge_off<D>(r, 8 * x + 2 * a4 + h)) =
                f32x4{st.oacc[x][4 * a4], st.oacc[x][4 * a4 + 1], st.oacc[x][4 * a4 + 2], st.oacc[x][4 * a4 + 3]};
    const float l_tot = sum_halves(st.l_run);
    if (h == 0) {
        ml[w][0][r] = st.m_s;
        ml[w][1][r] = l_tot;
    }
    __syncthreads();
    // ---- merge: thread t takes element (row, column) t, t + 64 W, ... of the chunk
    const int R = (Hq / Hkv) * Nq;
    for (int idx = threadIdx.x; idx < 32 * D; idx += 64 * W) {
        const int rr = idx / D, c = idx % D;
        if (rc * 32 + rr >= R) break;   // rows grow with idx
        float M = ml[0][0][rr];
#pragma unroll
        for (int ww = 1; ww < W; ++ww) M = vmax(M, ml[ww][0][rr]);
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < W; ++ww) {
            const float wt = fast_exp2(ml[ww][0][rr] - M);
            L = fmaf(wt, ml[ww][1][rr], L);
            acc = fmaf(wt, reinterpret_cast<const float*>(Vs[ww])[merge_off<D>(rr, c >> 2) + (c & 3)], acc);
        }
        const MfmaDecRow orow(b, hkv, rc, rr, Hq, Hkv, Nq, Nk);
        store_out1(o + orow.grow * D + c, acc / L);
        if (c == 0) lse[orow.grow] = (M + __log2f(L)) * kLn2;
    }
}

// Merge of the splits of one row: LSE = log2 sum_s 2^LSE_s (log2 units in lpart),
// O = sum_s 2^(LSE_s - LSE) O_s. CB = D / (2 NP) workgroups of 256 threads per
// row, each owning NP column pairs: with many splits NP = 16 (4 workgroups per
// row at d = 128, so a few dozen rows still spread over the CUs), with few one
// workgroup takes the whole row (NP = D / 2). In each, thread t takes the
// maximum and weight sum over split t (workgroup reductions through LDS, the
// weights kept in LDS; every workgroup of a row computes the same values), then
// thread t = (split group g, column pair p) accumulates its two columns over
// splits g, g + NG, ... (NG = 256 / NP groups), with the partial sums added
// across the groups through LDS in a fixed order. Every thread loads only its
// own splits; the first kMergePre of them before the split statistics, so their
// loads are in flight during the reductions rather than after them (the sums
// run in the same order either way). Split 0 holds key 0, visible to every row,
// so the maximum is finite.
constexpr int kMergeThreads = 256;
constexpr int kMergeColSplits = 32;   // more splits per row than this: column blocks of 16 pairs
constexpr int kMergePre = 4;          // partial-row loads per thread issued ahead of the statistics
template <typename OT, int D, int NP>
__global__ void __launch_bounds__(kMergeThreads)
decode_merge_kernel(const float* __restrict__ opart, const float* __restrict__ lpart, OT* __restrict__ o,
                    float* __restrict__ lse, int nrows, int nsplit) {
    constexpr int NW = kMergeThreads / 64;
    constexpr int MAXS = 256;                 // splits per row at most (decode_plan caps it)
    constexpr int CB = D / (2 * NP);          // workgroups per row
    constexpr int NG = kMergeThreads / NP;    // split groups
    static_assert(kMergeThreads % NP == 0 && NP * CB * 2 == D, "merge tiling");
    __shared__ float red[NW];
    __shared__ float wsh[MAXS];
    __shared__ float2 part[NG][NP];
    const int row = blockIdx.x / CB;
    const int c0 = 2 * NP * (blockIdx.x % CB);   // first column of this workgroup
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int p = tid % NP, g = tid / NP;
    float2 xe[kMergePre];
#pragma unroll
    for (int i = 0; i < kMergePre; ++i) {   // unconditional (clamped) loads: one wait for all of them
        const int sidx = min(g + i * NG, nsplit - 1);
        xe[i] = *reinterpret_cast<const float2*>(opart + ((size_t)sidx * nrows + row) * D + c0 + 2 * p);
    }
    const float ls = tid < nsplit ? lpart[(size_t)tid * nrows + row] : -INFINITY;
    float mx = ls;
#pragma unroll
    for (int st = 32; st > 0; st >>= 1) mx = vmax(mx, __shfl_xor(mx, st, 64));
    if (lane == 0) red[w] = mx;
    __syncthreads();
    mx = vmax(vmax(red[0], red[1]), vmax(red[2], red[3]));
    const float wt = tid < nsplit ? fast_exp2(ls - mx) : 0.f;
    wsh[tid] = wt;
    float sum = wt;
#pragma unroll
    for (int st = 32; st > 0; st >>= 1) sum += __shfl_xor(sum, st, 64);
    __syncthreads();
    if (lane == 0) red[w] = sum;
    __syncthreads();
    sum = (red[0] + red[1]) + (red[2] + red[3]);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < kMergePre; ++i) {
        const int sidx = g + i * NG;
        if (sidx < nsplit) {
            const float wgt = wsh[sidx];
            a0 = fmaf(wgt, xe[i].x, a0);
            a1 = fmaf(wgt, xe[i].y, a1);
        }
    }
#pragma unroll 4
    for (int sidx = g + kMergePre * NG; sidx < nsplit; sidx += NG) {
        const float2 x = *reinterpret_cast<const float2*>(opart + ((size_t)sidx * nrows + row) * D + c0 + 2 * p);
        const float wgt = wsh[sidx];
        a0 = fmaf(wgt, x.x, a0);
        a1 = fmaf(wgt, x.y, a1);
    }
    part[g][p] = float2{a0, a1};
    __syncthreads();
    if (g == 0) {
        float r0 = 0.f, r1 = 0.f;
#pragma unroll
        for (int gg = 0; gg < NG; ++gg) {
            r0 += part[gg][p].x;
            r1 += part[gg][p].y;
        }
        const float inv = 1.f / sum;
        store_out1(o + (size_t)row * D + c0 + 2 * p, r0 * inv);
        store_out1(o + (size_t)row * D + c0 + 2 * p + 1, r1 * inv);
    }
    if (c0 == 0 && tid == 0) lse[row] = (mx + __log2f(sum)) * kLn2;
}

// ---------------------------------------------------------------- host side
// Key splits for `items0` (batch, KV head, row chunk) groups: about kTargetWaves
// waves in all, at least kMinSplitKeys keys (a multiple of 64) per split, at most
// 256 splits per row.
static void plan_splits(DecodePlan& p, long long items0, int Nk) {
    long long want = (dec::kTargetWaves + items0 - 1) / items0;
    const long long cap = ((long long)Nk + dec::kMinSplitKeys - 1) / dec::kMinSplitKeys;
    want = want < 1 ? 1 : want;
    want = want > cap ? cap : want;
    want = want > 256 ? 256 : want;
    p.split_len = (int)((((long long)Nk + want - 1) / want + 63) / 64 * 64);
    if (p.split_len < 64) p.split_len = 64;
    p.nsplit = (int)(((long long)Nk + p.split_len - 1) / p.split_len);
    if (p.nsplit < 1) p.nsplit = 1;
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d, bool in32) {
    DecodePlan p;
    const int R = (Hq / Hkv) * Nq;
    p.rm = R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : 8;
    p.nrc = (R + p.rm - 1) / p.rm;
    const long long items0 = (long long)B * Hkv * p.nrc;
    plan_splits(p, items0, Nk);
    // merged in the workgroup when there are enough workgroups to fill the CUs: with
    // fewer, one CU streaming a whole row chunk's splits is slower than splits spread
    // over the chip plus a merge kernel
    p.fused = p.nsplit > 1 && p.nsplit <= dec::fused_waves(p.rm, in32) && items0 >= dec::kFusedMinGroups;
    p.mfma = false;
    // matrix-core splits, row chunks of 32 rows: measured faster from 3 rows per KV
    // head (2 at d = 64); with one or two rows the 32-column products sit nearly
    // empty and the VALU split, whose K reads are whole rows, is faster. With at
    // least 128 chunks their workgroup-merged form serves the call; otherwise they
    // replace the VALU's merged form only at d = 128 with 8 or more rows, and only
    // when their split partials fit the no-allocation scratch (so both entry points
    // keep serving the same calls).
    if (!in32 && (d == 64 || d == 128) && (R >= 3 || (R == 2 && d == 64))) {
        DecodePlan m = p;
        m.mfma = true;
        m.fused = false;
        m.rm = 32;
        m.nrc = (R + 31) / 32;
        const long long chunks = (long long)B * Hkv * m.nrc;
        plan_splits(m, chunks, Nk);
        const size_t rows = (size_t)B * Hq * Nq;
        const size_t part = m.nsplit <= 1 ? 0
                                          : ws_round((size_t)m.nsplit * rows * d * sizeof(float)) +
                                                ws_round((size_t)m.nsplit * rows * sizeof(float));
        if (chunks >= decm::kFusedMinChunks && m.nsplit > 1) {
            m.fused = true;   // the waves take 64-key tiles in turn; nsplit is not used
            p = m;
        } else if (!p.fused || (d == 128 && R >= 8 && part <= kDecodeScratchBytes)) {
            p = m;
        }
    }
    return p;
}

size_t decode_workspace_size(bool in32, int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    const DecodePlan p = decode_plan(B, Hq, Hkv, Nq, Nk, d, in32);
    if (p.nsplit <= 1 || p.fused) return 0;
    const size_t rows = (size_t)B * Hq * Nq;
    return ws_round((size_t)p.nsplit * rows * d * sizeof(float)) + ws_round((size_t)p.nsplit * rows * sizeof(float));
}

// The merge of the split partials (after either split kernel).
template <typename OT, int D>
static void launch_merge(const DecodeArgs& a, const DecodePlan& p, const float* opart, const float* lpart, int nrows,
                         hipStream_t st) {
    if (p.nsplit > kMergeColSplits && D >= 32) {
        constexpr int NP = D >= 32 ? 16 : D / 2;
        hipLaunchKernelGGL((decode_merge_kernel<OT, D, NP>), dim3((unsigned)((long long)nrows * (D / (2 * NP)))),
                           dim3(kMergeThreads), 0, st, opart, lpart, (OT*)a.o, a.lse, nrows, p.nsplit);
    } else if (p.nsplit > 1) {
        hipLaunchKernelGGL((decode_merge_kernel<OT, D, D / 2>), dim3((unsigned)nrows), dim3(kMergeThreads), 0, st,
                           opart, lpart, (OT*)a.o, a.lse, nrows, p.nsplit);
    }
}

// Split partials in the workspace: opart [nsplit][rows][D] floats, then lpart [nsplit][rows].
static void split_partials(const DecodeArgs& a, const DecodePlan& p, int nrows, float** opart, float** lpart) {
    *opart = nullptr;
    *lpart = nullptr;
    if (p.nsplit > 1) {
        *opart = static_cast<float*>(a.workspace);
        *lpart = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                          ws_round((size_t)p.nsplit * nrows * a.d * sizeof(float)));
    }
}

template <typename OT, int D>
static hipError_t launch_decode_mfma(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    if (p.fused) {
        hipLaunchKernelGGL((decode_mfma_fused_kernel<OT, D>), dim3((unsigned)(a.B * a.Hkv * p.nrc)),
                           dim3(64 * decm::kFusedWaves), 0, st, (const bf16_t*)a.q, (const bf16_t*)a.k,
                           (const bf16_t*)a.v, (OT*)a.o, a.lse, a.Hq, a.Hkv, a.Nq, a.Nk, a.causal,
                           score_scale(a.scale), p.nrc);
        return hipGetLastError();
    }
    const int nitems = a.B * a.Hkv * p.nrc * p.nsplit;
    const int nrows = a.B * a.Hq * a.Nq;
    float *opart, *lpart;
    split_partials(a, p, nrows, &opart, &lpart);
    hipLaunchKernelGGL((decode_mfma_kernel<OT, D>), dim3((unsigned)nitems), dim3(64), 0, st, (const bf16_t*)a.q,
                       (const bf16_t*)a.k, (const bf16_t*)a.v, (OT*)a.o, a.lse, opart, lpart, a.Hq, a.Hkv, a.Nq,
                       a.Nk, a.causal, score_scale(a.scale), p.nrc, p.nsplit, p.split_len, nrows);
    launch_merge<OT, D>(a, p, opart, lpart, nrows, st);
    return hipGetLastError();
}

template <typename T, typename OT, int D, int RM>
static hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    if (p.fused) {   // one workgroup per (batch, KV head, row chunk), one wave per split
        hipLaunchKernelGGL((decode_fused_kernel<T, OT, D, RM>), dim3((unsigned)(a.B * a.Hkv * p.nrc)),
                           dim3(64 * p.nsplit), 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, (OT*)a.o, a.lse,
                           a.Hq, a.Hkv, a.Nq, a.Nk, a.causal, a.scale, p.nrc, p.nsplit, p.split_len);
        return hipGetLastError();
    }
    const int nitems = a.B * a.Hkv * p.nrc * p.nsplit;
    const int nrows = a.B * a.Hq * a.Nq;
    float *opart, *lpart;
    split_partials(a, p, nrows, &opart, &lpart);
    const dim3 grid((unsigned)((nitems + dec::kWaves - 1) / dec::kWaves));
    hipLaunchKernelGGL((decode_split_kernel<T, OT, D, RM>), grid, dim3(64 * dec::kWaves), 0, st,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, (OT*)a.o, a.lse, opart, lpart, a.Hq,
                       a.Hkv, a.Nq, a.Nk, a.causal, a.scale, p.nrc, p.nsplit, p.split_len, nitems, nrows);
    launch_merge<OT, D>(a, p, opart, lpart, nrows, st);
    return hipGetLastError();
}

template <typename T, typename OT, int D>
static hipError_t launch_decode_rm(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    switch (p.rm) {
        case 1: return launch_decode_t<T, OT, D, 1>(a, p, st);
        case 2: return launch_decode_t<T, OT, D, 2>(a, p, st);
        case 4: return launch_decode_t<T, OT, D, 4>(a, p, st);
        default: return launch_decode_t<T, OT, D, 8>(a, p, st);
    }
}

template <typename T, typename OT>
static hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (p.mfma) return (a.d == 64) ? launch_decode_mfma<OT, 64>(a, p, st) : launch_decode_mfma<OT, 128>(a, p, st);
    }
    switch (a.d) {
        case 16: return launch_decode_rm<T, OT, 16>(a, p, st);
        case 32: return launch_decode_rm<T, OT, 32>(a, p, st);
        case 64: return launch_decode_rm<T, OT, 64>(a, p, st);
        case 128: return launch_decode_rm<T, OT, 128>(a, p, st);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- fixed scratch
// The split partials of attn_decode_noalloc live in this file-scope device array
// instead of a caller workspace, for callers that cannot allocate. Each GPU holds
// its own copy, at its own address, until the process ends. In host code the
// array's name is only a host-side stand-in: kernels and copies get the device
// address that hipGetSymbolAddress returns, taken once per device with that
// device current, kept below and used everywhere instead of the name. Nothing in
// it needs clearing: every partial the merge reads is written by the split
// kernel of the same call. Calls that overlap on one GPU share it and race.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptrs[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    const bool in32 = a.dtype == ATTN_F32, out32 = a.out_dtype == ATTN_F32;
    const DecodePlan p = decode_plan(a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d, in32);
    if (in32) return out32 ? launch_decode_d<float, float>(a, p, st) : launch_decode_d<float, bf16_t>(a, p, st);
    return out32 ? launch_decode_d<bf16_t, float>(a, p, st) : launch_decode_d<bf16_t, bf16_t>(a, p, st);
}

}  // namespace tca
