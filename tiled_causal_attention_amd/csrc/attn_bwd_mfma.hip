// attn_bwd_mfma.hip -- causal GQA attention backward on gfx950 matrix cores.
//
// The backward the pages hand-derive (P recomputed from the saved
// log-sum-exp, D = rowsum(dO o O), dS = P o (dP - D), then dQ, dK, dV) runs as
// two kernels with no atomics, so every output is written exactly once and is
// bitwise reproducible:
//
//   1. bwd_dq_kernel, query-tile parallel (the shape of the forward): for its
//      query rows it computes D from O and dO, writes D to the workspace, then
//      walks the visible K/V tiles: S^T = K Q^T, P, dP^T = V dO^T, dS, and
//      dQ^T += K^T dS^T; dQ is stored once at the end.
//   2. bwd_dkdv_kernel, K/V-tile parallel: a workgroup owns 64 keys of one
//      (batch, KV head), walks every query head of its GQA group and every
//      query tile at or below the diagonal, and accumulates dV += P^T dO and
//      dK += dS^T Q in registers (reading D from the workspace).
//
// Float32 atomics were measured at ~0.6 G adds/ms on this part (an L2 limit):
// accumulating dQ (or dK/dV across the query heads of a group) through them
// costs more than recomputing S and dP in a second kernel, which is why dQ has
// its own pass.
//
// Precision: S and dP are bf16 (dQ pass: dP) or fp16 (dK/dV pass, dQ pass S)
// products of the bf16 inputs -- identical values, since bf16 -> fp16 is
// exact for |x| >= 2^-14 -- with fp32 accumulation. P and dS, computed values,
// are rounded to fp16 (not bf16) for the products that consume them; their
// partner operands are converted to fp16 in registers or when staged to LDS.
#include <type_traits>

#include "tca_internal.h"

namespace tca {

// dQ pass layout: 4 waves per workgroup. d = 64: 64 query rows, row blocks of 32
// rows x 2 key halves (wave (rb, kh) takes keys 32kh .. 32kh+31 of each K/V
// tile); the two key halves' partial dQ are summed through LDS at the end; 3
// workgroups per CU. d = 128: 128 rows, one wave per row block taking both
// 32-key blocks of each tile in turn (P comes from the saved LSE, so the blocks
// are independent), no merge; with D taken from the workspace rather than held
// as a -D accumulator it stays within 256 registers, and two workgroups share a
// CU, so the two waves of a SIMD do not wait at the same barriers.
namespace bwdq {
template <int D> constexpr int kWaves = 4;
template <int D> constexpr int kKeyHalves = (D == 128) ? 1 : 2;   // waves sharing a row block
template <int D> constexpr int kThreads = 64 * kWaves<D>;
template <int D> constexpr int kRows = 32 * kWaves<D> / kKeyHalves<D>;   // query rows per workgroup
constexpr int BC = 64;           // keys per K/V tile
template <int D> constexpr int kPad = (D == 128) ? 24 : 8;   // K/V tile row padding, as the forward's
}  // namespace bwdq

// Global -> registers: the K and V chunks of one tile. K through a buffer resource
// over the head's N contiguous rows, koff this thread's byte offset of its first
// chunk (row tid / (D/8), chunk tid % (D/8) of the tile); V through vr, at this
// thread's in-tile offset vlane plus the tile's byte offset vtile_off. Thread tid
// owns chunks tid + T u, T threads (a wave reads whole rows); rows past the end
// of the sequence read as zero.
template <int D, int KCH, bool ROPE>
__device__ __forceinline__ void bwd_load_kv(u32x4 (&kreg)[KCH], u32x4 (&vreg)[KCH], __amdgpu_buffer_rsrc_t kr,
                                            uint32_t koff, const VRows<D, ROPE>& vr, uint32_t vlane,
                                            uint32_t vtile_off) {
    constexpr int ROWS_PER_U = bwdq::kThreads<D> / (D / 8);
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        kreg[u] = buf_load16(kr, koff + u * bwdq::kThreads<D> * 16);
        vreg[u] = vr.load16(vlane, vtile_off + u * ROWS_PER_U * vr.row_bytes);
    }
}

// Registers -> LDS: K as fp16 rows (converted from bf16, or as it is when KF16:
// the rotated keys come in fp16), V kept as bf16 rows. kdst/vdst point at this
// thread's chunk 0 (row tid / (D/8), column 8 (tid % (D/8))); chunk u sits
// T u / (D/8) rows further down (T threads).
template <int D, int KCH, bool KF16>
__device__ __forceinline__ void bwd_store_kv(const u32x4 (&kreg)[KCH], const u32x4 (&vreg)[KCH],
                                             _Float16* kdst, bf16_t* vdst) {
    constexpr int ROWS_PER_U = bwdq::kThreads<D> / (D / 8);
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        *reinterpret_cast<u32x4*>(kdst + u * ROWS_PER_U * (D + bwdq::kPad<D>)) =
            KF16 ? kreg[u] : bf16x8_to_f16x8(kreg[u]);
        *reinterpret_cast<u32x4*>(vdst + u * ROWS_PER_U * (D + bwdq::kPad<D>)) = vreg[u];
    }
}

// The table values a lane needs to turn its dQ row back (ROPE): frequency
// 32x + 8 a4 + 4h .. +3 of row qi for dim block x < D/64. Loaded on their own so
// that the kernel can issue them before its last barrier.
template <int D, bool ROPE>
struct DqTab {
    f32x4 c[D / 64][4], s[D / 64][4];
    __device__ __forceinline__ void load(const QRope& rq, int qi, int h) {
        if constexpr (ROPE) {
            const float* cr = rq.cs + (size_t)qi * (D / 2);
            const float* sr = rq.sn + (size_t)qi * (D / 2);
#pragma unroll
            for (int x = 0; x < D / 64; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    c[x][a4] = *reinterpret_cast<const f32x4*>(cr + 32 * x + 8 * a4 + 4 * h);
                    s[x][a4] = *reinterpret_cast<const f32x4*>(sr + 32 * x + 8 * a4 + 4 * h);
                }
        }
    }
};

// Store one query row's dQ (val[x][a4] holds dims 32x + 8 a4 + 4h .. +3). ROPE: the
// pairs (dim, dim + D/2) -- blocks x and x + D/64 of the same lane -- are turned
// back by the transpose rotation at row position qi (tab: that row's table values)
// and written through rq's dq strides; otherwise the row goes to `row` as it is.
template <int D, typename OT, bool ROPE>
__device__ __forceinline__ void store_dq_row(OT* row, const f32x4 (&val)[D / 32][4], const QRope& rq,
                                             const DqTab<D, ROPE>& tab, int b, int hq, int qi, int h) {
    constexpr int DB = D / 32;
    if constexpr (ROPE) {
        OT* dst = static_cast<OT*>(rq.dq) + b * rq.gb + hq * rq.gh + qi * rq.gn;
#pragma unroll
        for (int x = 0; x < DB / 2; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int i0 = 32 * x + 8 * a4 + 4 * h;
                const f32x4 c = tab.c[x][a4], s = tab.s[x][a4];
                const f32x4 g1 = val[x][a4], g2 = val[x + DB / 2][a4];
                store_out4(dst + i0, f32x4{g1[0] * c[0] + g2[0] * s[0], g1[1] * c[1] + g2[1] * s[1],
                                           g1[2] * c[2] + g2[2] * s[2], g1[3] * c[3] + g2[3] * s[3]});
                store_out4(dst + i0 + D / 2, f32x4{g2[0] * c[0] - g1[0] * s[0], g2[1] * c[1] - g1[1] * s[1],
                                                   g2[2] * c[2] - g1[2] * s[2], g2[3] * c[3] - g1[3] * s[3]});
            }
    } else {
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) store_out4(row + 32 * x + 8 * a4 + 4 * h, val[x][a4]);
    }
}

// OT: element type of o (read) and dq (written): float32 or bfloat16.
// ROPE: Q is read through rq's strides and rotated in registers into fp16 (so the
// fp16 Q copy left for the dK/dV pass is rotated too; K holds the rotated keys in
// fp16), and dQ is turned back by the transpose rotation and stored through rq's dq
// strides.
template <int D, typename OT, bool ROPE>
__global__ void __launch_bounds__(bwdq::kThreads<D>, (D == 64) ? 3 : 2)
bwd_dq_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
              const OT* __restrict__ o, const float* __restrict__ lse,
              const bf16_t* __restrict__ dout, float* __restrict__ delta, float* __restrict__ l2,
              _Float16* __restrict__ q16, _Float16* __restrict__ do16, OT* __restrict__ dq,
              int Hq, int Hkv, int N, int causal, float scale, ScoreScale sc, int nqt, int units, QRope rq) {
    using namespace bwdq;
    constexpr int DC = D / 16, DB = D / 32, LD = D + kPad<D>;
    constexpr int NKH = kKeyHalves<D>;   // key parts per tile (one wave each)
    constexpr int NT = kThreads<D>, BQ = kRows<D>, NRB = kWaves<D> / NKH;
    constexpr int KPW = BC / NKH, KB = KPW / 32;   // keys of a tile per wave, in 32-key blocks
    constexpr int CPR = D / 8, KCH = BC * CPR / NT;
    // -D as the starting dP accumulator saves a subtraction per element but
    // holds 16 more registers; at d = 128 the registers matter more
    constexpr bool kNegDAcc = (D == 64);
    // K and V tile buffers in one LDS block; after the loop (d = 64) it is the
    // exchange area of the key halves' partial dQ (NRB row blocks of 32 x D floats)
    constexpr int TILES_BYTES = 2 * 2 * BC * LD * 2, MERGE_BYTES = NRB * 32 * D * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[TILES_BYTES > MERGE_BYTES ? TILES_BYTES : MERGE_BYTES];
    _Float16 (*Ks)[BC][LD] = reinterpret_cast<_Float16 (*)[BC][LD]>(smem);
    bf16_t (*Vs)[BC][LD] = reinterpret_cast<bf16_t (*)[BC][LD]>(smem + 2 * BC * LD * 2);

    const int group = Hq / Hkv;
    const TileMap tm = map_workgroup(blockIdx.x, nqt, units, Hkv, group);
    const int hq = tm.hkv * group + tm.g;
    const size_t bh = (size_t)tm.b * Hq + hq;
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, scalar
    const int rb = (NKH == 2) ? (w >> 1) : w, khalf = (NKH == 2) ? (w & 1) : 0;   // row block, key half
    const int q0w = tm.qt * BQ + 32 * rb;
    const int qi = q0w + r;
    const int qc = min(qi, N - 1);
    const bool qok = qi < N;
    const bf16_t* kh = k + ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const float sl2 = sc.sl2;   // positive multiplier of Q' K^T (scale is dQ's factor)
    __shared__ float dsh[NKH == 2 ? BQ : 1];   // D of each row, from key half 0

    // Key half 0 computes D = rowsum(dO o O). Its O rows are the first loads, and the
    // first K/V tile's and this row's LSE follow before the Q and dO rows: every
    // prologue load is in flight before any of them is waited for.
    Row8<OT> orw[D / 16];
    if (khalf == 0) {
        const OT* orow = o + (bh * N + qc) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) orw[c].load(orow + 16 * c);
    }
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh, (uint32_t)N * D * 2);
    const VRows<D, ROPE> vrows(v, rq, tm.b, Hkv, tm.hkv, N);
    const uint32_t ld_off = (uint32_t)tid * 16;                      // byte offset of chunk 0 in a K tile
    const uint32_t vld_off = (uint32_t)(tid / CPR) * vrows.row_bytes + (uint32_t)(tid % CPR) * 16;
    const uint32_t vtile = BC * vrows.row_bytes;                       // bytes per V tile
    u32x4 kreg[KCH], vreg[KCH];
    bwd_load_kv<D, KCH, ROPE>(kreg, vreg, krs, ld_off, vrows, vld_off, 0);
    const float lse_i = lse[bh * N + qc];
    QRopeRow<D> qtab;   // ROPE: the row's table values, issued with the first loads
    if constexpr (ROPE) qtab.load(rq.cs + (size_t)qc * (D / 2), rq.sn + (size_t)qc * (D / 2), h);

    // Q (fp16) and dO (bf16) rows of this lane's query as B operands, and D_i:
    // key half 0 loads the O rows and computes D, key half 1 takes it from LDS
    // after the prologue barrier (half the O traffic at workgroup start)
    f16x8 qb[DC];
    bf16x8 db[DC];
    float Di;
    {
        const bf16_t* qrow = ROPE ? rq.q + tm.b * rq.qb + hq * rq.qh + qc * rq.qn + 8 * h
                                  : q + (bh * N + qc) * D + 8 * h;
        const bf16_t* drow = dout + (bh * N + qc) * D + 8 * h;
        u32x4 dvr[DC], qraw[DC];
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            qraw[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
            dvr[c] = *reinterpret_cast<const u32x4*>(drow + 16 * c);
        }
        if constexpr (ROPE) rope_rotate_q<D>(qraw, qtab);
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            // the rotated Q is fp16 already
            const u32x4 qh16 = ROPE ? apply_qsign(qraw[c], sc) : bf16x8_to_f16x8(apply_qsign(qraw[c], sc));
            qb[c] = qok ? __builtin_bit_cast(f16x8, qh16) : f16x8{};
            db[c] = qok ? __builtin_bit_cast(bf16x8, dvr[c]) : bf16x8{};
        }
        Di = 0.f;
        if (khalf == 0) {
            float part = 0.f;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const u32x4 dv = dvr[c];
                float ov[8];
                orw[c].get(ov);
                part = fmaf(bf16_lo(dv.x), ov[0], part);
                part = fmaf(bf16_hi(dv.x), ov[1], part);
                part = fmaf(bf16_lo(dv.y), ov[2], part);
                part = fmaf(bf16_hi(dv.y), ov[3], part);
                part = fmaf(bf16_lo(dv.z), ov[4], part);
                part = fmaf(bf16_hi(dv.z), ov[5], part);
                part = fmaf(bf16_lo(dv.w), ov[6], part);
                part = fmaf(bf16_hi(dv.w), ov[7], part);
            }
            Di = sum_halves(part);   // the two half-waves hold complementary dims of the row
            if constexpr (NKH == 2) {
                if (h == 0) dsh[32 * rb + r] = Di;
            }
            if (qok && h == 0) delta[bh * N + qi] = -Di;   // -D: the dK/dV pass starts dP from it
        }
    }
    const float Li = qok ? lse_i * kLog2e : 0.f;
    if (qok && h == 0 && khalf == 0) l2[bh * N + qi] = Li;

    f32x16 dqa[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) dqa[x] = f32x16{};

    const int last_q = min(N, (tm.qt + 1) * BQ) - 1;
    const int kend = causal ? last_q + 1 : N;
    const int ntile = (kend + BC - 1) / BC;
    const int krow_a = perm32(r);

    const int st_off = (tid / CPR) * LD + (tid % CPR) * 8;           // LDS slot of chunk 0 (elements)
    constexpr int TBUF = BC * LD;                                      // elements per LDS tile buffer

    bwd_store_kv<D, KCH, ROPE>(kreg, vreg, &Ks[0][0][0] + st_off, &Vs[0][0][0] + st_off);
    if (ntile > 1) bwd_load_kv<D, KCH, ROPE>(kreg, vreg, krs, ld_off + BC * D * 2, vrows, vld_off, vtile);
    __syncthreads();
    if constexpr (NKH == 2) {
        if (khalf == 1) Di = dsh[32 * rb + r];
    }

    for (int j = 0; j < ntile; ++j) {
        const int buf = j & 1, k0 = j * BC;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int kbr = KPW * khalf + 32 * kb;   // tile row of this wave's 32-key block
            const int kw0 = k0 + kbr;                // its first key
            if (causal && kw0 > q0w + 31) continue;
            // ---- S^T = K Q^T and dP^T - D = V dO^T - D (rows: the block's keys, permuted;
            // columns: queries): the dP product accumulates onto -D_i, so no subtraction follows
            f32x16 s = f32x16{}, dp;
            if constexpr (kNegDAcc)
                dp = f32x16{} - Di;   // -D_i in every accumulator of this lane's query column
            else
                dp = f32x16{};
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const f16x8 ak = *reinterpret_cast<const f16x8*>(&Ks[buf][kbr + krow_a][16 * c + 8 * h]);
                const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Vs[buf][kbr + krow_a][16 * c + 8 * h]);
                s = mfma_f16(ak, qb[c], s);
                dp = mfma_bf16(av, db[c], dp);
            }
            // ---- mask, only on blocks crossing the diagonal or the end of the sequence
            // (one wave-uniform branch; the common path carries no mask work):
            // accumulator e holds key kw0 + 8h + c_e, c_e = 16(e/8) + e%8, kept iff
            // key < N and (if causal) key <= qi
            if ((kw0 + 32 > N) || (causal && kw0 + 31 > q0w)) {
                const int lim = (causal ? min(qi, N - 1) : N - 1) - 8 * h - kw0;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s[e] = (16 * (e >> 3) + (e & 7) <= lim) ? s[e] : -INFINITY;
            }
            // ---- P, dS
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = fast_exp2(fmaf(s[e], sl2, -Li));
                s[e] = kNegDAcc ? p * dp[e] : p * (dp[e] - Di);   // dS = P (dP - D)
            }
            // ---- dQ^T += K^T dS^T  (A: the block's K rows read transposed; B: dS from registers)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const f16x8 dsb = to_f16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                                           s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
#pragma unroll
                for (int x = 0; x < DB; ++x) {
                    const f16x8 a = lds_tr_operand(&Ks[buf][0][0], LD, kbr + 16 * c2, 32 * x, h, r);
                    dqa[x] = mfma_f16(a, dsb, dqa[x]);
                }
            }
        }
        if (j + 1 < ntile) {
            bwd_store_kv<D, KCH, ROPE>(kreg, vreg, &Ks[0][0][0] + (buf ^ 1) * TBUF + st_off,
                                 &Vs[0][0][0] + (buf ^ 1) * TBUF + st_off);
            if (j + 2 < ntile)
                bwd_load_kv<D, KCH, ROPE>(kreg, vreg, krs, ld_off + (uint32_t)(j + 2) * (BC * D * 2), vrows,
                                          vld_off, (uint32_t)(j + 2) * vtile);
        }
        __syncthreads();
    }

    // ROPE: the storing waves issue the loads of their row's table values first, so
    // that they arrive during the copies and the key-half merge below
    DqTab<D, ROPE> dtab;
    if (ROPE && qok && khalf == 0) dtab.load(rq, qi, h);
    // key half 0 leaves fp16 copies of its Q and dO rows in the workspace for
    // the dK/dV phase, which copies them into LDS without conversion (stored
    // after the tile loop, where the writes overlap other workgroups' math)
    if (qok && khalf == 0) {
        _Float16* q16row = q16 + (bh * N + qi) * D + 8 * h;
        _Float16* d16row = do16 + (bh * N + qi) * D + 8 * h;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            *reinterpret_cast<u32x4*>(q16row + 16 * c) = __builtin_bit_cast(u32x4, qb[c]);
            *reinterpret_cast<u32x4*>(d16row + 16 * c) = bf16x8_to_f16x8(__builtin_bit_cast(u32x4, db[c]));
        }
    }
    // ---- store dQ (accumulator e of dim block x holds dim 32x + 8(e/4) + 4h + e%4 of
    // query qi); with two key halves, their partial sums are first added through LDS
    if constexpr (NKH == 1) {
        if (qok) {
            f32x4 val[DB][4];
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    val[x][a4] = f32x4{dqa[x][4 * a4 + 0] * scale, dqa[x][4 * a4 + 1] * scale,
                                       dqa[x][4 * a4 + 2] * scale, dqa[x][4 * a4 + 3] * scale};
            store_dq_row<D, OT, ROPE>(dq + (bh * N + qi) * D, val, rq, dtab, tm.b, hq, qi, h);
        }
    } else {
        // ---- sum the two key halves' partial dQ through LDS (the K buffers are free
        // after the last barrier) and store. Accumulator e of dim block x holds dim
        // 32x + 8(e/4) + 4h + e%4 of query qi.
        float* xo = reinterpret_cast<float*>(smem) + rb * (32 * D);   // [32 rows][D]
        if (khalf == 1) {
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    *reinterpret_cast<f32x4*>(xo + merge_off<D>(r, 8 * x + 2 * a4 + h)) =
                        f32x4{dqa[x][4 * a4 + 0], dqa[x][4 * a4 + 1], dqa[x][4 * a4 + 2], dqa[x][4 * a4 + 3]};
        }
        __syncthreads();
        if (khalf == 0 && qok) {
            f32x4 val[DB][4];
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + merge_off<D>(r, 8 * x + 2 * a4 + h));
                    val[x][a4] = f32x4{(dqa[x][4 * a4 + 0] + o1[0]) * scale, (dqa[x][4 * a4 + 1] + o1[1]) * scale,
                                       (dqa[x][4 * a4 + 2] + o1[2]) * scale, (dqa[x][4 * a4 + 3] + o1[3]) * scale};
                }
            store_dq_row<D, OT, ROPE>(dq + (bh * N + qi) * D, val, rq, dtab, tm.b, hq, qi, h);
        }
    }
}

// ---------------------------------------------------------------------------
// dK / dV: K/V-tile parallel.
//
// A workgroup owns the K/V tiles j and T-1-j (64 keys each) of one (batch, KV
// head) when causal -- tile j sees T-j query tiles and tile T-1-j sees j+1, so
// every workgroup does the same amount of work -- or one tile otherwise. Its
// waves are NKH = 2 key halves x NQW query sub-blocks: wave (kh, qw) handles
// keys 32kh .. 32kh+31 of the tile and rows 32qw .. 32qw+31 of each staged
// query tile (BQ = 32 NQW rows).
//
//   S  = Q K^T, dP = dO V^T  (rows: queries, permuted; columns: keys -> one key
//                             per lane, so P and dS are A operands in place)
//   dV += P^T dO, dK += dS^T Q (B operands: dO, Q tiles read transposed)
//
// Two forms (SPLIT):
// - exchange (d = 64, up to 1.5 workgroups per CU): 8 waves, 128-row query
//   tiles; each wave accumulates partial dK and dV for its keys over its own
//   rows, and at the end of a K/V tile the NQW = 4 partials of each key half are
//   summed in LDS in a fixed order (deterministic) and written out. One
//   workgroup per CU (133 KB of LDS), two waves per SIMD.
// - split by tensor (d = 128 always; d = 64 from 1.5 workgroups per CU): 4
//   waves, 64-row query tiles; wave (kh, 0) accumulates only dV and wave (kh, 1)
//   only dK, each over both 32-row blocks of the query tile: each wave keeps the
//   fp16 operand it needs of its own block (P or dS) and passes the other one to
//   its partner through 8 KB of LDS, one extra barrier per item, and there is no
//   end-of-tile exchange. At d = 128 (holding K, V, dK and dV in one wave would
//   take ~490 registers) that is 256 registers and 73 KB of LDS, two workgroups
//   per CU; at d = 64, 168 registers and 41 KB, three workgroups per CU. A staged
//   row feeds as many products per byte as in the exchange form, but a workgroup
//   has half the waves, so it needs three times the workgroups to fill the CUs:
//   exactly one per CU (the GQA shapes at N = 1024 and 4096) keeps the exchange.
namespace bwdkv {
constexpr int BC = 64;
template <int D, bool SPLIT> struct Cfg { static constexpr int NQW = 2; };   // 4 waves, 64-row query tiles
template <> struct Cfg<64, false> { static constexpr int NQW = 4; };           // 8 waves, 128-row query tiles
// d = 64 takes the split form from this many workgroups on (1.5 per CU)
constexpr long long kSplitMinWorkgroups64 = 384;

}  // namespace bwdkv

// OT: element type of dk and dv (float32, or bfloat16 rounded to nearest even).
// ROPE: V is read in place through rv's strides, K holds the rotated keys
// (contiguous, fp16), and dK is turned back by the transpose rotation at the store;
// dK and dV go through rv's strides.
template <int D, typename OT, bool ROPE, bool SPLIT>
__global__ void __launch_bounds__((64 * 2 * bwdkv::Cfg<D, SPLIT>::NQW), (D == 128) ? 2 : (SPLIT ? 3 : 1))
bwd_dkdv_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                const _Float16* __restrict__ q16, const _Float16* __restrict__ do16,
                const float* __restrict__ l2, const float* __restrict__ delta,
                OT* __restrict__ dk, OT* __restrict__ dv,
                int Hq, int Hkv, int N, int causal, ScoreScale sc, int ntiles, int wg_per_unit, KVRope rv) {
    using namespace bwdkv;
    static_assert(SPLIT || D == 64, "d = 128 runs split by tensor");
    constexpr int NQW = Cfg<D, SPLIT>::NQW;
    constexpr int NW = 2 * NQW;               // waves
    constexpr int BQ = 32 * NQW;              // query rows per staged tile
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int TILE_BYTES = BQ * D * 2;    // one staged Q or dO tile
    constexpr int IPW = TILE_BYTES / 1024 / NW;   // 1 KB copy instructions per wave per tile
    constexpr int NJ = BQ * 4 / 256;          // 256-byte copy instructions per row-statistic tile
    static_assert(IPW * NW * 1024 == TILE_BYTES && NJ * 256 == BQ * 4 && 2 * NJ <= NW, "staging split");
    // double buffer as distinct LDS objects, so the compiler can tell the copy
    // into one buffer from the reads of the other and does not make the reads
    // wait for the copy (the item loop is unrolled by two to name them statically)
    __shared__ __attribute__((aligned(16))) _Float16 Qs0[BQ * D], Qs1[BQ * D];
    __shared__ __attribute__((aligned(16))) _Float16 dOs0[BQ * D], dOs1[BQ * D];
    __shared__ __attribute__((aligned(16))) float Ls0[BQ], Ls1[BQ], Ds0[BQ], Ds1[BQ];
    // exchange form: partial-sum exchange area. Split by tensor: wave (kh, 0)
    // accumulates dV, wave (kh, 1) dK, each over the whole query tile; they trade
    // the fp16 dS (from qw 0) and P (from qw 1) operands of their blocks here
    constexpr bool kSplit = SPLIT;
    __shared__ __attribute__((aligned(16))) float red[kSplit ? 4 : (NQW / 2) * 2 * BC * D];
    __shared__ __attribute__((aligned(16))) _Float16 xch[kSplit ? 2 * 2 * 2 * 64 * 8 : 8];   // [kh][qw][c2][lane][8]

    const int group = Hq / Hkv;
    // all workgroups of one (batch, KV head) unit on one XCD (w mod 8), so the
    // unit's Q/dO stream is fetched into that XCD's L2 once
    int unit, slot;
    {
        const int w8 = blockIdx.x;
        const int units = gridDim.x / wg_per_unit;
        if ((units & 7) == 0) {
            const int i = w8 >> 3;
            unit = (i / wg_per_unit) * 8 + (w8 & 7);
            slot = i % wg_per_unit;
        } else {
            unit = w8 / wg_per_unit;
            slot = w8 % wg_per_unit;
        }
    }
    const int b = unit / Hkv, hkv = unit % Hkv;
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, scalar
    const int kh_ = w & 1, qw = w >> 1;       // key half, query sub-block
    const size_t kvoff = ((size_t)b * Hkv + hkv) * N * D;
    const float sl2 = sc.sl2;         // positive multiplier of Q' K^T (Q' is the stored copy)
    const float scale = sc.kscale;    // dK = s' dS^T Q'
    const int nqt = (N + BQ - 1) / BQ;

    // K/V tiles of this workgroup: causal -> {slot, ntiles-1-slot} (one if they coincide)
    const int tile_a = slot;
    const int tile_b = (causal && ntiles - 1 - slot != slot) ? ntiles - 1 - slot : -1;

    // items: for each of the workgroup's K/V tiles, every head g of the group
    // and every query tile qt at or below the diagonal (qt from first_qt(tile)).
    // Two cursors walk the sequence: `cur` (computed now) and `ld` (being
    // staged, one item ahead); advancing is a few scalar compares, no division.
    struct Cursor {
        int t, g, qt;   // t: 0 -> tile_a, 1 -> tile_b, 2 -> done
    };
    const int fa = causal ? (tile_a * BC) / BQ : 0;
    const int fb = (tile_b >= 0 && causal) ? (tile_b * BC) / BQ : 0;
    const int nitems = group * (nqt - fa) + ((tile_b >= 0) ? group * (nqt - fb) : 0);
    auto advance = [&](Cursor& c) {
        if (++c.qt < nqt) return;
        if (++c.g < group) {
            c.qt = c.t ? fb : fa;
            return;
        }
        c.g = 0;
        c.t += 1;
        c.qt = fb;
        if (c.t == 1 && tile_b < 0) c.t = 2;
    };
    auto tile_of = [&](const Cursor& c) { return c.t == 0 ? tile_a : tile_b; };

    // Staging is a direct global -> LDS copy (no registers, no conversion): the
    // workspace already holds Q and dO in fp16 and lse in log2 units. Copy
    // instruction i of a tile fills LDS bytes [1024 i, 1024 i + 1024), lane l
    // the 16 bytes at 1024 i + 16 l, i.e. row R = (1024 i + 16 l) / (2D) and
    // chunk position p; it reads source chunk p ^ tile_swz(R) of that row. Rows past
    // the end of the sequence lie outside the buffer resource and read as zero.
    uint32_t src_off[IPW];
#pragma unroll
    for (int u = 0; u < IPW; ++u) src_off[u] = tile_copy_src<D>(w * IPW + u, lane);
    auto stage = [&](const Cursor& c, _Float16* Qd, _Float16* dOd, float* Ld, float* Dd) {
        const size_t bh = (size_t)b * Hq + hkv * group + c.g;
        const int q0 = c.qt * BQ;
        const uint32_t rows = (uint32_t)(N - q0);
        const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q16 + (bh * N + q0) * D, rows * (D * 2));
        const __amdgpu_buffer_rsrc_t drs = make_rsrc(do16 + (bh * N + q0) * D, rows * (D * 2));
#pragma unroll
        for (int u = 0; u < IPW; ++u) {
            const int i = w * IPW + u;
            lds_copy16(qrs, Qd + i * 512, src_off[u]);
            lds_copy16(drs, dOd + i * 512, src_off[u]);
        }
        if (w < 2 * NJ) {   // row statistics: waves 0 .. NJ-1 copy L, NJ .. 2NJ-1 copy D
            const int j = (w < NJ) ? w : w - NJ;
            const float* src = (w < NJ) ? l2 : delta;
            float* dst = ((w < NJ) ? Ld : Dd) + j * 64;
            const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + bh * N + q0, rows * 4);
            lds_copy4(rs, dst, (uint32_t)(j * 64 + lane) * 4);
        }
    };

    f16x8 kb[DC], vb[DC];
    f32x16 dka[DB], dva[kSplit ? 1 : DB];   // split: dka is this wave's one tensor
    int cur_tile = -1;
    Cursor cur = {0, 0, fa}, ld = cur;

    if (nitems > 0) {
        stage(ld, Qs0, dOs0, Ls0, Ds0);
        advance(ld);
    }
    wait_vmem_all();   // the copies land before the barrier that publishes them
    __syncthreads();

    // one item; BUF (compile time) names the buffer it reads, the other one
    // receives the next item
    auto item = [&](const int it, auto bufc) {
        constexpr int BUF = decltype(bufc)::value;
        const _Float16* Qt = BUF ? Qs1 : Qs0;
        const _Float16* dOt = BUF ? dOs1 : dOs0;
        const float* Lt = BUF ? Ls1 : Ls0;
        const float* Dt = BUF ? Ds1 : Ds0;
        const int tile = tile_of(cur), qt = cur.qt;
        const int kw0 = tile * BC + 32 * kh_;   // first key of this wave
        const int kw = kw0 + r;                 // this lane's key
        if (tile != cur_tile) {
            // new K/V tile: this lane's K, V rows as fp16 B operands; clear partials
            cur_tile = tile;
            const bf16_t* krow = k + kvoff + (size_t)min(kw, N - 1) * D + 8 * h;
            const bf16_t* vrow = ROPE ? rv.v + b * rv.vb + hkv * rv.vh + (long long)min(kw, N - 1) * rv.vn + 8 * h
                                      : v + kvoff + (size_t)min(kw, N - 1) * D + 8 * h;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const u32x4 kw8 = *reinterpret_cast<const u32x4*>(krow + 16 * c);
                kb[c] = __builtin_bit_cast(f16x8, ROPE ? kw8 : bf16x8_to_f16x8(kw8));   // rotated keys: fp16
                vb[c] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(vrow + 16 * c)));
            }
#pragma unroll
            for (int x = 0; x < DB; ++x) dka[x] = f32x16{};
            if constexpr (!kSplit) {
#pragma unroll
                for (int x = 0; x < DB; ++x) dva[x] = f32x16{};
            }
        }
        // stage the next item into the other buffer (free since the last barrier)
        if (it + 1 < nitems) {
            if (BUF)
                stage(ld, Qs0, dOs0, Ls0, Ds0);
            else
                stage(ld, Qs1, dOs1, Ls1, Ds1);
            advance(ld);
        }
        const int q0 = qt * BQ + 32 * qw;        // first query row of this wave's block
        const bool live = !causal || q0 + 31 >= kw0;
        f16x8 own[kSplit ? 2 : 1];
        if (live) {
            // ---- S = Q K^T, dP - D = dO V^T - D (accumulator e: query q0 + 16(e/8) + 8h + e%8,
            // key kw): the row statistic arrives as -D, and the dP product accumulates onto it
            f32x16 s = f32x16{}, dp;
            {
                const int qq = 32 * qw + 8 * h;
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(Dt + qq);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(Dt + qq + 4);
                const f32x4 d2 = *reinterpret_cast<const f32x4*>(Dt + qq + 16);
                const f32x4 d3 = *reinterpret_cast<const f32x4*>(Dt + qq + 20);
                dp = f32x16{d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3],
                            d2[0], d2[1], d2[2], d2[3], d3[0], d3[1], d3[2], d3[3]};
            }
            const int arow = 32 * qw + perm32(r);
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const int off = tile_off<D>(arow, 16 * c + 8 * h);
                const f16x8 aq = *reinterpret_cast<const f16x8*>(Qt + off);
                const f16x8 ad = *reinterpret_cast<const f16x8*>(dOt + off);
                s = mfma_f16(aq, kb[c], s);
                dp = mfma_f16(ad, vb[c], dp);
            }
            // ---- mask, only on items crossing the diagonal or an end of the sequence
            // (one wave-uniform branch; the common path carries no mask work):
            // accumulator e holds query q0 + 8h + c_e, c_e = 16(e/8) + e%8, kept iff
            // query < N, kw < N and (if causal) kw <= query
            if ((q0 + 32 > N) || (kw0 + 32 > N) || (causal && q0 < kw0 + 31)) {
                const int lo = (causal ? kw : 0) - q0 - 8 * h;
                if constexpr (kSplit) {
                    // split by tensor: one two-sided test (the forms below cost the d = 128
                    // kernel registers it does not have: it spilled)
                    const int hi = (kw < N) ? N - q0 - 8 * h : lo;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ce = 16 * (e >> 3) + (e & 7);
                        s[e] = (ce >= lo && ce < hi) ? s[e] : -INFINITY;
                    }
                } else if (q0 + 32 <= N && kw0 + 32 <= N) {
                    // a diagonal item away from the end: only the causal bound c_e >= lo
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ce = 16 * (e >> 3) + (e & 7);
                        s[e] = (ce >= lo) ? s[e] : -INFINITY;
                    }
                } else {
                    // both bounds as one unsigned compare: lo <= c_e < hi iff
                    // c_e - lo < hi - lo (an empty range when hi <= lo)
                    const int hi = (kw < N) ? N - q0 - 8 * h : lo;
                    const unsigned span = (unsigned)(max(hi, lo) - lo);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ce = 16 * (e >> 3) + (e & 7);
                        s[e] = ((unsigned)(ce - lo) < span) ? s[e] : -INFINITY;
                    }
                }
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int qq = 32 * qw + 16 * c2 + 8 * h;   // tile row of accumulator 8c2
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(Lt + qq);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(Lt + qq + 4);
                const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int e = 8 * c2 + t;
                    const float p = fast_exp2(fmaf(s[e], sl2, -lv[t]));
                    s[e] = p;
                    dp[e] = p * dp[e];   // dS = P (dP - D)
                }
            }
            if constexpr (kSplit) {
                // keep this wave's own operand (qw 0: P, qw 1: dS), hand the other one to
                // the partner wave as lane-major 16-byte chunks (conflict-free)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const f16x8 pa = to_f16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                                              s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
                    const f16x8 da = to_f16x8(dp[8 * c2 + 0], dp[8 * c2 + 1], dp[8 * c2 + 2], dp[8 * c2 + 3],
                                              dp[8 * c2 + 4], dp[8 * c2 + 5], dp[8 * c2 + 6], dp[8 * c2 + 7]);
                    own[c2] = qw ? da : pa;
                    *reinterpret_cast<f16x8*>(xch + (((kh_ * 2 + qw) * 2 + c2) * 64 + lane) * 8) = qw ? pa : da;
                }
            } else {
                // ---- dV += P^T dO, dK += dS^T Q (B: dO, Q tiles read transposed, rows = queries)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const f16x8 pa = to_f16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                                              s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
                    const f16x8 da = to_f16x8(dp[8 * c2 + 0], dp[8 * c2 + 1], dp[8 * c2 + 2], dp[8 * c2 + 3],
                                              dp[8 * c2 + 4], dp[8 * c2 + 5], dp[8 * c2 + 6], dp[8 * c2 + 7]);
#pragma unroll
                    for (int x = 0; x < DB; ++x) {
                        const f16x8 bo = tile_tr_operand<D>(dOt, 32 * qw + 16 * c2, 32 * x, h, r);
                        const f16x8 bq = tile_tr_operand<D>(Qt, 32 * qw + 16 * c2, 32 * x, h, r);
                        dva[x] = mfma_f16(pa, bo, dva[x]);
                        dka[x] = mfma_f16(da, bq, dka[x]);
                    }
                }
            }
        }
        if constexpr (kSplit) {
            // ---- qw 0: dV += P^T dO, qw 1: dK += dS^T Q over both 32-row blocks of the
            // query tile, own block first (B: dO or Q tile read transposed, rows = queries)
            __syncthreads();
            const _Float16* Bt = qw ? Qt : dOt;
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                const int qb = pass ? 1 - qw : qw;
                if (pass && !(!causal || qt * BQ + 32 * qb + 31 >= kw0)) break;
                if (!pass && !live) continue;
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const f16x8 a = pass ? *reinterpret_cast<const f16x8*>(xch + (((kh_ * 2 + qb) * 2 + c2) * 64 + lane) * 8)
                                         : own[c2];
#pragma unroll
                    for (int x = 0; x < DB; ++x)
                        dka[x] = mfma_f16(a, tile_tr_operand<D>(Bt, 32 * qb + 16 * c2, 32 * x, h, r), dka[x]);
                }
            }
        }
        advance(cur);
        if constexpr (kSplit) {
            // ---- end of a K/V tile: each wave holds its tensor's final values for its 32 keys
            // (accumulator e of dim block x: key 32kh + 8(e/4) + 4h + e%4, dim 32x + r)
            if (it + 1 == nitems || tile_of(cur) != tile) {
                const float f = qw ? scale : 1.0f;
                if constexpr (ROPE) {
                    // dims 32x + r and 32x + r + D/2 (blocks x and x + DB/2 of this lane) form a
                    // rotation pair: dK is turned back with the key row's table entries
                    OT* const dst = static_cast<OT*>(qw ? rv.dk : rv.dv);
                    const long long sb = qw ? rv.kb : rv.db, sh = qw ? rv.kh : rv.dh, srow = qw ? rv.kn : rv.dn;
                    OT* const base = dst + b * sb + hkv * sh;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = kw0 + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key >= N) continue;
                        OT* const row = base + (long long)key * srow;
#pragma unroll
                        for (int x = 0; x < DB / 2; ++x) {
                            const int f0 = 32 * x + r;
                            const float g1 = dka[x][e] * f, g2 = dka[x + DB / 2][e] * f;
                            if (qw) {
                                const float c = rv.cs[(size_t)key * (D / 2) + f0], si = rv.sn[(size_t)key * (D / 2) + f0];
                                store_out1(row + f0, g1 * c + g2 * si);
                                store_out1(row + f0 + D / 2, g2 * c - g1 * si);
                            } else {
                                store_out1(row + f0, g1);
                                store_out1(row + f0 + D / 2, g2);
                            }
                        }
                    }
                } else {
                    OT* const dst = qw ? dk : dv;
#pragma unroll
                    for (int x = 0; x < DB; ++x)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = kw0 + 8 * (e >> 2) + 4 * h + (e & 3);
                            if (key < N) store_out1(dst + kvoff + (size_t)key * D + 32 * x + r, dka[x][e] * f);
                        }
                }
            }
        }
        // ---- end of a K/V tile: combine the NQW query sub-blocks' partial dK, dV
        else if (it + 1 == nitems || tile_of(cur) != tile) {
            // Wave (kh, qw) owns accumulators e in [E qw, E qw + E) of both tensors (accumulator
            // e of dim block x: key 32kh + 8(e/4) + 4h + e%4, dim 32x + r). It hands every
            // other owner its part through LDS, one (source, owner) block each, then adds the
            // NQW - 1 blocks addressed to it in source order (fixed order: deterministic) and
            // stores its keys. One exchange round; every wave shares the adds and the stores.
            // A block is lane-major 16-byte chunks (16 lanes of a cycle hit 256 contiguous
            // bytes: no bank conflicts). The blocks fill `red`, then this item's Q and
            // dO buffers, which every wave has finished reading at the barrier below.
            constexpr int E = 16 / NQW;                  // accumulators owned per wave
            constexpr int BS = 2 * DB * E * 64;          // floats per block (16-byte chunks, 64 lanes)
            constexpr int RED_FLOATS = (NQW / 2) * 2 * BC * D;
            constexpr int QF = BQ * D / 2;               // floats in one staged Q (or dO) buffer
            static_assert(2 * NQW * (NQW - 1) * BS <= RED_FLOATS + 2 * QF, "exchange blocks must fit");
            float* const redf = red;
            float* const qf = reinterpret_cast<float*>(BUF ? Qs1 : Qs0);
            float* const df = reinterpret_cast<float*>(BUF ? dOs1 : dOs0);
            auto block = [&](int src, int owner) -> float* {
                const int b = kh_ * NQW * (NQW - 1) + src * (NQW - 1) + (owner < src ? owner : owner - 1);
                const int off = b * BS;
                if (off < RED_FLOATS) return redf + off;
                return (off - RED_FLOATS < QF) ? qf + (off - RED_FLOATS) : df + (off - RED_FLOATS - QF);
            };
            __syncthreads();
            // chunk (t, x, j) of a block: tensor t (0 dK, 1 dV), dim block x, owner
            // accumulators 4j .. 4j+3; chunk index (t DB + x) E/4 + j
            constexpr int EQ = E / 4;
#pragma unroll
            for (int o = 0; o < NQW; ++o) {
                if (o == qw) continue;
                float* const dst = block(qw, o);
#pragma unroll
                for (int x = 0; x < DB; ++x)
#pragma unroll
                    for (int j = 0; j < EQ; ++j) {
                        const int e = E * o + 4 * j;
                        *reinterpret_cast<f32x4*>(dst + (((0 * DB + x) * EQ + j) * 64 + lane) * 4) =
                            f32x4{dka[x][e], dka[x][e + 1], dka[x][e + 2], dka[x][e + 3]};
                        *reinterpret_cast<f32x4*>(dst + (((1 * DB + x) * EQ + j) * 64 + lane) * 4) =
                            f32x4{dva[x][e], dva[x][e + 1], dva[x][e + 2], dva[x][e + 3]};
                    }
            }
            // own part (wave-uniform select: register indices stay compile-time)
            float sk[DB][E], sv[DB][E];
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    sk[x][i] = dka[x][i];
                    sv[x][i] = dva[x][i];
#pragma unroll
                    for (int o = 1; o < NQW; ++o)
                        if (qw == o) {
                            sk[x][i] = dka[x][E * o + i];
                            sv[x][i] = dva[x][E * o + i];
                        }
                }
            __syncthreads();
#pragma unroll
            for (int src = 0; src < NQW; ++src) {
                if (src == qw) continue;
                const float* const sb = block(src, qw);
#pragma unroll
                for (int x = 0; x < DB; ++x)
#pragma unroll
                    for (int j = 0; j < EQ; ++j) {
                        const f32x4 ak = *reinterpret_cast<const f32x4*>(sb + (((0 * DB + x) * EQ + j) * 64 + lane) * 4);
                        const f32x4 av = *reinterpret_cast<const f32x4*>(sb + (((1 * DB + x) * EQ + j) * 64 + lane) * 4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            sk[x][4 * j + i] += ak[i];
                            sv[x][4 * j + i] += av[i];
                        }
                    }
            }
            if constexpr (ROPE) {
                // dims 32x + r and 32x + r + D/2 (blocks x and x + DB/2 of this lane) form a
                // rotation pair: dK is turned back with the key row's table entries
                OT* const dkb = static_cast<OT*>(rv.dk) + b * rv.kb + hkv * rv.kh;
                OT* const dvb = static_cast<OT*>(rv.dv) + b * rv.db + hkv * rv.dh;
#pragma unroll
                for (int i = 0; i < E; ++i) {
                    const int e = E * qw + i;
                    const int key = tile * BC + 32 * kh_ + 8 * (e >> 2) + 4 * h + (e & 3);
                    if (key >= N) continue;
                    OT* const krow_o = dkb + (long long)key * rv.kn;
                    OT* const vrow_o = dvb + (long long)key * rv.dn;
#pragma unroll
                    for (int x = 0; x < DB / 2; ++x) {
                        const int f0 = 32 * x + r;
                        const float c = rv.cs[(size_t)key * (D / 2) + f0], si = rv.sn[(size_t)key * (D / 2) + f0];
                        const float g1 = sk[x][i] * scale, g2 = sk[x + DB / 2][i] * scale;
                        store_out1(krow_o + f0, g1 * c + g2 * si);
                        store_out1(krow_o + f0 + D / 2, g2 * c - g1 * si);
                        store_out1(vrow_o + f0, sv[x][i]);
                        store_out1(vrow_o + f0 + D / 2, sv[x + DB / 2][i]);
                    }
                }
            } else {
#pragma unroll
                for (int x = 0; x < DB; ++x)
#pragma unroll
                    for (int i = 0; i < E; ++i) {
                        const int e = E * qw + i;
                        const int key = tile * BC + 32 * kh_ + 8 * (e >> 2) + 4 * h + (e & 3);
                        if (key < N) {
                            const size_t off = kvoff + (size_t)key * D + 32 * x + r;
                            store_out1(dk + off, sk[x][i] * scale);
                            store_out1(dv + off, sv[x][i]);
                        }
                    }
            }
        }
        wait_vmem_all();   // the copies land before the barrier that publishes them
        __syncthreads();
    };
    for (int it = 0; it < nitems; it += 2) {
        item(it, std::integral_constant<int, 0>{});
        if (it + 1 < nitems) item(it + 1, std::integral_constant<int, 1>{});
    }
}

template <int D, typename OT, bool ROPE>
static hipError_t launch_bwd_dq_d(const AttnArgs& a, hipStream_t st) {
    const int nqt = (a.N + bwdq::kRows<D> - 1) / bwdq::kRows<D>;
    const int units = a.B * a.Hkv;
    const BwdWorkspace ws = bwd_workspace_layout(a.workspace, a.dtype, a.B, a.Hq, a.N, a.d);
    const QRope rq = ROPE ? *a.rope : QRope{};
    hipLaunchKernelGGL((bwd_dq_kernel<D, OT, ROPE>), dim3((unsigned)(nqt * a.B * a.Hq)), dim3(bwdq::kThreads<D>), 0, st,
                       (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const OT*)a.o,
                       (const float*)a.lse, (const bf16_t*)a.dout, ws.delta, ws.l2, ws.q16, ws.do16, (OT*)a.dq,
                       a.Hq, a.Hkv, a.N, a.causal, a.scale, score_scale(a.scale), nqt, units, rq);
    return hipGetLastError();
}

template <int D, typename OT, bool ROPE, bool SPLIT>
static hipError_t launch_bwd_dkdv_form(const AttnArgs& a, hipStream_t st, int ntiles, int per_unit) {
    const int threads = 64 * 2 * bwdkv::Cfg<D, SPLIT>::NQW;
    const BwdWorkspace ws = bwd_workspace_layout(a.workspace, a.dtype, a.B, a.Hq, a.N, a.d);
    const KVRope rv = ROPE ? *a.kvrope : KVRope{};
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, OT, ROPE, SPLIT>), dim3((unsigned)(per_unit * a.B * a.Hkv)), dim3(threads),
                       0, st, (const bf16_t*)a.k, (const bf16_t*)a.v, ws.q16, ws.do16, ws.l2, ws.delta, (OT*)a.dk,
                       (OT*)a.dv, a.Hq, a.Hkv, a.N, a.causal, score_scale(a.scale), ntiles, per_unit, rv);
    return hipGetLastError();
}

template <int D, typename OT, bool ROPE>
static hipError_t launch_bwd_dkdv_d(const AttnArgs& a, hipStream_t st) {
    const int ntiles = (a.N + bwdkv::BC - 1) / bwdkv::BC;
    const int per_unit = a.causal ? (ntiles + 1) / 2 : ntiles;
    if constexpr (D == 128) {
        return launch_bwd_dkdv_form<D, OT, ROPE, true>(a, st, ntiles, per_unit);
    } else {
        const long long wgs = (long long)per_unit * a.B * a.Hkv;
        return (wgs >= bwdkv::kSplitMinWorkgroups64) ? launch_bwd_dkdv_form<D, OT, ROPE, true>(a, st, ntiles, per_unit)
                                                     : launch_bwd_dkdv_form<D, OT, ROPE, false>(a, st, ntiles, per_unit);
    }
}

template <bool ROPE>
static hipError_t launch_bwd_dq_rope_or_not(const AttnArgs& a, hipStream_t st) {
    if (a.out_dtype == ATTN_BF16)
        return (a.d == 64) ? launch_bwd_dq_d<64, bf16_t, ROPE>(a, st) : launch_bwd_dq_d<128, bf16_t, ROPE>(a, st);
    return (a.d == 64) ? launch_bwd_dq_d<64, float, ROPE>(a, st) : launch_bwd_dq_d<128, float, ROPE>(a, st);
}

hipError_t launch_bwd_mfma_dq(const AttnArgs& a, hipStream_t st) {
    return a.rope ? launch_bwd_dq_rope_or_not<true>(a, st) : launch_bwd_dq_rope_or_not<false>(a, st);
}
template <bool ROPE>
static hipError_t launch_bwd_dkdv_rope_or_not(const AttnArgs& a, hipStream_t st) {
    if (a.out_dtype == ATTN_BF16)
        return (a.d == 64) ? launch_bwd_dkdv_d<64, bf16_t, ROPE>(a, st) : launch_bwd_dkdv_d<128, bf16_t, ROPE>(a, st);
    return (a.d == 64) ? launch_bwd_dkdv_d<64, float, ROPE>(a, st) : launch_bwd_dkdv_d<128, float, ROPE>(a, st);
}

hipError_t launch_bwd_mfma_dkdv(const AttnArgs& a, hipStream_t st) {
    return a.kvrope ? launch_bwd_dkdv_rope_or_not<true>(a, st) : launch_bwd_dkdv_rope_or_not<false>(a, st);
}

}  // namespace tca
