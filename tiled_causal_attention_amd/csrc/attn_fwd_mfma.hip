// attn_fwd_mfma.hip -- causal GQA attention forward on gfx950 matrix cores.
//
// The loop is the one of the NanoEuler "Tiled FlashAttention" section (one
// workgroup per query tile; for each K/V tile: stage it on chip, Q*K^T, online
// softmax, accumulate the output), re-shaped for CDNA4:
//
//  * d = 64: a workgroup covers 64 query rows with 4 waves, row blocks of 32
//    rows x 2 key halves. Wave (rb, kh) takes keys 32kh .. 32kh+31 of every K/V
//    tile for its 32 rows and runs its own online softmax over them; the two key
//    halves of a row block are merged once, through LDS, at the end. Splitting
//    the keys halves the serial work each wave does per tile, which is what
//    bounds short-sequence shapes (the last query tile's walk over all K/V
//    tiles), and doubles the waves available to hide latency.
//    d = 128: a workgroup covers 128 rows with 4 waves, each taking all 64 keys
//    of a tile for its 32 rows (no merge). Its ~190 registers allow two such
//    workgroups per CU, so the two waves of a SIMD belong to different
//    workgroups and do not wait at the same barriers (an 8-wave workgroup with
//    key halves needs 155 registers, which fits only one per CU).
//  * Each wave keeps its Q rows in registers as the B operand of
//    S^T = K * Q^T, so the score accumulator holds one query per lane
//    (lane = 32h + r -> query r): the row max and row sum are in-lane
//    reductions plus one half-wave exchange.
//  * K/V tiles (BC = 64 keys) are double-buffered in LDS and prefetched one
//    tile ahead into registers: the global loads for tile j+2 are issued while
//    tile j is computed and land in LDS after it, so their latency is hidden
//    behind a whole tile of math. Loads are branch-free (rows past the end are
//    clamped to the last row and masked out of the softmax).
//  * K stays bf16 (A operand of S^T, read at row perm32(m) so accumulator e
//    holds key 16(e/8) + 8h + e%8). V is converted to fp16 when it is written
//    to LDS and stays row-major; the transposing LDS load (ds_read_b64_tr_b16)
//    reads it as the A operand of O^T += V^T * P^T, whose B operand is the
//    probability tile taken straight from the score accumulator.
//  * P is rounded to fp16 (11-bit significand) rather than bf16: bf16 rounding
//    of P shifts O, hence the backward's D = rowsum(dO o O), enough to break
//    the bf16 accuracy bound on the peaked-softmax workloads. The row sum adds
//    the rounded fp16 values (v_dot2), so O is normalised by exactly the
//    weights it accumulated.
//  * Lazy rescaling: the running max m only moves when a tile's max exceeds it
//    by more than 8 (log2 units); otherwise probabilities are taken against the
//    stale max and stay <= 2^8, which fp16 and the fp32 accumulators hold
//    exactly as well. Most tiles therefore skip the O rescale entirely.
//  * Causal tile skipping: a query tile visits only the K/V tiles that start at
//    or below its last row; a wave whose rows all precede a tile skips its
//    math; the mask is applied only on tiles crossing the diagonal or the end.
//  * Grid order: longest (last) query tiles first; when the number of
//    (batch, KV head) units is a multiple of 8, the workgroups of one unit are
//    placed on one XCD (workgroups are dealt to the 8 XCDs round-robin), so
//    its K/V tiles stay in that XCD's L2.
#include "tca_internal.h"

namespace tca {

namespace fwd {
// Waves per workgroup: 4, as kWaves/kKeyHalves row blocks of 32 query rows x
// kKeyHalves key parts. d = 64: 2 key halves (64 rows): on the causal N = 1024
// shape 64-row workgroups (twice as many) leave a shorter tail than 128-row
// ones. d = 128: one wave per row block takes the whole tile (128 rows), so a
// K/V tile still serves 128 rows and two workgroups share a CU: 7-8% faster
// than 8-wave workgroups with key halves, which fit only one per CU.
template <int D> constexpr int kWaves = 4;
template <int D> constexpr int kKeyHalves = (D == 128) ? 1 : 2;   // waves sharing a row block
template <int D> constexpr int kThreads = 64 * kWaves<D>;
template <int D> constexpr int kRows = 32 * kWaves<D> / kKeyHalves<D>;   // query rows per workgroup
constexpr int BC = 64;           // keys per K/V tile (32 per key half)
// Row padding of the K/V tiles (16-bit elements). With 64 banks of 4 bytes, a
// stride of d + 8 leaves the 16-byte operand reads conflict-free and the
// transposing reads 2-way at d = 64 but 4-way at d = 128; d + 24 brings d = 128
// to 2-way as well (and two workgroups' tiles still fit one CU's LDS).
template <int D> constexpr int kPad = (D == 128) ? 24 : 8;
constexpr float kTau = 8.f;      // lazy-rescale threshold, log2 units
}  // namespace fwd

// Global -> registers: the K and V chunks of one tile. K through a buffer
// resource over the head's N contiguous rows, koff this thread's byte offset of
// its first chunk (row tid / (D/8), chunk tid % (D/8) of the tile); V through vr,
// at this thread's in-tile offset vlane plus the tile's byte offset vtile_off.
// Thread tid owns chunks tid + T u, T threads (a wave reads whole rows); rows
// past the end of the sequence read as zero.
template <int D, int KCH, bool ROPE>
__device__ __forceinline__ void load_kv_tile(u32x4 (&kreg)[KCH], u32x4 (&vreg)[KCH], __amdgpu_buffer_rsrc_t kr,
                                             uint32_t koff, const VRows<D, ROPE>& vr, uint32_t vlane,
                                             uint32_t vtile_off) {
    constexpr int ROWS_PER_U = fwd::kThreads<D> / (D / 8);
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        kreg[u] = buf_load16(kr, koff + u * fwd::kThreads<D> * 16);
        vreg[u] = vr.load16(vlane, vtile_off + u * ROWS_PER_U * vr.row_bytes);
    }
}

// Registers -> LDS: K as bf16 rows, V converted to fp16 rows. kdst/vdst point
// at this thread's chunk 0 (row tid / (D/8), column 8 (tid % (D/8))); chunk u
// sits T u / (D/8) rows further down (T threads).
template <int D, int KCH>
__device__ __forceinline__ void store_kv_tile(const u32x4 (&kreg)[KCH], const u32x4 (&vreg)[KCH], bf16_t* kdst,
                                              _Float16* vdst) {
    constexpr int ROWS_PER_U = fwd::kThreads<D> / (D / 8);
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        *reinterpret_cast<u32x4*>(kdst + u * ROWS_PER_U * (D + fwd::kPad<D>)) = kreg[u];
        *reinterpret_cast<u32x4*>(vdst + u * ROWS_PER_U * (D + fwd::kPad<D>)) = bf16x8_to_f16x8(vreg[u]);
    }
}

// OT: element type of o (float32, or bfloat16 rounded to nearest even at the store).
// ROPE: Q is read through rq's strides and rotated in registers (rotary embedding),
// V is read in place through rq's V strides, and K holds the rotated keys, contiguous,
// in fp16: the rotated Q and K meet in an fp16 product.
template <int D, typename OT, bool ROPE>
__global__ void __launch_bounds__(fwd::kThreads<D>, (D == 64) ? 4 : 2)
fwd_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                const bf16_t* __restrict__ v, OT* __restrict__ o, float* __restrict__ lse,
                int Hq, int Hkv, int N, int causal, ScoreScale sc, int nqt, int units, QRope rq) {
    using namespace fwd;
    constexpr int DC = D / 16;          // 16-deep chunks of the head dimension
    constexpr int DB = D / 32;          // 32-wide blocks of the head dimension
    constexpr int LD = D + kPad<D>;     // LDS row stride (elements)
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int NT = kThreads<D>;     // threads
    constexpr int BR = kRows<D>;        // query rows per workgroup
    constexpr int NKH = kKeyHalves<D>;  // key parts per tile (one wave each)
    constexpr int NRB = kWaves<D> / NKH;  // row blocks
    constexpr int KPW = BC / NKH;       // keys of a tile per wave
    constexpr int KB = KPW / 32;        // 32-key blocks per wave
    constexpr int KCH = BC * CPR / NT;  // chunks per thread per tensor per tile
    // K and V tile buffers, carved from one LDS block: after the loop (d = 64) the
    // whole block is the merge area of the key halves (NRB row blocks of 32 x D floats)
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * BC * LD * 2];
    bf16_t (*Ks)[BC][LD] = reinterpret_cast<bf16_t (*)[BC][LD]>(smem);
    _Float16 (*Vs)[BC][LD] = reinterpret_cast<_Float16 (*)[BC][LD]>(smem + 2 * BC * LD * 2);
    static_assert(NRB * 32 * D * 4 + NRB * 64 * 4 <= (int)sizeof(smem), "merge area exceeds the tile buffers");

    const int group = Hq / Hkv;
    const TileMap tm = map_workgroup(blockIdx.x, nqt, units, Hkv, group);
    const int hq = tm.hkv * group + tm.g;
    const size_t bh = (size_t)tm.b * Hq + hq;
    const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, scalar
    const int rb = (NKH == 2) ? (w >> 1) : w, khalf = (NKH == 2) ? (w & 1) : 0;   // row block, key half
    const int q0w = tm.qt * BR + 32 * rb;  // first query row of this wave
    const int qi = q0w + r;                // this lane's query row
    const bf16_t* qh = q + bh * N * D;
    const float sl2 = sc.sl2;              // scores in log2 units (positive multiplier)

    // Q rows of this wave as B operands: lane holds Q[qi][16c + 8h .. +7]. The operands
    // are formed (with ROPE: the row rotated, its table values loaded next to it) only
    // after the first K/V tile is staged, so the first tile's loads go out behind the
    // Q loads rather than after their arrival.
    bf16x8 qb[DC];
    u32x4 qraw[DC];
    QRopeRow<D> qtab;
    {
        const int qc = min(qi, N - 1);
        const bf16_t* qrow = ROPE ? rq.q + tm.b * rq.qb + hq * rq.qh + qc * rq.qn + 8 * h
                                  : qh + (size_t)qc * D + 8 * h;
#pragma unroll
        for (int c = 0; c < DC; ++c) qraw[c] = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
        if constexpr (ROPE) qtab.load(rq.cs + (size_t)qc * (D / 2), rq.sn + (size_t)qc * (D / 2), h);
    }

    // K/V tile prefetch registers: thread owns chunks tid + NT u (coalesced rows)
    u32x4 kreg[KCH], vreg[KCH];
    f32x16 oacc[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) oacc[x] = f32x16{};
    // Running (possibly stale) max in log2 units. It starts finite and far
    // below any score, so the first tile's rescale factor is exactly 0 and no
    // -inf - -inf can arise.
    float m_s = -0x1p100f;
    float l_run = 0.f;       // sum of this lane's fp16 probabilities (other half added at the end)

    const int last_q = min(N, (tm.qt + 1) * BR) - 1;
    const int kend = causal ? last_q + 1 : N;   // keys needed by this workgroup
    const int ntile = (kend + BC - 1) / BC;
    const int krow_a = perm32(r);
    // masking: accumulator e holds key kw0 + 8h + c_e with c_e = 16(e/8) + e%8;
    // it is kept iff c_e <= lim_row - kw0 (key < N, and key <= qi if causal)
    const int lim_row = (causal ? min(qi, N - 1) : N - 1) - 8 * h;

    const size_t kvoff = ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + kvoff, (uint32_t)N * D * 2);
    const VRows<D, ROPE> vrows(v, rq, tm.b, Hkv, tm.hkv, N);
    const uint32_t ld_off = (uint32_t)tid * 16;                     // byte offset of chunk 0 in a K tile
    const uint32_t vld_off = (uint32_t)(tid / CPR) * vrows.row_bytes + (uint32_t)(tid % CPR) * 16;
    const uint32_t vtile = BC * vrows.row_bytes;                      // bytes per V tile
    const int st_row = tid / CPR, st_col = (tid % CPR) * 8;           // LDS slot of chunk 0
    bf16_t* const kst0 = &Ks[0][st_row][st_col];
    _Float16* const vst0 = &Vs[0][st_row][st_col];
    constexpr int KBUF = BC * LD;                                     // elements per LDS buffer

    load_kv_tile<D, KCH, ROPE>(kreg, vreg, krs, ld_off, vrows, vld_off, 0);
    store_kv_tile<D, KCH>(kreg, vreg, kst0, vst0);
    if (ntile > 1) load_kv_tile<D, KCH, ROPE>(kreg, vreg, krs, ld_off + BC * D * 2, vrows, vld_off, vtile);
    __syncthreads();
    if constexpr (ROPE) rope_rotate_q<D>(qraw, qtab);
#pragma unroll
    for (int c = 0; c < DC; ++c) qb[c] = (qi < N) ? __builtin_bit_cast(bf16x8, apply_qsign(qraw[c], sc)) : bf16x8{};

    for (int j = 0; j < ntile; ++j) {
        const int buf = j & 1, k0 = j * BC;
        const int kw0 = k0 + KPW * khalf;       // first key of this wave's part of the tile
        const bool active = !causal || kw0 <= q0w + 31;
        if (active) {
            // a wave with two 32-key blocks (d = 128) skips the second one where it lies wholly
            // past the diagonal (the mask below then leaves it at -inf)
            const bool act1 = (KB > 1) && (!causal || kw0 + 32 <= q0w + 31);
            // ---- S^T = K * Q^T  (rows: 32 keys per block, permuted; columns: this wave's queries)
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                s[kb] = f32x16{};
                if (kb > 0 && !act1) continue;
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8 a =
                        *reinterpret_cast<const bf16x8*>(&Ks[buf][KPW * khalf + 32 * kb + krow_a][16 * c + 8 * h]);
                    if constexpr (ROPE)   // rotated K and Q hold fp16 bits
                        s[kb] = mfma_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, qb[c]), s[kb]);
                    else
                        s[kb] = mfma_bf16(a, qb[c], s[kb]);
                }
            }
            // ---- mask: only blocks crossing the diagonal or the end of the sequence
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int kwb = kw0 + 32 * kb;
                if ((kwb + 32 > N) || (causal && kwb + 31 > q0w)) {
                    const int lim = lim_row - kwb;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        s[kb][e] = (16 * (e >> 3) + (e & 7) <= lim) ? s[kb][e] : -INFINITY;
                }
            }
            // ---- online softmax with lazy rescaling (log2 domain)
            float mx = max16(s[0]);
#pragma unroll
            for (int kb = 1; kb < KB; ++kb) mx = vmax(mx, max16(s[kb]));
            const float mt = max_halves(mx) * sl2;
            if (__any(mt > m_s + kTau)) {
                const float m_new = vmax(m_s, mt);
                const float alpha = fast_exp2(m_s - m_new);
                l_run *= alpha;
#pragma unroll
                for (int x = 0; x < DB; ++x)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[x][e] *= alpha;
                m_s = m_new;
            }
            const float mb = m_s;
            // ---- P (fp16) and O^T += V^T * P^T over the wave's keys
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                if (kb > 0 && !act1) continue;
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    float p[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[kb][8 * c2 + t], sl2, -mb));
                    uint32_t pk[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        pk[t] = pack_f16(p[2 * t], p[2 * t + 1]);
                        l_run = add_f16_pair(pk[t], l_run);
                    }
                    const f16x8 pb = __builtin_bit_cast(f16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
                    for (int x = 0; x < DB; ++x) {
                        const f16x8 a =
                            lds_tr_operand(&Vs[buf][0][0], LD, KPW * khalf + 32 * kb + 16 * c2, 32 * x, h, r);
                        oacc[x] = mfma_f16(a, pb, oacc[x]);
                    }
                }
            }
        }
        if (j + 1 < ntile) {
            store_kv_tile<D, KCH>(kreg, vreg, kst0 + (buf ^ 1) * KBUF, vst0 + (buf ^ 1) * KBUF);
            if (j + 2 < ntile)
                load_kv_tile<D, KCH, ROPE>(kreg, vreg, krs, ld_off + (uint32_t)(j + 2) * (BC * D * 2), vrows,
                                           vld_off, (uint32_t)(j + 2) * vtile);
        }
        __syncthreads();
    }

    // ---- epilogue: normalise, store O (element type OT) and LSE (natural log). Accumulator e
    // of dim block x holds dim 32x + 8(e/4) + 4h + e%4 of query qi. With two key
    // halves, they are first merged through LDS (the K tile buffers are free after
    // the loop's last barrier).
    float l_tot = sum_halves(l_run);
    if constexpr (NKH == 1) {
        if (qi < N) {
            const float inv = 1.f / l_tot;
            OT* orow = o + (bh * N + qi) * D;
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const f32x4 val = {oacc[x][4 * a4 + 0] * inv, oacc[x][4 * a4 + 1] * inv,
                                       oacc[x][4 * a4 + 2] * inv, oacc[x][4 * a4 + 3] * inv};
                    store_out4(orow + 32 * x + 8 * a4 + 4 * h, val);
                }
            if (h == 0) lse[bh * N + qi] = (m_s + __log2f(l_tot)) * kLn2;
        }
    } else {
        float* xo = reinterpret_cast<float*>(smem) + rb * (32 * D);             // [32 rows][D]
        float* xs = reinterpret_cast<float*>(smem) + NRB * 32 * D + rb * 64;    // m[32], l[32]
        if (khalf == 1) {
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                    *reinterpret_cast<f32x4*>(xo + merge_off<D>(r, 8 * x + 2 * a4 + h)) =
                        f32x4{oacc[x][4 * a4 + 0], oacc[x][4 * a4 + 1], oacc[x][4 * a4 + 2], oacc[x][4 * a4 + 3]};
            if (h == 0) {
                xs[r] = m_s;
                xs[32 + r] = l_tot;
            }
        }
        __syncthreads();
        if (khalf == 0 && qi < N) {
            const float m1 = xs[r], l1 = xs[32 + r];
            const float m = vmax(m_s, m1);                // key half 0 always sees key 0
            const float a0 = fast_exp2(m_s - m), a1 = fast_exp2(m1 - m);
            const float l = l_tot * a0 + l1 * a1;
            const float inv = 1.f / l;
            const float c0 = a0 * inv, c1 = a1 * inv;
            OT* orow = o + (bh * N + qi) * D;
#pragma unroll
            for (int x = 0; x < DB; ++x)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const f32x4 o1 = *reinterpret_cast<const f32x4*>(xo + merge_off<D>(r, 8 * x + 2 * a4 + h));
                    const f32x4 val = {oacc[x][4 * a4 + 0] * c0 + o1[0] * c1, oacc[x][4 * a4 + 1] * c0 + o1[1] * c1,
                                       oacc[x][4 * a4 + 2] * c0 + o1[2] * c1, oacc[x][4 * a4 + 3] * c0 + o1[3] * c1};
                    store_out4(orow + 32 * x + 8 * a4 + 4 * h, val);
                }
            if (h == 0) lse[bh * N + qi] = (m + __log2f(l)) * kLn2;
        }
    }
}

bool mfma_path(const AttnArgs& a) { return mfma_shape(a.dtype, a.d); }

template <int D, typename OT, bool ROPE>
static hipError_t launch_fwd_d(const AttnArgs& a, hipStream_t st) {
    const int nqt = (a.N + fwd::kRows<D> - 1) / fwd::kRows<D>;
    const int units = a.B * a.Hkv;
    const dim3 grid((unsigned)(nqt * a.B * a.Hq));
    const QRope rq = ROPE ? *a.rope : QRope{};
    hipLaunchKernelGGL((fwd_mfma_kernel<D, OT, ROPE>), grid, dim3(fwd::kThreads<D>), 0, st, (const bf16_t*)a.q,
                       (const bf16_t*)a.k, (const bf16_t*)a.v, (OT*)a.o, a.lse, a.Hq, a.Hkv, a.N, a.causal,
                       score_scale(a.scale), nqt, units, rq);
    return hipGetLastError();
}

template <bool ROPE>
static hipError_t launch_fwd_rope_or_not(const AttnArgs& a, hipStream_t st) {
    if (a.out_dtype == ATTN_BF16)
        return (a.d == 64) ? launch_fwd_d<64, bf16_t, ROPE>(a, st) : launch_fwd_d<128, bf16_t, ROPE>(a, st);
    return (a.d == 64) ? launch_fwd_d<64, float, ROPE>(a, st) : launch_fwd_d<128, float, ROPE>(a, st);
}

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t st) {
    return a.rope ? launch_fwd_rope_or_not<true>(a, st) : launch_fwd_rope_or_not<false>(a, st);
}

}  // namespace tca
