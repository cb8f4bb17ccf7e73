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
#include "tca_internal.h"

namespace tca {

namespace bwdq {
constexpr int NW = 4;            // waves per workgroup
constexpr int BQ = 32 * NW;      // query rows per workgroup
constexpr int BC = 64;           // keys per K/V tile
constexpr int PAD = 8;
}  // namespace bwdq

// Global -> registers: K and V rows k0 .. k0 + BC - 1 (clamped to N - 1).
template <int D, int KCH>
__device__ __forceinline__ void bwd_load_kv(u32x4 (&kreg)[KCH], u32x4 (&vreg)[KCH], const bf16_t* kh,
                                            const bf16_t* vh, int k0, int N, int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int cid = tid + 256 * u;
        const int key = min(k0 + cid / CPR, N - 1);
        const size_t off = (size_t)key * D + (cid % CPR) * 8;
        kreg[u] = *reinterpret_cast<const u32x4*>(kh + off);
        vreg[u] = *reinterpret_cast<const u32x4*>(vh + off);
    }
}

// Registers -> LDS: K converted to fp16 rows, V kept as bf16 rows.
template <int D, int KCH>
__device__ __forceinline__ void bwd_store_kv(const u32x4 (&kreg)[KCH], const u32x4 (&vreg)[KCH],
                                             _Float16 (*Ks)[D + bwdq::PAD], bf16_t (*Vs)[D + bwdq::PAD],
                                             int tid) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
        const int cid = tid + 256 * u;
        const int row = cid / CPR, col = (cid % CPR) * 8;
        *reinterpret_cast<u32x4*>(&Ks[row][col]) = bf16x8_to_f16x8(kreg[u]);
        *reinterpret_cast<u32x4*>(&Vs[row][col]) = vreg[u];
    }
}

template <int D>
__global__ void __launch_bounds__(256, (D == 64) ? 2 : 1)
bwd_dq_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
              const float* __restrict__ o, const float* __restrict__ lse,
              const bf16_t* __restrict__ dout, float* __restrict__ delta, float* __restrict__ dq,
              int Hq, int Hkv, int N, int causal, float scale, int nqt, int units) {
    using namespace bwdq;
    constexpr int DC = D / 16, DB = D / 32, NB = BC / 32, LD = D + PAD;
    constexpr int CPR = D / 8, KCH = BC * CPR / 256;
    __shared__ __attribute__((aligned(16))) _Float16 Ks[2][BC][LD];
    __shared__ __attribute__((aligned(16))) bf16_t Vs[2][BC][LD];

    const int group = Hq / Hkv;
    const TileMap tm = map_workgroup(blockIdx.x, nqt, units, Hkv, group);
    const int hq = tm.hkv * group + tm.g;
    const size_t bh = (size_t)tm.b * Hq + hq;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int q0w = tm.qt * BQ + 32 * w;
    const int qi = q0w + r;
    const int qc = min(qi, N - 1);
    const bool qok = qi < N;
    const bf16_t* kh = k + ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const bf16_t* vh = v + ((size_t)tm.b * Hkv + tm.hkv) * N * D;
    const float sl2 = scale * kLog2e;

    // Q (fp16) and dO (bf16) rows of this lane's query as B operands, and D_i
    f16x8 qb[DC];
    bf16x8 db[DC];
    float Di;
    {
        const bf16_t* qrow = q + (bh * N + qc) * D + 8 * h;
        const bf16_t* drow = dout + (bh * N + qc) * D + 8 * h;
        const float* orow = o + (bh * N + qc) * D + 8 * h;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const u32x4 qv = *reinterpret_cast<const u32x4*>(qrow + 16 * c);
            const u32x4 dv = *reinterpret_cast<const u32x4*>(drow + 16 * c);
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(orow + 16 * c);
            const f32x4 o1 = *reinterpret_cast<const f32x4*>(orow + 16 * c + 4);
            qb[c] = qok ? __builtin_bit_cast(f16x8, bf16x8_to_f16x8(qv)) : f16x8{};
            db[c] = qok ? __builtin_bit_cast(bf16x8, dv) : bf16x8{};
            part = fmaf(bf16_lo(dv.x), o0[0], part);
            part = fmaf(bf16_hi(dv.x), o0[1], part);
            part = fmaf(bf16_lo(dv.y), o0[2], part);
            part = fmaf(bf16_hi(dv.y), o0[3], part);
            part = fmaf(bf16_lo(dv.z), o1[0], part);
            part = fmaf(bf16_hi(dv.z), o1[1], part);
            part = fmaf(bf16_lo(dv.w), o1[2], part);
            part = fmaf(bf16_hi(dv.w), o1[3], part);
        }
        Di = sum_halves(part);   // the two half-waves hold complementary dims of the row
        if (qok && h == 0) delta[bh * N + qi] = Di;
    }
    const float Li = qok ? lse[bh * N + qi] * kLog2e : 0.f;

    u32x4 kreg[KCH], vreg[KCH];
    f32x16 dqa[DB];
#pragma unroll
    for (int x = 0; x < DB; ++x) dqa[x] = f32x16{};

    const int last_q = min(N, (tm.qt + 1) * BQ) - 1;
    const int kend = causal ? last_q + 1 : N;
    const int ntile = (kend + BC - 1) / BC;
    const int krow_a = perm32(r);

    bwd_load_kv<D, KCH>(kreg, vreg, kh, vh, 0, N, tid);
    bwd_store_kv<D, KCH>(kreg, vreg, Ks[0], Vs[0], tid);
    if (ntile > 1) bwd_load_kv<D, KCH>(kreg, vreg, kh, vh, BC, N, tid);
    __syncthreads();

    for (int j = 0; j < ntile; ++j) {
        const int buf = j & 1, k0 = j * BC;
        if (!causal || k0 <= q0w + 31) {
            // ---- S^T = K Q^T and dP^T = V dO^T (rows: keys, permuted; columns: queries)
            f32x16 s[NB], dp[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                s[nb] = f32x16{};
                dp[nb] = f32x16{};
            }
#pragma unroll
            for (int c = 0; c < DC; ++c)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const f16x8 ak = *reinterpret_cast<const f16x8*>(&Ks[buf][32 * nb + krow_a][16 * c + 8 * h]);
                    const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Vs[buf][32 * nb + krow_a][16 * c + 8 * h]);
                    s[nb] = mfma_f16(ak, qb[c], s[nb]);
                    dp[nb] = mfma_bf16(av, db[c], dp[nb]);
                }
            // ---- P, dS (accumulator e of block nb: key k0 + 32nb + 16(e/8) + 8h + e%8)
            const bool need_mask = (k0 + BC > N) || (causal && k0 + BC - 1 > q0w);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float p = fast_exp2(fmaf(s[nb][e], sl2, -Li));
                    if (need_mask) {
                        const int key = k0 + 32 * nb + 16 * (e >> 3) + 8 * h + (e & 7);
                        if (key >= N || (causal && key > qi)) p = 0.f;
                    }
                    s[nb][e] = p * (dp[nb][e] - Di);   // dS
                }
            // ---- dQ^T += K^T dS^T  (A: K tile read transposed; B: dS from registers)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const f16x8 dsb = to_f16x8(s[nb][8 * c2 + 0], s[nb][8 * c2 + 1], s[nb][8 * c2 + 2],
                                               s[nb][8 * c2 + 3], s[nb][8 * c2 + 4], s[nb][8 * c2 + 5],
                                               s[nb][8 * c2 + 6], s[nb][8 * c2 + 7]);
#pragma unroll
                    for (int x = 0; x < DB; ++x) {
                        const f16x8 a = lds_tr_operand(&Ks[buf][0][0], LD, 32 * nb + 16 * c2, 32 * x, h, r);
                        dqa[x] = mfma_f16(a, dsb, dqa[x]);
                    }
                }
        }
        if (j + 1 < ntile) {
            bwd_store_kv<D, KCH>(kreg, vreg, Ks[buf ^ 1], Vs[buf ^ 1], tid);
            if (j + 2 < ntile) bwd_load_kv<D, KCH>(kreg, vreg, kh, vh, (j + 2) * BC, N, tid);
        }
        __syncthreads();
    }

    // ---- store dQ: accumulator e of dim block x holds dim 32x + 8(e/4) + 4h + e%4 of query qi
    if (qok) {
        float* row = dq + (bh * N + qi) * D;
#pragma unroll
        for (int x = 0; x < DB; ++x)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const f32x4 val = {dqa[x][4 * a4 + 0] * scale, dqa[x][4 * a4 + 1] * scale,
                                   dqa[x][4 * a4 + 2] * scale, dqa[x][4 * a4 + 3] * scale};
                *reinterpret_cast<f32x4*>(row + 32 * x + 8 * a4 + 4 * h) = val;
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
// query tile (BQ = 32 NQW rows), accumulating partial dK, dV for its keys in
// registers. At the end of a K/V tile the NQW partials of each key half are
// summed in LDS in a fixed order (deterministic) and written out.
//
//   S  = Q K^T, dP = dO V^T  (rows: queries, permuted; columns: keys -> one key
//                             per lane, so P and dS are A operands in place)
//   dV += P^T dO, dK += dS^T Q (B operands: dO, Q tiles read transposed)
namespace bwdkv {
constexpr int BC = 64;
constexpr int PAD = 8;
template <int D> struct Cfg;
template <> struct Cfg<64> { static constexpr int NQW = 4; };   // 8 waves, 128-row query tiles
template <> struct Cfg<128> { static constexpr int NQW = 2; };  // 4 waves, 64-row query tiles
}  // namespace bwdkv

template <int D>
__global__ void __launch_bounds__(64 * 2 * bwdkv::Cfg<D>::NQW, 1)
bwd_dkdv_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                const float* __restrict__ lse, const bf16_t* __restrict__ dout,
                const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
                int Hq, int Hkv, int N, int causal, float scale, int ntiles, int wg_per_unit) {
    using namespace bwdkv;
    constexpr int NQW = Cfg<D>::NQW;
    constexpr int NT = 64 * 2 * NQW;          // threads
    constexpr int BQ = 32 * NQW;              // query rows per staged tile
    constexpr int DC = D / 16, DB = D / 32, LD = D + PAD;
    constexpr int CPR = D / 8;
    constexpr int QCH = BQ * CPR / NT;        // 16-byte chunks per thread per tensor per tile
    __shared__ __attribute__((aligned(16))) _Float16 Qs[2][BQ][LD];
    __shared__ __attribute__((aligned(16))) _Float16 dOs[2][BQ][LD];
    __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
    __shared__ __attribute__((aligned(16))) float Ds[2][BQ];
    __shared__ __attribute__((aligned(16))) float red[2][BC][D];   // dK, dV partial sums

    const int group = Hq / Hkv;
    const int unit = blockIdx.x / wg_per_unit;
    const int slot = blockIdx.x % wg_per_unit;
    const int b = unit / Hkv, hkv = unit % Hkv;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, r = lane & 31;
    const int kh_ = w & 1, qw = w >> 1;       // key half, query sub-block
    const size_t kvoff = ((size_t)b * Hkv + hkv) * N * D;
    const float sl2 = scale * kLog2e;
    const int nqt = (N + BQ - 1) / BQ;

    // K/V tiles of this workgroup: causal -> {slot, ntiles-1-slot} (one if they coincide)
    const int tile_a = slot;
    const int tile_b = (causal && ntiles - 1 - slot != slot) ? ntiles - 1 - slot : -1;

    // items: (tile index t in {0,1}, head g, query tile i); for each tile, the
    // query tiles at or below the diagonal, for every head of the group
    auto first_qt = [&](int tile) { return causal ? (tile * BC) / BQ : 0; };
    const int na = group * (nqt - first_qt(tile_a));
    const int nbitems = (tile_b >= 0) ? group * (nqt - first_qt(tile_b)) : 0;
    const int nitems = na + nbitems;

    u32x4 qreg[QCH], dreg[QCH];
    float lreg = 0.f, dlreg = 0.f;
    // decode item -> (tile, head, query tile)
    auto item = [&](int it, int& tile, int& g, int& qt) {
        const int t = (it < na) ? 0 : 1;
        const int rel = t ? it - na : it;
        tile = t ? tile_b : tile_a;
        const int f = first_qt(tile), per = nqt - f;
        g = rel / per;
        qt = f + rel % per;
    };
    auto load_item = [&](int it) {
        int tile, g, qt;
        item(it, tile, g, qt);
        const size_t bh = (size_t)b * Hq + hkv * group + g;
        const bf16_t* qh = q + bh * N * D;
        const bf16_t* dh = dout + bh * N * D;
#pragma unroll
        for (int u = 0; u < QCH; ++u) {
            const int cid = tid + NT * u;
            const int row = min(qt * BQ + cid / CPR, N - 1);
            const size_t off = (size_t)row * D + (cid % CPR) * 8;
            qreg[u] = *reinterpret_cast<const u32x4*>(qh + off);
            dreg[u] = *reinterpret_cast<const u32x4*>(dh + off);
        }
        if (tid < BQ) {
            const int row = qt * BQ + tid;
            const int rc = min(row, N - 1);
            lreg = lse[bh * N + rc] * kLog2e;
            dlreg = delta[bh * N + rc];
        }
    };
    auto store_item = [&](int buf) {
#pragma unroll
        for (int u = 0; u < QCH; ++u) {
            const int cid = tid + NT * u;
            const int row = cid / CPR, col = (cid % CPR) * 8;
            *reinterpret_cast<u32x4*>(&Qs[buf][row][col]) = bf16x8_to_f16x8(qreg[u]);
            *reinterpret_cast<u32x4*>(&dOs[buf][row][col]) = bf16x8_to_f16x8(dreg[u]);
        }
        if (tid < BQ) {
            Ls[buf][tid] = lreg;
            Ds[buf][tid] = dlreg;
        }
    };

    f16x8 kb[DC], vb[DC];
    f32x16 dka[DB], dva[DB];
    int cur_tile = -1;

    if (nitems > 0) {
        load_item(0);
        store_item(0);
        if (nitems > 1) load_item(1);
    }
    __syncthreads();

    for (int it = 0; it < nitems; ++it) {
        const int buf = it & 1;
        int tile, g, qt;
        item(it, tile, g, qt);
        const int kw0 = tile * BC + 32 * kh_;   // first key of this wave
        const int kw = kw0 + r;                 // this lane's key
        if (tile != cur_tile) {
            // new K/V tile: this lane's K, V rows as fp16 B operands; clear partials
            cur_tile = tile;
            const bf16_t* krow = k + kvoff + (size_t)min(kw, N - 1) * D + 8 * h;
            const bf16_t* vrow = v + kvoff + (size_t)min(kw, N - 1) * D + 8 * h;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                kb[c] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(krow + 16 * c)));
                vb[c] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(*reinterpret_cast<const u32x4*>(vrow + 16 * c)));
            }
#pragma unroll
            for (int x = 0; x < DB; ++x) {
                dka[x] = f32x16{};
                dva[x] = f32x16{};
            }
        }
        const int q0 = qt * BQ + 32 * qw;        // first query row of this wave's block
        const bool live = !causal || q0 + 31 >= kw0;
        if (live) {
            // ---- S = Q K^T, dP = dO V^T (accumulator e: query q0 + 16(e/8) + 8h + e%8, key kw)
            f32x16 s = f32x16{}, dp = f32x16{};
            const int arow = 32 * qw + perm32(r);
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const f16x8 aq = *reinterpret_cast<const f16x8*>(&Qs[buf][arow][16 * c + 8 * h]);
                const f16x8 ad = *reinterpret_cast<const f16x8*>(&dOs[buf][arow][16 * c + 8 * h]);
                s = mfma_f16(aq, kb[c], s);
                dp = mfma_f16(ad, vb[c], dp);
            }
            const bool need_mask = (q0 + 32 > N) || (kw0 + 32 > N) || (causal && q0 < kw0 + 31);
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int qq = 32 * qw + 16 * c2 + 8 * h;   // tile row of accumulator 8c2
                const f32x4 l0 = *reinterpret_cast<const f32x4*>(&Ls[buf][qq]);
                const f32x4 l1 = *reinterpret_cast<const f32x4*>(&Ls[buf][qq + 4]);
                const f32x4 d0 = *reinterpret_cast<const f32x4*>(&Ds[buf][qq]);
                const f32x4 d1 = *reinterpret_cast<const f32x4*>(&Ds[buf][qq + 4]);
                const float lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
                const float dl[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int e = 8 * c2 + t;
                    float p = fast_exp2(fmaf(s[e], sl2, -lv[t]));
                    if (need_mask) {
                        const int qrow = qt * BQ + qq + t;
                        if (qrow >= N || kw >= N || (causal && kw > qrow)) p = 0.f;
                    }
                    s[e] = p;
                    dp[e] = p * (dp[e] - dl[t]);
                }
            }
            // ---- dV += P^T dO, dK += dS^T Q (B: dO, Q tiles read transposed, rows = queries)
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const f16x8 pa = to_f16x8(s[8 * c2 + 0], s[8 * c2 + 1], s[8 * c2 + 2], s[8 * c2 + 3],
                                          s[8 * c2 + 4], s[8 * c2 + 5], s[8 * c2 + 6], s[8 * c2 + 7]);
                const f16x8 da = to_f16x8(dp[8 * c2 + 0], dp[8 * c2 + 1], dp[8 * c2 + 2], dp[8 * c2 + 3],
                                          dp[8 * c2 + 4], dp[8 * c2 + 5], dp[8 * c2 + 6], dp[8 * c2 + 7]);
#pragma unroll
                for (int x = 0; x < DB; ++x) {
                    const f16x8 bo = lds_tr_operand(&dOs[buf][0][0], LD, 32 * qw + 16 * c2, 32 * x, h, r);
                    const f16x8 bq = lds_tr_operand(&Qs[buf][0][0], LD, 32 * qw + 16 * c2, 32 * x, h, r);
                    dva[x] = mfma_f16(pa, bo, dva[x]);
                    dka[x] = mfma_f16(da, bq, dka[x]);
                }
            }
        }
        if (it + 1 < nitems) {
            store_item(buf ^ 1);
            if (it + 2 < nitems) load_item(it + 2);
        }
        // ---- end of a K/V tile: fixed-order reduction of the query sub-block partials
        int ntile_next = -1;
        if (it + 1 < nitems) {
            int g2, qt2;
            item(it + 1, ntile_next, g2, qt2);
        }
        if (ntile_next != tile) {
            // accumulator e of dim block x: key 32kh + 8(e/4) + 4h + e%4, dim 32x + r
#pragma unroll 1
            for (int step = 0; step < NQW; ++step) {
                if (qw == step) {
#pragma unroll
                    for (int x = 0; x < DB; ++x)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int key = 32 * kh_ + 8 * (e >> 2) + 4 * h + (e & 3);
                            float* pk = &red[0][key][32 * x + r];
                            float* pv = &red[1][key][32 * x + r];
                            if (step == 0) {
                                *pk = dka[x][e];
                                *pv = dva[x][e];
                            } else {
                                *pk += dka[x][e];
                                *pv += dva[x][e];
                            }
                        }
                }
                __syncthreads();
            }
            // write the tile's dK (scaled) and dV rows
            const int key0 = tile * BC;
            constexpr int F4 = BC * D / 4;   // float4 per tensor
#pragma unroll
            for (int u = 0; u < F4 / NT; ++u) {
                const int idx = tid + NT * u;
                const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
                if (key0 + row < N) {
                    const f32x4 kv = *reinterpret_cast<const f32x4*>(&red[0][row][col]);
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(&red[1][row][col]);
                    const size_t off = kvoff + (size_t)(key0 + row) * D + col;
                    *reinterpret_cast<f32x4*>(dk + off) = kv * scale;
                    *reinterpret_cast<f32x4*>(dv + off) = vv;
                }
            }
        }
        __syncthreads();
    }
}

template <int D>
static hipError_t launch_bwd_dq_d(const AttnArgs& a, hipStream_t st) {
    const int nqt = (a.N + bwdq::BQ - 1) / bwdq::BQ;
    const int units = a.B * a.Hkv;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)(nqt * a.B * a.Hq)), dim3(256), 0, st,
                       (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const float*)a.o,
                       (const float*)a.lse, (const bf16_t*)a.dout, (float*)a.workspace, a.dq, a.Hq,
                       a.Hkv, a.N, a.causal, a.scale, nqt, units);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_dkdv_d(const AttnArgs& a, hipStream_t st) {
    const int ntiles = (a.N + bwdkv::BC - 1) / bwdkv::BC;
    const int per_unit = a.causal ? (ntiles + 1) / 2 : ntiles;
    const int threads = 64 * 2 * bwdkv::Cfg<D>::NQW;
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)(per_unit * a.B * a.Hkv)), dim3(threads), 0, st,
                       (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const float*)a.lse,
                       (const bf16_t*)a.dout, (const float*)a.workspace, a.dk, a.dv, a.Hq, a.Hkv, a.N,
                       a.causal, a.scale, ntiles, per_unit);
    return hipGetLastError();
}

hipError_t launch_bwd_mfma_dq(const AttnArgs& a, hipStream_t st) {
    return (a.d == 64) ? launch_bwd_dq_d<64>(a, st) : launch_bwd_dq_d<128>(a, st);
}
hipError_t launch_bwd_mfma_dkdv(const AttnArgs& a, hipStream_t st) {
    return (a.d == 64) ? launch_bwd_dkdv_d<64>(a, st) : launch_bwd_dkdv_d<128>(a, st);
}

}  // namespace tca
