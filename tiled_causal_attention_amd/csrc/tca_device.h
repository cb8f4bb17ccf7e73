// tca_device.h -- shared device helpers for the gfx950 attention kernels:
// vector types, matrix-core wrappers, conversions and lane exchanges.
//
// Matrix-core layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}, one
// wave of 64 lanes; lane = 32*h + r with h in {0,1}, r in [0,32)):
//   A (32 x 16): lane holds A[m = r][k = 8h .. 8h+7]      (8 packed 16-bit values)
//   B (16 x 32): lane holds B[k = 8h .. 8h+7][n = r]
//   C (32 x 32): lane holds C[m = 8(e/4) + 4h + e%4][n = r] in accumulator e = 0..15
// so a product's output column index n is fixed per lane and can feed the next
// product as its B operand (n stays the lane) or as its A operand transposed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tca {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // one 16-byte chunk
typedef uint16_t bf16_t;   // raw bfloat16 bits in memory
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// bfloat16 bits -> float32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Two float32 -> packed fp16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f16x2 h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Eight float32 accumulator values -> one fp16 operand.
__device__ __forceinline__ f16x8 to_f16x8(float a0, float a1, float a2, float a3,
                                          float a4, float a5, float a6, float a7) {
    f16x8 r = {(_Float16)a0, (_Float16)a1, (_Float16)a2, (_Float16)a3,
               (_Float16)a4, (_Float16)a5, (_Float16)a6, (_Float16)a7};
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// IEEE-754-2019 maximum (NaN-propagating). Unlike fmaxf it needs no operand
// canonicalisation, so a chain of them maps onto v_maximum3_f32 directly.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Maximum over the 16 accumulator values of a lane (8 v_maximum3_f32).
__device__ __forceinline__ float max16(const f32x16& s) {
    const float a = vmax3(s[0], s[1], s[2]), b = vmax3(s[3], s[4], s[5]), c = vmax3(s[6], s[7], s[8]);
    const float d = vmax3(s[9], s[10], s[11]), e = vmax3(s[12], s[13], s[14]);
    return vmax(vmax3(a, b, c), vmax3(d, e, s[15]));
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, stride 0). Loads
// through it at byte offsets >= bytes return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Direct global -> LDS copy through a buffer resource (no registers): lane l
// reads `bytes` (4 or 16) at byte offset voff and writes them to LDS at
// lds_dst + l * bytes; lds_dst must be the same in every lane. Completion is
// tracked by vmcnt: wait for it (s_waitcnt vmcnt(0)) and then barrier before
// any wave reads the destination.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rs, void* lds_dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t rs, void* lds_dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst, 4, voff, 0, 0, 0);
}
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x3f70); }   // vmcnt(0)

// One 16-byte chunk at byte offset voff (per lane) through a buffer resource.
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
}

// Eight bfloat16 (one 16-byte chunk) -> eight fp16, round to nearest even
// (exact for |x| in [2^-14, 65504]).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
    u32x4 r;
    r.x = pack_f16(bf16_lo(w.x), bf16_hi(w.x));
    r.y = pack_f16(bf16_lo(w.y), bf16_hi(w.y));
    r.z = pack_f16(bf16_lo(w.z), bf16_hi(w.z));
    r.w = pack_f16(bf16_lo(w.w), bf16_hi(w.w));
    return r;
}

// Sum of a packed fp16 pair added to acc in fp32 (v_dot2c_f32_f16 with (1, 1)).
__device__ __forceinline__ float add_f16_pair(uint32_t pair, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
}

// Matrix-core operand that contracts over the ROWS of a row-major 16-bit LDS
// tile, read with the transposing LDS load (ds_read_b64_tr_b16): lane (h, r)
// receives tile[row0 + 8h + t][col0 + r], t = 0..7 -- the A operand of a
// product whose m index is the tile column, or the B operand whose n index is.
// The transposing load hands lane i of each 16-lane group element (i mod 4) of
// the 8-byte chunks addressed by lanes 4k + i/4 (k = 0..3) of that group; the
// addresses below put row row0 + 8h + (r%16)/4 (+4 for the second load),
// columns col0 + 16(r/16) + 4(r%4) .. +3 behind each lane.
__device__ __forceinline__ f16x8 lds_tr_operand(const _Float16* tile, int stride, int row0, int col0,
                                                int h, int r) {
    const _Float16* p = tile + (row0 + 8 * h + ((r & 15) >> 2)) * stride + col0 + 16 * (r >> 4) + 4 * (r & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * stride));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(f16x8, v);
}

// LDS layout of the Q and dO tiles of the dK/dV pass, staged by direct
// global -> LDS copies: unpadded rows of D 16-bit elements (the copies land
// whole 1 KB blocks, so rows cannot be padded), 16-byte chunk c of row R at
// chunk position c ^ tile_swz(R). LDS serves a 16-byte read for 16
// consecutive lanes per cycle and a transposing 8-byte read for 32, from 64
// four-byte banks, so the two operand reads need:
//  - row-per-lane reads (rows R..R+15 of an aligned block, one chunk each):
//    the 16 rows on 16 different 16-byte bank groups;
//  - transposing reads (rows R..R+3, R = 0 mod 4, four consecutive chunks
//    from a multiple of 4): no bank shared by the four rows' chunks.
// On 64-element rows (two rows per 64 banks) both hold for
// tile_swz(R) = (R/4 mod 4) + 4 (R/2 mod 2): the rows of one parity in a
// 16-row block take eight different XOR values, and rows R and R+2 differ in
// the bit that moves a chunk to the other half of the row. 128-element rows
// span every bank; there tile_swz(R) = 4 (R mod 4) + (R/4 mod 4) serves both.
// rocprofv3's SQ_LDS_BANK_CONFLICT reads zero for both reads on both layouts.
// (The register-staged K/V tiles of the forward and the dQ pass keep padded
// rows, stride D + 8: conflict-free for row reads, two cycles per transposing
// read, but with additive operand addresses. The swizzle there removed the
// conflicts and cost more in address arithmetic than it saved.)
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
    return (D == 64) ? (((row >> 2) & 3) | ((row & 2) << 1)) : (((row & 3) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {   // element offset of (row, col)
    return row * D + ((((col >> 3) ^ tile_swz<D>(row))) << 3) + (col & 7);
}
// Source byte offset, within a tile of such rows, of the 16 bytes that lane
// `lane` of copy instruction i lands at LDS byte 1024 i + 16 lane: row R and
// chunk position p there hold source chunk p ^ tile_swz(R) of row R.
template <int D>
__device__ __forceinline__ uint32_t tile_copy_src(int i, int lane) {
    const int o = i * 1024 + lane * 16;
    const int row = o / (2 * D), p = (o % (2 * D)) / 16;
    return (uint32_t)(row * (2 * D) + ((p ^ tile_swz<D>(row)) * 16));
}
// lds_tr_operand for such a tile: lane (h, r) receives tile[row0 + 8h + t][col0 + r], t = 0..7
template <int D>
__device__ __forceinline__ f16x8 tile_tr_operand(const _Float16* tile, int row0, int col0, int h, int r) {
    const int row = row0 + 8 * h + ((r & 15) >> 2), col = col0 + 16 * (r >> 4) + 4 * (r & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + tile_off<D>(row, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + tile_off<D>(row + 4, col)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(f16x8, v);
}

// Float offset of 4-float chunk c of row r in a [rows][D] float32 exchange
// area (the key-half merges at the end of the forward and the dQ pass): chunk
// position c ^ (r mod 16). The 16 lanes of one LDS cycle write or read the
// same chunk of 16 consecutive rows; with rows of 64 or 128 floats (whole
// multiples of the 64 banks) they would all hit one bank group and serialise
// 16-fold, the swizzle spreads them over all 16. Needs D >= 64.
template <int D>
__device__ __forceinline__ int merge_off(int r, int c) {
    static_assert(D >= 64, "the swizzle spans 16 chunks");
    return r * D + 4 * (c ^ (r & 15));
}

// Reductions across the two half-waves with v_permlane32_swap: swapping a
// register with itself leaves, in every lane, the pair {own value, value of
// lane l ^ 32}, so max/sum over the pair combine the two halves.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value held by lane (lane ^ 32): the other half of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Row permutation that makes a 32x32 accumulator feed the next product's
// 16-deep operand in natural order: swaps bits 2 and 3 of the row index.
// If the A operand's row m is loaded from source row perm32(m), accumulator
// e of lane (h, r) holds source row 16(e/8) + 8h + (e%8).
__device__ __forceinline__ int perm32(int m) {
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Workgroup id -> (query tile, batch, KV head, head within the group) for the
// query-tile-parallel kernels. Longest (last) query tiles come first. When the
// number of (batch, KV head) units is a multiple of 8, all workgroups of a unit
// share w mod 8, i.e. land on one XCD (workgroups are dealt to the 8 XCDs
// round-robin), so the unit's K/V tiles stay in that XCD's L2.
struct TileMap {
    int qt, b, hkv, g;
};
__device__ __forceinline__ TileMap map_workgroup(int w, int nqt, int units, int Hkv, int group) {
    TileMap m;
    int t, u;
    if ((units & 7) == 0) {
        const int x = w & 7, i = w >> 3, upx = units >> 3;
        m.g = i % group;
        const int rest = i / group;
        u = (rest % upx) * 8 + x;
        t = rest / upx;
    } else {
        const int per = units * group;
        t = w / per;
        const int rem = w % per;
        u = rem / group;
        m.g = rem % group;
    }
    m.qt = nqt - 1 - t;
    m.b = u / Hkv;
    m.hkv = u % Hkv;
    return m;
}

// Output element stores: float32 as is, bfloat16 rounded to nearest even
// (v_cvt_pk_bf16_f32). store_out4 writes 4 consecutive elements (16 or 8 bytes).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 h = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ void store_out4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store_out4(bf16_t* p, f32x4 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
}
__device__ __forceinline__ void store_out1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out1(bf16_t* p, float v) {
    *p = (bf16_t)(pack_bf16(v, 0.f) & 0xffffu);
}
// Eight consecutive output-type elements held as raw registers, so a load can be
// issued early and converted later (float32: 32 bytes, bfloat16: 16 bytes).
template <typename T> struct Row8;
template <> struct Row8<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const f32x4*>(p);
        b = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void get(float (&x)[8]) const {
        x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
        x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    }
};
template <> struct Row8<bf16_t> {
    u32x4 w;
    __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const u32x4*>(p); }
    __device__ __forceinline__ void get(float (&x)[8]) const {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
};

// Eight consecutive elements (float32 or bfloat16) at p -> float32.
__device__ __forceinline__ void load8_f32(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
__device__ __forceinline__ void load8_f32(const bf16_t* p, float (&x)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// Scores for the matrix-core kernels, for any finite scale. They form
// s' (Q' K^T) with Q' = sgn(scale) Q and s' = |scale| (1 when scale is 0), which
// equals scale (Q K^T) exactly (a sign flip or a zero is exact in any format). The
// exponent's multiplier s' log2(e) is then always positive, so a key masked with
// -inf before the multiply stays -inf and the running max of the raw products is
// the max of the scaled ones. Gradients: dQ = scale dS K (the true scale),
// dK = s' dS^T Q' (the stored Q' copy carries the sign). Scale 0 zeroes Q', so every
// visible key gets the same weight and dK is zero.
struct ScoreScale {
    float sl2;        // s' log2(e)
    float kscale;     // s', the dK multiplier against Q'
    uint32_t qand;    // Q' bits = (Q bits & qand) ^ qxor on each 32-bit pair of 16-bit values
    uint32_t qxor;    // (bf16 and fp16 keep the sign in bit 15 of each half)
};
inline ScoreScale score_scale(float scale) {
    ScoreScale s;
    const float sp = (scale == 0.f) ? 1.f : fabsf(scale);
    s.sl2 = sp * kLog2e;
    s.kscale = sp;
    s.qand = (scale == 0.f) ? 0u : 0xffffffffu;
    s.qxor = (scale < 0.f) ? 0x80008000u : 0u;
    return s;
}
__device__ __forceinline__ u32x4 apply_qsign(u32x4 x, const ScoreScale& s) { return (x & s.qand) ^ s.qxor; }

// Rotary embedding of the query side, for kernels that rotate Q in registers
// (rotate-half pairing: dims i and i + D/2, cos/sin = table[n][i] at row n) and,
// in the dQ pass, turn dQ back by the transpose rotation at the store. Q and dQ
// are read / written through element strides (batch, head, row); the head
// dimension is contiguous and every row start 16-byte aligned.
struct QRope {
    const bf16_t* q;
    long long qb, qh, qn;    // q strides
    void* dq;                // dq in the output type
    long long gb, gh, gn;    // dq strides
    const float* cs;         // [N][D/2]
    const float* sn;
    const bf16_t* v;         // V read in place through its strides (row starts 16-byte aligned, vn >= D)
    long long vb, vh, vn;
};

// The dK/dV pass of the rotary path: V read in place through its strides, dK
// turned back by the transpose rotation and dK, dV written through their strides
// in the output type (one rounding).
struct KVRope {
    const bf16_t* v;
    long long vb, vh, vn;    // V strides (row starts 16-byte aligned)
    void* dk;
    long long kb, kh, kn;    // dk strides
    void* dv;
    long long db, dh, dn;    // dv strides
    const float* cs;         // [N][D/2]
    const float* sn;
};

// One KV head's V rows: in place through rq's strides (ROPE), else contiguous
// [N][D]. Rows at or past N lie outside the range (the row stride is at least D)
// and read as zero.
template <int D, bool ROPE>
struct VRows {
    const unsigned char* base;
    uint32_t bytes;       // readable bytes from base
    uint32_t row_bytes;   // byte stride of consecutive rows
    __device__ __forceinline__ VRows(const bf16_t* v, const QRope& rq, int b, int Hkv, int hkv, int N) {
        if constexpr (ROPE) {
            base = reinterpret_cast<const unsigned char*>(rq.v + b * rq.vb + hkv * rq.vh);
            row_bytes = (uint32_t)(rq.vn * 2);
            bytes = (uint32_t)(((long long)(N - 1) * rq.vn + D) * 2);
        } else {
            base = reinterpret_cast<const unsigned char*>(v + ((size_t)b * Hkv + hkv) * N * D);
            row_bytes = (uint32_t)(D * 2);
            bytes = (uint32_t)N * D * 2;
        }
    }
    // 16 bytes at byte offset lane_off + off (off the same in every lane), zero
    // past the range. With a runtime row stride the uniform part moves the
    // resource's base instead of adding to the lane's offset, so that one
    // register per lane serves every chunk and tile.
    __device__ __forceinline__ u32x4 load16(uint32_t lane_off, uint32_t off) const {
        if constexpr (ROPE) {
            // the clamped difference is a vector instruction: read back as a scalar
            // so that the resource stays in scalar registers
            const uint32_t left = __builtin_amdgcn_readfirstlane(bytes > off ? bytes - off : 0u);
            return buf_load16(make_rsrc(base + off, left), lane_off);
        }
        else
            return buf_load16(make_rsrc(base, bytes), lane_off + off);
    }
};

// The cos/sin values a lane needs to rotate its Q chunks: frequencies 16c + 8h .. +7
// for chunks c < D/32 of the row's table entries. Loaded on their own so that a
// kernel can issue them early and rotate later.
template <int D>
struct QRopeRow {
    f32x4 c[D / 32][2], s[D / 32][2];
    __device__ __forceinline__ void load(const float* cs_row, const float* sn_row, int h) {
#pragma unroll
        for (int k = 0; k < D / 32; ++k) {
            const int i0 = 16 * k + 8 * h;
            c[k][0] = *reinterpret_cast<const f32x4*>(cs_row + i0);
            c[k][1] = *reinterpret_cast<const f32x4*>(cs_row + i0 + 4);
            s[k][0] = *reinterpret_cast<const f32x4*>(sn_row + i0);
            s[k][1] = *reinterpret_cast<const f32x4*>(sn_row + i0 + 4);
        }
    }
};

// Rotate the Q chunks a lane holds: chunk c (dims 16c + 8h .. +7) pairs with chunk
// c + D/32 (the same dims + D/2). The rotated values are rounded to fp16 (11-bit
// significand; bfloat16 would add an input-sized rounding whose effect on the
// outputs grows with the scores), so the products that take them run on fp16.
template <int D>
__device__ __forceinline__ void rope_rotate_q(u32x4 (&qr)[D / 16], const QRopeRow<D>& tab) {
    constexpr int DC = D / 16;
#pragma unroll
    for (int c = 0; c < DC / 2; ++c) {
        const f32x4 c0 = tab.c[c][0], c1 = tab.c[c][1], s0 = tab.s[c][0], s1 = tab.s[c][1];
        const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
        const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const u32x4 a = qr[c], b = qr[c + DC / 2];
        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
        uint32_t ra[4], rbw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float a0 = bf16_lo(aw[t]), a1 = bf16_hi(aw[t]), b0 = bf16_lo(bw[t]), b1 = bf16_hi(bw[t]);
            const float c_0 = cv[2 * t], c_1 = cv[2 * t + 1], s_0 = sv[2 * t], s_1 = sv[2 * t + 1];
            ra[t] = pack_f16(a0 * c_0 - b0 * s_0, a1 * c_1 - b1 * s_1);
            rbw[t] = pack_f16(b0 * c_0 + a0 * s_0, b1 * c_1 + a1 * s_1);
        }
        qr[c] = u32x4{ra[0], ra[1], ra[2], ra[3]};
        qr[c + DC / 2] = u32x4{rbw[0], rbw[1], rbw[2], rbw[3]};
    }
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_as_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

}  // namespace tca
