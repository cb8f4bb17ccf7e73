/*
 * tca.h -- causal, GQA-capable tiled attention (forward and backward) for
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The operation is the tiled FlashAttention of the NanoEuler blog page
 * (section "Tiled FlashAttention": one block per query tile, a loop over K/V
 * tiles staged in on-chip memory, a Q*K^T tile product, an online softmax
 * update and an output accumulation), extended as follows:
 *   - causal masking (the model is a decoder-only transformer, section
 *     "Architecture Deep Dive"): query i attends to keys j <= i;
 *   - grouped-query attention (config "num_heads": 12, "num_kv_heads": 4 in
 *     section "Build and Run"; "GQA" in the FAQ): query head hq reads KV head
 *     hq / (Hq / Hkv), so consecutive query heads share one KV head;
 *   - the log-sum-exp of every query row is saved for the backward;
 *   - a hand-derived backward (the pages hand-write every backward pass,
 *     section "Hand-written Backpropagation"): D = rowsum(dO o O), P
 *     recomputed from the saved log-sum-exp, dS = P o (dP - D), and dQ, dK, dV.
 *
 * Definitions (for every batch b, query head hq, query row i):
 *   s_ij   = scale * <q_i, k_j>                 j visible: j <= i if causal, else all j
 *   lse_i  = log(sum_j exp(s_ij))               natural logarithm
 *   o_i    = sum_j exp(s_ij - lse_i) * v_j
 *   dv_j   = sum over hq in the group, i     of P_ij * dO_i
 *   dq_i   = scale * sum_j P_ij (dP_ij - D_i) k_j,   dP_ij = <dO_i, v_j>, D_i = <dO_i, o_i>
 *   dk_j   = scale * sum over hq in the group, i of P_ij (dP_ij - D_i) q_i
 *
 * Layout: every tensor is contiguous row-major. q, o, dO, dq: [B, Hq, N, d];
 * k, v, dk, dv: [B, Hkv, N, d]; lse: [B, Hq, N]. The head dimension d is the
 * fastest-moving index.
 *
 * Precision: inputs q, k, v, dO are float32 (ATTN_F32) or bfloat16 (ATTN_BF16)
 * (`dtype`). Outputs o, dq, dk, dv are float32 or bfloat16 (`out_dtype`); lse
 * is always float32. Every result is formed in float32 and, for bfloat16
 * outputs, rounded to nearest even only when it is stored: o in bfloat16 is
 * exactly the float32 o rounded. The backward takes o in `out_dtype`, as
 * attn_fwd wrote it, and forms D = rowsum(dO o O) from those values (what a
 * bfloat16 trainer holds). bfloat16 outputs serve the trainer step that follows
 * (the pages' hand-written GPT-2 trainer consumes these tensors); their extra
 * error is one bfloat16 rounding (relative 2^-9) per element. With ATTN_F32 every step is
 * computed in float32. With ATTN_BF16 and d in {64, 128} every product runs on
 * the matrix cores with float32 accumulation. Products of two inputs take them
 * as they are: in the forward Q*K^T is a bf16 product, in the backward dO*V^T
 * (dQ phase) is bf16 and the recomputed Q*K^T (both phases) and dO*V^T (dK/dV
 * phase) are fp16 products of the inputs converted to fp16, which is exact for
 * |x| >= 2^-14 (inputs must satisfy |x| < 65504). The probabilities P and the
 * score gradient dS are rounded to fp16 (11-bit significand) for the products
 * that consume them (P*V, P^T*dO, dS*K, dS^T*Q), whose other operand is
 * converted to fp16 likewise; dS = P o (dP - D) must therefore stay within the
 * fp16 range (|dS| < 65504, which |P| <= 1 leaves to dP = dO*V^T and D), and
 * values below 2^-14 lose precision as fp16 subnormals. bf16 inputs with d in
 * {16, 32} are computed in float32.
 *
 * Memory ownership: the caller owns every buffer. All tensor pointers are
 * device memory (hipMalloc or equivalent), 16-byte aligned, and must stay
 * alive until the work enqueued on `stream` completes. The library allocates
 * no memory and keeps no state between calls; calls are thread-safe.
 *
 * Asynchrony: every entry point validates its arguments, enqueues kernels on
 * `stream` (a hipStream_t; NULL means the default stream) and returns. Results
 * are valid after the caller synchronises with the stream.
 *
 * Errors: on any non-OK status nothing has been enqueued and no output has
 * been written, except ATTN_EHIP, which reports a HIP launch error after
 * enqueueing began. No exception crosses this interface and nothing is
 * printed. Inputs and outputs must not alias.
 *
 * Invalid dtype or out_dtype codes give ATTN_EINVAL.
 *
 * Supported shapes: B >= 0, N >= 0 (B*N == 0 is a no-op that returns ATTN_OK
 * and ignores every pointer), Hq >= 1, Hkv >= 1, Hq % Hkv == 0,
 * d in {16, 32, 64, 128}, (N+64)*d < 2^31, B*Hq*N < 2^31, causal in {0, 1},
 * scale finite. Any finite scale follows the definitions above, including 0
 * (every visible key gets the same weight; dq = dk = 0) and negative values
 * (masked keys stay excluded: the matrix-core kernels form the scores as
 * |scale| * <sgn(scale) q_i, k_j>, exactly equal to scale * <q_i, k_j>).
 */
#ifndef TCA_H
#define TCA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_dtype {
    ATTN_F32 = 0,   /* float32  */
    ATTN_BF16 = 1   /* bfloat16 */
} attn_dtype;

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_EINVAL = 1,        /* invalid argument: null or misaligned pointer, bad size, bad flag */
    ATTN_EUNSUPPORTED = 2,  /* valid but not supported (head dimension) */
    ATTN_EHIP = 3,          /* the HIP runtime reported an error while enqueueing */
    ATTN_ESCRATCH = 4       /* attn_decode_noalloc: the call needs more than its fixed scratch array */
} attn_status;

/* Version of this interface; bumped on any change (2: the out_dtype argument;
 * 3: attn_decode_noalloc and ATTN_ESCRATCH; 4: the k_rot argument of
 * attn_fwd_rope and attn_bwd_rope). */
int attn_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* attn_status_str(attn_status s);

/* Workspace bytes attn_fwd needs for these sizes (currently 0 for every
 * shape; a NULL workspace is accepted when this returns 0). */
size_t attn_fwd_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int N, int d);

/* Forward: o and lse from q, k, v.
 *   q [B,Hq,N,d], k and v [B,Hkv,N,d] in `dtype`;
 *   o [B,Hq,N,d] in `out_dtype` and lse [B,Hq,N] float32 are fully overwritten.
 * This is the tile loop of the "Tiled FlashAttention" section: per query tile,
 * K/V tiles in on-chip memory, Q*K^T, online softmax, output accumulation; the
 * causal variant visits only the K/V tiles at or below the diagonal. */
attn_status attn_fwd(attn_dtype dtype, attn_dtype out_dtype,
                     const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     void* stream);

/* Workspace bytes attn_bwd (and its two phases) need: the float32 row
 * statistic D = rowsum(dO o O) (B*Hq*N floats); for bf16 inputs with d in
 * {64, 128} also lse in base-2 units (B*Hq*N floats) and fp16 copies of q and
 * dO (B*Hq*N*d halves each), which the dQ phase writes and the dK/dV phase
 * reads. Each part is rounded up to 256 bytes. */
size_t attn_bwd_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int N, int d);

/* Backward: dq, dk, dv from q, k, v, the forward's o and lse, and dO.
 *   q, k, v, dO in `dtype`; o (in `out_dtype`) and lse exactly as written by
 *   attn_fwd with the same q, k, v, dtypes, sizes, causal flag and scale;
 *   dq [B,Hq,N,d], dk and dv [B,Hkv,N,d] in `out_dtype`, fully overwritten.
 *   `workspace` holds at least attn_bwd_workspace_bytes(...) bytes of device
 *   memory; its contents on entry do not matter. Every output element is
 *   written exactly once (no atomics), so dq, dk and dv are bitwise
 *   reproducible for fixed inputs.
 * Equivalent to attn_bwd_dq followed by attn_bwd_dkdv on `stream`. */
attn_status attn_bwd(attn_dtype dtype, attn_dtype out_dtype,
                     const void* q, const void* k, const void* v,
                     const void* o, const float* lse, const void* dO,
                     void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                     void* stream);

/* First phase of attn_bwd, query-tile parallel: writes D = rowsum(dO o O)
 * (and, for bf16 inputs with d in {64, 128}, lse in base-2 units and fp16
 * copies of q and dO) into `workspace`, then dq (recomputing P and dP for each
 * visible K/V tile). dk and dv are not touched. Arguments as for attn_bwd. */
attn_status attn_bwd_dq(attn_dtype dtype, attn_dtype out_dtype,
                        const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* dO,
                        void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                        void* stream);

/* Second phase of attn_bwd, K/V-tile parallel: dk and dv, reading what
 * attn_bwd_dq left in `workspace`. Requires attn_bwd_dq with the same arguments to have been
 * enqueued before it on the same stream (or completed). dq is not touched.
 * Arguments as for attn_bwd. */
attn_status attn_bwd_dkdv(attn_dtype dtype, attn_dtype out_dtype,
                          const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dO,
                          void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                          void* stream);

/* Element strides of a [B, H, N, d] tensor whose head dimension is contiguous:
 * element (b, h, n, c) sits at b*stride_b + h*stride_h + n*stride_n + c. For
 * q, k, v taken from one fused projection buffer [B, N, (Hq + 2*Hkv)*d]:
 * stride_b = N*W, stride_h = d, stride_n = W with W = (Hq + 2*Hkv)*d (k and v
 * start Hq*d and (Hq+Hkv)*d elements in). A NULL layout pointer means the
 * contiguous [B, H, N, d] layout. */
typedef struct attn_layout {
    long long stride_b, stride_h, stride_n;
} attn_layout;

/* Workspace bytes attn_fwd_rope / attn_bwd_rope need: contiguous copies of q,
 * k (rotated) and v in `dtype`; for the backward also float32 gradients, a
 * float32 copy of o for bfloat16 outputs, and attn_bwd's own workspace. Each
 * part rounded up to 256 bytes. */
size_t attn_fwd_rope_workspace_bytes(attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d);
size_t attn_bwd_rope_workspace_bytes(attn_dtype dtype, attn_dtype out_dtype, int B, int Hq, int Hkv, int N, int d);

/* Forward with rotary position embedding on q and k and strided inputs (the
 * blog page's FAQ lists RoPE among the trainer's techniques; q, k, v come from
 * one fused projection). Row n of every head sits at position n; with
 * rope_cos/rope_sin ([N, d/2] float32 device tables, normally cos/sin of
 * n * base^(-2i/d)) the pairs (x_i, x_{i+d/2}) of q and k are rotated to
 * (x_i cos - x_{i+d/2} sin, x_{i+d/2} cos + x_i sin) before the attention;
 * both NULL means no rotation (strided input only). d must be even for
 * tables. q, k, v are read through their layouts (NULL: contiguous); o and lse
 * are written as by attn_fwd. With bfloat16 inputs, d in {64, 128} and tables,
 * the matrix-core forward reads q through its strides and rotates it in
 * registers and reads v in place (each through an exact contiguous copy in
 * `workspace` instead when its rows do not start on 16-byte boundaries, or v's
 * rows are less than d elements apart); only k is rotated into a contiguous copy
 * in `workspace` (at least attn_fwd_rope_workspace_bytes), once for every query
 * tile that reads it. On that path the rotated q and k are rounded to fp16
 * (11-bit significand; |x| < 65504) and Q*K^T is an fp16 product, so the
 * rotation adds an eighth of an input rounding. Otherwise (float32 inputs, d in
 * {16, 32}, or no tables) the rotated q, k (rounded to `dtype`) and a contiguous
 * v are staged there and attn_fwd's kernels run on them. Pointers to
 * strided tensors need element alignment only; o and lse as for attn_fwd.
 * Strides must be >= 0 and the caller's buffers must hold every addressed
 * element.
 * k_rot: NULL, or device memory for B*Hkv*N*d elements of `dtype`'s size (2
 * bytes for bfloat16, 4 for float32), 16-byte aligned. The rotated keys (k itself
 * without tables), contiguous [B, Hkv, N, d] in the precision the path computes
 * with (fp16 on the matrix-core path, else `dtype`), are then written there
 * instead of into `workspace`, on every path, so that a training step can keep
 * them as a saved activation and hand them to attn_bwd_rope, which then skips its
 * own rotation of k. The buffer's contents are for attn_bwd_rope only. The
 * workspace size does not change. */
attn_status attn_fwd_rope(attn_dtype dtype, attn_dtype out_dtype,
                          const void* q, const attn_layout* q_layout,
                          const void* k, const attn_layout* k_layout,
                          const void* v, const attn_layout* v_layout,
                          const float* rope_cos, const float* rope_sin, void* k_rot,
                          void* o, float* lse,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                          void* stream);

/* Backward of attn_fwd_rope: dq, dk, dv with respect to the UNROTATED q, k and
 * to v, written through their layouts (NULL: contiguous) in `out_dtype`. o and
 * lse exactly as attn_fwd_rope wrote them (contiguous), dO contiguous in
 * `dtype`. dq and dk are turned back by the transpose rotation
 * (g_i cos + g_{i+d/2} sin, g_{i+d/2} cos - g_i sin) with a single rounding to
 * `out_dtype`. On the matrix-core path of attn_fwd_rope, k is rotated into
 * `workspace` again; the dQ pass reads q and v through their strides and stores
 * dq turned back through dq's (through a contiguous copy scattered afterwards
 * when dq's rows are not 16-byte aligned), and the dK/dV pass reads v in place
 * and stores dk turned back, and dv, through their layouts. Otherwise the
 * rotated copies are staged, attn_bwd's kernels write float32 gradients into
 * `workspace`, and one launch turns dq, dk back and scatters all three.
 * k_rot: NULL, or the k_rot that attn_fwd_rope filled for the same k, tables
 * and sizes, unchanged since (16-byte aligned). The backward then reads the
 * rotated keys from it instead of rotating k again, and does not read k (which
 * must still be a valid pointer). Given anything else the results are
 * undefined. */
attn_status attn_bwd_rope(attn_dtype dtype, attn_dtype out_dtype,
                          const void* q, const attn_layout* q_layout,
                          const void* k, const attn_layout* k_layout,
                          const void* v, const attn_layout* v_layout,
                          const float* rope_cos, const float* rope_sin, const void* k_rot,
                          const void* o, const float* lse, const void* dO,
                          void* dq, const attn_layout* dq_layout,
                          void* dk, const attn_layout* dk_layout,
                          void* dv, const attn_layout* dv_layout,
                          void* workspace, size_t workspace_bytes,
                          int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                          void* stream);

/* Workspace bytes attn_fwd_naive needs: the score matrix, B*Hq*N*N floats. */
size_t attn_fwd_naive_workspace_bytes(int B, int Hq, int N);

/* Unoptimised forward, for teaching and as a baseline (the NanoEuler article
 * lists a "naive", unoptimised version kept to understand every step): the
 * same o and lse as attn_fwd, computed the obvious way with the whole score
 * matrix in `workspace` (at least attn_fwd_naive_workspace_bytes(B, Hq, N)
 * bytes of device memory, 16-byte aligned): S = scale * Q K^T with masked
 * entries -inf, a row softmax in place (and lse), then O = P V, each step a
 * plain kernel reading global memory directly, in float32 for every dtype.
 * Arguments, layouts, sizes and errors as for attn_fwd; also ATTN_EINVAL when
 * B*Hq*N*N >= 2^39. */
attn_status attn_fwd_naive(attn_dtype dtype, attn_dtype out_dtype,
                           const void* q, const void* k, const void* v,
                           void* o, float* lse,
                           void* workspace, size_t workspace_bytes,
                           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                           void* stream);

/* Workspace bytes attn_decode needs for these sizes: the per-split partial
 * outputs and log-sum-exps when the keys are split into more ranges than one
 * workgroup merges itself (nsplit * B*Hq*Nq * (d + 1) floats, each part rounded
 * up to 256 bytes), else 0. A function of the sizes and `dtype` only; 0 for
 * invalid sizes. */
size_t attn_decode_workspace_bytes(attn_dtype dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d);

/* Few-query attention over a key/value cache (decode): o and lse for Nq query
 * rows that are the LAST Nq positions of a sequence of Nk tokens, whose keys
 * and values are all in k and v. This is the forward used for inference (the
 * blog page's FAQ: inference works and runs on 8 GB cards), one or a few new
 * tokens per step against the cache.
 *   q [B,Hq,Nq,d], k and v [B,Hkv,Nk,d] in `dtype`; o [B,Hq,Nq,d] in
 *   `out_dtype`; lse [B,Hq,Nq] float32 (natural log), fully overwritten.
 *   Query row i sits at sequence position Nk - Nq + i: causally it sees keys
 *   j <= Nk - Nq + i (bottom-right alignment); causal = 0 sees all Nk keys.
 *   With Nq = Nk the result is attn_fwd's (up to rounding order).
 *   GQA head map, scale and the definitions of o and lse as for attn_fwd.
 * The keys are split into ranges processed in parallel, whose partial outputs
 * are merged through their log-sum-exps. When a call has enough (batch, KV
 * head, query-row chunk) groups, a group's ranges are the waves of one workgroup
 * and merge in on-chip memory: one launch, no workspace. On the vector units
 * that takes at least 256 groups and up to 16 ranges per group (8 when a wave
 * holds 8 query rows, or 4 float32 ones); on the matrix cores (below) at least
 * 128 chunks of 32 rows, whose 8 waves take the key ranges in turn. With fewer
 * groups, bf16 calls at d = 128
 * with 8 or more query rows per KV head whose partials fit
 * ATTN_DECODE_SCRATCH_BYTES take the matrix-core ranges even where the vector
 * units would merge in a workgroup (measured faster). Otherwise each range writes its
 * partial output and log-sum-exp into `workspace` (at least
 * attn_decode_workspace_bytes(...) bytes of device memory, 16-byte aligned;
 * NULL allowed when that is 0) and a second kernel merges them. Arithmetic:
 * bf16 inputs at d = 64 or 128 with at least 3 query rows per KV head (Hq/Hkv *
 * Nq; 2 at d = 64) run on the matrix cores as
 * the forward does (bf16 Q K^T, fp32 accumulation, probabilities rounded to fp16
 * for P V, so |x| < 65504 is required of v as of attn_fwd's inputs); every other
 * call computes in float32 on the vector units.
 * Sizes: B >= 0, Nq >= 0 (B*Nq == 0 is a no-op), Nq <= Nk, Hq % Hkv == 0,
 * d in {16, 32, 64, 128}, (Nk+256)*d*4 < 2^31; otherwise ATTN_EINVAL (or
 * ATTN_EUNSUPPORTED for d). Results are bitwise reproducible. */
attn_status attn_decode(attn_dtype dtype, attn_dtype out_dtype,
                        const void* q, const void* k, const void* v,
                        void* o, float* lse,
                        void* workspace, size_t workspace_bytes,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                        void* stream);

/* Bytes of the fixed device array that attn_decode_noalloc uses as scratch. */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/* attn_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation). Arguments, results and errors are attn_decode's; the results
 * are bitwise those of attn_decode. The split partials go to a file-scope device
 * array of ATTN_DECODE_SCRATCH_BYTES bytes that each GPU the library runs on holds
 * until the process ends (its address is looked up on the first call on a device,
 * with that device current; `stream` must belong to the current device). A call
 * whose attn_decode_workspace_bytes(...) exceeds ATTN_DECODE_SCRATCH_BYTES returns
 * ATTN_ESCRATCH and enqueues nothing. The call itself allocates nothing. Every call
 * on one GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, or host threads) race and must be serialised by the caller. */
attn_status attn_decode_noalloc(attn_dtype dtype, attn_dtype out_dtype,
                                const void* q, const void* k, const void* v,
                                void* o, float* lse,
                                int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float scale,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TCA_H */
