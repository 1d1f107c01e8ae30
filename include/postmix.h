/*
 * postmix.h -- C ABI of the fused inverse-RoPE + VHA postmix library for
 * AMD Instinct MI355X (gfx950).  Library: libpostmix.so.
 *
 * The operation (PaddleFleet PR #1772, "Fuse HCA inverse RoPE into the VHA
 * postmix, and the sparse-attention KV index remap", PR body item 1 and the
 * description's part 一):  the HCA layer undoes the rotary position embedding
 * (RoPE) on the trailing pe channels of each head of the attention output O
 * and feeds the result to the ungrouped VHA postmix, an [nh,nh] matrix that
 * mixes heads.  Because the rotation acts on channels only and the mix
 * contracts heads, the channel axis is a pure N dimension and the two commute;
 * this library never materialises inv_rope(O).
 *
 *   forward        Y[s,g,c]  = sum_h W[g,h] * inv_rope(O)[s,h,c]
 *   input grad     dO[s,h,:] = rope( sum_g W[g,h] * dY[s,g,:] )
 *   weight grad    dW[g,h]   = sum_s sum_c dY[s,g,c] * inv_rope(O)[s,h,c]
 *                  (the pages' dM[h,h'] = sum_{t,c} dOut[t,h,c]*O_roped[t,h',c])
 *
 * RoPE convention (a reading; the pages name RoPE but do not print it):
 * rotate-half pairs (nope+i, nope+pe/2+i), i < pe/2, angle
 * phi = position * theta^(-2i/pe).  rope turns each pair by +phi:
 *   (a, b) -> (a cos - b sin, b cos + a sin);  inv_rope turns it by -phi.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - bf16 tensors are passed as raw bfloat16 bit patterns (uint16_t).
 *  - Activations O, Y, dY, dO: [sq, nh, nope+pe], row-major, channel fastest,
 *    the pe channels trailing each head.  Batch is folded into sq.
 *  - W, dW: [nh, nh] row-major, W[g,h] with g the OUTPUT head (matmul(M, X)).
 *  - rope_cos, rope_sin: fp32 [table_rows, pe/2]; row r holds position r.
 *  - positions: int32 [sq]; row s of O uses table row positions[s].  Values
 *    outside [0, table_rows) are clamped on the device (never read out of
 *    bounds); callers must not rely on clamping.
 *  - All pointers are DEVICE pointers, owned by the caller.  The library
 *    allocates, frees and synchronises nothing; work is enqueued on `stream`
 *    (a hipStream_t; NULL = the null stream) and the call returns at once.
 *  - Outputs are overwritten, never accumulated.  Inputs are not modified.
 *    In-place operation is not supported: an output range that overlaps an
 *    input range is rejected (postmix_kv_index_remap alone allows out == idx).
 *  - Limits: 1 <= nh <= 128; nope >= 0 with nope % 8 == 0; pe >= 0 with
 *    pe % 16 == 0; 0 < nope + pe <= 2^24; sq >= 0; sq * nh * (nope + pe)
 *    <= 2^40 elements, so any tensor that fits in device memory.  sq == 0 is
 *    a successful no-op.  The pages' shapes (nh = 3, 4, 64; 448 + 64 and
 *    48 + 16 channels) and the head counts up to 128 lie inside.  Why: one
 *    16-byte vector holds 8 channels, and each rotation half (pe/2 channels)
 *    and the nope range are whole vectors; W's rows and its MFMA fragments
 *    are staged for up to 128 heads; in-token offsets fit 31 bits.
 *  - Activation, table and workspace pointers must be 16-byte aligned; W must
 *    be 2-byte aligned (for nh of 32, 64 or 128 the tiled kernels read W in
 *    16-byte vectors and are used only when W is 16-byte aligned; other head
 *    counts read W element by element).
 *  - Return 0 on success, else a negative PM_ERR_* code; a thread-local
 *    message naming the offending argument is available from
 *    postmix_last_error().  Arguments are validated before any HIP call.
 *  - Calls are reentrant.  Concurrent postmix_bwd_dw / postmix_bwd calls need
 *    distinct workspaces.
 */
#ifndef POSTMIX_H
#define POSTMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pm_bf16;

enum {
    PM_OK = 0,
    PM_ERR_NULL = -1,      /* a required pointer is NULL                      */
    PM_ERR_SHAPE = -2,     /* sizes outside the limits above                  */
    PM_ERR_ALIGN = -3,     /* a pointer is not 16-byte aligned                */
    PM_ERR_OVERLAP = -4,   /* an output overlaps an input                     */
    PM_ERR_WORKSPACE = -5, /* workspace smaller than postmix_bwd_dw_workspace_bytes */
    PM_ERR_DEVICE = -6,    /* current device is not gfx950                    */
    PM_ERR_HIP = -7        /* a HIP runtime or launch error                   */
};

/*
 * Forward.  Y = inv_rope(W . O) per token, which equals W . inv_rope(O)
 * (PR #1772 body item 1: the nope columns are mixed directly; the pe columns
 * are rotated after the mix, in fp32 registers).  bf16 in, fp32 accumulate,
 * bf16 (round-to-nearest-even) out.
 *   O         [sq, nh, nope+pe] bf16, read
 *   W         [nh, nh] bf16, read
 *   rope_cos, rope_sin  [table_rows, pe/2] fp32, read (may be NULL if pe == 0)
 *   positions [sq] int32, read (may be NULL if pe == 0)
 *   Y         [sq, nh, nope+pe] bf16, written
 */
int postmix_fwd(const pm_bf16 *O, const pm_bf16 *W, const float *rope_cos,
                const float *rope_sin, int64_t table_rows,
                const int32_t *positions, int64_t sq, int32_t nh, int32_t nope,
                int32_t pe, pm_bf16 *Y, void *stream);

/*
 * Backward, input gradient.  dO = rope(W^T . dY) per token: the gradient of
 * the head mix (PR #1772, follow-up commit: the backward hands the gradient
 * through the GEMM's matmul_grad and then the RoPE backward), with the
 * transposed (+phi) rotation applied in fp32 registers.
 *   dY [sq, nh, nope+pe] bf16, read;  dO [sq, nh, nope+pe] bf16, written.
 *   Other arguments as postmix_fwd.
 */
int postmix_bwd_dx(const pm_bf16 *dY, const pm_bf16 *W, const float *rope_cos,
                   const float *rope_sin, int64_t table_rows,
                   const int32_t *positions, int64_t sq, int32_t nh,
                   int32_t nope, int32_t pe, pm_bf16 *dO, void *stream);

/*
 * Bytes of device workspace postmix_bwd_dw and postmix_bwd need for this
 * shape (a multiple of 256).  Not on the pages: it serves this library's
 * reading of their determinism requirement (backward reductions without
 * atomics that repeat bit for bit, PaddleFleet PR #1776; the weight gradient
 * dM[h,h'] = sum_{t,c} ... of PR #1772, description part 一).  Each token
 * block (and, for very wide rows, each channel span of it) writes one nh x nh
 * fp32 partial here, and a fixed-order tree adds them; the size is that of
 * the larger of the two partitions the calls may use.  Depends on
 * (sq, nh, nope, pe) only.  Returns 0 for sq == 0 and for shapes outside the
 * limits.
 */
size_t postmix_bwd_dw_workspace_bytes(int64_t sq, int32_t nh, int32_t nope,
                                      int32_t pe);

/*
 * Backward, weight gradient.  dW[g,h] = sum over tokens s and channels c of
 * dY[s,g,c] * inv_rope(O)[s,h,c] (PR #1772 description part 一: the weight
 * gradient contracts the full channel axis and cannot be split).
 * Deterministic: token blocks of equal size up to one token (a function of
 * the shape only) each produce an fp32 partial; the partials are summed in a
 * fixed pairwise tree.
 * No atomics; repeated calls give bitwise-identical dW (the atomic-free
 * principle of PaddleFleet PR #1776, "deterministic TileLang backend for
 * absorbed-MQA sparse backward").  The rotated pe operand is split into a
 * bf16 high part and a bf16 low correction (the compensated product of
 * tilelang-ascend PR #1640), both accumulated in fp32.
 * Accuracy: each element of a partial is one fp32 chain of k-steps (16
 * channels of one token each), whose norm-wise relative error grows like
 * 2^-24 * sqrt(length).  No chain is longer than 2^14 k-steps: blocks whose
 * tokens would exceed that are made smaller, and a token wider than 2^18
 * channels is split into channel spans with a partial each (one token of
 * 2^24 channels, a single 2^20-step chain, had measured 1.05e-4 relative;
 * the production blocks take 2^10 steps and are partitioned as before).
 *   dY, O     [sq, nh, nope+pe] bf16, read
 *   dW        [nh, nh] fp32, written
 *   workspace device scratch of workspace_bytes >= postmix_bwd_dw_workspace_bytes;
 *             clobbered.  May be NULL when that size is 0.
 */
int postmix_bwd_dw(const pm_bf16 *dY, const pm_bf16 *O, const float *rope_cos,
                   const float *rope_sin, int64_t table_rows,
                   const int32_t *positions, int64_t sq, int32_t nh,
                   int32_t nope, int32_t pe, float *dW, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Backward, both gradients in one call: dO as postmix_bwd_dx and dW as
 * postmix_bwd_dw, from a single pass over dY and O where the shape allows
 * (nope + pe a multiple of 128 and at most 2^24, pe <= 128, W 16-byte
 * aligned if nh is 64 or 128, and nh <= 64 with at most 32 tokens per 64-row chunk (for nh = 1
 * that needs pe >= 64, or pe >= 32 with 128-channel chunks, i.e. nope + pe
 * not a multiple of 256), or 64 < nh <= 128 with pe and nope multiples of
 * 32): each (token, channel chunk) of dY and O is read from HBM
 * once and feeds both the head-mix gradient and the weight-gradient partials.  That is one full read of dY
 * fewer than the two separate calls.  Other shapes run the two separate
 * computations.
 * dO is bitwise the same as postmix_bwd_dx's; dW is deterministic (token
 * blocks fixed by the shape, about half the size of postmix_bwd_dw's, and the
 * same fixed-order reduction), but it sums in a different order than
 * postmix_bwd_dw, so the two may differ in the last bits.
 *   dY, O [sq, nh, nope+pe] bf16, read;  W [nh, nh] bf16, read
 *   dO    [sq, nh, nope+pe] bf16, written;  dW [nh, nh] fp32, written
 *   workspace as postmix_bwd_dw (postmix_bwd_dw_workspace_bytes bytes).
 */
int postmix_bwd(const pm_bf16 *dY, const pm_bf16 *O, const pm_bf16 *W,
                const float *rope_cos, const float *rope_sin, int64_t table_rows,
                const int32_t *positions, int64_t sq, int32_t nh, int32_t nope,
                int32_t pe, pm_bf16 *dO, float *dW, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 * postmix_bwd without the workspace argument: the same computation, kernels
 * and partition (dO and dW are bitwise postmix_bwd's), with the weight-
 * gradient partials in a static device array of the library instead of a
 * caller workspace.  Allocates, frees and synchronises nothing.
 *   - The array is 32 MiB on each GPU the library runs on, held until the
 *     process ends (the production shape needs 16 MiB, 128 heads at 8192 or
 *     16384 tokens 32 MiB).  A shape whose partials need more
 *     (postmix_bwd_dw_workspace_bytes > 32 MiB) is rejected with
 *     PM_ERR_WORKSPACE before any device call; use postmix_bwd there.
 *   - Every call on one GPU uses that GPU's array: calls that overlap on one
 *     GPU (several streams, or several host threads) race and must be
 *     serialised by the caller.  Each call overwrites every partial it reads,
 *     so nothing carries over between calls.
 *   Other arguments, errors and limits as postmix_bwd.
 */
int postmix_bwd_noalloc(const pm_bf16 *dY, const pm_bf16 *O, const pm_bf16 *W,
                        const float *rope_cos, const float *rope_sin,
                        int64_t table_rows, const int32_t *positions, int64_t sq,
                        int32_t nh, int32_t nope, int32_t pe, pm_bf16 *dO,
                        float *dW, void *stream);

/*
 * RoPE tables from theta: row r (position r), column i < pe/2:
 *   cos_out[r, i] = cos(r * theta^(-2i/pe)),  sin_out likewise,
 * with the angle formed and evaluated in fp64, then rounded to fp32.
 * The pages state the problem with RoPE on the trailing qk_pos_emb_head_dim
 * channels (PR #1772 body item 1) but print neither its frequencies nor its
 * precision; both are readings: the usual frequency ladder over the pe
 * channels, and an fp64 angle (an fp32 position * frequency product is off
 * by up to ~1.2e-3 rad at positions near 32767, which moves outputs past the
 * forward tolerance).  The kernels take the tables, not theta, so callers
 * with other frequencies pass their own.
 * cos_out, sin_out: [table_rows, pe/2] fp32 device buffers, written.
 */
int postmix_rope_table(double theta, int32_t pe, int64_t table_rows,
                       float *cos_out, float *sin_out, void *stream);

/*
 * Full-width rotary embedding, out of place: the tensor the unfused route of
 * PR #1772 materialises (body item 1) and its final backward rebuilds
 * (rope_full_out_of_place, follow-up commit).  Provided so that route can be
 * run on this GPU next to the fused one; the fused entry points never need it.
 *   direction = -1: Out = inv_rope(X);  +1: Out = rope(X).
 *   X, Out [sq, nh, nope+pe] bf16 (RNE), nope channels copied; other
 *   arguments as postmix_fwd.  Out must not overlap X.
 */
int postmix_rope_apply(const pm_bf16 *X, const float *rope_cos,
                       const float *rope_sin, int64_t table_rows,
                       const int32_t *positions, int64_t sq, int32_t nh,
                       int32_t nope, int32_t pe, int32_t direction, pm_bf16 *Out,
                       void *stream);

/*
 * KV column index remap (PR #1772 body item 2, "sparse_attn_global_kv_idx_
 * remap_fusion", and description part 二): the sparse-attention index table
 * [rows = b*sq, topk] int32 holds per-batch-local KV column indices; the
 * flat-global index of row r (batch r / sq) is idx + batch * seqlen_kv.
 *   out[r, k] = idx[r, k] >= 0 ? idx[r, k] + (r / sq) * seqlen_kv : pad_value
 * Negative entries are padding (a reading: the pages name the unfused route's
 * steps, a fill, a >= 0 test, a batch arange, an expand, a scale, an add and
 * a select, but not the fill value; it is the caller's pad_value here).
 *   idx [rows, topk] int32 device, read;  out [rows, topk] int32 device,
 *   written; out == idx (in place) is allowed, a partial overlap is not.
 * rows % sq == 0; (rows / sq) * seqlen_kv must fit in int32 (valid entries
 * are expected below seqlen_kv; larger ones wrap as int32 arithmetic does).
 * 4-byte alignment; 16-byte alignment and topk % 4 == 0 take the vector path.
 */
int postmix_kv_index_remap(const int32_t *idx, int64_t rows, int64_t sq,
                           int64_t topk, int64_t seqlen_kv, int32_t pad_value,
                           int32_t *out, void *stream);

/* Static text for a PM_* code. */
const char *postmix_status_string(int status);

/* Message for the last failing call on this thread ("" if none). */
const char *postmix_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* POSTMIX_H */
