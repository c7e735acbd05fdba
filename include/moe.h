/*
 * moe.h - C ABI of the MI355X (gfx950) mixture-of-experts layer forward.
 *
 * One MoE layer forward on one GPU, in four calls that run back to back on a
 * HIP stream (deepmox ch.5 "The network becomes part of the forward pass": a
 * forward chunk dispatches tokens to experts, runs the expert MLP, combines;
 * zenaique "Why all to all dominates MoE step time": two exchanges per
 * forward, dispatch and combine):
 *
 *   moe_route       gate logits, sqrt(softplus) affinities, bias-adjusted
 *                   node-limited top-k, renormalised gate weights, per-block
 *                   expert histogram
 *   moe_dispatch    per-expert counts, exclusive scan, stable permutation,
 *                   packed expert-contiguous (= group-ordered) token rows
 *   moe_expert_ffn  grouped SwiGLU expert FFN (routed experts, or the shared
 *                   expert as one group over all tokens)
 *   moe_combine     gate-weighted sum of expert rows back in token order
 *
 * Conventions for every call
 *   - Pointers are device pointers unless marked "host".  The caller owns and
 *     allocates every buffer, including workspaces; the library never
 *     allocates, frees or synchronises, and reads no device value back to the
 *     host (data-dependent sizes such as per-expert counts stay on the device,
 *     so row buffers are sized for the worst case T*k).
 *   - Workspaces (`ws`, `ws_bytes`): device memory of at least
 *     moe_workspace_size(op, shape, dtype) bytes, 256-byte aligned, else
 *     MOE_ERR_WORKSPACE.  Calls that may execute at the same time (on other
 *     streams, or replays of captured graphs) need distinct workspaces.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) in call order.  Calls are reentrant given distinct buffers and
 *     workspaces; the library keeps no device state between calls.
 *   - Everything is row-major.  Weights are [out, in], so the reduction
 *     dimension is contiguous for both products.  bf16 is IEEE bfloat16 (bit
 *     pattern in a uint16), e4m3 is OCP E4M3FN in a uint8.
 *   - Return value: MOE_OK or a negative MOE_ERR_*.  Arguments are checked on
 *     the host before anything is launched; on an error nothing is launched
 *     and no output is touched.  MOE_ERR_HIP reports a failed launch
 *     (hipGetLastError); outputs are then undefined.  T = 0 is a no-op.
 *     Non-finite logits are outside the contract.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, inconsistent shape, bad range */
#define MOE_ERR_UNSUPPORTED (-2)  /* valid, but not a shape/dtype this library runs */
#define MOE_ERR_WORKSPACE (-3)    /* workspace smaller than *_workspace_size() */
#define MOE_ERR_HIP (-4)          /* a kernel launch failed */
#define MOE_ERR_SCRATCH (-5)      /* moe_dispatch_noalloc: the call needs more than its static scratch */

/* element types */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_E4M3 2

/* moe_route flags */
#define MOE_ROUTE_LOGITS_IN 1     /* skip the gate product: read `logits` as input */

/* moe_expert_ffn stages */
#define MOE_FFN_UP 1              /* h = silu(x W1^T) * (x W3^T)   */
#define MOE_FFN_DOWN 2            /* y = h W2^T                    */
#define MOE_FFN_ALL 3

/* moe_workspace_size operations */
#define MOE_OP_ROUTE 1
#define MOE_OP_DISPATCH 2
#define MOE_OP_EXPERT_FFN 3           /* also moe_expert_ffn_train */
#define MOE_OP_COMBINE 4
#define MOE_OP_ROUTE_BACKWARD 5
#define MOE_OP_EXPERT_FFN_BACKWARD 6

/* tokens per row of the block histogram written by moe_route */
#define MOE_ROUTE_BLOCK 64
/* fp8 scale granularity: 1 x 128 activation tiles, 128 x 128 weight blocks */
#define MOE_FP8_TILE 128

typedef void* moe_stream_t; /* hipStream_t */

/*
 * Layer shape.
 *   T tokens, d model width, E routed experts in G groups of E/G consecutive
 *   experts (group = "node" of node-limited routing: zenaique "MoE
 *   node-limited routing", definition; deepnotes "The real cluster": 4
 *   consecutive experts per GPU), at most M groups per token, k experts per
 *   token, group_topk affinities summed per group score (ceil(k/M)), d_ff
 *   expert hidden width.
 * Checked: T >= 0; d, E, G, M, k, group_topk, d_ff > 0; G divides E;
 *   M <= G; group_topk <= E/G; k <= M*E/G.
 */
typedef struct moe_shape {
  int64_t T;
  int32_t d, E, G, M, k, group_topk, d_ff;
} moe_shape;

int moe_abi_version(void);
const char* moe_status_str(int status);

/*
 * moe_workspace_size - bytes of device workspace a call needs (0: none).
 *   op     MOE_OP_*
 *   shape  the call's shape (moe_expert_ffn*: any shape; the size does not
 *          depend on it)
 *   dtype  MOE_OP_ROUTE: x's type; MOE_OP_DISPATCH: the output type (the
 *          e4m3 output needs a per-token scale table); otherwise ignored
 * MOE_OP_ROUTE covers a call with logits = NULL (the larger case; with
 * bf16 x and a split gate product both cases need the same);
 * MOE_OP_DISPATCH covers any expert range.  Returns 0 for an invalid shape
 * or op.
 */
size_t moe_workspace_size(int op, const moe_shape* shape, int dtype);

/*
 * moe_route - routing for T tokens (mastering-deepseek-v4 "MoE + Expert-
 * Parallel Overlap (Exp08)", Implemented: top-k gating over Sqrt(Softplus)
 * affinities, per-expert bias for balancing; zenaique "MoE node-limited
 * routing": at most M nodes per token).
 *   x             [T, d] in x_dtype (MOE_BF16 or MOE_F32); unused with LOGITS_IN
 *   w_gate        [d, E] fp32 router weight; unused with LOGITS_IN.  The
 *                 product runs on bf16 matrix cores and stays fp32-accurate:
 *                 w_gate is split into three bf16 planes hi + mid + lo == w
 *                 exactly (each the nearest bf16 of what the planes before it
 *                 leave), bf16 x times a plane is exact in fp32, and the
 *                 plane products accumulate in fp32 (the router is kept out of
 *                 low precision: deepnotes "The iteration loop", the FP8
 *                 recipe excludes the router gate)
 *   bias          [E] fp32 per-expert selection bias
 *   logit_offset  [E] fp32 added to every token's logits, or NULL
 *   logits        [T, E] fp32: out = x . W_g, or NULL (kept in ws, not
 *                 returned); in with MOE_ROUTE_LOGITS_IN (then required)
 *   topk_idx      [T, k] int32 out: chosen experts, biased affinity
 *                 descending, ties to the lower expert index
 *   topk_w        [T, k] fp32 out: s_j / (s_0 + s_1 + ... ) over the chosen
 *                 experts, s = unbiased affinity, left-to-right fp32 sum
 *   block_counts  [ceil(T/MOE_ROUTE_BLOCK), E] int32 out: pairs routed to each
 *                 expert within each block of MOE_ROUTE_BLOCK tokens
 * From logits on, every value is produced by a fixed operation sequence
 * (affinity = fp32 of sqrt(softplus(l)) evaluated in fp64 -- ln2 + l/2 + l*l/8
 * for |l| < 2^-14, else max(l,0) + log1p(exp(-|l|)) with a Cody-Waite exp and
 * the Goldberg log1p -- and rounded once, so it never decreases as l grows;
 * b = affinity + bias in fp32; group score = top group_topk biased affinities summed
 * largest first; top-M groups, ties to the lower group; experts outside kept
 * groups excluded), so results are reproducible bit for bit from the logits.
 * Supported: E <= 256 with E a multiple of 64 or E <= 64; E/G a multiple of
 * ceil(E/64) forming a power-of-two number of 64-lane wave lanes;
 * group_topk <= 4; k <= 16.  The matrix-core gate product needs bf16 x,
 * d % 64 == 0 and E % 64 == 0 (else fp32 vector products, same planes).
 *   ws            moe_workspace_size(MOE_OP_ROUTE, shape, x_dtype) bytes: the
 *                 planes [3, E, d] bf16 (rewritten by every call); for bf16 x
 *                 on the matrix cores the gate product runs split over its
 *                 reduction (the 3*d/64 plane-and-column steps) into S <= 8
 *                 fp32 partial products [S, T, E] that the selection sums in
 *                 order (((p0 + p1) + p2) + ...), with S chosen from T, d and E
 *                 alone, so the workspace then also holds, for S > 1, the
 *                 partial products, and for E % 256 == 0 the split's
 *                 counters; with S = 1 (or fp32 x) it holds the logits when
 *                 `logits` is NULL.  Nothing in it needs to start at zero.
 *                 Unused with LOGITS_IN (may be NULL).
 */
int moe_route(const moe_shape* shape, const void* x, int x_dtype, const float* w_gate,
              const float* bias, const float* logit_offset, float* logits, int32_t* topk_idx,
              float* topk_w, int32_t* block_counts, int flags, void* ws, size_t ws_bytes,
              moe_stream_t stream);

/*
 * moe_dispatch - pack token rows into an expert-contiguous buffer (deepmox
 * ch.5, dispatch; zenaique "Why all to all dominates": dispatch ships each
 * token's row to the holders of its k experts; shivam2003 "Worked example":
 * bytes = tokens x hidden x bytes per direction).  Only experts in
 * [e_begin, e_end) are packed (one expert-parallel rank's share; pass 0, E for
 * all).  With consecutive experts per group the buffer is group-ordered: it
 * is this GPU's all-to-all send layout.
 *   topk_idx, block_counts  from moe_route
 *   x        [T, d] in x_dtype (MOE_BF16 or MOE_F32)
 *   out_dtype  x_dtype (plain copy) or MOE_E4M3 from MOE_BF16 x (d % 128 == 0)
 *   counts   [n] int32 out, n = e_end - e_begin: pairs per local expert
 *   offsets  [n + 1] int32 out: exclusive prefix sum, offsets[0] = 0
 *   dest     [T, k] int32 out: packed row of pair (t, j), -1 if not local
 *   src      [T*k] int32 out: token of packed row r, for r < offsets[n]
 *   xp       [T*k, d] out: xp[r] = x[src[r]] (copied, or quantised to e4m3
 *            with one fp32 scale per 1 x 128 tile: scale = amax/448, or 1
 *            for an all-zero tile; code = e4m3(x / scale) rounded to
 *            nearest-even, saturating)
 *   xp_scale [d/128, T*k] fp32 out for MOE_E4M3, else ignored (may be NULL):
 *            block-major, the scale of row r's 128-column block b at
 *            xp_scale[b * T*k + r], so one block's scales are contiguous
 *            over rows (the layout moe_expert_ffn reads)
 *   ws       moe_workspace_size(MOE_OP_DISPATCH, shape, out_dtype) bytes: the
 *            per-(64-token block, expert) base rows and, for MOE_E4M3, a
 *            [d/128, T] fp32 table of each token's e4m3 scales (written once
 *            per token, then gathered into xp_scale by packed row)
 * Row numbering is stable: within an expert, rows follow token order.
 */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                 int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                 int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                 float* xp_scale, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_dispatch_noalloc - moe_dispatch without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, outputs
 * and checks as moe_dispatch; the workspace is a static array the library
 * holds on each device (8 MiB, MOE_DISPATCH_NOALLOC_SCRATCH bytes), so the
 * call allocates nothing.  A call whose workspace need
 * (moe_workspace_size(MOE_OP_DISPATCH, ...) for its expert range and output
 * type) exceeds it returns MOE_ERR_SCRATCH before anything is launched: with
 * 256 local experts that allows T up to 524288 for a bf16 or fp32 output, and
 * T up to about 34900 for the e4m3 output at d = 7168 (V3 shapes, T = 16384,
 * need 3.9 MiB).
 * Nothing in it needs to start at zero.  Every call on a device shares that
 * device's array and it keeps the last call's contents: calls that may
 * execute at the same time on one device (other streams, concurrent graph
 * replays) race on it and must use moe_dispatch with distinct workspaces.
 * The array belongs to the current device (the device of `stream`).
 */
#define MOE_DISPATCH_NOALLOC_SCRATCH 8388608  /* 8 MiB */
int moe_dispatch_noalloc(const moe_shape* shape, const int32_t* topk_idx, const int32_t* block_counts,
                         int32_t e_begin, int32_t e_end, const void* x, int x_dtype, int out_dtype,
                         int32_t* counts, int32_t* offsets, int32_t* dest, int32_t* src, void* xp,
                         float* xp_scale, moe_stream_t stream);

/*
 * moe_ffn_extra - one more group for moe_expert_ffn with buffers of its own:
 * the shared expert (mastering-deepseek-v4 "MoE + Expert-Parallel Overlap
 * (Exp08)", Implemented: shared experts are always active), computed with
 * the routed experts so its tiles fill the same launches.  Its rows are its
 * own (typically the T unpermuted token rows); types and layouts are the
 * routed groups':
 *   x [rows, d]   (+ x_scale [d/128, rows] for e4m3)   up-projection input
 *   w13 [2*d_ff, d] (+ w13_scale [2*d_ff/128, d/128]), w2 [d, d_ff]
 *                 (+ w2_scale [d/128, d_ff/128])
 *   h [rows, d_ff] (+ h_scale [d_ff/128, rows])          intermediate
 *   y [rows, d]                                          down-projection output
 * The bf16 matrix-core products take it into the routed launches (its tiles
 * after the routed ones); the other paths compute it in launches of its own
 * that follow on the stream.  Results are the same either way.
 */
typedef struct moe_ffn_extra {
  int64_t rows;
  const void* x;
  const float* x_scale;
  const void* w13;
  const float* w13_scale;
  const void* w2;
  const float* w2_scale;
  void* h;
  float* h_scale;
  void* y;
} moe_ffn_extra;

/*
 * moe_expert_ffn - grouped SwiGLU experts (mastering-deepseek-v4 Exp08,
 * Implemented: shared always-active experts plus fine-grained routed ones;
 * 6*d*d_ff flops per token-expert pair, i.e. three d x d_ff matrices).
 * Expert i processes rows [offsets[i], offsets[i+1]) of xp:
 *     h = silu(x W1_i^T) * (x W3_i^T),   y = h W2_i^T,   silu(a) = a/(1+e^-a)
 * The shared expert is the same call with n_exp = 1 over x itself
 * (offsets = {0, T}).
 *   n_exp     number of experts in this call (<= 1024)
 *   offsets   [n_exp + 1] int32 (device), non-decreasing, offsets[0] = 0,
 *             offsets[n_exp] <= max_rows
 *   max_rows  host upper bound on offsets[n_exp]: sizes the launch
 *   dtype     MOE_F32, MOE_BF16 or MOE_E4M3 (the storage type of xp, the
 *             weights and h); accumulation is fp32 throughout
 *   xp        [max_rows, d];  xp_scale [d/128, max_rows] fp32 for e4m3
 *             (block-major, as moe_dispatch writes it with max_rows = T*k)
 *   w13       [n_exp, 2*d_ff, d]: rows 0..d_ff-1 = W1 (gate), d_ff.. = W3 (up)
 *   w2        [n_exp, d, d_ff]
 *   w13_scale [n_exp, 2*d_ff/128, d/128], w2_scale [n_exp, d/128, d_ff/128]
 *             fp32 block scales for e4m3, else ignored
 *   h         [max_rows, d_ff] intermediate in dtype (bf16 for MOE_BF16);
 *             h_scale [d_ff/128, max_rows] for e4m3 (block-major)
 *   yp        [max_rows, d] out: fp32 for MOE_F32, bf16 otherwise
 *   stages    MOE_FFN_UP, MOE_FFN_DOWN or MOE_FFN_ALL
 *   extra     NULL, or one more group with its own buffers (moe_ffn_extra;
 *             rows = 0: none), for the stages asked for
 *   ws        moe_workspace_size(MOE_OP_EXPERT_FFN, ...) bytes: the ticket
 *             counters the persistent products schedule their tiles with (one
 *             set for the up and one for the down product).  It must be
 *             zero-filled before its first use; every call leaves it zero
 *             again when its kernels complete, so it can serve any number of
 *             calls in stream order (and replays of a captured graph).  Calls
 *             that may execute at the same time need distinct workspaces.
 * Supported: MOE_BF16 any d, d_ff: on the matrix cores when d % 256 == 0,
 * d_ff % 128 == 0 and d_ff >= 256, on the vector ALUs otherwise; MOE_E4M3
 * needs d % 256 == 0 and d_ff % 128 == 0 (a product whose reduction width,
 * d for the up-projection and d_ff for the down, is a multiple of 256 and
 * at least 512 runs persistent, a narrower one one tile per work-group);
 * MOE_F32 any d, d_ff.
 */
int moe_expert_ffn(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d,
                   int32_t d_ff, int dtype, const void* xp, const float* xp_scale,
                   const void* w13, const float* w13_scale, const void* w2,
                   const float* w2_scale, void* h, float* h_scale, void* yp, int stages,
                   const moe_ffn_extra* extra, void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_combine - out[t] = ysh[t] + sum_j topk_w[t,j] * yp[dest[t,j]]
 * (deepmox ch.5, combine), slots with dest = -1 skipped, summed in fp32 in
 * slot order starting from ysh (or from 0 without ysh).
 *   dest, topk_w  [T, k] from moe_dispatch / moe_route
 *   yp     [rows, d] in y_dtype (MOE_BF16 or MOE_F32)
 *   ysh    [T, d] in y_dtype (shared-expert output) or NULL
 *   out    [T, d] in out_dtype (MOE_BF16 or MOE_F32)
 *   accumulate  0: out = sum;  1: out += sum (out must be MOE_F32; one
 *               expert-parallel rank scatter-adding its share)
 */
int moe_combine(const moe_shape* shape, const int32_t* dest, const float* topk_w, const void* yp,
                int y_dtype, const void* ysh, void* out, int out_dtype, int accumulate,
                moe_stream_t stream);

/*
 * moe_quantize_rows_e4m3 - bf16 [rows, cols] -> e4m3 codes [rows, cols] with
 * one fp32 scale per 1 x 128 tile of a row, block-major [cols/128, rows] (the
 * same rule and layout as moe_dispatch's MOE_E4M3 output).  For the shared expert of the fp8 workload,
 * whose input is the unpermuted token rows.  cols must be a multiple of 128.
 */
int moe_quantize_rows_e4m3(int64_t rows, int32_t cols, const void* x, uint8_t* q, float* scale,
                           moe_stream_t stream);

/*
 * moe_quantize_blocks_e4m3 - fp32 [n, rows, cols] -> e4m3 codes
 * [n, rows, cols] with one fp32 scale per 128 x 128 block
 * [n, rows/128, cols/128] (scale = amax/448, or 1 for an all-zero block;
 * code = e4m3(w / scale), nearest-even, saturating).  Weight preparation for
 * the fp8 workload; rows and cols must be multiples of 128.
 */
int moe_quantize_blocks_e4m3(int64_t n, int32_t rows, int32_t cols, const float* w, uint8_t* q,
                             float* scale, moe_stream_t stream);

/*
 * ---------------------------------------------------------------- backward
 * The layer's backward (deepmox ch.5 "The network becomes part of the forward
 * pass": the backward carries its own communication and splits into the
 * gradient for the input and the gradient for the weights).  The pages give
 * no formulas; these are the exact derivatives of the forward above with the
 * expert selection held fixed (it is piecewise constant) and no gradient for
 * the routing bias (it steers selection and follows moe_bias_update).  Call
 * order for g = d loss / d out:
 *   moe_combine_backward     -> d_yp, d_topk_w          (d_ysh = g)
 *   moe_expert_ffn_backward  routed experts (d_yp) and the shared expert (g)
 *   moe_dispatch_backward    dx = shared-expert dx + sum over a token's rows
 *   moe_route_backward       dx += gate path, dW_g
 */

/*
 * moe_combine_backward - for out[t] = ysh[t] + sum_j w[t,j] yp[dest[t,j]]:
 *   d_yp[dest[t,j]] = topk_w[t,j] * grad_out[t]       bf16 [rows, d]
 *   d_topk_w[t,j]   = <grad_out[t], yp[dest[t,j]]>     fp32 [T, k] (0 for dest = -1)
 * yp in y_dtype, grad_out in g_dtype (MOE_BF16 or MOE_F32).  Rows of d_yp that
 * no slot points at are not written.  The dot products are reduced in a fixed
 * order (deterministic).
 */
int moe_combine_backward(const moe_shape* shape, const int32_t* dest, const float* topk_w, const void* yp,
                         int y_dtype, const void* grad_out, int g_dtype, void* d_yp, float* d_topk_w,
                         moe_stream_t stream);

/*
 * moe_expert_ffn_train - moe_expert_ffn (both stages, bf16) that also keeps
 * the pre-activations [a | u] = [x W1^T | x W3^T] (bf16 [max_rows, 2*d_ff])
 * for moe_expert_ffn_backward with MOE_BWD_AU_SAVED, which then skips
 * recomputing them.  h and yp are bit-identical to moe_expert_ffn's.
 * offsets may be NULL with n_exp = 1 (one group of max_rows rows); d and d_ff
 * multiples of 256.  ws as moe_expert_ffn's (MOE_OP_EXPERT_FFN).
 */
int moe_expert_ffn_train(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d, int32_t d_ff,
                         int dtype, const void* xp, const void* w13, const void* w2, void* h, void* au, void* yp,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

#define MOE_BWD_AU_SAVED 1  /* moe_expert_ffn_backward: au already holds [a | u] */

/*
 * moe_expert_ffn_backward - backward of the grouped SwiGLU experts
 * (y = (silu(x W1^T) * (x W3^T)) W2^T per group), bf16 products on the matrix
 * cores with fp32 accumulation:
 *   d_xp [max_rows, d]  bf16   d_yp W2 -> d_h; SwiGLU derivative; [da|du] W13
 *   dw13 [n_exp, 2*d_ff, d] fp32   [da|du]^T xp   (over each group's rows)
 *   dw2  [n_exp, d, d_ff]   fp32   d_yp^T h
 * Workspaces (caller-owned, bf16): au [max_rows, 2*d_ff] (the up-projection
 * is recomputed into it, unless flags has MOE_BWD_AU_SAVED and it holds
 * moe_expert_ffn_train's [a | u]), h [max_rows, d_ff] (d_h, then h), d_au
 * [max_rows, 2*d_ff].  offsets as moe_expert_ffn (device, [n_exp+1]); NULL with
 * n_exp = 1 means one group of max_rows rows (the shared expert on x).  Weight
 * gradients are written (not accumulated); a group with no rows gets zeros.
 * dtype must be MOE_BF16; d and d_ff multiples of 256.  ws:
 * moe_workspace_size(MOE_OP_EXPERT_FFN_BACKWARD, ...) bytes of ticket counters
 * for the recomputed up-projection, zero-filled before first use and left zero
 * by every call (as moe_expert_ffn's).
 */
int moe_expert_ffn_backward(int32_t n_exp, const int32_t* offsets, int64_t max_rows, int32_t d, int32_t d_ff,
                            int dtype, const void* xp, const void* w13, const void* w2, const void* d_yp,
                            void* au, void* h, void* d_au, void* d_xp, float* dw13, float* dw2, int flags,
                            void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_dispatch_backward - dx[t] (+)= d_extra[t] + sum_j d_xp[dest[t,j]] (slots
 * with dest = -1 skipped), fp32 [T, d].  d_xp [rows, d] and d_extra [T, d] (or
 * NULL) in xp_dtype (MOE_BF16 or MOE_F32).  accumulate = 1 adds into dx.
 */
int moe_dispatch_backward(const moe_shape* shape, const int32_t* dest, const void* d_xp, int xp_dtype,
                          const void* d_extra, float* dx, int accumulate, moe_stream_t stream);

/*
 * moe_route_backward - gate path.  With l = logits + logit_offset (as routed),
 * s = sqrt(softplus(l)) and w_j = s_j / S over a token's k experts:
 *   dlogits[t, idx_j] = (d_topk_w_j - sum_i w_i d_topk_w_i) / S * sig(l_j) / (2 s_j),
 *   zero elsewhere (fp32 [T, E], written);
 *   dx [T, d] fp32 += dlogits W_g^T;   dw_gate [d, E] fp32 = x^T dlogits.
 * x [T, d] in x_dtype; w_gate [d, E] fp32; logits [T, E] as moe_route wrote
 * them (without the offset); logit_offset [E] or NULL.  dw_gate sums over the
 * T tokens in up to 16 K-parts held in ws (moe_workspace_size(
 * MOE_OP_ROUTE_BACKWARD, shape, 0) bytes, enough for either path below;
 * MOE_ERR_WORKSPACE if smaller), added in part order (deterministic).  With bf16 x, d % 256 == 0 and E % 64 == 0
 * both products run on the matrix cores: each fp32 operand is split into
 * three bf16 planes (hi + mid + lo, 24 significant bits) and the plane
 * products above 2^-24 of a product are summed in fp32 (six for dx, three
 * for dw_gate, x being exact in bf16); otherwise fp32 vector products.
 */
int moe_route_backward(const moe_shape* shape, const void* x, int x_dtype, const float* w_gate,
                       const float* logit_offset, const float* logits, const int32_t* topk_idx,
                       const float* d_topk_w, float* dlogits, float* dx, float* dw_gate, void* ws,
                       size_t ws_bytes, moe_stream_t stream);

/*
 * moe_route_hash - hash router (mastering-deepseek-v4 "MoE + Expert-Parallel
 * Overlap (Exp08)", Implemented: a hash router emulates the early layers; a
 * token's experts follow from its token id).  Replaces moe_route; dispatch,
 * the expert FFN and combine are unchanged.  The pages do not give the hash;
 * this library uses Philox4x64-10 (Salmon et al., SC'11) keyed by (seed, 0)
 * with counter (token_ids[t] as uint32, block, 0, 0): each 64-bit word u of a
 * block picks expert floor(u * E / 2^64), repeats are skipped, the first k
 * distinct experts are listed in draw order; after 256 blocks any empty slot
 * takes the smallest unused experts.  Groups (G, M) play no part.
 *   shape      uses T, E, k (1 <= k <= min(E, 16), E <= 1024)
 *   token_ids  [T] int32 device (vocabulary ids; equal ids get equal experts)
 *   seed       key of the hash (one per layer)
 *   logits     [T, E] fp32 device or NULL.  NULL: topk_w = 1/k.  Otherwise
 *              topk_w[t,j] = s_j / (s_0 + ... + s_{k-1}) (left to right) with
 *              s = sqrt(softplus(logit)) by the same operation sequence as moe_route
 *   topk_idx   [T, k] int32, topk_w [T, k] fp32, block_counts as moe_route
 * T = 0 is a no-op returning MOE_OK.
 */
int moe_route_hash(const moe_shape* shape, const int32_t* token_ids, uint64_t seed,
                   const float* logits, int32_t* topk_idx, float* topk_w, int32_t* block_counts,
                   moe_stream_t stream);

/*
 * moe_bias_update - auxiliary-loss-free load balancing (mastering-deepseek-v4
 * "MoE + Expert-Parallel Overlap (Exp08)", Implemented and Measured: a
 * per-expert bias, updated from the observed expert load, replaces an
 * auxiliary balancing loss).  The pages do not print the rule; this is the
 * plainest reading:
 *     load[e] = sum over r of counts[r, e]
 *     bias[e] += gamma * sign(sum(load) / E - load[e])      (sign(0) = 0)
 * The comparison is exact (integer: sum(load) against E * load[e]); the update
 * is one fp32 addition of +gamma or -gamma, or none.
 *   n_rows, counts  [n_rows, E] int32 device, row-major: moe_route's
 *                   block_counts (n_rows = ceil(T/MOE_ROUTE_BLOCK)), a single
 *                   load vector (n_rows = 1, e.g. after an all-reduce over
 *                   data-parallel ranks), or one row per rank
 *   gamma   update step (finite)
 *   bias    [E] fp32 device, updated in place
 *   load    [E] int32 device, receives load[e]; may be NULL
 * 1 <= E <= 1024.  n_rows = 0 is a no-op returning MOE_OK (nothing written).
 * Ordered on the stream; overlapping calls on the same bias race.
 */
int moe_bias_update(int64_t n_rows, int32_t E, const int32_t* counts, float gamma, float* bias,
                    int32_t* load, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
