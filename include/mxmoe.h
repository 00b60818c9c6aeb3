/*
 * mxmoe.h -- C ABI of the MXFP8 MoE expert path for AMD MI355X (gfx950).
 *
 * The operations come from the tutorial on MoE training of biological
 * foundation models (BioNeMo MoE recipe with Transformer Engine), as retold by
 * "MoE-Training fuer biologische Grundmodelle optimieren" (hyper.ai, German),
 * "NVIDIA apresenta tecnicas para tornar mais eficiente o treinamento de
 * modelos biologicos baseados em arquitetura MoE" (conexaotc, Portuguese) and
 * "NVIDIA optimise l'entrainement MoE des modeles biologiques" (hyper.ai,
 * French):
 *   - GroupedLinear: the linear layers of all experts run in one call that is
 *     handed the number of tokens routed to each expert (German page, the
 *     paragraph on fragmented expert execution; Portuguese page, third
 *     paragraph; French page, first improvement).
 *   - MXFP8: 8 bits per value plus one scale per block of 32 values, with
 *     16-bit master weights and activations (German page, the paragraph on
 *     activation memory; Portuguese page, third paragraph; French page,
 *     second improvement).  Elements are OCP E4M3 (largest finite 448), scales
 *     E8M0; the scale of a block is 2^(floor(log2(amax)) - 8), elements are
 *     rounded to nearest even and saturate at +-448.
 *   - GroupedMLP: gate-up projection, SwiGLU scaled by the routing weight and
 *     the quantization fused into one forward and one backward pass whose
 *     intermediates are not held in memory (German page, the paragraph on the
 *     GroupedMLP fusion kernel; Portuguese page, third paragraph; French page,
 *     third improvement): the gate-up pre-activation h and the SwiGLU output
 *     stay on chip, only their requantized MXFP8 codes leave it, and the
 *     backward recomputes h from the saved X codes.  An optional mode
 *     (MX_MLP_SAVE_H) stores h as bf16 instead, trading 4 bytes per row and
 *     column of F for the recompute.
 *
 * Conventions shared by every entry point
 *   - All pointers named d_* and every tensor pointer are DEVICE pointers on
 *     the current HIP device.  Sizes are host scalars.  The library never
 *     synchronises: every call enqueues kernels on `stream` and returns.  The
 *     caller owns every buffer; the library allocates only the zero-padded
 *     operand copies of a GroupedLinear call whose K is not a multiple of 128
 *     (stream-ordered, freed on `stream` after its GEMM).
 *   - Rows are token-sorted: expert e owns rows [off[e], off[e+1]) of every
 *     [M, *] tensor; d_offsets is int64 [E+1] with off[0] = 0, off[E] = M,
 *     non-decreasing (not checked on the device).  Experts may be empty.
 *   - bf16 tensors are row-major with contiguous rows.  An MXFP8 tensor is a
 *     pair: codes (uint8 E4M3, same shape as the source, blocks of 32 along the
 *     last axis) and scales (uint8 E8M0, one per block, [rows][cols/32]).
 *   - A "columnwise" copy of X[R, C] is stored transposed: codes [C][ld] and
 *     scales [C][ld/32], blocks of 32 consecutive rows of X.  When X has row
 *     groups (experts), each group's rows start a new block and the group is
 *     padded with zero codes to a multiple of MX_TOKEN_ALIGN (128) rows; the
 *     start of group g in the padded axis is written to d_padded_offsets[g].
 *   - Errors: host-side validation returns a status and never touches the
 *     device; mx_last_error() gives the thread's last message.  Kernel launch
 *     failures return MX_ERR_LAUNCH.  Device-side contract violations (bad
 *     offsets) are undefined behaviour, unless MX_CHECK=1 is set in the
 *     environment: then every entry point that takes device offsets copies
 *     them to the host on its stream, waits for the copy (the one case where
 *     the library synchronises) and returns MX_ERR_INVALID_ARG, launching
 *     nothing, if they do not start at 0, decrease, or do not end at the row
 *     count (fp8_tensor_quantize: start >= 0, end <= rows).
 *   - Every call is re-entrant; calls on one stream are ordered.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* mx_stream_t; /* same type as hipStream_t */

typedef enum {
    MX_OK = 0,
    MX_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad combination */
    MX_ERR_UNSUPPORTED = 2,  /* size not a multiple the kernels need */
    MX_ERR_WORKSPACE = 3,    /* ctx or workspace smaller than required */
    MX_ERR_LAUNCH = 4        /* a HIP launch or query failed */
} mx_status;

enum { MX_DTYPE_BF16 = 0, MX_DTYPE_MXFP8 = 1 };
enum { MX_TOKEN_ALIGN = 128, MX_BLOCK = 32 };

/* Last error message of the calling thread ("" if none).  Never NULL. */
const char* mx_last_error(void);

/* Library version string. */
const char* mx_version(void);

/* Host-side check of a per-group offsets array in HOST memory: offsets[0] ==
 * 0, non-decreasing, offsets[G] == M.  MX_OK, or MX_ERR_INVALID_ARG with the
 * first violation in mx_last_error().  This is what MX_CHECK=1 runs on a copy
 * of the device offsets an entry point is given. */
mx_status mx_validate_offsets(const int64_t* h_offsets, int32_t G, int64_t M);

/* Upper bound of the padded length of G row groups holding M rows in total,
 * each padded to a multiple of `align`: the leading dimension the caller
 * allocates for a grouped columnwise copy.  Returns -1 on bad arguments. */
int64_t mx_padded_rows_bound(int64_t M, int32_t G, int32_t align);

/*
 * mxfp8_quantize -- block-quantize bf16 to MXFP8 (the MXFP8 paragraphs cited
 * above: 8-bit values, one scale per 32 values).
 *
 *   x            bf16 [batch][R][C], C % 32 == 0.
 *   row_codes    uint8 [batch][R][C] and row_scales [batch][R][C/32]: the
 *                rowwise copy (blocks along C).  Both NULL to skip.
 *   d_offsets    int64 [G+1] row groups of the columnwise copy (batch must be
 *                1), or NULL: each batch item is one group of R rows.
 *   col_codes    uint8 [batch][C][col_ld], col_scales [batch][C][col_ld/32]:
 *                the columnwise copy (blocks along R, restarting at every
 *                group, groups padded to MX_TOKEN_ALIGN with zero codes).
 *                Both NULL to skip.  col_ld % 128 == 0 and col_ld must be at
 *                least mx_padded_rows_bound(R, G, 128) (G = 1 if no groups).
 *                Columns past the last group's padded end are not written.
 *   d_padded_offsets  int64 [G+1], written (device) when col_codes is given
 *                with d_offsets; may be NULL otherwise.
 * At least one of the two copies must be requested.  x and the code buffers
 * must be 16-byte aligned, the scale buffers 4-byte aligned
 * (MX_ERR_INVALID_ARG otherwise).  With the columnwise copy, 256 * C must be
 * below 2^31 (MX_ERR_UNSUPPORTED otherwise: 32-bit tile offsets).
 */
mx_status mxfp8_quantize(const void* x, int64_t batch, int64_t R, int64_t C,
                         uint8_t* row_codes, uint8_t* row_scales,
                         const int64_t* d_offsets, int32_t G,
                         uint8_t* col_codes, uint8_t* col_scales,
                         int64_t col_ld, int64_t* d_padded_offsets,
                         mx_stream_t stream);

/*
 * grouped_linear_fwd -- GroupedLinear: for every expert e in ONE launch,
 *   Y[off[e]:off[e+1]] = X[off[e]:off[e+1]] . W[e]^T   (times r[row] if given)
 * (German page, the paragraph on fragmented expert execution; French page,
 * first improvement).  Accumulation in fp32, output rounded to bf16 (RNE).
 *
 *   dtype MX_DTYPE_BF16:  x bf16 [M][K], w bf16 [E][N][K]; x_scales, w_scales
 *                         must be NULL.  K % 32 == 0, N % 16 == 0.
 *   dtype MX_DTYPE_MXFP8: x = E4M3 codes [M][K] with x_scales [M][K/32];
 *                         w = codes [E][N][K] with w_scales [E][N][K/32]
 *                         (rowwise copies from mxfp8_quantize).
 *                         K % 32 == 0, N % 32 == 0.  K % 128 != 0 runs
 *                         through zero-padded copies of both operands to K
 *                         rounded up to 128 (codes 0, scales 2^0 past K),
 *                         in one device allocation made with hipMallocAsync
 *                         on `stream` and freed after the GEMM (a failed
 *                         allocation returns MX_ERR_LAUNCH).
 *   d_row_scale  fp32 [M] routing weight applied to each output row, or NULL.
 *   y            bf16 [M][N].
 */
mx_status grouped_linear_fwd(int32_t dtype, const void* x,
                             const uint8_t* x_scales, const int64_t* d_offsets,
                             int32_t E, int64_t M, const void* w,
                             const uint8_t* w_scales, int64_t N, int64_t K,
                             const float* d_row_scale, void* y,
                             mx_stream_t stream);

/*
 * Per-tensor scaled FP8, the plain FP8 format the German page names beside
 * MXFP8 (paragraph on activation memory; the page gives no recipe).  Every
 * expert's slice of a grouped operand is one tensor with one fp32 scale:
 * scale = 448 / amax (IEEE division; amax 0 gives 1, an overflowing quotient
 * the largest finite fp32), code = E4M3 of the fp32 product x * scale
 * (nearest even, saturating at +-448), scale_inv = 1 / scale.
 *
 * fp8_tensor_quantize -- codes uint8 [batch][R][C] of bf16 x [batch][R][C].
 *   Groups: with d_offsets (int64 [G+1], batch must be 1) group g is rows
 *   [off[g], off[g+1]) -- rows outside [off[0], off[G]) are neither counted
 *   nor written; without, group g is matrix g (G must equal batch).
 *   d_amax, d_scale_inv  fp32 [G], written (device).  C % 32 == 0,
 *   256 * C < 2^31 (MX_ERR_UNSUPPORTED otherwise); x and codes 16-byte aligned.
 *   Three launches on `stream` (amax reset, amax, cast); x is read twice.
 *
 * grouped_linear_fwd_fp8 -- GroupedLinear on per-tensor FP8 operands:
 *   Y[off[e]:off[e+1]] = (X_e codes . W_e codes^T) * x_scale_inv[e]
 *                        * w_scale_inv[e]  (times r[row] if given)
 *   x codes [M][K], w codes [E][N][K] (from fp8_tensor_quantize, x with the
 *   same offsets, w as E matrices), scale_inv fp32 [E] each (device), y bf16
 *   [M][N].  fp32 accumulation.  K % 32 == 0, N % 32 == 0 (K % 128 != 0:
 *   padded copies as for grouped_linear_fwd).
 */
mx_status fp8_tensor_quantize(const void* x, int64_t batch, int64_t R, int64_t C,
                              const int64_t* d_offsets, int32_t G, uint8_t* codes,
                              float* d_amax, float* d_scale_inv, mx_stream_t stream);
mx_status grouped_linear_fwd_fp8(const uint8_t* x, const float* d_x_scale_inv,
                                 const int64_t* d_offsets, int32_t E, int64_t M,
                                 const uint8_t* w, const float* d_w_scale_inv, int64_t N,
                                 int64_t K, const float* d_row_scale, void* y,
                                 mx_stream_t stream);

/*
 * grouped_mlp_fwd -- fused GroupedMLP forward (German page, the paragraph on
 * the GroupedMLP fusion kernel; Portuguese page, third paragraph; French page,
 * third improvement), in the order gate-up projection -> SwiGLU -> routing
 * weight scale -> down projection:
 *   h = Q(X_e) . Q(W1_e)^T          [rows of e, 2F]   (blocks along H)
 *   z = r * silu(h[:, :F]) * h[:, F:]                  (fp32, on chip)
 *   Y_e = Q(z) . Q(W2_e)^T          [rows of e, H]    (blocks along F)
 *
 *   x    bf16 [M][H];  w1 bf16 [E][2F][H] (rows [0,F) gate, [F,2F) up);
 *   w2   bf16 [E][H][F];  d_r fp32 [M];  y bf16 [M][H].  With M == 0, x, d_r
 *        and y may be NULL (the weights are still quantized into ctx).
 *   ctx  saved-for-backward buffer of grouped_mlp_ctx_bytes(.., 0) bytes,
 *        written here and read by grouped_mlp_bwd (opaque; 256-byte
 *        aligned): the MXFP8 copies of w1 and w2 (rowwise and columnwise),
 *        the rowwise and token-axis copies of x, the token-axis copy of z and
 *        the padded token offsets.  h is not stored (the backward recomputes
 *        it).
 *   ws   scratch of grouped_mlp_fwd_ws_bytes(.., 0) bytes (256-byte aligned):
 *        the rowwise MXFP8 copy of z, and 64 MiB (plus an 8 KiB header) for
 *        the fp32 partial tiles of the down GEMM's split tail round (the last
 *        round of output tiles, cut along K when it would leave more than
 *        half of the GPU idle).
 * H % 128 == 0, F % 128 == 0, E in [1, 1024], 2F * H < 2^31 (one expert's
 * weights), and mx_padded_rows_bound(M, E, 128) <= 65535 * 128 = 8,388,480
 * rows (MX_ERR_UNSUPPORTED otherwise).
 */
mx_status grouped_mlp_fwd(const void* x, const int64_t* d_offsets, int32_t E,
                          int64_t M, int64_t H, int64_t F, const void* w1,
                          const void* w2, const float* d_r, void* y,
                          void* ctx, size_t ctx_bytes, void* ws,
                          size_t ws_bytes, mx_stream_t stream);

/*
 * grouped_mlp_fwd_ex -- grouped_mlp_fwd with flags (0: same as
 * grouped_mlp_fwd).
 *
 * MX_FWD_REUSE_WEIGHTS: skip quantizing the weights and use the MXFP8 copies
 * that an earlier forward with the same w1, w2, E, H, F and MX_MLP_SAVE_H
 * setting left in this ctx: the caching of weight quantization across
 * micro-batches that the 16-bit master weights allow while they do not
 * change (German page, the paragraph on quantization between 16-bit master
 * weights and the 8-bit path).  The weight regions sit at the start of ctx,
 * so M may differ from that earlier call.  w1 and w2 are not read and may be
 * NULL.  The caller guarantees that the weights have not changed and that
 * nothing else has written those regions (grouped_mlp_bwd only reads them);
 * with any other contents the results are undefined, not an error.
 *
 * MX_MLP_SAVE_H: the save-h mode.  The forward stores the gate-up
 * pre-activation h as bf16 (RNE of the fp32 accumulator) in ctx and the
 * backward reads it instead of recomputing it: the backward then runs one
 * GEMM fewer over K = H per expert row block (2*M*2F*H fewer flops) for
 * M*2F*2 more bytes of ctx.  The backward's SwiGLU gradient then sees
 * bf16(h).  ctx and ws sizes, views and the backward must be given the same
 * flag (grouped_mlp_bwd_ex).
 *
 * Unknown flag bits: MX_ERR_INVALID_ARG.
 */
#define MX_FWD_REUSE_WEIGHTS 1u
#define MX_MLP_SAVE_H 2u
mx_status grouped_mlp_fwd_ex(const void* x, const int64_t* d_offsets, int32_t E,
                             int64_t M, int64_t H, int64_t F, const void* w1,
                             const void* w2, const float* d_r, void* y,
                             void* ctx, size_t ctx_bytes, void* ws,
                             size_t ws_bytes, uint32_t flags, mx_stream_t stream);

/*
 * grouped_mlp_bwd -- fused GroupedMLP backward with MXFP8 operands in every
 * GEMM (Portuguese page, fourth paragraph: MXFP8 active in forward and
 * backward).  Straight-through quantizers; each GEMM quantizes its operands
 * along its own contraction axis: rowwise copies feed the data gradients,
 * columnwise (token-axis) copies the weight gradients.
 *   dz  = Q(dY_e) . Q(W2_e)          (blocks along H)
 *   h   = Q(X_e) . Q(W1_e)^T = [a | b], recomputed in the same kernel tile
 *         as dz from the forward's saved codes (save-h mode: read from ctx)
 *   dr  = sum_f dz * s,  s = silu(a) * b
 *   dh  = [r dz b silu'(a) | r dz silu(a)]
 *   dX  = Q(dh) . Q(W1_e)            (blocks along 2F)
 *   dW2_e = Q_tok(dY_e)^T . Q_tok(z_e),  dW1_e = Q_tok(dh_e)^T . Q_tok(X_e)
 * Experts with no rows get dW1_e = dW2_e = 0.
 *
 *   dy bf16 [M][H]; outputs dx bf16 [M][H], dw1 bf16 [E][2F][H],
 *   dw2 bf16 [E][H][F], d_dr fp32 [M] (dy, d_r, dx and d_dr may be NULL when
 *   M == 0; dw1 and dw2 are then all zeros).  Same sizes, x-free: the forward's
 *   ctx holds what is needed, including the quantized copies of w1 and w2
 *   made by the forward (w1 and w2 must be the tensors given to the forward
 *   that wrote ctx; the backward only checks them for NULL and alignment).
 *   ws of grouped_mlp_bwd_ws_bytes(.., flags) bytes: the MXFP8 copies of dY
 *   and dh, the dr partial sums, and the split-tail scratch of the gate-up
 *   dgrad (as in the forward).
 *
 * grouped_mlp_bwd_ex -- grouped_mlp_bwd with flags: MX_MLP_SAVE_H for a ctx
 *   written by a forward with that flag (0: same as grouped_mlp_bwd).  A
 *   ctx read in the other mode than it was written gives undefined results.
 *   Unknown flag bits: MX_ERR_INVALID_ARG.
 */
mx_status grouped_mlp_bwd(const void* dy, const int64_t* d_offsets, int32_t E,
                          int64_t M, int64_t H, int64_t F, const void* w1,
                          const void* w2, const float* d_r, const void* ctx,
                          size_t ctx_bytes, void* dx, void* dw1, void* dw2,
                          float* d_dr, void* ws, size_t ws_bytes,
                          mx_stream_t stream);
mx_status grouped_mlp_bwd_ex(const void* dy, const int64_t* d_offsets, int32_t E,
                             int64_t M, int64_t H, int64_t F, const void* w1,
                             const void* w2, const float* d_r, const void* ctx,
                             size_t ctx_bytes, void* dx, void* dw1, void* dw2,
                             float* d_dr, void* ws, size_t ws_bytes,
                             uint32_t flags, mx_stream_t stream);

/* Byte sizes of the buffers above for the mode in flags (0 or
 * MX_MLP_SAVE_H); 0 on bad arguments. */
size_t grouped_mlp_ctx_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags);
size_t grouped_mlp_fwd_ws_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags);
size_t grouped_mlp_bwd_ws_bytes(int64_t M, int64_t H, int64_t F, int32_t E, uint32_t flags);

/*
 * Views into a forward ctx of the mode in flags, for inspection and tests
 * (offsets in bytes from the ctx base; all regions 256-byte aligned):
 *   MX_CTX_H        (save-h mode only) gate-up pre-activation h (bf16, RNE of fp32) in 16 x 16
 *                   blocks: block (pr/16, c/16), pr = padded row (expert e's
 *                   row off[e]+t sits at padded row poff[e]+t), c in [0, F),
 *                   is 1 KiB at byte ((pr/16)*(F/16) + c/16)*1024; within it
 *                   lane l = 16*q + r holds 16 bytes: gate h[pr+r][c+4q+v] for
 *                   v = 0..3, then up h[pr+r][F+c+4q+v].  Mp*F*4 bytes.
 *   MX_CTX_XROW     (recompute mode only) X rowwise codes [M][H] then scales
 *   MX_CTX_XCOL     X columnwise codes [H][Mp] then scales
 *   MX_CTX_ZCOL     z columnwise codes [F][Mp] then scales
 *   MX_CTX_POFF     int64 [E+1] padded token offsets
 *   MX_CTX_W1COL    W1 columnwise codes [E*H][2F] (blocks along 2F) + scales
 *   MX_CTX_W2COL    W2 columnwise codes [E*F][H] (blocks along H) + scales
 *   MX_CTX_W1ROW    W1 rowwise codes [E*2F][H] (blocks along H) + scales
 *   MX_CTX_W2ROW    W2 rowwise codes [E*H][F] (blocks along F) + scales
 * with Mp = mx_padded_rows_bound(M, E, 128).  In every codes-then-scales
 * pair here and below, the scales start at the first 256-byte boundary after
 * the last code byte, and (unlike the public entry points' row-major scales)
 * are K-step tiled: for codes [R][Kp], the scale of row r and block kb (codes
 * kb*32 .. kb*32+31) is byte ((r/32)*(Kp/128) + kb/4)*128 + (r%32)*4 + kb%4,
 * with R rounded up to a multiple of 32.  Returns -1 on bad arguments and for
 * a region the mode does not have.
 */
enum { MX_CTX_H = 0, MX_CTX_XCOL = 1, MX_CTX_ZCOL = 2, MX_CTX_POFF = 3, MX_CTX_W1COL = 4,
       MX_CTX_W2COL = 5, MX_CTX_XROW = 6, MX_CTX_W1ROW = 7, MX_CTX_W2ROW = 8 };
int64_t grouped_mlp_ctx_offset(int32_t which, int64_t M, int64_t H, int64_t F,
                               int32_t E, uint32_t flags);

/*
 * Views into the forward/backward workspaces of the mode in flags, for tests:
 * the rowwise z (codes [M][F] + K-step tiled scales) the forward fed its down
 * projection; the backward's rowwise dY (codes [M][H] + scales) and
 * token-axis dY (codes [H][Mp] + scales), and its rowwise and columnwise dh
 * (codes [M][2F] + scales; columnwise codes [2F][Mp] + scales).  Returns -1
 * on bad arguments.
 */
enum { MX_WS_ZROW = 0, MX_WS_DHROW = 1, MX_WS_DHCOL = 2, MX_WS_DYROW = 3, MX_WS_DYCOL = 4 };
int64_t grouped_mlp_ws_offset(int32_t which, int64_t M, int64_t H, int64_t F,
                              int32_t E, uint32_t flags);

/*
 * Routing around the expert path: the sorted-row plan of a top-k routing,
 * the permute that gathers token rows into that order (fused with MXFP8
 * quantization), and the combine back to token order with its backward.
 * The German page's paragraph on GroupedLinear: the caller hands over the
 * number of tokens per expert and the expert inputs are gathered into one
 * grouped call; the Portuguese page, third paragraph: routing weights send
 * each token to its experts.  Rows are sorted stably by (expert, token,
 * slot); the combine is out[t] = sum_j c[t][j] * Y[row_of[t][j]] with c = w
 * or, when the expert path already applied the routing weights (as the
 * GroupedMLP does), c = 1.  No host synchronisation; deterministic.
 *
 * moe_router -- the router: token t's experts d_ids int32 [T][k] are its k
 *   largest logits (d_logits fp32 [T][E], finite), taken one at a time (the
 *   lower expert index among equal values), and d_w fp32 [T][k] the softmax
 *   of those k logits.  1 <= k <= min(E, 64), E <= 1024 (MX_ERR_UNSUPPORTED
 *   above 64 or 1024).
 *
 * moe_route_ws_bytes -- scratch bytes moe_route_plan needs (0 on bad sizes).
 *
 * moe_route_plan
 *   d_ids       int32 [T][k], expert of token t's slot j, in [0, E).  Slots
 *               with other values are not routed: row_of = -1, no row.
 *   d_w         fp32 [T][k] routing weights, or NULL.
 *   d_offsets   int64 [E+1] out: expert e owns sorted rows
 *               [offsets[e], offsets[e+1]); offsets[E] = routed slots M.
 *   d_row_of    int32 [T][k] out: sorted row of each slot.
 *   d_tok_of    int32 [T*k] out: token of each sorted row (first M entries).
 *   d_r_sorted  fp32 [T*k] out: w of each sorted row; NULL iff d_w is NULL.
 *   ws          moe_route_ws_bytes(T, k, E) bytes, 4-byte aligned.
 *   1 <= k <= 64, 1 <= E <= 1024 (MX_ERR_UNSUPPORTED above), T*k < 2^31.
 *
 * moe_permute_quantize -- MXFP8 copies of the sorted rows X[tok_of[row]]
 *   straight from the token-order x, as mxfp8_quantize makes them from
 *   already sorted rows (row-major scales): rowwise codes [M][H] + scales
 *   [M][H/32], columnwise codes [H][col_ld] + scales [H][col_ld/32] with
 *   every expert padded to MX_TOKEN_ALIGN zero tokens; either copy may be
 *   skipped (both pointers NULL).  x bf16 [T][H]; d_offsets from
 *   moe_route_plan; M = the routed rows (T*k when every slot is routed);
 *   d_padded_offsets int64 [E+1] out.  H % 32 == 0, T*H*2 and 256*H below
 *   2^31; alignment as mxfp8_quantize.
 *
 * moe_combine -- out bf16 [T][H] = sum_j c[t][j] * y[row_of[t][j]] in fp32,
 *   j ascending, rounded once to bf16; y bf16 [M][H]; d_w NULL for c = 1.
 *   Unrouted slots contribute nothing.  H % 8 == 0; y, out 16-byte aligned.
 *
 * moe_combine_bwd -- dy bf16 [M][H]: dy[row_of[t][j]] = c[t][j] * dout[t]
 *   (with d_w NULL an exact copy: the token -> sorted-row permute of dout);
 *   d_dw fp32 [T][k] (or NULL): <dout[t], y[row_of[t][j]]>, needs d_w and y
 *   bf16 [M][H].  Rows that no slot maps to are not written.
 */
mx_status moe_router(const float* d_logits, int64_t T, int32_t E, int32_t k,
                     int32_t* d_ids, float* d_w, mx_stream_t stream);
size_t moe_route_ws_bytes(int64_t T, int32_t k, int32_t E);
mx_status moe_route_plan(const int32_t* d_ids, int64_t T, int32_t k, int32_t E,
                         const float* d_w, int64_t* d_offsets, int32_t* d_row_of,
                         int32_t* d_tok_of, float* d_r_sorted, void* ws,
                         size_t ws_bytes, mx_stream_t stream);
/*
 * moe_route_plan_noalloc -- moe_route_plan without a workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, outputs
 * and checks as moe_route_plan, minus ws / ws_bytes.  The per-chunk counts
 * go to a scratch array the library owns: 2^20 int32 (4 MiB) per GPU, held
 * from the first call on that GPU until the process ends; nothing is
 * allocated or freed by the call.  Limit: ceil(T*k/256) * E <= 2^20 (for
 * example T*k <= 33,554,432 at E = 8, or T*k <= 262,144 at E = 1024);
 * larger plans return MX_ERR_UNSUPPORTED (use moe_route_plan).  Every call
 * on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 * different streams, or from threads whose calls are not ordered) race and
 * give undefined results; calls on one stream are ordered and safe.  The
 * scratch needs no clearing (every counter a call reads it writes first).
 */
mx_status moe_route_plan_noalloc(const int32_t* d_ids, int64_t T, int32_t k, int32_t E,
                                 const float* d_w, int64_t* d_offsets,
                                 int32_t* d_row_of, int32_t* d_tok_of,
                                 float* d_r_sorted, mx_stream_t stream);
mx_status moe_permute_quantize(const void* x, int64_t T, int64_t H,
                               const int32_t* d_tok_of, int64_t M,
                               const int64_t* d_offsets, int32_t E,
                               uint8_t* row_codes, uint8_t* row_scales,
                               uint8_t* col_codes, uint8_t* col_scales,
                               int64_t col_ld, int64_t* d_padded_offsets,
                               mx_stream_t stream);
mx_status moe_combine(const void* y, int64_t M, int64_t H, const int32_t* d_row_of,
                      int64_t T, int32_t k, const float* d_w, void* out,
                      mx_stream_t stream);
mx_status moe_combine_bwd(const void* dout, int64_t T, int64_t H, int32_t k,
                          const int32_t* d_row_of, const float* d_w, const void* y,
                          int64_t M, void* dy, float* d_dw, mx_stream_t stream);

/*
 * Launch timing (diagnostics; not part of the computation).  Between
 * mx_profile_begin() and mx_profile_end(), every kernel the library launches
 * from the calling thread is bracketed by two HIP events recorded on the
 * launch's stream, up to `capacity` launches (later launches are not timed).
 * Each record carries the kernel's name and its algorithmic work: floating
 * point operations for GEMMs (2*M*N*K summed over experts), bytes moved for
 * memory-bound kernels.  The events are created by mx_profile_begin (the only
 * call here that allocates) and destroyed by the next mx_profile_begin.
 *   mx_profile_count  number of records of the last begin/end window.
 *   mx_profile_get    waits for record i's events, then returns its name
 *                     (static string), milliseconds, work and unit
 *                     (MX_WORK_FLOP or MX_WORK_BYTES).
 */
enum { MX_WORK_FLOP = 0, MX_WORK_BYTES = 1 };
mx_status mx_profile_begin(int32_t capacity);
mx_status mx_profile_end(void);
int32_t mx_profile_count(void);
mx_status mx_profile_get(int32_t i, const char** name, float* ms, double* work,
                         int32_t* unit);

#ifdef __cplusplus
}
#endif
#endif /* MXMOE_H */
