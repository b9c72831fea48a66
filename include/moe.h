/*
 * moe.h — C ABI of the MI355X (gfx950) MoE expert-layer library, one GPU's share of the
 * experts.
 *
 * The layer follows the "Mega MoE" page (Primus-Turbo documentation), section
 * Pipeline: a dispatch prologue builds routing tables from external top-k routing; the
 * dispatched token rows go through an L1 grouped GEMM (NT) into a [gate | up] projection;
 * SwiGLU; an L2 grouped GEMM (NT); and a combine that weights each row by its top-k weight
 * and sums the contributions of each token (a weighted scatter-add).  The backward entry
 * points follow the same section's backward: L2 dgrad (NN) with the gradient of the routing
 * weights, the SwiGLU transpose, dW2 with a variable K (the row count of each expert), dW1 (TN)
 * on re-gathered token rows, as in the page's Core Design section 2 (recompute the dispatched
 * x instead of saving it), and the L1 dgrad (NN) whose rows are summed back to token order.
 * Per-expert row counts are padded to the GEMM block (block-M alignment, "How Mega MoE
 * Overlaps Expert Parallelism Communication with Computation in DeepGEMM" page, section
 * Block-M Alignment), so every launch has a shape fixed on the host and nothing waits on the
 * host ("Mega MoE" page, Core Design section 3): every call only enqueues work on `stream`
 * and returns; the whole sequence can be captured into a HIP graph.
 *
 * Conventions shared by all entry points
 *   - Pointers marked [device] are device addresses; [host] are host addresses.
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense row-major.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 *   - Ownership: the caller owns every buffer (inputs, weights, outputs, workspace) and must
 *     keep it alive until the enqueued work completes.  The library allocates nothing, frees
 *     nothing, copies nothing between host and device and keeps no state between calls (beyond
 *     cached device properties and kernel attributes), so calls with distinct workspaces may run
 *     concurrently on different streams.
 *   - Workspace: `ws` is a device buffer of at least moe_workspace_bytes(shape) bytes, 256-B
 *     aligned.  The stages of one layer communicate through it and rely on stream order:
 *     moe_route_prologue, then moe_dispatch_gemm1, then moe_gemm2_combine, on one stream.
 *   - Errors: argument checks run on the host before any launch and return a negative
 *     moe_status without enqueuing anything.  A launch failure returns MOE_ERR_LAUNCH.
 *     Data-dependent conditions never trap on the device: an expert id outside [0, E) is
 *     ignored and counted (moe_workspace_layout().meta, entry 1).
 *   - No C++ exception crosses this interface.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,       /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,      /* a size is out of the supported range */
    MOE_ERR_BLOCK_M = -3,    /* block_m is not 32, 64, 128 or 256 */
    MOE_ERR_WORKSPACE = -4,  /* ws_bytes < moe_workspace_bytes(shape), or ws lacks train buffers */
    MOE_ERR_ALIGN = -5,      /* a pointer is not 16-byte aligned (ws: 256-byte) */
    MOE_ERR_LAUNCH = -6,     /* the HIP runtime rejected a launch */
    MOE_ERR_DEVICE = -7,     /* the current device is not a gfx950 GPU, or HIP failed */
    MOE_ERR_SCRATCH = -8     /* moe_forward_noalloc: the shape needs more than its fixed scratch */
} moe_status;

/*
 * Layer shape (host struct).
 *   T        tokens on this GPU (>= 0)
 *   H        hidden size (multiple of 128)
 *   I        intermediate size; the L1 output is [gate | up], 2*I wide (multiple of 128)
 *   E        experts in routing; ids in [0, E) are valid
 *   e_lo     first expert owned by this GPU; it owns ids [e_lo, e_lo + EL), e_lo + EL <= E
 *   EL       experts owned by this GPU (1 .. 1024)
 *   k        top-k slots per token (1 .. 32)
 *   block_m  GEMM row block; each expert's row count is padded up to a multiple of it
 *   train    nonzero: the workspace also holds the activations saved for the backward
 *            (pre-activation [gate | up] rows) and the backward's row gradients
 */
typedef struct moe_shape {
    int32_t T, H, I, E, e_lo, EL, k, block_m, train;
} moe_shape;

/*
 * Workspace layout: byte offsets of each region from the start of `ws`.  A hi / lo pair holds a
 * value v computed in fp32 as two bf16 arrays, hi = bf16(v) and lo = bf16(v - hi): the bf16
 * matrix cores take the pair as two operands, so the value enters a GEMM with about 16
 * significant bits instead of 8.
 *   rows_capacity  R_max = round_up(T*k + EL*(block_m - 1), block_m), the static bound on
 *                  padded rows every row-indexed region and grid is sized from
 *   counts         int32 [EL]           rows of each local expert
 *   padded_offsets int32 [EL + 1]       first row of each expert's segment (multiples of block_m)
 *   row_pair       int32 [R_max]        pair id p = t*k + j held by each row, -1 = padding/unused
 *   pair_row       int32 [T*k]          row of each pair, -1 = pair not handled by this GPU
 *   tile_expert    int32 [R_max/block_m] expert of each row block, -1 past the last segment
 *   tok_nloc       int32 [T]            local pairs of each token
 *   meta           int32 [4]            [0] padded row total R, [1] ids outside [0, E)
 *   act            bf16  [R_max, I]     SwiGLU output rows (L2 input)
 *   stage          fp32  [R_max, H]     weighted L2 rows of tokens with several local pairs
 *   hgu            fp32  [R_max, 2I]    pre-activation rows (train only, else 0)
 *   dact           fp32  [R_max, I]     L2 dgrad rows (train only, else 0)
 *   dhgu           bf16  [R_max, 2I]    [gate | up] gradient rows, hi part (train only, else 0)
 *   zeros          bf16  [max(H, 2I)]   a zero row (written by moe_route_prologue), read in place
 *                                       of the token row of a padding row
 *   scratch        prologue scratch (per-chunk expert histograms)
 *   tile_sync      int32 [512]          tile-scheduler counters of the forward GEMMs (zeroed by
 *                                       moe_route_prologue; zero again after each GEMM launch)
 *   dtw_part       fp32  [R_max, I/128] per-row partial sums of the routing-weight gradient, one
 *                                       per 128-column tile of the L2 dgrad (train only, else 0)
 *   dhgu_lo        bf16  [R_max, 2I]    lo part of the [gate | up] gradient rows (train only)
 *   wact           bf16  [R_max, I]     w * act, the activation row times its pair's routing
 *                                       weight, hi part (train only, else 0)
 *   wact_lo        bf16  [R_max, I]     its lo part (train only, else 0)
 */
typedef struct moe_ws_layout {
    size_t total_bytes;
    int64_t rows_capacity;
    int64_t num_blocks;
    size_t counts, padded_offsets, row_pair, pair_row, tile_expert, tok_nloc, meta;
    size_t act, stage, hgu, dact, dhgu, zeros, scratch, tile_sync, dtw_part;
    size_t dhgu_lo, wact, wact_lo;
} moe_ws_layout;

/* Message for a status code (static string). */
const char* moe_status_string(int32_t status);

/* Pure host functions of the shape. moe_workspace_bytes returns 0 for an invalid shape. */
size_t moe_workspace_bytes(const moe_shape* shape);
int32_t moe_workspace_layout(const moe_shape* shape, moe_ws_layout* out /* [host] */);

/* A block_m for a shape: the smallest of 64/128/256 whose padding stays small for the mean
 * rows per expert (the analogue of the block-M query on the "How Mega MoE Overlaps ..." page,
 * Block-M Alignment).  Returns 64 for an invalid shape. */
int32_t moe_preferred_block_m(const moe_shape* shape);

/*
 * One-time weight transform (untimed), as in the weight transform step that precedes the fused
 * call in the "How Mega MoE Overlaps ..." page's example: the logical x @ W weights become
 * fragment-major packed weights that the GEMMs stream straight into MFMA operand registers.
 *   w1  [device] bf16 [EL, H, 2I]  ->  w1p [device] bf16, EL * 2I * H elements
 *   w2  [device] bf16 [EL, I, H]   ->  w2p [device] bf16, EL * H * I elements
 * Packed layout.  Expert e's block starts at element e * N * K.  View the expert's matrix as
 * B[n][k] with n an output column (N = 2I for W1, H for W2) and k the reduction index (K = H
 * for W1, I for W2); element (n, k) sits at
 *     ((n / 32) * (K / 16) + k / 16) * 512 + ((k / 8) % 2 * 32 + n % 32) * 8 + k % 8
 * i.e. 1 KB blocks of 32 columns x 16 k, column-group major, each block the B operand of one
 * 32x32x16 MFMA.  For W2, n = h and k = i.  For W1, n is a packed column: L1 output column c
 * (c < I: gate column c; c >= I: up column c - I) is packed column
 *     ((c mod I) / 32) * 64 + (c >= I) * 32 + c mod 32,
 * so gate and up groups of the same 32 intermediate columns alternate.
 * Either pair may be NULL/NULL to skip it.  Inputs and outputs must not overlap.
 */
int32_t moe_pack_weights(const moe_shape* shape, const uint16_t* w1, const uint16_t* w2,
                         uint16_t* w1p, uint16_t* w2p, void* stream);

/* Inverse of moe_pack_weights: packed w1p / w2p (or weight gradients dw1p / dw2p, which share
 * the packed layout) -> logical w1 [EL, H, 2I] / w2 [EL, I, H].  Either pair may be NULL/NULL. */
int32_t moe_unpack_weights(const moe_shape* shape, const uint16_t* w1p, const uint16_t* w2p,
                           uint16_t* w1, uint16_t* w2, void* stream);

/*
 * Dispatch prologue ("Mega MoE" page, Implementation Map: routing tables): from topk_idx
 * [device] int32 [T, k] builds counts, padded_offsets, row_pair, pair_row, tile_expert,
 * tok_nloc and meta in ws.  Rows inside an expert's segment are in ascending pair order, so
 * the tables are deterministic.  A pair is local when e_lo <= id < e_lo + EL.
 */
int32_t moe_route_prologue(const moe_shape* shape, const int32_t* topk_idx, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Dispatch + L1 grouped GEMM, NT ("Mega MoE" page, Pipeline, dispatch_grouped_gemm): for every
 * row r of a real block, h[r] = x[row_pair[r] / k] @ W1[e] over the packed w1p [device]
 * (moe_pack_weights), with x [device] bf16 [T, H] gathered through row_pair inside the tile load
 * (padding rows are zero).  Writes, for rows [0, R):
 *   act_out [device] bf16 [R_max, I]  = silu(h[:, :I]) * h[:, I:]   (SwiGLU in the epilogue)
 *   hgu_out [device] fp32 [R_max, 2I] = h                            (pre-activation)
 * Either output may be NULL, not both.  Pass ws-relative regions (layout act / hgu) to feed
 * moe_gemm2_combine and the backward.
 */
int32_t moe_dispatch_gemm1(const moe_shape* shape, const uint16_t* x, const uint16_t* w1p,
                           void* ws, size_t ws_bytes, uint16_t* act_out, float* hgu_out,
                           void* stream);

/*
 * SwiGLU ("Mega MoE" page, Pipeline; Implementation Map, SwiGLU fwd): act[r, c] =
 * silu(hgu[r, c]) * hgu[r, I + c] for rows [0, R) (R read from ws on the device).
 *   hgu [device] fp32 [R_max, 2I], act [device] bf16 [R_max, I]
 */
int32_t moe_swiglu(const moe_shape* shape, const float* hgu, const void* ws,
                   size_t ws_bytes, uint16_t* act, void* stream);

/*
 * L2 grouped GEMM, NT + combine ("Mega MoE" page, Pipeline, grouped_gemm_combine, top-k
 * reduce as a weighted scatter-add): o[r] = act[r] @ W2[e] over the packed w2p [device],
 * then y[t] = sum over the local pairs (t, j) of topk_w[t, j] * o[row of (t, j)],
 * accumulated in fp32 and written as bf16; tokens with no local pair get y[t] = 0.
 *   act [device] bf16 [R_max, I]; topk_w [device] fp32 [T, k]; y [device] bf16 [T, H]
 */
int32_t moe_gemm2_combine(const moe_shape* shape, const uint16_t* act, const uint16_t* w2p,
                          const float* topk_w, void* ws, size_t ws_bytes, uint16_t* y,
                          void* stream);

/*
 * Fused forward: prologue, dispatch + L1 + SwiGLU, L2 + combine, in one call on one stream.
 * With shape->train nonzero the pre-activation rows are also kept in ws (layout hgu) for the
 * backward entry points.
 *   x [device] bf16 [T, H]; topk_idx [device] int32 [T, k]; topk_w [device] fp32 [T, k];
 *   w1p, w2p [device] packed weights (moe_pack_weights); y [device] bf16 [T, H]
 */
int32_t moe_forward(const moe_shape* shape, const uint16_t* x, const int32_t* topk_idx,
                    const float* topk_w, const uint16_t* w1p, const uint16_t* w2p, void* ws,
                    size_t ws_bytes, uint16_t* y, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same stages as moe_forward, with the workspace in a fixed device array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs on until the
 * process ends.  Nothing is allocated or freed by the call.
 *   Arguments as for moe_forward, without ws; shape->train must be 0 (MOE_ERR_SHAPE otherwise).
 *   MOE_ERR_SCRATCH when moe_workspace_bytes(shape) exceeds MOE_NOALLOC_SCRATCH_BYTES (e.g.
 *   256 tokens of the DeepSeek-V3 share with top-8 fit; 8192 do not).
 * Every call on one GPU uses that GPU's one array and leaves its contents behind: calls that
 * overlap on one GPU (two streams, or two threads) race and must be serialised by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (256u * 1024u * 1024u)
int32_t moe_forward_noalloc(const moe_shape* shape, const uint16_t* x, const int32_t* topk_idx,
                            const float* topk_w, const uint16_t* w1p, const uint16_t* w2p, uint16_t* y,
                            void* stream);

/*
 * Backward entry points ("Mega MoE" page, Pipeline, backward).  They need a workspace with
 * shape->train nonzero that a moe_forward of the same inputs filled (tables, act, hgu), and run
 * in this order on one stream: moe_bwd_gemm2_dgrad (or it without the SwiGLU transpose, then
 * moe_swiglu_bwd), then moe_wgrad2, moe_wgrad1 and moe_bwd_gemm1_dgrad_combine in any order.
 * They use ws regions that are dead at that point as scratch: moe_wgrad2 and moe_wgrad1 overwrite
 * ws stage (after the forward's combine has consumed it) to hold their operands in MFMA-fragment
 * order; when the expected rows per local expert (T * k / E) are at least 256 (and the shape
 * allows) the GEMMs run on the forward's pipeline, moe_bwd_gemm2_dgrad then overwrites ws stage
 * and moe_bwd_gemm1_dgrad_combine ws dact.
 *
 * L2 dgrad, NN: dact[r] = topk_w[p] * (dy[t] @ W2[e]^T) with p = row_pair[r], t = p / k, read
 * from the packed w2p as the [K = H, N = I] operand.  With fuse_swiglu_bwd nonzero the
 * epilogue applies the SwiGLU transpose and writes ws dhgu / dhgu_lo directly; else it writes
 * ws dact (fp32).  Either way it recomputes the activation a = silu(g) * u in fp32 from the saved
 * pre-activation and writes ws wact / wact_lo = topk_w[p] * a (the operand of moe_wgrad2).
 * With dtopk_w non-NULL it also writes the gradient of the routing weights, the derivative of
 * the weighted scatter-add y[t] = sum_j topk_w[t, j] * o_p:
 *   dtopk_w [device] fp32 [T, k]: dtopk_w[t, j] = <dy[t], o_p> for a local pair p = t*k + j,
 *   computed as <dy[t] @ W2[e]^T, a[r]> (the same value, since o_p = a[r] @ W2[e]); 0 for a pair
 *   this GPU does not handle (its partial of the gradient).
 *   dy [device] bf16 [T, H]; topk_w [device] fp32 [T, k]
 */
int32_t moe_bwd_gemm2_dgrad(const moe_shape* shape, const uint16_t* dy, const float* topk_w,
                            const uint16_t* w2p, void* ws, size_t ws_bytes,
                            int32_t fuse_swiglu_bwd, float* dtopk_w, void* stream);

/* SwiGLU transpose ("Mega MoE" page, SwiGLU bwd): from ws dact and ws hgu (both fp32), with
 * s = sigmoid(g): dgate = dact * u * s * (1 + g * (1 - s)), dup = dact * g * s -> ws dhgu /
 * dhgu_lo. */
int32_t moe_swiglu_bwd(const moe_shape* shape, void* ws, size_t ws_bytes, void* stream);

/*
 * L1 dgrad, NN, and its combine ("Mega MoE" page, Pipeline, backward: the conjugate of dispatch +
 * L1 sends each row's gradient back to its token): for every real row r of pair p = (t, j),
 * dX[r] = dhgu[r] @ W1[e]^T, read from the packed w1p as the [K = 2I, N = H] operand, then
 *   dx [device] bf16 [T, H]: dx[t] = sum over the local pairs of t of dX[row of the pair],
 *   summed in fp32 in slot order (deterministic); 0 for a token with no local pair.
 * Reads ws dhgu (moe_bwd_gemm2_dgrad with fuse_swiglu_bwd, or moe_swiglu_bwd); uses ws stage.
 */
int32_t moe_bwd_gemm1_dgrad_combine(const moe_shape* shape, const uint16_t* w1p, void* ws,
                                    size_t ws_bytes, uint16_t* dx, void* stream);

/* dW2 with variable K ("Mega MoE" page, backward: dW2 (variable-K)):
 * dW2[e] [I, H] = sum over rows r of e of (topk_w[p] * act[r])^T (x) dy[t]; K = count of e.
 * Reads the weighted activation rows ws wact / wact_lo that moe_bwd_gemm2_dgrad wrote; dy
 * [device] bf16 [T, H].  An expert without rows gets exact zeros.  dw2p [device] bf16,
 * EL * H * I elements, in the packed layout of w2p (moe_unpack_weights gives the logical
 * [EL, I, H]). */
int32_t moe_wgrad2(const moe_shape* shape, const uint16_t* dy, void* ws, size_t ws_bytes,
                   uint16_t* dw2p, void* stream);

/* dW1, TN with variable K ("Mega MoE" page, backward: dW1 (TN); Core Design section 2):
 * dW1[e] [H, 2I] = sum over rows r of e of x[row_pair[r] / k]^T (x) dhgu[r] (hi and lo parts),
 * re-gathering the token rows instead of saving them.  dw1p [device] bf16, EL * 2I * H elements, in the
 * packed layout of w1p (moe_unpack_weights gives the logical [EL, H, 2I]). */
int32_t moe_wgrad1(const moe_shape* shape, const uint16_t* x, void* ws, size_t ws_bytes,
                   uint16_t* dw1p, void* stream);

/* Fused backward: L2 dgrad with the SwiGLU transpose in its epilogue (and the routing-weight
 * gradient when dtopk_w is non-NULL), dW2, dW1, then the L1 dgrad with its combine when dx is
 * non-NULL (w1p is then required; it may be NULL otherwise).  Outputs as in the stage entry
 * points above: dw1p, dw2p packed bf16; dx bf16 [T, H]; dtopk_w fp32 [T, k]. */
int32_t moe_backward(const moe_shape* shape, const uint16_t* x, const uint16_t* dy,
                     const float* topk_w, const uint16_t* w1p, const uint16_t* w2p, void* ws,
                     size_t ws_bytes, uint16_t* dw1p, uint16_t* dw2p, uint16_t* dx,
                     float* dtopk_w, void* stream);

/*
 * MX variant ("How Mega MoE Overlaps ..." page, Code Example: FP8 activations cast per token with
 * UE8M0 scale factors over groups of 32 along K, weights transformed to FP4, a fused forward with
 * an activation clamp).  Formats (OCP microscaling): FP8 E4M3 (largest 448), FP4 E2M1 (values 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6); every 32 consecutive values along K share a scale 2^E stored as the
 * byte E + 127, E the smallest integer with max|v| <= (largest value) * 2^E (0 for a block of
 * zeros); values are v / 2^E rounded to nearest, ties to the even mantissa.
 *
 * FP8 cast of bf16 rows (the per-token cast):
 *   x      [device] bf16 [rows, cols], cols a multiple of 32
 *   codes  [device] uint8 [rows, cols]       FP8 E4M3 codes
 *   scales [device] uint8 [rows, cols / 32]  UE8M0 bytes
 * MOE_ERR_SHAPE for rows < 0 or cols not a positive multiple of 32; x and codes 16-byte aligned.
 */
int32_t moe_mx_cast_fp8(int64_t rows, int32_t cols, const uint16_t* x, uint8_t* codes, uint8_t* scales,
                        void* stream);

/*
 * One-time FP4 transform of the weights (the weight transform of the page's example), from the
 * logical w1 [EL, H, 2I] / w2 [EL, I, H] bf16 (each output column quantized in blocks of 32 along
 * its reduction index) into the operand layout of the block-scaled MFMA:
 *   w1q [device] uint8, EL * 2I * H / 2 bytes;  w1s [device] uint8, EL * 2I * H / 32 bytes
 *   w2q [device] uint8, EL * H * I / 2 bytes;   w2s [device] uint8, EL * H * I / 32 bytes
 * Per expert (N output columns, reduction length K; N = 2I, K = H for W1 and N = H, K = I for W2;
 * the expert's data starts at e * N * K / 2, its scales at e * N * K / 32), with j = k / 64 and
 * l = n % 32 + 32 * ((k % 64) / 32), the data of column n and reduction index k is nibble k % 32
 * (low nibble first) of the 16 bytes at (((n / 32) * (K / 64) + j) * 64 + l) * 16, and its block's
 * scale the byte at (n / 32) * (K / 64) * 64 + (j / 4) * 256 + l * 4 + j % 4 (one dword per lane
 * holds the scales of four K steps).  For W1, n is the packed L1 column (moe_pack_weights).
 * H and I must be multiples of 256 (MOE_ERR_SHAPE otherwise).  Either triple may be NULL.
 */
int32_t moe_mx_pack_weights(const moe_shape* shape, const uint16_t* w1, const uint16_t* w2, uint8_t* w1q,
                            uint8_t* w1s, uint8_t* w2q, uint8_t* w2s, void* stream);

/*
 * Fused MX forward: the routing prologue, the dispatch gather of FP8 x rows with L1 on the
 * block-scaled MFMA (FP8 x FP4 into fp32 accumulators; the instruction itself rounds more coarsely
 * than fp32, by up to 2^-12 of the magnitudes it sums), SwiGLU with its inputs clamped (gate to at
 * most clamp, up to [-clamp, clamp]; clamp <= 0: no clamp), the activation rows cast to FP8 per
 * group of 32, L2 on the block-scaled MFMA, and the combine of moe_gemm2_combine (y bf16).
 *   xq [device] uint8 [T, H], xs [device] uint8 [T, H / 32]  (moe_mx_cast_fp8 of x)
 *   w1q, w1s, w2q, w2s [device]                              (moe_mx_pack_weights)
 *   topk_idx, topk_w, ws, y as for moe_forward.  The act region of ws holds the FP8 activation
 *   codes [R_max, I] followed by their scale bytes slot-major, [I / 256][R_max][8]: byte b of row r
 *   in slot j is the scale of columns 32 (8 j + b) .. 32 (8 j + b) + 31 of row r (0 for a padding
 *   row of a tile).  The stage region is scratch (x's scale bytes in row order during L1).
 * H and I must be multiples of 256.
 */
int32_t moe_forward_mx(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs, const int32_t* topk_idx,
                       const float* topk_w, const uint8_t* w1q, const uint8_t* w1s, const uint8_t* w2q,
                       const uint8_t* w2s, float clamp, void* ws, size_t ws_bytes, uint16_t* y, void* stream);

/*
 * The two GEMM stages of moe_forward_mx on their own, after moe_route_prologue on the same ws:
 * moe_mx_dispatch_gemm1 writes the FP8 activation rows and their scales into the act region;
 * moe_mx_gemm2_combine reads them and writes y (its combine, as in moe_gemm2_combine).  Arguments
 * and errors as for moe_forward_mx.
 */
int32_t moe_mx_dispatch_gemm1(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs, const uint8_t* w1q,
                              const uint8_t* w1s, float clamp, void* ws, size_t ws_bytes, void* stream);
int32_t moe_mx_gemm2_combine(const moe_shape* shape, const uint8_t* w2q, const uint8_t* w2s, const float* topk_w,
                             void* ws, size_t ws_bytes, uint16_t* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
