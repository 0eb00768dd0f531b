/*
 * bi.h -- batch-invariant GEMM library for AMD Instinct MI355X (gfx950).
 *
 * A batch-invariant linear layer returns, for every row of X, the same bits
 * whatever the number of rows M it is computed with.  The library gets there
 * by making the whole reduction recipe -- matrix instruction, which k values
 * share one instruction and in which slot, the width BLOCK_K of a k tile, and
 * the order in which the k tiles are added -- a function of (dtype, N, K)
 * alone.  M only decides which kernel shape carries the recipe out, never the
 * recipe itself.
 *
 * Sources: "[BI][DSv4] Batch-invariant GateLinear router with fp32 persistent
 * matmul" (sections "What", "Tests", "Review follow-up" and "A correction to
 * why the key excludes M"), and "Batch-invariance generation with vLLM
 * fused-MoE backend" ("What's included" and the strict-review summary).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers on the current HIP device, owned
 *    by the caller.  The library allocates no device memory, never
 *    synchronises the host, enqueues its kernels on `stream` and returns.
 *  - Weights use the nn.Linear layout: W is [N, K] row-major with row pitch
 *    `ldw` elements, i.e. exactly the memory behind the transposed view
 *    W.t() ([K, N], strides (1, ldw)) that a linear layer hands to its matmul.
 *    No other weight layout is accepted.
 *  - X is [M, K] row-major with row pitch `ldx`; Y is [M, N] row-major with
 *    row pitch `ldy`.  Base pointers must be 16-byte aligned and row pitches
 *    must keep every row 16-byte aligned.
 *  - `ws` is a caller-owned device workspace of at least the size reported by
 *    the matching *_workspace_size() call (16-byte aligned; NULL when that
 *    size is 0).  Its first 16 KiB hold the arrival counters of the
 *    one-launch decode kernel: they must be ZERO when the workspace is first
 *    used (zero-fill it once at allocation), no call writes anything else
 *    there, and every call leaves them zero.  The rest holds intermediate
 *    tile partials and needs no initialisation (every byte of it a call reads
 *    it has written earlier in the same call).  One workspace serves calls of
 *    any shape in sequence; two calls in flight at the same time must not
 *    share one workspace.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    rejected call enqueues nothing.  There is no fallback to a
 *    non-invariant path: a shape the recipe table cannot serve returns
 *    BI_EUNSUPPORTED.  M == 0 returns BI_OK and enqueues nothing.
 *  - Global state and thread safety: the library's mutable global state is
 *    per-device values written once and then only read (the compute-unit
 *    count; the device address of bi_linear_f32_noalloc's static scratch,
 *    behind a once-flag) and that scratch array itself, which the calls of
 *    bi_linear_f32_noalloc on one GPU share.  Every other entry point reads
 *    and writes only caller memory, so calls from several host threads are
 *    safe as long as they do not share a workspace or an output.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BI_OK = 0,
    BI_EINVAL = 1,        /* null/misaligned pointer, negative size, bad pitch   */
    BI_EUNSUPPORTED = 2,  /* (dtype, N, K) outside what the recipe table serves  */
    BI_EWORKSPACE = 3,    /* ws missing or smaller than *_workspace_size()       */
    BI_EHIP = 4           /* a HIP launch failed; see hipGetLastError()         */
} bi_status_t;

typedef enum { BI_F32 = 0, BI_BF16 = 1 } bi_dtype_t;

/* How the per-element k reduction is carried out.
 * BI_R2_TILE_PARTIAL: K is cut into tiles of block_k; each tile's partial sum
 *   is formed from zero by a chain of matrix instructions in ascending k, and
 *   the tile partials are added into one fp32 accumulator in ascending tile
 *   order: acc = P_0; acc = acc + P_1; ... .  block_k == K is the fully
 *   chained recipe (one accumulator threaded through every k block).      */
typedef enum { BI_R2_TILE_PARTIAL = 2 } bi_reduce_t;

typedef enum {
    BI_MFMA_F32_16X16X4_F32 = 1,   /* fp32 operands, 4 products per instruction  */
    BI_MFMA_F32_16X16X32_BF16 = 2  /* bf16 operands, 32 products per instruction */
} bi_mfma_t;

/* The numeric recipe of a (dtype, N, K) key.  Every field is a function of
 * the key only; bi_describe_recipe() takes no M, by design. */
typedef struct {
    int32_t dtype;          /* bi_dtype_t of the operands                        */
    int32_t mfma;           /* bi_mfma_t                                         */
    int32_t k_group;        /* k values per lane slot in one 32-wide k block: 8.
                               Slot g (g = 0..3) of a block starting at k0 holds
                               k0+8g .. k0+8g+7; an fp32 instruction s (0..7)
                               takes element s of each slot, a bf16 instruction
                               takes all eight.                                  */
    int32_t reduce;         /* bi_reduce_t                                       */
    int32_t block_k;        /* width of one tile partial (multiple of 32)        */
    int32_t bias_last;      /* 1: bias is added once, after the full reduction   */
    int32_t m_decode_max;   /* largest M served by the k-tile-parallel decode
                               kernel; larger M uses the persistent kernel.  This
                               picks a kernel shape, never the numerics.         */
    int32_t reserved;
} bi_recipe_t;

/* Y[M,N] = X[M,K] . W^T + bias, all fp32, fp32 accumulation.
 * GateLinear page, "What": the router GEMM is computed in the input dtype
 * (fp32) and its scores never round through bf16; bias and skip-bias are
 * preserved ("Review follow-up").  bias may be NULL (no bias term). */
bi_status_t bi_linear_f32(const float* x, int64_t ldx,
                          const float* w, int64_t ldw,
                          const float* bias,
                          float* y, int64_t ldy,
                          int64_t M, int64_t N, int64_t K,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Y[M,N] = X[M,K] . W^T + bias with bf16 X and W (uint16 bit patterns), fp32
 * accumulation, fp32 bias (or NULL), and Y stored as bf16 (round to nearest
 * even, y_dtype == BI_BF16) or fp32 (y_dtype == BI_F32).  GateLinear page,
 * "A correction to why the key excludes M": the bf16 path goes through
 * matrix cores, so its recipe is pinned just as the fp32 one is. */
bi_status_t bi_linear_bf16(const uint16_t* x, int64_t ldx,
                           const uint16_t* w, int64_t ldw,
                           const float* bias,
                           void* y, int32_t y_dtype, int64_t ldy,
                           int64_t M, int64_t N, int64_t K,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* bi_linear_f32 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments, plan and kernels, hence the same bits, with no caller
 * workspace.  The workspace is a static device array of the library, 16 MiB
 * + 16 KiB per GPU, held until the process ends; a plan that splits the k
 * tiles of its fp32 ring tiles over workgroups (tile codes 28, 29) and needs
 * more runs those tiles unsplit, with the same bits and no workspace; any
 * other shape whose plan needs more (none of the compiled fp32 keys up to
 * its decode limit) returns BI_EWORKSPACE before anything is enqueued.  Its first call on a device
 * finds the array's address and clears its counters with a small kernel on
 * `stream`.  The library allocates nothing here.  All calls on one GPU share
 * the array: calls that overlap on one GPU (other streams, other host threads)
 * race and must be serialised by the caller. */
bi_status_t bi_linear_f32_noalloc(const float* x, int64_t ldx,
                                  const float* w, int64_t ldw,
                                  const float* bias,
                                  float* y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Batch-invariant MoE layer with gated SwiGLU experts (fused-MoE page, "What's
 * included"; strict-review summary):
 *   logits = fp32(x) . w_router^T (+ b_router)      fp32 router, recipe of
 *                                                    key (fp32, E, H)
 *   topk_ids[m, j]  : j-th largest logit, exact ties to the lower expert index,
 *                     -0.0 equal to +0.0
 *   topk_probs[m,j] : softmax over all E logits of the chosen expert (fp32,
 *                     not renormalised over the top-k)
 *   h   = bf16( x . w13[e]^T )       w13[e] = [gate rows 0..I-1 ; up rows I..2I-1]
 *   a   = bf16( silu(gate) * up * p )  fp32 math, one rounding; the routing
 *                                      probability is applied here
 *   y_j = a . w2[e]^T                 fp32 accumulation, fp32 partial per slot
 *   y[m] = fp32( sum_{j = 0..topk-1} (double) y_j )   unit weights, fp64, slot order
 * Layouts: x [M,H] bf16, w_router [E,H] fp32, b_router [E] fp32 or NULL,
 * w13 [E, 2I, H] bf16, w2 [E, H, I] bf16 (each expert an nn.Linear weight),
 * topk_ids [M,topk] int32, topk_probs [M,topk] fp32, y [M,H] fp32; all
 * contiguous.  Expert counts stay on the device (no host synchronisation).
 * Requires H % 32 == 0, I % 32 == 0, E <= 1024, topk <= E and topk <= 32. */
bi_status_t bi_moe_grouped_gemm(const uint16_t* x,
                                const float* w_router, const float* b_router,
                                const uint16_t* w13, const uint16_t* w2,
                                int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk,
                                int32_t* topk_ids, float* topk_probs, float* y,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* Deterministic per-row top-k of indexer scores (sparse-attention indexer;
 * "[BI][DSv4] Pin sparse-MLA decode and prefill scheduling under batch
 * invariance", commit notes of the deterministic per-row top-k).
 *   scores  [rows, cols] fp32, row pitch ld elements (ld >= cols); any fp32
 *           bit pattern, NaNs included.
 *   row_start, row_end  [rows] int64 or NULL (NULL: 0 and cols): row r's
 *           window is [clamp(row_start[r], 0, cols), clamp(row_end[r], 0, cols)).
 *   out     [rows, topk] int32, row pitch ld_out (>= topk).
 * Ranking: -0.0 counts as +0.0; scores are ranked by the monotone 32-bit key
 * of their bit pattern (positive NaNs above +inf, negative NaNs below -inf);
 * exact ties go to the lower column; lanes outside the window are never
 * selected and never take a tied slot.  Row r receives the min(topk, window
 * length) best lanes as window-relative column indices in ascending order,
 * followed by -1 in the remaining slots.  The result is a function of the
 * row's own scores and window only.  Requires cols <= 8192 (BI_EUNSUPPORTED
 * otherwise: there is no fallback).  Pointers are 4-byte (scores, out) and
 * 8-byte (bounds) aligned device pointers; no workspace. */
bi_status_t bi_indexer_topk(const float* scores, int64_t ld, int64_t rows, int64_t cols,
                            const int64_t* row_start, const int64_t* row_end, int64_t topk,
                            int32_t* out, int64_t ld_out, hipStream_t stream);

/* Activation and top-k-sum options of the MoE layer (fused-MoE page, "What's
 * included" and the strict-review summary: the batch-invariant MoE first
 * shipped a squared-ReLU activation; the top-k sum has an (apply_weights,
 * acc_fp64) option matrix, and every point of it must do what it says --
 * the unweighted fp32 point applies no weights). */
typedef enum { BI_ACT_SWIGLU = 0, BI_ACT_SQRELU = 1 } bi_activation_t;

typedef struct {
    int32_t activation;           /* bi_activation_t                                  */
    int32_t probs_at_activation;  /* 1: a = RN_bf16(act * p) (probability applied at
                                     the activation); 0: a = RN_bf16(act)             */
    int32_t apply_weights;        /* 1: the top-k sum weights slot j by p_j           */
    int32_t acc_fp64;             /* 1: the top-k sum runs in binary64, one rounding
                                     to fp32; 0: fp32 adds from +0 in slot order
                                     (fp32 products when weighted)                   */
} bi_moe_options_t;

/* The MoE layer with explicit options.  SwiGLU: w1 is [E, 2I, H] (gate rows,
 * then up rows), act = silu(g) * u; squared-ReLU: w1 is [E, I, H],
 * act = max(h, 0)^2 of the bf16 storage point h.  options == NULL is the
 * configuration of bi_moe_grouped_gemm (SwiGLU, probability at the
 * activation, unweighted binary64 sum).  Setting both probs_at_activation and
 * apply_weights would apply the probability twice and returns BI_EINVAL, as
 * does any field outside its range.  Everything else as bi_moe_grouped_gemm;
 * the workspace size does not depend on the options. */
bi_status_t bi_moe_grouped_gemm_ex(const uint16_t* x,
                                   const float* w_router, const float* b_router,
                                   const uint16_t* w1, const uint16_t* w2,
                                   int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk,
                                   const bi_moe_options_t* options,
                                   int32_t* topk_ids, float* topk_probs, float* y,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes the calls above need for a given problem (0 if none, or if
 * the arguments are invalid).  For the linear layer the workspace holds the
 * counter region and the k tile partials of the decode kernel M selects
 * (GateLinear page, "A correction to why the key excludes M": M picks the
 * kernel shape, never the recipe), so its size depends on M while the
 * results do not.  For the MoE layer it also holds the router logits, the
 * expert-sorted routing, the bf16 activations and the fp32 slot partials
 * (fused-MoE page, "What's included": expert counts and routing stay on the
 * device).  Pure host computations; nothing is enqueued. */
size_t bi_linear_workspace_size(int32_t dtype, int64_t M, int64_t N, int64_t K);
size_t bi_moe_workspace_size(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk);

/* The recipe of a key; takes no M (GateLinear page, "What" and "A correction
 * to why the key excludes M": the config is keyed on (dtype, N, K) and never
 * on M).  out: host pointer.  Returns BI_EUNSUPPORTED for keys the table
 * cannot serve, BI_EINVAL for a NULL out or an unknown dtype. */
bi_status_t bi_describe_recipe(int32_t dtype, int64_t N, int64_t K, bi_recipe_t* out);

/* Static, never-freed string naming a status code (Sparse-MLA page, the
 * fail-closed review notes: a call that cannot keep batch invariance reports
 * an error instead of returning a batch-dependent result). */
const char* bi_status_str(bi_status_t status);

/* ---------------------------------------------------------------------------
 * Experiment and control entry points.  Not for production use.
 * ------------------------------------------------------------------------- */

/* Path selectors for bi_lab_linear().  BI_PATH_DECODE: k tile partials on
 * separate waves across the chip, folded by a second launch (workspace).
 * BI_PATH_DECODE_XCD: the same waves and the same fold in one launch -- the
 * wave that arrives last at its output tile's counter folds the tile's
 * partials (workspace; recipes with several k tiles, N a multiple of 128 and
 * at most 128 output-tile groups; BI_EUNSUPPORTED otherwise).
 * BI_PATH_DECODE_WG: one workgroup per 16x16 output tile whose waves share
 * the k tile partials through LDS, one launch, no workspace (recipes with 2
 * to 64 k tiles; BI_EUNSUPPORTED otherwise).  BI_PATH_DECODE_DMA: fully
 * chained bf16 recipes at M <= 64, one workgroup per 16 columns whose loader
 * waves stream W and X into LDS with direct-to-LDS loads for one chain wave
 * (K a multiple of 512 at M <= 16, 256 at M <= 64;
 * BI_EUNSUPPORTED otherwise).  With BI_PATH_PERSISTENT, bits 8..15
 * of `path` may name a persistent tile shape (0: automatic; fp32: 1 = 64x64,
 * 2 = 32x64, 3 = 32x32, 4 = 64x64 on 8 waves, 5 = 128x64, 6 = 64x128,
 * 7 = 32x32 with 32-k stages, 8 = 64x256 with 32-k stages, 9 = 32x64 with
 * 128-k stages, 10 = 64x64 on 8 waves with 128-k stages, 23 = 32x32 on 8
 * waves fed by a ring of 64-k LDS stages through direct-to-LDS loads, four k
 * tiles at a time (two where four do not divide the number of k tiles),
 * 24 = 64x32 likewise, two k tiles at a time; 23 and 24 need K a multiple
 * of 64 and k tiles of an even number of 32-k blocks (23 with several k
 * tiles: at least four blocks); 28 and 29 = 23 and 24 with the k tiles of
 * each output tile split over 2 to 16 workgroups on one XCD whose last
 * arrival folds the partials in k tile order (workspace; a number of tiles
 * that is a multiple of 8 and at most 128, else they run as 23 and 24);
 * bf16: 11 = 128x128, 12 = 64x64, 13 = 128x128 with 128-k stages,
 * 14 = 256x128, 15 = 128x256, 16 = 64x128 with 128-k stages, 17 = 64x64
 * with 32-k stages, 18 = 256x256 on 2x4 waves, 19 = 256x256 on 4x2 waves,
 * 20 = 64x64 on 4x2 waves fed by a ring of eight 64-k LDS stages through
 * direct-to-LDS loads, 21 = 256x256 on 4x2 waves fed by a ring of four 32-k
 * LDS stages through direct-to-LDS loads issued by four of the waves, 22 =
 * the same with all eight waves loading; 18, 19, 21 and 22 serve fully
 * chained recipes only, 20-22 need K a multiple of 64; a shape that cannot
 * serve falls back to another).
 * With BI_PATH_DECODE or BI_PATH_DECODE_XCD, bits 8..15 may force the
 * number of 16-row M tiles one decode wave carries (1, 2 or 4; 0: automatic).
 * Tile shapes never change the numerics. */
enum { BI_PATH_AUTO = 0, BI_PATH_DECODE = 1, BI_PATH_PERSISTENT = 2, BI_PATH_DECODE_WG = 3,
       BI_PATH_DECODE_DMA = 4, BI_PATH_DECODE_XCD = 5 };

/* The same linear layer with an explicit recipe and an explicit kernel path,
 * for A/B experiments (e.g. fully chained vs tile-partial, or one BLOCK_K
 * against another) and for showing that the two kernel paths agree bit for
 * bit.  Results are batch-invariant only while the recipe is held fixed.
 * x/w are fp32 or bf16 per recipe->dtype; y is fp32 or bf16 per y_dtype. */
bi_status_t bi_lab_linear(const void* x, int64_t ldx, const void* w, int64_t ldw,
                          const float* bias, void* y, int32_t y_dtype, int64_t ldy,
                          int64_t M, int64_t N, int64_t K,
                          const bi_recipe_t* recipe, int32_t path,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes bi_lab_linear() needs for this recipe, path and shape. */
size_t bi_lab_workspace_size(const bi_recipe_t* recipe, int32_t path,
                             int64_t M, int64_t N, int64_t K);

/* Negative control (GateLinear page, "What" and "Tests": the default library
 * route split K and switched algorithm with M, so a row's scores changed with
 * the batch).  Same arguments as bi_linear_f32, but BLOCK_K is chosen from M
 * (twice the shipped width for M < 64, the shipped width otherwise): a
 * deliberately M-dependent recipe that is expected to break bitwise
 * invariance.  Its workspace never exceeds bi_linear_workspace_size(). */
bi_status_t bi_negctl_linear_f32(const float* x, int64_t ldx,
                                 const float* w, int64_t ldw,
                                 const float* bias,
                                 float* y, int64_t ldy,
                                 int64_t M, int64_t N, int64_t K,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Diagnostic for the one-launch decode, which needs every workgroup of an
 * output tile on one XCD (one L2): launches a grid_x x grid_y grid of
 * 64-thread workgroups, and workgroup (x, y) writes the id of the XCD it ran
 * on to out[y * grid_x + x].  out: device, 4-byte aligned, grid_x * grid_y
 * uint32 entries.  Workgroups are dispatched to the XCDs round-robin in
 * linear workgroup order, so ids that agree modulo 8 should report one XCD. */
bi_status_t bi_lab_xcc_ids(uint32_t* out, int32_t grid_x, int32_t grid_y, hipStream_t stream);

/* The kernel path (BI_PATH_*) the production entry points pick for M rows of
 * a (dtype, N, K) key -- M picks the kernel shape, never the recipe (GateLinear
 * page, "A correction to why the key excludes M").  path: host pointer to
 * one int32.  BI_EINVAL for M <= 0 or a NULL path, BI_EUNSUPPORTED for keys
 * the recipe table cannot serve. */
bi_status_t bi_lab_plan(int32_t dtype, int64_t M, int64_t N, int64_t K, int32_t* path);

/* Where a MoE call of this shape keeps its storage points in the workspace,
 * for stage-wise checks of the layer (fused-MoE page, "What's included": the
 * bf16 activation with the probability applied and the per-slot down
 * projection are the layer's storage points).  offsets: host int64[4] =
 * byte offsets of the pair list sorted by expert (int32 [M*topk], entry p is
 * the pair m*topk + j of sorted position p), of the activations (bf16
 * [M*topk, I] in sorted-position order) and of the fp32 slot partials
 * ([M*topk, H] in pair order), and the workspace size.  They hold a call's
 * values once it has completed, until the next call on the workspace. */
bi_status_t bi_lab_moe_layout(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk, int64_t* offsets);

/* Measurement floors (GateLinear page, "Update: is the M=4096 cost
 * avoidable?": a decode-sized kernel is judged by its device time, which sits
 * on a per-launch floor).  None of these is on the batch-invariant path.
 *  bi_lab_empty        launches an empty kernel of `grid` workgroups of
 *                      `threads` threads (a multiple of 64, <= 1024): its
 *                      device time is the floor every launch pays.
 *  bi_lab_stream_read  reads `bytes` (a multiple of 16) at `src` (device,
 *                      16-byte aligned) once with `grid` workgroups of 256
 *                      threads and writes one word per workgroup to sink
 *                      (device, `grid` uint32): the cold-read rate the
 *                      chip achieves, the practical HBM reference.
 *  bi_lab_l2_read      each of `grid` workgroups of 256 threads reads the
 *                      same `bytes` at `src` (device, 16-byte aligned; a
 *                      power of two from 32 KiB to 2 MiB, so that it stays
 *                      in every XCD's L2 after the first pass) `iters` times
 *                      and writes one word per workgroup to sink (device,
 *                      `grid` uint32): the rate at which the L2 delivers
 *                      data to the compute units (grid x iters x bytes per
 *                      call).
 *  bi_lab_clock        each of `grid` 64-thread workgroups runs iters x 64
 *                      dependent fp32 multiply-adds and writes three uint64
 *                      to out[3 wg ..]: shader-clock cycles (s_memtime),
 *                      constant-rate wall-clock ticks (s_memrealtime) and a
 *                      value that keeps the chain alive.
 *  bi_lab_lds_read     each of `grid` workgroups of 1024 threads fills 64 KiB
 *                      of LDS and reads it iters x 4 times with
 *                      conflict-free 16-byte loads (64 KiB per round):
 *                      the LDS read rate a compute unit sustains.
 *  bi_lab_mfma_rate    each of `grid` workgroups of 512 threads runs, per
 *                      wave, iters x 8 MFMAs of the recipe's instruction for
 *                      `dtype` (BI_F32: 16x16x4 f32, BI_BF16: 16x16x32
 *                      bf16) on register operands, spread over `chains`
 *                      (1, 2, 4 or 8) independent accumulators taken in
 *                      turn: with 8 the issue rate the matrix cores sustain
 *                      with nothing else in the way, with fewer the rate of
 *                      dependent chains like the recipe's tile partials.
 *                      Both write three uint64 per workgroup to out[3 wg ..]
 *                      (device, 8-byte aligned): shader cycles and wall ticks
 *                      of the loop, and a word that keeps its results alive.
 * Invalid arguments return BI_EINVAL before anything is enqueued. */
bi_status_t bi_lab_empty(int32_t grid, int32_t threads, hipStream_t stream);
bi_status_t bi_lab_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t grid,
                               hipStream_t stream);
bi_status_t bi_lab_l2_read(const void* src, int64_t bytes, int32_t iters, uint32_t* sink, int32_t grid,
                           hipStream_t stream);
bi_status_t bi_lab_clock(uint64_t* out, int32_t grid, int32_t iters, hipStream_t stream);
bi_status_t bi_lab_lds_read(uint64_t* out, int32_t grid, int32_t iters, hipStream_t stream);
bi_status_t bi_lab_mfma_rate(uint64_t* out, int32_t dtype, int32_t chains, int32_t grid, int32_t iters,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_H */
