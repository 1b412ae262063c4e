/*
 * sol_attn.h -- C ABI of the Sol-Attn block-sparse attention library for MI355X (gfx950).
 *
 * What is computed.  Sol-Attn is the training-free sparse attention of the Sol-H3
 * runtime: for every query it decides which parts of the attention computation
 * matter, and it is the largest single source of that runtime's speed-up; its
 * preparation step (the selection that precedes the attention) was itself
 * optimised ("Videomodel MiniMax-H3 rendert sneller dan afspelen", section
 * "Waar de snelheidswinst vandaan komt").  It runs in the high-resolution
 * refinement steps of the two-stage schedule ("NVIDIA Adds Two-Stage Generation
 * for MiniMax H3, ...", first paragraph).  The pages give no formula; this
 * library implements the following concrete reading, in three calls:
 *
 *   sol_attn_pool    Qbar_i = mean of the Bs query rows of block i, Kbar_j likewise
 *                    (tokens are frame-major; block i = tokens [i*Bs, (i+1)*Bs)).
 *   sol_attn_select  r_ij = Qbar_i . Kbar_j; per query block i keep the `topk` key
 *                    blocks j with the largest r_ij, ties to the lower j (the score
 *                    r_ij/sqrt(d) has the same order); emit them in ascending j.
 *   sol_attn_fwd     every query row of block i attends with exact
 *                    softmax(q k^T * scale) over the tokens of its selected key
 *                    blocks only; no mask.
 *
 * Around them: sol_attn_cube_permute, sol_attn_pool_cube and sol_attn_fwd_cube (3-D
 * cube blocks instead of runs of tokens),
 * sol_attn_window_blocks (a static windowed pattern for sol_attn_fwd),
 * sol_attn_check_block_idx (device check of an index list), sol_attn_frame_order (a
 * cache-friendly query-block schedule), sol_attn_quantize / sol_attn_dequantize (the
 * INT8 / FP8 formats of the exchange between GPUs) and sol_attn_probe_mfma (a
 * diagnostic of the sustained matrix-core rate).
 *
 * Layout.  Q, K, V and O are contiguous [B, H, L, d] row-major (d fastest), in the
 * element type given by `dtype`.  Pooled tensors are [B, H, n_blocks, d] float64.
 * The block index list is int32 [B, H, n_blocks, topk], ascending per row.
 *
 * Ownership and execution.  Every pointer argument is a DEVICE pointer owned by
 * the caller; the library allocates no memory and never retains a pointer.  Its only
 * state is one flag per device and select kernel: the first sol_attn_select on a
 * device raises that kernel's dynamic-LDS limit once.  Calls enqueue their kernel(s)
 * on `stream` (a hipStream_t; NULL = the default stream) and return without
 * synchronising; results are valid once the stream has reached that point.  Outputs
 * must not alias inputs.  Calls are thread-safe.
 *
 * Graph capture.  The device calls record kernel launches only (no allocation, memset
 * or copy), so a sequence of them -- e.g. pool, select, fwd -- can be captured into a
 * HIP graph from `stream` and replayed; a replay reads the inputs' current contents.
 * Make one sol_attn_select call on the device before capturing, so that the one-time
 * attribute change above happens outside the capture.
 *
 * Errors.  Argument errors are detected on the host before anything is enqueued
 * and leave every output untouched.  A failure reported by the HIP runtime at
 * launch returns SOL_ATTN_ERR_HIP.  sol_attn_last_error() describes the most
 * recent failure on the calling thread.  Faults inside a kernel surface at the
 * caller's next synchronisation, as for any HIP library.  Problems with zero
 * elements (B*H*L == 0) are valid and enqueue nothing (sol_attn_check_block_idx still
 * writes its count of 0).
 */
#ifndef SOL_ATTN_H_
#define SOL_ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SOL_ATTN_VERSION 102  /* major*100 + minor */

typedef enum {
  SOL_ATTN_BF16 = 0,  /* bfloat16 inputs/outputs, float32 accumulation */
  SOL_ATTN_FP32 = 1,  /* float32 inputs/outputs, float32 arithmetic */
  SOL_ATTN_DTYPE_INT_RANGE_ = 0x7fffffff  /* not a dtype: makes any int a valid value of the type, so an
                                             unknown code is rejected (SOL_ATTN_ERR_UNSUPPORTED), never UB */
} sol_attn_dtype_t;

typedef enum {
  SOL_ATTN_OK = 0,
  SOL_ATTN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  SOL_ATTN_ERR_SHAPE = 2,       /* negative size, d/block <= 0, or infinite scale      */
  SOL_ATTN_ERR_K = 3,           /* topk < 1 or topk > n_blocks                         */
  SOL_ATTN_ERR_UNSUPPORTED = 4, /* dtype / d / block combination not built (see calls) */
  SOL_ATTN_ERR_ALIGN = 5,       /* pointer not aligned as the call requires            */
  SOL_ATTN_ERR_HIP = 6          /* the HIP runtime rejected a launch                   */
} sol_attn_status_t;

/*
 * Blocks: the sequence of L tokens is cut into n_blocks = ceil(L / block) contiguous
 * blocks; block i holds tokens [i*block, min((i+1)*block, L)).  When block does not
 * divide L the last block is short: its mean is over its own tokens, as a key block it
 * contributes exactly those tokens, and as a query block only its existing rows are
 * written.
 *
 * Block mean-pooling of Q and K (the first half of the selection "preparation").
 *   q, k        [B,H,L,d] of `dtype`; 16-byte aligned.
 *   q_pooled,   [B,H,n_blocks,d] float64 outputs; 8-byte aligned.
 *   k_pooled    Element (b,h,i,e) = (sum over block i's rows of x[b,h,row,e]) / (its row count).
 *               The block sum is accumulated in float64 (exact whenever the block's
 *               values span less than ~2^35 in magnitude, so then order-independent);
 *               the division is IEEE-correctly rounded.
 * Supported: dtype BF16 with d % 8 == 0, or FP32 with d % 4 == 0; d <= 512; any block >= 1.
 */
sol_attn_status_t sol_attn_pool(const void* q, const void* k, sol_attn_dtype_t dtype, int B, int H, int L, int d, int block,
                                double* q_pooled, double* k_pooled, void* stream);

/*
 * Top-k key-block selection per query block (the second half of the preparation).
 *   q_pooled, k_pooled  [B,H,n_blocks,d] float64 (as written by sol_attn_pool); 8-byte aligned.
 *   block_idx           int32 [B,H,n_blocks,topk] output, ascending per row; 4-byte aligned.
 *                       Row (b,h,i) holds the first `topk` key blocks j in the order
 *                       (r_ij descending, j ascending), r_ij = sum_e Qbar_ie*Kbar_je in float64.
 *   scores_or_null      optional float64 [B,H,n_blocks,n_blocks] output of r_ij/sqrt(d).
 * Supported: 1 <= d <= 512, n_blocks <= 8192, 1 <= topk <= n_blocks.  -0.0 and +0.0 rank as equal.
 * Rows whose scores contain NaN get an unspecified (but in-range) selection.
 */
sol_attn_status_t sol_attn_select(const double* q_pooled, const double* k_pooled, int B, int H, int n_blocks, int d,
                                  int topk, int32_t* block_idx, double* scores_or_null, void* stream);

/*
 * Block-sparse exact softmax attention over the selected key blocks.
 *   q, k, v        [B,H,L,d] of `dtype`; 16-byte aligned.
 *   block_idx      int32 [B,H,n_blocks,topk]; every entry must lie in [0, n_blocks) and the
 *                  entries of a row must be strictly ascending (sol_attn_select and
 *                  sol_attn_window_blocks emit such rows; sol_attn_check_block_idx checks a
 *                  list on the device).  Out-of-range entries are clamped into range
 *                  instead of faulting, and other orders never fault either; the affected
 *                  rows' results are then unspecified.
 *   qblock_order_or_null
 *                  optional int32 [n_blocks] device array: a permutation of the query blocks
 *                  giving the order in which they are scheduled (shared by all (b,h)).
 *                  It changes only which blocks run concurrently -- and so how often K/V
 *                  tiles are re-read from cache rather than memory -- never the results.
 *                  NULL = ascending.  Entries outside [0, n_blocks) are clamped; a non-
 *                  permutation leaves some output rows unwritten.  See sol_attn_frame_order.
 *   softmax_scale  multiplier of q.k inside the softmax; a value <= 0 or NaN selects
 *                  1/sqrt(d); +infinity is rejected with SOL_ATTN_ERR_SHAPE.
 *   out            [B,H,L,d] of `dtype`: O = softmax(q K_sel^T * scale) V_sel per query row;
 *                  bf16 results are rounded to nearest-even from float32.
 *   lse_or_null    optional float32 [B,H,L]: natural-log log-sum-exp of the scaled logits.
 * Supported: BF16 with d == 128 and block == 128 (matrix-core path, float32 accumulation;
 * probabilities are rounded to bf16 before the P.V product), or FP32 with d in {64,128}
 * and 1 <= block <= 256.  16-byte alignment for q,k,v,out; 4-byte for lse and block_idx.
 *
 * Deliberate differences from the plain three-call interface (pool, select, fwd over
 * Q/K/V [B,H,L,d] plus block size and k), each a strict extension:
 *   - qblock_order_or_null is an extra argument; NULL gives the plain call.  It exists
 *     because the launch order decides how many gathered K/V tiles come from cache, and
 *     only the caller knows the latent grid that makes a good order.
 *   - L need not be a multiple of block (a short last block, described above) instead of
 *     being rejected with SOL_ATTN_ERR_SHAPE.
 *   - FP32 accepts any block in [1, 256], not only 64 and 128.
 *   - block_idx is not checked inside this call (no device error word); rows are clamped
 *     into range so a bad list cannot fault, and sol_attn_check_block_idx validates a
 *     list on the device when the caller wants it.
 */
sol_attn_status_t sol_attn_fwd(const void* q, const void* k, const void* v, sol_attn_dtype_t dtype, int B, int H, int L, int d,
                               int block, int topk, const int32_t* block_idx, const int32_t* qblock_order_or_null,
                               float softmax_scale, void* out, float* lse_or_null, void* stream);

/*
 * Device-side validation of a block index list (for lists not made by sol_attn_select,
 * e.g. static patterns): counts the rows of block_idx [B,H,n_blocks,topk] that
 * sol_attn_fwd does not accept -- an entry outside [0, n_blocks), or entries that are
 * not strictly ascending (a repeated entry included).
 *   bad_rows  device int32 output: the number of such rows (0: the list is valid).  It
 *             is zeroed and then counted on `stream`; read it after synchronising.
 * Returns SOL_ATTN_ERR_SHAPE for negative sizes, SOL_ATTN_ERR_NULL for a NULL bad_rows
 * (or a NULL block_idx with rows to check), SOL_ATTN_ERR_ALIGN for pointers not 4-byte
 * aligned.  topk == 0 or no rows: bad_rows is set to 0.
 */
sol_attn_status_t sol_attn_check_block_idx(const int32_t* block_idx, int B, int H, int n_blocks, int topk, int32_t* bad_rows,
                                           void* stream);

/*
 * Host helper (no GPU work): a query-block schedule for frame-major video tokens.
 * Tokens are frame-major with `frame_tokens` tokens per latent frame and `row_tokens`
 * per latent row (the latent grid of a clip is frames x rows x cols; Sol-H3-VAE model
 * card, section "Usage").  Query blocks covering the same latent rows in different
 * frames select similar key blocks, so the order sorts blocks by (row of their first
 * token, frame, index): neighbouring entries then share K/V tiles in cache.
 *   order_host  HOST int32 [n_blocks] output (caller-owned).
 * Returns SOL_ATTN_ERR_SHAPE unless block > 0, L >= 0, frame_tokens > 0 and
 * 0 < row_tokens <= frame_tokens.
 */
sol_attn_status_t sol_attn_frame_order(int L, int block, int frame_tokens, int row_tokens, int32_t* order_host);

/*
 * Host helper (no GPU work): a static block-sparse pattern for sol_attn_fwd, the
 * decoder-style windowed attention (Sol-H3-VAE model card: whole frames with windowed
 * attention, each native 5-latent block decoded bidirectionally) expressed as a fixed
 * key-block list.  Query block i attends to the `topk` consecutive key blocks
 * [s, s + topk) with s = clamp(i - (topk - 1) / 2, 0, n_blocks - topk): a window of
 * frame-major tokens centred on the query block (for even topk one more block after it
 * than before it) and shifted inwards at the ends, so every row has exactly topk
 * entries, contains i and is ascending.
 *   idx_host  HOST int32 [n_blocks][topk] output (caller-owned); pass it (copied to the
 *             device, once per (b, h)) as block_idx of sol_attn_fwd.
 * Returns SOL_ATTN_ERR_SHAPE if n_blocks < 0, SOL_ATTN_ERR_K unless 1 <= topk <= n_blocks
 * (when n_blocks > 0), SOL_ATTN_ERR_NULL for a NULL output with n_blocks > 0.
 */
sol_attn_status_t sol_attn_window_blocks(int n_blocks, int topk, int32_t* idx_host);

/*
 * Token reordering for 3-D cube blocks (device copy).  The tokens of a clip form a
 * T x h x w latent grid (frames x rows x cols; Sol-H3-VAE model card, section "Usage"),
 * stored frame-major: token n = (t*h + y)*w + x.  A cube block is a bt x by x bx box of
 * that grid.  Cube-major order numbers the boxes like the tokens (time slowest, then
 * row, then column) and keeps the frame-major order of the tokens inside a box, so box
 * c is tokens [c*V, (c+1)*V) of the reordered sequence, V = bt*by*bx.  Pooling, scoring
 * and softmax only see token sets, so block-sparse attention with cube blocks is:
 *   1. cube_permute Q, K, V (inverse = 0);
 *   2. sol_attn_pool / sol_attn_select / sol_attn_fwd with block = V on the reordered
 *      tensors (block_idx then indexes boxes);
 *   3. cube_permute O (and lse, with row_bytes = 4) back with inverse = 1.
 * A model whose token-wise layers do not care about order can keep its activations in
 * cube-major order and skip steps 1 and 3.  sol_attn_pool_cube and sol_attn_fwd_cube
 * (below) do steps 1-3 without the copies, reading the frame-major tensors in place.
 *   src, dst    [B,H,T*h*w] rows of row_bytes bytes each (a [B,H,L,d] tensor has
 *               row_bytes = d * element size); must not overlap; 4-byte aligned (16-byte
 *               alignment and bx*row_bytes % 16 == 0 select 16-byte accesses).
 *   inverse     0: dst row p = src row n(p) (frame-major -> cube-major); 1: the reverse.
 * Returns SOL_ATTN_ERR_SHAPE for negative sizes, row_bytes not a positive multiple of 4,
 * a box that does not divide the grid (no partial boxes), inverse not 0/1, or B*H > 65535.
 */
sol_attn_status_t sol_attn_cube_permute(const void* src, void* dst, int B, int H, int T, int h, int w, int row_bytes, int bt,
                                        int by, int bx, int inverse, void* stream);

/*
 * Cube blocks read in place: sol_attn_pool with the blocks replaced by the bt x by x bx
 * boxes of the frame-major T x h x w latent grid (boxes numbered time, row, column as
 * for sol_attn_cube_permute; block c of the output is box c).  q, k stay frame-major
 * [B,H,T*h*w,d]; no reordered copy is made.  The pooled values equal those of
 * sol_attn_pool on the cube_permute'd tensors with block = bt*by*bx, bit for bit.
 *   q_pooled, k_pooled  float64 [B,H,n_boxes,d], n_boxes = (T/bt)*(h/by)*(w/bx).
 * Errors: as sol_attn_cube_permute for the grid and box (SOL_ATTN_ERR_SHAPE), then as
 * sol_attn_pool for dtype, d, B*H, NULL and alignment.
 */
sol_attn_status_t sol_attn_pool_cube(const void* q, const void* k, sol_attn_dtype_t dtype, int B, int H, int T, int h, int w, int d, int bt,
                                     int by, int bx, double* q_pooled, double* k_pooled, void* stream);

/*
 * Cube blocks read in place: the bf16 sol_attn_fwd (d = 128) with query and key block
 * c = box c of the frame-major latent grid, which must hold 128 tokens
 * (bt*by*bx == 128).  q, k, v, out [B,H,T*h*w,128] bf16 and lse [B,H,T*h*w] stay
 * frame-major; every output row is written (boxes tile the grid).  block_idx
 * [B,H,n_boxes,topk] indexes boxes, strictly ascending per row as for sol_attn_fwd;
 * qblock_order_or_null orders boxes.  The results equal those of sol_attn_fwd on the
 * cube_permute'd tensors, permuted back, bit for bit.
 * Errors: SOL_ATTN_ERR_SHAPE for the grid and box as sol_attn_cube_permute;
 * SOL_ATTN_ERR_UNSUPPORTED for a box of other than 128 tokens or a head of 2^31 bytes
 * or more; then as sol_attn_fwd.
 */
sol_attn_status_t sol_attn_fwd_cube(const void* q, const void* k, const void* v, int B, int H, int T, int h, int w, int bt, int by,
                                    int bx, int topk, const int32_t* block_idx, const int32_t* qblock_order_or_null,
                                    float softmax_scale, void* out, float* lse_or_null, void* stream);

/*
 * 8-bit exchange formats.  Between GPUs the Sol-H3 runtime sends Q, K and V as INT8 and
 * the attention output as FP8, shrinking the exchanged data ("Videomodel MiniMax-H3
 * rendert sneller dan afspelen", section "Waar de snelheidswinst vandaan komt": by
 * 51.6 percent).  Each token row of one head (d values) gets one float32 scale, so a
 * row costs d + 4 bytes instead of 2d (51.6 % of the bf16 bytes at d = 128).  With
 * amax = max |x| over the row:
 *   SOL_ATTN_INT8      scale = amax/127, code = round-half-even(x * (127/amax)), in [-127, 127]
 *   SOL_ATTN_FP8_E4M3  scale = amax/448, code = x * (448/amax) rounded to nearest-even OCP
 *                      E4M3 (bias 7, 3 mantissa bits, largest finite 448), saturated
 * A row of zeros has scale 0 and zero codes.  Every step is float32 with IEEE rounding,
 * so codes are reproducible bit for bit.  Decoding: code * scale, rounded to bf16.
 */
typedef enum { SOL_ATTN_INT8 = 0, SOL_ATTN_FP8_E4M3 = 1 } sol_attn_qformat_t;

/*
 * Quantise bf16 rows.
 *   x       [B,H,L,d] bf16 (rows of d values); 16-byte aligned.
 *   codes   [B,H,L,d] one byte per value (int8 or E4M3) output; 8-byte aligned.
 *   scales  [B,H,L] float32 output (one per row); 4-byte aligned.
 * Supported: d % 8 == 0, d <= 512.  Inputs must be finite.
 */
sol_attn_status_t sol_attn_quantize(const void* x, int B, int H, int L, int d, int format, void* codes, float* scales,
                                    void* stream);

/*
 * Decode rows written by sol_attn_quantize (same format) to bf16.
 *   codes [B,H,L,d] bytes (8-byte aligned), scales [B,H,L] float32 (4-byte aligned),
 *   out   [B,H,L,d] bf16 output (16-byte aligned).  Same support as sol_attn_quantize.
 */
sol_attn_status_t sol_attn_dequantize(const void* codes, const float* scales, int B, int H, int L, int d, int format, void* out,
                                      void* stream);

/*
 * Diagnostic (not part of the method): launches `workgroups` workgroups of 4 waves, each
 * wave running `iters` x 4 independent bf16 32x32x16 matrix-core products on register
 * operands (32768 flops each), no memory traffic.  Timing the launch gives the matrix
 * rate the chip sustains, a practical ceiling beside the nominal 2516.6 TFLOP/s.
 *   sink  device float[workgroups], written only in a case that does not occur (it keeps
 *         the products from being optimised away); 4-byte aligned.
 * Returns SOL_ATTN_ERR_SHAPE unless workgroups, iters >= 1; SOL_ATTN_ERR_NULL for a NULL sink.
 */
sol_attn_status_t sol_attn_probe_mfma(int workgroups, int iters, float* sink, void* stream);

/* Human-readable description of the last failure on the calling thread ("" if none). */
const char* sol_attn_last_error(void);

/* SOL_ATTN_VERSION of the built library. */
int sol_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SOL_ATTN_H_ */
