/*
 * nm.h -- C ABI of libnmsparse: N:M structured-sparse linear layers on AMD MI355X (gfx950).
 *
 * The library computes Y = S(X) . W^T where S keeps, in every group of m contiguous
 * values along the reduction dimension K, the n values of largest magnitude (ties to
 * the lower index), and the sparse operand is contracted in compressed form (values
 * plus index metadata).  Sources, by page title and section:
 *   [FLEX]   "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity
 *            via Benchmarking Lightweight Post-Training Sparsification Approaches",
 *            technical summary sections 1, 2.A (ACT: activation magnitude), 2.C (patterns).
 *   [SLIDE]  "SlideSparse: Fast and Flexible (2N-2):2N Structured Sparsity",
 *            technical summary sections 2.A (sliding windows), 2.B (activation lifting),
 *            2.C (packer, load-time compression, online kernel).
 *   [SPENSE] "SpenseGPT: Practical One-shot Pruning Enabling Sparse and Dense GEMMs for
 *            LLM Inference", technical summary sections 2.A (dense + 2:4 regions,
 *            input split with accumulation) and 2.B (dense indices permuted contiguous).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or keeps a pointer past the call.
 *  - bf16 tensors are 16-bit bf16 bit patterns; row-major with an explicit leading
 *    dimension in ELEMENTS (ld >= K).  Compressed arrays are dense row-major with no
 *    padding: values [rows][K*n/m] (bf16), U8 metadata [rows][K*n/m] (one byte per kept
 *    value = its in-group position 0..m-1, kept values in ascending position), 2-bit
 *    metadata [rows][ceil(K/8)] bytes (2:4 only; kept slot j of a row -> byte j/4,
 *    bits 2*(j%4)..2*(j%4)+1).  Bitmasks are uint32 words [rows][ceil(K/32)], bit k%32 of
 *    word k/32 set iff position k is kept.
 *  - Magnitude order is the order of the low 15 bits of the bf16 pattern: |x| order for
 *    every finite and infinite value, +0 ties -0, NaN ranks above infinity.  Pruned
 *    outputs are +0.0; kept values are copied bit for bit.
 *  - Every call validates its arguments on the host first and returns an nm_status.  On
 *    NM_OK the work has been ENQUEUED on `stream` (a hipStream_t passed as void*, NULL =
 *    the default stream); nothing is synchronised.  A device-side fault surfaces at the
 *    caller's next synchronisation.  No call throws; all are thread-safe and stateless.
 *  - Alignment: every device pointer must be 16-byte aligned and every bf16 leading
 *    dimension a multiple of 8 elements (nm_sparsify / nm_compress / nm_decompress with
 *    m = 4 accept a multiple of 4, with m in {6, 10, 12, 14} a multiple of 2,
 *    nm_slide_lift any); fp8 weights need a leading dimension that is a multiple of 16
 *    bytes (NM_EALIGN otherwise).  fp32 outputs take any leading dimension >= O.
 *  - Supported patterns: m in {4, 8, 16, 32}, 1 <= n <= m, K % m == 0.  nm_sparsify,
 *    nm_compress and nm_decompress also take m in {6, 10, 12, 14} (the group widths of
 *    the (2N-2):2N weight family, [SLIDE] 2.A) without a bitmask, since such groups
 *    straddle the 32-bit mask words (NM_EUNSUPPORTED with a mask).
 *  - Sizes are int64_t; rows, K, T, O >= 0 (zero-size calls return NM_OK and launch
 *    nothing, except that nm_spmm / nm_hybrid_gemm with K == 0 still write Y = 0 (or
 *    leave it unchanged when accumulating)).
 */
#ifndef NM_SPARSE_H
#define NM_SPARSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_EINVAL = 1,        /* null required pointer, bad enum value, n or m out of range  */
  NM_ESHAPE = 2,        /* inconsistent sizes: K % m, ld < K, negative or overflowing  */
  NM_EALIGN = 3,        /* pointer not 16-byte aligned or leading dimension % 8 != 0    */
  NM_EUNSUPPORTED = 4,  /* well-formed request outside what the kernels implement       */
  NM_EHIP = 5,          /* the HIP runtime reported an error when launching            */
  NM_ESCRATCH = 6       /* nm_spmm_noalloc: the call needs more scratch than it holds  */
} nm_status;

typedef enum { NM_META_U8 = 0, NM_META_2BIT = 1 } nm_meta;
typedef enum { NM_W_BF16 = 0, NM_W_FP8E4M3 = 1 } nm_wdtype;

/* Human-readable name of a status code (static storage). */
const char* nm_status_str(nm_status s);
/* Library version: major*10000 + minor*100 + patch. */
int nm_version(void);

/*
 * nm_sparsify -- S(X): per-group magnitude top-n along K.  [FLEX] 2.A (ACT score) and
 * 2.C (N:M patterns along the reduction dimension).
 *   x     bf16 [rows][ldx]                      input
 *   y     bf16 [rows][ldy] or NULL              S(X): kept values copied, pruned = +0.0
 *   mask  uint32 [rows][ceil(k/32)] or NULL     keep bitmask
 * At least one of y, mask must be non-NULL (NM_EINVAL).  y may alias x when ldy == ldx.
 */
nm_status nm_sparsify(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m,
                      void* y, int64_t ldy, uint32_t* mask, void* stream);

typedef enum {
  NM_SCORE_ACT_WEIGHTED = 0,   /* score = |x[k]| * col_score[k]  (activation weighted by    */
                               /*         the magnitude of the weights it multiplies)       */
  NM_SCORE_WEIGHT = 1          /* score = col_score[k]           (weight magnitude alone)   */
} nm_score;

/*
 * nm_sparsify_scored -- S(X) under an alternative selection score: per group of m along
 * K keep the n largest scores, ties to the lower index.  [FLEX] 2.A lists, besides ACT,
 * a weight-magnitude score (WT) and Amber-Pruner, which weights activation importance by
 * the magnitude of the corresponding weights; the pages give neither statistic, so the
 * per-column magnitude is the caller's (e.g. the L2 norm of each column of W, after any
 * outlier clipping).  The score is one fp32 multiply, rounded to nearest even with
 * subnormals kept: score = fp32(|x|) * col_score[k].
 *   x          bf16 [rows][ldx], finite
 *   col_score  fp32 [k], device, 16-byte aligned, every entry finite and >= 0
 *   mode       an nm_score value (NM_EINVAL otherwise)
 *   y, mask    as for nm_sparsify (at least one non-NULL)
 * m in {4, 8, 16, 32} (other widths: NM_EUNSUPPORTED).  Results are bit-exact.
 */
nm_status nm_sparsify_scored(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m,
                             const float* col_score, nm_score mode, void* y, int64_t ldy,
                             uint32_t* mask, void* stream);

/*
 * Error mitigation of activation sparsity.  [FLEX] 2.B names light-weight corrections that
 * need little or no calibration data: a per-token shift centring the activations before
 * pruning, dynamic (D-PTS) or static (S-PTS), and a per-token variance correction after it
 * (VAR); [FLEX] 4.C ranks them among the most effective.  The page gives no formulas; this
 * library's readings:
 *   NM_PTS_DYNAMIC  x~ = bf16(fp32(x - mu_t)), mu_t = the mean of token row t.  mu_t is
 *                   computed reproducibly: every value is rounded to a multiple of
 *                   q = 2^(E-162) (E = exponent field of the row's largest magnitude), the
 *                   integers are summed exactly and mu = fp32(fp64(sum * q) / k) -- the
 *                   row mean to within 2^-37 max|x|, the same bits in any summation order.
 *                   The product adds back mu_t * (W . 1)_o.
 *   NM_PTS_STATIC   x~ = bf16(fp32(x - c_k)) with the caller's per-channel shift c (a
 *                   scalar shift is c_k = s); the product adds back (W . c)_o.
 *   NM_PTS_VAR      alpha_t = sqrt(Var(x~_t) / Var(S(x~_t))) (population variances over the
 *                   k entries, pruned entries as zeros; 1 when the pruned row has no
 *                   variance); the product scales token t by alpha_t.
 * The selection is the ACT rule on x~ (bit-exact); with the mitigation the layer is
 *   Y[t][o] = alpha_t * sum_k S(x~)[t][k] W[o][k] + beta_t * v_o,
 * beta_t = mu_t (dynamic) or 1 (static), v = nm_weight_sums(W, shift) (W . 1 or W . c).
 */
enum { NM_PTS_DYNAMIC = 1, NM_PTS_STATIC = 2, NM_PTS_VAR = 4 };

/*
 * nm_sparsify_pts -- shift (pts & (NM_PTS_DYNAMIC | NM_PTS_STATIC), at most one), select
 * and, with NM_PTS_VAR, the variance correction factor.  [FLEX] 2.A, 2.B, 2.C.
 *   x          bf16 [rows][ldx], every value finite; k % 8 == 0, k <= 65536
 *   shift      fp32 [k] (NM_PTS_STATIC; NULL otherwise), finite
 *   y          bf16 [rows][ldy]: S(x~), required
 *   mask       uint32 [rows][ceil(k/32)] or NULL
 *   row_shift  fp32 [rows] or NULL: receives mu_t (NM_PTS_DYNAMIC)
 *   row_scale  fp32 [rows]: receives alpha_t (required with NM_PTS_VAR)
 * m in {4, 8, 16, 32}.  y, mask and row_shift are bit-exact; row_scale is the fp64 ratio
 * rounded to fp32 (summation order free, so equal to the definition within a few ulp).
 */
nm_status nm_sparsify_pts(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m, int pts,
                          const float* shift, void* y, int64_t ldy, uint32_t* mask, float* row_shift,
                          float* row_scale, void* stream);

/*
 * nm_weight_sums -- the per-output term that undoes a shift of the activations:
 *   out[o] = fp32( s_o * sum_k dec(W[o][k]) * c_k )
 * c = shift (fp32 [k], the static shift) or 1 when NULL (the dynamic shift's W . 1),
 * s = w_scale[o] for fp8 weights, 1 for bf16; summed in fp64.  w bf16 [o][ldw] or e4m3 codes
 * [o][ldw] bytes (w_dtype); out fp32 [o].  An offline step, once per weight (and shift).
 */
nm_status nm_weight_sums(const void* w, int64_t o, int64_t k, int64_t ldw, int w_dtype, const float* w_scale,
                         const float* shift, float* out, void* stream);

/*
 * nm_compress -- select and compact in one pass, straight from the dense input.
 * [FLEX] 1 (values plus index metadata), [SLIDE] 2.C (load-time compression).
 *   x       bf16 [rows][ldx]
 *   values  bf16 [rows][k*n/m]                    kept values, ascending position
 *   meta    U8: uint8 [rows][k*n/m]; 2BIT: uint8 [rows][ceil(k/8)] (needs n == 2, m == 4)
 *   mask    uint32 [rows][ceil(k/32)] or NULL     optional keep bitmask
 */
nm_status nm_compress(const void* x, int64_t rows, int64_t k, int64_t ldx, int n, int m,
                      void* values, void* meta, nm_meta fmt, uint32_t* mask, void* stream);

/*
 * nm_decompress -- inverse of nm_compress: scatter values to their positions, +0.0
 * elsewhere.  [SLIDE] 2.C: the packed form (values plus index metadata) is produced once
 * at load time and expanded again only where a dense operand is needed; [FLEX] 1 (values
 * plus index metadata).  y bf16 [rows][ldy].  Metadata entries must be valid positions
 * (< m, strictly ascending within a group); other metadata is a caller error with an
 * unspecified (but in-bounds) result.
 */
nm_status nm_decompress(const void* values, const void* meta, nm_meta fmt, int64_t rows,
                        int64_t k, int n, int m, void* y, int64_t ldy, void* stream);

/*
 * nm_lower_slide -- offline packer for (2N-2):2N weights.  [SLIDE] 2.A and 2.C.
 * Input: the compressed form (values bf16 [rows][k*(2N-2)/(2N)], idx uint8 same shape,
 * in-group positions 0..2N-1 ascending) of a matrix with exactly 2N-2 kept per group of
 * 2N.  Output: the equivalent 2:4 matrix over K' = k*(N-1)/N*2 = k*(2N-2)/N: each group
 * becomes N-1 overlapping windows of width 4 and stride 2 (window w covers positions
 * 2w..2w+3); kept positions are placed in ascending order, each in the lowest covering
 * window that holds fewer than two.  Window w of group g occupies lowered positions
 * g*4(N-1) + 4w + s.  values_out bf16 [rows][K'/2]; meta_out U8 [rows][K'/2] (in-window
 * slot 0..3) or 2BIT [rows][ceil(K'/8)].  Requires k % (2N) == 0 and 2 <= N <= 8.
 * Input that is not (2N-2):2N (a window overflow) is a caller error: the affected
 * group's output is unspecified but every access stays in bounds.
 */
nm_status nm_lower_slide(const void* values, const uint8_t* idx, int64_t rows, int64_t k,
                         int ns, void* values_out, void* meta_out, nm_meta fmt, void* stream);

/*
 * nm_quant_lift -- per-token fp8 quantization of the activations fused with the lift
 * ([SLIDE] 2.B; the page gives no quantization scheme).  Per row t:
 *   amax = max_k |x[t][k]|,  r = fp32(448 / amax),  xs[t] = fp32(amax / 448)  (1, 1 if amax = 0)
 *   q[k] = e4m3fn(clamp(fp32(x[t][k] * r), -448, 448)), round to nearest even (OCP E4M3FN)
 * written lifted: xq[t][g*4(N-1) + 4w + s] = q[g*2N + 2w + s] (N = ns; ns = 2: no lift),
 * uint8 codes [t][ldq] with ldq >= K' = k(2N-2)/N and ldq % 16 == 0 (codes past K' are
 * zero); xs fp32 [t].  x must be finite.  nm_spmm does this itself for fp8 weights in
 * the W_* modes; this call exists for inspection and tests.
 */
nm_status nm_quant_lift(const void* x, int64_t t, int64_t k, int64_t ldx, int ns, void* xq, int64_t ldq,
                        float* xs, void* stream);

/*
 * nm_slide_lift -- explicit activation lifting, X' [t][ldo] over K' = k*(2N-2)/N:
 * X'[t][g*4(N-1) + 4w + s] = X[t][g*2N + 2w + s].  [SLIDE] 2.B.  nm_spmm performs the
 * same lifting inside its operand loader; this call exists for inspection and tests.
 */
nm_status nm_slide_lift(const void* x, int64_t t, int64_t k, int64_t ldx, int ns,
                        void* x_out, int64_t ldo, void* stream);

/*
 * Route hints of nm_spmm (nm_spmm_args.route) and nm_hybrid_gemm (its `route` argument).
 * A hint chooses WHICH kernels compute a call, never WHAT is computed: every route gives
 * the same bitmask bit for bit and products within the same tolerance of the same
 * definition.  NM_ROUTE_AUTO (0) lets the library choose by shape; the other bits exist
 * so that every kernel can be tested and measured on any shape.  A hint that does not
 * apply to a call, or whose kernel does not take the shape, is ignored (the report below
 * says what ran).
 */
enum {
  NM_ROUTE_AUTO = 0,
  NM_ROUTE_ACT_FUSED = 1u << 0,     /* ACT_DYNAMIC above the few-token sizes: top-n selected
                                       inside the product's X-tile loader                   */
  NM_ROUTE_ACT_MASK = 1u << 1,      /* ... a select pass writes the bitmask to the
                                       workspace, the product applies it to X fragments     */
  NM_ROUTE_ACT_SX = 1u << 2,        /* ... a select pass writes S(X) to the workspace, the
                                       product streams it                                   */
  NM_ROUTE_NO_FEW = 1u << 3,        /* never the few-token (t <= 128) kernels, nor the split
                                       tile kernel above 128 tokens                         */
  NM_ROUTE_FEW_STREAM = 1u << 4,    /* few tokens: the weight-streaming kernels             */
  NM_ROUTE_FEW_TILE = 1u << 5,      /* few tokens: the split-K tile kernels where they apply*/
  NM_ROUTE_NO_META_BLOCK = 1u << 6, /* large-token 2:4 products read the row-major 2-bit
                                       positions (no K-blocked copy in the workspace)       */
  NM_ROUTE_FP8_WIDEN = 1u << 7,     /* large-token fp8 weights widened to bf16 in the
                                       workspace first                                      */
  NM_ROUTE_NO_XLDS = 1u << 8,       /* one token: X fragments in registers, not staged in LDS*/
  NM_ROUTE_NO_FEW_SELECT = 1u << 9, /* one token: a separate select pass rather than the
                                       selection inside the product's staged X row          */
  NM_ROUTE_TILE_LDS = 1u << 10,     /* tile products: the direct-to-LDS large-tile kernels
                                       at any size                                          */
  NM_ROUTE_TILE_REGS = 1u << 11,    /* tile products: the register-staged kernels           */
  NM_ROUTE_LIFT_COPY = 1u << 12,    /* W_SLIDE tile products: lift X into the workspace
                                       first (otherwise the tile loads build the lifted
                                       rows from the raw X)                                 */
  NM_ROUTE_ACT_SPARSE_X = 1u << 13, /* ACT_DYNAMIC 2:4 above the few-token sizes: compress
                                       X, then the sparse matrix instruction with X as the
                                       sparse operand (otherwise S(X) on dense tiles)       */
  NM_ROUTE_ROW_SX = 1u << 14        /* ACT_DYNAMIC, 2-32 tokens on the streaming kernel:
                                       S(X) staged row-major (otherwise in blocks of 16
                                       token rows, each 32-position piece contiguous)       */
};

/*
 * Report of the kernels a call enqueued (bits OR-ed into *route_taken when the caller
 * passes a host pointer; the call never clears it).
 */
enum {
  NM_TAKEN_SELECT = 1u << 0,        /* a separate select / compress pass                    */
  NM_TAKEN_FEW_STREAM = 1u << 1,    /* a few-token weight-streaming kernel                  */
  NM_TAKEN_FEW_XLDS = 1u << 2,      /* ... with the X row staged in LDS                     */
  NM_TAKEN_FEW_SELECT = 1u << 3,    /* ... selecting inside the staged X row                */
  NM_TAKEN_TILE_SPLIT = 1u << 4,    /* a split-K tile kernel (partial tiles in workspace)   */
  NM_TAKEN_REDUCE = 1u << 5,        /* a pass adding partial sums in a fixed order          */
  NM_TAKEN_TILE_LDS = 1u << 6,      /* a direct-to-LDS tile kernel                          */
  NM_TAKEN_TILE_REGS = 1u << 7,     /* a register-staged tile kernel                        */
  NM_TAKEN_FUSED_SELECT = 1u << 8,  /* selection inside a tile kernel's X loader            */
  NM_TAKEN_MASK = 1u << 9,          /* a product applying a bitmask to X                    */
  NM_TAKEN_GATHER1 = 1u << 10,      /* the single-token K-major gather                      */
  NM_TAKEN_LIFT = 1u << 11,         /* X lifted into the workspace                          */
  NM_TAKEN_META_BLOCK = 1u << 12,   /* 2-bit positions K-blocked into the workspace         */
  NM_TAKEN_PERMUTE = 1u << 13,      /* hybrid columns of X permuted into the workspace      */
  NM_TAKEN_QUANT = 1u << 14,        /* per-token fp8 quantization (and lift) pass           */
  NM_TAKEN_WIDEN = 1u << 15,        /* fp8 weights widened to bf16 in the workspace         */
  NM_TAKEN_DECOMPRESS = 1u << 16,   /* compressed X expanded into the workspace             */
  NM_TAKEN_SPARSE_MMA = 1u << 17    /* a product on the sparse matrix instructions          */
};

/* Operating modes of nm_spmm. */
typedef enum {
  NM_ACT_DYNAMIC = 0,    /* X dense; select n:m of X inside the call, then contract     */
  NM_ACT_COMPRESSED = 1, /* X given compressed (values + meta from nm_compress)          */
  NM_W_COMPRESSED = 2,   /* W given as 2:4 compressed (values + meta); X dense           */
  NM_W_SLIDE = 3,        /* W given lowered by nm_lower_slide (2:4 over K'); X lifted on
                            the fly inside the operand loader                            */
  NM_ACT_MASKED = 4      /* X dense plus its keep bitmask from nm_sparsify (x_meta =
                            uint32 [t][ceil(k/32)]), or X = S(X) already (x_meta NULL):
                            the two-pass forms of ACT_DYNAMIC                            */
} nm_spmm_mode;

/*
 * Arguments of nm_spmm.  Y[t][o] (fp32, row stride ldy) = sum_k A[t][k] * B[o][k] with
 *   ACT_DYNAMIC:    A = S_{n:m}(x),         B = w (bf16 [o][ldw] or fp8 [o][ldw] bytes)
 *   ACT_COMPRESSED: A = decompress(x, x_meta) (x = values [t][k*n/m]), B = w as above
 *   ACT_MASKED:     A = x with the positions whose bit in x_meta is clear zeroed; the
 *                   mask must come from nm_sparsify with the same n, m (then A = S(x)).
 *                   x_meta may be NULL when x already holds S(x) (nm_sparsify's y).
 *   W_COMPRESSED:   A = x (bf16 [t][ldx]),  B = decompress(w, w_meta), 2:4 over k
 *   W_SLIDE:        A = lift_ns(x),          B = decompress(w, w_meta), 2:4 over
 *                   K' = k*(2ns-2)/ns  (equals x . Wpruned^T)
 *   W_* with w_dtype NM_W_FP8E4M3 (w: e4m3 codes [o][K'/2], w_scale required): x is
 *                   quantized per token to e4m3 and lifted first (nm_quant_lift), and
 *                   Y = xs[t] * (sum_k' dec(xq[t][k']) * dec(W'[o][k'])) * w_scale[o], on the
 *                   fp8 sparse matrix instruction ([SLIDE]: FP8 serving).  Requires
 *                   K' % 128 == 0 (NM_EUNSUPPORTED otherwise) and a workspace of
 *                   nm_spmm_workspace_size bytes (NM_EINVAL otherwise).
 * then, when w_scale != NULL (fp8 weights), Y[t][o] *= w_scale[o]; finally Y = result
 * (accumulate == 0) or Y += result (accumulate == 1).
 * Optional fields (may be NULL / 0):
 *   x_mask_out  ACT_DYNAMIC only: receives the selection bitmask of x [t][ceil(k/32)]
 *   w_kmajor    ACT_DYNAMIC, bf16 W only: the same weights stored K-major [k][o]
 *               (row stride o, 16-byte aligned).  Single-token calls (t == 1) with
 *               o % 8 == 0, no w_scale and a workspace of nm_spmm_workspace_size bytes
 *               then read only the selected K-rows of W (n/m of its bytes).
 *   workspace   device scratch (16-byte aligned).  With workspace_bytes >=
 *               nm_spmm_workspace_size(args): ACT_DYNAMIC may run select and product as
 *               two passes (S(x) staged in the workspace), ACT_COMPRESSED stages the
 *               decompressed x there (required unless n:m = 2:4 with 2BIT metadata),
 *               W_SLIDE calls that run the register-staged tile kernel (or carry the
 *               NM_ROUTE_LIFT_COPY hint) stage the lifted x there (the direct-to-LDS tile
 *               kernels build the lifted rows from x in their own loads), W_* calls
 *               above 128 tokens also place a K-blocked copy of the 2-bit positions
 *               there (o * kc / 8 bytes: fewer, larger loads per tile), and few-token
 *               calls (t <= 128), and larger calls whose 256 x 256 output tiles number
 *               under 128, may split the reduction across workgroups, writing fp32
 *               partial sums there that a second kernel adds in a fixed order (at most
 *               256 partial tiles of 128 x 128; the split-K tile route needs this).  With
 *               less, the call takes a route that needs none (slower).  Contents after the call are
 *               unspecified.  Calls sharing a workspace must be ordered (same stream).
 *   pts, pts_shift, col_shift, row_scale, row_shift   the activation-sparsity
 *               mitigations ([FLEX] 2.B): ACT_DYNAMIC with pts != 0 shifts, selects and
 *               (NM_PTS_VAR) computes alpha inside the call (x finite, k % 8 == 0,
 *               k <= 65536, m in {4, 8, 16, 32}, a workspace of nm_spmm_workspace_size
 *               bytes required), then Y = alpha_t * (S(x~) W^T) + beta_t * col_shift[o].
 *               In ACT_MASKED / ACT_COMPRESSED the terms come from the caller (the two-pass
 *               form with nm_sparsify_pts): Y = row_scale[t] * (...) + beta_t * col_shift[o],
 *               beta_t = row_shift[t] (1 when row_shift is NULL); NULL drops a factor or
 *               term.  row_shift needs col_shift; all need 16-byte alignment.  W_* modes
 *               take none of them (NM_EUNSUPPORTED).
 *   route       NM_ROUTE_* hint bits (0: the library chooses by shape)
 *   few_wpb     few-token streaming kernels: waves per workgroup (4, 8 or 16; 0 = chosen)
 *   few_splits  few-token streaming kernels: reduction splits across workgroups (0 = chosen)
 *   tile_wg     split-K tile kernels: target workgroup count (0 = one per CU)
 *   route_taken host pointer or NULL: receives NM_TAKEN_* bits (OR-ed in) of the kernels
 *               the call enqueued
 *   The route fields change which kernels run and the workspace the size query asks for,
 *   never the result beyond the stated tolerance.
 * Results are deterministic: the same call on the same inputs gives the same bits.
 */
typedef struct {
  int mode;               /* nm_spmm_mode                                          */
  int n, m;               /* activation pattern (ACT_*); ignored for W_* modes     */
  int ns;                 /* N of the (2N-2):2N family (W_SLIDE only)              */
  int64_t t, o, k;        /* tokens, output features, ORIGINAL reduction length    */
  const void* x;          /* see mode                                              */
  int64_t ldx;            /* elements; ignored for ACT_COMPRESSED                  */
  const void* x_meta;     /* ACT_COMPRESSED metadata                               */
  int x_meta_fmt;         /* nm_meta                                               */
  const void* w;          /* see mode                                              */
  int64_t ldw;            /* elements (bf16) or bytes (fp8); ignored for W_* modes */
  int w_dtype;            /* nm_wdtype (fp8 in W_* modes: fp8 x fp8, see above)     */
  const void* w_meta;     /* W_* metadata                                          */
  int w_meta_fmt;         /* nm_meta                                               */
  const float* w_scale;   /* fp32 [o] per-row scale (required for fp8, else NULL)  */
  const void* w_kmajor;   /* optional, see above                                   */
  float* y;               /* fp32 [t][ldy]                                         */
  int64_t ldy;
  int accumulate;         /* 0: Y = result, 1: Y += result                         */
  uint32_t* x_mask_out;   /* optional                                              */
  void* workspace;        /* optional                                              */
  int64_t workspace_bytes;
  uint32_t route;         /* NM_ROUTE_* hints (0 = the library's choice)           */
  int32_t few_wpb;        /* tuning of the chosen kernels (0 = the library's)      */
  int32_t few_splits;
  int32_t tile_wg;
  uint32_t* route_taken;  /* optional host pointer: NM_TAKEN_* bits of what ran    */
  /* error mitigation and output terms (ACT_* modes), see NM_PTS_*:                */
  int pts;                /* ACT_DYNAMIC: NM_PTS_* applied inside the call          */
  const float* pts_shift; /* NM_PTS_STATIC: fp32 [k]                                */
  const float* col_shift; /* fp32 [o]: v (nm_weight_sums); required with a shift    */
  const float* row_scale; /* ACT_MASKED / ACT_COMPRESSED: fp32 [t] alpha_t, or NULL */
  const float* row_shift; /* ACT_MASKED / ACT_COMPRESSED: fp32 [t] beta_t, or NULL  */
} nm_spmm_args;

/*
 * nm_spmm -- the structured-sparse linear layer.  [FLEX] 2.A/2.C (activation N:M),
 * [SLIDE] 2.A-2.C (lowered (2N-2):2N weights with lifted activations), 2:4 weights as
 * the special case N = 2.  W_COMPRESSED and W_SLIDE run on the gfx950 sparse matrix
 * instructions (2:4 along K); activation patterns other than 2:4 run on dense matrix
 * instructions over the selected (zero-filled) operand.
 */
nm_status nm_spmm(const nm_spmm_args* args, void* stream);

/*
 * nm_spmm_noalloc -- nm_spmm for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  It computes
 * what nm_spmm computes (the same kernels and routes, bit-identical results, except as
 * below) but takes its scratch from a buffer inside the library instead of
 * args->workspace, which must be NULL with workspace_bytes 0 (NM_EINVAL otherwise):
 *   - the buffer is NM_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory per GPU, part of the
 *     library's code object, held until the process ends;
 *   - when nm_spmm_workspace_size exceeds it because the preferred route splits the
 *     reduction of its 256 x 256 tiles, the call runs those tiles unsplit (another
 *     summation order, the same tolerance); a call that still needs more returns
 *     NM_ESCRATCH and enqueues nothing;
 *   - the first call on a GPU looks up that GPU's copy of the buffer (no allocation);
 *   - every call on a GPU shares that GPU's buffer: calls that may overlap in time on one
 *     GPU (different streams, or different threads without ordering) race on it and must
 *     be serialised by the caller; calls on one stream are ordered and safe;
 *   - no route needs the buffer zeroed; it keeps whatever the last call left in it.
 * Allocates nothing: no hipMalloc, hipFree or allocating library routine.
 */
#define NM_NOALLOC_SCRATCH_BYTES (64ll << 20)
nm_status nm_spmm_noalloc(const nm_spmm_args* args, void* stream);

/* Bytes of workspace for nm_spmm's preferred route with these arguments (0 if it uses
 * none).  Depends on mode, n, m, ns, t, o, k, w_dtype, w_scale, ldx, x_meta and the route
 * fields only. */
int64_t nm_spmm_workspace_size(const nm_spmm_args* args);

/*
 * nm_hybrid_pack -- offline packing of the hybrid dense + 2:4 format.  [SPENSE] 2.A
 * (a dense region and a 2:4 region) and 2.B (chosen dense indices permuted into one
 * contiguous block).  Dense columns = the k_dense columns of W with the largest L2 norm
 * over the output dimension (sum of squares in fp64, accumulated in ascending o; ties to
 * the lower column).  Outputs:
 *   sparse_cols int32 [k - k_dense] ascending; dense_cols int32 [k_dense] ascending
 *   ws_values bf16 [o][(k-k_dense)/2], ws_meta (U8 [o][(k-k_dense)/2] or 2BIT
 *   [o][ceil((k-k_dense)/8)]): W restricted to sparse_cols, pruned 2:4 by magnitude
 *   wd bf16 [o][ldwd]: W restricted to dense_cols
 *   workspace: device scratch of at least nm_hybrid_pack_workspace_size(k) bytes
 *   (column norms and flags; its contents after the call are unspecified).
 * Requires (k - k_dense) % 4 == 0, 0 <= k_dense <= k, k <= 65536.
 */
nm_status nm_hybrid_pack(const void* w, int64_t o, int64_t k, int64_t ldw, int64_t k_dense,
                         int32_t* sparse_cols, int32_t* dense_cols, void* ws_values,
                         void* ws_meta, nm_meta fmt, void* wd, int64_t ldwd, void* workspace,
                         int64_t workspace_bytes, void* stream);

/* Workspace bytes nm_hybrid_pack needs for a reduction length k. */
int64_t nm_hybrid_pack_workspace_size(int64_t k);

/*
 * nm_hybrid_gemm -- input-split product of the hybrid format, one accumulator:
 *   Y[t][o] (=|+=) sum_{j<K_s} x[t][sparse_cols[j]] * Ws[o][j]
 *                + sum_{j<K_d} x[t][dense_cols[j]]  * Wd[o][j]
 * with Ws the 2:4 compressed sparse region (sparse matrix instructions) and Wd the dense
 * region (dense matrix instructions).  [SPENSE] 2.A (input split with accumulation).
 * x is bf16 [t][ldx] with ldx >= K_s + K_d.  sparse_cols / dense_cols (as written by
 * nm_hybrid_pack: a partition of [0, K_s + K_d)) may both be NULL, in which case x is
 * taken as already permuted: columns [0, K_s) are the sparse region and [K_s, K_s+K_d)
 * the dense one (then K_s % 8 == 0 when K_d > 0).  Column indices outside
 * [0, K_s + K_d) are clamped into it.  ws_meta must be 2BIT.  Requires K_s % 4 == 0.
 * workspace: device scratch (16-byte aligned) of workspace_bytes bytes.  The gathered
 * form (column lists given) stages the column-permuted x there and requires at least
 * t * (ceil8(K_s) + ceil8(K_d)) * 2 bytes (NM_EINVAL otherwise); above 128 tokens the
 * preferred route also places a K-blocked copy of ws_meta after it (o * K_s / 8 bytes).
 * nm_hybrid_gemm_workspace_size gives the amount for the preferred route.  Contents
 * after the call are unspecified; calls sharing it must be ordered.
 * route: NM_ROUTE_* hints (0 = the library's choice; the ACT_* and fp8 bits do not apply);
 * route_taken: host pointer or NULL, receives NM_TAKEN_* bits as for nm_spmm.
 */
nm_status nm_hybrid_gemm(const void* x, int64_t t, int64_t ldx, const int32_t* sparse_cols,
                         int64_t k_s, const int32_t* dense_cols, int64_t k_d,
                         const void* ws_values, const void* ws_meta, nm_meta fmt,
                         const void* wd, int64_t ldwd, int64_t o, float* y, int64_t ldy,
                         int accumulate, void* workspace, int64_t workspace_bytes,
                         uint32_t route, uint32_t* route_taken, void* stream);

/* Workspace bytes of nm_hybrid_gemm's preferred route (gathered: column lists given) under
 * the route hints `route`. */
int64_t nm_hybrid_gemm_workspace_size(int64_t t, int64_t k_s, int64_t k_d, int64_t o,
                                      int gathered, uint32_t route);

/*
 * Spense layout of a GLU MLP ([SPENSE] 2.A, 2.B).  The intermediate indices of
 * down(act(gate x) * up x) can be permuted without changing the result, so the indices
 * kept dense are moved into one block at the end: gate and up are split by output rows
 * (output-split: a 2:4 product and a dense product write disjoint column ranges of y),
 * down by input columns (input-split: nm_hybrid_gemm with the column lists NULL, since
 * the GLU output already comes in the permuted order).
 */
typedef enum {
  NM_SPENSE_LOSS = 0,   /* dense = the n_dense indices of largest loss-aware score      */
  NM_SPENSE_TAIL = 1    /* dense = the last n_dense indices (identity permutation)      */
} nm_spense_strategy;

/*
 * nm_spense_glu_order -- which intermediate indices stay dense, and the permutation.
 * [SPENSE] 2.B: the loss-aware score of index i sums the per-weight score
 * |W_ij| * sqrt(H_jj) over the three projections:
 *   S_i = (sum_j |Wg[i][j]| hs_in[j] + sum_j |Wu[i][j]| hs_in[j]) + hs_mid[i] * sum_o |Wd[o][i]|
 * in fp64, each sum in ascending index order, every product and sum rounded once.
 *   w_gate, w_up  bf16 [inter][ld_gu] (row i = intermediate index i), w_down bf16 [hidden][ld_d]
 *   hs_in         fp64 [hidden]: square roots of the MLP input's Hessian diagonal (X^T X)
 *   hs_mid        fp64 [inter]:  the same for the down projection's input
 *                 (weights and hs_* are not read for NM_SPENSE_TAIL and may be NULL)
 *   perm          int32 [inter] out: sparse indices ascending, then the n_dense dense ones
 *                 ascending (ties in the score go to the lower index)
 *   scores        fp64 [inter] out, or NULL (then the scores live in the workspace)
 *   workspace     >= nm_spense_glu_order_workspace_size(inter) bytes
 * Offline step (once per weight set).  Deterministic.
 */
nm_status nm_spense_glu_order(const void* w_gate, const void* w_up, int64_t ld_gu, const void* w_down,
                              int64_t ld_d, int64_t hidden, int64_t inter, const double* hs_in,
                              const double* hs_mid, int64_t n_dense, nm_spense_strategy strategy,
                              int32_t* perm, double* scores, void* workspace, int64_t workspace_bytes,
                              void* stream);
int64_t nm_spense_glu_order_workspace_size(int64_t inter);

/*
 * nm_spense_pack -- split W [o][k] by a permutation into a 2:4 region and a dense region.
 * [SPENSE] 2.A.
 *   axis 0 (output-split, gate / up): rows perm[0:n_sparse] are pruned 2:4 along k and
 *          compressed (values [n_sparse][k/2], meta); rows perm[n_sparse:o] go to
 *          wd [o - n_sparse][ldwd] (ldwd >= k).  k % 4 == 0.
 *   axis 1 (input-split, down): columns perm[0:n_sparse] are pruned 2:4 in that order
 *          (values [o][n_sparse/2], meta); columns perm[n_sparse:k] go to wd [o][ldwd]
 *          (ldwd >= k - n_sparse).  n_sparse % 4 == 0.
 * Meta is U8 or 2BIT as in nm_compress.  perm entries outside the axis are clamped into
 * it.  The workspace takes nm_spense_pack_workspace_size(o, k, axis, n_sparse) bytes
 * (axis 0: a gathered copy of the sparse rows).  Offline step.
 */
nm_status nm_spense_pack(const void* w, int64_t o, int64_t k, int64_t ldw, int axis, const int32_t* perm,
                         int64_t n_sparse, void* ws_values, void* ws_meta, nm_meta fmt, void* wd,
                         int64_t ldwd, void* workspace, int64_t workspace_bytes, void* stream);
int64_t nm_spense_pack_workspace_size(int64_t o, int64_t k, int axis, int64_t n_sparse);

/*
 * nm_spense_outsplit_gemm -- output-split product ([SPENSE] 2.A):
 *   y[:, 0:o_s]        (=|+=) x . W_s^T   (W_s: 2:4 rows as packed by nm_spense_pack axis 0,
 *                                          2BIT meta)
 *   y[:, o_s:o_s+o_d]  (=|+=) x . W_d^T   (dense rows wd [o_d][ldwd])
 * x bf16 [t][ldx]; k % 4 == 0; ldy >= o_s + o_d; o_s % 4 == 0 when both parts are
 * present (the dense part starts at y + o_s).  The two parts run as the corresponding
 * nm_spmm calls (W_COMPRESSED and the plain product), in order on `stream`, sharing the
 * workspace: nm_spense_outsplit_workspace_size(t, k, o_s, o_d) bytes for the preferred
 * routes.
 */
nm_status nm_spense_outsplit_gemm(const void* x, int64_t t, int64_t k, int64_t ldx, const void* ws_values,
                                  const void* ws_meta, int64_t o_s, const void* wd, int64_t ldwd, int64_t o_d,
                                  float* y, int64_t ldy, int accumulate, void* workspace,
                                  int64_t workspace_bytes, void* stream);
int64_t nm_spense_outsplit_workspace_size(int64_t t, int64_t k, int64_t o_s, int64_t o_d);

#ifdef __cplusplus
}
#endif

#endif /* NM_SPARSE_H */
