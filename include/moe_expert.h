/*
 * moe_expert.h -- C ABI of the MI355X (gfx950) MoE expert-mapping, dispatch
 * and combine library (libmoe_expert.so).
 *
 * One device's share of a Mixture-of-Experts layer's token dispatch and
 * combine, as described by the Ascend CANN operator pages
 * "aclnnMoeUpdateExpert", "aclnnMoeDistributeDispatchV2" and
 * "aclnnMoeDistributeCombineAddRmsNorm".  The three calls run in that fixed
 * order for a layer (update-expert page, calling-sequence constraint).
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     allocates, frees, synchronises and retains nothing; each call only
 *     validates its scalar arguments on the host and enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the legacy default stream).  Calls are
 *     asynchronous, safe to capture in a HIP graph, reentrant across streams
 *     and deterministic (bitwise-repeatable), as the pages require
 *     (确定性计算 / "deterministic computation" notes).
 *   - All arrays are dense row-major.  bf16 data is IEEE bfloat16 bit
 *     patterns; fp8 data is OCP FP8 E4M3 bytes; int8 is two's complement.
 *   - Row pointers (x, expand_x, expert_out, shared_x, residual_x, y, x_out,
 *     gamma) must be 16-byte aligned.
 *   - Host-checkable errors return a non-zero moe_status BEFORE anything is
 *     enqueued (the role of the pages' first-phase parameter check).
 *     Data-dependent errors that cannot be seen without reading device
 *     memory set bits in the optional device word *dev_err (atomic OR,
 *     sticky until the caller clears it); the offending entry is then
 *     treated as pruned.  MOE_ELAUNCH reports a HIP launch failure.
 *
 * Shape limits (combine page 约束说明 item 4; update-expert page shape
 * restrictions): 0 < Bs <= 512, 0 < K <= 16, 1024 <= H <= 8192, at most
 * 1024 expert instances in total.  This library also requires H % 32 == 0
 * (whole 16-byte row chunks and whole 32-element mxfp8 blocks).
 */
#ifndef MOE_EXPERT_H
#define MOE_EXPERT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,   /* a scalar out of range, a NULL required pointer, misalignment */
    MOE_ENOTSUP = 2,  /* a valid option this library does not implement */
    MOE_ELAUNCH = 3   /* the HIP runtime rejected a kernel launch */
} moe_status;

/* Dispatch quantisation modes (dispatch page 计算公式 cases 1-5). */
typedef enum {
    MOE_Q_NONE = 0,        /* expand_x rows are bit copies of x (bf16)                  */
    MOE_Q_STATIC = 1,      /* static int8: code = sat(round_half_even(x * scales))     */
    MOE_Q_INT8_TOKEN = 2,  /* per-token dynamic int8                                    */
    MOE_Q_INT8_TILE = 3,   /* per-tile dynamic int8 ("pertile" / "pergroup")            */
    MOE_Q_MXFP8 = 4,       /* mxfp8: E4M3 codes, one E8M0 exponent per 32 elements      */
    MOE_Q_MXFP8_GM = 5,    /* the same codes, exponents group-major (moe_expert_gemm's
                              order): a layout of case 5, not another format           */
    MOE_Q_STATIC_E4M3 = 6  /* static, the second output type (read as E4M3; one
                              coefficient only): code = E4M3(x * scale)               */
} moe_quant;

/* Shape of the dispatch's scales input (dispatch page 计算公式: xFp32 =
 * CastToFp32(X) * scales in cases 2-4; quantMode constraints for the shapes).
 * A device pointer carries no shape, so the caller names it. */
typedef enum {
    MOE_SCALES_NONE = 0,   /* no scales input (scales pointer NULL)                     */
    MOE_SCALES_ONE = 1,    /* f32 [1]: one coefficient (static mode only)                */
    MOE_SCALES_ROW = 2,    /* f32 [H]: one row shared by all experts (static mode only)  */
    MOE_SCALES_EXPERT = 3  /* f32 [E, H]: one row per instance, picked by the instance a
                              copy is sent to; every copy is then quantised on its own */
} moe_scales_kind;

/* Weight of the shared-expert output in the combine (combine page 计算公式). */
typedef enum {
    MOE_SHARED_PAGE = 0,   /* sum over the token's dispatched k of expertScales[i,k]     */
    MOE_SHARED_ADD = 1     /* 1                                                         */
} moe_shared_mode;

/* dev_err bits */
#define MOE_ERR_ID 1        /* an active expert / instance id outside its range          */
#define MOE_ERR_TABLE 2     /* mapping-table replica count not in [1, F-1], or an
                               instance id in the table outside [0, n_instances)         */
#define MOE_ERR_MASK1D 4    /* a 1-D token mask that is not all-true-then-all-false      */
#define MOE_ERR_ROW 8       /* combine: an assist_dst entry >= Bs*K                      */
#define MOE_ERR_OFFSETS 16  /* expert GEMM: offsets not non-decreasing within [0, rows]   */

/*
 * moe_update_expert -- load balancing and expert pruning
 * ("aclnnMoeUpdateExpert": map each token's top-K logical expert ids to
 * deployed instances; prune entries by a threshold broadcast over the batch).
 *
 * For entry f = i*K + k with logical id e = expert_ids[f]:
 *   n                = table[e*F + 0]                (replica count, 1 <= n <= F-1)
 *   balanced_ids[f]  = table[e*F + 1 + (i mod n)]    (global instance id,
 *                                                     rank * local_experts + slot)
 *   balanced_mask[f] = token_mask[i] (1 if token_mask is NULL)
 *                      AND NOT (expert_scales[f] < prune_thr[k])
 *                      (the threshold test is skipped if either pointer is NULL;
 *                       a NaN score is kept)
 * An entry whose lookup fails gets id -1 and mask 0, and raises MOE_ERR_ID /
 * MOE_ERR_TABLE only if it would otherwise have been kept.  A token_mask that
 * is not all-true-then-all-false (dispatch page: {true,false,true} is
 * illegal) raises MOE_ERR_MASK1D and is still applied as given.
 *
 *   expert_ids    int32 [Bs, K]            logical ids in [0, n_logical)
 *   expert_scales f32   [Bs, K] or NULL     routing scores
 *   table         int32 [n_logical, F]      col 0 = replica count, cols 1.. = instance ids
 *   prune_thr     f32   [K] or NULL         threshold for column k
 *   token_mask    u8    [Bs] or NULL        1 = token takes part
 *   balanced_ids  int32 [Bs, K]   (out)
 *   balanced_mask u8    [Bs, K]   (out)     1 = dispatch, 0 = pruned
 *   dev_err       int32 [1] or NULL
 * Limits: 0 < Bs <= 512, 0 < K <= 16, K <= n_logical <= 1024,
 *         2 <= F <= n_logical + 1, 0 < n_instances <= 1024.
 */
int moe_update_expert(const int32_t *expert_ids, const float *expert_scales,
                      const int32_t *table, const float *prune_thr, const uint8_t *token_mask,
                      int Bs, int K, int n_logical, int F, int n_instances,
                      int32_t *balanced_ids, uint8_t *balanced_mask, int32_t *dev_err,
                      void *stream);

/*
 * moe_dispatch -- quantise tokens and scatter them expert-major
 * ("aclnnMoeDistributeDispatchV2" 计算公式: expandX = AllToAllV(quantOut);
 * here the single device's share: the rows this device would send, laid out
 * [rank][local expert][token] as the all-to-all delivers them).
 *
 * E = n_ranks * local_experts instances; N = Bs*K entries f = i*K + k.
 * Entry f is active if active_mask is NULL or active_mask[f] != 0, and
 * token_mask is NULL or token_mask[i] != 0, and its id is in [0, E) (else
 * MOE_ERR_ID and it is dropped).  The two masks are the 2-D (Bs, K) and 1-D
 * (Bs,) forms of the page's active mask (参数说明 of the dispatch page); a
 * 1-D mask must be all true, then all false: otherwise MOE_ERR_MASK1D is set
 * and the mask is applied as given.
 *   expert_counts[e]  = number of active entries with id e
 *   expert_offsets    = exclusive prefix sum of counts; offsets[E] = rows written
 *   assist_dst[f]     = row of entry f: offsets[id] + number of active g < f
 *                       with the same id (stable, ascending f); -1 if inactive
 *   expand_src[r]     = entry placed in row r; -1 for r >= offsets[E]
 *   expand_x[r]       = token i = f / K sent to instance e = id of f, coded
 *                       from v = x[i] (no scales) or v = x[i] * s (one fp32
 *                       multiply per element; s by quant_scales_kind):
 *     MOE_Q_NONE       bf16 [N, H] bit copy of x[i]
 *     MOE_Q_STATIC     int8 [N, H]: code = clamp(round_half_even(v), -128, 127),
 *                      NaN -> 0; no expand_scales (may be NULL)
 *     MOE_Q_STATIC_E4M3  E4M3 [N, H]: code = E4M3(v) rounded to nearest even and
 *                      saturated at +-448, a NaN v (NaN in x, or +-inf times a zero
 *                      coefficient) -> 0x7F; no expand_scales (may be NULL).  The
 *                      page's second static output type, whose name the extracted
 *                      text lost, read as the E4M3 of case 5; the quantMode
 *                      constraints give that type the one-coefficient shape only
 *     MOE_Q_INT8_TOKEN int8 [N, H]: m = max|v|, d = 127/m (fp32, IEEE),
 *                      code = clamp(round_half_even(x*d), -127, 127);
 *                      expand_scales f32 [N] = 1/d  (m == 0: codes 0, scale 0)
 *     MOE_Q_INT8_TILE  the same per tile of `tile` elements along H (the last
 *                      tile may be partial); expand_scales f32 [N, ceil(H/tile)];
 *                      tile must be a power of two in [16, 1024]
 *     MOE_Q_MXFP8      E4M3 [N, H]: per block of 32, se = floor(log2 max|x|) - 8
 *                      clamped to [-127, 127] (-127 for an all-zero block),
 *                      code = E4M3(x / 2^se) rounded to nearest even and
 *                      saturated at +-448; expand_scales u8 [N, H/32] = se + 127
 *                      (E8M0 code of the dequantisation multiplier 2^se)
 *     MOE_Q_MXFP8_GM   the codes and exponents of MOE_Q_MXFP8, the exponents
 *                      stored group-major: expand_scales u8 [ceil(H/512), N, 16],
 *                      exponent b of row r at [b/16][r][b%16] (the pad bytes of a
 *                      last, partial group are not written), so that the expert
 *                      GEMM copies one group of 64 rows' exponents as 1 KB
 * Infinities and NaNs in x (the page defines no rule): every maximum skips
 * NaN; an infinite maximum gives se = 127, or d = 127/inf = 0 with scale +inf
 * (every int8 code 0); E4M3 codes NaN as 0x7F with its sign and +-inf as
 * +-448; int8 codes NaN as 0; the static cast takes +-inf to 127 / -128.
 * Rows at or past offsets[E] of expand_x / expand_scales are not written.
 *
 *   x              bf16 [Bs, H]
 *   expert_ids     int32 [Bs, K]     instance ids (e.g. balanced_ids)
 *   active_mask    u8 [Bs, K] or NULL (e.g. balanced_mask)
 *   token_mask     u8 [Bs] or NULL
 *   quant_scales   f32, shape by quant_scales_kind (16-byte aligned for ROW and
 *                  EXPERT), or NULL with MOE_SCALES_NONE.  MOE_Q_STATIC takes
 *                  ONE, ROW or EXPERT; MOE_Q_STATIC_E4M3 takes ONE;
 *                  MOE_Q_INT8_TOKEN / _TILE take NONE or EXPERT; MOE_Q_NONE and
 *                  the mxfp8 modes take NONE (else MOE_EINVAL).
 *   expand_x       [N, H] elements of the mode's type (out)
 *   expand_scales  see above; NULL for MOE_Q_NONE and the static modes (out)
 *   expert_counts  int32 [E]  (out)      expert_offsets int32 [E+1] (out)
 *   expand_src     int32 [N]  (out)      assist_dst     int32 [N]   (out)
 *   dev_err        int32 [1] or NULL
 * Limits: 0 < Bs <= 512, 0 < K <= 16, K <= E <= 1024, H in [1024, 8192] with
 *         H % 32 == 0, n_ranks >= 1, local_experts >= 1.
 */
int moe_dispatch(const void *x, const int32_t *expert_ids, const uint8_t *active_mask,
                 const uint8_t *token_mask, int Bs, int H, int K, int n_ranks,
                 int local_experts, int quant_mode,
                 int tile, const float *quant_scales, int quant_scales_kind, void *expand_x,
                 void *expand_scales, int32_t *expert_counts, int32_t *expert_offsets,
                 int32_t *expand_src, int32_t *assist_dst, int32_t *dev_err, void *stream);

/*
 * moe_update_dispatch -- moe_update_expert followed by moe_dispatch in one
 * launch (the pages' fixed calling sequence UpdateExpert -> DispatchV2).
 *
 * Same results as
 *   moe_update_expert(expert_ids, expert_scales, table, prune_thr, token_mask,
 *                     Bs, K, n_logical, F, n_ranks * local_experts, ids', mask', ...)
 *   moe_dispatch(x, ids', mask', Bs, H, K, n_ranks, local_experts, quant_mode, tile, ...)
 * with the intermediate ids' / mask' written to balanced_ids / balanced_mask
 * when those are non-NULL, and dev_err collecting the bits of both calls.
 * Every dispatch block maps the entries it counts through an LDS copy of the
 * table, which saves the second launch but repeats the mapping in each of the
 * Bs + 1 blocks: measured on MI355X it pays off up to about Bs*K = 4096
 * entries (Bs=512, K=8: 10.2 us against 3.3 + 9.0 us for the two calls) and
 * not at Bs*K = 8192 with pruning (Bs=512, K=16: 17.0 us against 3.5 + 10.9).
 * So above 4096 entries, when balanced_ids and balanced_mask are given (the
 * mask 4-byte aligned), the call enqueues the two launches itself; with either
 * of them NULL it stays one launch at any size.
 *
 *   expert_ids    int32 [Bs, K]  logical ids (16-byte aligned)
 *   expert_scales f32   [Bs, K] or NULL (16-byte aligned when prune_thr is given)
 *   table, prune_thr, token_mask, n_logical, F: as moe_update_expert
 *   balanced_ids  int32 [Bs, K] or NULL (out); balanced_mask u8 [Bs, K] or NULL (out)
 *   the rest: as moe_dispatch.
 * Limits: those of both calls, and n_logical * F <= 8192 (the table a block
 * stages in LDS); a larger table returns MOE_ENOTSUP (make the two calls).
 */
int moe_update_dispatch(const void *x, const int32_t *expert_ids, const float *expert_scales,
                        const int32_t *table, const float *prune_thr, const uint8_t *token_mask,
                        int Bs, int H, int K, int n_logical, int F, int n_ranks,
                        int local_experts, int quant_mode, int tile, const float *quant_scales,
                        int quant_scales_kind, int32_t *balanced_ids,
                        uint8_t *balanced_mask, void *expand_x, void *expand_scales,
                        int32_t *expert_counts, int32_t *expert_offsets, int32_t *expand_src,
                        int32_t *assist_dst, int32_t *dev_err, void *stream);

/*
 * moe_combine_add_rmsnorm -- weighted gather of expert outputs, shared
 * expert and residual add, RMSNorm ("aclnnMoeDistributeCombineAddRmsNorm"
 * 计算公式: combineOut = Sum(expertScales*ataOut + expertScales*sharedExpertX),
 * x = combineOut + residualX, y = x / RMS(x) * gamma,
 * RMS(x) = sqrt(mean(x^2) + normEps)).
 *
 * For token i, with fp32 accumulation:
 *   acc  = sum over k with r = assist_dst[i*K+k] >= 0 of
 *          expert_scales[i*K+k] * expert_out[r]
 *   acc += w * shared_x[i]   (w = sum of those scales for MOE_SHARED_PAGE,
 *                             1 for MOE_SHARED_ADD; skipped if shared_x is NULL)
 *   x    = acc + residual_x[i];  x_out[i] = bf16(x)
 *   rstd = 1 / sqrt(mean(x^2) + eps);  y[i] = bf16(x * rstd * gamma)
 * The RMS is taken over the fp32 x before rounding.
 *
 *   expert_out   bf16 [Bs*K, H]   rows in dispatch order (expert FFN output)
 *   assist_dst   int32 [Bs, K]    from moe_dispatch (-1 = not dispatched)
 *   expert_scales f32 [Bs, K]
 *   shared_x     bf16 [Bs, H] or NULL
 *   residual_x   bf16 [Bs, H]
 *   gamma        bf16 [H]
 *   y            bf16 [Bs, H] (out)
 *   x_out        bf16 [Bs, H] or NULL (out)
 *   rstd         f32 [Bs] or NULL (out)
 *   dev_err      int32 [1] or NULL: MOE_ERR_ROW for an entry >= Bs*K (skipped)
 * Limits: 0 < Bs <= 512, 0 < K <= 16, H in [1024, 8192] with H % 32 == 0,
 *         eps >= 0 and finite, shared_mode in {0, 1}.
 */
int moe_combine_add_rmsnorm(const void *expert_out, const int32_t *assist_dst,
                            const float *expert_scales, const void *shared_x,
                            const void *residual_x, const void *gamma, float eps, int Bs,
                            int H, int K, int shared_mode, void *y, void *x_out, float *rstd,
                            int32_t *dev_err, void *stream);

/*
 * moe_expert_gemm -- the expert computation between dispatch and combine
 * (the calling sequence of "aclnnMoeUpdateExpert" places it there; the pages
 * do not define it).  One linear layer per instance over the rows dispatch
 * wrote for it, reading expand_x and expand_scales as dispatch leaves them
 * ("aclnnMoeDistributeDispatchV2", case 5: mxfp8):
 *
 *   for e < n_instances, r in [expert_offsets[e], expert_offsets[e+1]), n < N:
 *     y[r][n] = bf16( sum_k  A(r, k) * W(e, n, k) )        (fp32 accumulation)
 *     A(r, k)    = e4m3(expand_x[r][k])   * 2^(expand_scales[r][k/32] - 127)
 *     W(e, n, k) = e4m3(weights[e][n][k]) * 2^(S(e, n, k/32) - 127)
 *     S(e, n, b) = weight_scales[e][b/16][n][b%16]
 *
 * or, for the int8 outputs of dispatch cases 3 (MOE_Q_INT8_TOKEN) and 4
 * (MOE_Q_INT8_TILE, tiles of 128):
 *     y[r][n] = bf16( ws[e][n] * sum_t as[r][t] * sum_{k in tile t} a[r][k] * w[e][n][k] )
 * with one tile covering all of H (per token) or tiles of 128 (per tile);
 * integer sums are exact (int32), scaling and the sum over tiles are fp32.
 *
 *   expand_x       E4M3 or int8 [rows, H]                    16-byte aligned
 *   expand_scales  mxfp8: u8 E8M0 [rows, H/32] (MOE_Q_MXFP8), or group-major
 *                  [H/512 rounded up, rows, 16] (MOE_Q_MXFP8_GM: the dispatch's
 *                  layout for N = rows, so rows is the N of that call, the
 *                  capacity Bs*K); per token: f32 [rows]; per tile: f32
 *                  [rows, H/128]                             4-byte aligned
 *   expert_offsets int32 [n_instances+1] (moe_dispatch's offsets, or a slice
 *                  of them for a subset of instances; values are absolute rows)
 *   weights        E4M3 or int8 [n_instances, N, H]          16-byte aligned
 *   weight_scales  mxfp8: u8 E8M0 [n_instances, ceil(H/512), N, 16], group-major:
 *                  group q holds the exponents of K blocks 16q .. 16q+15 of every
 *                  column, 16 bytes per column (a last, partial group is padded; the
 *                  pad is never read), so the kernel's copies of one group for a
 *                  run of columns are contiguous.  A weight-preparation step, done
 *                  once per weight set: pack_mx_weight_scales in the binding.
 *                  int8: f32 [n_instances, N].                4-byte aligned
 *   y              bf16 [rows, N] (out; rows outside every instance's range
 *                  are not written)  16-byte aligned
 *   dev_err        int32 [1] or NULL: MOE_ERR_OFFSETS when the offsets are not
 *                  non-decreasing within [0, rows]; every range is then
 *                  clamped into [0, rows] and the output is unspecified
 *                  (but no access leaves the buffers)
 * Limits: 1 <= n_instances <= 1024, 0 <= rows <= 4194304, H and N multiples of
 * 128 in [128, 16384], quant_mode MOE_Q_MXFP8, MOE_Q_MXFP8_GM, MOE_Q_INT8_TOKEN
 * or MOE_Q_INT8_TILE (MOE_Q_NONE and the static modes: MOE_ENOTSUP).
 */
int moe_expert_gemm(const void *expand_x, const void *expand_scales,
                    const int32_t *expert_offsets, int n_instances, int rows,
                    const void *weights, const void *weight_scales, int N, int H,
                    int quant_mode, void *y, int32_t *dev_err, void *stream);

/*
 * moe_expert_swiglu -- the activation between the expert computation's two
 * projections, for the second projection's moe_expert_gemm.  The pages place
 * the expert step in the calling sequence of "aclnnMoeUpdateExpert" without
 * defining it; this library reads it as the gated FFN of a DeepSeek-V3-shaped
 * layer: a first moe_expert_gemm with N = 2I whose output row holds the gate g
 * (columns [0, I)) and the up projection u (columns [I, 2I)), this call, and a
 * second moe_expert_gemm with H = I whose output rows are the combine's
 * expert_out.  For every row r in [expert_offsets[0], expert_offsets[n_instances]):
 *
 *   act[r][j] = bf16( silu(g) * u ),  silu(g) = g / (1 + exp(-g))   (fp32, j < I)
 *
 * and act's row is coded with the mxfp8 quantiser of the dispatch
 * ("aclnnMoeDistributeDispatchV2", 计算公式 case 5), with the same rules as
 * moe_dispatch's MOE_Q_MXFP8 (infinities and NaNs included).  The fp32
 * expression may round to a bf16 one step away from the exact value's.
 *
 *   y1             bf16 [rows, 2I] (the first projection's output)  16-byte aligned
 *   expert_offsets int32 [n_instances+1] (as for moe_expert_gemm)
 *   quant_mode     MOE_Q_MXFP8 (act_scales u8 E8M0 [rows, I/32]) or MOE_Q_MXFP8_GM
 *                  (group-major [I/512 rounded up, rows, 16], the order the second
 *                  moe_expert_gemm reads fastest; rows is then that call's rows);
 *                  the int8 modes: MOE_ENOTSUP
 *   act_codes      E4M3 [rows, I] (out)                             16-byte aligned
 *   act_scales     E8M0 bytes, layout by quant_mode (out)
 *   act            bf16 [rows, I] or NULL (out)                     16-byte aligned
 *   dev_err        int32 [1] or NULL: MOE_ERR_OFFSETS when offsets[0] < 0,
 *                  offsets[n_instances] > rows or offsets[n_instances] < offsets[0];
 *                  the range is then clamped into [0, rows]
 * Rows outside the range are not written.  Limits: 1 <= n_instances <= 1024,
 * 0 <= rows <= 4194304, I a multiple of 128 in [128, 8192].
 */
int moe_expert_swiglu(const void *y1, const int32_t *expert_offsets, int n_instances, int rows,
                      int I, int quant_mode, void *act_codes, void *act_scales, void *act,
                      int32_t *dev_err, void *stream);

/* A static, human-readable name for a moe_status value. */
const char *moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERT_H */
