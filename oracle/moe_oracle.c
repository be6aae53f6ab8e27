/*
 * moe_oracle.c -- plain CPU oracle for the single-GPU share of an MoE layer's
 * expert mapping, token dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources (Ascend CANN operator documentation pages):
 *   [UPD] "aclnnMoeUpdateExpert": load balancing (map each token's top-K
 *         logical expert ids to deployed instances), expert pruning by a
 *         threshold broadcast over the batch, and the mapping-table format
 *         (column 0 = replica count > 0, columns 1.. = instance ids).
 *   [DSP] "aclnnMoeDistributeDispatchV2", 计算公式 (formula): case 1
 *         (quantMode 0, no quantisation), case 2 (quantMode 1, static), the
 *         scales factor of cases 2-4, case 3 (quantMode 2, per-token
 *         dynamic int8), case 4 (quantMode 3, per-tile dynamic int8), case 5
 *         (quantMode 4, mxfp8), and the note that emax is the exponent of
 *         the target type's largest normal number; 约束说明 (constraints) for
 *         the 1-D / 2-D active mask and the quantMode-dependent shapes of
 *         the scales input.
 *   [CMB] "aclnnMoeDistributeCombineAddRmsNorm", 计算公式 (formula): the
 *         weighted sum of expert outputs and shared-expert output, the
 *         residual add and RMSNorm.
 *   [SEQ] "aclnnMoeUpdateExpert", calling sequence: the expert computation
 *         sits between dispatch and combine and consumes expandX with its
 *         dynamicScales.  The pages do not define that computation; the
 *         oracle takes it as one linear layer per expert instance (below).
 *
 * Readings where the pages are silent or garbled:
 *   - instance ids are global: instance = rank * local_experts + local slot;
 *   - the replica used by token i is column 1 + (i mod replica count);
 *   - pruning keeps an entry unless score < threshold[k] (NaN is kept);
 *   - rows of one instance are ordered by ascending flat index f = i*K + k;
 *   - static int8 (quantMode 1): the cast rounds half to even and saturates
 *     to [-128, 127]; the scales input is one coefficient, one row of H
 *     shared by all experts, or one row per instance ([E, H], indexed by the
 *     instance a copy is sent to);
 *   - the second static output type (garbled on the page; it takes the
 *     (1,) scales shape only) is read as OCP E4M3, the type the mxfp8 mode
 *     writes: the cast rounds to nearest even and saturates at +-448, and a
 *     NaN product codes to 0x7F;
 *   - int8: dstTypeMax = 127, round half to even, clamp to [-127, 127],
 *     scale written = 1 / dynamicScales, all-zero segment -> codes 0, scale 0;
 *     if 127 / max overflows fp32 (max below about 3.7e-38), zero elements
 *     code to 0 and the others saturate to +-127 (scale 1/inf = 0);
 *   - per-tile mode: tiles of `tile` elements along H (128 in the workloads);
 *   - mxfp8: blocks of 32 along H, max(x) read as max |x|, emax = 8 (E4M3),
 *     fp8 cast rounds to nearest even and saturates at +-448, the scale byte
 *     is the E8M0 code of 2^sharedExp (the dequantisation multiplier),
 *     all-zero block -> exponent -127;
 *   - the shared-expert term is weighted by the sum of the token's active
 *     scales (the formula's literal reading) or by 1 (selectable);
 *   - RMS is taken over the unrounded x; y = x * (1 / RMS(x)) * gamma;
 *   - expert computation: rows offsets[e] .. offsets[e+1]-1 of expandX belong
 *     to instance e and are multiplied by that instance's weight matrix W[e]
 *     ([N, H], one row per output column); for mxfp8 both operands are
 *     dequantised as code value * 2^(scale byte - 127) per block of 32 along
 *     H, the products are summed exactly (fp64) and rounded once to bf16; for
 *     int8 (the per-token and per-tile outputs of [DSP] cases 3 and 4) the
 *     activations are dequantised as code * scale of their row (per token) or
 *     of their row's tile of 128 (per tile), the weights as code * one scale
 *     per output column, the integer products summed exactly per tile.
 *
 * Precision: the quantisers work in fp32 exactly as the dispatch formula's
 * CastToFp32 prescribes (IEEE division, no contraction; build with
 * -ffp-contract=off -fno-fast-math).  The combine is computed in fp64 and
 * rounded once to bf16.
 *
 * Parity pins: every exported function is pinned by CPU tests against brute
 * force, library routines, closed forms and invariants (tests/test_oracle_*.py).
 *
 * Threads: the per-token loops of the quantise-and-copy step and of the
 * combine run their tokens on OpenMP threads (each token's arithmetic is
 * unchanged and touches only its own rows); the routing (histogram, scan,
 * stable rank) stays sequential.  oracle_set_threads picks the count.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Threads for the per-token loops (n <= 0: all available); returns the count
 * now in effect. */
int oracle_set_threads(int n)
{
    omp_set_num_threads(n > 0 ? n : omp_get_num_procs());
    return omp_get_max_threads();
}

enum { ORC_ERR_ID = 1, ORC_ERR_TABLE = 2, ORC_ERR_MASK1D = 4 };

/* ---------------------------------------------------------------- numbers */

/* bf16 bit pattern -> value (exact: bf16 is the top half of an fp32). */
static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Nearest bf16 to a double, ties to even.  bf16 keeps 8 significant bits,
 * normal exponents [-126, 127], subnormal spacing 2^-133. */
static uint16_t bf16_from_double(double v)
{
    if (isnan(v))
        return 0x7FC0;
    double a = fabs(v), r = 0.0;
    if (a != 0.0) {
        int e = ilogb(a);          /* a in [2^e, 2^(e+1)) */
        int q = e - 7;             /* exponent of one unit in the last place */
        if (q < -133)
            q = -133;              /* subnormal grid */
        r = ldexp(nearbyint(ldexp(a, -q)), q);
    }
    float f = (r >= 0x1p128) ? INFINITY : (float)r;  /* r is exact in fp32 */
    if (signbit(v))
        f = -f;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* OCP FP8 E4M3 code of an fp32 value: bias 7, 3 mantissa bits, largest
 * finite 448 = 1.75 * 2^8, no infinities, 0x7F/0xFF = NaN.  Rounds to nearest
 * with ties to the even code and saturates at +-448.  Codes increase
 * monotonically with magnitude, so the subnormal grid m * 2^-9 and each
 * binade's grid (8 + m) * 2^(e-3) map to consecutive codes. */
static uint8_t e4m3_from_float(float v)
{
    uint8_t s = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return s | 0x7F;
    float a = fabsf(v);
    if (a >= 448.0f)
        return s | 0x7E;
    if (a < 0x1p-6f)                            /* below the smallest normal */
        return s | (uint8_t)nearbyintf(a * 512.0f);  /* 0..8; 8 is 2^-6 */
    int e = ilogbf(a);                          /* -6 .. 8 */
    int q = (int)nearbyintf(ldexpf(a, 3 - e));  /* 8 .. 16 */
    return s | (uint8_t)((e + 7) * 8 + (q - 8));
}

/* ---------------------------------------------------------------- quantisers */

/* [DSP] cases 3/4: dynamicScales = 127 / max|v| over the segment of fp32
 * values v (xFp32 of the formula); code = CastToInt8(v * dynamicScales); the
 * scale sent is 1 / dynamicScales. */
static void quant_int8_values(const float *v, int n, int8_t *q, float *scale)
{
    float m = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(v[j]);
        if (a > m)
            m = a;
    }
    if (m == 0.0f) {
        for (int j = 0; j < n; ++j)
            q[j] = 0;
        *scale = 0.0f;
        return;
    }
    float d = 127.0f / m;  /* +inf when m < 127 / FLT_MAX (a tiny subnormal maximum) */
    for (int j = 0; j < n; ++j) {
        float w = v[j] * d;
        float r = (w != w) ? 0.0f : nearbyintf(w);  /* 0 * inf: a zero element stays 0 */
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        q[j] = (int8_t)r;
    }
    *scale = 1.0f / d;
}

/* The same on bf16 input: xFp32 = CastToFp32(X) (exact). */
static void quant_int8_segment(const uint16_t *x, int n, int8_t *q, float *scale)
{
    float *v = (float *)malloc((size_t)n * sizeof(float));
    if (!v) {
        *scale = -1.0f;  /* never happens at the sizes tested */
        return;
    }
    for (int j = 0; j < n; ++j)
        v[j] = bf16_value(x[j]);
    quant_int8_values(v, n, q, scale);
    free(v);
}

/* [DSP] case 2 (static): quantOut = Cast(xFp32, int8): the nearest integer,
 * ties to even, saturated to [-128, 127]; NaN codes to 0. */
static int8_t int8_cast(float v)
{
    if (v != v)
        return 0;
    float r = nearbyintf(v);
    if (r > 127.0f)
        r = 127.0f;
    if (r < -128.0f)
        r = -128.0f;
    return (int8_t)r;
}

/* [DSP] case 2 (static) with the second output type, read as OCP E4M3:
 * quantOut = Cast(xFp32, E4M3), the cast of CastToFp8 (nearest, ties to the
 * even code, saturated at +-448).  A NaN product (a NaN in x, or an infinity
 * times a zero coefficient) codes to 0x7F: its sign is not fixed across
 * processors, so the code does not follow it. */
static uint8_t e4m3_static_cast(float v)
{
    if (v != v)
        return 0x7F;
    return e4m3_from_float(v);
}

/* [DSP] case 5: sharedExp = floor(log2(max|x|)) - emax with emax = 8;
 * code = CastToFp8(x / 2^sharedExp); scale byte = E8M0(2^sharedExp). */
static void quant_mxfp8_block(const uint16_t *x, int n, uint8_t *codes, uint8_t *scale_byte)
{
    float m = 0.0f;
    for (int j = 0; j < n; ++j) {
        float a = fabsf(bf16_value(x[j]));
        if (a > m)
            m = a;
    }
    int se = -127;
    if (m != 0.0f) {
        se = ilogbf(m) - 8;   /* exact floor(log2 m), subnormals included */
        if (se < -127)
            se = -127;
        if (se > 127)
            se = 127;
    }
    for (int j = 0; j < n; ++j)
        codes[j] = e4m3_from_float(ldexpf(bf16_value(x[j]), -se));
    *scale_byte = (uint8_t)(se + 127);
}

/* ---------------------------------------------------------------- exports */

void oracle_e4m3_encode(const float *v, int n, uint8_t *out)
{
    for (int j = 0; j < n; ++j)
        out[j] = e4m3_from_float(v[j]);
}

void oracle_bf16_round(const double *v, int n, uint16_t *out)
{
    for (int j = 0; j < n; ++j)
        out[j] = bf16_from_double(v[j]);
}

void oracle_quant_int8(const uint16_t *x, int n, int8_t *q, float *scale)
{
    quant_int8_segment(x, n, q, scale);
}

void oracle_quant_mxfp8(const uint16_t *x, int n, uint8_t *codes, uint8_t *scale_byte)
{
    quant_mxfp8_block(x, n, codes, scale_byte);
}

/* [UPD] map + prune.  For entry f = i*K + k with logical id e:
 *   keep      = token_mask[i] (if given) and not (score[f] < thr[k]) (if given)
 *   instance  = table[e][1 + (i mod table[e][0])]
 * An entry whose lookup fails (id, replica count or instance out of range)
 * gets instance -1 and keep 0; it raises an error bit only if it would have
 * been kept.  A 1-D token mask that is not all-true-then-all-false raises
 * bit 4 and is still applied as given. */
int oracle_update_expert(const int32_t *ids, const float *scores, const int32_t *table,
                         const float *thr, const uint8_t *token_mask, int Bs, int K,
                         int n_logical, int F, int n_instances, int32_t *out_ids,
                         uint8_t *out_mask, int32_t *err)
{
    if (Bs <= 0 || K <= 0 || n_logical <= 0 || F < 2 || n_instances <= 0)
        return -1;
    int32_t bits = 0;
    if (token_mask)
        for (int i = 1; i < Bs; ++i)
            if (token_mask[i] && !token_mask[i - 1])
                bits |= ORC_ERR_MASK1D;
    for (int i = 0; i < Bs; ++i) {
        for (int k = 0; k < K; ++k) {
            int f = i * K + k;
            int keep = (token_mask == NULL) || token_mask[i] != 0;
            if (scores && thr && scores[f] < thr[k])
                keep = 0;
            int e = ids[f], inst = -1, fail = 0;
            if (e < 0 || e >= n_logical) {
                fail = ORC_ERR_ID;
            } else {
                int n = table[(size_t)e * F];
                if (n < 1 || n > F - 1) {
                    fail = ORC_ERR_TABLE;
                } else {
                    inst = table[(size_t)e * F + 1 + (i % n)];
                    if (inst < 0 || inst >= n_instances) {
                        fail = ORC_ERR_TABLE;
                        inst = -1;
                    }
                }
            }
            if (fail) {
                if (keep)
                    bits |= fail;
                keep = 0;
            }
            out_ids[f] = inst;
            out_mask[f] = (uint8_t)keep;
        }
    }
    if (err)
        *err |= bits;
    return 0;
}

/* Expert-major routing of N = Bs*K entries over E instances: a stable
 * counting sort by instance id.
 *   counts[e]   = number of active entries with id e
 *   offsets     = exclusive prefix sum of counts, offsets[E] = total rows
 *   assist[f]   = destination row of entry f (-1 if not active)
 *   src[r]      = entry f placed in row r (-1 for r >= total)
 * Within an instance, rows follow ascending f.  An active entry whose id is
 * outside [0, E) raises bit 1 and is treated as inactive. */
int oracle_route(const int32_t *ids, const uint8_t *mask, int N, int E, int32_t *counts,
                 int32_t *offsets, int32_t *assist, int32_t *src, int32_t *err)
{
    if (N <= 0 || E <= 0)
        return -1;
    int32_t bits = 0;
    uint8_t *act = (uint8_t *)malloc((size_t)N);
    int32_t *cursor = (int32_t *)malloc((size_t)E * sizeof(int32_t));
    if (!act || !cursor) {
        free(act);
        free(cursor);
        return -2;
    }
    for (int f = 0; f < N; ++f) {
        act[f] = (mask == NULL) || mask[f] != 0;
        if (act[f] && (ids[f] < 0 || ids[f] >= E)) {
            bits |= ORC_ERR_ID;
            act[f] = 0;
        }
    }
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int f = 0; f < N; ++f)
        if (act[f])
            counts[ids[f]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int f = 0; f < N; ++f) {
        if (act[f]) {
            int r = cursor[ids[f]]++;
            assist[f] = r;
            src[r] = f;
        } else {
            assist[f] = -1;
        }
    }
    for (int r = offsets[E]; r < N; ++r)
        src[r] = -1;
    free(act);
    free(cursor);
    if (err)
        *err |= bits;
    return 0;
}

/* [DSP] dispatch on one device: route, then quantise each token once and copy
 * its coded row (and scales) into each of its destination rows.
 *   quant_mode 0: expand_x is bf16 [N, H], bit copies of x; no scales
 *   quant_mode 2: expand_x int8 [N, H]; scales f32 [N]
 *   quant_mode 3: expand_x int8 [N, H]; scales f32 [N, ceil(H / tile)]
 *   quant_mode 4: expand_x e4m3 [N, H]; scales E8M0 u8 [N, H / 32]
 * Rows at or past offsets[E] are not written. */
int oracle_dispatch(const uint16_t *x, const int32_t *ids, const uint8_t *mask, int Bs, int H,
                    int K, int n_ranks, int local_experts, int quant_mode, int tile,
                    void *expand_x, void *expand_scales, int32_t *counts, int32_t *offsets,
                    int32_t *expand_src, int32_t *assist_dst, int32_t *err)
{
    if (Bs <= 0 || H <= 0 || K <= 0 || n_ranks <= 0 || local_experts <= 0)
        return -1;
    if (quant_mode == 3 && tile <= 0)
        return -1;
    if (quant_mode == 4 && H % 32 != 0)
        return -1;
    if (quant_mode != 0 && quant_mode != 2 && quant_mode != 3 && quant_mode != 4)
        return -1;
    int E = n_ranks * local_experts, N = Bs * K;
    int rc = oracle_route(ids, mask, N, E, counts, offsets, assist_dst, expand_src, err);
    if (rc)
        return rc;

    int n_sc = 0;  /* scale entries per row */
    if (quant_mode == 2)
        n_sc = 1;
    else if (quant_mode == 3)
        n_sc = (H + tile - 1) / tile;
    else if (quant_mode == 4)
        n_sc = H / 32;

    int fail = 0;
#pragma omp parallel
    {
        int8_t *q = (int8_t *)malloc((size_t)H);
        float *fs = (float *)malloc((size_t)(n_sc > 0 ? n_sc : 1) * sizeof(float));
        uint8_t *bs = (uint8_t *)malloc((size_t)(n_sc > 0 ? n_sc : 1));
        if (!q || !fs || !bs) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int i = 0; i < Bs; ++i) {
            if (!q || !fs || !bs)
                continue;
            const uint16_t *xi = x + (size_t)i * H;
            if (quant_mode == 2) {
                quant_int8_segment(xi, H, q, &fs[0]);
            } else if (quant_mode == 3) {
                for (int t = 0; t < n_sc; ++t) {
                    int n = H - t * tile < tile ? H - t * tile : tile;
                    quant_int8_segment(xi + (size_t)t * tile, n, q + (size_t)t * tile, &fs[t]);
                }
            } else if (quant_mode == 4) {
                for (int b = 0; b < n_sc; ++b)
                    quant_mxfp8_block(xi + (size_t)b * 32, 32, (uint8_t *)q + (size_t)b * 32,
                                      &bs[b]);
            }
            for (int k = 0; k < K; ++k) {
                int r = assist_dst[i * K + k];
                if (r < 0)
                    continue;
                if (quant_mode == 0) {
                    memcpy((uint16_t *)expand_x + (size_t)r * H, xi, (size_t)H * sizeof(uint16_t));
                } else {
                    memcpy((int8_t *)expand_x + (size_t)r * H, q, (size_t)H);
                    if (quant_mode == 4)
                        memcpy((uint8_t *)expand_scales + (size_t)r * n_sc, bs, (size_t)n_sc);
                    else
                        memcpy((float *)expand_scales + (size_t)r * n_sc, fs,
                               (size_t)n_sc * sizeof(float));
                }
            }
        }
        free(q);
        free(fs);
        free(bs);
    }
    return fail ? -2 : 0;
}

/* [DSP] cases 2-4 with the scales input: xFp32 = CastToFp32(X) * scales, then
 *   quant_mode 1 (static):     code = Cast(xFp32, int8)            (int8_cast)
 *   quant_mode 6 (static):     code = Cast(xFp32, E4M3)            (e4m3_static_cast)
 *   quant_mode 2 (per token):  the dynamic int8 quantiser on xFp32
 *   quant_mode 3 (per tile):   the same per tile of `tile` elements
 * The scale applied to element j of the copy of token i sent to instance e is
 *   qscales_kind 0: none (1)    1: qscales[0]    2: qscales[j]
 *   qscales_kind 3: qscales[e * H + j]   (one row per instance, [E, H])
 * each one fp32 multiply.  Every (token, instance) copy is quantised on its
 * own (with kinds 0-2 all copies of a token are equal).  Outputs as
 * oracle_dispatch; quant_mode 1 writes no scales (expand_scales unused).
 * quant_mode 1 needs qscales_kind >= 1; modes 0 and 4 are oracle_dispatch's.
 * quant_mode 6 (the second static output type) takes one coefficient only
 * (qscales_kind 1: the quantMode constraints allow that type the (1,) shape
 * alone) and writes E4M3 bytes and no scales. */
int oracle_dispatch_scaled(const uint16_t *x, const int32_t *ids, const uint8_t *mask, int Bs,
                           int H, int K, int n_ranks, int local_experts, int quant_mode,
                           int tile, const float *qscales, int qscales_kind, void *expand_x,
                           void *expand_scales, int32_t *counts, int32_t *offsets,
                           int32_t *expand_src, int32_t *assist_dst, int32_t *err)
{
    if (Bs <= 0 || H <= 0 || K <= 0 || n_ranks <= 0 || local_experts <= 0)
        return -1;
    if (quant_mode < 1 || (quant_mode > 3 && quant_mode != 6) || qscales_kind < 0 ||
        qscales_kind > 3)
        return -1;
    if ((quant_mode == 1 && qscales_kind == 0) || (quant_mode == 6 && qscales_kind != 1) ||
        (qscales_kind != 0 && qscales == NULL))
        return -1;
    if (quant_mode == 3 && tile <= 0)
        return -1;
    int E = n_ranks * local_experts, N = Bs * K;
    int rc = oracle_route(ids, mask, N, E, counts, offsets, assist_dst, expand_src, err);
    if (rc)
        return rc;
    int n_sc = quant_mode == 2 ? 1 : quant_mode == 3 ? (H + tile - 1) / tile : 0;
    float *v = (float *)malloc((size_t)H * sizeof(float));
    if (!v)
        return -2;
    for (int f = 0; f < N; ++f) {
        int r = assist_dst[f];
        if (r < 0)
            continue;
        int i = f / K, e = ids[f];
        const uint16_t *xi = x + (size_t)i * H;
        for (int j = 0; j < H; ++j) {
            float s = 1.0f;
            if (qscales_kind == 1)
                s = qscales[0];
            else if (qscales_kind == 2)
                s = qscales[j];
            else if (qscales_kind == 3)
                s = qscales[(size_t)e * H + j];
            v[j] = qscales_kind == 0 ? bf16_value(xi[j]) : bf16_value(xi[j]) * s;
        }
        int8_t *q = (int8_t *)expand_x + (size_t)r * H;
        if (quant_mode == 6) {
            uint8_t *c = (uint8_t *)expand_x + (size_t)r * H;
            for (int j = 0; j < H; ++j)
                c[j] = e4m3_static_cast(v[j]);
        } else if (quant_mode == 1) {
            for (int j = 0; j < H; ++j)
                q[j] = int8_cast(v[j]);
        } else if (quant_mode == 2) {
            quant_int8_values(v, H, q, (float *)expand_scales + r);
        } else {
            for (int t = 0; t < n_sc; ++t) {
                int n = H - t * tile < tile ? H - t * tile : tile;
                quant_int8_values(v + (size_t)t * tile, n, q + (size_t)t * tile,
                                  (float *)expand_scales + (size_t)r * n_sc + t);
            }
        }
    }
    free(v);
    return 0;
}

/* [CMB] combine + add + RMSNorm for each token i, in fp64:
 *   acc  = sum over active k of s[i,k] * Eout[assist[i,k]]
 *   acc += w * shared[i]   with w = sum of active s[i,k] (shared_mode 0)
 *                          or w = 1 (shared_mode 1); skipped without shared
 *   x    = acc + residual[i]                 -> x_out = bf16(x)
 *   rstd = 1 / sqrt(mean(x^2) + eps)         -> y = bf16(x * rstd * gamma)
 * An entry with assist < 0 was not dispatched and contributes nothing. */
int oracle_combine_add_rmsnorm(const uint16_t *expert_out, const int32_t *assist,
                               const float *scales, const uint16_t *shared,
                               const uint16_t *residual, const uint16_t *gamma, float eps,
                               int Bs, int H, int K, int shared_mode, uint16_t *y,
                               uint16_t *x_out, float *rstd_out)
{
    if (Bs <= 0 || H <= 0 || K <= 0 || (shared_mode != 0 && shared_mode != 1))
        return -1;
    int fail = 0;
#pragma omp parallel
    {
        double *xf = (double *)malloc((size_t)H * sizeof(double));
        if (!xf) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(static)
        for (int i = 0; i < Bs; ++i) {
            if (!xf)
                continue;
            double ws = 0.0;
            for (int h = 0; h < H; ++h)
                xf[h] = 0.0;
            for (int k = 0; k < K; ++k) {
                int r = assist[i * K + k];
                if (r < 0)
                    continue;
                double s = scales[i * K + k];
                ws += s;
                const uint16_t *row = expert_out + (size_t)r * H;
                for (int h = 0; h < H; ++h)
                    xf[h] += s * (double)bf16_value(row[h]);
            }
            if (shared) {
                double w = shared_mode == 0 ? ws : 1.0;
                for (int h = 0; h < H; ++h)
                    xf[h] += w * (double)bf16_value(shared[(size_t)i * H + h]);
            }
            double ss = 0.0;
            for (int h = 0; h < H; ++h) {
                xf[h] += (double)bf16_value(residual[(size_t)i * H + h]);
                ss += xf[h] * xf[h];
            }
            double rstd = 1.0 / sqrt(ss / H + (double)eps);
            for (int h = 0; h < H; ++h) {
                if (x_out)
                    x_out[(size_t)i * H + h] = bf16_from_double(xf[h]);
                y[(size_t)i * H + h] =
                    bf16_from_double(xf[h] * rstd * (double)bf16_value(gamma[h]));
            }
            if (rstd_out)
                rstd_out[i] = (float)rstd;
        }
        free(xf);
    }
    return fail ? -2 : 0;
}

/* ---------------------------------------------------------------- expert GEMM */

/* OCP E4M3 code -> value, from the format: sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 is the subnormal grid m * 2^-9;
 * S.1111.111 is NaN. */
static double e4m3_value(uint8_t c)
{
    int ef = (c >> 3) & 15, m = c & 7;
    double v;
    if (ef == 15 && m == 7)
        return NAN;
    if (ef == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(8.0 + m, ef - 10);   /* (1 + m/8) * 2^(ef - 7) */
    return (c & 0x80) ? -v : v;
}

/* OCP E8M0 scale code -> 2^(c - 127); 255 is NaN. */
static double e8m0_value(uint8_t c)
{
    return c == 255 ? NAN : ldexp(1.0, (int)c - 127);
}

void oracle_e4m3_decode(const uint8_t *codes, int n, double *out)
{
    for (int j = 0; j < n; ++j)
        out[j] = e4m3_value(codes[j]);
}

/* [SEQ] expert computation, mxfp8 operands (the expandX / dynamicScales
 * layout of [DSP] case 5): for each instance e < E and each row r in
 * [offsets[e], offsets[e+1]):
 *   y[r][n] = bf16( sum_k  A(r, k) * W(e, n, k) ),  n < N, k < Kd
 *   A(r, k)    = e4m3(a[r][k])    * 2^(a_sc[r][k/32] - 127)
 *   W(e, n, k) = e4m3(w[e][n][k]) * 2^(w_sc[e][n][k/32] - 127)
 * Every product is exact in fp64 and the sum is taken in fp64.  y64 (if
 * given) receives the unrounded sums and abs64 (if given) the sums of the
 * products' magnitudes, both [rows, N].  Rows outside every instance's range
 * are left untouched.  Returns -1 for bad sizes or offsets that are not
 * non-decreasing within [0, rows]. */
int oracle_expert_gemm_mx(const uint8_t *a, const uint8_t *a_sc, const int32_t *offsets, int E,
                          int rows, const uint8_t *w, const uint8_t *w_sc, int N, int Kd,
                          uint16_t *y, double *y64, double *abs64)
{
    if (E <= 0 || rows < 0 || N <= 0 || Kd <= 0 || Kd % 32 != 0)
        return -1;
    if (offsets[0] < 0 || offsets[E] > rows)
        return -1;
    for (int e = 0; e < E; ++e)
        if (offsets[e] > offsets[e + 1])
            return -1;
    const int nb = Kd / 32;
    for (int e = 0; e < E; ++e) {
        const uint8_t *we = w + (size_t)e * N * Kd;
        const uint8_t *wse = w_sc + (size_t)e * N * nb;
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
            for (int n = 0; n < N; ++n) {
                double sum = 0.0, mag = 0.0;
                for (int k = 0; k < Kd; ++k) {
                    double av = e4m3_value(a[(size_t)r * Kd + k]) * e8m0_value(a_sc[(size_t)r * nb + k / 32]);
                    double wv = e4m3_value(we[(size_t)n * Kd + k]) * e8m0_value(wse[(size_t)n * nb + k / 32]);
                    sum += av * wv;
                    mag += fabs(av * wv);
                }
                y[(size_t)r * N + n] = bf16_from_double(sum);
                if (y64)
                    y64[(size_t)r * N + n] = sum;
                if (abs64)
                    abs64[(size_t)r * N + n] = mag;
            }
        }
    }
    return 0;
}

/* [SEQ] expert computation, int8 operands (the expandX / dynamicScales of
 * [DSP] case 3, per token, or case 4 with tiles of 128, per tile): for each
 * instance e < E and each row r in [offsets[e], offsets[e+1]), n < N:
 *   y[r][n] = bf16( sum_t a_sc[r][t] * w_sc[e][n] * sum_{k in tile t} a[r][k] * w[e][n][k] )
 * with n_tiles = 1 (one scale per row, the tile is all of Kd) or Kd / 128 (one
 * scale per row and tile of 128).  The integer sums are exact (int64), the
 * scaling and the sum over tiles are fp64, rounded once to bf16.  y64 / abs64
 * as for mxfp8 (abs64 = sum over k of |dequantised a * dequantised w|).
 * Returns -1 for bad sizes or offsets. */
int oracle_expert_gemm_i8(const int8_t *a, const float *a_sc, int n_tiles, const int32_t *offsets,
                          int E, int rows, const int8_t *w, const float *w_sc, int N, int Kd,
                          uint16_t *y, double *y64, double *abs64)
{
    if (E <= 0 || rows < 0 || N <= 0 || Kd <= 0)
        return -1;
    if (!(n_tiles == 1 || (Kd % 128 == 0 && n_tiles == Kd / 128)))
        return -1;
    if (offsets[0] < 0 || offsets[E] > rows)
        return -1;
    for (int e = 0; e < E; ++e)
        if (offsets[e] > offsets[e + 1])
            return -1;
    const int tl = Kd / n_tiles;
    for (int e = 0; e < E; ++e) {
        const int8_t *we = w + (size_t)e * N * Kd;
        for (int r = offsets[e]; r < offsets[e + 1]; ++r) {
            for (int n = 0; n < N; ++n) {
                const double ws = (double)w_sc[(size_t)e * N + n];
                double sum = 0.0, mag = 0.0;
                for (int t = 0; t < n_tiles; ++t) {
                    int64_t isum = 0, iabs = 0;
                    for (int k = t * tl; k < (t + 1) * tl; ++k) {
                        int64_t prod = (int64_t)a[(size_t)r * Kd + k] * (int64_t)we[(size_t)n * Kd + k];
                        isum += prod;
                        iabs += prod < 0 ? -prod : prod;
                    }
                    const double as = (double)a_sc[(size_t)r * n_tiles + t];
                    sum += as * ws * (double)isum;
                    mag += fabs(as * ws) * (double)iabs;
                }
                y[(size_t)r * N + n] = bf16_from_double(sum);
                if (y64)
                    y64[(size_t)r * N + n] = sum;
                if (abs64)
                    abs64[(size_t)r * N + n] = mag;
            }
        }
    }
    return 0;
}

/* [SEQ] expert computation, the activation between its two projections.  The
 * pages name the expert step and its operand formats only; the reading here is
 * the gated FFN of a DeepSeek-V3-shaped layer: the first projection's output
 * row holds the gate g (columns [0, I)) and the up projection u (columns
 * [I, 2I)) side by side, and
 *   act[r][j] = bf16( silu(g) * u ),  silu(g) = g / (1 + exp(-g))
 * evaluated in fp64 and rounded once to bf16.  Each act row is then coded for
 * the second projection with the quantiser of [DSP] case 5 (blocks of 32,
 * sharedExp = floor(log2 max|act|) - 8, E4M3 codes, E8M0 byte sharedExp + 127).
 * For every row r in [offsets[0], offsets[E]):
 *   y1    bf16 [rows, 2I]  (in)
 *   act   bf16 [rows, I]   (out, may be NULL)
 *   codes E4M3 [rows, I], scales E8M0 [rows, I/32]  (out)
 * Rows outside that range are left untouched.  Returns -1 for bad sizes or
 * offsets that are not non-decreasing within [0, rows]. */
int oracle_swiglu_mx(const uint16_t *y1, const int32_t *offsets, int E, int rows, int I,
                     uint16_t *act, uint8_t *codes, uint8_t *scales)
{
    if (E <= 0 || rows < 0 || I <= 0 || I % 32 != 0)
        return -1;
    if (offsets[0] < 0 || offsets[E] > rows)
        return -1;
    for (int e = 0; e < E; ++e)
        if (offsets[e] > offsets[e + 1])
            return -1;
    uint16_t *a = (uint16_t *)malloc((size_t)I * sizeof(uint16_t));
    if (!a)
        return -2;
    for (int r = offsets[0]; r < offsets[E]; ++r) {
        const uint16_t *row = y1 + (size_t)r * 2 * I;
        for (int j = 0; j < I; ++j) {
            double g = bf16_value(row[j]), u = bf16_value(row[I + j]);
            a[j] = bf16_from_double(g / (1.0 + exp(-g)) * u);
        }
        if (act)
            memcpy(act + (size_t)r * I, a, (size_t)I * sizeof(uint16_t));
        for (int b = 0; b < I / 32; ++b)
            quant_mxfp8_block(a + 32 * b, 32, codes + (size_t)r * I + 32 * b,
                              scales + (size_t)r * (I / 32) + b);
    }
    free(a);
    return 0;
}
