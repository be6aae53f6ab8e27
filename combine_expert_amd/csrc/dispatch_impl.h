// dispatch_impl.h -- the dispatch kernels (see dispatch.hip for the design),
// shared by the translation units that instantiate them, one per quantisation
// mode (dispatch_m0.hip .. dispatch_m4.hip), so that they compile in parallel.
#pragma once

#include "device.h"
#include "kernels.h"

namespace moe {


constexpr int kHistSlots = 1024;  // one LDS counter per instance (E <= 1024)
// Tokens (rows) per token block.  Two would halve the per-row routing work
// (the loads of every id, the histogram, the table lookups) but measured
// slower (c3: 9.2 against 7.8 us; fused mapping 12.3 against 9.5): with one
// block per compute unit, each block's barrier holds all of its rows.  The
// body works for any count; the per-instance scales variant would not fit
// its registers in 1024 threads.
template <bool PE>
constexpr int tokens_per_block() { return 1; }
constexpr int kDispatchWaves = kMaxWaves * 2;
constexpr int kPreOne = 0x10001;  // packed counter increment: all (low) and before-token (high)
constexpr int kMaxTokens = 512;   // Bs limit: staged token mask
constexpr int kMaxTopK = 16;      // K limit: staged thresholds

constexpr int kStageTab = 4;      // mapping-table words per thread staged through registers
constexpr int kStageTok = 4;      // token-mask bytes per thread staged through registers

// floor(a / d) for 0 <= a < 2^23, 1 <= d <= 1024: fp32 reciprocal estimate
// (off by far less than one unit here) and one correction step.
__device__ __forceinline__ int small_div(int a, int d)
{
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)d));
    const int r = a - q * d;
    q += r < 0 ? -1 : (r >= d ? 1 : 0);
    return q;
}

// The staged copy of the mapping table is prepared for lookups: the first
// word of row e packs its replica count n (bits 0-10; 1 if the row is
// malformed), m = ceil(2^19 / n) (bits 11-30) and a malformed-row flag (bit
// 31, count outside [1, F-1]); the instance words hold -1 where the table's
// instance is outside [0, E).  Then i mod n = i - n * ((i * m) >> 19), exact
// for token indices i < 512 and n <= 1024.
__device__ __forceinline__ int staged_table_word(int v, int col, int F, int E)
{
    const int inst = (unsigned)v < (unsigned)E ? v : -1;
    const bool ok = v >= 1 && v <= F - 1;
    const int nn = ok ? v : 1;
    const int m = small_div((1 << 19) + nn - 1, nn);
    const int head = (ok ? 0 : (int)0x80000000) | (m << 11) | nn;
    return col == 0 ? head : inst;  // straight-line: no branch between loads and waits
}

__device__ __forceinline__ int replica_slot(int head, int i)
{
    const unsigned nn = (unsigned)head & 2047u;
    const unsigned m = ((unsigned)head >> 11) & 0xfffffu;
    return i - (int)(nn * ((unsigned)i * m >> 19));
}

// Entry sources.  Both load 16-byte groups of four [Bs, K] ids plus a
// per-group side word (mask bytes or scores) and turn each entry into
// (instance id or -1, active), raising device error bits.

// Routed: instance ids and an optional [Bs, K] mask.  Ids outside [0, E) of
// active entries raise bit 1.
struct Routed {
    static constexpr bool kMapped = false;
    static constexpr bool kKeep = false;
    using Side = uint32_t;
    const int32_t *ids;
    const uint8_t *mask;  // null: every entry is active
    int E;

    __device__ Side side4(int g4) const
    {
        return mask ? reinterpret_cast<const uint32_t *>(mask)[g4] : 0x01010101u;
    }
    // the four entries of group g4 as f(inst, on, g)
    template <typename Fn>
    __device__ void group(const int4 &v, Side m, int g4, bool in, int &err, Fn &&f) const
    {
        const int idv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool act = in && ((m >> (8 * j)) & 0xffu) != 0;
            const bool ok = (unsigned)idv[j] < (unsigned)E;
            err |= act && !ok ? 1 : 0;
            const bool on = act && ok;
            f(on ? idv[j] : -1, on, g4 * 4 + j);
        }
    }
    __device__ int entry1(int g, bool &on, int &err) const
    {
        const int id = ids[g];
        const bool act = mask == nullptr || mask[g] != 0;
        const bool ok = (unsigned)id < (unsigned)E;
        err |= act && !ok ? 1 : 0;
        on = act && ok;
        return on ? id : -1;
    }
};

// Mapped (expert mapping and pruning fused in): logical ids go through the
// mapping table, staged in LDS (prepared as staged_table_word describes).
// With KEEP, the token mask (all ones when absent) and the thresholds (-inf
// when absent, so that the scores -- or the ids read in their place -- never
// prune) are staged too and tested; without, every entry is kept.  Token
// index i = g / K and i mod n are multiply-shifts (24-bit multiplies).  The
// LDS reads of an entry are the row head, then the instance slot.  Lookup
// failures raise bit 1 (logical id out of range) or 2 (malformed row,
// instance out of range), for entries that would otherwise be kept only.
template <bool KEEP>
struct Mapped {
    static constexpr bool kMapped = true;
    static constexpr bool kKeep = KEEP;
    using Side = float4;
    const int32_t *ids;
    const float *scores;  // [Bs, K], or the ids when nothing is pruned
    const int *tab;       // LDS [n_logical, F]
    const uint8_t *tok;   // LDS [Bs]
    const float *thr;     // LDS [K]
    int n_logical, F, E, K;
    unsigned mK;          // ceil(2^17 / K): g / K = (g * mK) >> 17 for g < 8192

    __device__ Side side4(int g4) const
    {
        if (KEEP)
            return reinterpret_cast<const float4 *>(scores)[g4];
        return make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ int token_of(int g) const { return (int)(__umul24((unsigned)g, mK) >> 17); }
    __device__ bool keep_of(int i, int k, float score) const
    {
        if (!KEEP)
            return true;
        const int tv = tok[i];    // both read, no short circuit:
        const float th = thr[k];  // the reads are then issued together
        return (tv != 0) & !(score < th);
    }
    __device__ int lookup(int head, int at, int i) const
    {
        const unsigned nn = (unsigned)head & 2047u;
        const unsigned m = ((unsigned)head >> 11) & 0xfffffu;
        const int slot = i - (int)__umul24(nn, __umul24((unsigned)i, m) >> 19);
        return tab[at + 1 + slot];
    }
    // entry (token i, column k) with logical id e
    __device__ int map(int e, int i, int k, float score, bool in, bool &on, int &err) const
    {
        const bool keep = in && keep_of(i, k, score);
        const bool e_ok = (unsigned)e < (unsigned)n_logical;
        const int at = (int)__umul24(e_ok ? (unsigned)e : 0u, (unsigned)F);
        const int head = tab[at];
        const int inst = lookup(head, at, i);
        const int fail = !e_ok ? 1 : (head < 0 || inst < 0) ? 2 : 0;
        err |= keep ? fail : 0;
        on = keep && fail == 0;
        return fail ? -1 : inst;
    }
    // The four entries of group g4, mapped phase by phase -- row heads (and
    // token / threshold reads), then instance slots -- so that each phase's
    // LDS reads are in flight together, then visited as f(inst, on, g).
    // (Entry by entry, the LDS reads would queue behind the previous
    // counter update.)
    template <typename Fn>
    __device__ void group(const int4 &v, Side sc, int g4, bool in, int &err, Fn &&f) const
    {
        const int idv[4] = {v.x, v.y, v.z, v.w};
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
        const int g0 = in ? g4 * 4 : 0;
        int ii[4], at[4], hv[4];
        bool keep[4], e_ok[4];
        if ((K & 3) == 0) {
            // the group is one token's columns k0 .. k0 + 3: one token index,
            // one mask byte and one 16-byte threshold read
            const int i0 = token_of(g0);
            const int k0 = g0 - (int)__umul24((unsigned)i0, (unsigned)K);
            bool kp[4] = {true, true, true, true};
            if (KEEP) {
                const int tv = tok[i0];
                const float4 th = *reinterpret_cast<const float4 *>(thr + k0);
                kp[0] = (tv != 0) & !(scv[0] < th.x);
                kp[1] = (tv != 0) & !(scv[1] < th.y);
                kp[2] = (tv != 0) & !(scv[2] < th.z);
                kp[3] = (tv != 0) & !(scv[3] < th.w);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                keep[j] = in && kp[j];
                ii[j] = i0;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = token_of(g0 + j);
                keep[j] =
                    in && keep_of(i, g0 + j - (int)__umul24((unsigned)i, (unsigned)K), scv[j]);
                ii[j] = i;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            e_ok[j] = (unsigned)idv[j] < (unsigned)n_logical;
            at[j] = (int)__umul24(e_ok[j] ? (unsigned)idv[j] : 0u, (unsigned)F);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            hv[j] = tab[at[j]];
        int inst[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            inst[j] = lookup(hv[j], at[j], ii[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int fail = !e_ok[j] ? 1 : (hv[j] < 0 || inst[j] < 0) ? 2 : 0;
            err |= keep[j] ? fail : 0;
            const bool on = keep[j] && fail == 0;
            f(on ? inst[j] : -1, on, g4 * 4 + j);
        }
    }
    __device__ int entry1(int g, bool &on, int &err) const
    {
        const int i = token_of(g);
        return map(ids[g], i, g - i * K, KEEP ? scores[g] : 0.0f, true, on, err);
    }
};

// Visits every entry g this thread owns -- int4 groups g4 = t, t + T, ...,
// then the scalar tail -- as f(inst, on, g) with inst = -1 unless on.  Each
// batch issues four 16-byte id loads (and side words) before using any;
// indices past the end are clamped and visited as inactive.
// after_first_issue() runs once, right after the first batch is issued:
// loads placed there stay in flight while the batch is consumed.
template <typename Src, typename Fn, typename G>
__device__ __forceinline__ void for_each_entry(const Src &s, int N, int &err, Fn &&f,
                                               G &&after_first_issue)
{
    const int t = threadIdx.x, T = blockDim.x;
    const int N4 = N >> 2;
    const int4 *ids4 = reinterpret_cast<const int4 *>(s.ids);
    bool first = true;
    for (int base = t; base < N4 || first; base += 4 * T) {
        int4 v[4];
        typename Src::Side m[4];
        if (N4 > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int g4 = min(base + u * T, N4 - 1);
                v[u] = ids4[g4];
                m[u] = s.side4(g4);
            }
        }
        if (first) {
            after_first_issue();
            first = false;
        }
        if (N4 == 0)
            break;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g4 = base + u * T;
            // groups past the end for the whole wave (its first lane has the
            // smallest g4) are skipped with a uniform branch
            if (__builtin_amdgcn_readfirstlane(g4) < N4)
                s.group(v[u], m[u], g4, g4 < N4, err, f);
        }
    }
    for (int g = N4 * 4 + t; g < N; g += T) {
        bool on;
        const int inst = s.entry1(g, on, err);
        f(inst, on, g);
    }
}

struct DispatchArgs {
    const uint16_t *x;
    const int32_t *ids;          // instance ids (routed) or logical ids (mapped)
    const uint8_t *mask;         // routed: [Bs, K] or null
    const float *scores;         // mapped: [Bs, K], or null when nothing is pruned
    const int32_t *table;        // mapped: [n_logical, F]
    const float *thr;            // mapped: [K], or null when nothing is pruned
    const uint8_t *token_mask;   // mapped: [Bs] or null
    int n_logical, F;            // mapped
    int Bs, H, K, E, tile;
    const float *qs;             // scales input: [1], [H] or [E, H] by qs_kind, or null
    int qs_kind;                 // MOE_SCALES_*: 0 none, 1 one, 2 row, 3 one row per instance
    void *expand_x, *expand_scales;
    int32_t *counts, *offsets, *expand_src, *assist_dst;
    int32_t *balanced_ids;       // mapped, may be null
    uint8_t *balanced_mask;      // mapped, may be null
    int32_t *dev_err;
};

// Mapped source: the table (prepared by staged_table_word), the token mask
// (all ones when absent) and the thresholds (-inf when absent) go to LDS.
// issue() loads the first kStageTab table words and kStageTok mask bytes of
// this thread into registers; store() writes them to LDS.  Both use clamped
// indices and no branches (threads past the end rewrite the last word with
// the value it gets anyway), so that the compiler can wait for exactly these
// loads.  rest() stages whatever lies beyond, with plain loops; it runs at
// the start of the kernel, before other loads are in flight, and only when
// the table or the batch is that large.  The caller puts a barrier after
// store().
template <bool KEEP>
struct Stage {
    int tabv[kStageTab];
    uint8_t tokv[kStageTok];
    float thrv;

    __device__ __forceinline__ void issue(const DispatchArgs &a)
    {
        const int t = threadIdx.x, T = blockDim.x;
        const int tabsz = a.n_logical * a.F;
#pragma unroll
        for (int u = 0; u < kStageTab; ++u)
            tabv[u] = a.table[min(t + u * T, tabsz - 1)];
        if (!KEEP)
            return;
        const uint8_t *tm = a.token_mask ? a.token_mask : reinterpret_cast<const uint8_t *>(a.table);
#pragma unroll
        for (int u = 0; u < kStageTok; ++u)
            tokv[u] = tm[a.token_mask ? min(t + u * T, a.Bs - 1) : 0];
        const float *th = a.thr ? a.thr : reinterpret_cast<const float *>(a.table);
        thrv = th[a.thr ? min(t, a.K - 1) : 0];
    }

    // The empty asm statements pin the loaded words: nothing computed from
    // them can be moved above this point, ahead of loads issued before it.
    __device__ __forceinline__ void store(const DispatchArgs &a, int *s_tab, uint8_t *s_tok,
                                          float *s_thr)
    {
        const int t = threadIdx.x, T = blockDim.x;
        const int tabsz = a.n_logical * a.F;
#pragma unroll
        for (int u = 0; u < kStageTab; ++u) {
            asm volatile("" : "+v"(tabv[u]));
            const int j = min(t + u * T, tabsz - 1);
            s_tab[j] = staged_table_word(tabv[u], j - a.F * small_div(j, a.F), a.F, a.E);
        }
        if (!KEEP)
            return;
#pragma unroll
        for (int u = 0; u < kStageTok; ++u)
            s_tok[min(t + u * T, a.Bs - 1)] = a.token_mask ? tokv[u] : 1;
        s_thr[min(t, a.K - 1)] = a.thr ? thrv : -__builtin_inff();
    }

    static __device__ __forceinline__ void rest(const DispatchArgs &a, int *s_tab,
                                                uint8_t *s_tok)
    {
        const int t = threadIdx.x, T = blockDim.x;
        const int tabsz = a.n_logical * a.F;
        if (tabsz > kStageTab * T) {
            for (int j = t + kStageTab * T; j < tabsz; j += T)
                s_tab[j] = staged_table_word(a.table[j], j - a.F * small_div(j, a.F), a.F, a.E);
        }
        if (KEEP && a.Bs > kStageTok * T) {
            for (int j = t + kStageTok * T; j < a.Bs; j += T)
                s_tok[j] = a.token_mask ? a.token_mask[j] : 1;
        }
    }
};

// ------------------------------------------------------------------ block 0

template <typename Src>
__device__ void route_summary(const DispatchArgs &a, const Src &s, int *s_hist, int *s_wave,
                              int *s_tab, uint8_t *s_tok, float *s_thr)
{
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const int N = a.Bs * a.K, E = a.E;
    if (Src::kMapped)
        Stage<Src::kKeep>::rest(a, s_tab, s_tok);
    for (int e = t; e < E; e += T)
        s_hist[e] = 0;
    int err = 0;
    for_each_entry(
        s, N, err,
        [&](int inst, bool on, int) {
            if (on)
                atomicAdd(&s_hist[inst], 1);
        },
        [&] {
            if (Src::kMapped) {
                Stage<Src::kKeep> st;
                st.issue(a);
                st.store(a, s_tab, s_tok, s_thr);
            }
            lds_barrier();
        });
    if (Src::kKeep) {  // a 1-D token mask is all true, then all false
        for (int i = 1 + t; i < a.Bs; i += T)
            err |= s_tok[i] && !s_tok[i - 1] ? 4 : 0;
    }
    if (err && a.dev_err)
        atomicOr(a.dev_err, err);
    lds_barrier();

    // exclusive scan: each thread owns a contiguous run of counters
    const int per = (E + T - 1) / T;
    const int e0 = min(t * per, E), e1 = min(e0 + per, E);
    int local = 0;
    for (int e = e0; e < e1; ++e)
        local += s_hist[e];
    const int incl = wave_incl_scan(local);
    if (lane == kWave - 1)
        s_wave[w] = incl;
    lds_barrier();
    int base = 0, total = 0;
    for (int j = 0; j < nw; ++j) {
        const int v = s_wave[j];
        base += j < w ? v : 0;
        total += v;
    }
    int run = base + incl - local;
    for (int e = e0; e < e1; ++e) {
        const int c = s_hist[e];
        a.counts[e] = c;
        a.offsets[e] = run;
        run += c;
    }
    if (t == 0)
        a.offsets[E] = total;
    for (int r = total + t; r < N; r += T)
        a.expand_src[r] = -1;
}

// ------------------------------------------------------------------ token blocks

// Token blocks use the row layout of device.h: lane l of wave w holds part 0
// (elements e0 = 1024 w + 8 l .. + 7) and part 1 (e1 = e0 + 512 .. + 7) of
// the token's row, and writes the codes of each part as 8 bytes (16 for bf16
// rows), so every store instruction of a wave covers 512 contiguous bytes of
// codes (1 KB of bf16).  A part past the row end reads zeros and its stores
// go to an offset past the buffer (dropped).  Coded rows are stored with the
// device-scope policy, which writes them through to memory: for these
// scattered rows it measured faster than non-temporal or default stores
// (c3: 5.5 against 6.3-6.5 us for the bare scatter), and it leaves no dirty
// lines for the end of the kernel to write back.  Scales (a few bytes per
// lane, partial lines) keep the default policy, so that L2 merges the pieces
// of a line: written through, they cost 0.3 us more at c3.
struct Lane {
    int e0, e1;    // first element of each part
    bool v0, v1;   // part inside the row
};

__device__ __forceinline__ Lane lane_parts(int t, int H)
{
    Lane L;
    L.e0 = part_elem(t, 0);
    L.e1 = part_elem(t, 1);
    L.v0 = L.e0 < H;
    L.v1 = L.e1 < H;
    return L;
}

__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)d << 24);
}

// Largest |x| bit pattern among 8 bf16 (sign cleared).  For non-negative
// values the integer order of bf16 patterns is the numeric order.
__device__ __forceinline__ uint32_t amax_bits8(const uint4 &a)
{
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        m = max(m, w[j] & 0x7fffu);
        m = max(m, (w[j] >> 16) & 0x7fffu);
    }
    return m;
}

// int8 codes of 8 values with multiplier d: clamp(rint(v * d), -127, 127).
// d is +inf when 127 / max overflows (a tiny subnormal maximum): zeros then
// give 0 * inf = NaN and are coded 0, the rest saturate.
__device__ __forceinline__ uint2 int8_codes8(const float *v, float d)
{
    int q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float r = __builtin_rintf(v[j] * d);
        r = r != r ? 0.0f : r;
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q[j] = (int)r;
    }
    return make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
}

// int8 codes of 8 fp32 values for the static mode: the nearest integer, ties
// to even, saturated to [-128, 127]; NaN codes to 0.
__device__ __forceinline__ uint2 int8_static_codes8(const float *v)
{
    int q[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float r = __builtin_rintf(v[j]);
        r = r != r ? 0.0f : r;
        r = fminf(fmaxf(r, -128.0f), 127.0f);
        q[j] = (int)r;
    }
    return make_uint2(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]));
}

// E4M3 codes of 8 values multiplied by the power of two f (an exact product):
// clamp to +-448 (saturation), then the gfx950 packed conversion, which
// rounds to nearest even and keeps the sign of zero.
__device__ __forceinline__ uint2 e4m3_codes8(const float *v, float f)
{
    uint32_t w[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float a = fminf(fmaxf(v[4 * q] * f, -448.0f), 448.0f);
        const float b = fminf(fmaxf(v[4 * q + 1] * f, -448.0f), 448.0f);
        const float c = fminf(fmaxf(v[4 * q + 2] * f, -448.0f), 448.0f);
        const float d = fminf(fmaxf(v[4 * q + 3] * f, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
        w[q] = (uint32_t)p;
    }
    return make_uint2(w[0], w[1]);
}

// floor(log2(m)) of a positive bf16 magnitude pattern (normal or subnormal)
__device__ __forceinline__ int bf16_ilogb(uint32_t m)
{
    const int ex = (int)(m >> 7);
    return ex ? ex - 127 : (31 - __clz((int)(m & 0x7f))) - 133;
}

// mxfp8 shared exponent of a block whose largest |x| pattern is m
__device__ __forceinline__ int mx_exponent(uint32_t m)
{
    int se = -127;
    if (m) {
        se = bf16_ilogb(m) - 8;
        se = max(-127, min(127, se));
    }
    return se;
}

// Maximum over the lanes of one tile of a part (tile / 8 lanes, tile <= 512),
// in each of them: DPP steps up to 16 lanes, then lane shuffles.
__device__ __forceinline__ uint32_t tile_max(uint32_t m, int lanes)
{
    m = group_max_u32(m, lanes < 32 ? lanes : 32);
    if (lanes >= 64)
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
    return m;
}

// this thread's 8 + 8 values of scales row e ([E, H] or [H]); a part past the
// row end reads the row's first chunk (its values are not used)
__device__ __forceinline__ void scale_row_parts(const float *qs, int e, int H, const Lane &L,
                                                float4 (&s)[4])
{
    const float *row = qs + (size_t)e * H;
    const float4 *p0 = reinterpret_cast<const float4 *>(row + (L.v0 ? L.e0 : 0));
    const float4 *p1 = reinterpret_cast<const float4 *>(row + (L.v1 ? L.e1 : 0));
    s[0] = p0[0];
    s[1] = p0[1];
    s[2] = p1[0];
    s[3] = p1[1];
}

// w = v * s for the lane's 16 values; a part past the row end gives zeros
__device__ __forceinline__ void scaled16(const float *v, const float4 (&s)[4], const Lane &L,
                                         float *w)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool ok = q < 2 ? L.v0 : L.v1;
        w[4 * q] = ok ? v[4 * q] * s[q].x : 0.0f;
        w[4 * q + 1] = ok ? v[4 * q + 1] * s[q].y : 0.0f;
        w[4 * q + 2] = ok ? v[4 * q + 2] * s[q].z : 0.0f;
        w[4 * q + 3] = ok ? v[4 * q + 3] * s[q].w : 0.0f;
    }
}

__device__ __forceinline__ uint32_t absmax_bits_f(const float *w, int n)
{
    float m = 0.0f;
    for (int j = 0; j < n; ++j)
        m = fmaxf(m, fabsf(w[j]));
    return __float_as_uint(m);  // non-negative floats order like their bit patterns
}

// Output buffers of one dispatch launch.
struct Out {
    rsrc_t x, sc;
    uint32_t row_bytes;   // bytes of one expand_x row
    uint32_t sc_row;      // scale entries per row (modes 2-4)
};

__device__ __forceinline__ Out out_buffers(const DispatchArgs &a, int MODE)
{
    const int N = a.Bs * a.K;
    const int elt = MODE == 0 ? 2 : 1;
    Out o;
    o.row_bytes = (uint32_t)a.H * elt;
    o.x = buffer_rsrc(a.expand_x, (uint32_t)N * o.row_bytes);
    o.sc_row = MODE == 2 ? 1u : MODE == 3 ? (uint32_t)((a.H + a.tile - 1) / a.tile)
                                          : MODE == 4 ? (uint32_t)(a.H / 32) : 0u;
    const uint32_t sc_bytes = MODE == 4 ? 1u : 4u;
    o.sc = buffer_rsrc(a.expand_scales ? a.expand_scales : a.expand_x,
                       a.expand_scales ? (uint32_t)N * o.sc_row * sc_bytes : 0u);
    return o;
}

// Writes one tile scale of part p of a per-tile int8 row: the tile's first
// lane in the part stores it (tiles of 1024 span both parts of a wave: lane 0
// of part 0 stores it).
__device__ __forceinline__ void store_tile_scale(const Out &o, uint32_t row, int tile, int lane,
                                                 int e, bool ok, int p, float f)
{
    const int lanes = tile >= kWaveElems ? 2 * kWave : tile / kPartElems;
    const bool first = tile >= kWaveElems ? (lane == 0 && p == 0) : (lane & (lanes - 1)) == 0;
    if (ok && first)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f), o.sc,
                                              (row * o.sc_row + (uint32_t)(e / tile)) * 4u, 0,
                                              kPlain);
}

// One scales row per instance (the scales input of shape [E, H]): every copy
// k of the token is quantised on its own from xFp32 = x * row(eid[k]).  Rows
// are prefetched kPrefetch copies ahead (they come from L2 or the Infinity
// Cache: the table is E * H * 4 bytes).  Per-token dynamic int8 needs each
// copy's maximum over the whole row first: a pass computes all K maxima
// (one barrier for all of them), a second pass codes.  s_pmax: LDS
// [kDispatchWaves][KMAX]; tr is the thread's index in its token's row, w its
// wave in the block, waves [w0, w0 + rw) the token's.
constexpr int kPrefetch = 4;

template <int MODE, int KMAX>
__device__ __forceinline__ void code_store_rows(const DispatchArgs &a, int tr, int w, int w0,
                                                int rw, const Lane &L, const uint4 &xa,
                                                const uint4 &xb, const int *rank,
                                                const int *eid, uint32_t *s_pmax)
{
    constexpr int D = KMAX < kPrefetch ? KMAX : kPrefetch;
    const int H = a.H;
    const int lane = tr & (kWave - 1);
    const Out o = out_buffers(a, MODE);
    float v[16];
    unpack8(xa, v);
    unpack8(xb, v + 8);
    int ek[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        ek[k] = rank[k] >= 0 ? eid[k] : 0;  // copies not sent read a valid row, unused
    float4 ring[D][4];

    float amax[KMAX];
    if (MODE == 2) {
#pragma unroll
        for (int p = 0; p < D; ++p)
            scale_row_parts(a.qs, ek[p], H, L, ring[p]);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            float x16[16];
            scaled16(v, ring[k % D], L, x16);
            const uint32_t m = wave_max_u32(absmax_bits_f(x16, 16));
            if (lane == 0)
                s_pmax[w * KMAX + k] = m;
            if (k + D < KMAX)
                scale_row_parts(a.qs, ek[k + D], H, L, ring[k % D]);
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            uint32_t m = 0;
            for (int j = w0; j < w0 + rw; ++j)  // the token's waves
                m = max(m, s_pmax[j * KMAX + k]);
            amax[k] = __uint_as_float(m);
        }
    }

#pragma unroll
    for (int p = 0; p < D; ++p)
        scale_row_parts(a.qs, ek[p], H, L, ring[p]);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        float x16[16];
        scaled16(v, ring[k % D], L, x16);
        if (k + D < KMAX)
            scale_row_parts(a.qs, ek[k + D], H, L, ring[k % D]);
        const uint32_t row = rank[k] >= 0 ? (uint32_t)rank[k] : 0u;
        const uint32_t base = rank[k] >= 0 ? row * o.row_bytes : kNoRow;
        const uint32_t p0 = L.v0 ? (uint32_t)L.e0 : kNoPart, p1 = L.v1 ? (uint32_t)L.e1 : kNoPart;
        uint2 c0, c1;
        if (MODE == 1) {
            c0 = int8_static_codes8(x16);
            c1 = int8_static_codes8(x16 + 8);
        } else if (MODE == 2) {
            const float m = amax[k];
            const float d = m != 0.0f ? 127.0f / m : 0.0f;
            c0 = int8_codes8(x16, d);
            c1 = int8_codes8(x16 + 8, d);
            if (tr == 0 && rank[k] >= 0)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(m != 0.0f ? 1.0f / d : 0.0f), o.sc, row * 4u, 0, kPlain);
        } else {  // MODE == 3
            const int tile = a.tile;
            uint32_t m0 = absmax_bits_f(x16, 8), m1 = absmax_bits_f(x16 + 8, 8);
            if (tile >= kWaveElems) {
                m0 = m1 = wave_max_u32(max(m0, m1));
            } else {
                m0 = tile_max(m0, tile / kPartElems);
                m1 = tile_max(m1, tile / kPartElems);
            }
            const float mf0 = __uint_as_float(m0), mf1 = __uint_as_float(m1);
            const float d0 = m0 ? 127.0f / mf0 : 0.0f, d1 = m1 ? 127.0f / mf1 : 0.0f;
            c0 = int8_codes8(x16, d0);
            c1 = int8_codes8(x16 + 8, d1);
            if (rank[k] >= 0) {
                store_tile_scale(o, row, tile, lane, L.e0, L.v0, 0, m0 ? 1.0f / d0 : 0.0f);
                store_tile_scale(o, row, tile, lane, L.e1, L.v1, 1, m1 ? 1.0f / d1 : 0.0f);
            }
        }
        buf_store8<kDevice>(o.x, base + p0, c0.x, c0.y);
        buf_store8<kDevice>(o.x, base + p1, c1.x, c1.y);
    }
}

// A token's coded parts (this lane's 8 + 8 elements) and their scales.
struct Coded {
    uint2 c0, c1;  // modes 1-4: codes of part 0 and part 1
    float f0, f1;  // mode 2: the token's 1 / dynamicScales (f0); mode 3: each part's tile's
    int se0, se1;  // mode 4: each part's block exponent
};

// Codes a token's row once (this lane's parts in xa, xb; zeros past the row
// end); no memory writes, so it can run before the rows are known.  amax_row
// is the token's largest |x| pattern (per-token int8 only).
template <int MODE>
__device__ __forceinline__ Coded code_row(const DispatchArgs &a, const Lane &L, const uint4 &xa,
                                          const uint4 &xb, uint32_t amax_row)
{
    Coded c{};
    if (MODE == 0)
        return c;
    float v[16];
    unpack8(xa, v);
    unpack8(xb, v + 8);
    if (MODE == 1) {  // static: one coefficient or one row shared by all experts
        float sv[16];
        if (a.qs_kind == 2) {
            float4 s[4];
            scale_row_parts(a.qs, 0, a.H, L, s);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                sv[4 * q] = s[q].x;
                sv[4 * q + 1] = s[q].y;
                sv[4 * q + 2] = s[q].z;
                sv[4 * q + 3] = s[q].w;
            }
        } else {
            const float cst = a.qs[0];
#pragma unroll
            for (int j = 0; j < 16; ++j)
                sv[j] = cst;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] *= sv[j];
        c.c0 = int8_static_codes8(v);
        c.c1 = int8_static_codes8(v + 8);
    } else if (MODE == 2) {
        const uint32_t m = amax_row;
        const float mf = __uint_as_float(m << 16);
        const float d = m ? 127.0f / mf : 0.0f;
        c.f0 = m ? 1.0f / d : 0.0f;
        c.c0 = int8_codes8(v, d);
        c.c1 = int8_codes8(v + 8, d);
    } else if (MODE == 3) {
        const int tile = a.tile;
        uint32_t m0 = amax_bits8(xa), m1 = amax_bits8(xb);
        if (tile >= kWaveElems) {
            m0 = m1 = wave_max_u32(max(m0, m1));
        } else {
            m0 = tile_max(m0, tile / kPartElems);
            m1 = tile_max(m1, tile / kPartElems);
        }
        const float mf0 = __uint_as_float(m0 << 16), mf1 = __uint_as_float(m1 << 16);
        const float d0 = m0 ? 127.0f / mf0 : 0.0f, d1 = m1 ? 127.0f / mf1 : 0.0f;
        c.f0 = m0 ? 1.0f / d0 : 0.0f;
        c.f1 = m1 ? 1.0f / d1 : 0.0f;
        c.c0 = int8_codes8(v, d0);
        c.c1 = int8_codes8(v + 8, d1);
    } else {  // MODE == 4: blocks of 32 are 4 lanes of one part
        const uint32_t m0 = tile_max(amax_bits8(xa), 4), m1 = tile_max(amax_bits8(xb), 4);
        c.se0 = mx_exponent(m0);
        c.se1 = mx_exponent(m1);
        const float f0 = __uint_as_float((uint32_t)(127 - c.se0) << 23);  // 2^-se, normal
        const float f1 = __uint_as_float((uint32_t)(127 - c.se1) << 23);
        c.c0 = e4m3_codes8(v, f0);
        c.c1 = e4m3_codes8(v + 8, f1);
    }
    return c;
}

// Writes the coded parts (mode 0: the raw bf16 parts), with their scales, to
// each destination row rank[k] >= 0.
template <int MODE, int KMAX>
__device__ __forceinline__ void store_row(const DispatchArgs &a, int tr, const Lane &L,
                                          const uint4 &xa, const uint4 &xb, const Coded &c,
                                          const int *rank)
{
    if (!L.v0 && !L.v1)
        return;  // a wave past the row end
    const Out o = out_buffers(a, MODE);
    const int lane = tr & (kWave - 1);
    const int elt = MODE == 0 ? 2 : 1;
    const uint32_t p0 = L.v0 ? (uint32_t)(L.e0 * elt) : kNoPart;
    const uint32_t p1 = L.v1 ? (uint32_t)(L.e1 * elt) : kNoPart;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (rank[k] < 0)
            continue;
        const uint32_t row = (uint32_t)rank[k];
        const uint32_t base = row * o.row_bytes;
        if (MODE == 0) {
            buf_store16<kDevice>(o.x, base + p0, xa);
            buf_store16<kDevice>(o.x, base + p1, xb);
            continue;
        }
        buf_store8<kDevice>(o.x, base + p0, c.c0.x, c.c0.y);
        buf_store8<kDevice>(o.x, base + p1, c.c1.x, c.c1.y);
        if (MODE == 2 && tr == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(c.f0), o.sc, row * 4u, 0,
                                                  kPlain);
        if (MODE == 3) {
            store_tile_scale(o, row, a.tile, lane, L.e0, L.v0, 0, c.f0);
            store_tile_scale(o, row, a.tile, lane, L.e1, L.v1, 1, c.f1);
        }
        if (MODE == 4 && (lane & 3) == 0) {
            if (L.v0)
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(c.se0 + 127), o.sc,
                                                     row * o.sc_row + (uint32_t)(L.e0 / 32), 0,
                                                     kPlain);
            if (L.v1)
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(c.se1 + 127), o.sc,
                                                     row * o.sc_row + (uint32_t)(L.e1 / 32), 0,
                                                     kPlain);
        }
    }
}

// Destination row of this lane's entry (lanes k < K hold entry k of the
// token, id my_id >= 0 if active; other lanes -1) from the packed histograms
// (low 16 bits: active entries of each instance; high 16 bits: those before
// this token).  Every wave works the rows out on its own, so no barrier
// follows: lane c sums the low halves of counters [c*per, (c+1)*per) (per a
// multiple of 4 with 64 * per >= E, read as 16-byte words), a DPP scan gives
// each chunk's exclusive prefix, and lane k adds its chunk's prefix (one lane
// shuffle), the low halves before its id in the chunk, the high half of its
// own counter and the token's earlier entries with the same id.
template <int KMAX>
__device__ __forceinline__ int entry_row(const int *s_cnt, int E, int K, int lane, int my_id)
{
    const int per = ((E + kWave - 1) / kWave + 3) & ~3;  // 4, 8, 12 or 16
    const int q = per >> 2;
    const int4 *c4 = reinterpret_cast<const int4 *>(s_cnt);
    const bool on = my_id >= 0;
    const int id = on ? my_id : 0;
    const int chunk = small_div(id, per);
    const int within = id - chunk * per;
    int local = 0, part = 0, high = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < q) {
            const int4 v = c4[lane * q + j];
            const int4 u = c4[chunk * q + j];
            local += (v.x & 0xffff) + (v.y & 0xffff) + (v.z & 0xffff) + (v.w & 0xffff);
            const int uv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                part += 4 * j + b < within ? (uv[b] & 0xffff) : 0;
                high += 4 * j + b == within ? (uv[b] >> 16) : 0;
            }
        }
    }
    const int excl = wave_incl_scan(local) - local;
    const int off = __shfl(excl, chunk);
    int dup = 0;  // earlier entries of this token with the same id
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        const int v = j < K ? __builtin_amdgcn_readlane(my_id, j) : -1;
        dup += (j < lane && v == my_id) ? 1 : 0;
    }
    return on ? off + part + high + dup : -1;
}

template <int MODE, int KMAX, typename Src, bool PE>
__device__ __forceinline__ void dispatch_body(const DispatchArgs &a)
{
    // low 16 bits: active entries with id e; high: those before this block's
    // tokens
    __shared__ __align__(16) int s_cnt[kHistSlots];
    __shared__ int s_wave[kDispatchWaves];
    __shared__ uint32_t s_wmax[kDispatchWaves];
    __shared__ uint32_t s_pmax[PE && MODE == 2 ? kDispatchWaves * KMAX : 1];
    __shared__ uint8_t s_tok[Src::kMapped ? kMaxTokens : 1];
    __shared__ __align__(16) float s_thr[Src::kMapped ? kMaxTopK : 1];
    extern __shared__ int s_tab[];  // mapped: the [n_logical, F] table
    constexpr int kTPB = tokens_per_block<PE>();

    const int Bs = a.Bs, H = a.H, K = a.K, E = a.E;
    const int N = Bs * K;
    Src s;
    if constexpr (Src::kMapped)
        s = Src{a.ids, a.scores ? a.scores : reinterpret_cast<const float *>(a.ids), s_tab,
                s_tok, s_thr, a.n_logical, a.F, E, K, (unsigned)(((1 << 17) + K - 1) / K)};
    else
        s = Routed{a.ids, a.mask, E};
    if (blockIdx.x == 0) {
        route_summary(a, s, s_cnt, s_wave, s_tab, s_tok, s_thr);
        return;
    }
    // Block 1 + b holds tokens kTPB * b + j, one row of waves each
    // (rw waves per row); lanes below KB = kTPB * K carry the
    // block's entries g0 + lane in order.
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const int rw = kTPB == 1 ? nw : nw / kTPB;
    const int tk = kTPB == 1 ? 0 : w / rw;  // this wave's token in the block (wave-uniform)
    const int i = (blockIdx.x - 1) * kTPB + tk;
    const int tr = t - tk * rw * kWave;  // thread index in the token's row
    const Lane L = lane_parts(tr, H);
    const rsrc_t r_x = buffer_rsrc(a.x, (uint32_t)Bs * H * 2);
    const int KB = kTPB * K;
    const int g0 = (blockIdx.x - 1) * KB;

    // 1. the block's own entries, one per lane: the first loads issued are
    //    the first ones waited for (after the rare large-table staging)
    if (Src::kMapped)
        Stage<Src::kKeep>::rest(a, s_tab, s_tok);
    const bool mine = lane < KB && g0 + lane < N;
    const int gm = min(g0 + min(lane, KB - 1), N - 1);
    const int raw_id = a.ids[gm];
    const uint8_t *mp =
        !Src::kMapped && a.mask ? a.mask : reinterpret_cast<const uint8_t *>(a.ids);
    const uint8_t raw_on = Src::kMapped ? 1 : mp[gm];
    const float *sp = Src::kMapped && a.scores ? a.scores : reinterpret_cast<const float *>(a.ids);
    const float raw_sc = Src::kMapped ? sp[gm] : 0.0f;
    for (int e = t; e < kHistSlots; e += T)  // entry_row reads whole 16-byte groups
        s_cnt[e] = 0;

    // 2. the packed histograms.  The tokens' rows (two 8-element parts per
    //    lane) are loaded after the first batch of ids, so they stay in flight
    //    meanwhile.
    uint4 xa, xb;
    int err = 0;
    for_each_entry(
        s, N, err,
        [&](int inst, bool on, int g) {
            if (on)
                atomicAdd(&s_cnt[inst], g < g0 ? kPreOne : 1);
        },
        [&] {
            // mapped source: the staging loads go out with the first ids and
            // before the token's row, so that storing them waits for neither
            // (issued earlier, the compiler would wait for them before the ids)
            Stage<Src::kKeep> st;
            if (Src::kMapped)
                st.issue(a);
            const uint32_t tok = i < Bs ? (uint32_t)i * H * 2 : kNoRow;
            xa = buf_load16<kPlain>(r_x, tok + (L.v0 ? (uint32_t)L.e0 * 2 : kNoPart));
            xb = buf_load16<kPlain>(r_x, tok + (L.v1 ? (uint32_t)L.e1 * 2 : kNoPart));
            if (Src::kMapped)
                st.store(a, s_tab, s_tok, s_thr);
            lds_barrier();  // histograms zeroed (and mapping data staged) before use
        });
    int my_id;
    if constexpr (Src::kMapped) {
        bool on;
        int e2 = 0;  // block 0 reports the errors
        const int ie = s.token_of(gm);
        const int inst = s.map(raw_id, ie, gm - ie * K, raw_sc, true, on, e2);
        if (w == 0 && mine) {  // the update-expert outputs of the block's entries
            if (a.balanced_ids)
                a.balanced_ids[g0 + lane] = inst;
            if (a.balanced_mask)
                a.balanced_mask[g0 + lane] = on ? 1 : 0;
        }
        my_id = mine && on ? inst : -1;
    } else {
        const bool my_on =
            mine && (a.mask == nullptr || raw_on != 0) && (unsigned)raw_id < (unsigned)E;
        my_id = my_on ? raw_id : -1;
    }
    // After the histogram barrier each wave works out the block's rows itself
    // (entry_row) and codes its parts, then stores: no further barrier.
    // Per-token int8 publishes its wave maxima before the barrier.
    Coded cd{};
    if (MODE == 2 && !PE) {
        const uint32_t m = wave_max_u32(max(amax_bits8(xa), amax_bits8(xb)));
        if (lane == 0)
            s_wmax[w] = m;
    }
    lds_barrier();  // histograms complete

    // 3. rows of the block's entries (lane j = entry g0 + j), in every wave,
    //    before the coding: their LDS reads then overlap the row's HBM load
    const int my_row = entry_row<KMAX * kTPB>(s_cnt, E, KB, lane, my_id);
    if (!PE && MODE != 2)
        cd = code_row<MODE>(a, L, xa, xb, 0u);
    if (!PE && MODE == 2) {
        uint32_t amax = 0;
        for (int j = tk * rw; j < (tk + 1) * rw; ++j)  // the token's waves
            amax = max(amax, s_wmax[j]);
        cd = code_row<MODE>(a, L, xa, xb, amax);
    }
    if (w == 0 && mine) {
        a.assist_dst[g0 + lane] = my_row;
        if (my_row >= 0)
            a.expand_src[my_row] = g0 + lane;
    }
    int rank[KMAX];  // rows of this wave's token's entries
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        rank[k] = k < K ? __builtin_amdgcn_readlane(my_row, tk * K + k) : -1;

    if constexpr (PE) {
        int eid[KMAX];  // instance of each copy
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            eid[k] = k < K ? __builtin_amdgcn_readlane(my_id, tk * K + k) : -1;
        code_store_rows<MODE, KMAX>(a, tr, w, tk * rw, rw, L, xa, xb, rank, eid, s_pmax);
    } else {
        store_row<MODE, KMAX>(a, tr, L, xa, xb, cd, rank);
    }
}

// routed entries (moe_dispatch); PE: one scales row per instance
template <int MODE, int KMAX, bool PE>
__global__ __launch_bounds__(kMaxThreads * tokens_per_block<PE>()) void k_dispatch(DispatchArgs a)
{
    dispatch_body<MODE, KMAX, Routed, PE>(a);
}

// mapped entries (moe_update_dispatch); KEEP: a token mask or thresholds
template <int MODE, int KMAX, bool KEEP, bool PE>
__global__ __launch_bounds__(kMaxThreads * tokens_per_block<PE>()) void k_update_dispatch(DispatchArgs a)
{
    dispatch_body<MODE, KMAX, Mapped<KEEP>, PE>(a);
}

template <int MODE, int KMAX, typename Src, bool PE>
void launch_kernel(const DispatchArgs &a, hipStream_t stream)
{
    constexpr int kTPB = tokens_per_block<PE>();
    const dim3 grid(1 + (a.Bs + kTPB - 1) / kTPB), block(row_threads(a.H) * kTPB);
    if constexpr (Src::kMapped)
        hipLaunchKernelGGL((k_update_dispatch<MODE, KMAX, Src::kKeep, PE>), grid, block,
                           (size_t)a.n_logical * a.F * sizeof(int), stream, a);
    else
        hipLaunchKernelGGL((k_dispatch<MODE, KMAX, PE>), grid, block, 0, stream, a);
}

template <int MODE, typename Src, bool PE>
hipError_t launch_dispatch_mode(const DispatchArgs &a, hipStream_t stream)
{
    switch (a.K <= 2 ? 2 : a.K <= 4 ? 4 : a.K <= 8 ? 8 : 16) {
    case 2: launch_kernel<MODE, 2, Src, PE>(a, stream); break;
    case 4: launch_kernel<MODE, 4, Src, PE>(a, stream); break;
    case 8: launch_kernel<MODE, 8, Src, PE>(a, stream); break;
    default: launch_kernel<MODE, 16, Src, PE>(a, stream); break;
    }
    return hipGetLastError();
}

// Sources of entries: 0 routed (moe_dispatch), 1 mapped without a keep test,
// 2 mapped with a token mask or thresholds (moe_update_dispatch).
enum SrcKind { kRouted = 0, kMappedPlain = 1, kMappedKeep = 2 };

// The launcher of one quantisation mode for every source and scales layout
// (pe: one scales row per instance; only modes 1-3 take it).
template <int MODE>
hipError_t launch_mode(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    if constexpr (MODE >= 1 && MODE <= 3) {
        if (pe) {
            switch (src) {
            case kRouted: return launch_dispatch_mode<MODE, Routed, true>(a, stream);
            case kMappedPlain: return launch_dispatch_mode<MODE, Mapped<false>, true>(a, stream);
            default: return launch_dispatch_mode<MODE, Mapped<true>, true>(a, stream);
            }
        }
    }
    switch (src) {
    case kRouted: return launch_dispatch_mode<MODE, Routed, false>(a, stream);
    case kMappedPlain: return launch_dispatch_mode<MODE, Mapped<false>, false>(a, stream);
    default: return launch_dispatch_mode<MODE, Mapped<true>, false>(a, stream);
    }
}

hipError_t launch_mode0(const DispatchArgs &a, int src, bool pe, hipStream_t stream);
hipError_t launch_mode1(const DispatchArgs &a, int src, bool pe, hipStream_t stream);
hipError_t launch_mode2(const DispatchArgs &a, int src, bool pe, hipStream_t stream);
hipError_t launch_mode3(const DispatchArgs &a, int src, bool pe, hipStream_t stream);
hipError_t launch_mode4(const DispatchArgs &a, int src, bool pe, hipStream_t stream);

}  // namespace moe
