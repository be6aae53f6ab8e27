// dispatch_impl.h -- the dispatch kernels (see dispatch.hip for the design),
// shared by the translation units that instantiate them, one per quantisation
// mode (dispatch_m0.hip .. dispatch_m4.hip), so that they compile in parallel.
#pragma once

#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kChunk = 16;        // row elements owned by one thread (16 consecutive)

constexpr int kHistSlots = 1024;  // one LDS counter per instance (E <= 1024)
constexpr int kDispatchWaves = kMaxWaves + 1;
constexpr int kPreOne = 0x10001;  // packed counter increment: all (low) and before-token (high)
constexpr int kMaxTokens = 512;   // Bs limit: staged token mask
constexpr int kMaxTopK = 16;      // K limit: staged thresholds

constexpr int kStageTab = 4;      // mapping-table words per thread staged through registers
constexpr int kStageTok = 4;      // token-mask bytes per thread staged through registers

// Above this many entries the routed dispatch loads the token's row after its id loop
// rather than right after the first id batch.  Measured on MI355X, inputs cold: with
// 8192 entries (Bs=512, K=16; 40 KB of ids and mask per block) the early row load held
// the ids back (10.14 against 10.48 us), with 4096 it is the late one that costs (Bs=512,
// K=8: 9.10 against 8.73 us; fused 11.38 against 10.16, so the mapped source keeps it early).
constexpr int kLateRowEntries = 4096;

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

// Routed: instance ids, an optional [Bs, K] mask and an optional [Bs] token
// mask (staged in LDS; an entry is active only if both allow it).  Ids
// outside [0, E) of active entries raise bit 1.
struct Routed {
    static constexpr bool kMapped = false;
    static constexpr bool kKeep = false;
    using Side = uint32_t;
    const int32_t *ids;
    const uint8_t *mask;  // null: every entry is active
    const uint8_t *tok;   // LDS [Bs], or null: every token is active
    int E, K;
    unsigned mK;          // ceil(2^17 / K): g / K = (g * mK) >> 17 for g < 8192

    __device__ int token_of(int g) const { return (int)(__umul24((unsigned)g, mK) >> 17); }
    __device__ Side side4(int g4) const
    {
        return mask ? reinterpret_cast<const uint32_t *>(mask)[g4] : 0x01010101u;
    }
    // the four entries of group g4 as f(inst, on, g, inst)
    template <typename Fn>
    __device__ void group(const int4 &v, Side m, int g4, bool in, int &err, Fn &&f) const
    {
        const int idv[4] = {v.x, v.y, v.z, v.w};
        if (tok) {  // clear the mask bytes of entries whose token is off
            const int g0 = in ? g4 * 4 : 0;
            uint32_t keep = 0;
            if ((K & 3) == 0) {
                keep = tok[token_of(g0)] ? 0xffffffffu : 0u;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    keep |= tok[token_of(g0 + j)] ? 0xffu << (8 * j) : 0u;
            }
            m &= keep;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool act = in && ((m >> (8 * j)) & 0xffu) != 0;
            const bool ok = (unsigned)idv[j] < (unsigned)E;
            err |= act && !ok ? 1 : 0;
            const bool on = act && ok;
            f(on ? idv[j] : -1, on, g4 * 4 + j, on ? idv[j] : -1);
        }
    }
    __device__ int entry1(int g, bool &on, int &err) const
    {
        const int id = ids[g];
        const bool act = (mask == nullptr || mask[g] != 0) && (tok == nullptr || tok[g / K] != 0);
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
    // LDS reads are in flight together, then visited as f(inst, on, g, mapped)
    // (mapped: the instance looked up, -1 if the lookup failed, whether or
    // not the entry is kept).
    // (Entry by entry, the LDS reads would queue behind the previous
    // counter update.)
    template <typename Fn>
    __device__ void group(const int4 &v, Side sc, int g4, bool in, int &err, Fn &&f) const
    {
        // a group past the end shares its first indices with the scalar tail's
        // entries when N % 4 != 0: it visits nothing, since the token blocks'
        // visitor also records the token's own entries and their outputs
        if (!in)
            return;
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
            f(on ? inst[j] : -1, on, g4 * 4 + j, fail ? -1 : inst[j]);
        }
    }
    __device__ int entry1(int g, bool &on, int &err) const
    {
        const int i = token_of(g);
        return map(ids[g], i, g - i * K, KEEP ? scores[g] : 0.0f, true, on, err);
    }
};

// Visits every entry g this thread owns -- int4 groups g4 = t, t + T, ...,
// then the scalar tail -- as f(inst, on, g, mapped) with inst = -1 unless on
// (mapped: the source's instance before the keep test, -1 if none).  Each
// batch issues four 16-byte id loads (and side words) before using any;
// indices past the end are clamped and visited as inactive.
// after_first_issue() runs once, right after the first batch is issued:
// loads placed there stay in flight while the batch is consumed.
template <typename Src, typename Fn, typename G>
__device__ __forceinline__ void for_each_entry(const Src &s, int N, int T, int &err, Fn &&f,
                                               G &&after_first_issue)
{
    const int t = threadIdx.x;
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
        const int m = s.entry1(g, on, err);
        f(on ? m : -1, on, g, m);
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
    int static_e4m3;             // mode 1: E4M3 codes in place of int8 (one coefficient)
    void *expand_x, *expand_scales;
    // mxfp8 exponent b of row r sits at byte r * sc_row + (b / 16) * sc_group + b % 16:
    // row-major (H / 32, 16) or group-major (16, 16 * Bs * K)
    int sc_row, sc_group;
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
        const int t = threadIdx.x, T = dispatch_threads(a.H);
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
        const int t = threadIdx.x, T = dispatch_threads(a.H);
        const int tabsz = a.n_logical * a.F;
#pragma unroll
        for (int u = 0; u < kStageTab; ++u) {
            asm volatile("" : "+v"(tabv[u]));
            const int j = min(t + u * T, tabsz - 1);
            // the clamped copies past the end would all write the last word: they skip
            // the store (measured: fused dispatch at Bs=512, K=8, 256 x 2 table, 10.07
            // against 10.17 us)
            if (u == 0 || t + u * T < tabsz)
                s_tab[j] = staged_table_word(tabv[u], j - a.F * small_div(j, a.F), a.F, a.E);
        }
        if (!KEEP)
            return;
#pragma unroll
        for (int u = 0; u < kStageTok; ++u)
            if (u == 0 || t + u * T < a.Bs)
                s_tok[min(t + u * T, a.Bs - 1)] = a.token_mask ? tokv[u] : 1;
        if (t < a.K)
            s_thr[t] = a.thr ? thrv : -__builtin_inff();
    }

    static __device__ __forceinline__ void rest(const DispatchArgs &a, int *s_tab,
                                                uint8_t *s_tok)
    {
        const int t = threadIdx.x, T = dispatch_threads(a.H);
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
    const int t = threadIdx.x, T = dispatch_threads(a.H);
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const int N = a.Bs * a.K, E = a.E;
    if (Src::kMapped)
        Stage<Src::kKeep>::rest(a, s_tab, s_tok);
    for (int e = t; e < E; e += T)
        s_hist[e] = 0;
    int err = 0;
    for_each_entry(
        s, N, T, err,
        [&](int inst, bool on, int, int) {
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
    if (Src::kKeep || (!Src::kMapped && a.token_mask)) {  // a 1-D token mask is all true, then all false
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

__device__ __forceinline__ uint32_t pack_i8x4(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)d << 24);
}

// int8 codes of 16 values with multiplier d: clamp(rint(v * d), -127, 127),
// NaN products coded 0.  d is +inf when 127 / max overflows (a tiny subnormal
// maximum): zeros then give 0 * inf = NaN and are coded 0, the rest saturate.
// d is 0 when the maximum is infinite: every value then codes 0 (an infinity
// through inf * 0 = NaN).  NaN inputs code 0; the maxima skip them.
__device__ __forceinline__ uint4 int8_codes(const float *v, float d)
{
    int q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float r = __builtin_rintf(v[j] * d);
        r = r != r ? 0.0f : r;
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q[j] = (int)r;
    }
    return make_uint4(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]),
                      pack_i8x4(q[8], q[9], q[10], q[11]), pack_i8x4(q[12], q[13], q[14], q[15]));
}

// E4M3 codes of 16 values multiplied by the power of two f (an exact product):
// clamp to +-448 (saturation), then the gfx950 packed conversion, which
// rounds to nearest even and keeps the sign of zero.
__device__ __forceinline__ uint4 e4m3_codes(const float *v, float f)
{
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float a = fminf(fmaxf(v[4 * q] * f, -448.0f), 448.0f);
        const float b = fminf(fmaxf(v[4 * q + 1] * f, -448.0f), 448.0f);
        const float c = fminf(fmaxf(v[4 * q + 2] * f, -448.0f), 448.0f);
        const float d = fminf(fmaxf(v[4 * q + 3] * f, -448.0f), 448.0f);
        int p = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
        p = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, p, true);
        w[q] = (uint32_t)p;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// The E4M3 NaN code (sign of the input, all other bits set) in place of the
// code of each NaN among the 16 bf16 inputs: the clamp in e4m3_codes has
// turned a NaN into -448.
__device__ __forceinline__ uint4 e4m3_nan_codes(uint4 code, const uint4 &xa, const uint4 &xb)
{
    const uint32_t w[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    uint32_t c[4] = {code.x, code.y, code.z, code.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        if ((h & 0x7fffu) > 0x7f80u) {
            const int sh = 8 * (e & 3);
            c[e >> 2] = (c[e >> 2] & ~(0xffu << sh)) | ((((h >> 8) & 0x80u) | 0x7fu) << sh);
        }
    }
    return make_uint4(c[0], c[1], c[2], c[3]);
}

// floor(log2(m)) of a positive bf16 magnitude pattern (normal or subnormal)
__device__ __forceinline__ int bf16_ilogb(uint32_t m)
{
    const int ex = (int)(m >> 7);
    return ex ? ex - 127 : (31 - __clz((int)(m & 0x7f))) - 133;
}

// E4M3 codes of 16 fp32 values for the static mode's second output type: the
// saturating conversion of e4m3_codes, then the NaN code 0x7F in place of each
// NaN value (a NaN in x, or an infinity times a zero coefficient), whose sign
// is not kept: the sign of such a product is not the same on every processor.
__device__ __forceinline__ uint4 e4m3_static_codes(const float *v)
{
    uint4 code = e4m3_codes(v, 1.0f);
    uint32_t c[4] = {code.x, code.y, code.z, code.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        if (v[e] != v[e]) {
            const int sh = 8 * (e & 3);
            c[e >> 2] = (c[e >> 2] & ~(0xffu << sh)) | (0x7fu << sh);
        }
    }
    return make_uint4(c[0], c[1], c[2], c[3]);
}

// int8 codes of 16 fp32 values for the static mode: the nearest integer, ties
// to even, saturated to [-128, 127]; NaN codes to 0.
__device__ __forceinline__ uint4 int8_static_codes(const float *v)
{
    int q[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        float r = __builtin_rintf(v[j]);
        r = r != r ? 0.0f : r;
        r = fminf(fmaxf(r, -128.0f), 127.0f);
        q[j] = (int)r;
    }
    return make_uint4(pack_i8x4(q[0], q[1], q[2], q[3]), pack_i8x4(q[4], q[5], q[6], q[7]),
                      pack_i8x4(q[8], q[9], q[10], q[11]), pack_i8x4(q[12], q[13], q[14], q[15]));
}

// this thread's 16 values of scales row e ([E, H]); lanes past the row end
// (tc = 0) read the row's first chunk
__device__ __forceinline__ void scale_row16(const float *qs, int e, int H, int tc, float4 (&s)[4])
{
    const float4 *p = reinterpret_cast<const float4 *>(qs + (size_t)e * H) + 4 * tc;
    s[0] = p[0];
    s[1] = p[1];
    s[2] = p[2];
    s[3] = p[3];
}

__device__ __forceinline__ void scaled16(const float *v, const float4 (&s)[4], float *w)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        w[4 * q] = v[4 * q] * s[q].x;
        w[4 * q + 1] = v[4 * q + 1] * s[q].y;
        w[4 * q + 2] = v[4 * q + 2] * s[q].z;
        w[4 * q + 3] = v[4 * q + 3] * s[q].w;
    }
}

__device__ __forceinline__ uint32_t absmax_bits16(const float *w)
{
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        m = fmaxf(m, fabsf(w[j]));
    return __float_as_uint(m);  // non-negative floats order like their bit patterns
}

// One scales row per instance (the scales input of shape [E, H]): every copy
// k of the token is quantised on its own from xFp32 = x * row(eid[k]).  Rows
// are prefetched kPrefetch copies ahead (they come from L2 or the Infinity
// Cache: the table is E * H * 4 bytes).  Per-token dynamic int8 needs each
// copy's maximum over the whole row first: a pass computes all K maxima
// (one barrier for all of them), a second pass codes.  s_pmax: LDS
// [kDispatchWaves][KMAX].
constexpr int kPrefetch = 4;

template <int MODE, int KMAX>
__device__ __forceinline__ void code_store_rows(const DispatchArgs &a, int t, bool has,
                                                const uint4 &xa, const uint4 &xb,
                                                const int *rank, const int *eid,
                                                uint32_t *s_pmax)
{
    constexpr int D = KMAX < kPrefetch ? KMAX : kPrefetch;
    const int H = a.H;
    const int tc = has ? t : 0;
    const int lane = t & (kWave - 1), w = t / kWave, nw = dispatch_threads(a.H) / kWave;
    float v[16];
    unpack16(xa, xb, v);
    int ek[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        ek[k] = rank[k] >= 0 ? eid[k] : 0;  // copies not sent read a valid row, unused
    float4 ring[D][4];

    float amax[KMAX];
    if (MODE == 2) {
#pragma unroll
        for (int p = 0; p < D; ++p)
            scale_row16(a.qs, ek[p], H, tc, ring[p]);
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            float x16[16];
            scaled16(v, ring[k % D], x16);
            const uint32_t m = wave_max_u32(has ? absmax_bits16(x16) : 0u);
            if (lane == 0)
                s_pmax[w * KMAX + k] = m;
            if (k + D < KMAX)
                scale_row16(a.qs, ek[k + D], H, tc, ring[k % D]);
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            uint32_t m = 0;
            for (int j = 0; j < nw; ++j)
                m = max(m, s_pmax[j * KMAX + k]);
            amax[k] = __uint_as_float(m);
        }
    }

#pragma unroll
    for (int p = 0; p < D; ++p)
        scale_row16(a.qs, ek[p], H, tc, ring[p]);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        float x16[16];
        scaled16(v, ring[k % D], x16);
        if (k + D < KMAX)
            scale_row16(a.qs, ek[k + D], H, tc, ring[k % D]);
        const bool put = has && rank[k] >= 0;
        int8_t *dst = static_cast<int8_t *>(a.expand_x) + (size_t)(rank[k] >= 0 ? rank[k] : 0) * H;
        if (MODE == 1) {
            const uint4 code = int8_static_codes(x16);
            if (put)
                store_nt16(reinterpret_cast<uint4 *>(dst) + t, code);
        } else if (MODE == 2) {
            const float m = amax[k];
            const float d = m != 0.0f ? 127.0f / m : 0.0f;
            const uint4 code = int8_codes(x16, d);
            if (put) {
                store_nt16(reinterpret_cast<uint4 *>(dst) + t, code);
                if (t == 0)
                    static_cast<float *>(a.expand_scales)[rank[k]] = m != 0.0f ? 1.0f / d : 0.0f;
            }
        } else {  // MODE == 3
            const int tile = a.tile;
            const int lanes = tile / kChunk;
            uint32_t m = has ? absmax_bits16(x16) : 0u;
            for (int o = 1; o < lanes; o <<= 1)
                m = max(m, (uint32_t)__shfl_xor((int)m, o));
            const float mf = __uint_as_float(m);
            const float d = m ? 127.0f / mf : 0.0f;
            const uint4 code = int8_codes(x16, d);
            if (put) {
                store_nt16(reinterpret_cast<uint4 *>(dst) + t, code);
                if ((t & (lanes - 1)) == 0) {
                    const int nt = (H + tile - 1) / tile;
                    static_cast<float *>(a.expand_scales)[(size_t)rank[k] * nt +
                                                          (t * kChunk) / tile] = m ? 1.0f / d : 0.0f;
                }
            }
        }
    }
}

// A token's coded chunk (this thread's 16 elements) and its scale.
struct Coded {
    uint4 code;    // modes 1-4
    float fscale;  // modes 2 and 3: 1 / dynamicScales of the token / tile
    int se;        // mode 4: the block's shared exponent
};

// Codes a token's row once (this thread's 16 elements in xa, xb); no memory
// writes, so it can run before the rows are known.  amax_row is the token's
// largest |x| pattern (per-token int8 only).
template <int MODE>
__device__ __forceinline__ Coded code_row(const DispatchArgs &a, int t, bool has, const uint4 &xa,
                                          const uint4 &xb, uint32_t amax_row)
{
    Coded c{};
    if (MODE == 0)
        return c;
    float v[16];
    unpack16(xa, xb, v);
    if (MODE == 1) {  // static: one coefficient or one row shared by all experts
        const int tc = has ? t : 0;
        float sv[16];
        if (a.qs_kind == 2) {
            const float4 *p = reinterpret_cast<const float4 *>(a.qs) + 4 * tc;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 f = p[q];
                sv[4 * q] = f.x;
                sv[4 * q + 1] = f.y;
                sv[4 * q + 2] = f.z;
                sv[4 * q + 3] = f.w;
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
        c.code = a.static_e4m3 ? e4m3_static_codes(v) : int8_static_codes(v);
    } else if (MODE == 2) {
        const uint32_t m = amax_row;
        const float mf = __uint_as_float(m << 16);
        const float d = m ? 127.0f / mf : 0.0f;
        c.fscale = m ? 1.0f / d : 0.0f;
        c.code = int8_codes(v, d);
    } else if (MODE == 3) {
        const int lanes = a.tile / kChunk;  // lanes per tile: 1 .. 64
        // lanes past the row end hold a copy of chunk 0: keep it out of the
        // last (partial) tile's maximum
        uint32_t m = has ? amax_bits16(xa, xb) : 0u;
        for (int o = 1; o < lanes; o <<= 1)
            m = max(m, (uint32_t)__shfl_xor((int)m, o));
        const float mf = __uint_as_float(m << 16);
        const float d = m ? 127.0f / mf : 0.0f;
        c.fscale = m ? 1.0f / d : 0.0f;
        c.code = int8_codes(v, d);
    } else {  // MODE == 4
        bool nan;
        uint32_t m = amax_bits16(xa, xb, &nan);
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        int se = -127;
        if (m) {  // an infinite maximum takes the largest exponent, 127
            se = m >= 0x7f80u ? 127 : max(-127, bf16_ilogb(m) - 8);
        }
        // 2^-se is a normal float except at se = 127 (only an infinite
        // maximum gives it): the scaling then takes two exact steps
        float f = __uint_as_float((uint32_t)(127 - se) << 23);
        if (se == 127) {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j] *= 0x1p-64f;
            f = 0x1p-63f;
        }
        c.code = e4m3_codes(v, f);
        if (nan)
            c.code = e4m3_nan_codes(c.code, xa, xb);
        c.se = se;
    }
    return c;
}

// Writes the coded chunk (mode 0: the raw bf16 chunk), with its scales, to
// each destination row rank[k] >= 0.
template <int MODE, int KMAX>
__device__ __forceinline__ void store_row(const DispatchArgs &a, int t, bool has, const uint4 &xa,
                                          const uint4 &xb, const Coded &c, const int *rank)
{
    const int H = a.H;
    if (!has)
        return;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        if (rank[k] < 0)
            continue;
        if (MODE == 0) {
            uint4 *dst = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.expand_x) +
                                                   (size_t)rank[k] * H) + 2 * t;
            store_nt16(dst, xa);
            store_nt16(dst + 1, xb);
            continue;
        }
        store_nt16(reinterpret_cast<uint4 *>(static_cast<int8_t *>(a.expand_x) +
                                             (size_t)rank[k] * H) + t, c.code);
        if (MODE == 2 && t == 0)
            static_cast<float *>(a.expand_scales)[rank[k]] = c.fscale;
        if (MODE == 3) {
            const int lanes = a.tile / kChunk;
            if ((t & (lanes - 1)) == 0) {
                const int nt = (H + a.tile - 1) / a.tile;
                static_cast<float *>(a.expand_scales)[(size_t)rank[k] * nt +
                                                      (t * kChunk) / a.tile] = c.fscale;
            }
        }
        if (MODE == 4 && (t & 1) == 0) {
            const int b = t / 2;
            static_cast<uint8_t *>(a.expand_scales)[(size_t)rank[k] * a.sc_row +
                                                    (size_t)(b >> 4) * a.sc_group + (b & 15)] =
                (uint8_t)(c.se + 127);
        }
    }
}

// LATE: the token's row is loaded after the id loop instead of right after the first id
// batch (routed entries above kLateRowEntries)
template <int MODE, int KMAX, typename Src, bool PE, bool LATE>
__device__ __forceinline__ void dispatch_body(const DispatchArgs &a)
{
    // low 16 bits: active entries with id e; high: those before this token.
    // After the scan the low half holds offsets[e].
    __shared__ __align__(16) int s_cnt[kHistSlots];
    __shared__ int s_wave[kDispatchWaves];
    __shared__ int s_rank[KMAX];
    __shared__ int s_my[KMAX];
    __shared__ uint32_t s_wmax[kDispatchWaves];
    __shared__ uint32_t s_pmax[PE && MODE == 2 ? kDispatchWaves * KMAX : 1];
    __shared__ uint8_t s_tok[kMaxTokens];
    __shared__ __align__(16) float s_thr[Src::kMapped ? kMaxTopK : 1];
    extern __shared__ int s_tab[];  // mapped: the [n_logical, F] table

    const int Bs = a.Bs, H = a.H, K = a.K, E = a.E;
    const int N = Bs * K;
    Src s;
    if constexpr (Src::kMapped)
        s = Src{a.ids, a.scores ? a.scores : reinterpret_cast<const float *>(a.ids), s_tab,
                s_tok, s_thr, a.n_logical, a.F, E, K, (unsigned)(((1 << 17) + K - 1) / K)};
    else
        s = Routed{a.ids, a.mask, a.token_mask ? s_tok : nullptr, E, K,
                   (unsigned)(((1 << 17) + K - 1) / K)};
    if (!Src::kMapped && a.token_mask) {  // staged before the first use (a barrier follows)
        for (int j = threadIdx.x; j < Bs; j += dispatch_threads(H))
            s_tok[j] = a.token_mask[j];
    }
    if (blockIdx.x == 0) {
        route_summary(a, s, s_cnt, s_wave, s_tab, s_tok, s_thr);
        return;
    }
    const int i = blockIdx.x - 1;
    const int t = threadIdx.x, T = dispatch_threads(a.H);
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const bool has = t * kChunk < H;

    // 1. routed source: the token's own K entries, one per lane, are the first
    //    loads issued and the first waited for.  (With the mapping fused in
    //    they are picked up in step 2 instead, already mapped.)  The
    //    histograms of step 2 are zeroed, all of them: the rank wave reads
    //    whole runs.
    if (Src::kMapped)
        Stage<Src::kKeep>::rest(a, s_tab, s_tok);
    const int f0 = i * K;
    int raw_id = -1;
    uint8_t raw_m = 1;
    if constexpr (!Src::kMapped) {  // both loads unconditional: no wait before the ids go out
        const int kk = min(lane, K - 1);
        raw_id = a.ids[f0 + kk];
        const uint8_t *mp = a.mask ? a.mask : reinterpret_cast<const uint8_t *>(a.ids);
        raw_m = mp[f0 + kk];  // without a mask: a byte of the ids, not used
    }
    for (int e = t; e < kHistSlots; e += T)
        s_cnt[e] = 0;

    // 2. the packed histograms.  The token's row (16 elements per thread) is
    //    loaded after the first batch of ids, so it stays in flight meanwhile
    //    (with LATE, after the whole id loop).
    //    With the mapping fused in, the token's own entries are picked up on
    //    the way (s_my: instance or -1) and their update-expert outputs
    //    written there, which saves mapping them again after the loop.
    uint4 xa, xb;
    int err = 0;
    for_each_entry(
        s, N, T, err,
        [&](int inst, bool on, int g, int mapped) {
            if (on)
                atomicAdd(&s_cnt[inst], g < f0 ? kPreOne : 1);
            if constexpr (Src::kMapped) {
                const unsigned k = (unsigned)(g - f0);
                if (k < (unsigned)K) {
                    s_my[k] = inst;
                    if (a.balanced_ids)
                        a.balanced_ids[g] = mapped;
                    if (a.balanced_mask)
                        a.balanced_mask[g] = on ? 1 : 0;
                }
            }
        },
        [&] {
            // mapped source: the staging loads go out with the first ids and
            // before the token's row, so that storing them waits for neither
            // (issued earlier, the compiler would wait for them before the ids)
            Stage<Src::kKeep> st;
            if (Src::kMapped)
                st.issue(a);
            if constexpr (!LATE) {
                const uint4 *src =
                    reinterpret_cast<const uint4 *>(a.x + (size_t)i * H) + 2 * (has ? t : 0);
                xa = src[0];
                xb = src[1];
            }
            if (Src::kMapped)
                st.store(a, s_tab, s_tok, s_thr);
            lds_barrier();  // histograms zeroed (and mapping data staged) before use
        });
    if constexpr (LATE) {
        const uint4 *src =
            reinterpret_cast<const uint4 *>(a.x + (size_t)i * H) + 2 * (has ? t : 0);
        xa = src[0];
        xb = src[1];
    }
    int my_id = -1;  // lane k: entry k's instance, -1 if not dispatched
    if constexpr (!Src::kMapped) {  // the token mask, when given, is staged in LDS
        const bool on = lane < K && (a.mask == nullptr || raw_m != 0) &&
                        (a.token_mask == nullptr || s_tok[i] != 0);
        my_id = on && (unsigned)raw_id < (unsigned)E ? raw_id : -1;
    }
    // Coding needs no ranks: after the histogram barrier the row's waves code
    // their chunks while the block's last wave, which holds no row data (the
    // block has one wave more than the row needs), works out the rows.
    // Per-token int8 publishes its wave maxima before the barrier.
    Coded cd{};
    if (MODE == 2 && !PE) {
        const uint32_t m = wave_max_u32(amax_bits16(xa, xb));
        if (lane == 0)
            s_wmax[w] = m;
    }
    const int rw = nw - 1;  // the rank wave: holds no row data
    lds_barrier();  // histograms complete
    if constexpr (Src::kMapped)
        my_id = lane < K ? s_my[lane < KMAX ? lane : 0] : -1;
    const bool my_on = my_id >= 0;
    if (!PE && MODE != 2 && w != rw)
        cd = code_row<MODE>(a, t, has, xa, xb, 0u);
    if (!PE && MODE == 2 && w != rw) {
        uint32_t amax = 0;
        for (int j = 0; j < nw; ++j)
            amax = max(amax, s_wmax[j]);
        cd = code_row<MODE>(a, t, has, xa, xb, amax);
    }

    // 3. rows of the token's entries (the rank wave, lane k = entry k).  Lane c
    //    owns counters [16c, 16c + 16) (four 16-byte LDS reads; the array is
    //    zeroed to its end): the low halves are prefix-summed in registers and
    //    across the wave, and each counter is rewritten in place with its
    //    exclusive prefix (offsets[e]) plus its high half (the active entries
    //    with that id before this token).  An entry's row is then that word
    //    plus the token's earlier entries with the same id.
    int my_row = -1;
    if (w == rw) {
        // raised issue priority: the row's waves are coding on the same SIMDs
        __builtin_amdgcn_s_setprio(3);
        static_assert(kHistSlots == 16 * kWave, "16 counters per lane");
        int4 *run4 = reinterpret_cast<int4 *>(s_cnt) + 4 * lane;
        int4 c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            c[q] = run4[q];
        int v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[4 * q] = c[q].x;
            v[4 * q + 1] = c[q].y;
            v[4 * q + 2] = c[q].z;
            v[4 * q + 3] = c[q].w;
        }
        int tot = 0, ex[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            ex[j] = tot;
            tot += v[j] & 0xffff;
        }
        const int base = wave_incl_scan(tot) - tot;
#pragma unroll
        for (int j = 0; j < 16; ++j)
            ex[j] += base + (int)((unsigned)v[j] >> 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            run4[q] = make_int4(ex[4 * q], ex[4 * q + 1], ex[4 * q + 2], ex[4 * q + 3]);
        int dup = 0;  // earlier entries of this token with the same id
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int u = j < K ? __builtin_amdgcn_readlane(my_id, j) : -1;
            dup += (j < lane && u == my_id) ? 1 : 0;
        }
        my_row = my_on ? s_cnt[my_id] + dup : -1;
        if (lane < K)
            s_rank[lane] = my_row;
        __builtin_amdgcn_s_setprio(0);
    }
    lds_barrier();  // rows published
    int rank[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        rank[k] = k < K ? s_rank[k] : -1;
    // the routing outputs go out after the barrier: issued before it, they
    // would wait for room in the CU's memory pipeline behind the row stores
    // of other blocks, and hold up the barrier with them
    if (w == rw && lane < K) {
        a.assist_dst[f0 + lane] = my_row;
        if (my_row >= 0)
            a.expand_src[my_row] = f0 + lane;
    }

    if constexpr (PE) {
        int eid[KMAX];  // instance of each copy
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            eid[k] = k < K ? __builtin_amdgcn_readlane(my_id, k) : -1;
        code_store_rows<MODE, KMAX>(a, t, has, xa, xb, rank, eid, s_pmax);
    } else {
        store_row<MODE, KMAX>(a, t, has, xa, xb, cd, rank);
    }
}

// routed entries (moe_dispatch); PE: one scales row per instance; LATE: see dispatch_body
template <int MODE, int KMAX, bool PE, bool LATE>
__global__ __launch_bounds__(kMaxThreads + kWave) void k_dispatch(DispatchArgs a)
{
    dispatch_body<MODE, KMAX, Routed, PE, LATE>(a);
}

// mapped entries (moe_update_dispatch); KEEP: a token mask or thresholds
template <int MODE, int KMAX, bool KEEP, bool PE>
__global__ __launch_bounds__(kMaxThreads + kWave) void k_update_dispatch(DispatchArgs a)
{
    dispatch_body<MODE, KMAX, Mapped<KEEP>, PE, false>(a);
}

template <int MODE, int KMAX, typename Src, bool PE>
void launch_kernel(const DispatchArgs &a, hipStream_t stream)
{
    const dim3 grid(a.Bs + 1), block(dispatch_threads(a.H));
    if constexpr (Src::kMapped) {
        hipLaunchKernelGGL((k_update_dispatch<MODE, KMAX, Src::kKeep, PE>), grid, block,
                           (size_t)a.n_logical * a.F * sizeof(int), stream, a);
    } else if constexpr (KMAX == 16) {  // more than 4096 entries needs K > 8
        if (a.Bs * a.K > kLateRowEntries)
            hipLaunchKernelGGL((k_dispatch<MODE, KMAX, PE, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((k_dispatch<MODE, KMAX, PE, false>), grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL((k_dispatch<MODE, KMAX, PE, false>), grid, block, 0, stream, a);
    }
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
