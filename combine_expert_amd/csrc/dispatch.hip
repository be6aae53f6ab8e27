// dispatch.hip -- quantise tokens and scatter them expert-major
// ("aclnnMoeDistributeDispatchV2", 计算公式 cases 1, 3, 4 and 5: the rows
// this device sends, laid out [rank][local expert][token] exactly as the
// all-to-all would deliver them).
//
// One launch, Bs + 1 blocks, no inter-block communication:
//   block 0      histogram of the active entries (LDS atomics; counts are
//                order-free), exclusive scan, counts/offsets, -1 for the
//                unused tail of expand_src, and the device error bits;
//   block 1 + i  token i: loads its row once, works out the destination row
//                of each of its K entries, codes the row once and writes it
//                K times.
// The row of entry f with instance id e is offsets[e] plus the number of
// active entries before f with the same id (a stable counting sort).  Each
// token block derives it on its own from LDS histograms of all N = Bs*K
// entries (at most 8192 four-byte ids, read with 16-byte loads from L2): one
// over every entry and one over the entries before its token, packed as the
// low and high 16 bits of one counter (each count is at most 8192), so each
// entry costs one LDS atomic.  An in-place exclusive scan of the low halves
// gives offsets[e]; one lane per entry of the token then adds the high half
// and the token's own earlier duplicates.  This replaces a serial routing
// kernel between two launches with redundant LDS work that overlaps the HBM
// load of the token's row.  (Two tokens per block, sharing the histograms,
// measured slower: one block per compute unit hides less latency than two.)
// Nothing depends on scheduling: bitwise repeatable.
//
// Row layout: one thread owns 16 consecutive elements (two 16-byte loads of
// bf16), so a 32-element mxfp8 block is a lane pair and a 128-element int8
// tile is 8 lanes; per-block maxima are lane shuffles, the per-token maximum
// is a wave reduction plus one LDS step.
//
// Load order matters: wait counters retire in issue order, so the loads a
// phase waits for are issued before the ones it does not (the token's row),
// and loads are unconditional (clamped indices) so that no control-flow join
// makes a wait cover loads issued after it on another path.
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kHistSlots = 1024;  // one LDS counter per instance (E <= 1024)
constexpr int kPreOne = 0x10001;  // packed counter increment: all (low) and before-token (high)

// Where the entries come from: [Bs, K] instance ids and an optional mask.
struct Entries {
    const int32_t *ids;
    const uint8_t *mask;  // null: every entry is active
    int E;
};

// Visits every entry g this thread owns -- int4 groups g4 = t, t + T, ...,
// then the scalar tail -- as f(inst, on, g) with inst = -1 unless on.  Each
// batch issues four 16-byte id loads (and mask words) before using any;
// indices past the end are clamped and visited as inactive.  Ids outside
// [0, E) of active entries raise error bit 1 in err.
// after_first_issue() runs once, right after the first batch is issued:
// loads placed there stay in flight while the batch is consumed.
template <typename Fn, typename G>
__device__ __forceinline__ void for_each_entry(const Entries &s, int N, int &err, Fn &&f,
                                               G &&after_first_issue)
{
    const int t = threadIdx.x, T = blockDim.x;
    const int N4 = N >> 2;
    const int4 *ids4 = reinterpret_cast<const int4 *>(s.ids);
    const uint32_t *mask4 = reinterpret_cast<const uint32_t *>(s.mask);
    bool first = true;
    for (int base = t; base < N4 || first; base += 4 * T) {
        int4 v[4];
        uint32_t m[4];
        if (N4 > 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int g4 = min(base + u * T, N4 - 1);
                v[u] = ids4[g4];
                m[u] = s.mask ? mask4[g4] : 0x01010101u;
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
            const int g = g4 * 4;
            const int idv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            const uint32_t mu = g4 < N4 ? m[u] : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool on = ((mu >> (8 * j)) & 0xffu) != 0;
                const bool ok = (unsigned)idv[j] < (unsigned)s.E;
                if (on && !ok)
                    err |= 1;
                f(on && ok ? idv[j] : -1, on && ok, g + j);
            }
        }
    }
    for (int g = N4 * 4 + t; g < N; g += T) {
        const int id = s.ids[g];
        const bool on = s.mask == nullptr || s.mask[g] != 0;
        const bool ok = (unsigned)id < (unsigned)s.E;
        if (on && !ok)
            err |= 1;
        f(on && ok ? id : -1, on && ok, g);
    }
}

struct DispatchArgs {
    const uint16_t *x;
    const int32_t *ids;
    const uint8_t *mask;
    int Bs, H, K, E, tile;
    void *expand_x, *expand_scales;
    int32_t *counts, *offsets, *expand_src, *assist_dst;
    int32_t *dev_err;
};

// ------------------------------------------------------------------ block 0

__device__ void route_summary(const DispatchArgs &a, const Entries &s, int *s_hist, int *s_wave)
{
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const int N = a.Bs * a.K, E = a.E;
    for (int e = t; e < E; e += T)
        s_hist[e] = 0;
    int err = 0;
    for_each_entry(
        s, N, err,
        [&](int inst, bool on, int) {
            if (on)
                atomicAdd(&s_hist[inst], 1);
        },
        [&] { lds_barrier(); });
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

// int8 codes of 16 values with multiplier d: clamp(rint(v * d), -127, 127).
// d is +inf when 127 / max overflows (a tiny subnormal maximum): zeros then
// give 0 * inf = NaN and are coded 0, the rest saturate.
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

// floor(log2(m)) of a positive bf16 magnitude pattern (normal or subnormal)
__device__ __forceinline__ int bf16_ilogb(uint32_t m)
{
    const int ex = (int)(m >> 7);
    return ex ? ex - 127 : (31 - __clz((int)(m & 0x7f))) - 133;
}

// Codes a token's row once (this thread's 16 elements in xa, xb) and writes it,
// with its scales, to each destination row rank[k] >= 0.  amax_row is the
// token's largest |x| pattern (per-token int8 only).
template <int MODE, int KMAX>
__device__ __forceinline__ void code_store(const DispatchArgs &a, int t, bool has, const uint4 &xa,
                                           const uint4 &xb, const int *rank, uint32_t amax_row)
{
    const int H = a.H;
    if (MODE == 0) {
        if (!has)
            return;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (rank[k] < 0)
                continue;
            uint4 *dst = reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.expand_x) +
                                                   (size_t)rank[k] * H) + 2 * t;
            store_nt16(dst, xa);
            store_nt16(dst + 1, xb);
        }
        return;
    }

    float v[16];
    unpack16(xa, xb, v);
    uint4 code;
    if (MODE == 2) {
        const uint32_t m = amax_row;
        const float mf = __uint_as_float(m << 16);
        const float d = m ? 127.0f / mf : 0.0f;
        const float scale = m ? 1.0f / d : 0.0f;
        code = int8_codes(v, d);
        if (has) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (rank[k] < 0)
                    continue;
                store_nt16(reinterpret_cast<uint4 *>(static_cast<int8_t *>(a.expand_x) +
                                                     (size_t)rank[k] * H) + t, code);
                if (t == 0)
                    static_cast<float *>(a.expand_scales)[rank[k]] = scale;
            }
        }
    } else if (MODE == 3) {
        const int tile = a.tile;
        const int lanes = tile / kChunk;  // lanes per tile: 1 .. 64
        // lanes past the row end hold a copy of chunk 0: keep it out of the
        // last (partial) tile's maximum
        uint32_t m = has ? amax_bits16(xa, xb) : 0u;
        for (int o = 1; o < lanes; o <<= 1)
            m = max(m, (uint32_t)__shfl_xor((int)m, o));
        const float mf = __uint_as_float(m << 16);
        const float d = m ? 127.0f / mf : 0.0f;
        const float scale = m ? 1.0f / d : 0.0f;
        code = int8_codes(v, d);
        const int nt = (H + tile - 1) / tile;
        const bool lead = has && (t & (lanes - 1)) == 0;
        if (has) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (rank[k] < 0)
                    continue;
                store_nt16(reinterpret_cast<uint4 *>(static_cast<int8_t *>(a.expand_x) +
                                                     (size_t)rank[k] * H) + t, code);
                if (lead)
                    static_cast<float *>(a.expand_scales)[(size_t)rank[k] * nt +
                                                          (t * kChunk) / tile] = scale;
            }
        }
    } else {  // MODE == 4
        uint32_t m = amax_bits16(xa, xb);
        m = max(m, (uint32_t)__shfl_xor((int)m, 1));
        int se = -127;
        if (m) {
            se = bf16_ilogb(m) - 8;
            se = max(-127, min(127, se));
        }
        const float f = __uint_as_float((uint32_t)(127 - se) << 23);  // 2^-se, normal
        code = e4m3_codes(v, f);
        const int nb = H / 32;
        const bool lead = has && (t & 1) == 0;
        if (has) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (rank[k] < 0)
                    continue;
                store_nt16(reinterpret_cast<uint4 *>(static_cast<uint8_t *>(a.expand_x) +
                                                     (size_t)rank[k] * H) + t, code);
                if (lead)
                    static_cast<uint8_t *>(a.expand_scales)[(size_t)rank[k] * nb + t / 2] =
                        (uint8_t)(se + 127);
            }
        }
    }
}

// Exclusive scan of the low 16 bits of s[0, n) in place by the whole block,
// keeping the high 16 bits (s_wave: one int per wave).  Each thread owns a
// contiguous run of counters.  Ends with a barrier.
__device__ void block_exclusive_scan_lo16(int *s, int n, int *s_wave)
{
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const int per = (n + T - 1) / T;
    const int e0 = min(t * per, n), e1 = min(e0 + per, n);
    int local = 0;
    for (int e = e0; e < e1; ++e)
        local += s[e] & 0xffff;
    const int incl = wave_incl_scan(local);
    if (lane == kWave - 1)
        s_wave[w] = incl;
    lds_barrier();
    int run = incl - local;
    for (int j = 0; j < nw; ++j)
        run += j < w ? s_wave[j] : 0;
    for (int e = e0; e < e1; ++e) {
        const int c = s[e];
        s[e] = run | (c & ~0xffff);
        run += c & 0xffff;
    }
    lds_barrier();
}

template <int MODE, int KMAX>
__global__ __launch_bounds__(kMaxThreads) void k_dispatch(DispatchArgs a)
{
    // low 16 bits: active entries with id e; high: those before this token.
    // After the scan the low half holds offsets[e].
    __shared__ int s_cnt[kHistSlots];
    __shared__ int s_wave[kMaxWaves];
    __shared__ int s_rank[KMAX];
    __shared__ uint32_t s_wmax[kMaxWaves];

    const int Bs = a.Bs, H = a.H, K = a.K, E = a.E;
    const int N = Bs * K;
    const Entries s{a.ids, a.mask, E};
    if (blockIdx.x == 0) {
        route_summary(a, s, s_cnt, s_wave);
        return;
    }
    const int i = blockIdx.x - 1;
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const bool has = t * kChunk < H;

    // 1. the token's own K entries, one per lane: the first loads issued are
    //    the first ones waited for
    const int f0 = i * K;
    const int kk = min(lane, K - 1);
    const int raw_id = a.ids[f0 + kk];
    const uint8_t *mp = a.mask ? a.mask : reinterpret_cast<const uint8_t *>(a.ids);
    const uint8_t raw_on = mp[f0 + kk];
    for (int e = t; e < E; e += T)
        s_cnt[e] = 0;

    // 2. the packed histograms.  The token's row (16 elements per thread) is
    //    loaded after the first batch of ids, so it stays in flight meanwhile.
    uint4 xa, xb;
    int err = 0;
    for_each_entry(
        s, N, err,
        [&](int inst, bool on, int g) {
            if (on)
                atomicAdd(&s_cnt[inst], g < f0 ? kPreOne : 1);
        },
        [&] {
            const uint4 *src =
                reinterpret_cast<const uint4 *>(a.x + (size_t)i * H) + 2 * (has ? t : 0);
            xa = src[0];
            xb = src[1];
            lds_barrier();  // histograms zeroed before the first increment
        });
    const bool my_on =
        lane < K && (a.mask == nullptr || raw_on != 0) && (unsigned)raw_id < (unsigned)E;
    const int my_id = my_on ? raw_id : -1;
    lds_barrier();
    block_exclusive_scan_lo16(s_cnt, E, s_wave);

    // 3. rows of the token's entries (wave 0, lane k = entry k)
    if (w == 0) {
        int dup = 0;  // earlier entries of this token with the same id
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int v = j < K ? __builtin_amdgcn_readlane(my_id, j) : -1;
            dup += (j < lane && v == my_id) ? 1 : 0;
        }
        if (lane < K) {
            const int c = my_on ? s_cnt[my_id] : 0;
            const int r = my_on ? (c & 0xffff) + (c >> 16) + dup : -1;
            s_rank[lane] = r;
            a.assist_dst[f0 + lane] = r;
            if (r >= 0)
                a.expand_src[r] = f0 + lane;
        }
    }
    if (MODE == 2) {  // per-token maximum: wave maxima, then across the waves
        const uint32_t m = wave_max_u32(amax_bits16(xa, xb));
        if (lane == 0)
            s_wmax[w] = m;
    }
    lds_barrier();
    uint32_t amax = 0;
    if (MODE == 2) {
        for (int j = 0; j < nw; ++j)
            amax = max(amax, s_wmax[j]);
    }
    int rank[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
        rank[k] = k < K ? s_rank[k] : -1;

    code_store<MODE, KMAX>(a, t, has, xa, xb, rank, amax);
}

template <int MODE>
static hipError_t launch_dispatch_mode(int kmax, const DispatchArgs &a, hipStream_t stream)
{
    const dim3 grid(a.Bs + 1), block(row_threads(a.H));
    switch (kmax) {
    case 2: hipLaunchKernelGGL((k_dispatch<MODE, 2>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((k_dispatch<MODE, 4>), grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((k_dispatch<MODE, 8>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((k_dispatch<MODE, 16>), grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_dispatch(const uint16_t *x, const int32_t *ids, const uint8_t *mask, int Bs,
                           int H, int K, int E, int quant_mode, int tile, void *expand_x,
                           void *expand_scales, int32_t *counts, int32_t *offsets,
                           int32_t *expand_src, int32_t *assist_dst, int32_t *dev_err,
                           hipStream_t stream)
{
    const DispatchArgs a{x, ids, mask, Bs, H, K, E, tile, expand_x, expand_scales,
                         counts, offsets, expand_src, assist_dst, dev_err};
    const int kmax = K <= 2 ? 2 : K <= 4 ? 4 : K <= 8 ? 8 : 16;
    switch (quant_mode) {
    case 0: return launch_dispatch_mode<0>(kmax, a, stream);
    case 2: return launch_dispatch_mode<2>(kmax, a, stream);
    case 3: return launch_dispatch_mode<3>(kmax, a, stream);
    default: return launch_dispatch_mode<4>(kmax, a, stream);
    }
}

}  // namespace moe
