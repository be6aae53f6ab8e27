// calib.hip -- measurement kernels of libmoe_calib.so (include/moe_calib.h):
// byte movers in the access shapes of the dispatch and combine kernels, with
// none of their arithmetic, and streams with their read/write mixes.  They
// set the ceilings the method's kernels are measured against.
#include <stddef.h>
#include <stdint.h>

#include "device.h"
#include "kernels.h"
#include "moe_calib.h"

namespace moe {
namespace {

constexpr int kStreamThreads = 256;
constexpr uint32_t kStreamChunk = kStreamThreads * 16;  // bytes one pass of a block moves
constexpr int kChunksPerBlock = 4;
constexpr int kMaxReads = 8;                      // read chunks a block takes at most

// Block b reads chunks [b*CR/nb, (b+1)*CR/nb) of src and writes chunks
// [b*CW/nb, (b+1)*CW/nb) of dst: every block moves reads and writes in the
// whole kernel's proportion, so the two interleave over time.
template <int SP>
__global__ __launch_bounds__(kStreamThreads) void k_stream(const void *src, uint32_t rbytes,
                                                           void *dst, uint32_t wbytes,
                                                           uint32_t cr, uint32_t cw)
{
    const uint32_t nb = gridDim.x, b = blockIdx.x, t = threadIdx.x;
    const uint32_t r0 = (uint32_t)((uint64_t)b * cr / nb), r1 = (uint32_t)((uint64_t)(b + 1) * cr / nb);
    const uint32_t w0 = (uint32_t)((uint64_t)b * cw / nb), w1 = (uint32_t)((uint64_t)(b + 1) * cw / nb);
    const rsrc_t rs = buffer_rsrc(src, rbytes), rd = buffer_rsrc(dst, wbytes);
    uint4 v[kMaxReads];
#pragma unroll
    for (int j = 0; j < kMaxReads; ++j)
        v[j] = buf_load16<kStream>(rs, r0 + j < r1 ? (r0 + j) * kStreamChunk + t * 16 : kNoRow);
    uint4 acc = make_uint4(t, b, 0, 0);
#pragma unroll
    for (int j = 0; j < kMaxReads; ++j) {
        acc.x ^= v[j].x;
        acc.y ^= v[j].y;
        acc.z ^= v[j].z;
        acc.w ^= v[j].w;
    }
    for (uint32_t c = w0; c < w1; ++c)
        buf_store16<SP>(rd, c * kStreamChunk + t * 16, make_uint4(acc.x ^ c, acc.y, acc.z, acc.w));
    // a block with no chunk to write still needs its loads: a store the data
    // decides (practically never taken) keeps them from being dropped
    if (w0 == w1 && acc.x == 0x9e3779b9u && acc.y == acc.z)
        buf_store16<SP>(rd, t * 16, acc);
}

// high byte of each of the 8 bf16 in a
__device__ __forceinline__ uint2 high_bytes(const uint4 &a)
{
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    uint32_t o[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
        o[q] = ((w[2 * q] >> 8) & 0xffu) | ((w[2 * q] >> 16) & 0xff00u) |
               ((w[2 * q + 1] << 8) & 0xff0000u) | (w[2 * q + 1] & 0xff000000u);
    return make_uint2(o[0], o[1]);
}

template <int SP>
__global__ __launch_bounds__(kMaxThreads) void k_scatter_shape(const uint16_t *x,
                                                               const int32_t *assist, int Bs,
                                                               int H, int K, int n_rows,
                                                               uint8_t *out)
{
    const int i = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1);
    int my = assist[i * K + min(lane, K - 1)];
    if (lane >= K || my >= n_rows)
        my = -1;
    const int e0 = part_elem(t, 0), e1 = part_elem(t, 1);
    const uint32_t p0 = e0 < H ? (uint32_t)e0 : kNoPart, p1 = e1 < H ? (uint32_t)e1 : kNoPart;
    const rsrc_t rx = buffer_rsrc(x, (uint32_t)Bs * H * 2);
    const rsrc_t ro = buffer_rsrc(out, (uint32_t)n_rows * H);
    const uint32_t tok = (uint32_t)i * H * 2;
    const uint2 c0 = high_bytes(buf_load16<kPlain>(rx, tok + 2 * p0));
    const uint2 c1 = high_bytes(buf_load16<kPlain>(rx, tok + 2 * p1));
    for (int k = 0; k < K; ++k) {
        const int r = __builtin_amdgcn_readlane(my, k);
        if (r < 0)
            continue;
        const uint32_t base = (uint32_t)r * H;
        buf_store8<SP>(ro, base + p0, c0.x, c0.y);
        buf_store8<SP>(ro, base + p1, c1.x, c1.y);
    }
}

__device__ __forceinline__ void add_words(uint4 &acc, const uint4 &v)
{
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
}

constexpr int kGroup = 8;

template <int SP>
__global__ __launch_bounds__(kMaxThreads) void k_gather_shape(
    const uint16_t *rows, const int32_t *assist, const uint16_t *a, const uint16_t *b,
    const uint16_t *gamma, int Bs, int H, int K, int n_rows, uint16_t *out1, uint16_t *out2)
{
    __shared__ uint32_t s_part[kMaxWaves];
    const int i = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int nw = row_threads(H) / kWave;
    int my = assist[i * K + min(lane, K - 1)];
    if (lane >= K || my >= n_rows)
        my = -1;
    const uint32_t rowb = (uint32_t)H * 2;
    const int e0 = part_elem(t, 0), e1 = part_elem(t, 1);
    const uint32_t o0 = e0 < H ? (uint32_t)e0 * 2 : kNoPart, o1 = e1 < H ? (uint32_t)e1 * 2 : kNoPart;
    const rsrc_t rr = buffer_rsrc(rows, (uint32_t)n_rows * rowb);
    const rsrc_t ra = buffer_rsrc(a, (uint32_t)Bs * rowb);
    const rsrc_t rb = buffer_rsrc(b ? b : a, b ? (uint32_t)Bs * rowb : 0u);  // no b: reads zeros
    const rsrc_t rg = buffer_rsrc(gamma, rowb);
    const uint32_t tok = (uint32_t)i * rowb;
    uint4 s0 = buf_load16<kPlain>(ra, tok + o0), s1 = buf_load16<kPlain>(ra, tok + o1);
    add_words(s0, buf_load16<kPlain>(rb, tok + o0));
    add_words(s1, buf_load16<kPlain>(rb, tok + o1));
    const uint4 g0 = buf_load16<kPlain>(rg, o0), g1 = buf_load16<kPlain>(rg, o1);
    uint64_t live = __ballot(my >= 0);
    while (live) {
        uint4 v0[kGroup], v1[kGroup];
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            uint32_t base = kNoRow;
            if (live) {
                const int k = __builtin_ctzll(live);
                live &= live - 1;
                base = (uint32_t)__builtin_amdgcn_readlane(my, k) * rowb;
            }
            v0[j] = buf_load16<kStream>(rr, base + o0);
            v1[j] = buf_load16<kStream>(rr, base + o1);
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            add_words(s0, v0[j]);
            add_words(s1, v1[j]);
        }
    }
    const rsrc_t r1 = buffer_rsrc(out1, (uint32_t)Bs * rowb), r2 = buffer_rsrc(out2, (uint32_t)Bs * rowb);
    buf_store16<SP>(r1, tok + o0, s0);
    buf_store16<SP>(r1, tok + o1, s1);
    const uint32_t part = wave_max_u32(s0.x ^ s1.y);
    if (lane == 0)
        s_part[w] = part;
    lds_barrier();
    uint32_t m = 0;
    for (int j = 0; j < nw; ++j)
        m ^= s_part[j];
    add_words(s0, g0);
    add_words(s1, g1);
    s0.x ^= m;
    buf_store16<SP>(r2, tok + o0, s0);
    buf_store16<SP>(r2, tok + o1, s1);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool bad_shape(int Bs, int H, int K, int n_rows)
{
    return Bs <= 0 || Bs > 512 || H < 1024 || H > 8192 || H % 32 != 0 || K <= 0 || K > 16 ||
           n_rows <= 0 || n_rows > Bs * K;
}

int status(hipError_t e) { return e == hipSuccess ? MOE_CALIB_OK : MOE_CALIB_ELAUNCH; }

bool bad_policy(int p) { return p < MOE_CALIB_STORE_PLAIN || p > MOE_CALIB_STORE_DEVICE; }

// a kernel template's instance for a store policy
template <template <int> class F, typename... A>
hipError_t by_policy(int policy, A... args)
{
    switch (policy) {
    case MOE_CALIB_STORE_PLAIN: return F<kPlain>::run(args...);
    case MOE_CALIB_STORE_STREAM: return F<kStream>::run(args...);
    default: return F<kDevice>::run(args...);
    }
}

template <int SP> struct StreamK {
    static hipError_t run(dim3 g, hipStream_t st, const void *src, uint32_t rb, void *dst,
                          uint32_t wb, uint32_t cr, uint32_t cw)
    {
        hipLaunchKernelGGL(k_stream<SP>, g, dim3(kStreamThreads), 0, st, src, rb, dst, wb, cr, cw);
        return hipGetLastError();
    }
};
template <int SP> struct ScatterK {
    static hipError_t run(dim3 g, dim3 b, hipStream_t st, const uint16_t *x, const int32_t *assist,
                          int Bs, int H, int K, int n_rows, uint8_t *out)
    {
        hipLaunchKernelGGL(k_scatter_shape<SP>, g, b, 0, st, x, assist, Bs, H, K, n_rows, out);
        return hipGetLastError();
    }
};
template <int SP> struct GatherK {
    static hipError_t run(dim3 g, dim3 b, hipStream_t st, const uint16_t *rows,
                          const int32_t *assist, const uint16_t *a, const uint16_t *bb,
                          const uint16_t *gamma, int Bs, int H, int K, int n_rows, uint16_t *o1,
                          uint16_t *o2)
    {
        hipLaunchKernelGGL(k_gather_shape<SP>, g, b, 0, st, rows, assist, a, bb, gamma, Bs, H, K,
                           n_rows, o1, o2);
        return hipGetLastError();
    }
};

}  // namespace
}  // namespace moe

extern "C" {

int moe_calib_stream(const void *src, size_t read_bytes, void *dst, size_t write_bytes,
                     int store_policy, void *stream)
{
    using namespace moe;
    const size_t lim = (size_t)1 << 31;
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || read_bytes % 16 ||
        write_bytes % 16 || read_bytes > lim || write_bytes > lim ||
        read_bytes + write_bytes == 0 || bad_policy(store_policy))
        return MOE_CALIB_EINVAL;
    const uint32_t cr = (uint32_t)((read_bytes + kStreamChunk - 1) / kStreamChunk);
    const uint32_t cw = (uint32_t)((write_bytes + kStreamChunk - 1) / kStreamChunk);
    uint32_t nb = (cr + cw + kChunksPerBlock - 1) / kChunksPerBlock;
    // at most kMaxReads read chunks per block
    nb = nb > (cr + kMaxReads - 1) / kMaxReads ? nb : (cr + kMaxReads - 1) / kMaxReads;
    return status(by_policy<StreamK>(store_policy, dim3(nb), static_cast<hipStream_t>(stream),
                                     src, (uint32_t)read_bytes, dst, (uint32_t)write_bytes, cr,
                                     cw));
}

int moe_calib_scatter_shape(const void *x, const int32_t *assist, int Bs, int H, int K,
                            int n_rows, void *out, int store_policy, void *stream)
{
    using namespace moe;
    if (!x || !assist || !out || !aligned16(x) || !aligned16(out) ||
        bad_shape(Bs, H, K, n_rows) || bad_policy(store_policy))
        return MOE_CALIB_EINVAL;
    return status(by_policy<ScatterK>(store_policy, dim3(Bs), dim3(row_threads(H)),
                                      static_cast<hipStream_t>(stream),
                                      static_cast<const uint16_t *>(x), assist, Bs, H, K, n_rows,
                                      static_cast<uint8_t *>(out)));
}

int moe_calib_gather_shape(const void *rows, const int32_t *assist, const void *a,
                           const void *b, const void *gamma, int Bs, int H, int K, int n_rows,
                           void *out1, void *out2, int store_policy, void *stream)
{
    using namespace moe;
    if (!rows || !assist || !a || !gamma || !out1 || !out2 || !aligned16(rows) ||
        !aligned16(a) || (b && !aligned16(b)) || !aligned16(gamma) || !aligned16(out1) ||
        !aligned16(out2) || bad_shape(Bs, H, K, n_rows) || bad_policy(store_policy))
        return MOE_CALIB_EINVAL;
    return status(by_policy<GatherK>(store_policy, dim3(Bs), dim3(row_threads(H)),
                                     static_cast<hipStream_t>(stream),
                                     static_cast<const uint16_t *>(rows), assist,
                                     static_cast<const uint16_t *>(a),
                                     static_cast<const uint16_t *>(b),
                                     static_cast<const uint16_t *>(gamma), Bs, H, K, n_rows,
                                     static_cast<uint16_t *>(out1), static_cast<uint16_t *>(out2)));
}

}  // extern "C"
