// expert_gemm.hip -- the expert computation between dispatch and combine: a
// grouped GEMM over the dispatch output, one weight matrix per instance, on
// the gfx950 block-scaled MFMA (mxfp8 x mxfp8 -> fp32 -> bf16).
//
// Rows offsets[e] .. offsets[e+1]-1 of the expandX buffer belong to instance
// e (the instance-major order of "aclnnMoeDistributeDispatchV2"); each is
// multiplied by W[e] ([N, K], one row per output column), both operands
// dequantised per block of 32 along K as E4M3 value x 2^(E8M0 code - 127) --
// the mxfp8 expandX / dynamicScales layout of that page's case 5.
//
// Tiling.  A block computes a 128 x 128 output tile (128 rows of one
// instance x 128 output columns) with four waves of 64 x 64 each.  K is
// walked 128 at a time; both operand tiles (16 KB each) and their scale bytes
// go through registers into a double-buffered LDS stage, so the global loads
// of step s+1 are in flight while the MFMAs of step s run, with one LDS
// barrier per step.  Each 128-byte LDS row keeps its eight 16-byte chunks in
// XOR-swizzled order (chunk c at c ^ (row & 7)) so that the fragment reads of
// sixteen consecutive rows spread over the banks.
//
// MFMA operand layout (v_mfma_scale_f32_16x16x128_f8f6f4, measured): lane l
// holds 32 K-bytes of row l % 16 of its operand: bytes 0-15 are K offsets
// 16 * (l / 16) .. +15 and bytes 16-31 are K offsets 64 + 16 * (l / 16) .. +15;
// its scale byte covers row l % 16, K block l / 16 (32 elements).  The
// result lane l, slot i is D[4 * (l / 16) + i][l % 16].  The weight tile is
// the first operand and the activation tile the second, so D is the
// transposed output tile and each lane ends with four consecutive output
// columns of one row: one 8-byte bf16 store.
//
// Scheduling.  Each instance needs ceil(rows_e / 128) row tiles; a block
// prefix-sums those counts into LDS once and then walks the flattened
// (column tile, row tile) space grid-stride, row tiles fastest so that the
// blocks working on one weight tile run together.  Consecutive block ids are
// spread over the eight XCDs round-robin by the hardware, so the block id is
// remapped to give each XCD (and its L2) a contiguous range of tiles.
#include <stdint.h>

#include <algorithm>

#include "device.h"
#include "kernels.h"
#include "moe_expert.h"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per tile
constexpr int kBN = 128;        // output columns per tile
constexpr int kBK = 128;        // K elements (bytes) per step
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;
constexpr int kMaxInstances = 1024;
constexpr int kGemmGrid = 1024;  // grid-stride cap (a multiple of the XCD count)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint8_t *a;        // [rows, K] E4M3
    const uint8_t *a_sc;     // [rows, K/32] E8M0
    const int32_t *offsets;  // [E+1]
    const uint8_t *w;        // [E, N, K] E4M3
    const uint8_t *w_sc;     // [E, N, K/32] E8M0
    uint16_t *y;             // [rows, N] bf16
    int32_t *dev_err;
    int E, rows, N, K;
};

struct Stage {
    uint8_t x[kBM * kBK];
    uint8_t w[kBN * kBK];
    uint32_t sc[kBM + kBN];  // the step's four scale bytes of each row: activations, weights
};

// Clamped row range of instance e: [lo, hi) within [0, rows); *bad is set
// when the offsets are not non-decreasing within [0, rows].
__device__ __forceinline__ void instance_rows(const GemmArgs &p, int e, int &lo, int &hi,
                                              bool *bad)
{
    const int o0 = p.offsets[e], o1 = p.offsets[e + 1];
    lo = min(max(o0, 0), p.rows);
    hi = min(max(o1, lo), p.rows);
    if (bad)
        *bad = o0 < 0 || o1 < o0 || o1 > p.rows;
}

__global__ __launch_bounds__(kGemmThreads, 2) void k_expert_gemm_mx(GemmArgs p)
{
    __shared__ __align__(16) Stage s_stage[2];
    __shared__ int s_tiles[kMaxInstances + 1];  // exclusive prefix of row tiles per instance
    __shared__ int s_wave_sum[kGemmThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // ---- row tiles per instance, prefix-summed (thread t owns instances 4t .. 4t+3)
    int c[4], tsum = 0;
    bool bad_any = false;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        c[q] = 0;
        if (e < p.E) {
            int lo, hi;
            bool bad;
            instance_rows(p, e, lo, hi, &bad);
            bad_any |= bad;
            c[q] = (hi - lo + kBM - 1) / kBM;
        }
        tsum += c[q];
    }
    if (bad_any && blockIdx.x == 0 && p.dev_err)
        atomicOr(p.dev_err, MOE_ERR_OFFSETS);
    const int incl = wave_incl_scan(tsum);
    if (lane == kWave - 1)
        s_wave_sum[wave] = incl;
    lds_barrier();
    int excl = incl - tsum;
    for (int w = 0; w < wave; ++w)
        excl += s_wave_sum[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        if (e < p.E)
            s_tiles[e] = excl;
        if (e == p.E - 1)
            s_tiles[p.E] = excl + c[q];
        excl += c[q];
    }
    lds_barrier();
    const int m_tiles = s_tiles[p.E];
    const int n_tiles = p.N / kBN;
    const int total = m_tiles * n_tiles;

    // ---- XCD-grouped virtual block id
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int v = (G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;

    const int nk = p.K / kBK;
    const int kb = p.K / 32;                  // scale bytes per row
    const int g = lane >> 4;                  // lane group: K chunk / scale block
    const int r16 = lane & 15;
    const int wn = wave & 1, wm = wave >> 1;  // wave's 64 x 64 quadrant (columns, rows)

    // global -> register staging: thread owns 16-byte chunk (tid & 7) of rows (tid >> 3) + 32 j
    const int ld_chunk = tid & 7;
    const int ld_row = tid >> 3;
    const int sw_chunk = (ld_chunk ^ (ld_row & 7)) << 4;  // swizzled LDS byte offset in the row

    for (int t = v; t < total; t += G) {
        const int tm = t % m_tiles;
        const int tn = t / m_tiles;
        // instance of row tile tm: the last e with s_tiles[e] <= tm
        int lo_e = 0, hi_e = p.E;
        while (hi_e - lo_e > 1) {
            const int mid = (lo_e + hi_e) >> 1;
            if (s_tiles[mid] <= tm)
                lo_e = mid;
            else
                hi_e = mid;
        }
        const int e = lo_e;
        int row_lo, row_hi;
        instance_rows(p, e, row_lo, row_hi, nullptr);
        const int m0 = row_lo + (tm - s_tiles[e]) * kBM;   // first row of the tile
        const int n0 = tn * kBN;

        // per-thread global sources for the step (rows past the instance are clamped to its
        // last row: loaded, multiplied, never stored)
        const uint8_t *xsrc[4];
        const uint8_t *wsrc[4];
        const uint8_t *w_e = p.w + (size_t)e * p.N * p.K;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = min(m0 + ld_row + 32 * j, row_hi - 1);
            xsrc[j] = p.a + (size_t)r * p.K + ld_chunk * 16;
            wsrc[j] = w_e + (size_t)(n0 + ld_row + 32 * j) * p.K + ld_chunk * 16;
        }
        const uint8_t *scsrc;
        if (tid < kBM)
            scsrc = p.a_sc + (size_t)min(m0 + tid, row_hi - 1) * kb;
        else
            scsrc = p.w_sc + ((size_t)e * p.N + n0 + (tid - kBM)) * kb;

        u32x4 rx[4], rw[4];
        uint32_t rsc;
#define MOE_GEMM_LOAD_STEP(s_)                                                             \
    do {                                                                                   \
        const int k0_ = (s_) * kBK;                                                        \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                      \
        {                                                                                  \
            rx[j] = *reinterpret_cast<const u32x4 *>(xsrc[j] + k0_);                       \
            rw[j] = *reinterpret_cast<const u32x4 *>(wsrc[j] + k0_);                       \
        }                                                                                  \
        rsc = *reinterpret_cast<const uint32_t *>(scsrc + k0_ / 32);                       \
    } while (0)
#define MOE_GEMM_STORE_STEP(st_)                                                           \
    do {                                                                                   \
        _Pragma("unroll") for (int j = 0; j < 4; ++j)                                      \
        {                                                                                  \
            const int row_ = ld_row + 32 * j;                                              \
            *reinterpret_cast<u32x4 *>(&(st_).x[row_ * kBK + sw_chunk]) = rx[j];           \
            *reinterpret_cast<u32x4 *>(&(st_).w[row_ * kBK + sw_chunk]) = rw[j];           \
        }                                                                                  \
        (st_).sc[tid] = rsc;                                                               \
    } while (0)

        v4f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

        MOE_GEMM_LOAD_STEP(0);
        MOE_GEMM_STORE_STEP(s_stage[0]);
        lds_barrier();

        const int fr_c0 = ((g ^ (r16 & 7)) << 4);   // swizzled offsets of chunks g and g + 4
        const int fr_c1 = (((g + 4) ^ (r16 & 7)) << 4);
        for (int s = 0; s < nk; ++s) {
            // prefetch the next step (the last step reloads itself: no branch in the body,
            // which would let the compiler sink the MFMAs below the stores)
            const int s_next = min(s + 1, nk - 1);
            MOE_GEMM_LOAD_STEP(s_next);
            __builtin_amdgcn_sched_barrier(0);   // issue the loads before the MFMAs
            const Stage &st = s_stage[s & 1];
            v8i xf[4];
            int xs[4];
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) {
                const int row = wm * 64 + fm * 16 + r16;
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c0]);
                const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c1]);
                xf[fm] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                xs[fm] = (int)((st.sc[row] >> (8 * g)) & 0xffu);
            }
#pragma unroll
            for (int fn = 0; fn < 4; ++fn) {
                const int row = wn * 64 + fn * 16 + r16;
                const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c0]);
                const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c1]);
                const v8i wf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                const int ws = (int)((st.sc[kBM + row] >> (8 * g)) & 0xffu);
#pragma unroll
                for (int fm = 0; fm < 4; ++fm)
                    acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf, xf[fm], acc[fn][fm], 0, 0, 0, ws, 0, xs[fm]);
            }
            // keep the next stage's LDS stores (which wait for this step's global loads)
            // behind the MFMAs, so the load latency hides under them
            __builtin_amdgcn_sched_barrier(0);
            MOE_GEMM_STORE_STEP(s_stage[(s + 1) & 1]);
            lds_barrier();
        }

#undef MOE_GEMM_LOAD_STEP
#undef MOE_GEMM_STORE_STEP

        // ---- epilogue: lane holds columns n0 + wn*64 + fn*16 + 4g .. +3 of row m0 + wm*64 + fm*16 + r16
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
            const int r = m0 + wm * 64 + fm * 16 + r16;
            if (r < row_hi) {
                uint16_t *yrow = p.y + (size_t)r * p.N + n0 + wn * 64 + 4 * g;
#pragma unroll
                for (int fn = 0; fn < 4; ++fn) {
                    const v4f d = acc[fn][fm];
                    const uint2 o = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
                    *reinterpret_cast<uint2 *>(yrow + fn * 16) = o;
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_expert_gemm_mx(const uint8_t *a, const uint8_t *a_sc, const int32_t *offsets,
                                 int E, int rows, const uint8_t *w, const uint8_t *w_sc, int N,
                                 int K, uint16_t *y, int32_t *dev_err, hipStream_t stream)
{
    GemmArgs p{a, a_sc, offsets, w, w_sc, y, dev_err, E, rows, N, K};
    // Upper bound on row tiles: sum of ceil(rows_e / 128) <= ceil(rows / 128) + E.
    const long m_cap = (rows + kBM - 1) / kBM + E;
    const long tiles_cap = m_cap * (N / kBN);
    const int grid = (int)std::min<long>(tiles_cap, kGemmGrid);
    hipLaunchKernelGGL(k_expert_gemm_mx, dim3(grid), dim3(kGemmThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace moe
