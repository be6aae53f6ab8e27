// combine.hip -- weighted gather of expert outputs + shared expert + residual,
// fused with RMSNorm ("aclnnMoeDistributeCombineAddRmsNorm", 计算公式:
// combineOut = Sum(expertScales*ataOut + expertScales*sharedExpertX),
// x = combineOut + residualX, y = x / RMS(x) * gamma with
// RMS(x) = sqrt(mean(x^2) + normEps)).
//
// One block per token, one thread per 16 elements of the row: every input
// row is read once with 16-byte loads, the fp32 sum stays in registers, the
// sum of squares is a wave butterfly plus one LDS step, and y / x_out are
// written once.  The kernel is bound by HBM bandwidth: per token it moves
// (n_dispatched + 2 or 3) rows in and 2 rows out.
//
// Every wave reads the token's K (row, weight) pairs itself, one per lane,
// and broadcasts them with readlane, so the only block barrier is the one of
// the sum of squares.  Row loads are issued back to back, CH rows at a time,
// with no loads for entries that were not dispatched.
#include "device.h"
#include "kernels.h"

namespace moe {

template <int CH>
__global__ __launch_bounds__(kMaxThreads) void k_combine(
    const uint16_t *__restrict__ eo, const int32_t *__restrict__ assist,
    const float *__restrict__ scales, const uint16_t *__restrict__ shared,
    const uint16_t *__restrict__ residual, const uint16_t *__restrict__ gamma, float eps,
    int Bs, int H, int K, int shared_mode, uint16_t *__restrict__ y,
    uint16_t *__restrict__ x_out, float *__restrict__ rstd_out, int32_t *__restrict__ dev_err)
{
    __shared__ float s_part[kMaxWaves];

    const int i = blockIdx.x;
    const int t = threadIdx.x, T = blockDim.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = T / kWave;
    const bool has = t * kChunk < H;
    const size_t rowoff = (size_t)i * H;

    // 1. the token's K entries, one per lane, loaded first: the expert-row
    //    loads depend on them, and wait counters retire in issue order
    //    (all loads here are unconditional -- lanes past K or past the row end
    //    re-read a valid address -- so that waiting for one load never has to
    //    assume a shorter queue on some other path and wait for later ones)
    const int kk = min(lane, K - 1);
    int my_r = assist[i * K + kk];
    float my_s = scales[i * K + kk];
    if (lane >= K)
        my_r = -1;

    // 2. residual, shared and gamma do not depend on the routing
    const int tc = has ? t : 0;
    const uint16_t *shp = shared ? shared : residual;
    const uint4 *pr = reinterpret_cast<const uint4 *>(residual + rowoff) + 2 * tc;
    const uint4 *pg = reinterpret_cast<const uint4 *>(gamma) + 2 * tc;
    const uint4 *ps = reinterpret_cast<const uint4 *>(shp + rowoff) + 2 * tc;
    const uint4 ra = pr[0], rb = pr[1];
    const uint4 ga = pg[0], gb = pg[1];
    const uint4 sa = ps[0], sb = ps[1];

    // 3. the dispatched entries' rows, CH at a time; entries that were not
    //    dispatched (row -1) or point outside the buffer load nothing
    if (my_r >= Bs * K) {
        if (w == 0 && dev_err)
            atomicOr(dev_err, 8);
        my_r = -1;
    }
    const float ws = wave_sum_f32(my_r >= 0 ? my_s : 0.0f);
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        acc[j] = 0.0f;
    // Every one of CH == K entries dispatched (the usual case without pruning): the row
    // loads are unconditional straight-line code, so the compiler counts them and each
    // row's sums start as soon as that row has arrived, overlapping the arithmetic with
    // the later rows' loads (with a branch per row it must wait for all of them first)
    const uint64_t live = __ballot(my_r >= 0);
    if (K == CH && live == (1ull << CH) - 1) {
        uint4 ea[CH], eb[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int r = __builtin_amdgcn_readlane(my_r, j);
            const uint4 *p = reinterpret_cast<const uint4 *>(eo + (size_t)r * H) + 2 * tc;
            ea[j] = load_nt16(p);
            eb[j] = load_nt16(p + 1);
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
            float v[16];
            unpack16(ea[j], eb[j], v);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[e] = fmaf(sk, v[e], acc[e]);
        }
    }
    for (int k0 = 0; k0 < K && !(K == CH && live == (1ull << CH) - 1); k0 += CH) {
        uint4 ea[CH], eb[CH];
        int rr[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            rr[j] = k0 + j < K ? __builtin_amdgcn_readlane(my_r, k0 + j) : -1;
            if (rr[j] >= 0) {
                const uint4 *p = reinterpret_cast<const uint4 *>(eo + (size_t)rr[j] * H) + 2 * tc;
                ea[j] = load_nt16(p);
                eb[j] = load_nt16(p + 1);
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (rr[j] >= 0) {
                const float sk =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k0 + j));
                float v[16];
                unpack16(ea[j], eb[j], v);
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[e] = fmaf(sk, v[e], acc[e]);
            }
        }
    }

    float xf[16];
    {
        float rv[16];
        unpack16(ra, rb, rv);
        if (shared) {
            const float wsh = shared_mode == 0 ? ws : 1.0f;
            float sv[16];
            unpack16(sa, sb, sv);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[e] = fmaf(wsh, sv[e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
            xf[e] = acc[e] + rv[e];
    }

    // lanes past the row end loaded nothing: they add nothing to the sum of squares
    float ss = 0.0f;
    if (has) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ss = fmaf(xf[e], xf[e], ss);
    }
    ss = wave_sum_f32(ss);
    if (lane == 0)
        s_part[w] = ss;

    if (has && x_out) {
        uint4 *p = reinterpret_cast<uint4 *>(x_out + rowoff) + 2 * t;
        p[0] = make_uint4(pack_bf16x2(xf[0], xf[1]), pack_bf16x2(xf[2], xf[3]),
                          pack_bf16x2(xf[4], xf[5]), pack_bf16x2(xf[6], xf[7]));
        p[1] = make_uint4(pack_bf16x2(xf[8], xf[9]), pack_bf16x2(xf[10], xf[11]),
                          pack_bf16x2(xf[12], xf[13]), pack_bf16x2(xf[14], xf[15]));
    }
    lds_barrier();
    float tot = 0.0f;
    for (int j = 0; j < nw; ++j)
        tot += s_part[j];
    const float rstd = 1.0f / __builtin_sqrtf(tot / (float)H + eps);
    if (t == 0 && rstd_out)
        rstd_out[i] = rstd;
    if (!has)
        return;
    float g[16], o[16];
    unpack16(ga, gb, g);
#pragma unroll
    for (int e = 0; e < 16; ++e)
        o[e] = xf[e] * rstd * g[e];
    uint4 *p = reinterpret_cast<uint4 *>(y + rowoff) + 2 * t;
    p[0] = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                      pack_bf16x2(o[6], o[7]));
    p[1] = make_uint4(pack_bf16x2(o[8], o[9]), pack_bf16x2(o[10], o[11]),
                      pack_bf16x2(o[12], o[13]), pack_bf16x2(o[14], o[15]));
}

hipError_t launch_combine(const uint16_t *expert_out, const int32_t *assist,
                          const float *scales, const uint16_t *shared,
                          const uint16_t *residual, const uint16_t *gamma, float eps, int Bs,
                          int H, int K, int shared_mode, uint16_t *y, uint16_t *x_out,
                          float *rstd, int32_t *dev_err, hipStream_t stream)
{
    hipLaunchKernelGGL((k_combine<8>), dim3(Bs), dim3(row_threads(H)), 0, stream, expert_out,
                       assist, scales, shared, residual, gamma, eps, Bs, H, K, shared_mode, y,
                       x_out, rstd, dev_err);
    return hipGetLastError();
}

}  // namespace moe
