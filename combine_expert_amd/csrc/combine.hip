// combine.hip -- weighted gather of expert outputs + shared expert + residual,
// fused with RMSNorm ("aclnnMoeDistributeCombineAddRmsNorm", 计算公式:
// combineOut = Sum(expertScales*ataOut + expertScales*sharedExpertX),
// x = combineOut + residualX, y = x / RMS(x) * gamma with
// RMS(x) = sqrt(mean(x^2) + normEps)).
//
// One block per token in the row layout of device.h (a wave per 1024
// elements, two 8-element parts per lane, so every 16-byte access of a wave
// covers one contiguous kilobyte).  Every input row is read once, the fp32
// sum stays in registers, the sum of squares is a wave butterfly plus one LDS
// step, and y / x_out are written once.  The kernel is bound by HBM
// bandwidth: per token it moves (n_dispatched + 2 or 3) rows in and 2 rows
// out.
//
// Every wave reads the token's K (row, weight) pairs itself, one per lane,
// so the only block barrier is the one of the sum of squares.  The
// dispatched entries are taken in order of k into eight register slots:
// straight-line code (a missing entry loads at an offset past the buffer,
// which reads zeros with no memory traffic), so the compiler counts the loads
// and each row's sums start as soon as that row has arrived.  A token with
// more than eight rows refills each slot as soon as its row is summed.
// Expert rows are read once and marked non-temporal; residual, shared and
// gamma rows use the default policy; y and x_out are stored non-temporal,
// which streams them out instead of leaving them dirty in L2 for the end of
// the kernel to write back (c3, inputs cold: 15.7 against 17.8 us with
// default-policy stores).
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kGroup = 8;  // expert rows loaded together

__global__ __launch_bounds__(kMaxThreads) void k_combine(
    const uint16_t *__restrict__ eo, const int32_t *__restrict__ assist,
    const float *__restrict__ scales, const uint16_t *__restrict__ shared,
    const uint16_t *__restrict__ residual, const uint16_t *__restrict__ gamma, float eps,
    int Bs, int H, int K, int shared_mode, uint16_t *__restrict__ y,
    uint16_t *__restrict__ x_out, float *__restrict__ rstd_out, int32_t *__restrict__ dev_err)
{
    __shared__ float s_part[kMaxWaves];

    const int i = blockIdx.x;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1), w = t / kWave, nw = row_threads(H) / kWave;
    const uint32_t rowb = (uint32_t)H * 2;
    // byte offsets of this lane's two parts in a row; a part past the row end
    // reads at kNoPart (zeros) and is not stored
    const int e0 = part_elem(t, 0), e1 = part_elem(t, 1);
    const bool v0 = e0 < H, v1 = e1 < H;
    const uint32_t o0 = v0 ? (uint32_t)e0 * 2 : kNoPart, o1 = v1 ? (uint32_t)e1 * 2 : kNoPart;
    const rsrc_t r_eo = buffer_rsrc(eo, (uint32_t)(Bs * K) * rowb);
    const rsrc_t r_tok = buffer_rsrc(residual, (uint32_t)Bs * rowb);
    const rsrc_t r_sh = buffer_rsrc(shared ? shared : residual, shared ? (uint32_t)Bs * rowb : 0u);
    const rsrc_t r_g = buffer_rsrc(gamma, rowb);
    const uint32_t tok = (uint32_t)i * rowb;

    // 1. the token's K entries, one per lane, loaded first: the expert-row
    //    loads depend on them, and wait counters retire in issue order
    const int kk = min(lane, K - 1);
    int my_r = assist[i * K + kk];
    const float my_s = scales[i * K + kk];
    if (lane >= K)
        my_r = -1;

    // 2. residual, shared (zeros without one) and gamma do not depend on the routing
    const uint4 ra = buf_load16<kPlain>(r_tok, tok + o0), rb = buf_load16<kPlain>(r_tok, tok + o1);
    const uint4 sa = buf_load16<kPlain>(r_sh, tok + o0), sb = buf_load16<kPlain>(r_sh, tok + o1);
    const uint4 ga = buf_load16<kPlain>(r_g, o0), gb = buf_load16<kPlain>(r_g, o1);

    // 3. the dispatched entries' rows through kGroup register slots; entries
    //    that were not dispatched (row -1) or point outside the buffer are skipped
    if (my_r >= Bs * K) {
        if (w == 0 && dev_err)
            atomicOr(dev_err, 8);
        my_r = -1;
    }
    const float ws = wave_sum_f32(my_r >= 0 ? my_s : 0.0f);
    uint64_t live = __ballot(my_r >= 0);
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
        acc[j] = 0.0f;
    uint4 ea[kGroup], eb[kGroup];
    float sk[kGroup];
    // the next dispatched entry in order of k into slot j (a far offset, weight 0, when
    // none is left): its row's two parts and its weight
    auto issue = [&](int j) {
        uint32_t base = kNoRow;
        sk[j] = 0.0f;
        if (live) {
            const int k = __builtin_ctzll(live);
            live &= live - 1;
            base = (uint32_t)__builtin_amdgcn_readlane(my_r, k) * rowb;
            sk[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
        }
        ea[j] = buf_load16<kStream>(r_eo, base + o0);
        eb[j] = buf_load16<kStream>(r_eo, base + o1);
    };
    auto sum = [&](int j) {
        float v[16];
        unpack8(ea[j], v);
        unpack8(eb[j], v + 8);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            acc[e] = fmaf(sk[j], v[e], acc[e]);
    };
    const bool two_groups = __popcll(live) > kGroup;  // the same in every wave of the block
    if (!two_groups) {
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            issue(j);
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            sum(j);
    } else {
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            issue(j);
        // up to 2 * kGroup rows (K <= 16): each slot is refilled with the row kGroup
        // entries later as soon as its row is summed, so the second group's loads go out
        // while the first group is still arriving.  Rows are summed in the same order as
        // with one group after the other.
#pragma unroll
        for (int j = 0; j < kGroup; ++j) {
            sum(j);
            // the sums are done and the slot is free before its next load goes out:
            // without this the compiler hoists the second group's loads above the
            // sums and keeps both groups in registers (216 instead of 120 VGPRs)
#pragma unroll
            for (int e = 0; e < 16; e += 4)
                asm volatile("" : "+v"(acc[e]), "+v"(acc[e + 1]), "+v"(acc[e + 2]),
                             "+v"(acc[e + 3])::"memory");
            issue(j);
        }
#pragma unroll
        for (int j = 0; j < kGroup; ++j)
            sum(j);
    }

    float xf[16];
    {
        float rv[16];
        unpack8(ra, rv);
        unpack8(rb, rv + 8);
        if (shared) {
            const float wsh = shared_mode == 0 ? ws : 1.0f;
            float sv[16];
            unpack8(sa, sv);
            unpack8(sb, sv + 8);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[e] = fmaf(wsh, sv[e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e)
            xf[e] = acc[e] + rv[e];
    }

    // parts past the row end add nothing to the sum of squares
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        ss = fmaf(v0 ? xf[e] : 0.0f, v0 ? xf[e] : 0.0f, ss);
        ss = fmaf(v1 ? xf[8 + e] : 0.0f, v1 ? xf[8 + e] : 0.0f, ss);
    }
    ss = wave_sum_f32(ss);
    if (lane == 0)
        s_part[w] = ss;

    if (x_out) {
        const rsrc_t r_xo = buffer_rsrc(x_out, (uint32_t)Bs * rowb);
        buf_store16<kStream>(r_xo, tok + o0, pack8_bf16(xf));
        buf_store16<kStream>(r_xo, tok + o1, pack8_bf16(xf + 8));
    }
    lds_barrier();
    float tot = 0.0f;
    for (int j = 0; j < nw; ++j)
        tot += s_part[j];
    const float rstd = 1.0f / __builtin_sqrtf(tot / (float)H + eps);
    if (t == 0 && rstd_out)
        rstd_out[i] = rstd;
    float g[16], o[16];
    unpack8(ga, g);
    unpack8(gb, g + 8);
#pragma unroll
    for (int e = 0; e < 16; ++e)
        o[e] = xf[e] * rstd * g[e];
    const rsrc_t r_y = buffer_rsrc(y, (uint32_t)Bs * rowb);
    buf_store16<kStream>(r_y, tok + o0, pack8_bf16(o));
    buf_store16<kStream>(r_y, tok + o1, pack8_bf16(o + 8));
}

hipError_t launch_combine(const uint16_t *expert_out, const int32_t *assist,
                          const float *scales, const uint16_t *shared,
                          const uint16_t *residual, const uint16_t *gamma, float eps, int Bs,
                          int H, int K, int shared_mode, uint16_t *y, uint16_t *x_out,
                          float *rstd, int32_t *dev_err, hipStream_t stream)
{
    hipLaunchKernelGGL(k_combine, dim3(Bs), dim3(row_threads(H)), 0, stream, expert_out, assist,
                       scales, shared, residual, gamma, eps, Bs, H, K, shared_mode, y, x_out,
                       rstd, dev_err);
    return hipGetLastError();
}

}  // namespace moe
