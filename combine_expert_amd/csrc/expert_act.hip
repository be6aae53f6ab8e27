// expert_act.hip -- the activation between the expert FFN's two projections.
// The pages place the expert computation between dispatch and combine in the
// fixed calling sequence ("aclnnMoeUpdateExpert") without defining it; it is
// read as the gated FFN of a DeepSeek-V3-shaped layer.  The first projection's
// output row holds the gate g (columns [0, I)) and the up projection u
// (columns [I, 2I)); this kernel computes act = bf16(silu(g) * u) with
// silu(g) = g / (1 + exp(-g)) and codes act for the second projection with the
// mxfp8 quantiser of "aclnnMoeDistributeDispatchV2", 计算公式 case 5 (blocks of
// 32, sharedExp = floor(log2 max|act|) - 8, E4M3 codes, E8M0 byte sharedExp + 127).
//
// One thread per 16 consecutive act elements: two 16-byte loads of gate and two
// of up (a wave covers 2 KB of each contiguously), fp32 arithmetic, one RNE
// rounding to bf16, then the dispatch's block coder on the bf16 values (a lane
// pair is one block of 32; its maximum is a lane swap).  Rows outside
// [offsets[0], offsets[E]) are not touched.  Bound by HBM: per row 4I bytes
// read and I + I/32 written (2I more with the optional bf16 act output).
#include "dispatch_impl.h"
#include "moe_expert.h"

namespace moe {

constexpr int kActThreads = 256;

__global__ __launch_bounds__(kActThreads) void k_expert_swiglu(
    const uint16_t *__restrict__ y1, const int32_t *__restrict__ offsets, int E, int rows,
    int I, int sc_row, int sc_group, uint8_t *__restrict__ codes, uint8_t *__restrict__ sc,
    uint16_t *__restrict__ act, int32_t *__restrict__ dev_err)
{
    const int o0 = offsets[0], o1 = offsets[E];
    const unsigned g = blockIdx.x * kActThreads + threadIdx.x;
    if (g == 0 && dev_err && (o0 < 0 || o1 > rows || o1 < o0))
        atomicOr(dev_err, MOE_ERR_OFFSETS);
    const unsigned cpr = (unsigned)I / 16;  // chunks per row: even, so a block never straddles rows
    const int r = (int)(g / cpr), c = (int)(g - (unsigned)r * cpr);
    // both lanes of a pair share r: they leave together, before the lane swap
    if (r < max(o0, 0) || r >= min(o1, rows))
        return;
    const uint16_t *row = y1 + (size_t)r * 2 * I + 16 * c;
    const uint4 *gp = reinterpret_cast<const uint4 *>(row);
    const uint4 *up = reinterpret_cast<const uint4 *>(row + I);
    const uint4 ga = gp[0], gb = gp[1], ua = up[0], ub = up[1];
    float gv[16], uv[16], a[16];
    unpack16(ga, gb, gv);
    unpack16(ua, ub, uv);
    // silu(g) = g / (1 + exp(-g)) with e = exp(-|g|): g / (1 + e) for g >= 0 and
    // g * e / (1 + e) below, the same function without exp(-g) overflowing fp32 for
    // g < -88 (where silu(g) is still a normal bf16 down to about g = -93).  e is
    // 2^t with t = -|g| log2(e) by the hardware exp2; below t = -126 its result
    // would be a subnormal, so it is taken at t + 64 and scaled by 2^-64 (exact).
    // The quotient is a hardware reciprocal and a product.  Each step is within a
    // few fp32 ulps (about 2^-21 relative), against the 2^-8 of a bf16 step; the
    // kernel is bound by issue, not HBM, with expf and IEEE division (52 vector
    // instructions per element, 12.6 us at 4096 rows x I = 2048).
    // When no gate of the wave lies below -87, exp(-g) stays a normal float and the plain
    // form g / (1 + exp(-g)) needs none of that (a branch uniform over the wave).
    float gmin = gv[0];
#pragma unroll
    for (int j = 1; j < 16; ++j)
        gmin = fminf(gmin, gv[j]);
    if (__builtin_amdgcn_ballot_w64(!(gmin >= -87.0f)) == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float e = __builtin_amdgcn_exp2f(gv[j] * -1.44269504f);
            a[j] = gv[j] * __builtin_amdgcn_rcpf(1.0f + e) * uv[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float g = gv[j];
            const float t = -fabsf(g) * 1.44269504f;
            const bool sub = t < -126.0f;
            float e = __builtin_amdgcn_exp2f(sub ? t + 64.0f : t);
            e = sub ? e * 0x1p-64f : e;
            const float s = (g >= 0.0f ? g : g * e) * __builtin_amdgcn_rcpf(1.0f + e);
            a[j] = s * uv[j];
        }
    }
    const uint4 xa = pack8_bf16(a), xb = pack8_bf16(a + 8);

    // the case-5 coder on the bf16 values, as the dispatch codes a token's row
    float v[16];
    unpack16(xa, xb, v);
    bool nan;
    uint32_t m = amax_bits16(xa, xb, &nan);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    int se = -127;
    if (m)  // an infinite maximum takes the largest exponent, 127
        se = m >= 0x7f80u ? 127 : max(-127, bf16_ilogb(m) - 8);
    float f = __uint_as_float((uint32_t)(127 - se) << 23);
    if (se == 127) {  // 2^-127 is not a normal float: two exact steps
#pragma unroll
        for (int j = 0; j < 16; ++j)
            v[j] *= 0x1p-64f;
        f = 0x1p-63f;
    }
    uint4 code = e4m3_codes(v, f);
    if (nan)
        code = e4m3_nan_codes(code, xa, xb);
    *reinterpret_cast<uint4 *>(codes + (size_t)r * I + 16 * c) = code;
    if ((c & 1) == 0) {
        const int b = c / 2;
        sc[(size_t)r * sc_row + (size_t)(b >> 4) * sc_group + (b & 15)] = (uint8_t)(se + 127);
    }
    if (act) {
        uint4 *ap = reinterpret_cast<uint4 *>(act + (size_t)r * I + 16 * c);
        ap[0] = xa;
        ap[1] = xb;
    }
}

hipError_t launch_expert_swiglu(const uint16_t *y1, const int32_t *offsets, int E, int rows,
                                int I, bool group_major, uint8_t *codes, uint8_t *sc,
                                uint16_t *act, int32_t *dev_err, hipStream_t stream)
{
    if (rows == 0)
        return hipSuccess;
    const unsigned threads = (unsigned)rows * (unsigned)(I / 16);
    const unsigned blocks = (threads + kActThreads - 1) / kActThreads;
    const int sc_row = group_major ? 16 : I / 32;
    const int sc_group = group_major ? 16 * rows : 16;
    hipLaunchKernelGGL(k_expert_swiglu, dim3(blocks), dim3(kActThreads), 0, stream, y1, offsets,
                       E, rows, I, sc_row, sc_group, codes, sc, act, dev_err);
    return hipGetLastError();
}

}  // namespace moe
