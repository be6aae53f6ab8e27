// device.h -- gfx950 device helpers for the MoE mapping / dispatch / combine
// kernels: bf16 conversions, streaming loads/stores, an LDS-only block
// barrier, wave64 reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxThreads = 512;        // a row of H <= 8192 elements: 16 per thread
constexpr int kMaxWaves = kMaxThreads / kWave;

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even: one v_cvt_pk_bf16_f32 on gfx950
// (two scalar casts compile to one conversion each, plus the masks and shifts that
// pack them).
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const moe_f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, moe_bf16x2));
}

__device__ __forceinline__ uint4 pack8_bf16(const float *f)
{
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
}

// 16 bf16 (two uint4) -> 16 fp32
__device__ __forceinline__ void unpack16(const uint4 &a, const uint4 &b, float *v)
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_lo(w[j]);
        v[2 * j + 1] = bf16_hi(w[j]);
    }
}

// Largest |x| among 16 bf16 as a magnitude pattern (sign cleared), NaN
// skipped and infinity included; *nan tells whether a NaN was seen.  For
// non-negative values the integer order of bf16 patterns is the numeric order.
// With p the 15-bit magnitude, (p + 0x7f) mod 2^15 keeps the order of every
// non-NaN pattern (0 .. 0x7f80 map to 0x7f .. 0x7fff) and sends the NaN
// patterns (0x7f81 .. 0x7fff) below zero's image; bit 15 of p + 0x7f marks a
// NaN.  Both halves of a word are handled at once with packed 16-bit integer
// arithmetic.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t amax_bits16(const uint4 &a, const uint4 &b, bool *nan = nullptr)
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const u16x2 bias = {0x7f, 0x7f}, mag = {0x7fff, 0x7fff};
    u16x2 m = {0, 0}, seen = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u16x2 p = (__builtin_bit_cast(u16x2, w[j]) & mag) + bias;
        seen |= p;
        m = __builtin_elementwise_max(m, p & mag);
    }
    if (nan)
        *nan = ((seen.x | seen.y) & 0x8000u) != 0;
    const uint32_t mm = max((uint32_t)m.x, (uint32_t)m.y);
    return mm > 0x7fu ? mm - 0x7fu : 0u;
}

// ---------------------------------------------------------------- streaming access

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads / stores marked non-temporal: data read or written exactly
// once by this kernel (expert rows in, coded rows out) should not displace
// reusable lines in the caches.
__device__ __forceinline__ uint4 load_nt16(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt16(void *p, const uint4 &v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// ---------------------------------------------------------------- buffer access

// Raw buffer loads and stores with an explicit cache policy.  The address is
// a 32-bit byte offset from a base (every buffer here is below 2 GB), and an
// access at an offset at or past the buffer's size reads zeros and writes
// nothing, with no memory traffic: a load of a row that does not exist
// (kNoRow) is still issued, so straight-line load sequences keep a fixed
// count for the wait counters.  Every buffer passed here is below 256 MB, so
// a row base below 256 MB plus kNoPart, or kNoRow plus any in-row offset or
// kNoPart, is past the end without wrapping around 2^32.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kPlain = 0;      // default policy
constexpr int kStream = 2;     // non-temporal: read or written once
constexpr int kDevice = 16;    // device scope: stores write through to memory
constexpr uint32_t kNoRow = 0x80000000u;   // row base of a row that does not exist
constexpr uint32_t kNoPart = 0x40000000u;  // in-row offset of a part past the row end

__device__ __forceinline__ rsrc_t buffer_rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

template <int POL>
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t off)
{
    const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL));
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int POL>
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, const uint4 &v)
{
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, POL);
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int POL>
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, uint32_t lo, uint32_t hi)
{
    const u32x2 w = {lo, hi};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, POL);
}

// ---------------------------------------------------------------- row layout

// Row layout of the dispatch and combine kernels: wave w of a row block owns
// elements [1024 w, 1024 w + 1024) of the row, and lane l holds two chunks of
// eight, part 0 at 1024 w + 8 l and part 1 at 1024 w + 512 + 8 l.  A wave's
// 16-byte accesses to a bf16 row then each cover one contiguous kilobyte
// (eight whole cache lines); with each lane's 16 elements consecutive, every
// access instruction would touch 16 half-used lines, which measured about 12%
// slower for the same bytes.  A 32-element block is 4 lanes of one part and a
// power-of-two tile of up to 512 elements is tile/8 lanes of one part.
constexpr int kPartElems = 8;
constexpr int kWaveElems = 1024;

__device__ __forceinline__ int part_elem(int t, int p)
{
    return (t >> 6) * kWaveElems + p * (kWaveElems / 2) + (t & (kWave - 1)) * kPartElems;
}

// 8 bf16 (one uint4) -> 8 fp32
__device__ __forceinline__ void unpack8(const uint4 &a, float *v)
{
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}

// ---------------------------------------------------------------- block barrier

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (vmcnt(0)), which would
// serialise the HBM traffic in flight behind each barrier; the barriers in
// these kernels only publish LDS data, so global accesses stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- wave ops

// Wave-wide reductions and scans use DPP lane moves (VALU operands, a few
// cycles each) rather than LDS-path lane shuffles.  DPP controls: row_shr:n
// 0x110 + n, row_mirror 0x140, row_half_mirror 0x141, row_bcast:15 0x142,
// row_bcast:31 0x143, quad_perm 0x00-0xff.  A row is 16 lanes.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, true);
}

constexpr int kQuadXor1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;  // quad_perm [2,3,0,1]

// Reduces v over the wave into lane 63 with op (commutative, associative on
// the values used), then returns lane 63's value in every lane: the same
// bits everywhere, and the same order of operations on every run.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op)
{
    auto mv = [](T x, auto ctrl) {
        return __builtin_bit_cast(T, dpp<decltype(ctrl)::value>(__builtin_bit_cast(int, x)));
    };
    v = op(v, mv(v, std::integral_constant<int, kQuadXor1>{}));
    v = op(v, mv(v, std::integral_constant<int, kQuadXor2>{}));
    v = op(v, mv(v, std::integral_constant<int, 0x141>{}));  // half-row mirror: 8 lanes
    v = op(v, mv(v, std::integral_constant<int, 0x140>{}));  // row mirror: 16 lanes
    // rows 1 and 3 add the last lane of rows 0 and 2, then rows 2 and 3 add lane 31
    const T b15 = __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
    v = op(v, b15);
    const T b31 = __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(
                                            0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
    v = op(v, b31);
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ int wave_sum_i32(int v)
{
    return wave_reduce(v, [](int a, int b) { return a + b; });
}

// Every lane gets the same bits (the total is read from one lane).
__device__ __forceinline__ float wave_sum_f32(float v)
{
    return wave_reduce(v, [](float a, float b) { return a + b; });
}

// Inclusive prefix sum over the wave: Hillis-Steele steps inside each row of
// 16 lanes (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read
// 0), then the row broadcasts carry rows 0 and 2 into rows 1 and 3 and the
// first half into the second.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    v += dpp<0x118>(v);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
    return v;
}

// Maximum over aligned groups of n lanes (n = 1, 2, 4, 8, 16 or 32), the
// group's maximum in each of its lanes: quad permutes, then the half-row and
// row mirrors (lane i and its mirror lie in different halves of the group),
// then, for 32, a lane shuffle.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t m, int n)
{
    if (n >= 2)
        m = max(m, (uint32_t)dpp<kQuadXor1>((int)m));
    if (n >= 4)
        m = max(m, (uint32_t)dpp<kQuadXor2>((int)m));
    if (n >= 8)
        m = max(m, (uint32_t)dpp<0x141>((int)m));
    if (n >= 16)
        m = max(m, (uint32_t)dpp<0x140>((int)m));
    if (n >= 32)
        m = max(m, (uint32_t)__shfl_xor((int)m, 16));
    return m;
}

}  // namespace moe
