// device.h -- gfx950 device helpers for the MoE mapping / dispatch / combine
// kernels: bf16 conversions, streaming loads/stores, an LDS-only block
// barrier, wave64 reductions and scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxThreads = 512;        // H <= 8192 elements / 16 per thread
constexpr int kMaxWaves = kMaxThreads / kWave;
constexpr int kChunk = 16;              // row elements owned by one thread

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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

// Largest |x| bit pattern among 16 bf16 (sign cleared).  For non-negative
// values the integer order of bf16 patterns is the numeric order.
__device__ __forceinline__ uint32_t amax_bits16(const uint4 &a, const uint4 &b)
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        m = max(m, w[j] & 0x7fffu);
        m = max(m, (w[j] >> 16) & 0x7fffu);
    }
    return m;
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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Every lane gets the same bits: the butterfly adds the same pairs in every lane.
__device__ __forceinline__ float wave_sum_f32(float v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o);
        if (lane >= o)
            v += t;
    }
    return v;
}

}  // namespace moe
