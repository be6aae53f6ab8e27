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
// Tiling.  One block per CU computes a 128 x 256 output tile (128 rows of one
// instance x 256 output columns) with eight waves of 64 x 64 each, two per SIMD
// (measured 9% faster than four waves of 64 x 128: one wave's MFMAs run while
// the other waits on its LDS reads or the step barrier).  The tile
// size is set by the L2 -> CU load rate (about 50 B/clk per CU measured): a
// K step of 128 brings (128 + 256) x 128 bytes for 128 x 256 x 128 MACs,
// which keeps the loads under that rate at full MFMA speed, where a 128 x 128
// tile does not.
//
// Pipeline.  K is walked 128 at a time through a three-stage LDS ring.  The
// operand tiles go global -> LDS with global_load_lds_dwordx4 (no register
// staging, no LDS store instructions: those run at about a third of the LDS
// read rate) two steps ahead of the MFMAs, so each step waits only for loads
// issued two steps earlier.  A wave's DMA instruction fills 1 KB of LDS
// lane-contiguously; each 128-byte LDS row keeps its eight 16-byte chunks in
// XOR-swizzled order (slot s holds chunk s ^ ((row >> 1) & 7)), which the lanes
// realise by fetching the permuted global chunk, so that the MFMA fragment
// reads of sixteen consecutive rows spread over the banks: two rows share the
// 64 banks, so the sixteen rows are eight in each half and need eight distinct
// slots (row & 7 gives four: a two-way conflict).  The scale bytes
// travel separately: when a row's scales for four K steps are 16 contiguous
// bytes (K a multiple of 512) one 16-byte copy per row brings them every
// fourth step into a two-group ring; otherwise a 4-byte copy per row each step.
// Either way a copy touches one line per row, so the scales cost as many L2
// line requests as the tiles they scale unless they are grouped.
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
// Two tilings for mxfp8 (grouped scales).  Besides the 128 x 256 tiles described here,
// 256 x 256 tiles (further down) need a third fewer line requests per flop and win by
// 11-14% on shapes that fill whole rounds of them; on uneven row counts their last,
// partial round costs more than it saves.  The launch computes both row-tile counts on
// the device and takes the tiling a cost model of whole and partial rounds estimates
// faster (every block decides alike).  int8 and ungrouped scales use the 128 x 256 tiles.
//
// Scheduling.  Each instance needs ceil(rows_e / 128) row tiles; a block
// prefix-sums those counts into LDS once and then walks the flattened
// (column tile, row tile) space grid-stride, row tiles fastest so that the
// blocks working on one weight tile run together.  Consecutive block ids are
// spread over the eight XCDs round-robin by the hardware, so the block id is
// remapped to give each XCD (and its L2) a contiguous range of tiles.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "moe_expert.h"

namespace moe {
namespace {

constexpr int kBM = 128;        // rows per tile
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 128;        // K elements (bytes) per step
constexpr int kStages = 3;
constexpr int kAhead = kStages - 1;   // K steps between issuing a stage's copies and using it
constexpr int kWavesM = 2;      // waves along the rows of a tile
constexpr int kWavesN = 4;      // waves along the columns
constexpr int kGemmWaves = kWavesM * kWavesN;
constexpr int kGemmThreads = kGemmWaves * 64;
constexpr int kFragM = kBM / kWavesM / 16;   // 16-row MFMA fragments per wave (activations)
// per wave and step: 1 KB DMA runs of the two tiles (8 rows x 128 bytes each)
constexpr int kXRuns = kBM / 8 / kGemmWaves;
constexpr int kXcds = 8;
constexpr int kCus = 256;
constexpr int kMaxInstances = 1024;
constexpr int kGroupM = 8;      // row tiles per patch of the tile order
constexpr int kScaleGroup = 4;  // K steps per grouped scale copy (16 bytes per row)

// scale copies go in runs of 64 rows: weight run j to wave j, activation run j to wave
// (kBN / 64 + j) mod waves; at most one of each per wave
static_assert(kBM / 64 <= kGemmWaves && kBN / 64 <= kGemmWaves, "scale runs: one per wave");

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

// operand formats (the dispatch's quantisation modes)
constexpr int kModeI8Token = 2;   // int8, one f32 scale per row; weights int8, f32 per column
constexpr int kModeI8Tile = 3;    // int8, one f32 scale per row and 128-element tile
constexpr int kModeMx = 4;        // E4M3 with E8M0 scales per 32 elements, both operands

struct GemmArgs {
    const uint8_t *a;        // [rows, K] E4M3 or int8
    const uint8_t *a_sc;     // [rows, K/32] E8M0, or f32 [rows] / [rows, K/128]
    const int32_t *offsets;  // [E+1]
    const uint8_t *w;        // [E, N, K] E4M3 or int8
    const uint8_t *w_sc;     // [E, N, K/32] E8M0, or f32 [E, N]
    uint16_t *y;             // [rows, N] bf16
    int32_t *dev_err;
    int E, rows, N, K;
    // activation scale bytes: row r, byte offset `off` of the row-major layout, at
    // r * x_pitch + (off / 16) * x_group + off % 16.  Row-major: (K / 32, 16); mxfp8
    // exponents group-major ([K/512 rounded up][rows][16]): (16, 16 * rows).
    int x_pitch;
    size_t x_group;
};

struct Stage {
    uint8_t x[kBM * kBK];    // 16 KB: activation rows, swizzled 16-byte chunks
    uint8_t w[kBN * kBK];    // 32 KB: weight rows
};

// Scale words of one K step (4 bytes per row) or of a group of four steps (16 bytes per row).
template <int STEPS>
struct Scales {
    uint32_t x[kBM][STEPS];
    uint32_t w[kBN][STEPS];
};

// A grouped scale row holds four K steps, one word each, the word's byte b being the E8M0
// exponent of 32-element block b of that step's 128 bytes.  A lane needs only block g of
// every step: one 16-byte read per group, packed here into one word (step j in byte j).
// Per-step reads of one step's exponents (a word or a byte per lane) hit LDS rows 16 bytes
// apart and show bank conflicts on the counters; 16-byte reads of whole rows do not.
__device__ __forceinline__ uint32_t pack_block_exponents(const u32x4 q, int g)
{
    const int sh = 8 * g;
    return ((q.x >> sh) & 0xffu) | ((q.y >> sh) & 0xffu) << 8 | ((q.z >> sh) & 0xffu) << 16 |
           ((q.w >> sh) & 0xffu) << 24;
}
__device__ __forceinline__ uint32_t pack_block_exponents(const uint32_t *row, int g)
{
    return pack_block_exponents(*reinterpret_cast<const u32x4 *>(row), g);
}

// s_waitcnt immediate (gfx9 layout): vmcnt <= n, expcnt and lgkmcnt not waited on
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// One lane's share of a wave-wide global -> LDS copy: lane i's bytes land at
// LDS address lds + i * size, lds being the same for the whole wave (it goes
// through M0).  Written as inline asm on purpose: the compiler would make
// every later LDS read, and every LDS fence, wait for all such copies in
// flight, which caps the pipeline at one step; here the waits are explicit.
// The asm has no output registers (the data goes to LDS), and the address
// registers are read when the instruction issues.  M0 is listed as clobbered, so
// the compiler assumes nothing about it after the statement and sets it again
// before any use of its own (LDS-direct or message instructions); the kernel's
// own LDS accesses are ordinary ds_ instructions, which do not read M0 on gfx950.
__device__ __forceinline__ void dma16(const uint8_t *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ void dma4(const uint8_t *src, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(lds) : "memory", "m0");
}

// Global chunk offset a DMA lane fetches for copy run `run` (8 rows starting at LDS row
// 8 * run): lane l fills LDS row 8 * run + l / 8, slot l % 8, which holds chunk
// slot ^ ((row >> 1) & 7) = slot ^ (4 * (run & 1) + l / 16).
__device__ __forceinline__ int dma_chunk_of(int run, int lane)
{
    return ((lane & 7) ^ (((run & 1) << 2) | (lane >> 4))) << 4;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)p);
}

// s_waitcnt needs an immediate: the count, known per wave at run time (wave-uniform),
// picks one of the immediates (counts above 31 wait for everything)
__device__ __forceinline__ void wait_vm(int n)
{
#define MOE_WAIT_CASE(c) \
    case c: __builtin_amdgcn_s_waitcnt(vmcnt_imm(c)); break;
    switch (n) {
        MOE_WAIT_CASE(1) MOE_WAIT_CASE(2) MOE_WAIT_CASE(3) MOE_WAIT_CASE(4) MOE_WAIT_CASE(5)
        MOE_WAIT_CASE(6) MOE_WAIT_CASE(7) MOE_WAIT_CASE(8) MOE_WAIT_CASE(9) MOE_WAIT_CASE(10)
        MOE_WAIT_CASE(11) MOE_WAIT_CASE(12) MOE_WAIT_CASE(13) MOE_WAIT_CASE(14)
        MOE_WAIT_CASE(15) MOE_WAIT_CASE(16) MOE_WAIT_CASE(17) MOE_WAIT_CASE(18)
        MOE_WAIT_CASE(19) MOE_WAIT_CASE(20) MOE_WAIT_CASE(21) MOE_WAIT_CASE(22)
        MOE_WAIT_CASE(23) MOE_WAIT_CASE(24) MOE_WAIT_CASE(25) MOE_WAIT_CASE(26)
        MOE_WAIT_CASE(27) MOE_WAIT_CASE(28) MOE_WAIT_CASE(29) MOE_WAIT_CASE(30)
        MOE_WAIT_CASE(31)
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    }
#undef MOE_WAIT_CASE
}

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

// LDS of one block: the copy ring, the scale ring (per step, or in groups of four steps),
// the row-tile prefix of the instances and a scan scratch
template <bool GROUPED>
struct GemmSmem {
    static constexpr int kScaleSteps = GROUPED ? kScaleGroup : 1;
    static constexpr int kScaleBufs = GROUPED ? 2 : kStages;
    Stage stage[kStages];
    Scales<kScaleSteps> scale[kScaleBufs];
    uint16_t tiles[kMaxInstances + 1];   // exclusive prefix of row tiles per instance
    int wave_sum[kGemmWaves];
};

// One output tile: rows [m0, m0 + kBM) of instance e (valid below row_hi) by columns
// [n0, n0 + BN).  MODE: operand format (kModeMx, kModeI8Tile, kModeI8Token).  GROUPED:
// per-step scales in 16-byte groups of four K steps (needs K % 512 == 0), else 4 bytes per
// step.  BN: 256 for whole tiles; 128 or 64 for the pieces the last round is split into.
template <int MODE, bool GROUPED, int BN>
__device__ __forceinline__ void run_tile(const GemmArgs &p, GemmSmem<GROUPED> &sm, int e,
                                         int m0, int row_hi, int n0)
{
    // the accumulator: fp32 (mxfp8; int8 per tile, where each step's exact int32 sum is scaled
    // into it) or int32 (int8 per token: exact over all of K, scaled at the end)
    using Acc = std::conditional_t<MODE == kModeI8Token, v4i, v4f>;
    using Stg = Stage;
    using Sc = Scales<GemmSmem<GROUPED>::kScaleSteps>;
    constexpr bool kStepScales = MODE != kModeI8Token;   // scale copies along K
    constexpr bool kWeightStepScales = MODE == kModeMx;
    constexpr int kWRunsT = BN / 8 / kGemmWaves;          // weight copy runs per wave
    constexpr int kFragNT = BN / kWavesN / 16;            // weight fragments per wave
    constexpr int kDataLoadsT = kXRuns + kWRunsT;
    static_assert(kWRunsT >= 1 && kFragNT >= 1 && BN <= kBN, "tile width");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nk = p.K / kBK;
    const int g = lane >> 4;                  // lane group: K chunk / scale block
    const int r16 = lane & 15;
    const int wn = wave % kWavesN, wm = wave / kWavesN;   // the wave's part of the tile
    // the wave's scale runs of 64 rows: weight run j to wave j, activation run j to wave
    // (BN / 64 + j) mod waves
    const bool w_run = wave < BN / 64;
    const int x_idx = (wave - BN / 64 + kGemmWaves) % kGemmWaves;   // activation run, if any
    const bool x_run = x_idx < kBM / 64;
    // scale copies per issue (wave-uniform)
    const int n_scale = (kWeightStepScales && w_run ? 1 : 0) + (kStepScales && x_run ? 1 : 0);
    // DMA lane mapping: one instruction covers 8 rows x 128 bytes; lane -> row lane / 8, LDS
    // slot lane % 8, global chunk per dma_chunk_of
    const int dma_row = lane >> 3;
    // swizzled offsets of chunks g and g + 4 (fragments start at multiples of 16 rows, so
    // (row >> 1) & 7 = r16 / 2)
    const int fr_c0 = ((g ^ (r16 >> 1)) << 4);
    const int fr_c1 = (((g + 4) ^ (r16 >> 1)) << 4);
    const uint8_t *w_e = p.w + (size_t)e * p.N * p.K;

    // this thread's DMA sources at K offset 0.  Rows past the instance (or past N) are
    // clamped to its last row (column): loaded, multiplied, never stored.
    const uint8_t *xsrc[kXRuns];
    const uint8_t *wsrc[kWRunsT];
#pragma unroll
    for (int q = 0; q < kXRuns; ++q) {
        const int r = min(m0 + (wave * kXRuns + q) * 8 + dma_row, row_hi - 1);
        xsrc[q] = p.a + (size_t)r * p.K + dma_chunk_of(wave * kXRuns + q, lane);
    }
#pragma unroll
    for (int q = 0; q < kWRunsT; ++q) {
        const int n = min(n0 + (wave * kWRunsT + q) * 8 + dma_row, p.N - 1);
        wsrc[q] = w_e + (size_t)n * p.K + dma_chunk_of(wave * kWRunsT + q, lane);
    }
    // mxfp8 weight scales are group-major ([E][ceil(K/512)][N][16]): a scale offset `off`
    // along K (bytes of the row-major layout) is group off / 16, byte off % 16
    const int n_groups = (p.K + kBK * kScaleGroup - 1) / (kBK * kScaleGroup);
    const uint8_t *wsc_src =
        p.w_sc + ((size_t)e * n_groups * p.N + min(n0 + (w_run ? wave : 0) * 64 + lane, p.N - 1)) * 16;
    const size_t wsc_group = (size_t)p.N * 16;   // bytes between groups
    const uint8_t *xsc_src =
        p.a_sc + (size_t)min(m0 + (x_run ? x_idx : 0) * 64 + lane, row_hi - 1) * p.x_pitch;

    // copies of K step s into stage s % kStages
    auto issue_data = [&](int s) {
        const int k0 = s * kBK;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(&sm.stage[s % kStages]);
#pragma unroll
        for (int q = 0; q < kXRuns; ++q)
            dma16(xsrc[q] + k0, lds_addr(base + offsetof(Stg, x) + (wave * kXRuns + q) * 1024));
#pragma unroll
        for (int q = 0; q < kWRunsT; ++q)
            dma16(wsrc[q] + k0, lds_addr(base + offsetof(Stg, w) + (wave * kWRunsT + q) * 1024));
    };
    // scale copies: buffer `buf`, scale bytes from byte offset `off` of each row
    auto issue_scales = [&](int buf, int off) {
        Sc &sc = sm.scale[buf];
        if (GROUPED) {
            if (kWeightStepScales && w_run)
                dma16(wsc_src + (off >> 4) * wsc_group, lds_addr(&sc.w[wave * 64][0]));
            if (x_run)
                dma16(xsc_src + (off >> 4) * p.x_group, lds_addr(&sc.x[x_idx * 64][0]));
        } else {
            if (kWeightStepScales && w_run)
                dma4(wsc_src + (off >> 4) * wsc_group + (off & 15), lds_addr(&sc.w[wave * 64][0]));
            if (x_run)
                dma4(xsc_src + (off >> 4) * p.x_group + (off & 15), lds_addr(&sc.x[x_idx * 64][0]));
        }
    };

    Acc acc[kFragNT][kFragM];
#pragma unroll
    for (int i = 0; i < kFragNT; ++i)
#pragma unroll
        for (int j = 0; j < kFragM; ++j)
            acc[i][j] = Acc{0, 0, 0, 0};

    // copies of one step: the tiles and, unless grouped, that step's scales
    const int step_loads = kDataLoadsT + (kStepScales && !GROUPED ? n_scale : 0);
    // prologue: steps 0 .. kAhead-1 (the first scale group right after step 0's tiles);
    // wait for step 0
    issue_data(0);
    if (kStepScales)
        issue_scales(0, 0);
#pragma unroll
    for (int i = 1; i < kAhead; ++i) {
        issue_data(min(i, nk - 1));
        if (kStepScales && !GROUPED)
            issue_scales(i % kStages, 4 * min(i, nk - 1));
    }
    wait_vm((kAhead - 1) * step_loads);
    lds_barrier();

    // mxfp8 with grouped scales: the loop runs whole groups of four steps, so the step within
    // the group is known at compile time.  The group's first step reads each fragment row's
    // exponents whole, where a per-step read would sit, and packs them (step j in byte j);
    // the other three steps read none.  (With a run-time test of the step in the step's
    // body instead, the same reads were slower than per-step reads.)
    constexpr bool kPackedScales = MODE == kModeMx && GROUPED;
    // int8 per tile with grouped scales: each activation fragment row's four tile scales,
    // read whole at the group's first step
    constexpr bool kTileRows = MODE == kModeI8Tile && GROUPED;
    uint32_t wsp[kFragNT], xsp[kFragM];
    u32x4 xrow[kFragM];
    auto step = [&](const int s, const auto sw_c) {
        constexpr int kSw = decltype(sw_c)::value;   // -1: not known at compile time
        constexpr bool kUseW = kPackedScales, kUseX = kPackedScales;
        const Stg &st = sm.stage[s % kStages];
        const Sc &sc = sm.scale[GROUPED ? (s / kScaleGroup) & 1 : s % kStages];
        const int sw = kSw >= 0 ? kSw : (GROUPED ? s % kScaleGroup : 0);
        // fragment reads: all weight fragments and the first two activation fragments go
        // out before this step's copies are issued; the other activation fragments two
        // ahead of the MFMAs that use them
        v8i xf[kFragM], wf[kFragNT];
        int xs[kFragM], ws[kFragNT];   // E8M0 scale bytes (mxfp8), f32 bits (int8 per tile)
#pragma unroll
        for (int fn = 0; fn < kFragNT; ++fn) {
            const int row = wn * (BN / kWavesN) + fn * 16 + r16;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c0]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c1]);
            wf[fn] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if constexpr (kUseW) {
                if constexpr (kSw == 0)
                    wsp[fn] = pack_block_exponents(sc.w[row], g);
                ws[fn] = (int)((wsp[fn] >> (8 * sw)) & 0xffu);
            }
            else if (kWeightStepScales)
                ws[fn] = (int)((sc.w[row][sw] >> (8 * g)) & 0xffu);
        }
        auto read_x = [&](int fm) {
            const int row = wm * (kBM / kWavesM) + fm * 16 + r16;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c0]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c1]);
            xf[fm] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            if constexpr (kUseX) {
                if constexpr (kSw == 0)
                    xsp[fm] = pack_block_exponents(sc.x[row], g);
                xs[fm] = (int)((xsp[fm] >> (8 * sw)) & 0xffu);
            }
            else if (MODE == kModeMx)
                xs[fm] = (int)((sc.x[row][sw] >> (8 * g)) & 0xffu);
            else if (MODE == kModeI8Tile) {
                if constexpr (kTileRows && kSw >= 0) {
                    if constexpr (kSw == 0)
                        xrow[fm] = *reinterpret_cast<const u32x4 *>(sc.x[row]);
                    xs[fm] = (int)xrow[fm][kSw];
                } else {
                    xs[fm] = (int)sc.x[row][sw];
                }
            }
        };
        read_x(0);
        if (kFragM > 1)
            read_x(1);

        // copies kAhead steps ahead (the last steps reload the final K step into stages
        // nobody reads any more: no branch in the count of copies in flight)
        const int s2 = min(s + kAhead, nk - 1);
        issue_data(s2);
        bool grouped_issue = false;
        if (!kStepScales) {
        } else if (GROUPED) {
            // every fourth step, the next group into the other buffer (the last group
            // reloads itself there, unused)
            if (s % kScaleGroup == 0) {
                const int gi = min(s / kScaleGroup + 1, nk / kScaleGroup - 1);
                issue_scales((s / kScaleGroup + 1) & 1, 16 * gi);
                grouped_issue = true;
            }
        } else {
            issue_scales((s + kAhead) % kStages, 4 * s2);
        }

#pragma unroll
        for (int fm = 0; fm < kFragM; ++fm) {
            if (fm + 2 < kFragM)
                read_x(fm + 2);
#pragma unroll
            for (int fn = 0; fn < kFragNT; ++fn) {
                if constexpr (MODE == kModeMx) {
                    acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf[fn], xf[fm], acc[fn][fm], 0, 0, 0, ws[fn], 0, xs[fm]);
                } else {
                    // K = 128 as two int8 MFMAs of 64: chunk g, then chunk g + 4 (both
                    // operands packed alike, which is all the instruction needs)
                    const v4i wlo = {wf[fn][0], wf[fn][1], wf[fn][2], wf[fn][3]};
                    const v4i whi = {wf[fn][4], wf[fn][5], wf[fn][6], wf[fn][7]};
                    const v4i xlo = {xf[fm][0], xf[fm][1], xf[fm][2], xf[fm][3]};
                    const v4i xhi = {xf[fm][4], xf[fm][5], xf[fm][6], xf[fm][7]};
                    if constexpr (MODE == kModeI8Token) {
                        acc[fn][fm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, xlo,
                                                                            acc[fn][fm], 0, 0, 0);
                        acc[fn][fm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, xhi,
                                                                            acc[fn][fm], 0, 0, 0);
                    } else {
                        v4i t = __builtin_amdgcn_mfma_i32_16x16x64_i8(wlo, xlo, v4i{0, 0, 0, 0},
                                                                     0, 0, 0);
                        t = __builtin_amdgcn_mfma_i32_16x16x64_i8(whi, xhi, t, 0, 0, 0);
                        const float as = __int_as_float(xs[fm]);   // the row's tile scale
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[fn][fm][i] = __builtin_fmaf((float)t[i], as, acc[fn][fm][i]);
                    }
                }
            }
        }
        // step s+1's copies went out kAhead - 1 steps ago: wait for this thread's (only the
        // steps issued since, and a scale group issued this step, may stay in flight; an
        // older group must have landed), then for everyone's
        wait_vm((kAhead - 1) * step_loads + (grouped_issue ? n_scale : 0));
        lds_barrier();
    };
    if constexpr (kPackedScales || kTileRows) {
        for (int s = 0; s < nk; s += kScaleGroup) {   // nk is a multiple of four here
            step(s, std::integral_constant<int, 0>{});
            step(s + 1, std::integral_constant<int, 1>{});
            step(s + 2, std::integral_constant<int, 2>{});
            step(s + 3, std::integral_constant<int, 3>{});
        }
    } else {
        for (int s = 0; s < nk; ++s)
            step(s, std::integral_constant<int, -1>{});
    }
    // the reloads of the last steps must land, and every wave be done with the rings,
    // before the epilogue reuses them
    wait_vm(0);
    lds_barrier();

    // ---- epilogue: lane holds columns wn*(BN/kWavesN) + fn*16 + 4g .. +3 of tile row
    //      wm*(kBM/kWavesM) + fm*16 + r16.  int8: times the weight column scales (and, per
    //      token, the row scale), in that order.  The bf16 tile goes through LDS (the
    //      rings are free now) so that the stores write whole rows: written straight from
    //      the MFMA layout, each store instruction would touch 16 rows with 32 bytes each.
    constexpr int kPitch = BN * 2 + 16;   // bytes per LDS row; the pad spreads the rows' banks
    static_assert(kBM * kPitch <= (int)sizeof(sm.stage), "output tile fits the rings");
    uint8_t *otile = reinterpret_cast<uint8_t *>(&sm.stage[0]);
    const float *wcol = reinterpret_cast<const float *>(p.w_sc) + (size_t)e * p.N;
#pragma unroll
    for (int fm = 0; fm < kFragM; ++fm) {
        const int lr = wm * (kBM / kWavesM) + fm * 16 + r16;
        float rs = 1.0f;
        if (MODE == kModeI8Token)
            rs = reinterpret_cast<const float *>(p.a_sc)[min(m0 + lr, row_hi - 1)];
#pragma unroll
        for (int fn = 0; fn < kFragNT; ++fn) {
            const int lc = wn * (BN / kWavesN) + fn * 16 + 4 * g;
            const int n = min(n0 + lc, p.N - 4);   // columns past N: computed, never stored
            v4f d;
            if constexpr (MODE == kModeMx) {
                d = acc[fn][fm];
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (MODE == kModeI8Token)
                        d[i] = (float)acc[fn][fm][i] * rs * wcol[n + i];
                    else
                        d[i] = acc[fn][fm][i] * wcol[n + i];
                }
            }
            *reinterpret_cast<uint2 *>(otile + lr * kPitch + lc * 2) =
                make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
        }
    }
    lds_barrier();
    // 16-byte chunks, row-major over the tile: a wave instruction stores whole rows
    constexpr int kRowChunks = BN / 8;
#pragma unroll
    for (int c = tid; c < kBM * kRowChunks; c += kGemmThreads) {
        const int lr = c / kRowChunks, cc = c % kRowChunks;
        const int r = m0 + lr, n = n0 + cc * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(otile + lr * kPitch + cc * 16);
        if (r < row_hi && n < p.N)
            *reinterpret_cast<uint4 *>(p.y + (size_t)r * p.N + n) = v;
    }
    lds_barrier();   // the next tile's copies rewrite the rings
}

// Row tiles of `bm` rows per instance, prefix-summed into tiles[0 .. E] in LDS (thread t
// owns instances 4t .. 4t+3); returns the total.  Offsets that are not non-decreasing within
// [0, rows] raise the error bit (once, from block 0, when `report`).
__device__ __forceinline__ int tile_prefix(const GemmArgs &p, int bm, uint16_t *tiles,
                                           int *wave_sum, bool report)
{
    static_assert(kGemmThreads * 4 >= kMaxInstances, "prefix covers every instance");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
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
            c[q] = (hi - lo + bm - 1) / bm;
        }
        tsum += c[q];
    }
    if (report && bad_any && blockIdx.x == 0 && p.dev_err)
        atomicOr(p.dev_err, MOE_ERR_OFFSETS);
    const int incl = wave_incl_scan(tsum);
    if (lane == kWave - 1)
        wave_sum[wave] = incl;
    lds_barrier();
    int excl = incl - tsum;
    for (int w = 0; w < wave; ++w)
        excl += wave_sum[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * tid + q;
        if (e < p.E)
            tiles[e] = (uint16_t)excl;
        if (e == p.E - 1)
            tiles[p.E] = (uint16_t)(excl + c[q]);
        excl += c[q];
    }
    lds_barrier();
    return tiles[p.E];
}

// The tiles of 128 rows x 256 columns, walked by the grid (see the kernel below).
template <int MODE, bool GROUPED>
__device__ __forceinline__ void narrow_tiles(const GemmArgs &p, GemmSmem<GROUPED> &sm,
                                             int m_tiles)
{
    const int n_tiles = (p.N + kBN - 1) / kBN;
    const int total = m_tiles * n_tiles;

    // ---- XCD-grouped virtual block id
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int v = (G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;

    // tile t -> instance e, rows [m0, row_hi), columns from n0.  Patch order: kGroupM row
    // tiles x every column tile, row tiles fastest, so the 32 blocks an XCD runs at once
    // share about 8 row tiles and 4 column tiles
    auto locate = [&](int t, int &e, int &m0, int &row_hi, int &n0) {
        const int grp = t / (kGroupM * n_tiles);
        const int tin = t - grp * kGroupM * n_tiles;
        const int gm = min(kGroupM, m_tiles - grp * kGroupM);
        const int tm = grp * kGroupM + tin % gm;
        const int tn = tin / gm;
        // instance of row tile tm: the last e with tiles[e] <= tm
        int lo_e = 0, hi_e = p.E;
        while (hi_e - lo_e > 1) {
            const int mid = (lo_e + hi_e) >> 1;
            if (sm.tiles[mid] <= tm)
                lo_e = mid;
            else
                hi_e = mid;
        }
        e = lo_e;
        int row_lo;
        instance_rows(p, e, row_lo, row_hi, nullptr);
        m0 = row_lo + (tm - sm.tiles[e]) * kBM;
        n0 = tn * kBN;
    };

    // whole rounds of whole tiles; the tiles left over for a last, partial round are cut along
    // the columns into 2 or 4 pieces so that it keeps (nearly) every CU busy, in a fraction of
    // a round (a piece loads the same activation tile and a part of the weight tile)
    const int rounds = total / G;
    const int tail = total - rounds * G;
    const int split = tail == 0 ? 1 : (G / tail >= 4 ? 4 : (G / tail >= 2 ? 2 : 1));
    for (int r = 0; r < rounds; ++r) {
        int e, m0, row_hi, n0;
        locate(r * G + v, e, m0, row_hi, n0);
        run_tile<MODE, GROUPED, kBN>(p, sm, e, m0, row_hi, n0);
    }
    if (v < tail * split) {
        int e, m0, row_hi, n0;
        locate(rounds * G + v / split, e, m0, row_hi, n0);
        const int piece = v % split;
        if (split == 1) {
            run_tile<MODE, GROUPED, kBN>(p, sm, e, m0, row_hi, n0);
        } else if (split == 2) {
            if (n0 + piece * (kBN / 2) < p.N)
                run_tile<MODE, GROUPED, kBN / 2>(p, sm, e, m0, row_hi, n0 + piece * (kBN / 2));
        } else {
            if (n0 + piece * (kBN / 4) < p.N)
                run_tile<MODE, GROUPED, kBN / 4>(p, sm, e, m0, row_hi, n0 + piece * (kBN / 4));
        }
    }
}

template <int MODE, bool GROUPED>
__global__ __launch_bounds__(kGemmThreads, 1) void k_expert_gemm(GemmArgs p)
{
    __shared__ __align__(16) GemmSmem<GROUPED> sm;
    const int m_tiles = tile_prefix(p, kBM, sm.tiles, sm.wave_sum, true);
    narrow_tiles<MODE, GROUPED>(p, sm, m_tiles);
}

// ---------------------------------------------------------------- 256 x 256 tiles (mxfp8)
//
// The same computation with 256 x 256 output tiles, for mxfp8 with grouped scales.  A K
// step then brings 512 rows of 128 bytes for twice the MACs of a 128 x 256 tile: a third
// fewer line requests per flop, which is what bounds the smaller tile (its copies cannot
// keep its MFMAs busy).  Eight waves of 64 x 128 (two per SIMD), two LDS stages of 64 KB:
// a step's 32 MFMAs per wave, 64 per SIMD (about 2048 cycles), cover the copies of the
// next step, issued right after the barrier that opens the step.
constexpr int kWBM = 256;
constexpr int kWBN = 256;
constexpr int kWWaves = 8;
constexpr int kWThreads = kWWaves * 64;
constexpr int kWWavesM = 4;                      // waves along the rows (64 rows each)
constexpr int kWFragM = kWBM / kWWavesM / 16;    // 4 fragments of 16 rows per wave
constexpr int kWXRuns = kWBM / 8 / kWWaves;      // 4 copy runs of 8 rows per wave and step
constexpr int kWGroupM = 4;                      // row tiles per patch of the tile order

struct WStage {
    uint8_t x[kWBM * kBK];   // 32 KB: activation rows, swizzled 16-byte chunks
    uint8_t w[kWBN * kBK];   // 32 KB: weight rows
};

struct WScales {
    uint32_t x[kWBM][kScaleGroup];
    uint32_t w[kWBN][kScaleGroup];
};

struct WSmem {
    WStage stage[2];
    WScales scale[2];
    uint16_t tiles[kMaxInstances + 1];   // exclusive prefix of row tiles per instance
    int wave_sum[kWWaves];
};

// One 256 x BN output tile (BN 256, or 128 / 64 for the pieces of the last round).
template <int BN>
__device__ __forceinline__ void run_wtile(const GemmArgs &p, WSmem &sm, int e, int m0,
                                          int row_hi, int n0)
{
    constexpr int kFragNT = BN / 2 / 16;          // weight fragments per wave
    constexpr int kWRunsT = BN / 8 / kWWaves;     // weight copy runs per wave and step
    static_assert(kFragNT >= 1 && kWRunsT >= 1, "tile width");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nk = p.K / kBK;
    const int n_groups = nk / kScaleGroup;       // K % 512 == 0 on this path
    const int g = lane >> 4;
    const int r16 = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;     // the wave's 64 x (BN / 2) part
    const int dma_row = lane >> 3;
    const int fr_c0 = ((g ^ (r16 >> 1)) << 4);
    const int fr_c1 = (((g + 4) ^ (r16 >> 1)) << 4);
    const uint8_t *w_e = p.w + (size_t)e * p.N * p.K;

    // copy sources are recomputed at each issue (a handful of integer operations per copy)
    // rather than held in registers; rows past the instance / columns past N are clamped:
    // loaded, multiplied, never stored
    // scale runs of 64 rows / columns: activation run j to wave j (4 runs), weight run j
    // to wave 4 + j (BN / 64 runs)
    const bool x_run = wave < kWBM / 64;
    const int wj = wave - kWBM / 64;
    const bool w_run = wj >= 0 && wj < BN / 64;
    const uint8_t *xsc_src =
        p.a_sc + (size_t)min(m0 + (x_run ? wave : 0) * 64 + lane, row_hi - 1) * p.x_pitch;
    const uint8_t *wsc_src =
        p.w_sc + ((size_t)e * n_groups * p.N + min(n0 + (w_run ? wj : 0) * 64 + lane, p.N - 1)) * 16;
    const size_t wsc_group = (size_t)p.N * 16;

    auto issue_data = [&](int s) {
        const int k0 = s * kBK;
        const uint8_t *base = reinterpret_cast<const uint8_t *>(&sm.stage[s & 1]);
#pragma unroll
        for (int q = 0; q < kWXRuns; ++q) {
            const int r = min(m0 + (wave * kWXRuns + q) * 8 + dma_row, row_hi - 1);
            dma16(p.a + (size_t)r * p.K + k0 + dma_chunk_of(wave * kWXRuns + q, lane),
                  lds_addr(base + offsetof(WStage, x) + (wave * kWXRuns + q) * 1024));
        }
#pragma unroll
        for (int q = 0; q < kWRunsT; ++q) {
            const int n = min(n0 + (wave * kWRunsT + q) * 8 + dma_row, p.N - 1);
            dma16(w_e + (size_t)n * p.K + k0 + dma_chunk_of(wave * kWRunsT + q, lane),
                  lds_addr(base + offsetof(WStage, w) + (wave * kWRunsT + q) * 1024));
        }
    };
    auto issue_scales = [&](int gi) {
        WScales &sc = sm.scale[gi & 1];
        if (x_run)
            dma16(xsc_src + gi * p.x_group, lds_addr(&sc.x[wave * 64][0]));
        if (w_run)
            dma16(wsc_src + gi * wsc_group, lds_addr(&sc.w[wj * 64][0]));
    };

    v4f acc[kFragNT][kWFragM];
#pragma unroll
    for (int i = 0; i < kFragNT; ++i)
#pragma unroll
        for (int j = 0; j < kWFragM; ++j)
            acc[i][j] = v4f{0, 0, 0, 0};

    issue_data(0);
    issue_scales(0);
    // the current group's block exponents (step j of the group in byte j), read at the
    // group's first step (read at the end of the previous group instead, the registers
    // spill)
    uint32_t wsp[kFragNT], xsp[kWFragM];
    auto load_group = [&](const WScales &sc) {
#pragma unroll
        for (int fm = 0; fm < kWFragM; ++fm)
            xsp[fm] = pack_block_exponents(sc.x[wm * (kWBM / kWWavesM) + fm * 16 + r16], g);
#pragma unroll
        for (int fn = 0; fn < kFragNT; ++fn)
            wsp[fn] = pack_block_exponents(sc.w[wn * (BN / 2) + fn * 16 + r16], g);
    };
    for (int s = 0; s < nk; ++s) {
        // step s's copies (and its scale group) have landed for this wave, then for every
        // wave; every wave is also past step s - 1, so its stage and, at a group start,
        // the previous group's scale buffer are free
        wait_vm(0);
        lds_barrier();
        if (s + 1 < nk)
            issue_data(s + 1);
        if (s % kScaleGroup == 0 && s / kScaleGroup + 1 < n_groups)
            issue_scales(s / kScaleGroup + 1);
        if (s % kScaleGroup == 0)
            load_group(sm.scale[(s / kScaleGroup) & 1]);

        const WStage &st = sm.stage[s & 1];
        const int sw = s % kScaleGroup;
        // all activation fragments first (32 registers), then the weight fragments one
        // ahead of the four MFMAs that use each
        v8i xf[kWFragM];
        int xs[kWFragM];
#pragma unroll
        for (int fm = 0; fm < kWFragM; ++fm) {
            const int row = wm * (kWBM / kWWavesM) + fm * 16 + r16;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c0]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.x[row * kBK + fr_c1]);
            xf[fm] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                         (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            xs[fm] = (int)((xsp[fm] >> (8 * sw)) & 0xffu);
        }
        auto read_w = [&](int fn, v8i &wf, int &ws) {
            const int row = wn * (BN / 2) + fn * 16 + r16;
            const u32x4 lo = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c0]);
            const u32x4 hi = *reinterpret_cast<const u32x4 *>(&st.w[row * kBK + fr_c1]);
            wf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            ws = (int)((wsp[fn] >> (8 * sw)) & 0xffu);
        };
        v8i wcur, wnext;
        int scur, snext;
        read_w(0, wcur, scur);
#pragma unroll
        for (int fn = 0; fn < kFragNT; ++fn) {
            if (fn + 1 < kFragNT)
                read_w(fn + 1, wnext, snext);
#pragma unroll
            for (int fm = 0; fm < kWFragM; ++fm)
                acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    wcur, xf[fm], acc[fn][fm], 0, 0, 0, scur, 0, xs[fm]);
            wcur = wnext;
            scur = snext;
        }
    }
    // every wave is done with the rings before the epilogue reuses them
    lds_barrier();

    // epilogue through LDS (the rings and the scale buffers, contiguous): whole rows out
    constexpr int kPitch = BN * 2 + 16;
    static_assert(offsetof(WSmem, scale) == sizeof(WStage) * 2, "contiguous rings");
    static_assert(kWBM * kPitch <= (int)(sizeof(WStage) * 2 + sizeof(WScales) * 2),
                  "output tile fits the rings");
    uint8_t *otile = reinterpret_cast<uint8_t *>(&sm.stage[0]);
#pragma unroll
    for (int fm = 0; fm < kWFragM; ++fm) {
        const int lr = wm * (kWBM / kWWavesM) + fm * 16 + r16;
#pragma unroll
        for (int fn = 0; fn < kFragNT; ++fn) {
            const int lc = wn * (BN / 2) + fn * 16 + 4 * g;
            const v4f d = acc[fn][fm];
            *reinterpret_cast<uint2 *>(otile + lr * kPitch + lc * 2) =
                make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
        }
    }
    lds_barrier();
    constexpr int kRowChunks = BN / 8;
#pragma unroll 4
    for (int c = tid; c < kWBM * kRowChunks; c += kWThreads) {
        const int lr = c / kRowChunks, cc = c % kRowChunks;
        const int r = m0 + lr, n = n0 + cc * 8;
        const uint4 v = *reinterpret_cast<const uint4 *>(otile + lr * kPitch + cc * 16);
        if (r < row_hi && n < p.N)
            *reinterpret_cast<uint4 *>(p.y + (size_t)r * p.N + n) = v;
    }
    lds_barrier();   // the next tile's copies rewrite the rings
}

// The tiles of 256 x 256, walked by the grid like the narrow ones.
__device__ __forceinline__ void wide_tiles(const GemmArgs &p, WSmem &sm, int m_tiles)
{
    const int n_tiles = (p.N + kWBN - 1) / kWBN;
    const int total = m_tiles * n_tiles;

    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int v = (G % kXcds == 0) ? (b % kXcds) * (G / kXcds) + b / kXcds : b;
    auto locate = [&](int t, int &e, int &m0, int &row_hi, int &n0) {
        const int grp = t / (kWGroupM * n_tiles);
        const int tin = t - grp * kWGroupM * n_tiles;
        const int gm = min(kWGroupM, m_tiles - grp * kWGroupM);
        const int tm = grp * kWGroupM + tin % gm;
        const int tn = tin / gm;
        int lo_e = 0, hi_e = p.E;
        while (hi_e - lo_e > 1) {
            const int mid = (lo_e + hi_e) >> 1;
            if (sm.tiles[mid] <= tm)
                lo_e = mid;
            else
                hi_e = mid;
        }
        e = lo_e;
        int row_lo;
        instance_rows(p, e, row_lo, row_hi, nullptr);
        m0 = row_lo + (tm - sm.tiles[e]) * kWBM;
        n0 = tn * kWBN;
    };
    const int rounds = total / G;
    const int tail = total - rounds * G;
    const int split = tail == 0 ? 1 : (G / tail >= 4 ? 4 : (G / tail >= 2 ? 2 : 1));
    for (int r = 0; r < rounds; ++r) {
        int e, m0, row_hi, n0;
        locate(r * G + v, e, m0, row_hi, n0);
        run_wtile<kWBN>(p, sm, e, m0, row_hi, n0);
    }
    if (v < tail * split) {
        int e, m0, row_hi, n0;
        locate(rounds * G + v / split, e, m0, row_hi, n0);
        const int piece = v % split;
        if (split == 1) {
            run_wtile<kWBN>(p, sm, e, m0, row_hi, n0);
        } else if (split == 2) {
            if (n0 + piece * (kWBN / 2) < p.N)
                run_wtile<kWBN / 2>(p, sm, e, m0, row_hi, n0 + piece * (kWBN / 2));
        } else {
            if (n0 + piece * (kWBN / 4) < p.N)
                run_wtile<kWBN / 4>(p, sm, e, m0, row_hi, n0 + piece * (kWBN / 4));
        }
    }
}

// Estimated time of a tiling, in rounds of narrow (128 x 256) tiles: its whole rounds
// times the cost of one, plus the last partial round at the cost of its pieces (the split
// the tile loops use).  Measured on MI355X (H = 7168 -> N = 4096), each tiling forced at
// run time: a round of 256 x 256 tiles costs 1.83-1.93 narrow rounds (one instance of
// 4096 or 8192 rows, four of 2048, sixteen of 512); a last round cut into pieces of a
// quarter (half) of the columns costs about 0.5 (0.67) of a round for narrow tiles and
// 0.5 (0.6) for wide ones (Zipf split of 4096 rows over 8 instances, six of 1500 rows, two
// of 3072).
__device__ __forceinline__ float tiling_cost(int tiles, int G, float round_cost, float quarter,
                                             float half)
{
    const int rounds = tiles / G;
    const int tail = tiles - rounds * G;
    const int split = tail == 0 ? 1 : (G / tail >= 4 ? 4 : (G / tail >= 2 ? 2 : 1));
    const float last = tail == 0 ? 0.0f : (split == 4 ? quarter : split == 2 ? half : 1.0f);
    return round_cost * ((float)rounds + last);
}

// mxfp8 with grouped scales: both tilings' row-tile counts are prefix-summed (each block
// alike, so every block takes the same decision), and the launch runs the one the cost
// model estimates faster.  The two LDS layouts share the block's LDS; their prefix arrays
// do not overlap each other, and the chosen tiling only touches its own layout.
union MxSmem {
    GemmSmem<true> narrow;
    WSmem wide;
};

__global__ __launch_bounds__(kGemmThreads, 1) void k_expert_gemm_mx(GemmArgs p)
{
    static_assert(kWThreads == kGemmThreads, "one block shape for both tilings");
    static_assert(offsetof(WSmem, wave_sum) + sizeof(int) * kWWaves <=
                      offsetof(GemmSmem<true>, tiles),
                  "the two prefix arrays do not overlap");
    __shared__ __align__(16) MxSmem sm;
    const int m_narrow = tile_prefix(p, kBM, sm.narrow.tiles, sm.narrow.wave_sum, true);
    const int m_wide = tile_prefix(p, kWBM, sm.wide.tiles, sm.wide.wave_sum, false);
    const int G = gridDim.x;
    const int n_narrow = m_narrow * ((p.N + kBN - 1) / kBN);
    const int n_wide = m_wide * ((p.N + kWBN - 1) / kWBN);
    if (tiling_cost(n_wide, G, 1.9f, 0.5f, 0.6f) < tiling_cost(n_narrow, G, 1.0f, 0.5f, 0.67f))
        wide_tiles(p, sm.wide, m_wide);
    else
        narrow_tiles<kModeMx, true>(p, sm.narrow, m_narrow);
}

}  // namespace

hipError_t launch_expert_gemm(int quant_mode, const void *a, const void *a_sc,
                              const int32_t *offsets, int E, int rows, const void *w,
                              const void *w_sc, int N, int K, uint16_t *y, int32_t *dev_err,
                              hipStream_t stream)
{
    // mode 5: mxfp8 with the activation exponents group-major, as the dispatch writes them
    // for a buffer of `rows` rows
    const bool x_gm = quant_mode == 5;
    GemmArgs p{static_cast<const uint8_t *>(a), static_cast<const uint8_t *>(a_sc), offsets,
               static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(w_sc), y, dev_err,
               E, rows, N, K, x_gm ? 16 : K / 32, x_gm ? (size_t)16 * rows : (size_t)16};
    if (x_gm)
        quant_mode = kModeMx;
    // Upper bound on row tiles: sum of ceil(rows_e / 128) <= ceil(rows / 128) + E.
    const long m_cap = (rows + kBM - 1) / kBM + E;
    const long tiles_cap = m_cap * ((N + kBN - 1) / kBN);
    // one resident block per CU, walking the tiles grid-stride
    const dim3 grid((unsigned)std::min<long>(tiles_cap, kCus)), block(kGemmThreads);
    // grouped scale copies read 16 bytes per row: K a multiple of 512 (whole groups) and
    // 16-byte aligned scale arrays (the row pitch, 4 bytes per K step, is then a multiple of
    // 16 as well)
    const bool grouped = K % (kBK * kScaleGroup) == 0 &&
                         (reinterpret_cast<uintptr_t>(a_sc) & 15) == 0 &&
                         (reinterpret_cast<uintptr_t>(w_sc) & 15) == 0;
    switch (quant_mode) {
    case kModeMx:
        if (grouped)
            hipLaunchKernelGGL(k_expert_gemm_mx, grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((k_expert_gemm<kModeMx, false>), grid, block, 0, stream, p);
        break;
    case kModeI8Tile:
        if (grouped)
            hipLaunchKernelGGL((k_expert_gemm<kModeI8Tile, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((k_expert_gemm<kModeI8Tile, false>), grid, block, 0, stream, p);
        break;
    case kModeI8Token:
        hipLaunchKernelGGL((k_expert_gemm<kModeI8Token, false>), grid, block, 0, stream, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace moe
