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
// entry costs one LDS atomic.  Only the token's K offsets are needed, so one
// wave alone scans chunk sums of the low halves; each of its first K lanes
// takes its chunk's prefix by a lane shuffle, adds the counters before its id
// in the chunk, the high half and the token's own earlier duplicates.  That
// wave is an extra one holding no row data, so the row's waves code their
// chunks (codes need no ranks) while it works out the rows; only the stores
// wait for it.  This replaces a serial routing
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
//
// Files: the kernels live in dispatch_impl.h; dispatch_m0.hip .. dispatch_m4.hip
// instantiate them, one quantisation mode each; this file holds the host
// launchers.
#include "dispatch_impl.h"

namespace moe {

// The host has checked the (mode, scales) pairing: modes 0, 4 and 5 take no
// scales, mode 1 takes one coefficient, one row or one row per instance,
// modes 2 and 3 take none or one row per instance.  Mode 5 is mode 4 with the
// exponents group-major: [H/512 rounded up][Bs*K rows][16 bytes].
static hipError_t launch_any(int quant_mode, const DispatchArgs &args, int src,
                             hipStream_t stream)
{
    DispatchArgs a = args;
    const bool gm = quant_mode == 5;
    a.static_e4m3 = quant_mode == 6;  // the static kernel, E4M3 codes
    a.sc_row = gm ? 16 : a.H / 32;
    a.sc_group = gm ? 16 * a.Bs * a.K : 16;
    const bool pe = a.qs_kind == 3;
    switch (quant_mode) {
    case 0: return launch_mode0(a, src, false, stream);
    case 1:
    case 6: return launch_mode1(a, src, pe, stream);
    case 2: return launch_mode2(a, src, pe, stream);
    case 3: return launch_mode3(a, src, pe, stream);
    default: return launch_mode4(a, src, false, stream);
    }
}

hipError_t launch_dispatch(const uint16_t *x, const int32_t *ids, const uint8_t *mask,
                           const uint8_t *token_mask, int Bs, int H, int K, int E,
                           int quant_mode, int tile, const float *qs,
                           int qs_kind, void *expand_x, void *expand_scales, int32_t *counts,
                           int32_t *offsets, int32_t *expand_src, int32_t *assist_dst,
                           int32_t *dev_err, hipStream_t stream)
{
    DispatchArgs a{};
    a.x = x;
    a.ids = ids;
    a.mask = mask;
    a.token_mask = token_mask;
    a.Bs = Bs;
    a.H = H;
    a.K = K;
    a.E = E;
    a.tile = tile;
    a.qs = qs;
    a.qs_kind = qs ? qs_kind : 0;
    a.expand_x = expand_x;
    a.expand_scales = expand_scales;
    a.counts = counts;
    a.offsets = offsets;
    a.expand_src = expand_src;
    a.assist_dst = assist_dst;
    a.dev_err = dev_err;
    return launch_any(quant_mode, a, kRouted, stream);
}

hipError_t launch_update_dispatch(const uint16_t *x, const int32_t *ids, const float *scores,
                                  const int32_t *table, const float *thr,
                                  const uint8_t *token_mask, int n_logical, int F, int Bs, int H,
                                  int K, int E, int quant_mode, int tile, const float *qs,
                                  int qs_kind, int32_t *balanced_ids, uint8_t *balanced_mask,
                                  void *expand_x, void *expand_scales, int32_t *counts,
                                  int32_t *offsets, int32_t *expand_src, int32_t *assist_dst,
                                  int32_t *dev_err, hipStream_t stream)
{
    const bool prune = thr && scores;  // the threshold test needs both
    DispatchArgs a{};
    a.x = x;
    a.ids = ids;
    a.scores = prune ? scores : nullptr;
    a.table = table;
    a.thr = prune ? thr : nullptr;
    a.token_mask = token_mask;
    a.n_logical = n_logical;
    a.F = F;
    a.Bs = Bs;
    a.H = H;
    a.K = K;
    a.E = E;
    a.tile = tile;
    a.qs = qs;
    a.qs_kind = qs ? qs_kind : 0;
    a.expand_x = expand_x;
    a.expand_scales = expand_scales;
    a.counts = counts;
    a.offsets = offsets;
    a.expand_src = expand_src;
    a.assist_dst = assist_dst;
    a.balanced_ids = balanced_ids;
    a.balanced_mask = balanced_mask;
    a.dev_err = dev_err;
    return launch_any(quant_mode, a, prune || token_mask ? kMappedKeep : kMappedPlain, stream);
}

}  // namespace moe
