// api.hip -- C ABI of libmoe_expert.so (declared in include/moe_expert.h).
//
// Each entry point checks every host-visible argument (the pages' first-phase
// parameter check) and returns a non-zero status before anything is
// enqueued; otherwise it enqueues its kernels on the caller's stream and
// returns.  Nothing is allocated, synchronised or kept between calls.
#include <math.h>
#include <stdint.h>

#include "kernels.h"
#include "moe_expert.h"

namespace {

constexpr int kMaxBs = 512;       // combine / update-expert pages: 0 < Bs <= 512
constexpr int kMaxK = 16;         // 0 < K <= 16
constexpr int kMinH = 1024;       // combine page: H in [1024, 8192]
constexpr int kMaxH = 8192;
constexpr int kMaxExperts = 1024; // update-expert page: at most 1024 instances
constexpr int kMaxGemmDim = 16384; // expert GEMM: H and N (multiples of 128)
constexpr int kMaxGemmRows = 1 << 22; // expert GEMM: row tiles counted in 16 bits on the device
constexpr int kMaxStagedTable = 8192;  // table words a fused dispatch block stages in LDS (32 KB)
constexpr int kFusedMaxEntries = 4096; // moe_update_dispatch: one launch up to this many entries

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool bad_bs_k(int Bs, int K) { return Bs <= 0 || Bs > kMaxBs || K <= 0 || K > kMaxK; }

bool bad_h(int H) { return H < kMinH || H > kMaxH || H % 32 != 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

}  // namespace

extern "C" {

const char *moe_status_string(int status)
{
    switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: argument out of range, NULL or misaligned";
    case MOE_ENOTSUP: return "MOE_ENOTSUP: option not implemented";
    case MOE_ELAUNCH: return "MOE_ELAUNCH: kernel launch failed";
    default: return "unknown moe_status";
    }
}

int moe_update_expert(const int32_t *expert_ids, const float *expert_scales,
                      const int32_t *table, const float *prune_thr, const uint8_t *token_mask,
                      int Bs, int K, int n_logical, int F, int n_instances,
                      int32_t *balanced_ids, uint8_t *balanced_mask, int32_t *dev_err,
                      void *stream)
{
    if (!expert_ids || !table || !balanced_ids || !balanced_mask)
        return MOE_EINVAL;
    if (bad_bs_k(Bs, K) || n_logical <= 0 || n_logical > kMaxExperts || K > n_logical)
        return MOE_EINVAL;
    if (F < 2 || F > n_logical + 1 || n_instances <= 0 || n_instances > kMaxExperts)
        return MOE_EINVAL;
    if (!aligned(expert_ids, 4) || !aligned(table, 4) || !aligned(balanced_ids, 4) ||
        (expert_scales && !aligned(expert_scales, 4)) || (prune_thr && !aligned(prune_thr, 4)) ||
        (dev_err && !aligned(dev_err, 4)))
        return MOE_EINVAL;
    return from_hip(moe::launch_update_expert(expert_ids, expert_scales, table, prune_thr,
                                              token_mask, Bs, K, n_logical, F, n_instances,
                                              balanced_ids, balanced_mask, dev_err,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks shared by moe_dispatch and moe_update_dispatch.
int check_dispatch(const void *x, const int32_t *ids, int Bs, int H, int K, int n_ranks,
                   int local_experts, int quant_mode, int tile, const float *qs, int qs_kind,
                   const void *expand_x, const void *expand_scales, const int32_t *counts,
                   const int32_t *offsets, const int32_t *expand_src,
                   const int32_t *assist_dst, const int32_t *dev_err)
{
    if (!x || !ids || !expand_x || !counts || !offsets || !expand_src || !assist_dst)
        return MOE_EINVAL;
    if (bad_bs_k(Bs, K) || bad_h(H) || n_ranks < 1 || local_experts < 1)
        return MOE_EINVAL;
    const long long E = (long long)n_ranks * local_experts;
    if (E > kMaxExperts || K > E)
        return MOE_EINVAL;
    // the scales input: its shape must be one the mode takes (quantMode
    // constraints of the dispatch page), and present iff named
    if (qs_kind < MOE_SCALES_NONE || qs_kind > MOE_SCALES_EXPERT ||
        (qs_kind == MOE_SCALES_NONE) != (qs == nullptr))
        return MOE_EINVAL;
    if ((qs_kind == MOE_SCALES_ROW || qs_kind == MOE_SCALES_EXPERT) ? !aligned(qs, 16)
                                                                     : (qs && !aligned(qs, 4)))
        return MOE_EINVAL;
    switch (quant_mode) {
    case MOE_Q_NONE:
    case MOE_Q_MXFP8:
    case MOE_Q_MXFP8_GM:
        if (qs_kind != MOE_SCALES_NONE)
            return MOE_EINVAL;
        break;
    case MOE_Q_STATIC:
        if (qs_kind == MOE_SCALES_NONE)
            return MOE_EINVAL;
        break;
    case MOE_Q_STATIC_E4M3:
        if (qs_kind != MOE_SCALES_ONE)
            return MOE_EINVAL;
        break;
    case MOE_Q_INT8_TOKEN:
    case MOE_Q_INT8_TILE:
        if (qs_kind != MOE_SCALES_NONE && qs_kind != MOE_SCALES_EXPERT)
            return MOE_EINVAL;
        break;
    default:
        return MOE_EINVAL;
    }
    switch (quant_mode) {
    case MOE_Q_NONE:
    case MOE_Q_STATIC:
    case MOE_Q_STATIC_E4M3:
        break;
    case MOE_Q_INT8_TOKEN:
    case MOE_Q_MXFP8:
    case MOE_Q_MXFP8_GM:
        if (!expand_scales)
            return MOE_EINVAL;
        break;
    case MOE_Q_INT8_TILE:
        if (!expand_scales || tile <= 0)
            return MOE_EINVAL;
        if (tile < 16 || tile > 1024 || (tile & (tile - 1)) != 0)
            return MOE_ENOTSUP;
        break;
    default:
        return MOE_EINVAL;
    }
    if (!aligned(x, 16) || !aligned(expand_x, 16) || !aligned(ids, 16) || !aligned(counts, 4) ||
        !aligned(offsets, 4) || !aligned(expand_src, 4) || !aligned(assist_dst, 4) ||
        (dev_err && !aligned(dev_err, 4)) ||
        ((quant_mode == MOE_Q_INT8_TOKEN || quant_mode == MOE_Q_INT8_TILE) &&
         !aligned(expand_scales, 4)))
        return MOE_EINVAL;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_dispatch(const void *x, const int32_t *expert_ids, const uint8_t *active_mask,
                 const uint8_t *token_mask, int Bs,
                 int H, int K, int n_ranks, int local_experts, int quant_mode, int tile,
                 const float *quant_scales, int quant_scales_kind, void *expand_x,
                 void *expand_scales, int32_t *expert_counts, int32_t *expert_offsets,
                 int32_t *expand_src, int32_t *assist_dst, int32_t *dev_err, void *stream)
{
    const int rc = check_dispatch(x, expert_ids, Bs, H, K, n_ranks, local_experts, quant_mode,
                                  tile, quant_scales, quant_scales_kind, expand_x, expand_scales,
                                  expert_counts, expert_offsets, expand_src, assist_dst, dev_err);
    if (rc != MOE_OK)
        return rc;
    if (active_mask && !aligned(active_mask, 4))
        return MOE_EINVAL;
    return from_hip(moe::launch_dispatch(
        static_cast<const uint16_t *>(x), expert_ids, active_mask, token_mask, Bs, H, K,
        n_ranks * local_experts, quant_mode, quant_mode == MOE_Q_INT8_TILE ? tile : 0,
        quant_scales, quant_scales_kind, expand_x, expand_scales, expert_counts, expert_offsets,
        expand_src, assist_dst, dev_err, static_cast<hipStream_t>(stream)));
}

int moe_update_dispatch(const void *x, const int32_t *expert_ids, const float *expert_scales,
                        const int32_t *table, const float *prune_thr, const uint8_t *token_mask,
                        int Bs, int H, int K, int n_logical, int F, int n_ranks,
                        int local_experts, int quant_mode, int tile, const float *quant_scales,
                        int quant_scales_kind, int32_t *balanced_ids, uint8_t *balanced_mask,
                        void *expand_x, void *expand_scales, int32_t *expert_counts,
                        int32_t *expert_offsets, int32_t *expand_src, int32_t *assist_dst,
                        int32_t *dev_err, void *stream)
{
    const int rc = check_dispatch(x, expert_ids, Bs, H, K, n_ranks, local_experts, quant_mode,
                                  tile, quant_scales, quant_scales_kind, expand_x, expand_scales,
                                  expert_counts, expert_offsets, expand_src, assist_dst, dev_err);
    if (rc != MOE_OK)
        return rc;
    if (!table || n_logical <= 0 || n_logical > kMaxExperts || K > n_logical || F < 2 ||
        F > n_logical + 1)
        return MOE_EINVAL;
    if ((long long)n_logical * F > kMaxStagedTable)
        return MOE_ENOTSUP;
    const bool prune = expert_scales && prune_thr;
    if (!aligned(table, 4) || (prune && !aligned(expert_scales, 16)) ||
        (prune_thr && !aligned(prune_thr, 4)) || (balanced_ids && !aligned(balanced_ids, 4)))
        return MOE_EINVAL;
    // Every block of the single launch maps all Bs*K entries (that is what lets it skip a
    // second launch), which costs more than the second launch beyond about 4096 entries
    // (measured: 4096 entries 10.2 us fused against 3.2 + 8.6 us; 8192 with pruning 17.2
    // against 3.0 + 11.0).  Past that size, when the caller provides the mapped ids and mask,
    // the mapping and the dispatch run as two launches, with the same results.
    if (Bs * K > kFusedMaxEntries && balanced_ids && balanced_mask &&
        aligned(balanced_mask, 4)) {
        const hipError_t e = moe::launch_update_expert(
            expert_ids, expert_scales, table, prune_thr, token_mask, Bs, K, n_logical, F,
            n_ranks * local_experts, balanced_ids, balanced_mask, dev_err,
            static_cast<hipStream_t>(stream));
        if (e != hipSuccess)
            return from_hip(e);
        return from_hip(moe::launch_dispatch(
            static_cast<const uint16_t *>(x), balanced_ids, balanced_mask, nullptr, Bs, H, K,
            n_ranks * local_experts, quant_mode, quant_mode == MOE_Q_INT8_TILE ? tile : 0,
            quant_scales, quant_scales_kind, expand_x, expand_scales, expert_counts,
            expert_offsets, expand_src, assist_dst, dev_err, static_cast<hipStream_t>(stream)));
    }
    return from_hip(moe::launch_update_dispatch(
        static_cast<const uint16_t *>(x), expert_ids, expert_scales, table, prune_thr,
        token_mask, n_logical, F, Bs, H, K, n_ranks * local_experts, quant_mode,
        quant_mode == MOE_Q_INT8_TILE ? tile : 0, quant_scales, quant_scales_kind,
        balanced_ids, balanced_mask, expand_x,
        expand_scales, expert_counts, expert_offsets, expand_src, assist_dst, dev_err,
        static_cast<hipStream_t>(stream)));
}

int moe_combine_add_rmsnorm(const void *expert_out, const int32_t *assist_dst,
                            const float *expert_scales, const void *shared_x,
                            const void *residual_x, const void *gamma, float eps, int Bs,
                            int H, int K, int shared_mode, void *y, void *x_out, float *rstd,
                            int32_t *dev_err, void *stream)
{
    if (!expert_out || !assist_dst || !expert_scales || !residual_x || !gamma || !y)
        return MOE_EINVAL;
    if (bad_bs_k(Bs, K) || bad_h(H))
        return MOE_EINVAL;
    if (!(eps >= 0.0f) || !isfinite(eps) || (shared_mode != MOE_SHARED_PAGE &&
                                            shared_mode != MOE_SHARED_ADD))
        return MOE_EINVAL;
    if (!aligned(expert_out, 16) || !aligned(residual_x, 16) || !aligned(gamma, 16) ||
        !aligned(y, 16) || (shared_x && !aligned(shared_x, 16)) ||
        (x_out && !aligned(x_out, 16)) || !aligned(assist_dst, 4) ||
        !aligned(expert_scales, 4) || (rstd && !aligned(rstd, 4)) ||
        (dev_err && !aligned(dev_err, 4)))
        return MOE_EINVAL;
    return from_hip(moe::launch_combine(
        static_cast<const uint16_t *>(expert_out), assist_dst, expert_scales,
        static_cast<const uint16_t *>(shared_x), static_cast<const uint16_t *>(residual_x),
        static_cast<const uint16_t *>(gamma), eps, Bs, H, K, shared_mode,
        static_cast<uint16_t *>(y), static_cast<uint16_t *>(x_out), rstd, dev_err,
        static_cast<hipStream_t>(stream)));
}

int moe_expert_gemm(const void *expand_x, const void *expand_scales,
                    const int32_t *expert_offsets, int n_instances, int rows,
                    const void *weights, const void *weight_scales, int N, int H,
                    int quant_mode, void *y, int32_t *dev_err, void *stream)
{
    if (!expand_x || !expand_scales || !expert_offsets || !weights || !weight_scales || !y)
        return MOE_EINVAL;
    if (n_instances < 1 || n_instances > kMaxExperts || rows < 0 || rows > kMaxGemmRows)
        return MOE_EINVAL;
    if (H < 128 || H > kMaxGemmDim || H % 128 != 0 || N < 128 || N > kMaxGemmDim ||
        N % 128 != 0)
        return MOE_EINVAL;
    if (quant_mode < MOE_Q_NONE || quant_mode > MOE_Q_STATIC_E4M3)
        return MOE_EINVAL;
    if (quant_mode != MOE_Q_MXFP8 && quant_mode != MOE_Q_MXFP8_GM &&
        quant_mode != MOE_Q_INT8_TOKEN && quant_mode != MOE_Q_INT8_TILE)
        return MOE_ENOTSUP;
    if (!aligned(expand_x, 16) || !aligned(weights, 16) || !aligned(y, 16) ||
        !aligned(expand_scales, 4) || !aligned(weight_scales, 4) ||
        !aligned(expert_offsets, 4) || (dev_err && !aligned(dev_err, 4)))
        return MOE_EINVAL;
    return from_hip(moe::launch_expert_gemm(quant_mode, expand_x, expand_scales, expert_offsets,
                                            n_instances, rows, weights, weight_scales, N, H,
                                            static_cast<uint16_t *>(y), dev_err,
                                            static_cast<hipStream_t>(stream)));
}

int moe_expert_swiglu(const void *y1, const int32_t *expert_offsets, int n_instances, int rows,
                      int I, int quant_mode, void *act_codes, void *act_scales, void *act,
                      int32_t *dev_err, void *stream)
{
    if (!y1 || !expert_offsets || !act_codes || !act_scales)
        return MOE_EINVAL;
    if (n_instances < 1 || n_instances > kMaxExperts || rows < 0 || rows > kMaxGemmRows)
        return MOE_EINVAL;
    if (I < 128 || I > kMaxGemmDim / 2 || I % 128 != 0)
        return MOE_EINVAL;
    if (quant_mode < MOE_Q_NONE || quant_mode > MOE_Q_STATIC_E4M3)
        return MOE_EINVAL;
    if (quant_mode != MOE_Q_MXFP8 && quant_mode != MOE_Q_MXFP8_GM)
        return MOE_ENOTSUP;
    if (!aligned(y1, 16) || !aligned(act_codes, 16) || (act && !aligned(act, 16)) ||
        !aligned(expert_offsets, 4) || (dev_err && !aligned(dev_err, 4)))
        return MOE_EINVAL;
    return from_hip(moe::launch_expert_swiglu(
        static_cast<const uint16_t *>(y1), expert_offsets, n_instances, rows, I,
        quant_mode == MOE_Q_MXFP8_GM, static_cast<uint8_t *>(act_codes),
        static_cast<uint8_t *>(act_scales), static_cast<uint16_t *>(act), dev_err,
        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
