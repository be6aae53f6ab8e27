// Host-side driver of the C ABI's argument checking and launch selection
// (api.hip), built with AddressSanitizer and UndefinedBehaviorSanitizer and
// linked against stand-in launchers that record their calls instead of
// enqueuing kernels: no GPU and no kernel is involved.  Every entry point is
// called with valid arguments (the expected launchers must be called with
// the arguments passed through) and with invalid ones (a non-zero status and
// no launcher call).  Pointers are stand-in addresses that nothing reads.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "moe_expert.h"

namespace {
std::vector<std::string> g_calls;
int g_last_Bs = -1, g_last_K = -1, g_last_q = -1;
hipError_t record(const char *name, int Bs, int K, int q)
{
    g_calls.push_back(name);
    g_last_Bs = Bs;
    g_last_K = K;
    g_last_q = q;
    return hipSuccess;
}
}  // namespace

namespace moe {
hipError_t launch_update_expert(const int32_t *, const float *, const int32_t *, const float *,
                                const uint8_t *, int Bs, int K, int, int, int, int32_t *,
                                uint8_t *, int32_t *, hipStream_t)
{
    return record("update_expert", Bs, K, -1);
}
hipError_t launch_dispatch(const uint16_t *, const int32_t *, const uint8_t *, const uint8_t *,
                           int Bs, int, int K, int, int q, int, const float *, int, void *,
                           void *, int32_t *, int32_t *, int32_t *, int32_t *, int32_t *,
                           hipStream_t)
{
    return record("dispatch", Bs, K, q);
}
hipError_t launch_update_dispatch(const uint16_t *, const int32_t *, const float *,
                                  const int32_t *, const float *, const uint8_t *, int, int,
                                  int Bs, int, int K, int, int q, int, const float *, int,
                                  int32_t *, uint8_t *, void *, void *, int32_t *, int32_t *,
                                  int32_t *, int32_t *, int32_t *, hipStream_t)
{
    return record("update_dispatch", Bs, K, q);
}
hipError_t launch_combine(const uint16_t *, const int32_t *, const float *, const uint16_t *,
                          const uint16_t *, const uint16_t *, float, int Bs, int, int K, int,
                          uint16_t *, uint16_t *, float *, int32_t *, hipStream_t)
{
    return record("combine", Bs, K, -1);
}
hipError_t launch_expert_gemm(int q, const void *, const void *, const int32_t *, int, int,
                              const void *, const void *, int, int, uint16_t *, int32_t *,
                              hipStream_t)
{
    return record("expert_gemm", -1, -1, q);
}
hipError_t launch_expert_swiglu(const uint16_t *, const int32_t *, int, int rows, int I,
                                bool group_major, uint8_t *, uint8_t *, uint16_t *, int32_t *,
                                hipStream_t)
{
    return record("expert_swiglu", rows, I, group_major ? MOE_Q_MXFP8_GM : MOE_Q_MXFP8);
}
}  // namespace moe

namespace {
int g_fail = 0;
void expect(bool ok, const char *what)
{
    if (!ok) {
        std::printf("FAIL: %s\n", what);
        ++g_fail;
    }
}
// a 256-byte aligned stand-in address (never dereferenced)
template <typename T> T *P() { return reinterpret_cast<T *>(static_cast<uintptr_t>(0x100000)); }

int dispatch(int Bs, int H, int K, int R, int L, int q, int tile, const float *qs, int qk,
             const uint8_t *token_mask = nullptr)
{
    return moe_dispatch(P<void>(), P<int32_t>(), nullptr, token_mask, Bs, H, K, R, L, q, tile,
                        qs, qk, P<void>(), q ? P<void>() : nullptr, P<int32_t>(), P<int32_t>(),
                        P<int32_t>(), P<int32_t>(), nullptr, nullptr);
}
int fused(int Bs, int K, int nl, int F, int R, int L, int q, int tile, bool outs)
{
    return moe_update_dispatch(P<void>(), P<int32_t>(), nullptr, P<int32_t>(), nullptr, nullptr,
                               Bs, 7168, K, nl, F, R, L, q, tile, nullptr, 0,
                               outs ? P<int32_t>() : nullptr, outs ? P<uint8_t>() : nullptr,
                               P<void>(), q ? P<void>() : nullptr, P<int32_t>(), P<int32_t>(),
                               P<int32_t>(), P<int32_t>(), nullptr, nullptr);
}
}  // namespace

int main()
{
    // valid calls reach their launchers with the sizes passed
    g_calls.clear();
    expect(dispatch(512, 7168, 8, 32, 8, MOE_Q_MXFP8, 0, nullptr, 0) == MOE_OK, "dispatch c3");
    expect(g_calls.size() == 1 && g_calls[0] == "dispatch" && g_last_Bs == 512 && g_last_K == 8 &&
               g_last_q == MOE_Q_MXFP8, "dispatch c3 launcher");
    g_calls.clear();
    std::vector<uint8_t> tm(512, 1);
    expect(dispatch(512, 4096, 8, 8, 8, MOE_Q_INT8_TOKEN, 0, nullptr, 0, tm.data()) == MOE_OK,
           "dispatch with a token mask");
    g_calls.clear();
    expect(dispatch(512, 7168, 8, 32, 8, MOE_Q_STATIC_E4M3, 0, P<float>(), MOE_SCALES_ONE) ==
               MOE_OK, "static E4M3 with one coefficient");
    expect(g_calls.size() == 1 && g_last_q == MOE_Q_STATIC_E4M3, "static E4M3 launcher");
    g_calls.clear();
    // the fused call: one launch up to 4096 entries, two above when the mapped outputs are given
    expect(fused(512, 8, 256, 2, 32, 8, MOE_Q_MXFP8, 0, true) == MOE_OK, "fused c3");
    expect(g_calls.size() == 1 && g_calls[0] == "update_dispatch", "fused c3 is one launch");
    g_calls.clear();
    expect(fused(512, 16, 512, 3, 64, 16, MOE_Q_INT8_TILE, 128, true) == MOE_OK, "fused c4");
    expect(g_calls.size() == 2 && g_calls[0] == "update_expert" && g_calls[1] == "dispatch",
           "fused c4 is mapping then dispatch");
    g_calls.clear();
    expect(fused(512, 16, 512, 3, 64, 16, MOE_Q_INT8_TILE, 128, false) == MOE_OK,
           "fused c4 without mapped outputs");
    expect(g_calls.size() == 1 && g_calls[0] == "update_dispatch",
           "fused c4 without mapped outputs is one launch");
    g_calls.clear();
    expect(moe_update_expert(P<int32_t>(), nullptr, P<int32_t>(), nullptr, nullptr, 512, 8, 256, 2,
                             256, P<int32_t>(), P<uint8_t>(), nullptr, nullptr) == MOE_OK,
           "update_expert");
    expect(moe_combine_add_rmsnorm(P<void>(), P<int32_t>(), P<float>(), P<void>(), P<void>(),
                                   P<void>(), 1e-6f, 512, 7168, 8, MOE_SHARED_PAGE, P<void>(),
                                   P<void>(), P<float>(), nullptr, nullptr) == MOE_OK,
           "combine");
    expect(moe_expert_gemm(P<void>(), P<void>(), P<int32_t>(), 8, 4096, P<void>(), P<void>(), 4096,
                           7168, MOE_Q_MXFP8, P<void>(), nullptr, nullptr) == MOE_OK,
           "expert gemm");
    expect(g_calls.size() == 3 && g_calls[0] == "update_expert" && g_calls[1] == "combine" &&
               g_calls[2] == "expert_gemm", "update / combine / gemm launchers");
    g_calls.clear();
    expect(moe_expert_swiglu(P<void>(), P<int32_t>(), 8, 4096, 2048, MOE_Q_MXFP8_GM, P<void>(),
                             P<void>(), nullptr, nullptr, nullptr) == MOE_OK, "expert swiglu");
    expect(g_calls.size() == 1 && g_calls[0] == "expert_swiglu" && g_last_Bs == 4096 &&
               g_last_K == 2048 && g_last_q == MOE_Q_MXFP8_GM, "expert swiglu launcher");
    g_calls.clear();
    expect(moe_expert_swiglu(P<void>(), P<int32_t>(), 8, 4096, 2000, MOE_Q_MXFP8, P<void>(),
                             P<void>(), nullptr, nullptr, nullptr) == MOE_EINVAL, "swiglu I % 128");
    expect(moe_expert_swiglu(P<void>(), P<int32_t>(), 8, 4096, 2048, MOE_Q_INT8_TOKEN, P<void>(),
                             P<void>(), nullptr, nullptr, nullptr) == MOE_ENOTSUP, "swiglu int8");
    expect(g_calls.empty(), "rejected swiglu calls launch nothing");

    // invalid calls: a status and no launcher
    g_calls.clear();
    expect(dispatch(0, 7168, 8, 32, 8, MOE_Q_MXFP8, 0, nullptr, 0) == MOE_EINVAL, "Bs = 0");
    expect(dispatch(513, 7168, 8, 32, 8, MOE_Q_MXFP8, 0, nullptr, 0) == MOE_EINVAL, "Bs = 513");
    expect(dispatch(512, 7168 + 16, 8, 32, 8, MOE_Q_MXFP8, 0, nullptr, 0) == MOE_EINVAL, "H % 32");
    expect(dispatch(512, 7168, 17, 32, 8, MOE_Q_MXFP8, 0, nullptr, 0) == MOE_EINVAL, "K = 17");
    expect(dispatch(512, 7168, 8, 32, 8, 7, 0, nullptr, 0) == MOE_EINVAL, "quant mode 7");
    expect(dispatch(512, 7168, 8, 32, 8, MOE_Q_INT8_TILE, 96, nullptr, 0) == MOE_ENOTSUP, "tile 96");
    expect(dispatch(512, 7168, 8, 32, 8, MOE_Q_STATIC, 0, nullptr, 0) == MOE_EINVAL,
           "static without scales");
    expect(dispatch(512, 7168, 8, 32, 8, MOE_Q_STATIC_E4M3, 0, P<float>(), MOE_SCALES_ROW) ==
               MOE_EINVAL, "static E4M3 with a scales row");
    expect(fused(512, 8, 256, 1, 32, 8, MOE_Q_MXFP8, 0, true) == MOE_EINVAL, "F = 1");
    expect(moe_combine_add_rmsnorm(P<void>(), P<int32_t>(), P<float>(), nullptr, P<void>(),
                                   P<void>(), -1.0f, 512, 7168, 8, 0, P<void>(), nullptr,
                                   nullptr, nullptr, nullptr) == MOE_EINVAL, "eps < 0");
    expect(moe_expert_gemm(P<void>(), P<void>(), P<int32_t>(), 8, 4096, P<void>(), P<void>(), 100,
                           7168, MOE_Q_MXFP8, P<void>(), nullptr, nullptr) == MOE_EINVAL, "N = 100");
    expect(g_calls.empty(), "no launcher after a rejected call");

    for (int s = -1; s <= 4; ++s)
        expect(std::strlen(moe_status_string(s)) > 0, "status string");
    std::printf(g_fail ? "%d failures\n" : "all passed\n", g_fail);
    return g_fail ? 1 : 0;
}
