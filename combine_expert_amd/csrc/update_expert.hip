// update_expert.hip -- load-balance mapping and threshold pruning of top-K
// expert ids ("aclnnMoeUpdateExpert": map each token's logical expert ids to
// deployed instances; prune entries by a threshold broadcast over the batch).
//
// One lane per entry f = i*K + k.  The work is a few scattered 4-byte reads
// per entry (the table row of the logical expert), so the kernel is bound by
// latency, not bandwidth (about 3.3 us per launch back to back at Bs=512,
// K=8, however the row is read).  It is kept separate from the dispatch: the
// pages define it as its own call in a fixed sequence before the dispatch,
// and folding the mapping into the dispatch (each of its Bs + 1 blocks maps
// all Bs*K entries from an LDS copy of the table) measured slower than the
// two launches, as did a routing kernel plus a row-scatter kernel.
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kUpdateThreads = 256;

__global__ __launch_bounds__(kUpdateThreads) void k_update_expert(
    const int32_t *__restrict__ ids, const float *__restrict__ scores,
    const int32_t *__restrict__ table, const float *__restrict__ thr,
    const uint8_t *__restrict__ token_mask, int Bs, int K, int n_logical, int F, int n_instances,
    int32_t *__restrict__ out_ids, uint8_t *__restrict__ out_mask, int32_t *__restrict__ dev_err)
{
    const int f = blockIdx.x * kUpdateThreads + threadIdx.x;
    if (f >= Bs * K)
        return;
    const int i = f / K;
    const int k = f - i * K;
    int bits = 0;
    // 1-D mask must be all-true then all-false: a true after a false is illegal
    if (token_mask && k == 0 && i > 0 && token_mask[i] && !token_mask[i - 1])
        bits |= 4;
    bool keep = token_mask == nullptr || token_mask[i] != 0;
    if (scores && thr && scores[f] < thr[k])
        keep = false;
    const int e = ids[f];
    int inst = -1;
    int fail = 0;
    if (e < 0 || e >= n_logical) {
        fail = 1;
    } else {
        const int n = table[(size_t)e * F];
        if (n < 1 || n > F - 1) {
            fail = 2;
        } else {
            inst = table[(size_t)e * F + 1 + i % n];
            if (inst < 0 || inst >= n_instances) {
                fail = 2;
                inst = -1;
            }
        }
    }
    if (fail) {
        if (keep)
            bits |= fail;
        keep = false;
    }
    out_ids[f] = inst;
    out_mask[f] = keep ? 1 : 0;
    if (bits && dev_err)
        atomicOr(dev_err, bits);
}

hipError_t launch_update_expert(const int32_t *ids, const float *scores, const int32_t *table,
                                const float *thr, const uint8_t *token_mask, int Bs, int K,
                                int n_logical, int F, int n_instances, int32_t *out_ids,
                                uint8_t *out_mask, int32_t *dev_err, hipStream_t stream)
{
    const int N = Bs * K;
    const int threads = kUpdateThreads;
    hipLaunchKernelGGL(k_update_expert, dim3((N + threads - 1) / threads), dim3(threads), 0,
                       stream, ids, scores, table, thr, token_mask, Bs, K, n_logical, F,
                       n_instances, out_ids, out_mask, dev_err);
    return hipGetLastError();
}

}  // namespace moe
