// dispatch_m0.hip -- instantiates the dispatch kernels of quantisation mode 0.
#include "dispatch_impl.h"

namespace moe {

hipError_t launch_mode0(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    return launch_mode<0>(a, src, pe, stream);
}

}  // namespace moe
