// dispatch_m1.hip -- instantiates the dispatch kernels of quantisation mode 1.
#include "dispatch_impl.h"

namespace moe {

hipError_t launch_mode1(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    return launch_mode<1>(a, src, pe, stream);
}

}  // namespace moe
