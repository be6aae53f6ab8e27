// dispatch_m2.hip -- instantiates the dispatch kernels of quantisation mode 2.
#include "dispatch_impl.h"

namespace moe {

hipError_t launch_mode2(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    return launch_mode<2>(a, src, pe, stream);
}

}  // namespace moe
