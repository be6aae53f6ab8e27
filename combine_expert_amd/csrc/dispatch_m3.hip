// dispatch_m3.hip -- instantiates the dispatch kernels of quantisation mode 3.
#include "dispatch_impl.h"

namespace moe {

hipError_t launch_mode3(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    return launch_mode<3>(a, src, pe, stream);
}

}  // namespace moe
