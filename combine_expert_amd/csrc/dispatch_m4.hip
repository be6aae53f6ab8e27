// dispatch_m4.hip -- instantiates the dispatch kernels of quantisation mode 4.
#include "dispatch_impl.h"

namespace moe {

hipError_t launch_mode4(const DispatchArgs &a, int src, bool pe, hipStream_t stream)
{
    return launch_mode<4>(a, src, pe, stream);
}

}  // namespace moe
