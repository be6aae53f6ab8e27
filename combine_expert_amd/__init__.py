"""MI355X (gfx950) MoE expert mapping, token dispatch and combine.

The compute lives in libmoe_expert.so (HIP kernels behind the C ABI in
include/moe_expert.h); `combine_expert_amd.moe` is its ctypes binding and
`combine_expert_amd.workloads` draws seeded synthetic inputs.  Importing the
package itself loads nothing, so the input generators work without the
library; `from combine_expert_amd import moe` fails loudly if it is absent.
"""
__all__ = ["moe", "workloads", "build"]
