// pa_decode_balanced.hip -- instantiations of the partial kernel
// (partial_kernel.h) for the length-balanced schedule: a ragged batch's
// visible pages are split evenly over the waves of each KV head, computed in
// the kernel from the context lengths, so the longest sequences no longer set
// the step time.  Kept in a translation unit of its own so that the two
// schedules' instantiations compile in parallel.
#include "partial_kernel.h"

namespace pa {

hipError_t launch_partial_balanced(int dtype, int head_dim, int group_t, const PartialParams& p,
                                   dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                   LaunchEvents ev)
{
    return launch_partial_any<true>(dtype, head_dim, group_t, p, grid, block, lds, stream, ev);
}

int partial_balanced_waves_per_cu(int dtype, int head_dim, int group_t, bool rotary, int waves,
                                  size_t lds)
{
    return partial_waves_any<true>(dtype, head_dim, group_t, rotary, waves, lds);
}

}  // namespace pa
