// Stand-ins for the kernel-side functions of libgqa, so that the host
// planner and C ABI (gqa_api.cpp) can be built alone -- with the host
// sanitizers, and without any GPU code.  No kernel is ever launched.
#include "gqa_internal.h"

namespace gqa {

hipError_t launch_decode(const Plan&, const Args&, hipStream_t) { return hipErrorNoDevice; }

int resident_groups_per_cu(const Plan&) { return 0; }

hipError_t noalloc_scratch(void** ptr)
{
    *ptr = nullptr;
    return hipErrorNoDevice;
}

hipError_t launch_clear_counters(int32_t*, int, hipStream_t) { return hipErrorNoDevice; }

}  // namespace gqa
