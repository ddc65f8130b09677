// kernels_m1.hip -- the persistent kernel for a single slot (its own
// translation unit so the kernel variants compile in parallel).
#include "kernels.h"

namespace mk {

hipError_t launch_persistent_m1(const DevPlan *d, const CallArgs &ca, int grid, hipStream_t s) {
  void *args[] = {(void *)&d, (void *)&ca};
  // all workers must be resident at once (each may wait on any other), which
  // a cooperative launch guarantees or refuses
  return hipLaunchCooperativeKernel((const void *)mk_persistent_kernel<1>, dim3(grid),
                                    dim3(kThreads), args, 0, s);
}

}  // namespace mk
