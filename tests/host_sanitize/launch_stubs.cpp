// The library's launch functions replaced by counters, so that the C-ABI
// validation layer (moe_api.hip) can run on the host alone under the
// address and undefined-behaviour sanitizers.  Nothing here touches a GPU
// or dereferences a pointer argument.
#include <hip/hip_runtime.h>

#include "expert_gemm.h"
#include "moe_launch.h"

namespace moe {

int g_launches = 0;

hipError_t launch_route(const void*, const void*, int, const float*, int,
                        int, int, int, int, int32_t*, float*, int32_t*,
                        int32_t*, float*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_plan(const int32_t*, int, int, int, int, int32_t*,
                       int32_t*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dispatch(const void*, int, int, int, const int32_t*, int,
                           int, const int32_t*, const int32_t*, const void*,
                           int, void*, size_t, float*, int32_t*, int32_t*,
                           hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dispatch_noalloc(const void*, int, int, int,
                                   const int32_t*, int, int, int,
                                   const int32_t*, const int32_t*, int, void*,
                                   size_t, float*, int32_t*, int32_t*,
                                   hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_route_dispatch(const void*, const void*, int, const float*,
                                 int, int, int, int, int, int32_t*, float*,
                                 int32_t*, int32_t*, float*, void*, int,
                                 void*, size_t, float*, int32_t*, int32_t*,
                                 hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_route_dispatch_one_launch(const void*, const void*,
                                            const float*, int, int, int, int,
                                            int, int32_t*, float*, int32_t*,
                                            int32_t*, float*, void*, int,
                                            void*, size_t, float*, int32_t*,
                                            int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_plan_dispatch_small(const void*, int, int, int,
                                      const int32_t*, int, int, int,
                                      int32_t*, int32_t*, int, void*, size_t,
                                      float*, int32_t*, int32_t*,
                                      hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine(const void*, int, int, size_t, const int32_t*,
                          const float*, int, int, const void*, const void*,
                          void*, void*, void*, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_farskip_aux(const void*, const void*, void*, int, int,
                              hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine_backward(const void*, const void*, int, int,
                                   size_t, const int32_t*, const float*, int,
                                   int, void*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fixture(const void*, int, const float*, int,
                          const int32_t*, const int32_t*, int, const float*,
                          size_t, void*, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_expert_gemm(const void*, const float*, int, size_t,
                              const int32_t*, const int32_t*, int,
                              const void*, const float*, int, void*, int,
                              void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace moe
