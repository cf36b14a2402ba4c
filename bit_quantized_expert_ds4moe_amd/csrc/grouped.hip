// grouped.hip -- token->expert permutation launch and the batched
// (several tokens per expert) expert FFN path (gfx950).
#include "dev_common.h"

namespace ds4 {

__global__ __launch_bounds__(1024) void k_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                                  int32_t* offsets, int32_t* perm, int32_t* inv,
                                                  uint32_t* status);

inline ds4moe_status launch_permute(const int32_t* ids, int n, int E, int32_t* counts,
                                    int32_t* offsets, int32_t* perm, int32_t* inv,
                                    uint32_t* status, hipStream_t st) {
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  size_t lds = (size_t)n2 * 4;
  if (hipFuncSetAttribute((const void*)k_permute, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds) != hipSuccess)
    return DS4MOE_EDEVICE;
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), lds, st, ids, n, E, counts, offsets, perm, inv,
                     status);
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_EDEVICE;
}

inline bool grouped_eligible(const ds4moe_shape&, const ds4moe_experts&, const ds4moe_experts*,
                             const void*, int32_t, int32_t) {
  return false;
}

inline ds4moe_status run_grouped(const ds4moe_shape&, const ds4moe_experts&, const ds4moe_experts*,
                                 const uint16_t*, int32_t, const int32_t*, const float*, float*,
                                 float*, int32_t*, int32_t*, uint16_t*, float*, uint32_t*,
                                 hipStream_t) {
  return DS4MOE_EUNSUPPORTED;
}

}  // namespace ds4
