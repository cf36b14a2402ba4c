/*
 * ds4gen_fill.hip -- device fill of quantised expert tensors from the same
 * counter-based stream as the host generator (ds4gen.h), so that tens of GB
 * of synthetic 2-bit blocks can be written straight into HBM.  Each thread
 * builds one block in LDS; the workgroup then copies its LDS tile to global
 * memory with coalesced 4-byte stores.  Bit-identical to ds4gen_blocks().
 *
 * Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off -fPIC -shared
 */
#include <hip/hip_runtime.h>

#include "ds4gen.h"

#define FILL_THREADS 256
#define FILL_MAX_BYTES 144

template <int QT, int BB>
__global__ __launch_bounds__(FILL_THREADS) void gen_fill_kernel(uint64_t key, uint64_t first,
                                                                 uint64_t n, uint8_t* out) {
  __shared__ __align__(16) uint8_t tile[FILL_THREADS * BB];
  uint64_t b0 = (uint64_t)blockIdx.x * FILL_THREADS;
  uint64_t nb = n - b0 < (uint64_t)FILL_THREADS ? n - b0 : (uint64_t)FILL_THREADS;
  if ((uint64_t)threadIdx.x < nb) {
    uint8_t blk[BB];
    gen_block(QT, key, first + b0 + threadIdx.x, blk);
    for (int i = 0; i < BB; i++) tile[threadIdx.x * BB + i] = blk[i];
  }
  __syncthreads();
  uint64_t nbytes = nb * BB;
  uint8_t* dst = out + b0 * BB;
  /* The tile start is a multiple of BB*256 bytes from a 4-aligned base. */
  uint32_t* dst4 = reinterpret_cast<uint32_t*>(dst);
  const uint32_t* src4 = reinterpret_cast<const uint32_t*>(tile);
  uint64_t nw = nbytes / 4;
  for (uint64_t w = threadIdx.x; w < nw; w += FILL_THREADS) dst4[w] = src4[w];
  for (uint64_t i = nw * 4 + threadIdx.x; i < nbytes; i += FILL_THREADS) dst[i] = tile[i];
}

extern "C" __attribute__((visibility("default"))) int ds4gen_dev_blocks(
    int qtype, uint64_t seed, uint64_t stream, uint64_t first, uint64_t n, void* dev_out,
    hipStream_t st) {
  if (n == 0) return 0;
  if (((uintptr_t)dev_out & 3u) != 0) return -1;
  uint64_t key = gen_key(seed, stream);
  uint64_t grid = (n + FILL_THREADS - 1) / FILL_THREADS;
  if (grid > 0x7FFFFFFFULL) return -1;
  uint8_t* o = static_cast<uint8_t*>(dev_out);
  if (qtype == DS4GEN_Q2_K)
    hipLaunchKernelGGL((gen_fill_kernel<DS4GEN_Q2_K, DS4GEN_Q2K_BYTES>), dim3((unsigned)grid),
                       dim3(FILL_THREADS), 0, st, key, first, n, o);
  else if (qtype == DS4GEN_Q2_K_ZM)
    hipLaunchKernelGGL((gen_fill_kernel<DS4GEN_Q2_K_ZM, DS4GEN_Q2K_BYTES>), dim3((unsigned)grid),
                       dim3(FILL_THREADS), 0, st, key, first, n, o);
  else if (qtype == DS4GEN_IQ2_XXS)
    hipLaunchKernelGGL((gen_fill_kernel<DS4GEN_IQ2_XXS, DS4GEN_IQ2_BYTES>), dim3((unsigned)grid),
                       dim3(FILL_THREADS), 0, st, key, first, n, o);
  else if (qtype == DS4GEN_Q8_0)
    hipLaunchKernelGGL((gen_fill_kernel<DS4GEN_Q8_0, DS4GEN_Q80_BYTES>), dim3((unsigned)grid),
                       dim3(FILL_THREADS), 0, st, key, first, n, o);
  else if (qtype == DS4GEN_Q4_K)
    hipLaunchKernelGGL((gen_fill_kernel<DS4GEN_Q4_K, DS4GEN_Q4K_BYTES>), dim3((unsigned)grid),
                       dim3(FILL_THREADS), 0, st, key, first, n, o);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
