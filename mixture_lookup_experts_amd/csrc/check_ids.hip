// Device-side check of token ids (MoLE article, inference section: a token's
// table rows are found by direct addressing on its id, so an id outside
// [0, V) would address memory outside the table).  The combines do not check
// device-resident ids; a caller that wants the check runs this kernel first.
#include "mole_device.hpp"
#include "mole_kernels.hpp"

namespace mole {

__global__ __launch_bounds__(256) void check_ids_kernel(const int64_t* __restrict__ ids, int64_t T, int64_t V,
                                                        int* __restrict__ count) {
  int bad = 0;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t id = ids[t];
    bad += (id < 0 || id >= V) ? 1 : 0;
  }
  // wavefront sum, one atomic per wavefront that saw a bad id
#pragma unroll
  for (int m = kWave / 2; m >= 1; m >>= 1) bad += __shfl_xor(bad, m, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0 && bad != 0) atomicAdd(count, bad);
}

hipError_t launch_check_ids(const int64_t* ids, int64_t T, int64_t V, int* count, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int64_t blocks = (T + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(check_ids_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ids, T, V, count);
  return hipGetLastError();
}

}  // namespace mole
