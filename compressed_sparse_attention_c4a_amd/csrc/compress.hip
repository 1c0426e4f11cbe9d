// compress.hip -- the compressor kernel: one workgroup per (sequence,
// candidate group, job); the routines are in compress_dev.hpp.  Memory-bound
// and tiny next to the indexer and attention.
#include "compress_dev.hpp"

#include <algorithm>
#include <cmath>

namespace csa {

// blockIdx.z selects the job (j0 or j1): both compressors of a CSA layer
// (main KV and index keys) run in one launch.
template <typename T>
__global__ __launch_bounds__(256) void compress_kernel(CompressJob j0, CompressJob j1, const int32_t* __restrict__ pos0,
                                                       int L, int ratio, float eps, double log2_base) {
  __shared__ float red4[4];
  compress_task<T>(blockIdx.z == 0 ? j0 : j1, pos0, blockIdx.y, blockIdx.x, true, L, ratio, eps, log2_base, red4);
}

// Entries with more than 32 slots (C128A): 1024 threads per (sequence,
// candidate group, job), the slots split in four quarters.
template <typename T>
__global__ __launch_bounds__(1024) void compress_kernel_wide(CompressJob j0, CompressJob j1,
                                                             const int32_t* __restrict__ pos0, int L, int ratio,
                                                             float eps, double log2_base) {
  __shared__ float4 red[2048];
  __shared__ float red4[4];
  compress_task_wide<T>(blockIdx.z == 0 ? j0 : j1, pos0, blockIdx.y, blockIdx.x, L, ratio, eps, log2_base, red, red4);
}

}  // namespace csa

namespace csa_host {
using namespace csa;

hipError_t launch_compress(const CompressJob* jobs, int njobs, const int32_t* pos0, int B, int L, int ratio,
                           float eps, float base, int dtype, hipStream_t st) {
  // Candidate groups per sequence: compress_gx (a complete group lies inside the buffer).
  dim3 grid((unsigned)compress_gx(L, ratio), (unsigned)B, (unsigned)njobs);
  const CompressJob j1 = njobs > 1 ? jobs[1] : jobs[0];
  const double l2b = std::log2((double)base);
  const int nslot = std::max(jobs[0].overlap ? 2 * ratio : ratio, j1.overlap ? 2 * ratio : ratio);
  if (nslot > 32) {
    if (dtype == CSA_F32)
      hipLaunchKernelGGL(compress_kernel_wide<float>, grid, dim3(1024), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
    else
      hipLaunchKernelGGL(compress_kernel_wide<bf16>, grid, dim3(1024), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
    return hipGetLastError();
  }
  if (dtype == CSA_F32)
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(256), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
  else
    hipLaunchKernelGGL(compress_kernel<bf16>, grid, dim3(256), 0, st, jobs[0], j1, pos0, L, ratio, eps, l2b);
  return hipGetLastError();
}

}  // namespace csa_host
