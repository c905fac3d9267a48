// Device builders of the paged and tree calls' index inputs
// (TensorRT-Edge-LLM C++ API, "Dflash Runtime Kernels":
// launchDFlashPrepareDeltaMetadata, launchDFlashBuildLinearTreeMetadata).
//
// One thread per output row; both arrays of a row are written by the same
// thread.  The work is a few thousand rows per launch, so the launch itself
// dominates; the kernels only need to be branch-light and bounds-checked.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rkv_launch.hpp"

namespace rkv {

namespace {

constexpr int kMetaBlock = 256;

// Row i = b * width + j is token j of sequence b's delta when
// j < min(deltaLengths[b], width): position old[b] + j (padding if that
// exceeds int32), owner b; otherwise -1 / -1.
__global__ __launch_bounds__(kMetaBlock) void delta_metadata_kernel(
    const int32_t* __restrict__ old_lengths, const int32_t* __restrict__ delta_lengths,
    int32_t width, FastDiv div_width, int32_t* __restrict__ positions,
    int32_t* __restrict__ owners, int32_t rows) {
  const int32_t i = (int32_t)(blockIdx.x * kMetaBlock + threadIdx.x);
  if (i >= rows) return;
  const int32_t b = (int32_t)fast_div((uint32_t)i, div_width);
  const int32_t j = i - b * width;
  const long long pos = (long long)old_lengths[b] + j;
  const bool ok = j < delta_lengths[b] && pos <= INT32_MAX;
  positions[i] = ok ? (int32_t)pos : -1;
  owners[i] = ok ? b : -1;
}

// Linear path of `verify` nodes per sequence: parent i-1 (-1 at the root),
// depth i.
__global__ __launch_bounds__(kMetaBlock) void linear_tree_kernel(int32_t* __restrict__ parents,
                                                                 int32_t* __restrict__ depths,
                                                                 FastDiv div_verify,
                                                                 int32_t verify, int32_t nodes) {
  const int32_t i = (int32_t)(blockIdx.x * kMetaBlock + threadIdx.x);
  if (i >= nodes) return;
  const int32_t node = i - (int32_t)fast_div((uint32_t)i, div_verify) * verify;
  parents[i] = node - 1;
  depths[i] = node;
}

unsigned meta_blocks(int32_t n) { return (unsigned)((n + kMetaBlock - 1) / kMetaBlock); }

}  // namespace

hipError_t launch_delta_metadata(const int32_t* old_lengths, const int32_t* delta_lengths,
                                 int32_t width, int32_t* positions, int32_t* owners,
                                 int32_t rows, hipStream_t stream) {
  hipLaunchKernelGGL(delta_metadata_kernel, dim3(meta_blocks(rows)), dim3(kMetaBlock), 0, stream,
                     old_lengths, delta_lengths, width, make_fastdiv((uint32_t)width), positions,
                     owners, rows);
  return hipGetLastError();
}

hipError_t launch_linear_tree(int32_t* parents, int32_t* depths, int32_t verify, int32_t nodes,
                              hipStream_t stream) {
  hipLaunchKernelGGL(linear_tree_kernel, dim3(meta_blocks(nodes)), dim3(kMetaBlock), 0, stream,
                     parents, depths, make_fastdiv((uint32_t)verify), verify, nodes);
  return hipGetLastError();
}

}  // namespace rkv
