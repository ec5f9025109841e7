// Weight packing: plain row-major [G][R][C] matrices into the tiled layout
// the kernels read (layout described in moe_internal.h).  Done once when the
// weights are loaded.  A thread moves 8 consecutive elements of one row,
// which stay consecutive in the packed layout (8 divides the step and the
// strip widths).
#include "moe_internal.h"

namespace moe {

template <typename V>
__global__ void pack_kernel(const V* __restrict__ src, long groups, int R, int C, int neuron_major,
                            V* __restrict__ dst) {
  const int cv = C / 8;  // 8-element vectors per row
  const long n = groups * R * cv;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const long g = i / ((long)R * cv);
    const long rem = i - g * R * cv;
    const int r = (int)(rem / cv), c = (int)(rem - (long)r * cv) * 8;
    const long o = neuron_major ? packed_neuron_major_offset(r, c, R, C) : packed_out_in_offset(r, c, R, C);
    dst[(g * R * C + o) / 8] = src[i];
  }
}

struct Vec4 { uint32_t v; };
struct Vec8 { uint2 v; };
struct Vec16 { uint4 v; };
struct Vec32 { uint4 a, b; };

hipError_t launch_pack_weight(const void* src, int elem_bytes, int neuron_major, int G, int R, int C,
                              void* dst, hipStream_t s) {
  const long n = (long)G * R * (C / 8);
  if (n == 0) return hipSuccess;
  int grid = (int)((n + 255) / 256);
  if (grid > 65536) grid = 65536;
  if (elem_bytes == 0)  // MXFP4 codes: 8 elements are 4 bytes
    hipLaunchKernelGGL(pack_kernel<Vec4>, dim3(grid), dim3(256), 0, s, (const Vec4*)src, (long)G, R, C,
                       neuron_major, (Vec4*)dst);
  else if (elem_bytes == 1)
    hipLaunchKernelGGL(pack_kernel<Vec8>, dim3(grid), dim3(256), 0, s, (const Vec8*)src, (long)G, R, C,
                       neuron_major, (Vec8*)dst);
  else if (elem_bytes == 2)
    hipLaunchKernelGGL(pack_kernel<Vec16>, dim3(grid), dim3(256), 0, s, (const Vec16*)src, (long)G, R, C,
                       neuron_major, (Vec16*)dst);
  else
    hipLaunchKernelGGL(pack_kernel<Vec32>, dim3(grid), dim3(256), 0, s, (const Vec32*)src, (long)G, R, C,
                       neuron_major, (Vec32*)dst);
  return hipGetLastError();
}

}  // namespace moe
