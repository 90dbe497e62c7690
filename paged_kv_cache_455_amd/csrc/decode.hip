// Paged decode attention: split-context online softmax + second-pass merge
// (the device templates and their description are in decode_impl.h).
#include <stdlib.h>

#include "decode_impl.h"

namespace pa {

template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(kDecodeWaves *kWave) void pa_decode_stream_kernel(DecodeArgs a) {
  if constexpr (Q8Geom<KV, D, G>::kOn)
    decode_stream_q8<KV, QT>(a);
  else
    decode_stream<KV, QT, D, G>(a);
}

// One wave per (sequence, query head); four per workgroup.
template <int QT, int D>
__global__ __launch_bounds__(4 * kWave) void pa_decode_stream_merge_kernel(DecodeArgs a) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // s * num_q_heads + hq
  if (row >= a.num_seqs * a.num_q_heads) return;
  merge_stream<QT, D>(a, row / a.num_q_heads, row % a.num_q_heads, threadIdx.x % kWave);
}

// ---------------------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------------------
// Workgroups of one balanced-split kernel instantiation that fit on the device at once.
template <int KV, int QT, int D, int G>
static int resident_groups() {
  static int cached = 0;  // one value per instantiation
  if (cached > 0) return cached;
  auto kernel = pa_decode_stream_kernel<KV, QT, D, G>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeWaves * kWave, 0) !=
      hipSuccess)
    return 0;
  cached = cus * (per_cu > 0 ? per_cu : 1);
  return cached;
}

template <int KV, int QT, int D, int G>
static hipError_t launch_stream_kg(DecodeArgs a, int num_seqs, hipStream_t st) {
  auto kern = pa_decode_stream_kernel<KV, QT, D, G>;
  static const int oversub = [] {
    const char *v = getenv("PA_STREAM_OVERSUB");
    const int x = v ? atoi(v) : 0;
    return x > 0 ? x : 1;
  }();
  const int groups = resident_groups<KV, QT, D, G>() * oversub;
  if (groups <= 0) return hipErrorInvalidDeviceFunction;
  a.num_waves = groups * kDecodeWaves;
  hipLaunchKernelGGL(kern, dim3(groups), dim3(kDecodeWaves * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid((num_seqs * a.num_q_heads + 3) / 4);
  hipLaunchKernelGGL((pa_decode_stream_merge_kernel<QT, D>), mgrid, dim3(4 * kWave), 0, st, a);
  return hipGetLastError();
}

template <int KV, int QT, int D>
static hipError_t launch_stream_g(const DecodeArgs &a, int G, int num_seqs, hipStream_t st) {
  switch (G) {
    case 1: return launch_stream_kg<KV, QT, D, 1>(a, num_seqs, st);
    case 2: return launch_stream_kg<KV, QT, D, 2>(a, num_seqs, st);
    case 4: return launch_stream_kg<KV, QT, D, 4>(a, num_seqs, st);
    case 8: return launch_stream_kg<KV, QT, D, 8>(a, num_seqs, st);
  }
  return hipErrorInvalidValue;
}

template <int KV, int QT>
static hipError_t launch_stream_d(const DecodeArgs &a, int D, int G, int num_seqs, hipStream_t st) {
  if (D == 64) return launch_stream_g<KV, QT, 64>(a, G, num_seqs, st);
  if (D == 128) return launch_stream_g<KV, QT, 128>(a, G, num_seqs, st);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_stream(const DecodeArgs &a, int kv_dtype, int q_dtype, int head_dim,
                                int group, int num_seqs, hipStream_t st) {
  switch (kv_dtype) {
    case PA_F32: return launch_stream_d<PA_F32, PA_F32>(a, head_dim, group, num_seqs, st);
    case PA_F16: return launch_stream_d<PA_F16, PA_F16>(a, head_dim, group, num_seqs, st);
    case PA_BF16: return launch_stream_d<PA_BF16, PA_BF16>(a, head_dim, group, num_seqs, st);
    case PA_FP8_E4M3:
      return q_dtype == PA_F16
                 ? launch_stream_d<PA_FP8_E4M3, PA_F16>(a, head_dim, group, num_seqs, st)
                 : launch_stream_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, num_seqs, st);
    case PA_I8:
      return q_dtype == PA_F16 ? launch_stream_d<PA_I8, PA_F16>(a, head_dim, group, num_seqs, st)
                               : launch_stream_d<PA_I8, PA_BF16>(a, head_dim, group, num_seqs, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
