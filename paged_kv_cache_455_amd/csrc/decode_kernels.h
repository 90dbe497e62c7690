// Decode kernels and their launch templates.  Each decode_<dtype>.hip includes this
// header and instantiates the launchers of one KV storage type, so the (many)
// kernel instantiations compile in parallel translation units.
#pragma once

#include "decode_impl.h"

namespace pa {

template <int KV, int QT, int D, int G, bool NT>
__global__ __launch_bounds__(kDecodeWaves *kWave) void pa_decode_stream_kernel(DecodeArgs a) {
  decode_stream<KV, QT, D, G, NT>(a);
}

// 1-byte KV with a GQA group of 8 (both products on MFMA): its state fits two waves
// per SIMD without spilling, which hides more of each wave's load latency.
template <int KV, int QT, bool NT>
__global__ __launch_bounds__(kDecodeWaves *kWave, 2) void pa_decode_stream_q8_kernel(DecodeArgs a) {
  decode_stream_q8<KV, QT, NT>(a);
}

// One wave per (sequence, query head); four per workgroup.
template <int QT, int D>
__global__ __launch_bounds__(4 * kWave) void pa_decode_stream_merge_kernel(DecodeArgs a) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // s * num_q_heads + hq
  if (row >= a.num_seqs * a.num_q_heads) return;
  merge_stream<QT, D>(a, row / a.num_q_heads, row % a.num_q_heads, threadIdx.x % kWave);
}

template <int KV, int QT, int D, int G, bool NT>
static constexpr auto stream_kernel() {
  if constexpr (Q8Geom<KV, D, G>::kOn)
    return pa_decode_stream_q8_kernel<KV, QT, NT>;
  else
    return pa_decode_stream_kernel<KV, QT, D, G, NT>;
}

// Workgroups of one balanced-split kernel instantiation that fit on the device at once.
template <int KV, int QT, int D, int G, bool NT>
static int resident_groups() {
  static int cached = 0;  // one value per instantiation
  if (cached > 0) return cached;
  auto kernel = stream_kernel<KV, QT, D, G, NT>();
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeWaves * kWave, 0) !=
      hipSuccess)
    return 0;
  cached = cus * (per_cu > 0 ? per_cu : 1);
  return cached;
}

template <int KV, int QT, int D, int G, bool NT>
static hipError_t launch_stream_kg(DecodeArgs a, int num_seqs, hipStream_t st) {
  auto kern = stream_kernel<KV, QT, D, G, NT>();
  // one workgroup per resident slot: every wave streams one equal share of the work
  const int groups = resident_groups<KV, QT, D, G, NT>();
  if (groups <= 0) return hipErrorInvalidDeviceFunction;
  a.num_waves = groups * kDecodeWaves;
  hipLaunchKernelGGL(kern, dim3(groups), dim3(kDecodeWaves * kWave), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 mgrid((num_seqs * a.num_q_heads + 3) / 4);
  hipLaunchKernelGGL((pa_decode_stream_merge_kernel<QT, D>), mgrid, dim3(4 * kWave), 0, st, a);
  return hipGetLastError();
}

template <int KV, int QT, int D, bool NT>
static hipError_t launch_stream_g(const DecodeArgs &a, int G, int num_seqs, hipStream_t st) {
  switch (G) {
    case 1: return launch_stream_kg<KV, QT, D, 1, NT>(a, num_seqs, st);
    case 2: return launch_stream_kg<KV, QT, D, 2, NT>(a, num_seqs, st);
    case 4: return launch_stream_kg<KV, QT, D, 4, NT>(a, num_seqs, st);
    case 8: return launch_stream_kg<KV, QT, D, 8, NT>(a, num_seqs, st);
  }
  return hipErrorInvalidValue;
}

template <int KV, int QT, bool NT>
static hipError_t launch_stream_d(const DecodeArgs &a, int D, int G, int num_seqs, hipStream_t st) {
  if (D == 64) return launch_stream_g<KV, QT, 64, NT>(a, G, num_seqs, st);
  if (D == 128) return launch_stream_g<KV, QT, 128, NT>(a, G, num_seqs, st);
  return hipErrorInvalidValue;
}

template <int KV, int QT>
static hipError_t launch_stream_kvq(const DecodeArgs &a, int D, int G, int num_seqs,
                                    bool stream_loads, hipStream_t st) {
  return stream_loads ? launch_stream_d<KV, QT, true>(a, D, G, num_seqs, st)
                      : launch_stream_d<KV, QT, false>(a, D, G, num_seqs, st);
}

}  // namespace pa
