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

// Both products on MFMA (MxGeom::kOn).  PER_CU workgroups per CU
// (stream_kernel_per_cu): two where a wave's K+V tile is at most 4 KiB (1-byte
// pools; 16-bit ones at head_dim 64) or the pool's blocks are shared, whose state
// then fits two waves per SIMD without spilling and hides more of each wave's load
// latency; else one.
template <int KV, int QT, int D, int G, bool NT, int PER_CU>
__global__ __launch_bounds__(kDecodeWaves *kWave, PER_CU) void pa_decode_stream_mx_kernel(DecodeArgs a) {
  decode_stream_mx<KV, QT, D, G, NT>(a);
}

// One wave per (sequence, query head); four per workgroup.
template <int QT, int D>
__global__ __launch_bounds__(4 * kWave) void pa_decode_stream_merge_kernel(DecodeArgs a) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // s * num_q_heads + hq
  if (row >= a.num_seqs * a.num_q_heads) return;
  merge_stream<QT, D>(a, row / a.num_q_heads, row % a.num_q_heads, threadIdx.x % kWave);
}

// Workgroups per CU of the stream kernel of (KV, D, G, NT): stream_per_cu's rule by
// tile size, and two for the MFMA tile over a shared-block pool (cached loads), whose
// hits in L2 and the Infinity Cache leave each wave waiting on latency more than on
// HBM (128 bf16 requests over a 1024-token shared prefix: 143.5 against 138.8 us at
// two; the unshared Llama-3-8B-shaped decode layer is 2.3 us slower at two).
template <int KV, int D, int G, bool NT>
constexpr int stream_kernel_per_cu() {
  return MxGeom<KV, D, G>::kOn && !NT ? 2 : stream_per_cu<KV, D>();
}

template <int KV, int QT, int D, int G, bool NT>
static constexpr auto stream_kernel() {
  if constexpr (MxGeom<KV, D, G>::kOn)
    return pa_decode_stream_mx_kernel<KV, QT, D, G, NT, stream_kernel_per_cu<KV, D, G, NT>()>;
  else
    return pa_decode_stream_kernel<KV, QT, D, G, NT>;
}

// Workgroups of one balanced-split kernel instantiation that fit on the device at
// once, and how many of them share a CU.
struct Residency {
  int groups, per_cu;
};
template <int KV, int QT, int D, int G, bool NT>
static Residency resident_groups() {
  static Residency cached{0, 0};  // one value per instantiation
  if (cached.groups > 0) return cached;
  auto kernel = stream_kernel<KV, QT, D, G, NT>();
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return Residency{0, 0};
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return Residency{0, 0};
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecodeWaves * kWave, 0) !=
      hipSuccess)
    return Residency{0, 0};
  // Kernels whose K+V tile is 8 KiB or more run one workgroup per CU (a wave per
  // SIMD) even where their registers would allow two: twice the waves split twice
  // as many segments: the Llama-3-8B-shaped decode layer (64 sequences, 32/8 heads)
  // measured 98.0 against 95.2 us at two on the VALU path, the 16-bit MFMA tile 105.6
  // against 99.5 us at a group of 8.  Tiles of at
  // most 4 KiB run two (the 16 x 32768-token fp8 decode: 179 against 198 us at one;
  // MHA-shaped fp8 at head_dim 64 on the VALU path 52.3 against 36.4 us).
  const int cap = stream_kernel_per_cu<KV, D, G, NT>();
  per_cu = per_cu > cap ? cap : per_cu;
  per_cu = per_cu > 0 ? per_cu : 1;
  cached = Residency{cus * per_cu, per_cu};
  return cached;
}

// Two workgroups per CU: the waves of the grid's second round (the second wave on
// each SIMD) stream slower than the first's, which the instruction arbiter serves
// first; per-wave timestamps of the 16 x 32768-token fp8 decode put their median
// end 5-17 us later.  The first round takes skew/256 of its share more, the second
// as much less.
constexpr int kTwoRoundSkew = 6;

template <int KV, int QT, int D, int G, bool NT>
static hipError_t launch_stream_kg(DecodeArgs a, int num_seqs, hipStream_t st) {
  auto kern = stream_kernel<KV, QT, D, G, NT>();
  // one workgroup per resident slot: every wave streams one equal share of the work
  const Residency res = resident_groups<KV, QT, D, G, NT>();
  const int groups = res.groups;
  if (groups <= 0) return hipErrorInvalidDeviceFunction;
  a.num_waves = groups * kDecodeWaves;
  a.skew = res.per_cu == 2 ? kTwoRoundSkew : 0;
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
