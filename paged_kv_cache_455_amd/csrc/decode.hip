// Paged decode attention: split-context online softmax + second-pass merge
// (the device templates and their description are in decode_impl.h).
#include "decode_impl.h"

namespace pa {

template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(kDecodeWaves *kWave) void pa_decode_partition_kernel(DecodeArgs a) {
  const int s = blockIdx.z;
  decode_partition<KV, QT, D, G>(a, s, blockIdx.y, blockIdx.x, s, a.ctx[s], s);
}

// Second pass: combine a sequence's partitions, one workgroup per (seq, q head).
//   M = max_p m_p,  L = sum_p 2^(m_p - M) l_p,  out = sum_p 2^(m_p - M) acc_p / L
// Rows whose sequence fits in one partition were finished by the first pass.
template <int QT, int D>
__global__ __launch_bounds__(D) void pa_decode_merge_kernel(DecodeArgs a) {
  const int s = blockIdx.y;
  merge_partitions<QT, D>(a, s, blockIdx.x, threadIdx.x, a.ctx[s]);
}

// ---------------------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------------------
template <int KV, int QT, int D>
static hipError_t launch_g(const DecodeArgs &a, int G, dim3 grid, hipStream_t st) {
  dim3 blk(kDecodeWaves * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((pa_decode_partition_kernel<KV, QT, D, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((pa_decode_partition_kernel<KV, QT, D, 2>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((pa_decode_partition_kernel<KV, QT, D, 4>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((pa_decode_partition_kernel<KV, QT, D, 8>), grid, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV, int QT>
static hipError_t launch_d(const DecodeArgs &a, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64) return launch_g<KV, QT, 64>(a, G, grid, st);
  if (D == 128) return launch_g<KV, QT, 128>(a, G, grid, st);
  return hipErrorInvalidValue;
}

template <int QT>
static hipError_t launch_merge(const DecodeArgs &a, int D, int num_seqs, hipStream_t st) {
  dim3 grid(a.num_q_heads, num_seqs);
  if (D == 64) hipLaunchKernelGGL((pa_decode_merge_kernel<QT, 64>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((pa_decode_merge_kernel<QT, 128>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int kv_dtype, int q_dtype, int head_dim, int group,
                         int num_seqs, hipStream_t st) {
  dim3 grid(a.max_parts, a.num_kv_heads, num_seqs);
  hipError_t e = hipErrorInvalidValue;
  switch (kv_dtype) {
    case PA_F32: e = launch_d<PA_F32, PA_F32>(a, head_dim, group, grid, st); break;
    case PA_F16: e = launch_d<PA_F16, PA_F16>(a, head_dim, group, grid, st); break;
    case PA_BF16: e = launch_d<PA_BF16, PA_BF16>(a, head_dim, group, grid, st); break;
    case PA_FP8_E4M3:
      e = q_dtype == PA_F16 ? launch_d<PA_FP8_E4M3, PA_F16>(a, head_dim, group, grid, st)
                            : launch_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, grid, st);
      break;
    case PA_I8:
      e = q_dtype == PA_F16 ? launch_d<PA_I8, PA_F16>(a, head_dim, group, grid, st)
                            : launch_d<PA_I8, PA_BF16>(a, head_dim, group, grid, st);
      break;
  }
  if (e != hipSuccess || a.max_parts <= 1) return e;
  switch (q_dtype) {
    case PA_F32: return launch_merge<PA_F32>(a, head_dim, num_seqs, st);
    case PA_F16: return launch_merge<PA_F16>(a, head_dim, num_seqs, st);
    default: return launch_merge<PA_BF16>(a, head_dim, num_seqs, st);
  }
}

}  // namespace pa
