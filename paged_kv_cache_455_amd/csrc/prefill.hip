// Mixed continuous-batching step: chunked prefills and decodes in one launch.
//
// uml.org.cn "Continuous Batching": new requests' prefill work and running
// requests' decode steps share one batch.  5688vip chapter 3, section 3.1:
// generation is autoregressive, so query row i of a chunk that extends a
// sequence to seq_len tokens sits at position seq_len - q_len + i and attends
// to keys 0 .. that position.
//
// Every query row is one work item per (kv head, context partition), run by the
// decode partition path with the row's own causal context length; partitions
// are merged by a second pass.
#include "decode_impl.h"

namespace pa {

// Sequence that owns packed query row t, and the row's causal context length.
__device__ __forceinline__ void row_owner(const int32_t *qsl, const int32_t *seq_lens,
                                          int num_seqs, int t, int &s, int &n) {
  int lo = 0, hi = num_seqs;  // invariant: qsl[lo] <= t < qsl[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid;
  }
  s = lo;
  const int q_len = qsl[lo + 1] - qsl[lo];
  n = seq_lens[lo] - q_len + (t - qsl[lo]) + 1;
}

template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(kDecodeWaves *kWave) void pa_mixed_rows_kernel(PrefillArgs a) {
  const int t = blockIdx.z;
  int s, n;
  row_owner(a.qsl, a.dec.ctx, a.num_seqs, t, s, n);
  decode_partition<KV, QT, D, G>(a.dec, s, blockIdx.y, blockIdx.x, t, n, t);
}

template <int QT, int D>
__global__ __launch_bounds__(D) void pa_mixed_merge_kernel(PrefillArgs a) {
  const int t = blockIdx.y;
  int s, n;
  row_owner(a.qsl, a.dec.ctx, a.num_seqs, t, s, n);
  merge_partitions<QT, D>(a.dec, t, blockIdx.x, threadIdx.x, n);
}

template <int KV, int QT, int D>
static hipError_t launch_rows(const PrefillArgs &a, int G, dim3 grid, hipStream_t st) {
  dim3 blk(kDecodeWaves * kWave);
  switch (G) {
    case 1: hipLaunchKernelGGL((pa_mixed_rows_kernel<KV, QT, D, 1>), grid, blk, 0, st, a); break;
    case 2: hipLaunchKernelGGL((pa_mixed_rows_kernel<KV, QT, D, 2>), grid, blk, 0, st, a); break;
    case 4: hipLaunchKernelGGL((pa_mixed_rows_kernel<KV, QT, D, 4>), grid, blk, 0, st, a); break;
    case 8: hipLaunchKernelGGL((pa_mixed_rows_kernel<KV, QT, D, 8>), grid, blk, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int KV, int QT>
static hipError_t launch_rows_d(const PrefillArgs &a, int D, int G, dim3 grid, hipStream_t st) {
  if (D == 64) return launch_rows<KV, QT, 64>(a, G, grid, st);
  if (D == 128) return launch_rows<KV, QT, 128>(a, G, grid, st);
  return hipErrorInvalidValue;
}

template <int QT>
static hipError_t launch_mixed_merge(const PrefillArgs &a, int D, int num_rows, hipStream_t st) {
  dim3 grid(a.dec.num_q_heads, num_rows);
  if (D == 64) hipLaunchKernelGGL((pa_mixed_merge_kernel<QT, 64>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((pa_mixed_merge_kernel<QT, 128>), grid, dim3(128), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, int kv_dtype, int q_dtype, int head_dim, int group,
                          int num_rows, hipStream_t st) {
  dim3 grid(a.dec.max_parts, a.dec.num_kv_heads, num_rows);
  hipError_t e = hipErrorInvalidValue;
  switch (kv_dtype) {
    case PA_F32: e = launch_rows_d<PA_F32, PA_F32>(a, head_dim, group, grid, st); break;
    case PA_F16: e = launch_rows_d<PA_F16, PA_F16>(a, head_dim, group, grid, st); break;
    case PA_BF16: e = launch_rows_d<PA_BF16, PA_BF16>(a, head_dim, group, grid, st); break;
    case PA_FP8_E4M3:
      e = q_dtype == PA_F16 ? launch_rows_d<PA_FP8_E4M3, PA_F16>(a, head_dim, group, grid, st)
                            : launch_rows_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, grid, st);
      break;
    case PA_I8:
      e = q_dtype == PA_F16 ? launch_rows_d<PA_I8, PA_F16>(a, head_dim, group, grid, st)
                            : launch_rows_d<PA_I8, PA_BF16>(a, head_dim, group, grid, st);
      break;
  }
  if (e != hipSuccess || a.dec.max_parts <= 1) return e;
  switch (q_dtype) {
    case PA_F32: return launch_mixed_merge<PA_F32>(a, head_dim, num_rows, st);
    case PA_F16: return launch_mixed_merge<PA_F16>(a, head_dim, num_rows, st);
    default: return launch_mixed_merge<PA_BF16>(a, head_dim, num_rows, st);
  }
}

}  // namespace pa
