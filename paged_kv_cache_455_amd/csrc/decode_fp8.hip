// Decode kernels for one KV storage type (see decode_kernels.h).
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_fp8(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                             bool stream_loads, hipStream_t st) {
  return q_dtype == PA_F16
             ? launch_stream_kvq<PA_FP8_E4M3, PA_F16>(a, D, G, num_seqs, stream_loads, st)
             : launch_stream_kvq<PA_FP8_E4M3, PA_BF16>(a, D, G, num_seqs, stream_loads, st);
}

}  // namespace pa
