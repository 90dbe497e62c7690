// Decode kernels for one KV storage type (see decode_kernels.h).
#include "decode_kernels.h"

namespace pa {

hipError_t launch_decode_bf16(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                              bool stream_loads, hipStream_t st) {
  (void)q_dtype;
  return launch_stream_kvq<PA_BF16, PA_BF16>(a, D, G, num_seqs, stream_loads, st);
}

}  // namespace pa
