// Paged decode attention, host-side dispatch by KV storage type.  The kernels are
// in decode_kernels.h (device templates in decode_impl.h); each storage type's
// instantiations live in their own translation unit, decode_<dtype>.hip.
#include "../../include/pa.h"
#include "pa_launch.h"

namespace pa {

hipError_t launch_decode_stream(const DecodeArgs &a, int kv_dtype, int q_dtype, int head_dim,
                                int group, int num_seqs, bool stream_loads, hipStream_t st) {
  switch (kv_dtype) {
    case PA_F32: return launch_decode_f32(a, q_dtype, head_dim, group, num_seqs, stream_loads, st);
    case PA_F16: return launch_decode_f16(a, q_dtype, head_dim, group, num_seqs, stream_loads, st);
    case PA_BF16: return launch_decode_bf16(a, q_dtype, head_dim, group, num_seqs, stream_loads, st);
    case PA_FP8_E4M3:
      return launch_decode_fp8(a, q_dtype, head_dim, group, num_seqs, stream_loads, st);
    case PA_I8: return launch_decode_i8(a, q_dtype, head_dim, group, num_seqs, stream_loads, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
