// Data movement around the paged pools: slot mapping, cache write, block copy.
//
// 5688vip chapter 3, section 3.2: prefill writes every prompt token's K/V into
// the request's blocks; a decode step writes the new token at the end of the
// current block and moves on to a new physical block (through the block table)
// when that one is full.  uml.org.cn "Prefix Sharing": a request that diverges
// from a shared page gets a copy of it (copy-on-write) and writes there.
//
// All three are bandwidth- or launch-bound bit movement; lanes move 16-byte
// chunks so every wave-wide access is contiguous.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Logical position of query row t of sequence s is seq_len - q_len + i; its
// slot is block_table[s][pos / bs] * bs + pos % bs (bs = 16 or 32 tokens).
__global__ __launch_bounds__(256) void pa_slot_mapping_kernel(const int32_t *bt, int32_t mbps,
                                                              int32_t bs, const int32_t *qsl,
                                                              const int32_t *seq_lens,
                                                              int64_t *slots) {
  const int s = blockIdx.x;
  const int a = qsl[s], b = qsl[s + 1];
  const int q_len = b - a;
  const int first = seq_lens[s] - q_len;
  const int32_t *row = bt + (int64_t)s * mbps;
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    const int pos = first + i;
    slots[a + i] = (int64_t)row[pos / bs] * bs + pos % bs;
  }
}

// One thread per 16-byte chunk of one (token, kv head) row of K or V.
__global__ __launch_bounds__(256) void kv_cache_write_kernel(CacheWriteArgs a, int64_t total) {
  const int cpr = a.row_bytes / 16;  // chunks per row
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t per_pool = total / 2;
    const bool is_v = i >= per_pool;
    const int64_t r = is_v ? i - per_pool : i;
    const int c = (int)(r % cpr);
    const int64_t row = r / cpr;  // token * Hkv + head
    const int h = (int)(row % a.num_kv_heads);
    const int64_t t = row / a.num_kv_heads;
    const int64_t slot = a.slots[t];
    if (slot < 0) continue;
    const int64_t blk = slot / a.block_size;
    const int off = (int)(slot % a.block_size);
    const char *src = reinterpret_cast<const char *>(is_v ? a.v_new : a.k_new) +
                      row * a.row_bytes + c * 16;
    char *dst = reinterpret_cast<char *>(is_v ? a.v : a.k) +
                ((blk * a.num_kv_heads + h) * a.block_size + off) * (int64_t)a.row_bytes + c * 16;
    *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
  }
}

// ---- quantise-on-write into a 1-byte pool ----------------------------------------
// "从KV Cache到vLLM" §2.2-2.3 store the cache as INT8 or FP8 codes; one fp32 scale
// per (block, kv head) maps codes to values.  The rows one call writes into a
// block are that block's next rows, contiguous in token order (a "run").  One
// wave per (run, kv head, K or V):
//   amax   = largest |x| over the run's rows (every dim)
//   s_new  = max(s_old, amax / qmax)      s_old = 0 when the run starts at row 0
//   if s_new > s_old: earlier rows c -> encode(value(c) * (s_old / s_new))
//   new rows x -> encode(x / s_new)       (code 0 while s_new is 0)
// All arithmetic is fp32, rounded to nearest even; encode clamps to +-qmax and
// rounds to nearest even (E4M3FN by the hardware convert, int8 by v_rndne).
template <int ST>
__device__ __forceinline__ float src_value(const void *p, int64_t i) {
  if constexpr (ST == PA_F32) return reinterpret_cast<const float *>(p)[i];
  else if constexpr (ST == PA_F16) return (float)reinterpret_cast<const _Float16 *>(p)[i];
  else return __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}

template <int KV>
__device__ __forceinline__ uint8_t encode_code(float y) {
  constexpr float qmax = KV == PA_FP8_E4M3 ? 448.f : 127.f;
  y = fminf(fmaxf(y, -qmax), qmax);
  if constexpr (KV == PA_FP8_E4M3) {
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xff);
  } else {
    return (uint8_t)(int8_t)(int)__builtin_rintf(y);
  }
}

template <int KV>
__device__ __forceinline__ float code_value(uint8_t c) {
  if constexpr (KV == PA_FP8_E4M3) {
    float f[4];
    fp8x4_to_f32((uint32_t)c, f);
    return f[0];
  } else {
    return (float)(int8_t)c;
  }
}

template <int KV, int ST, int D>
__global__ __launch_bounds__(64) void kv_cache_write_quant_kernel(CacheWriteArgs a) {
  constexpr float qmax = KV == PA_FP8_E4M3 ? 448.f : 127.f;
  constexpr int EPL = D / 64;  // dims per lane
  const int t = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const bool is_v = blockIdx.z != 0;
  const int bs = a.block_size;
  int64_t slot;
  int len = 1;
  if (a.slots == nullptr) {  // decode append: one row per sequence, each a run of its own
    const int n = a.ctx[t];
    slot = n > 0 ? (int64_t)a.bt[(int64_t)t * a.mbps + (n - 1) / bs] * bs + (n - 1) % bs : -1;
    if (a.slots_out != nullptr && h == 0 && !is_v && lane == 0) a.slots_out[t] = slot;
    if (slot < 0) return;
  } else {
    slot = a.slots[t];
    if (slot < 0) return;
    if (t > 0) {  // not the first row of its run: the run's first row does the work
      const int64_t prev = a.slots[t - 1];
      if (prev >= 0 && prev / bs == slot / bs) return;
    }
    while (len < bs - (int)(slot % bs) && t + len < a.num_tokens && a.slots[t + len] >= 0 &&
           a.slots[t + len] / bs == slot / bs)
      ++len;
  }
  const int64_t blk = slot / bs;
  const int off = (int)(slot % bs);

  const void *src = is_v ? a.v_new : a.k_new;
  uint8_t *tile = reinterpret_cast<uint8_t *>(is_v ? a.v : a.k) +
                  (blk * a.num_kv_heads + h) * (int64_t)(bs * D);
  float *scale = (is_v ? a.v_scale : a.k_scale) + blk * a.num_kv_heads + h;
  const int d0 = lane * EPL;

  auto src_at = [&](int i, int e) {
    return src_value<ST>(src, ((int64_t)(t + i) * a.num_kv_heads + h) * D + d0 + e);
  };
  float amax = 0.f;
  for (int i = 0; i < len; ++i)
#pragma unroll
    for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(src_at(i, e)));
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float s_old = off > 0 ? *scale : 0.f;
  const float s_new = fmaxf(s_old, amax / qmax);
  if (off > 0 && s_new > s_old) {
    const float ratio = s_old / s_new;
    for (int r = 0; r < off; ++r) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        uint8_t *c = tile + r * D + d0 + e;
        *c = encode_code<KV>(code_value<KV>(*c) * ratio);
      }
    }
  }
  for (int i = 0; i < len; ++i) {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      tile[(off + i) * D + d0 + e] = s_new > 0.f ? encode_code<KV>(src_at(i, e) / s_new) : (uint8_t)0;
  }
  if (lane == 0) *scale = s_new;
}

// One thread per 16-byte chunk of a block's K or V (all kv heads), plus the
// per-(block, kv head) scales of 1-byte pools.
__global__ __launch_bounds__(256) void kv_block_copy_kernel(BlockCopyArgs a, int64_t total) {
  const int64_t per_blk = (int64_t)a.num_kv_heads * a.tile_bytes / 16;  // chunks per block
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t per_pool = total / 2;
    const bool is_v = i >= per_pool;
    const int64_t r = is_v ? i - per_pool : i;
    const int pair = (int)(r / per_blk);
    const int64_t c = r % per_blk;
    const int64_t src_b = a.pairs[2 * pair];
    const int64_t dst_b = a.pairs[2 * pair + 1];
    const char *src = reinterpret_cast<const char *>(is_v ? a.src_v : a.src_k);
    char *dst = reinterpret_cast<char *>(is_v ? a.dst_v : a.dst_k);
    const int64_t blk_bytes = per_blk * 16;
    *reinterpret_cast<u32x4 *>(dst + dst_b * blk_bytes + c * 16) =
        *reinterpret_cast<const u32x4 *>(src + src_b * blk_bytes + c * 16);
    const float *ss = is_v ? a.src_vs : a.src_ks;
    float *ds = is_v ? a.dst_vs : a.dst_ks;
    if (ds != nullptr && c < a.num_kv_heads)
      ds[dst_b * a.num_kv_heads + c] = ss[src_b * a.num_kv_heads + c];
  }
}

static int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return (int)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

hipError_t launch_slot_mapping(const int32_t *bt, int32_t mbps, int32_t block_size,
                               const int32_t *qsl,
                               const int32_t *seq_lens, int32_t num_seqs, int64_t *slots,
                               hipStream_t st) {
  hipLaunchKernelGGL(pa_slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, st, bt, mbps,
                     block_size, qsl,
                     seq_lens, slots);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t st) {
  const int64_t total = 2 * (int64_t)a.num_tokens * a.num_kv_heads * (a.row_bytes / 16);
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, total);
  return hipGetLastError();
}

template <int KV, int ST>
static hipError_t launch_quant_d(const CacheWriteArgs &a, int D, hipStream_t st) {
  dim3 grid(a.num_tokens, a.num_kv_heads, 2);
  if (D == 64) hipLaunchKernelGGL((kv_cache_write_quant_kernel<KV, ST, 64>), grid, dim3(64), 0, st, a);
  else hipLaunchKernelGGL((kv_cache_write_quant_kernel<KV, ST, 128>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

template <int KV>
static hipError_t launch_quant_s(const CacheWriteArgs &a, int src_dtype, int D, hipStream_t st) {
  switch (src_dtype) {
    case PA_F32: return launch_quant_d<KV, PA_F32>(a, D, st);
    case PA_F16: return launch_quant_d<KV, PA_F16>(a, D, st);
    case PA_BF16: return launch_quant_d<KV, PA_BF16>(a, D, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_cache_write_quant(const CacheWriteArgs &a, int kv_dtype, int src_dtype,
                                    int head_dim, hipStream_t st) {
  return kv_dtype == PA_FP8_E4M3 ? launch_quant_s<PA_FP8_E4M3>(a, src_dtype, head_dim, st)
                                 : launch_quant_s<PA_I8>(a, src_dtype, head_dim, st);
}

hipError_t launch_block_copy(const BlockCopyArgs &a, hipStream_t st) {
  const int64_t total = 2 * (int64_t)a.num_pairs * a.num_kv_heads * (a.tile_bytes / 16);
  hipLaunchKernelGGL(kv_block_copy_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, total);
  return hipGetLastError();
}

}  // namespace pa
