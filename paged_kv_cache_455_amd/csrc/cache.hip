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
// slot is block_table[s][pos / 16] * 16 + pos % 16.
__global__ __launch_bounds__(256) void pa_slot_mapping_kernel(const int32_t *bt, int32_t mbps,
                                                              const int32_t *qsl,
                                                              const int32_t *seq_lens,
                                                              int64_t *slots) {
  const int s = blockIdx.x;
  const int a = qsl[s], b = qsl[s + 1];
  const int q_len = b - a;
  const int first = seq_lens[s] - q_len;
  const int32_t *row = bt + (int64_t)s * mbps;
  for (int i = threadIdx.x; i < q_len; i += blockDim.x) {
    const int pos = first + i;
    slots[a + i] = (int64_t)row[pos / kBlock] * kBlock + pos % kBlock;
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
    const int64_t blk = slot / kBlock;
    const int off = (int)(slot % kBlock);
    const char *src = reinterpret_cast<const char *>(is_v ? a.v_new : a.k_new) +
                      row * a.row_bytes + c * 16;
    char *dst = reinterpret_cast<char *>(is_v ? a.v : a.k) +
                ((blk * a.num_kv_heads + h) * kBlock + off) * (int64_t)a.row_bytes + c * 16;
    *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
  }
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
    char *base = reinterpret_cast<char *>(is_v ? a.v : a.k);
    const int64_t blk_bytes = per_blk * 16;
    *reinterpret_cast<u32x4 *>(base + dst_b * blk_bytes + c * 16) =
        *reinterpret_cast<const u32x4 *>(base + src_b * blk_bytes + c * 16);
    float *sc = is_v ? a.v_scale : a.k_scale;
    if (sc != nullptr && c < a.num_kv_heads)
      sc[dst_b * a.num_kv_heads + c] = sc[src_b * a.num_kv_heads + c];
  }
}

static int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return (int)(g < 8192 ? (g < 1 ? 1 : g) : 8192);
}

hipError_t launch_slot_mapping(const int32_t *bt, int32_t mbps, const int32_t *qsl,
                               const int32_t *seq_lens, int32_t num_seqs, int64_t *slots,
                               hipStream_t st) {
  hipLaunchKernelGGL(pa_slot_mapping_kernel, dim3(num_seqs), dim3(256), 0, st, bt, mbps, qsl,
                     seq_lens, slots);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t st) {
  const int64_t total = 2 * (int64_t)a.num_tokens * a.num_kv_heads * (a.row_bytes / 16);
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, total);
  return hipGetLastError();
}

hipError_t launch_block_copy(const BlockCopyArgs &a, hipStream_t st) {
  const int64_t total = 2 * (int64_t)a.num_pairs * a.num_kv_heads * (a.tile_bytes / 16);
  hipLaunchKernelGGL(kv_block_copy_kernel, dim3(grid_for(total)), dim3(256), 0, st, a, total);
  return hipGetLastError();
}

}  // namespace pa
