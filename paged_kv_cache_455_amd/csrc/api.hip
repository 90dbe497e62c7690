// C ABI of the paged-attention library: argument checks, workspace sizing,
// split-context policy and kernel dispatch.  Declarations and contracts are in
// include/pa.h.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>

#include <mutex>
#include <new>

#include "pa_launch.h"
#include "status.h"
#include "../../include/pa.h"

namespace {

pa_status_t fail(pa_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status_t fail(pa_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  pa::set_errorv(st, fmt, ap);
  va_end(ap);
  return st;
}

pa_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kTileRows = 16;  // rows per tile; the splits and workspaces count tiles

int elem_bytes(int dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16: case PA_BF16: return 2;
    case PA_FP8_E4M3: case PA_I8: return 1;
    default: return 0;
  }
}

bool is_quantised(int dt) { return dt == PA_FP8_E4M3 || dt == PA_I8; }

pa_status_t check_pool(const pa_kv_pool_t *pool, bool need_scales_if_quantised) {
  if (pool == nullptr) return fail(PA_E_ARG, "pool is NULL");
  if (pool->k == nullptr || pool->v == nullptr) return fail(PA_E_ARG, "pool k/v pointer is NULL");
  if (pool->num_blocks <= 0) return fail(PA_E_ARG, "num_blocks must be > 0");
  if (pool->num_kv_heads <= 0) return fail(PA_E_ARG, "num_kv_heads must be > 0");
  if (pool->block_size != 16 && pool->block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size %d unsupported (16 or 32)", pool->block_size);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(PA_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", pool->head_dim);
  if (elem_bytes(pool->kv_dtype) == 0) return fail(PA_E_ARG, "unknown kv_dtype %d", pool->kv_dtype);
  if (need_scales_if_quantised && is_quantised(pool->kv_dtype) &&
      (pool->k_scale == nullptr || pool->v_scale == nullptr))
    return fail(PA_E_ARG, "1-byte kv_dtype needs k_scale and v_scale");
  if (!is_quantised(pool->kv_dtype) && (pool->k_scale != nullptr || pool->v_scale != nullptr))
    return fail(PA_E_ARG, "scales are only meaningful for 1-byte kv_dtype");
  if (((uintptr_t)pool->k | (uintptr_t)pool->v) & 15)
    return fail(PA_E_ARG, "pool k/v must be 16-byte aligned");
  if (pool->flags & ~PA_POOL_SHARED_BLOCKS) return fail(PA_E_ARG, "unknown pool flags 0x%x", pool->flags);
  return PA_OK;
}

pa_status_t check_q_dtype(int kv, int q) {
  if (is_quantised(kv)) {
    if (q != PA_F16 && q != PA_BF16)
      return fail(PA_E_UNSUPPORTED, "1-byte KV takes f16 or bf16 queries (got %d)", q);
  } else if (q != kv) {
    return fail(PA_E_UNSUPPORTED, "q_dtype %d must equal kv_dtype %d for float KV", q, kv);
  }
  return PA_OK;
}

pa_status_t check_heads(int num_q_heads, int num_kv_heads, int *group) {
  if (num_q_heads <= 0) return fail(PA_E_ARG, "num_q_heads must be > 0");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_E_ARG, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                num_kv_heads);
  const int g = num_q_heads / num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_E_UNSUPPORTED, "GQA group %d unsupported (1, 2, 4 or 8)", g);
  *group = g;
  return PA_OK;
}

// ---- split-context policy ---------------------------------------------------------------
// A context of nblk blocks is cut into partitions of part_blocks blocks, each one
// workgroup.  The default keeps partitions long (little merge traffic) and only
// shortens them when there would be too few workgroups to fill 256 CUs.
int decode_part_blocks(int64_t num_rows, int num_kv_heads, int max_blocks) {
  int pb = 32;
  const int64_t kMinGroups = 1024;
  while (pb > 8) {
    const int64_t parts = (max_blocks + pb - 1) / pb;
    if (num_rows * num_kv_heads * parts >= kMinGroups) break;
    pb /= 2;
  }
  return pb;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t acc_off, m_off, l_off, hdr_off, total;
};

WsLayout ws_layout(int64_t rows, int num_q_heads, int head_dim, int max_parts) {
  WsLayout w{};
  if (max_parts <= 1) return w;
  const size_t n_ml = (size_t)rows * num_q_heads * max_parts;
  w.acc_off = 0;
  w.m_off = align256(n_ml * head_dim * sizeof(float));
  w.l_off = w.m_off + align256(n_ml * sizeof(float));
  w.total = w.l_off + align256(n_ml * sizeof(float));
  return w;
}

// Balanced-split decode: every wave streams at least this many tiles, which bounds
// how many waves (pieces) can share one (sequence, kv head) segment.
constexpr int kMinTilesPerWave = 8;
// Cost, in tiles, of starting a (sequence, kv head) segment in the balanced split
// (emitting its result, switching q): 0 -> 4 took the Llama-3-8B-shaped decode layer
// from 110 to 103 us and the mixed step's lognormal decode rows from 224 to 190 us;
// once the emit became a reduce-scatter (0.55 instead of 1.8 us per segment end),
// 2 beat 1, 3 and 4 (stream kernel 95.0 vs 95.9 us at 4, mixed decode rows 185.5 vs
// 188.0 us, prefix-sharing decode 162.8 vs 164.2 us).
constexpr int kSegCost = 2;

int stream_pieces(int max_ctx) {
  const int max_blocks = (max_ctx + kTileRows - 1) / kTileRows;
  return (max_blocks + kMinTilesPerWave - 1) / kMinTilesPerWave + 1;
}

WsLayout stream_layout(int64_t num_seqs, int num_q_heads, int head_dim, int max_ctx) {
  const int pieces = stream_pieces(max_ctx);
  WsLayout w{};
  const size_t n_ml = (size_t)num_seqs * num_q_heads * pieces;
  w.acc_off = 0;
  w.m_off = align256(n_ml * head_dim * sizeof(float));
  w.l_off = w.m_off + align256(n_ml * sizeof(float));
  w.hdr_off = w.l_off + align256(n_ml * sizeof(float));
  w.total = w.hdr_off + align256((size_t)(num_seqs + 2) * sizeof(int32_t));
  return w;
}

int max_parts_for(int max_ctx, int part_blocks) {
  const int max_blocks = (max_ctx + kTileRows - 1) / kTileRows;
  return (max_blocks + part_blocks - 1) / part_blocks;
}

}  // namespace

extern "C" {

pa_status_t pa_slot_mapping(const int32_t *block_tables, int32_t max_blocks_per_seq,
                            int32_t block_size, const int32_t *query_start_loc, const int32_t *seq_lens,
                            int32_t num_seqs, int32_t num_tokens, int64_t *slot_mapping,
                            hipStream_t stream) {
  if (num_seqs < 0 || num_tokens < 0) return fail(PA_E_ARG, "negative num_seqs/num_tokens");
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!block_tables || !query_start_loc || !seq_lens || !slot_mapping)
    return fail(PA_E_ARG, "NULL array argument");
  if (max_blocks_per_seq <= 0) return fail(PA_E_ARG, "max_blocks_per_seq must be > 0");
  if (block_size != 16 && block_size != 32)
    return fail(PA_E_UNSUPPORTED, "block_size %d unsupported (16 or 32)", block_size);
  return hip_status(pa::launch_slot_mapping(block_tables, max_blocks_per_seq, block_size,
                                            query_start_loc,
                                            seq_lens, num_seqs, slot_mapping, stream),
                    "pa_slot_mapping launch");
}

// The input checks need the pool's geometry only.
static pa_status_t check_geometry(const pa_kv_pool_t *pool, int32_t *flags) {
  if (!pool || !flags) return fail(PA_E_ARG, "NULL pool or flags");
  if (pool->num_blocks <= 0) return fail(PA_E_ARG, "num_blocks must be > 0");
  if (pool->block_size != 16 && pool->block_size != 32)
    return fail(PA_E_ARG, "block_size %d (16 or 32)", pool->block_size);
  return PA_OK;
}

pa_status_t pa_check_tables(const pa_kv_pool_t *pool, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t num_seqs, int32_t max_seq_len,
                            int32_t *flags, hipStream_t stream) {
  pa_status_t st = check_geometry(pool, flags);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_E_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  if (!block_tables || !seq_lens) return fail(PA_E_ARG, "NULL array argument");
  if (max_blocks_per_seq <= 0) return fail(PA_E_ARG, "max_blocks_per_seq must be > 0");
  pa::CheckTablesArgs a{block_tables, seq_lens, query_start_loc, flags, pool->num_blocks,
                        max_blocks_per_seq, pool->block_size, max_seq_len};
  return hip_status(pa::launch_check_tables(a, num_seqs, stream), "pa_check_tables launch");
}

pa_status_t pa_check_slots(const pa_kv_pool_t *pool, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t *flags, hipStream_t stream) {
  pa_status_t st = check_geometry(pool, flags);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_E_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping) return fail(PA_E_ARG, "NULL slot_mapping");
  return hip_status(pa::launch_check_slots(slot_mapping, num_tokens,
                                           pool->num_blocks * pool->block_size, flags, stream),
                    "pa_check_slots launch");
}

pa_status_t pa_check_copy_pairs(const pa_kv_pool_t *pool, const int32_t *src_dst,
                                int32_t num_pairs, int32_t *flags, hipStream_t stream) {
  pa_status_t st = check_geometry(pool, flags);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_E_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_E_ARG, "NULL src_dst");
  return hip_status(pa::launch_check_pairs(src_dst, num_pairs, pool->num_blocks, flags, stream),
                    "pa_check_copy_pairs launch");
}

pa_status_t kv_cache_write(const pa_kv_pool_t *pool, const void *k_new, const void *v_new,
                           const int64_t *slot_mapping, int32_t num_tokens, hipStream_t stream) {
  pa_status_t st = check_pool(pool, false);
  if (st != PA_OK) return st;
  if (is_quantised(pool->kv_dtype))
    return fail(PA_E_UNSUPPORTED, "1-byte pools are written by kv_cache_write_quant");
  if (num_tokens < 0) return fail(PA_E_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_E_ARG, "NULL array argument");
  pa::CacheWriteArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.num_blocks = pool->num_blocks;
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool->num_kv_heads;
  a.row_bytes = pool->head_dim * elem_bytes(pool->kv_dtype);
  a.block_size = pool->block_size;
  return hip_status(pa::launch_cache_write(a, stream), "kv_cache_write launch");
}

pa_status_t kv_cache_write_quant(const pa_kv_pool_t *pool, const void *k_new, const void *v_new,
                                 int32_t src_dtype, const int64_t *slot_mapping,
                                 int32_t num_tokens, hipStream_t stream) {
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (!is_quantised(pool->kv_dtype))
    return fail(PA_E_UNSUPPORTED, "kv_cache_write_quant needs a 1-byte pool (use kv_cache_write)");
  if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_E_UNSUPPORTED, "src_dtype %d: f32, f16 or bf16 values only", src_dtype);
  if (num_tokens < 0) return fail(PA_E_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_E_ARG, "NULL array argument");
  if (pool->num_kv_heads > 65535)  // grid y limit
    return fail(PA_E_UNSUPPORTED, "too many kv heads for one launch");
  pa::CacheWriteArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  a.num_blocks = pool->num_blocks;
  a.num_tokens = num_tokens;
  a.num_kv_heads = pool->num_kv_heads;
  a.row_bytes = pool->head_dim;
  a.block_size = pool->block_size;
  return hip_status(pa::launch_cache_write_quant(a, pool->kv_dtype, src_dtype, pool->head_dim,
                                                 stream),
                    "kv_cache_write_quant launch");
}

pa_status_t kv_block_copy(const pa_kv_pool_t *pool, const int32_t *src_dst, int32_t num_pairs,
                          hipStream_t stream) {
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_E_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_E_ARG, "src_dst is NULL");
  pa::BlockCopyArgs a{};
  a.src_k = a.dst_k = pool->k;
  a.src_v = a.dst_v = pool->v;
  a.src_ks = a.dst_ks = pool->k_scale;
  a.src_vs = a.dst_vs = pool->v_scale;
  a.pairs = src_dst;
  a.num_pairs = num_pairs;
  a.num_kv_heads = pool->num_kv_heads;
  a.tile_bytes = pool->block_size * pool->head_dim * elem_bytes(pool->kv_dtype);
  return hip_status(pa::launch_block_copy(a, stream), "kv_block_copy launch");
}

// The address a kernel uses for p: p itself for device (or managed) memory, the
// mapped device address for pinned host memory; pageable host memory is refused.
static pa_status_t device_address(const void *p, const char *what, void **out) {
  *out = nullptr;
  if (p == nullptr) return PA_OK;
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_E_ARG, "%s is neither device memory nor pinned host memory", what);
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = const_cast<void *>(p);
  } else if (at.type == hipMemoryTypeHost && at.devicePointer != nullptr) {
    *out = at.devicePointer;
  } else {
    return fail(PA_E_ARG, "%s is neither device memory nor pinned host memory", what);
  }
  return PA_OK;
}

pa_status_t kv_swap(const pa_kv_pool_t *dst, const pa_kv_pool_t *src, const int32_t *src_dst,
                    int32_t num_pairs, hipStream_t stream) {
  pa_status_t st = check_pool(dst, true);
  if (st != PA_OK) return st;
  if ((st = check_pool(src, true)) != PA_OK) return st;
  if (dst->kv_dtype != src->kv_dtype || dst->num_kv_heads != src->num_kv_heads ||
      dst->head_dim != src->head_dim || dst->block_size != src->block_size)
    return fail(PA_E_ARG, "kv_swap pools differ in kv_dtype, num_kv_heads, head_dim or block_size");
  if (num_pairs < 0) return fail(PA_E_ARG, "num_pairs must be >= 0");
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_E_ARG, "src_dst is NULL");
  void *p[8];
  const void *in[8] = {src->k, src->v, src->k_scale, src->v_scale,
                       dst->k, dst->v, dst->k_scale, dst->v_scale};
  static const char *names[8] = {"src k", "src v", "src k_scale", "src v_scale",
                                 "dst k", "dst v", "dst k_scale", "dst v_scale"};
  for (int i = 0; i < 8; ++i)
    if ((st = device_address(in[i], names[i], &p[i])) != PA_OK) return st;
  void *pairs_dev;
  if ((st = device_address(src_dst, "src_dst", &pairs_dev)) != PA_OK) return st;
  pa::BlockCopyArgs a{};
  a.src_k = p[0];
  a.src_v = p[1];
  a.src_ks = static_cast<const float *>(p[2]);
  a.src_vs = static_cast<const float *>(p[3]);
  a.dst_k = p[4];
  a.dst_v = p[5];
  a.dst_ks = static_cast<float *>(p[6]);
  a.dst_vs = static_cast<float *>(p[7]);
  a.pairs = static_cast<const int32_t *>(pairs_dev);
  a.num_pairs = num_pairs;
  a.num_kv_heads = src->num_kv_heads;
  a.tile_bytes = src->block_size * src->head_dim * elem_bytes(src->kv_dtype);
  return hip_status(pa::launch_block_copy(a, stream), "kv_swap launch");
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      max_context_len <= 0)
    return 0;
  return stream_layout(num_seqs, num_q_heads, head_dim, max_context_len).total;
}

static pa_status_t fill_decode_args(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                                    void *out, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *lens,
                                    int64_t rows, int32_t num_q_heads, int32_t max_len,
                                    float scale, void *workspace, size_t workspace_bytes,
                                    pa::DecodeArgs &a, int &group, bool partitioned = true) {
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if ((st = check_q_dtype(pool->kv_dtype, q_dtype)) != PA_OK) return st;
  if ((st = check_heads(num_q_heads, pool->num_kv_heads, &group)) != PA_OK) return st;
  if (!q || !out || !block_tables || !lens) return fail(PA_E_ARG, "NULL array argument");
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)workspace) & 15)
    return fail(PA_E_ARG, "q, out and workspace must be 16-byte aligned");
  if (max_blocks_per_seq <= 0) return fail(PA_E_ARG, "max_blocks_per_seq must be > 0");
  if (max_len <= 0) return fail(PA_E_ARG, "max length must be > 0");
  if ((int64_t)max_len > (int64_t)max_blocks_per_seq * pool->block_size)
    return fail(PA_E_ARG, "max length %d exceeds max_blocks_per_seq * block_size", max_len);
  if (!(scale > 0.f) || !(scale <= FLT_MAX))
    return fail(PA_E_ARG, "scale %g must be positive and finite", (double)scale);
  const int max_blocks = (max_len + kTileRows - 1) / kTileRows;
  const int pb = decode_part_blocks(rows, pool->num_kv_heads, max_blocks);
  const int parts = max_parts_for(max_len, pb);
  const WsLayout w =
      partitioned ? ws_layout(rows, num_q_heads, pool->head_dim, parts) : WsLayout{};
  if (w.total > 0 && (workspace == nullptr || workspace_bytes < w.total))
    return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  a = pa::DecodeArgs{};
  a.k = pool->k;
  a.v = pool->v;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.q = q;
  a.out = out;
  a.bt = block_tables;
  a.ctx = lens;
  char *ws = reinterpret_cast<char *>(workspace);
  a.ws_acc = w.total ? reinterpret_cast<float *>(ws + w.acc_off) : nullptr;
  a.ws_m = w.total ? reinterpret_cast<float *>(ws + w.m_off) : nullptr;
  a.ws_l = w.total ? reinterpret_cast<float *>(ws + w.l_off) : nullptr;
  a.num_kv_heads = pool->num_kv_heads;
  a.num_q_heads = num_q_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_blocks = pb;
  a.max_parts = parts;
  a.qk_scale = scale * 1.4426950408889634f;
  a.bs_shift = pool->block_size == 32 ? 1 : 0;
  return PA_OK;
}

// pa_decode, and pa_decode_append when k_new is set (new rows read by the decode,
// stored into the pool by its merge kernel).
static pa_status_t decode_call(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                               const void *k_new, const void *v_new, void *out,
                               const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int64_t *slot_mapping,
                               int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                               float scale, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (num_seqs < 0) return fail(PA_E_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  pa::DecodeArgs a;
  int group = 0;
  pa_status_t st = fill_decode_args(pool, q, q_dtype, out, block_tables, max_blocks_per_seq,
                                    context_lens, num_seqs, num_q_heads, max_context_len, scale,
                                    nullptr, 0, a, group, /*partitioned=*/false);
  if (st != PA_OK) return st;
  const WsLayout w = stream_layout(num_seqs, num_q_heads, pool->head_dim, max_context_len);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  char *ws = reinterpret_cast<char *>(workspace);
  a.ws_acc = reinterpret_cast<float *>(ws + w.acc_off);
  a.ws_m = reinterpret_cast<float *>(ws + w.m_off);
  a.ws_l = reinterpret_cast<float *>(ws + w.l_off);
  a.hdr = reinterpret_cast<int32_t *>(ws + w.hdr_off);
  a.max_parts = stream_pieces(max_context_len);
  a.num_seqs = num_seqs;
  a.min_tpw = kMinTilesPerWave;
  a.seg_cost = kSegCost;
  if (k_new != nullptr) {
    a.k_new = k_new;
    a.v_new = v_new;
    a.pool_k = pool->k;
    a.pool_v = pool->v;
    a.slots_out = slot_mapping;
  }
  const bool stream_loads = (pool->flags & PA_POOL_SHARED_BLOCKS) == 0;
  return hip_status(pa::launch_decode_stream(a, pool->kv_dtype, q_dtype, pool->head_dim, group,
                                             num_seqs, stream_loads, stream),
                    k_new ? "pa_decode_append launch" : "pa_decode launch");
}

pa_status_t pa_decode(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype, void *out,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_context_len, float scale, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return decode_call(pool, q, q_dtype, nullptr, nullptr, out, block_tables, max_blocks_per_seq,
                     context_lens, nullptr, num_seqs, num_q_heads, max_context_len, scale,
                     workspace, workspace_bytes, stream);
}

pa_status_t pa_decode_append(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                             const void *k_new, const void *v_new, void *out,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int64_t *slot_mapping,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                             float scale, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (!k_new || !v_new) return fail(PA_E_ARG, "NULL k_new / v_new");
  if (((uintptr_t)k_new | (uintptr_t)v_new) & 15)
    return fail(PA_E_ARG, "k_new and v_new must be 16-byte aligned");
  if ((uintptr_t)slot_mapping & 7) return fail(PA_E_ARG, "slot_mapping must be 8-byte aligned");
  if (!is_quantised(pool->kv_dtype))
    return decode_call(pool, q, q_dtype, k_new, v_new, out, block_tables, max_blocks_per_seq,
                       context_lens, slot_mapping, num_seqs, num_q_heads, max_context_len, scale,
                       workspace, workspace_bytes, stream);
  // 1-byte pools: the new rows (in q's dtype) are quantised on write, their slots
  // taken from the tables, then the decode reads them from the pool
  if (num_seqs < 0) return fail(PA_E_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  pa::DecodeArgs probe;
  int group = 0;
  st = fill_decode_args(pool, q, q_dtype, out, block_tables, max_blocks_per_seq, context_lens,
                        num_seqs, num_q_heads, max_context_len, scale, nullptr, 0, probe, group,
                        /*partitioned=*/false);
  if (st != PA_OK) return st;
  if (workspace == nullptr ||
      workspace_bytes < stream_layout(num_seqs, num_q_heads, pool->head_dim, max_context_len).total)
    return decode_call(pool, q, q_dtype, nullptr, nullptr, out, block_tables, max_blocks_per_seq,
                       context_lens, nullptr, num_seqs, num_q_heads, max_context_len, scale,
                       workspace, workspace_bytes, stream);  // reports the workspace error
  pa::CacheWriteArgs w{};
  w.k = pool->k;
  w.v = pool->v;
  w.k_scale = pool->k_scale;
  w.v_scale = pool->v_scale;
  w.k_new = k_new;
  w.v_new = v_new;
  w.slots = nullptr;
  w.num_blocks = pool->num_blocks;
  w.num_tokens = num_seqs;
  w.num_kv_heads = pool->num_kv_heads;
  w.row_bytes = pool->head_dim;
  w.block_size = pool->block_size;
  w.bt = block_tables;
  w.ctx = context_lens;
  w.slots_out = slot_mapping;
  w.mbps = max_blocks_per_seq;
  st = hip_status(pa::launch_cache_write_quant(w, pool->kv_dtype, q_dtype, pool->head_dim, stream),
                  "pa_decode_append quantised write");
  if (st != PA_OK) return st;
  return decode_call(pool, q, q_dtype, nullptr, nullptr, out, block_tables, max_blocks_per_seq,
                     context_lens, nullptr, num_seqs, num_q_heads, max_context_len, scale,
                     workspace, workspace_bytes, stream);
}

pa_status_t pa_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (bytes == 0) return PA_OK;
  if (!src || !sink) return fail(PA_E_ARG, "NULL src or sink");
  if (((uintptr_t)src & 15) || (bytes & 15))
    return fail(PA_E_ARG, "src must be 16-byte aligned and bytes a multiple of 16");
  return hip_status(pa::launch_stream_read(src, bytes, sink, stream), "pa_stream_read launch");
}

// ---- pa_decode_append_noalloc: the same call with its scratch in a static array ----
// Device memory of fixed size that the library holds for the life of the process
// (the code object's static data: one copy on every GPU the library runs on).  In
// host code `scratch` names a host-side stand-in, never the device copy: its device
// address comes from hipGetSymbolAddress, once per device with that device current,
// and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

static pa_status_t scratch_address(void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices];  // device address of scratch on each device, or null
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_E_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                        "hipGetSymbolAddress(scratch)");
    addr[dev] = p;
  }
  *out = addr[dev];
  return PA_OK;
}

size_t pa_noalloc_scratch_bytes(void) { return kScratchBytes; }

pa_status_t pa_decode_append_noalloc(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                                     const void *k_new, const void *v_new, void *out,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int64_t *slot_mapping,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_context_len, float scale, hipStream_t stream) {
  if (num_seqs < 0) return fail(PA_E_ARG, "num_seqs must be >= 0");
  if (num_seqs == 0) return PA_OK;
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (num_q_heads <= 0 || max_context_len <= 0)
    return fail(PA_E_ARG, "num_q_heads and max_context_len must be > 0");
  // the decode's pieces, (m, l) and split header, as pa_decode_workspace_size counts
  // them; nothing in that region needs to start at zero
  const size_t need = stream_layout(num_seqs, num_q_heads, pool->head_dim, max_context_len).total;
  if (need > kScratchBytes)
    return fail(PA_E_WORKSPACE,
                "pa_decode_append_noalloc: these sizes need %zu bytes of scratch, the static "
                "scratch holds %zu (use pa_decode_append with a workspace)",
                need, kScratchBytes);
  void *ws = nullptr;
  if ((st = scratch_address(&ws)) != PA_OK) return st;
  return pa_decode_append(pool, q, q_dtype, k_new, v_new, out, block_tables, max_blocks_per_seq,
                          context_lens, slot_mapping, num_seqs, num_q_heads, max_context_len,
                          scale, ws, kScratchBytes, stream);
}

// Workspace of the mixed step.  f16, bf16, fp8 and int8 KV (MFMA prefill tiles): a
// header int, the prefill tile list, then the balanced-split decode workspace of
// the one-token rows (pieces for every sequence, as pa_decode lays them out).  fp32
// KV runs every query row through the partitioned decode path (per-row
// partitions).
struct MixedLayout {
  size_t hdr_off, p_off, acc_off, m_off, l_off, stream_off, total;
  WsLayout stream;  // offsets relative to stream_off
  int p_bound, part_blocks, max_parts, qtok;
};

MixedLayout mixed_layout(int kv_dtype, int64_t S, int64_t T, int Hq, int Hkv, int D,
                         int max_seq_len) {
  MixedLayout w{};
  const int max_blocks = (max_seq_len + kTileRows - 1) / kTileRows;
  if (pa::mixed_uses_tiles(kv_dtype)) {
    w.qtok = pa::mixed_tile_rows() / (Hq / Hkv);
    w.p_bound = (int)((T + w.qtok - 1) / w.qtok + S);
    w.max_parts = stream_pieces(max_seq_len);
    w.stream = stream_layout(S, Hq, D, max_seq_len);
    w.hdr_off = 0;
    w.p_off = align256(sizeof(int32_t));
    w.stream_off = w.p_off + align256((size_t)w.p_bound * sizeof(int32_t));
    w.total = w.stream_off + w.stream.total;
    return w;
  }
  w.part_blocks = decode_part_blocks(T, Hkv, max_blocks);
  w.max_parts = (max_blocks + w.part_blocks - 1) / w.part_blocks;
  const size_t n_ml = (size_t)T * Hq * w.max_parts;
  w.acc_off = 0;
  w.m_off = w.acc_off + align256(n_ml * D * sizeof(float));
  w.l_off = w.m_off + align256(n_ml * sizeof(float));
  w.total = w.l_off + align256(n_ml * sizeof(float));
  return w;
}

size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t kv_dtype) {
  (void)max_query_len;
  if (num_seqs <= 0 || num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || max_seq_len <= 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  const int g = num_q_heads / num_kv_heads;  // the groups pa_prefill_chunk accepts
  if (g != 1 && g != 2 && g != 4 && g != 8) return 0;
  return mixed_layout(kv_dtype, num_seqs, num_q_tokens, num_q_heads, num_kv_heads, head_dim,
                      max_seq_len)
      .total;
}

pa_status_t pa_prefill_chunk(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                             void *out, const int32_t *query_start_loc, const int32_t *seq_lens,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                             int32_t max_query_len, int32_t max_seq_len, float scale,
                             void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs < 0 || num_q_tokens < 0) return fail(PA_E_ARG, "negative num_seqs/num_q_tokens");
  if (num_seqs == 0 || num_q_tokens == 0) return PA_OK;
  if (!query_start_loc) return fail(PA_E_ARG, "query_start_loc is NULL");
  if (max_query_len <= 0 || max_query_len > max_seq_len)
    return fail(PA_E_ARG, "max_query_len %d must be in [1, max_seq_len]", max_query_len);
  if (num_seqs >= (1 << 19)) return fail(PA_E_UNSUPPORTED, "num_seqs must be < 2^19");
  pa::MixedArgs m{};
  int group = 0;
  pa_status_t st = fill_decode_args(pool, q, q_dtype, out, block_tables, max_blocks_per_seq,
                                    seq_lens, num_q_tokens, num_q_heads, max_seq_len, scale,
                                    nullptr, 0, m.dec, group, /*partitioned=*/false);
  if (st != PA_OK) return st;
  const MixedLayout w = mixed_layout(pool->kv_dtype, num_seqs, num_q_tokens, num_q_heads,
                                     pool->num_kv_heads, pool->head_dim, max_seq_len);
  const bool tiles = pa::mixed_uses_tiles(pool->kv_dtype);
  if (tiles && max_query_len > 4096 * w.qtok)
    return fail(PA_E_UNSUPPORTED, "max_query_len %d too long (limit %d)", max_query_len,
                4096 * w.qtok);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(PA_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  char *ws = reinterpret_cast<char *>(workspace);
  m.qsl = query_start_loc;
  m.num_seqs = num_seqs;
  if (tiles) {
    char *sw = ws + w.stream_off;
    m.hdr = reinterpret_cast<int32_t *>(ws + w.hdr_off);
    m.p_items = reinterpret_cast<int32_t *>(ws + w.p_off);
    m.p_bound = w.p_bound;
    m.qtok = w.qtok;
    m.dec.ws_acc = reinterpret_cast<float *>(sw + w.stream.acc_off);
    m.dec.ws_m = reinterpret_cast<float *>(sw + w.stream.m_off);
    m.dec.ws_l = reinterpret_cast<float *>(sw + w.stream.l_off);
    m.dec.hdr = reinterpret_cast<int32_t *>(sw + w.stream.hdr_off);
    m.dec.max_parts = w.max_parts;
    m.dec.num_seqs = num_seqs;
    m.dec.min_tpw = kMinTilesPerWave;
    m.dec.seg_cost = kSegCost;
    m.dec.qsl = query_start_loc;
  } else {
    m.dec.ws_acc = reinterpret_cast<float *>(ws + w.acc_off);
    m.dec.ws_m = reinterpret_cast<float *>(ws + w.m_off);
    m.dec.ws_l = reinterpret_cast<float *>(ws + w.l_off);
    m.dec.part_blocks = w.part_blocks;
    m.dec.max_parts = w.max_parts;
  }
  const bool stream_loads = (pool->flags & PA_POOL_SHARED_BLOCKS) == 0;
  return hip_status(pa::launch_mixed(m, pool->kv_dtype, q_dtype, pool->head_dim, group,
                                     num_q_tokens, stream_loads, stream),
                    "pa_prefill_chunk launch");
}

}  // extern "C"

struct pa_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

// Capture one decode step -- slot mapping, the new rows' K/V write (quantising
// for 1-byte pools), the balanced-split decode and its merge -- into a HIP graph,
// built once and replayed every step ("从KV Cache到vLLM" 4.2, 6.2).  Every launch
// is validated as in the eager calls; no memset node is recorded.
pa_status_t pa_decode_step_graph(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                                 const void *k_new, const void *v_new, int32_t new_dtype,
                                 void *out, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *context_lens,
                                 const int32_t *query_start_loc, int64_t *slot_mapping,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 float scale, void *workspace, size_t workspace_bytes,
                                 pa_graph_t **graph) {
  if (!graph) return fail(PA_E_ARG, "graph is NULL");
  *graph = nullptr;
  if (num_seqs <= 0) return fail(PA_E_ARG, "num_seqs must be > 0");
  pa_status_t st = check_pool(pool, true);
  if (st != PA_OK) return st;
  if (!is_quantised(pool->kv_dtype) && new_dtype != pool->kv_dtype)
    return fail(PA_E_UNSUPPORTED, "new_dtype %d must equal kv_dtype %d for float KV", new_dtype,
                pool->kv_dtype);
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess)
    return hip_status(hipGetLastError(), "capture stream");
  // relaxed: the first launch of a kernel instantiation queries its occupancy
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_status(e, "hipStreamBeginCapture");
  }
  if (is_quantised(pool->kv_dtype) && new_dtype != q_dtype) {
    st = pa_slot_mapping(block_tables, max_blocks_per_seq, pool->block_size, query_start_loc,
                         context_lens, num_seqs, num_seqs, slot_mapping, cs);
    if (st == PA_OK)
      st = kv_cache_write_quant(pool, k_new, v_new, new_dtype, slot_mapping, num_seqs, cs);
    if (st == PA_OK)
      st = pa_decode(pool, q, q_dtype, out, block_tables, max_blocks_per_seq, context_lens,
                     num_seqs, num_q_heads, max_context_len, scale, workspace, workspace_bytes,
                     cs);
  } else {  // the write rides in the decode call (pa_decode_append)
    st = pa_decode_append(pool, q, q_dtype, k_new, v_new, out, block_tables, max_blocks_per_seq,
                          context_lens, slot_mapping, num_seqs, num_q_heads, max_context_len,
                          scale, workspace, workspace_bytes, cs);
  }
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (st != PA_OK || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return st != PA_OK ? st : hip_status(e, "hipStreamEndCapture");
  }
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_status(e, "hipGraphInstantiate");
  }
  pa_graph *h = new (std::nothrow) pa_graph();
  if (!h) {
    (void)hipGraphExecDestroy(x);
    (void)hipGraphDestroy(g);
    return fail(PA_E_ARG, "out of host memory");
  }
  h->graph = g;
  h->exec = x;
  *graph = h;
  return PA_OK;
}

pa_status_t pa_graph_launch(pa_graph_t *graph, hipStream_t stream) {
  if (!graph || !graph->exec) return fail(PA_E_ARG, "graph is NULL");
  return hip_status(hipGraphLaunch(graph->exec, stream), "hipGraphLaunch");
}

void pa_graph_destroy(pa_graph_t *graph) {
  if (!graph) return;
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  if (graph->graph) (void)hipGraphDestroy(graph->graph);
  delete graph;
}

}  // extern "C"
