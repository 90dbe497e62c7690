// Kernel argument blocks and launchers shared between the C-ABI layer and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

struct DecodeArgs {
  const void *k;
  const void *v;
  const float *k_scale;
  const float *v_scale;
  const void *q;
  void *out;
  const int32_t *bt;   // [num_seqs][max_blocks_per_seq]
  const int32_t *ctx;  // [num_seqs] context (KV) length per sequence
  float *ws_acc;       // [num_seqs][num_q_heads][max_parts][head_dim]
  float *ws_m;         // [num_seqs][num_q_heads][max_parts]
  float *ws_l;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_blocks_per_seq;
  int32_t part_blocks;  // blocks per context partition (partitioned path)
  int32_t max_parts;    // partitions (or pieces) of the longest context
  float qk_scale;       // softmax scale * log2(e)
  // balanced split: waves share the work evenly; see decode_stream
  int32_t *hdr;         // [2 + num_seqs]: cost units per first-round wave, each sequence's
                        // first cost unit, cost units per later wave
  int32_t num_seqs;
  int32_t num_waves;    // waves launched
  int32_t min_tpw;      // lower bound on cost units per wave
  int32_t seg_cost;     // cost units charged for each (sequence, kv head) segment start
  int32_t skew;         // two workgroups per CU: the first round's waves take tpw + d cost
                        // units and the second round's tpw - d, d = tpw * skew / 256
  int32_t bs_shift;     // log2(block size / 16): tiles of 16 rows per block, as a shift
  // mixed step: [num_seqs + 1] query starts; only q_len == 1 sequences are decoded,
  // sequence s's query/output row being qsl[s] (nullptr: every sequence, row s)
  const int32_t *qsl;
  // fused append (pa_decode_append; nullptr otherwise): each sequence's new K/V row,
  // [num_seqs][num_kv_heads][head_dim] in the pool's type, at position ctx[s] - 1.
  // The decode reads it from here in place of the pool row; the merge kernel then
  // stores it into the pool (pool_k / pool_v) and its slot into slots_out (if set).
  const void *k_new;
  const void *v_new;
  void *pool_k;
  void *pool_v;
  int64_t *slots_out;
};

struct MixedArgs {
  DecodeArgs dec;       // pools, q/out, tables, seq_lens (as ctx); with the MFMA tiles (all
                        // but fp32 KV) also the balanced-split decode of the one-token rows
                        // (dec.qsl set)
  const int32_t *qsl;   // [num_seqs + 1]
  int32_t *hdr;         // [1]: prefill tiles listed (written by the prep kernel)
  int32_t *p_items;     // [p_bound]
  int32_t num_seqs;
  int32_t p_bound;
  int32_t qtok;         // query tokens per prefill tile (tile rows / G)
};

struct CacheWriteArgs {
  void *k;
  void *v;
  float *k_scale;     // 1-byte pools (quantise-on-write)
  float *v_scale;
  const void *k_new;
  const void *v_new;
  const int64_t *slots;
  int64_t num_blocks;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t row_bytes;   // head_dim * element bytes
  int32_t block_size;  // tokens per physical block (16 or 32)
  // decode append (slots == nullptr): token t is sequence t's new row at position
  // ctx[t] - 1 of its table row; its slot is computed here and stored to slots_out
  const int32_t *bt;
  const int32_t *ctx;
  int64_t *slots_out;
  int32_t mbps;
};

// Block tiles (and scales) copied from one pool to another of the same geometry;
// the same pool on both sides is the copy-on-write case.  Any of the pointers may
// be device addresses of pinned host memory.
struct BlockCopyArgs {
  const void *src_k;
  const void *src_v;
  const float *src_ks;
  const float *src_vs;
  void *dst_k;
  void *dst_v;
  float *dst_ks;
  float *dst_vs;
  const int32_t *pairs;
  int32_t num_pairs;
  int32_t num_kv_heads;
  int32_t tile_bytes;  // 16 * head_dim * element bytes
};

// Input checks (debugging aid): tables and lengths of one call.
struct CheckTablesArgs {
  const int32_t *bt;    // [num_seqs][mbps]
  const int32_t *lens;  // [num_seqs]
  const int32_t *qsl;   // [num_seqs + 1] or nullptr
  int32_t *flags;       // OR-ed PA_CHECK_* bits
  int64_t num_blocks;
  int32_t mbps;
  int32_t block_size;
  int32_t max_len;
};
hipError_t launch_check_tables(const CheckTablesArgs &a, int32_t num_seqs, hipStream_t st);
hipError_t launch_check_slots(const int64_t *slots, int32_t n, int64_t num_slots, int32_t *flags,
                              hipStream_t st);
hipError_t launch_check_pairs(const int32_t *pairs, int32_t n, int64_t num_blocks,
                              int32_t *flags, hipStream_t st);

// stream_loads: read K/V tiles with the nontemporal hint (off when blocks are shared)
hipError_t launch_decode_stream(const DecodeArgs &a, int kv_dtype, int q_dtype, int head_dim,
                                int group, int num_seqs, bool stream_loads, hipStream_t st);
hipError_t launch_decode_f32(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                             bool stream_loads, hipStream_t st);
hipError_t launch_decode_f16(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                             bool stream_loads, hipStream_t st);
hipError_t launch_decode_bf16(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                              bool stream_loads, hipStream_t st);
hipError_t launch_decode_fp8(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                             bool stream_loads, hipStream_t st);
hipError_t launch_decode_i8(const DecodeArgs &a, int q_dtype, int D, int G, int num_seqs,
                            bool stream_loads, hipStream_t st);
bool mixed_uses_tiles(int kv_dtype);
int mixed_tile_rows();  // query rows (token, head) per prefill tile of the mixed kernel
hipError_t launch_mixed(const MixedArgs &a, int kv_dtype, int q_dtype, int head_dim, int group,
                        int num_rows, bool stream_loads, hipStream_t st);
hipError_t launch_cache_write(const CacheWriteArgs &a, hipStream_t st);
hipError_t launch_cache_write_quant(const CacheWriteArgs &a, int kv_dtype, int src_dtype,
                                    int head_dim, hipStream_t st);
hipError_t launch_block_copy(const BlockCopyArgs &a, hipStream_t st);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t st);
hipError_t launch_slot_mapping(const int32_t *bt, int32_t mbps, int32_t block_size,
                               const int32_t *qsl,
                               const int32_t *seq_lens, int32_t num_seqs, int64_t *slots,
                               hipStream_t st);


}  // namespace pa
