/*
 * pa.h -- paged KV-cache attention on one MI355X (gfx950): the C ABI.
 *
 * Sources for what each call computes (the pages are the authority):
 *  [P1] "vLLM ... PagedAttention / Prefix Sharing / Continuous Batching"
 *       (uml.org.cn), sections PagedAttention, Prefix Sharing, Continuous Batching.
 *  [P2] "3、核心概念：LLM推理原理、KV Cache、PagedAttention、连续批处理"
 *       (5688vip.com course, chapter 3), sections 3.1-3.3.
 *  [P3] "从KV Cache到vLLM：大模型推理提速与显存优化实战" (xxqk.cn),
 *       sections 1.1-1.2 (attention against the cache), 2.1-2.3 (KV size,
 *       GQA, INT8/FP8 storage), 3.2 (16-token pages).
 *
 * Conventions shared by every call
 *  - Every pointer is a DEVICE pointer unless its comment says "host".
 *  - The pools (k, v) and the q, out and workspace arrays of the attention calls
 *    must be 16-byte aligned (PA_E_ARG otherwise); kernels move 16 bytes per lane.
 *  - Calls validate their scalar arguments on the host, then only enqueue
 *    work on `stream`; they never allocate, free or synchronise.  A non-OK
 *    status means nothing was enqueued (PA_E_HIP: a launch was attempted and
 *    failed; pa_last_error() holds the HIP message).
 *  - The caller owns every buffer.  Scratch memory comes from the caller's
 *    `workspace` (size from the matching *_workspace_size call).
 *  - Contents of device arrays are NOT checked (that would need a sync):
 *    block ids outside [0, num_blocks), negative or too-long lengths,
 *    duplicate write slots or overlapping copy pairs are undefined behaviour.
 *
 * KV pool layout (the pages fix the paging, not the memory layout):
 *    k, v : [num_blocks][num_kv_heads][block_size][head_dim], kv_dtype
 *    k_scale, v_scale : float32 [num_blocks][num_kv_heads] for 1-byte codes
 *  with block_size 16 or 32 tokens ([P2] 3.2), so one (block, kv head) tile of
 *  block_size token rows is contiguous: 4 KiB for fp16/bf16 at head_dim 128 and
 *  16 tokens, 2 KiB for fp8/int8; a 32-token block holds two such 16-row
 *  halves per kv head, under one scale.
 *
 * GQA ([P3] 2.2): query head h reads kv head h / (num_q_heads / num_kv_heads).
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3, /* OCP E4M3FN codes: bias 7, max 448, NaN = S.1111.111 */
  PA_I8 = 4        /* symmetric int8 codes, value = code * scale */
} pa_dtype_t;

typedef enum pa_status {
  PA_OK = 0,
  PA_E_ARG = 1,         /* a null pointer or an out-of-range scalar */
  PA_E_UNSUPPORTED = 2, /* a valid but unimplemented shape or dtype combination */
  PA_E_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
  PA_E_HIP = 4,         /* a HIP launch failed */
  PA_E_NO_BLOCKS = 5    /* block manager: the free list cannot cover the request */
} pa_status_t;

/* Host struct describing caller-owned device memory. */
/* pa_kv_pool_t.flags */
#define PA_POOL_SHARED_BLOCKS 1 /* some physical blocks appear in several sequences'
                                   tables (prefix sharing, [P1] Prefix Sharing): pa_decode
                                   then reads K/V tiles with ordinary cached loads so that
                                   repeated reads of a shared tile can hit in cache.
                                   Without it every tile is read once per call and is
                                   streamed with a nontemporal hint. */

typedef struct pa_kv_pool {
  void *k;          /* [num_blocks][num_kv_heads][block_size][head_dim] */
  void *v;          /* same shape */
  float *k_scale;   /* [num_blocks][num_kv_heads]; NULL unless kv_dtype is 1 byte */
  float *v_scale;
  int64_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size; /* 16 or 32 tokens ([P2] 3.2; [P3] 3.2 names 16) */
  int32_t head_dim;   /* 64 or 128 */
  int32_t kv_dtype;   /* pa_dtype_t */
  int32_t flags;      /* PA_POOL_* bits; 0 for none */
} pa_kv_pool_t;

/* Version string of the library (static storage). */
const char *pa_version(void);

/* Text of a status code (static storage). */
const char *pa_status_string(pa_status_t s);

/* Detail of the last non-OK status returned on the calling thread. */
const char *pa_last_error(void);

/*
 * pa_slot_mapping -- where each new token's K/V goes ([P2] 3.2: a decode
 * step writes the new token at the end of the current block; a block that is
 * full is followed by a new physical block from the block table).
 *
 * For sequence s, query rows t in [query_start_loc[s], query_start_loc[s+1])
 * are the q_len newest tokens; row t sits at logical position
 *     p = seq_lens[s] - q_len + (t - query_start_loc[s])
 * and its slot is   block_tables[s][p / bs] * bs + p % bs,  bs = block_size
 * (16 or 32; PA_E_UNSUPPORTED otherwise).
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, [0] = 0,
 *                   [num_seqs] = num_tokens
 *   seq_lens        int32 [num_seqs], KV length including the new rows
 *   slot_mapping    int64 [num_tokens] (output)
 */
pa_status_t pa_slot_mapping(const int32_t *block_tables, int32_t max_blocks_per_seq,
                            int32_t block_size, const int32_t *query_start_loc,
                            const int32_t *seq_lens,
                            int32_t num_seqs, int32_t num_tokens, int64_t *slot_mapping,
                            hipStream_t stream);

/*
 * kv_cache_write -- scatter new tokens' K and V into the pools by slot
 * ([P2] 3.2 prefill writes every prompt token, decode appends one token).
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim], dtype = pool kv_dtype
 *   slot_mapping  int64 [num_tokens]; slot = block * block_size + offset; slot < 0
 *                 means "no token" and is skipped.
 * A pure bit copy.  Pools with 1-byte codes return PA_E_UNSUPPORTED: they are
 * written by kv_cache_write_quant.
 */
pa_status_t kv_cache_write(const pa_kv_pool_t *pool, const void *k_new, const void *v_new,
                           const int64_t *slot_mapping, int32_t num_tokens,
                           hipStream_t stream);

/*
 * kv_cache_write_quant -- write new tokens' K and V into a pool of 1-byte codes
 * (fp8 E4M3FN or int8), keeping one scale per (block, kv head) ([P3] 2.2-2.3:
 * the cache may be stored as INT8 or FP8, one byte per element).
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim] values of src_dtype
 *                 (PA_F32, PA_F16 or PA_BF16)
 *   slot_mapping  int64 [num_tokens]; slot < 0 means "no token" and is skipped.
 * The rows one call writes into a block must be that block's next rows, in
 * order and contiguous in token order (pa_slot_mapping of one step gives
 * exactly that); rows below them already hold data.  The pages fix no scale
 * policy for a block that fills over several steps; this one, per (block, kv
 * head), in fp32 with round-to-nearest-even:
 *   s_new = max(s_old, amax / qmax)   amax over the new rows, qmax 448 or 127,
 *                                     s_old = 0 when the new rows start at row 0
 *   if s_new > s_old, each earlier code c becomes encode(value(c) * (s_old / s_new))
 *   each new value x becomes encode(x / s_new)   (code 0 while s_new is 0)
 *   encode = clamp to [-qmax, qmax], then nearest code, ties to even.
 * A tile whose rows are all zero has scale 0.  PA_E_UNSUPPORTED for pools of
 * other types (see kv_cache_write).
 */
pa_status_t kv_cache_write_quant(const pa_kv_pool_t *pool, const void *k_new, const void *v_new,
                                 int32_t src_dtype, const int64_t *slot_mapping,
                                 int32_t num_tokens, hipStream_t stream);

/*
 * kv_block_copy -- copy-on-write duplication of physical blocks ([P1]
 * Prefix Sharing: when a request that shares a page diverges, the shared page
 * stays as it is and the new token goes into a copy of it).
 *   src_dst int32 [num_pairs][2]: every kv head's K and V tile of block src
 *           (and both scales, for 1-byte pools) is copied to block dst.
 * Destinations must be unique and disjoint from the sources.
 */
pa_status_t kv_block_copy(const pa_kv_pool_t *pool, const int32_t *src_dst, int32_t num_pairs,
                          hipStream_t stream);

/*
 * kv_swap -- move blocks between two pools of the same kv_dtype, num_kv_heads
 * and head_dim, typically the device pool and a host pool in pinned memory
 * ([P1] PagedAttention: under memory pressure pages go out to CPU memory and come
 * back when the request runs again).
 *   src_dst int32 [num_pairs][2] (device or pinned host memory): every kv head's
 *           K and V tile (and both scales, for 1-byte pools) of block src of
 *           `src` is copied to block dst of `dst`.
 * Each pool's k, v and scales must be device memory or pinned host memory
 * (hipHostMalloc, torch pin_memory); pageable memory gives PA_E_ARG.  One kernel
 * moves every pair: the copies to or from host memory cross PCIe.  Destinations
 * must be unique; when src and dst are one pool, also disjoint from the sources.
 */
pa_status_t kv_swap(const pa_kv_pool_t *dst, const pa_kv_pool_t *src, const int32_t *src_dst,
                    int32_t num_pairs, hipStream_t stream);

/* Workspace bytes pa_decode needs for these sizes (0 is a valid answer). */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_context_len);

/*
 * pa_decode -- one decode step: every sequence's single new query token
 * attends to all of its cached tokens through its block table ([P2] 3.2: the
 * kernel reads the scattered blocks by indirection through the block table;
 * [P3] 1.1: dot the query with every cached key, softmax, weight the values).
 *   q            [num_seqs][num_q_heads][head_dim], q_dtype
 *   out          same shape and dtype as q (fp32 accumulation, rounded to
 *                nearest even on store)
 *   block_tables int32 [num_seqs][max_blocks_per_seq]
 *   context_lens int32 [num_seqs], >= 1: cached tokens including this step's
 *                token, whose K/V must already be written
 *   max_context_len  host upper bound of context_lens (sizes the split)
 *   scale        softmax scale applied to q.k (1/sqrt(head_dim) usually); it
 *                must be positive and finite (PA_E_ARG otherwise), here and in
 *                pa_decode_append and pa_prefill_chunk
 * dtypes: kv f32/f16/bf16 need q_dtype == kv_dtype; fp8/int8 KV take f16 or
 * bf16 queries.  num_q_heads / num_kv_heads must be 1, 2, 4 or 8.
 */
pa_status_t pa_decode(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype, void *out,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_context_len, float scale, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_append -- a decode step with its cache write fused in: for every
 * sequence the new token's K/V row goes to the end of its last block ([P2] 3.2:
 * compute the token's K/V, write it at the end of the current block, then
 * attend) and its query attends to all context_lens[s] tokens, the new one
 * included.  The result equals pa_slot_mapping (one row per sequence at
 * position context_lens[s] - 1), kv_cache_write and pa_decode run in that order:
 * out is bit-identical and the pools byte-identical.  For f32/f16/bf16 pools
 * the attention reads the new rows from k_new / v_new, so the write needs no
 * launch of its own (two launches); the pool rows are stored within the call,
 * after every read of the pool.
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim], 16-byte aligned: the
 *                 pool's kv_dtype for f32/f16/bf16 pools; for fp8/int8 pools
 *                 q_dtype, quantised on write by kv_cache_write_quant's policy
 *                 (the result then equals pa_slot_mapping, kv_cache_write_quant
 *                 and pa_decode; three launches, the write's slots taken from the
 *                 block tables)
 *   slot_mapping  int64 [num_seqs] receives each row's slot
 *                 (block * block_size + offset; -1 for a context length < 1);
 *                 may be NULL
 *   the rest      as pa_decode; the workspace is pa_decode_workspace_size's
 * Errors as pa_decode, plus PA_E_ARG for NULL or misaligned k_new / v_new.
 * Sequences' new rows must sit in distinct blocks (each writes the end of a last
 * block it owns alone, as copy-on-write guarantees).
 */
pa_status_t pa_decode_append(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                             const void *k_new, const void *v_new, void *out,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int64_t *slot_mapping,
                             int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                             float scale, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * pa_decode_append_noalloc -- pa_decode_append for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It takes no workspace: the decode's scratch (its
 * partial pieces, their (m, l) and the split header) lives in a static device
 * array of pa_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on
 * every GPU it runs on until the process ends.  Arguments, results and errors
 * are pa_decode_append's (bit-identical outputs, pools and slots), plus
 * PA_E_WORKSPACE, with nothing enqueued, when the sizes need more scratch than
 * that (pa_decode_workspace_size of the same sizes > pa_noalloc_scratch_bytes();
 * e.g. 64 sequences x 32 query heads x head_dim 128 up to 4096 tokens need 35 MB).
 * The call allocates nothing and calls no allocating routine.  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents (nothing in
 * it needs to start at zero): calls that overlap on one GPU (other streams,
 * other threads) race and give undefined results; serialise them.  The first
 * call on each device looks up the array's device address
 * (hipGetSymbolAddress) with that device current.
 */
pa_status_t pa_decode_append_noalloc(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                                     const void *k_new, const void *v_new, void *out,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *context_lens, int64_t *slot_mapping,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_context_len, float scale, hipStream_t stream);

/* Bytes of the static scratch pa_decode_append_noalloc uses (a host constant). */
size_t pa_noalloc_scratch_bytes(void);

/*
 * pa_stream_read -- a measurement reference, not part of the attention path:
 * reads `bytes` of device memory at src once (16-byte nontemporal loads, the
 * cache hint the decode kernels use for K/V tiles) and XORs the words into
 * *sink (a device uint32; its old value is folded in, nothing needs zeroing),
 * so the achievable HBM read rate can be timed beside the attention calls in
 * the same run.  src 16-byte aligned, bytes a multiple of 16 (PA_E_ARG
 * otherwise); bytes == 0 enqueues nothing.
 */
pa_status_t pa_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Workspace bytes pa_prefill_chunk needs for these sizes and KV storage type
 * (0 for invalid sizes, including a GQA group num_q_heads / num_kv_heads other
 * than 1, 2, 4 or 8). */
size_t pa_prefill_workspace_size(int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                 int32_t max_seq_len, int32_t kv_dtype);

/*
 * pa_prefill_chunk -- one continuous-batching step ([P1] Continuous
 * Batching): chunked prefills and decodes of many sequences in one call.
 *   q               [num_q_tokens][num_q_heads][head_dim], rows packed by
 *                   sequence; out has the same shape and dtype
 *   query_start_loc int32 [num_seqs + 1]; q_len = qsl[s+1] - qsl[s] >= 1
 *                   (q_len == 1 is a decode)
 *   seq_lens        int32 [num_seqs]: KV length including the q_len new
 *                   tokens, whose K/V must already be written
 * Causality ([P2] 3.1, autoregressive order): row i of sequence s sits at
 * position seq_lens[s] - q_len + i and sees keys 0 .. that position.
 */
pa_status_t pa_prefill_chunk(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                             void *out, const int32_t *query_start_loc, const int32_t *seq_lens,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             int32_t num_seqs, int32_t num_q_tokens, int32_t num_q_heads,
                             int32_t max_query_len, int32_t max_seq_len, float scale,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ---- Input checks: a debugging aid for the arrays the calls take on trust ----
 * The calls above never read their index arrays back (that would need a
 * synchronisation): a block id outside the pool, a length past its table, a
 * repeated slot or overlapping copy pairs are undefined behaviour there.  These
 * enqueue a kernel that reads the same arrays, compares values only (no id is used
 * as an address) and ORs one bit per kind of violation into *flags, an int32 in
 * device memory that the caller zeroes beforehand and reads after synchronising.
 * The slot and pair checks compare every two entries (quadratic in the count).
 * Only num_blocks and block_size of the pool are used.  Errors: PA_E_ARG for NULL
 * arrays or flags, negative counts or a bad pool geometry; PA_E_HIP on launch.
 */
#define PA_CHECK_LEN 1      /* a length < 1, above the bound given, or past its table row */
#define PA_CHECK_BLOCK 2    /* an id in the used part of a table row outside [0, num_blocks) */
#define PA_CHECK_QSL 4      /* query_start_loc[0] != 0, or a q_len < 1 or above its seq_len */
#define PA_CHECK_SLOT 8     /* a slot >= num_blocks * block_size (negative = skipped, allowed) */
#define PA_CHECK_SLOT_DUP 16 /* two tokens with one slot (>= 0) */
#define PA_CHECK_PAIR 32    /* a copy pair id out of range, a repeated destination, or a
                               source that is some pair's destination */

/* block_tables / seq_lens (/ query_start_loc) as pa_decode or pa_prefill_chunk
 * read them: query_start_loc may be NULL (one row per sequence); max_seq_len is
 * the host bound passed to those calls. */
pa_status_t pa_check_tables(const pa_kv_pool_t *pool, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t num_seqs, int32_t max_seq_len,
                            int32_t *flags, hipStream_t stream);
/* slot_mapping as kv_cache_write / kv_cache_write_quant read it. */
pa_status_t pa_check_slots(const pa_kv_pool_t *pool, const int64_t *slot_mapping,
                           int32_t num_tokens, int32_t *flags, hipStream_t stream);
/* src_dst as kv_block_copy reads it. */
pa_status_t pa_check_copy_pairs(const pa_kv_pool_t *pool, const int32_t *src_dst,
                                int32_t num_pairs, int32_t *flags, hipStream_t stream);

/*
 * ---- A captured decode step ([P3] 4.2: the serving engine builds graphs of
 * its step at start-up; 6.2: running eagerly instead saves that memory but adds
 * latency to every step; here a HIP graph). ----
 * pa_decode_step_graph records, on a stream of its own, the calls of one
 * decode step over fixed buffers: pa_decode_append (slot mapping, the write of
 * each sequence's new K/V row -- quantised for 1-byte pools -- and the decode
 * with its merge); for a 1-byte pool whose new rows are not in q_dtype,
 * pa_slot_mapping (block_size from the pool), kv_cache_write_quant from
 * new_dtype, then pa_decode.  Arguments
 * mean what they mean in those calls (one query row per sequence:
 * query_start_loc is 0, 1, .., num_seqs; slot_mapping int64 [num_seqs] is the
 * step's scratch for the slots) and are validated at capture; nothing runs
 * then.  pa_graph_launch replays the step on `stream`, reading the buffers'
 * contents at that time: q, k_new, v_new, block tables and context lengths may
 * change between replays (contexts >= 1 and within max_blocks_per_seq *
 * block_size -- longer than max_context_len only costs balance, the split keeps
 * its pieces within the workspace); the buffers, num_seqs and the pool must
 * stay as captured.  Copy-on-write pairs vary in number per step and are not
 * part of the graph: run kv_block_copy before the replay.  Replays on one
 * stream run in order; the caller owns every buffer.
 */
typedef struct pa_graph pa_graph_t;
pa_status_t pa_decode_step_graph(const pa_kv_pool_t *pool, const void *q, int32_t q_dtype,
                                 const void *k_new, const void *v_new, int32_t new_dtype,
                                 void *out, const int32_t *block_tables,
                                 int32_t max_blocks_per_seq, const int32_t *context_lens,
                                 const int32_t *query_start_loc, int64_t *slot_mapping,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 float scale, void *workspace, size_t workspace_bytes,
                                 pa_graph_t **graph);
pa_status_t pa_graph_launch(pa_graph_t *graph, hipStream_t stream);
void pa_graph_destroy(pa_graph_t *graph);

/*
 * ---- Host block manager ([P1] PagedAttention, Prefix Sharing, Continuous
 * Batching; [P2] 3.2) -- host memory only, no device calls. ----
 * A request's cache is a list of physical blocks of block_size (16 or 32)
 * tokens, the device pool's, taken from a free list
 * of num_blocks (the device pool's blocks) as it grows: a token goes at the end of
 * the last block, a full block is followed by a fresh one.  Blocks are reference
 * counted: pa_bm_fork shares every block of a request with a new one (parallel
 * sampling), and a request that appends into a shared, partly filled last block
 * first moves to a copy of it (copy-on-write).  Full blocks enter a prefix cache
 * under a hash of the tokens up to their end; pa_bm_add reuses cached blocks for
 * a new prompt's leading full blocks (a hit is checked token by token and block
 * by block, so a hash collision cannot share wrong rows).  A block returns to the
 * free list, and leaves the prefix cache, with its last reference.
 *
 * Step protocol.  After adds, appends, forks and releases, pa_bm_step hands out
 * one step's host arrays; the caller then runs, in this order on one stream:
 * kv_block_copy over the pairs, the K/V writes of the query tokens (slot mapping
 * from the arrays), attention.  A request's query rows in a step are all its
 * tokens not yet written (the cached prefix of a prompt excluded); a block
 * enters the prefix cache in the step that writes its last token.  With that
 * order the pairs' destinations are unique and disjoint from their sources, and
 * no slot is written twice in a step.  Not thread safe: one manager per thread.
 */
typedef struct pa_block_manager pa_block_manager_t;

/* A manager over device blocks 0 .. num_blocks-1 of block_size tokens (16 or
 * 32, the pool's) and host slots 0 .. num_host_blocks-1 (a host pool for
 * swapping; 0 for none), all free.  NULL for num_blocks <= 0, num_host_blocks
 * < 0, another block_size or out of host memory. */
pa_block_manager_t *pa_bm_create(int32_t num_blocks, int32_t num_host_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager_t *bm);
/* Free device blocks (-1 for a NULL manager).  A copy source whose last
 * reference went in this step counts as free only after the next pa_bm_step. */
int32_t pa_bm_num_free(const pa_block_manager_t *bm);
/* Free host slots (-1 for a NULL manager); a slot a pending swap-in reads is
 * free again after the next pa_bm_step. */
int32_t pa_bm_num_free_host(const pa_block_manager_t *bm);
/* References to a block (-1 out of range); for tests and diagnostics. */
int32_t pa_bm_refcount(const pa_block_manager_t *bm, int32_t block);

/* New request `req` with its n >= 1 prompt tokens (host array).  *cached (may
 * be NULL) receives how many leading prompt tokens already sit in shared cached
 * blocks -- a multiple of block_size, at most n - 1 -- which the next step does not
 * compute.  PA_E_NO_BLOCKS (nothing changed) when the free list is short;
 * PA_E_ARG for a used id. */
pa_status_t pa_bm_add(pa_block_manager_t *bm, int64_t req, const int32_t *tokens, int32_t n,
                      int32_t *cached);
/* New request `child` sharing every block of `parent` (reference counts + 1).
 * PA_E_ARG if the parent has tokens no step has handed out yet. */
pa_status_t pa_bm_fork(pa_block_manager_t *bm, int64_t parent, int64_t child);
/* Append n tokens to `req` (one per decode step, or a prompt chunk); may queue
 * a copy-on-write pair.  PA_E_NO_BLOCKS (nothing changed) when the free list is
 * short. */
pa_status_t pa_bm_append(pa_block_manager_t *bm, int64_t req, const int32_t *tokens, int32_t n);
/* Drop `req`: its device blocks lose a reference each, its host slots are freed. */
pa_status_t pa_bm_release(pa_block_manager_t *bm, int64_t req);

/* ---- Swapping ([P1] PagedAttention: under memory pressure a request's pages
 * go out to CPU memory and come back when it runs again). ----
 * pa_bm_swap_out moves every block `req` holds alone to a host slot (queued as
 * a (device block, host slot) pair) and frees those device blocks; blocks it
 * shares with other requests stay on the device.  *moved (may be NULL) gets the
 * number of blocks moved.  The request must have all its tokens written; until
 * pa_bm_swap_in it cannot be appended, forked or stepped.  pa_bm_swap_in takes
 * fresh device blocks for its host slots (queued as (host slot, device block)
 * pairs).  A request moves at most once between two steps (PA_E_ARG otherwise);
 * PA_E_NO_BLOCKS (nothing changed) when slots or blocks are short.
 * Before pa_bm_step, pa_bm_swaps hands out the queued pairs (pa_bm_step refuses
 * while any are queued); the step's device work is then: kv_swap(host pool <-
 * device pool, out pairs), kv_swap(device pool <- host pool, in pairs),
 * kv_block_copy, the K/V writes, attention. */
pa_status_t pa_bm_swap_out(pa_block_manager_t *bm, int64_t req, int32_t *moved);
pa_status_t pa_bm_swap_in(pa_block_manager_t *bm, int64_t req);
/* *req = the resident request that the fewest recent steps listed (least
 * recently used; ties to the smaller id) among those with all tokens written
 * and not moved since the last step.  PA_E_NO_BLOCKS if there is none. */
pa_status_t pa_bm_lru(const pa_block_manager_t *bm, int64_t *req);
/* Where `req`'s logical blocks are: device_blocks[i] (-1 if in a host slot) and
 * host_slots[i] (-1 if on the device), *num_blocks entries. */
pa_status_t pa_bm_blocks(const pa_block_manager_t *bm, int64_t req, int32_t *device_blocks,
                         int32_t *host_slots, int32_t max_blocks, int32_t *num_blocks);
/* Hand out (and clear) the queued swap pairs: out_pairs [max_out][2] (device
 * block, host slot), in_pairs [max_in][2] (host slot, device block).  PA_E_ARG
 * (nothing changed) if either has too little room. */
pa_status_t pa_bm_swaps(pa_block_manager_t *bm, int32_t *out_pairs, int32_t max_out,
                        int32_t *num_out, int32_t *in_pairs, int32_t max_in, int32_t *num_in);
/* The host arrays of one step over the n distinct requests `reqs`, each with at
 * least one token not yet written; those tokens are its query rows:
 *   block_tables    int32 [n][max_blocks_per_seq], -1 past each request's blocks
 *   seq_lens        int32 [n]: each request's length (its tokens so far)
 *   query_start_loc int32 [n + 1]: prefix sums of the query row counts
 *   copy_pairs      int32 [max_pairs][2]: every copy-on-write pair queued since
 *                   the last step, then *num_pairs = their count (may be NULL
 *                   when none are queued).  The queue is emptied.
 * PA_E_ARG (nothing changed) for an unknown, repeated or swapped-out request,
 * one with no new token or more than max_blocks_per_seq blocks, too little pair
 * room, or swap pairs not yet handed out by pa_bm_swaps. */
pa_status_t pa_bm_step(pa_block_manager_t *bm, const int64_t *reqs, int32_t n,
                       int32_t max_blocks_per_seq, int32_t *block_tables, int32_t *seq_lens,
                       int32_t *query_start_loc, int32_t *copy_pairs, int32_t max_pairs,
                       int32_t *num_pairs);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
