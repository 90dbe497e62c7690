"""Paged attention, written out as its plain definition in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is blocked,
fused or reordered beyond what the definition states.

Pages and the facts taken from them:

* uml.org.cn vLLM article, "PagedAttention": the KV cache of each request is cut
  into fixed-size logical pages (e.g. 16 tokens); a per-request page table
  records which physical page holds each logical page, and attention stitches
  the pages back together through that table.
* 5688vip.com chapter 3, §3.2: blocks of 16 or 32 tokens; a block table maps
  logical to physical blocks, which need not be contiguous.  Prefill writes every
  prompt token's K/V into the allocated blocks; each decode step computes the
  new token's K/V and writes it at the end of the current block, taking a new
  physical block through the table when the current one is full; the kernel
  reads the scattered KV by indirection through the block table.
* "从KV Cache到vLLM" (xxqk.cn) §1.1-1.2: attention of the current query is the
  dot product with every cached key followed by the value sum weighted by the
  softmax of those products; with the cache, a step only computes the new
  token's query and appends its K/V.  §2.1: KV bytes closed form.  §2.2:
  grouped-query attention lets several query heads share one K/V head.
* uml.org.cn "Prefix Sharing": requests with a common prefix point at the same
  physical pages; a diverging token triggers copy-on-write -- the shared page is
  left untouched and the new token goes into a copied page.

Data model (logical, layout-free): a pool is an array
``[num_blocks][num_kv_heads][block_size][head_dim]``; element ``[b][h][o][:]``
is the K (or V) vector of kv head ``h`` for the token stored at offset ``o`` of
physical block ``b``.  How the GPU library lays a pool out in memory is its own
business; the tests convert.
"""
import numpy as np

from .codec import e4m3fn_decode, e4m3fn_encode, int8_decode, int8_encode

BLOCK_SIZE = 16


def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, batch, bytes_per_elem):
    """KV cache size in bytes ("从KV Cache到vLLM" §2.1).

    The factor 2 is one K and one V vector per token, per layer and per KV head.
    """
    return 2 * layers * kv_heads * head_dim * seq_len * batch * bytes_per_elem


def slot_for_position(block_table_row, pos, block_size=BLOCK_SIZE):
    """Flat slot of the token at logical position ``pos`` (5688vip §3.2).

    Logical block ``pos // block_size`` is looked up in the request's block
    table; the token sits at offset ``pos % block_size`` inside that physical
    block.  ``slot = physical_block * block_size + offset``.
    """
    logical_block = pos // block_size
    offset = pos % block_size
    return int(block_table_row[logical_block]) * block_size + offset


def _decode_values(x, codec):
    if codec is None:
        return np.asarray(x, dtype=np.float64)
    if codec == "e4m3fn":
        return e4m3fn_decode(x)
    if codec == "int8":
        return int8_decode(x)
    raise ValueError(f"unknown codec {codec!r}")


def gather_sequence(pool, block_table_row, n, scales=None, codec=None):
    """K (or V) of one request as a contiguous float64 array ``[n][H][D]``.

    The block size ``bs`` is the pool's third axis (16 or 32 tokens, 5688vip
    §3.2).  Concatenates physical blocks ``block_table_row[0 .. ceil(n/bs)-1]``
    along the token axis and keeps the first ``n`` tokens.  For 1-byte pools the
    codes are decoded and multiplied by that block's per-(block, kv_head)
    scale, ``scales[b][h]``.
    """
    bs = pool.shape[2]
    n_blocks = -(-n // bs)
    pieces = []
    for j in range(n_blocks):
        b = int(block_table_row[j])
        tile = _decode_values(pool[b], codec)  # [H][bs][D]
        if scales is not None:
            tile = tile * np.asarray(scales[b], dtype=np.float64)[:, None, None]
        pieces.append(np.transpose(tile, (1, 0, 2)))  # [bs][H][D]
    return np.concatenate(pieces, axis=0)[:n]


def attention_rows(q, K, V, scale, visible):
    """Softmax attention of query rows against one request's keys and values.

    q:       ``[nq][Hq][D]`` float64
    K, V:    ``[n][Hkv][D]`` float64
    visible: ``[nq]`` -- query row ``i`` attends to keys ``0 .. visible[i]-1``
    Query head ``h`` uses kv head ``h // (Hq // Hkv)`` (contiguous groups).

    For each row and head: ``s_t = scale * q . k_t``, ``w = softmax(s)`` over the
    visible keys, output ``sum_t w_t v_t``.
    """
    nq, hq, d = q.shape
    n, hkv, _ = K.shape
    g = hq // hkv
    out = np.zeros((nq, hq, d), dtype=np.float64)
    key_idx = np.arange(n)
    for h in range(hq):
        kvh = h // g
        s = scale * (q[:, h, :] @ K[:, kvh, :].T)  # [nq][n]
        s = np.where(key_idx[None, :] < np.asarray(visible)[:, None], s, -np.inf)
        m = np.max(s, axis=1, keepdims=True)
        e = np.exp(s - m)
        w = e / np.sum(e, axis=1, keepdims=True)
        out[:, h, :] = w @ V[:, kvh, :]
    return out


def decode(q, k_pool, v_pool, block_tables, context_lens, scale,
           k_scale=None, v_scale=None, codec=None):
    """One decode step: each request's single new query against its whole cache.

    ``context_lens[s]`` counts the tokens in the cache *including* this step's
    token, whose K/V was written before attention (5688vip §3.2 orders the
    write before the read).  Returns float64 ``[S][Hq][D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros_like(q)
    for s in range(q.shape[0]):
        n = int(context_lens[s])
        K = gather_sequence(k_pool, block_tables[s], n, k_scale, codec)
        V = gather_sequence(v_pool, block_tables[s], n, v_scale, codec)
        out[s] = attention_rows(q[s][None], K, V, scale, [n])[0]
    return out


def prefill_chunk(q, k_pool, v_pool, query_start_loc, seq_lens, block_tables, scale,
                  k_scale=None, v_scale=None, codec=None):
    """Mixed batch of chunked prefills and decodes (uml.org.cn "Continuous Batching").

    Request ``s`` owns query rows ``query_start_loc[s] .. query_start_loc[s+1]-1``
    (``q_len`` rows; ``q_len == 1`` is a decode).  ``seq_lens[s]`` is its KV
    length including those rows, already written.  Query ``i`` of the chunk sits
    at absolute position ``seq_lens[s] - q_len + i`` and sees keys ``0 .. that
    position`` inclusive (autoregressive order, 5688vip §3.1).
    """
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros_like(q)
    for s in range(len(seq_lens)):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        q_len = b - a
        n = int(seq_lens[s])
        K = gather_sequence(k_pool, block_tables[s], n, k_scale, codec)
        V = gather_sequence(v_pool, block_tables[s], n, v_scale, codec)
        visible = [n - q_len + i + 1 for i in range(q_len)]
        out[a:b] = attention_rows(q[a:b], K, V, scale, visible)
    return out


def cache_write(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Scatter new tokens' K/V into the pools by slot; returns new pools.

    Token ``t`` goes to block ``slot // bs``, offset ``slot % bs`` (``bs`` the
    pools' third axis, 16 or 32); a negative
    slot means "no token" and is skipped.  Values are stored as given (the pool's
    own element type), so the result is an exact bit copy.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for t, slot in enumerate(np.asarray(slot_mapping)):
        if slot < 0:
            continue
        b, o = int(slot) // k_pool.shape[2], int(slot) % k_pool.shape[2]
        k_out[b, :, o, :] = k_new[t]
        v_out[b, :, o, :] = v_new[t]
    return k_out, v_out


def quantised_cache_write(codes, scales, x_new, slot_mapping, kind):
    """Write new tokens' K (or V) into a 1-byte pool, keeping one scale per
    (block, kv head) ("从KV Cache到vLLM" §2.2-2.3 store the cache as INT8 or FP8,
    one byte per element).  Returns new (codes, scales).

    The pages fix no scale policy for a block that fills up over several steps;
    the reading here (all arithmetic in float32, rounding to nearest even):

    * the rows one call writes into a block are the block's next rows in order;
      rows below the first of them already hold data (none when it is row 0);
    * the tile's scale never shrinks: s_new = max(s_old, amax_new / qmax), with
      s_old = 0 for a tile with no earlier rows, amax_new the largest magnitude
      among the new rows (every dim) and qmax 448 (FP8 E4M3FN) or 127 (INT8);
    * when the scale grows, each earlier code c is encoded again as
      encode(value(c) * (s_old / s_new));
    * a new value x is stored as encode(x / s_new), or code 0 while s_new is 0;
    * encode clamps to [-qmax, qmax] and rounds to nearest even (E4M3FN by the
      code grid, INT8 by rint).

    codes  [NB][H][bs][D] uint8 (fp8) or int8 (bs = 16 or 32 tokens per block);
           scales float32 [NB][H]
    x_new  [T][H][D] float values (float32 or narrower; read as float32)
    """
    codes = np.array(codes, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    x_new = np.asarray(x_new, dtype=np.float32)
    qmax = np.float32(448.0 if kind == "fp8" else 127.0)
    encode = e4m3fn_encode if kind == "fp8" else int8_encode
    values = e4m3fn_decode if kind == "fp8" else int8_decode
    slots = np.asarray(slot_mapping)
    # group the call's tokens by block, in token order
    runs = {}
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        runs.setdefault(int(slot) // codes.shape[2], []).append((int(slot) % codes.shape[2], t))
    for b, rows in runs.items():
        offs = [o for o, _ in rows]
        off0 = min(offs)
        for h in range(codes.shape[1]):
            s_old = scales[b, h] if off0 > 0 else np.float32(0.0)
            xs = np.stack([x_new[t, h] for _, t in rows])
            amax = np.float32(np.max(np.abs(xs)))
            s_new = np.maximum(s_old, np.float32(amax / qmax))
            if s_new > s_old and off0 > 0:
                ratio = np.float32(s_old / s_new)
                old = values(codes[b, h, :off0]).astype(np.float32)
                y = np.clip((old * ratio).astype(np.float32), -qmax, qmax)
                codes[b, h, :off0] = encode(y)
            for o, t in rows:
                if s_new > 0:
                    y = np.clip((x_new[t, h] / s_new).astype(np.float32), -qmax, qmax)
                    codes[b, h, o] = encode(y)
                else:
                    codes[b, h, o] = 0
            scales[b, h] = s_new
    return codes, scales


def block_copy(k_pool, v_pool, pairs, k_scale=None, v_scale=None):
    """Copy-on-write block duplication (uml.org.cn "Prefix Sharing").

    For each ``(src, dst)`` pair every kv head's K and V tile of block ``src``
    (and its scales, for 1-byte pools) is copied to block ``dst``.  All sources
    are read before any destination is written.  Returns new arrays.
    """
    pairs = np.asarray(pairs).reshape(-1, 2)
    srcs, dsts = pairs[:, 0], pairs[:, 1]
    outs = []
    for arr in (k_pool, v_pool, k_scale, v_scale):
        if arr is None:
            outs.append(None)
            continue
        new = np.array(arr, copy=True)
        src_data = np.array(arr[srcs], copy=True)
        new[dsts] = src_data
        outs.append(new)
    return tuple(outs)


def swap_blocks(dst, src, pairs):
    """Move blocks between two pools of one geometry (uml.org.cn "PagedAttention":
    under memory pressure a request's pages go out to CPU memory and come back
    when it runs again).

    ``dst`` and ``src`` are ``(k, v, k_scale, v_scale)`` tuples (scales None for
    pools without them).  For each ``(s, d)`` pair, every kv head's K and V tile
    of block ``s`` of ``src``, and its scales, becomes block ``d`` of ``dst``.
    Returns the new ``dst`` tuple; ``src`` is left as it is.
    """
    pairs = np.asarray(pairs).reshape(-1, 2)
    out = []
    for a_dst, a_src in zip(dst, src):
        if a_dst is None:
            out.append(None)
            continue
        new = np.array(a_dst, copy=True)
        for s, d in pairs:
            new[int(d)] = a_src[int(s)]
        out.append(new)
    return tuple(out)
