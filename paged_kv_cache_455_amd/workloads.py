"""Seeded synthetic inputs for the paged-attention path.

This module draws random numbers and deals out physical blocks; it holds none
of the attention arithmetic, no slot computation and no dequantisation.  It
is shared by the tests (which feed the same arrays to the CPU oracle and to the
HIP library), by ``bench.py`` and by the smoke check.

Workloads (no public dataset is involved; these synthetic batches stand in for
the serving scenarios the pages describe):

1. tiny fp32 decode: contexts {5,16,17,40}, 4 query / 2 KV heads, head_dim 64,
   pool of 32 blocks, N(0,1) data, scale 1/8;
2. Llama-3-8B-shaped decode layer: 64 sequences, contexts uniform in
   [128, 4096], 32 query / 8 KV heads, head_dim 128, fp16, N(0,1)/sqrt(128);
3. prefix sharing + copy-on-write: 128 requests over one 1024-token prefix
   (64 shared blocks) and a private suffix uniform in [16, 2048], bf16; 16 of
   them are forked (parallel sampling) and the child's copy of the shared,
   partially filled last block is staged as a (src, dst) copy pair;
4. mixed continuous-batching step: 8 prefill chunks of 512 tokens over
   0..2048 tokens of prior context plus 256 decodes with lognormal contexts
   (median 600, sigma 1, clipped to [16, 8192]), fp16;
5. long-context quantised KV: 16 x 32768 tokens, 64 query / 8 KV heads, KV
   stored as fp8 E4M3FN or int8 codes with one fp32 scale per (block, kv head),
   bf16 queries and outputs.

All tensors are CPU torch tensors; the pool layout is
``[num_blocks][num_kv_heads][16][head_dim]``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BLOCK = 16

TORCH_DTYPE = {
    "f32": torch.float32,
    "f16": torch.float16,
    "bf16": torch.bfloat16,
    "fp8": torch.uint8,   # E4M3FN bit patterns
    "i8": torch.int8,
}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "i8": 1}
QUANTISED = ("fp8", "i8")


@dataclass
class PagedBatch:
    name: str
    kind: str                      # "decode" (one query row per sequence) or "mixed"
    kv_dtype: str
    q_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    q: torch.Tensor                # [T][Hq][D]
    k_pool: torch.Tensor           # [NB][Hkv][block_size][D]
    v_pool: torch.Tensor
    block_tables: torch.Tensor     # int32 [S][MB], -1 past the last used block
    seq_lens: torch.Tensor         # int32 [S], KV length including this step's tokens
    query_start_loc: torch.Tensor  # int32 [S+1]
    k_scale: Optional[torch.Tensor] = None   # f32 [NB][Hkv]
    v_scale: Optional[torch.Tensor] = None
    k_new: Optional[torch.Tensor] = None     # [T][Hkv][D] this step's K/V, pool dtype
    v_new: Optional[torch.Tensor] = None
    copy_pairs: Optional[torch.Tensor] = None  # int32 [P][2] (src, dst)
    extra: dict = field(default_factory=dict)
    block_size: int = BLOCK        # tokens per block, 16 or 32 (the pools' third axis)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    @property
    def shares_blocks(self) -> bool:
        """True when a physical block appears in more than one sequence's used table
        entries (prefix sharing): the pool is then declared with shared blocks."""
        used = []
        for s in range(self.num_seqs):
            nb = -(-int(self.seq_lens[s]) // self.block_size)
            used.append(self.block_tables[s, :nb])
        ids = torch.cat(used) if used else torch.empty(0, dtype=torch.int32)
        return int(torch.unique(ids).numel()) < int(ids.numel())

    @property
    def max_query_len(self) -> int:
        qsl = self.query_start_loc
        return int((qsl[1:] - qsl[:-1]).max())


# ----------------------------------------------------------------------------------
# building blocks: random draws, block dealing, dtype casts
# ----------------------------------------------------------------------------------
def _normal(rng, shape, div=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if div != 1.0:
        x /= np.float32(div)
    return x


def _cast(x: np.ndarray, dt: str) -> torch.Tensor:
    """float32 numpy -> CPU tensor of a float storage dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DTYPE[dt])


def _deal_tables(perm: np.ndarray, blocks_per_seq: List[int], start: int = 0):
    """Hand out physical ids ``perm[start:]`` in order, one row per sequence."""
    mb = max(1, max(blocks_per_seq))
    bt = np.full((len(blocks_per_seq), mb), -1, dtype=np.int32)
    i = start
    for s, nb in enumerate(blocks_per_seq):
        bt[s, :nb] = perm[i:i + nb]
        i += nb
    return bt, i


def _float_pool(rng, nb, hkv, d, div, dt, chunk=2048, bs=BLOCK):
    """[nb][hkv][bs][d] of N(0,1)/div, drawn in chunks to bound host memory."""
    out = torch.empty((nb, hkv, bs, d), dtype=TORCH_DTYPE[dt])
    for a in range(0, nb, chunk):
        b = min(nb, a + chunk)
        out[a:b] = _cast(_normal(rng, (b - a, hkv, bs, d), div), dt)
    return out


def _quantised_pool(rng, nb, hkv, d, div, kv, chunk=2048, bs=BLOCK):
    """Codes and per-(block, kv head) scales for N(0,1)/div data.

    Each (block, head) tile gets ``scale = amax(|tile|) / qmax`` (qmax 448 for
    E4M3FN, 127 for int8; an all-zero tile gets 1).  Codes come from torch's
    float8_e4m3fn cast (round to nearest even) or from rint+clip for int8.  The
    codes are the stored data the attention path is given; how they were made
    does not enter the comparison, which decodes the same stored codes.
    """
    qmax = 448.0 if kv == "fp8" else 127.0
    codes = torch.empty((nb, hkv, bs, d), dtype=TORCH_DTYPE[kv])
    scales = torch.empty((nb, hkv), dtype=torch.float32)
    for a in range(0, nb, chunk):
        b = min(nb, a + chunk)
        x = torch.from_numpy(_normal(rng, (b - a, hkv, bs, d), div))
        amax = x.abs().amax(dim=(2, 3))
        sc = torch.where(amax > 0, amax / qmax, torch.ones_like(amax))
        y = x / sc[:, :, None, None]
        if kv == "fp8":
            y = y.clamp(-qmax, qmax).to(torch.float8_e4m3fn).view(torch.uint8)
        else:
            y = torch.round(y).clamp(-127, 127).to(torch.int8)
        codes[a:b] = y
        scales[a:b] = sc
    return codes, scales


def _poison_unused(pool: torch.Tensor, used: np.ndarray, kv: str):
    unused = torch.from_numpy(~used)
    if not bool(unused.any()):
        return
    if kv == "fp8":
        pool[unused] = 0x7F          # the E4M3FN NaN pattern
    elif kv == "i8":
        pool[unused] = 127
    else:
        pool[unused] = float("nan")


def _used_mask(bt: np.ndarray, nb: int) -> np.ndarray:
    used = np.zeros(nb, dtype=bool)
    ids = bt[bt >= 0]
    used[ids] = True
    return used


# ----------------------------------------------------------------------------------
# generic decode batch (configs 1, 2, 5 and their small variants)
# ----------------------------------------------------------------------------------
def decode_batch(seed: int, ctx, hq: int, hkv: int, d: int, kv: str, qd: str, *,
                 div: float = 1.0, pool_blocks: Optional[int] = None, pool_extra: float = 0.10,
                 scale: Optional[float] = None, poison: bool = False, name: str = "decode",
                 with_new: bool = True, block_size: int = BLOCK) -> PagedBatch:
    """One query token per sequence against ``ctx[s]`` cached tokens.

    Physical blocks come from one seeded permutation of the pool, dealt in
    sequence order.  ``with_new`` also draws this step's K/V (``k_new``) for the
    cache-write that precedes the attention; the pool slot it goes to holds an
    older random value until then.
    """
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int64)
    bs = block_size
    nbs = [int(-(-int(n) // bs)) for n in ctx]
    need = sum(nbs)
    nb = pool_blocks if pool_blocks is not None else int(math.ceil((1.0 + pool_extra) * need))
    assert nb >= need
    perm = rng.permutation(nb).astype(np.int32)
    bt, _ = _deal_tables(perm, nbs)
    S = len(ctx)
    q = _cast(_normal(rng, (S, hq, d), div), qd)
    if kv in QUANTISED:
        # the draw order does not depend on kv, so an fp8 and an int8 batch with the
        # same seed quantise the same N(0,1) data
        k_pool, k_scale = _quantised_pool(rng, nb, hkv, d, div, kv, bs=bs)
        v_pool, v_scale = _quantised_pool(rng, nb, hkv, d, div, kv, bs=bs)
        if with_new:  # this step's K/V in the model's dtype, quantised on write
            k_new = _cast(_normal(rng, (S, hkv, d), div), qd)
            v_new = _cast(_normal(rng, (S, hkv, d), div), qd)
        else:
            k_new = v_new = None
    else:
        k_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
        v_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
        k_scale = v_scale = None
        if with_new:
            k_new = _cast(_normal(rng, (S, hkv, d), div), kv)
            v_new = _cast(_normal(rng, (S, hkv, d), div), kv)
        else:
            k_new = v_new = None
    if poison:
        used = _used_mask(bt, nb)
        _poison_unused(k_pool, used, kv)
        _poison_unused(v_pool, used, kv)
    return PagedBatch(
        name=name, kind="decode", kv_dtype=kv, q_dtype=qd, num_q_heads=hq, num_kv_heads=hkv,
        head_dim=d, scale=(1.0 / math.sqrt(d)) if scale is None else scale, q=q,
        k_pool=k_pool, v_pool=v_pool, block_tables=torch.from_numpy(bt),
        seq_lens=torch.from_numpy(ctx.astype(np.int32)),
        query_start_loc=torch.arange(S + 1, dtype=torch.int32),
        k_scale=k_scale, v_scale=v_scale, k_new=k_new, v_new=v_new, block_size=bs)


# ----------------------------------------------------------------------------------
# prefix sharing with forked requests
# ----------------------------------------------------------------------------------
def fork_batch(seed: int, n_req: int, prefix_tokens: int, suffix_lo: int, suffix_hi: int,
               n_forks: int, hq: int, hkv: int, d: int, kv: str, qd: str, *, div: float = 1.0,
               pool_extra: float = 0.10, poison: bool = False, name: str = "fork",
               block_size: int = BLOCK) -> PagedBatch:
    """Requests over one shared prefix; some are forked just before a decode step.

    Request ``r`` holds ``L_r = prefix + suffix_r`` cached tokens; the prefix's
    blocks are one physical set shared by every request.  ``n_forks`` requests
    with a partially filled last block are forked (parallel sampling): the child
    shares all of the parent's blocks, so before either writes its new token
    into that shared partial block the child gets a fresh block, to be filled by
    a block copy ``(parent_last, fresh)``, and its table row points there.  The
    batch has ``n_req + n_forks`` decode rows (parents first, then children in
    fork order), each with context ``L + 1``.
    """
    bs = block_size
    assert prefix_tokens % bs == 0
    rng = np.random.default_rng(seed)
    suffix = rng.integers(suffix_lo, suffix_hi, size=n_req, endpoint=True)
    L = prefix_tokens + suffix
    eligible = np.nonzero(L % bs != 0)[0]
    forks = np.sort(rng.choice(eligible, size=n_forks, replace=False)) if n_forks else np.zeros(0, np.int64)
    pre_blocks = prefix_tokens // bs
    # blocks each request needs after its new token: ceil((L+1)/bs)
    own = [int(-(-(int(l) + 1) // bs)) - pre_blocks for l in L]
    need = pre_blocks + sum(own) + n_forks
    nb = int(math.ceil((1.0 + pool_extra) * need))
    perm = rng.permutation(nb).astype(np.int32)
    shared = perm[:pre_blocks]
    rows = []
    i = pre_blocks
    for r in range(n_req):
        rows.append(list(shared) + list(perm[i:i + own[r]]))
        i += own[r]
    pairs = []
    for f in forks:
        child = list(rows[f])
        fresh = int(perm[i])
        i += 1
        pairs.append((child[-1], fresh))
        child[-1] = fresh
        rows.append(child)
    mb = max(len(r) for r in rows)
    bt = np.array([r + [-1] * (mb - len(r)) for r in rows], dtype=np.int32)
    ctx = np.concatenate([L + 1, L[forks] + 1]).astype(np.int32)
    S = len(ctx)
    q = _cast(_normal(rng, (S, hq, d), div), qd)
    k_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
    v_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
    k_new = _cast(_normal(rng, (S, hkv, d), div), kv)
    v_new = _cast(_normal(rng, (S, hkv, d), div), kv)
    if poison:
        used = _used_mask(bt, nb)
        _poison_unused(k_pool, used, kv)
        _poison_unused(v_pool, used, kv)
    return PagedBatch(
        name=name, kind="decode", kv_dtype=kv, q_dtype=qd, num_q_heads=hq, num_kv_heads=hkv,
        head_dim=d, scale=1.0 / math.sqrt(d), q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.from_numpy(bt), seq_lens=torch.from_numpy(ctx),
        query_start_loc=torch.arange(S + 1, dtype=torch.int32), k_new=k_new, v_new=v_new,
        copy_pairs=torch.tensor(pairs, dtype=torch.int32).reshape(-1, 2),
        extra={"forks": forks, "n_req": n_req, "shared_blocks": shared.copy()}, block_size=bs)


# ----------------------------------------------------------------------------------
# mixed prefill chunks + decodes
# ----------------------------------------------------------------------------------
def mixed_batch(seed: int, n_chunks: int, chunk_len: int, prior_lo: int, prior_hi: int,
                n_dec: int, dec_median: float, dec_sigma: float, dec_lo: int, dec_hi: int,
                hq: int, hkv: int, d: int, kv: str, qd: str, *, div: float = 1.0,
                pool_extra: float = 0.10, poison: bool = False, priors=None, dec_ctx=None,
                name: str = "mixed", block_size: int = BLOCK) -> PagedBatch:
    """Chunked prefills and decodes in one batch.

    Chunk ``i`` adds ``chunk_len`` tokens on top of ``prior_i`` cached tokens
    (``seq_len = prior + chunk_len``); each decode adds one token to a context
    drawn from a lognormal (``seq_len`` = that context).  Rows are packed
    chunks first, then decodes.  ``k_new``/``v_new`` hold every new token's K/V.
    """
    rng = np.random.default_rng(seed)
    if priors is None:
        priors = rng.integers(prior_lo, prior_hi, size=n_chunks, endpoint=True)
    priors = np.asarray(priors, dtype=np.int64)
    if dec_ctx is None:
        dec_ctx = np.clip(np.rint(np.exp(rng.normal(math.log(dec_median), dec_sigma, size=n_dec))),
                          dec_lo, dec_hi)
    dec_ctx = np.asarray(dec_ctx, dtype=np.int64)
    seq_lens = np.concatenate([priors + chunk_len, dec_ctx]).astype(np.int32)
    q_lens = np.concatenate([np.full(len(priors), chunk_len), np.ones(len(dec_ctx))]).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    bs = block_size
    nbs = [int(-(-int(n) // bs)) for n in seq_lens]
    need = sum(nbs)
    nb = int(math.ceil((1.0 + pool_extra) * need))
    perm = rng.permutation(nb).astype(np.int32)
    bt, _ = _deal_tables(perm, nbs)
    T = int(qsl[-1])
    q = _cast(_normal(rng, (T, hq, d), div), qd)
    if kv in QUANTISED:  # codes + per-(block, kv head) scales; new rows in q's dtype
        k_pool, k_scale = _quantised_pool(rng, nb, hkv, d, div, kv, bs=bs)
        v_pool, v_scale = _quantised_pool(rng, nb, hkv, d, div, kv, bs=bs)
        k_new = _cast(_normal(rng, (T, hkv, d), div), qd)
        v_new = _cast(_normal(rng, (T, hkv, d), div), qd)
    else:
        k_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
        v_pool = _float_pool(rng, nb, hkv, d, div, kv, bs=bs)
        k_scale = v_scale = None
        k_new = _cast(_normal(rng, (T, hkv, d), div), kv)
        v_new = _cast(_normal(rng, (T, hkv, d), div), kv)
    if poison:
        used = _used_mask(bt, nb)
        _poison_unused(k_pool, used, kv)
        _poison_unused(v_pool, used, kv)
    return PagedBatch(
        name=name, kind="mixed", kv_dtype=kv, q_dtype=qd, num_q_heads=hq, num_kv_heads=hkv,
        head_dim=d, scale=1.0 / math.sqrt(d), q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=torch.from_numpy(bt), seq_lens=torch.from_numpy(seq_lens),
        query_start_loc=torch.from_numpy(qsl), k_scale=k_scale, v_scale=v_scale,
        k_new=k_new, v_new=v_new,
        extra={"n_chunks": len(priors), "chunk_len": chunk_len}, block_size=bs)


# ----------------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------------
def tiny_fp32(poison: bool = True, block_size: int = BLOCK) -> PagedBatch:
    """Contexts {5,16,17,40}, Hq 4 / Hkv 2, D 64, fp32, pool 32 blocks."""
    return decode_batch(1, [5, 16, 17, 40], 4, 2, 64, "f32", "f32", pool_blocks=32,
                        scale=1.0 / 8.0, poison=poison, name="tiny-fp32", block_size=block_size)


def llama3_8b_decode(batch: int = 64, ctx_lo: int = 128, ctx_hi: int = 4096, seed: int = 2,
                     poison: bool = False, block_size: int = BLOCK) -> PagedBatch:
    """Llama-3-8B-shaped decode layer: Hq 32 / Hkv 8, D 128, fp16, N(0,1)/sqrt(128)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi, size=batch, endpoint=True)
    return decode_batch(seed + 1000, ctx, 32, 8, 128, "f16", "f16", div=math.sqrt(128.0),
                        poison=poison, name=f"llama3-8b-decode-b{batch}", block_size=block_size)


def prefix_cow(n_req: int = 128, suffix_hi: int = 2048, n_forks: int = 16, seed: int = 3,
               poison: bool = False, block_size: int = BLOCK) -> PagedBatch:
    """128 requests over a 1024-token shared prefix, 16 forks, bf16, Llama-3-8B heads."""
    return fork_batch(seed, n_req, 1024, 16, suffix_hi, n_forks, 32, 8, 128, "bf16", "bf16",
                      div=math.sqrt(128.0), poison=poison, name=f"prefix-cow-r{n_req}",
                      block_size=block_size)


def mixed_step(n_chunks: int = 8, chunk_len: int = 512, n_dec: int = 256, seed: int = 4,
               poison: bool = False, priors=None, block_size: int = BLOCK) -> PagedBatch:
    """8 chunks x 512 over 0..2048 prior tokens + 256 lognormal decodes, fp16."""
    return mixed_batch(seed, n_chunks, chunk_len, 0, 2048, n_dec, 600.0, 1.0, 16, 8192,
                       32, 8, 128, "f16", "f16", div=math.sqrt(128.0), poison=poison,
                       priors=priors, name=f"mixed-c{n_chunks}x{chunk_len}-d{n_dec}",
                       block_size=block_size)


def long_quantised(kv: str = "fp8", batch: int = 16, ctx: int = 32768, seed: int = 5,
                   poison: bool = False, block_size: int = BLOCK) -> PagedBatch:
    """16 x 32768 tokens, Hq 64 / Hkv 8, D 128, fp8 or int8 KV, bf16 q/out.

    The int8 batch quantises the same N(0,1) draws as the fp8 batch.
    """
    return decode_batch(seed, [ctx] * batch, 64, 8, 128, kv, "bf16", poison=poison,
                        name=f"long-{kv}-b{batch}x{ctx}", block_size=block_size)


WORKLOADS = {
    1: tiny_fp32,
    2: llama3_8b_decode,
    3: prefix_cow,
    4: mixed_step,
    5: long_quantised,
}
