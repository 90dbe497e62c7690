"""Glue between the seeded workloads, the CPU oracle and the HIP library (tests only)."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
from paged_kv_cache_455_amd import workloads as W

CODEC = {"fp8": "e4m3fn", "i8": "int8"}
# max-abs tolerances on attention outputs, by KV storage type
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3, "fp8": 2e-2, "i8": 2e-2}


def np_of(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy without changing any value (bf16 widens to float32 exactly)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy()
    return t.numpy()


def oracle_pools(b: W.PagedBatch):
    kw = {}
    if b.kv_dtype in W.QUANTISED:
        kw = dict(k_scale=np_of(b.k_scale).astype(np.float64), v_scale=np_of(b.v_scale).astype(np.float64),
                  codec=CODEC[b.kv_dtype])
    return np_of(b.k_pool), np_of(b.v_pool), kw


def poison_tails(b: W.PagedBatch):
    """NaN (or a NaN code) in every slot past a sequence's context in its last block."""
    bt = b.block_tables.numpy()
    kf = b.k_pool.view(-1, b.head_dim)
    vf = b.v_pool.view(-1, b.head_dim)
    hkv = b.num_kv_heads
    bad = 0x7F if b.kv_dtype == "fp8" else (127 if b.kv_dtype == "i8" else float("nan"))
    bs = b.block_size
    for s, n in enumerate(b.seq_lens.tolist()):
        nb = -(-n // bs)
        for pos in range(n, nb * bs):
            slot = oracle.slot_for_position(bt[s], pos, bs)
            blk, off = divmod(slot, bs)
            for h in range(hkv):
                r = (blk * hkv + h) * bs + off
                kf[r] = bad
                vf[r] = bad
    return b


def oracle_slots(b: W.PagedBatch) -> np.ndarray:
    bt = b.block_tables.numpy()
    qsl = b.query_start_loc.numpy()
    out = []
    for s, n in enumerate(b.seq_lens.tolist()):
        q_len = int(qsl[s + 1] - qsl[s])
        for i in range(q_len):
            out.append(oracle.slot_for_position(bt[s], n - q_len + i, b.block_size))
    return np.array(out, dtype=np.int64)


def oracle_decode_rows(b: W.PagedBatch, rows=None) -> np.ndarray:
    """oracle.decode on the listed sequences (all by default): float64 [len(rows)][Hq][D]."""
    kp, vp, kw = oracle_pools(b)
    rows = list(range(b.num_seqs)) if rows is None else list(rows)
    q = np_of(b.q).astype(np.float64)[rows]
    bt = b.block_tables.numpy()[rows]
    ctx = b.seq_lens.numpy()[rows]
    return oracle.decode(q, kp, vp, bt, ctx, b.scale, **kw)


def oracle_mixed(b: W.PagedBatch, seqs=None):
    """oracle.prefill_chunk restricted to some sequences: (row indices, float64 outputs)."""
    kp, vp, kw = oracle_pools(b)
    qsl = b.query_start_loc.numpy()
    seqs = list(range(b.num_seqs)) if seqs is None else list(seqs)
    rows = np.concatenate([np.arange(qsl[s], qsl[s + 1]) for s in seqs])
    sub_qsl = np.concatenate([[0], np.cumsum([qsl[s + 1] - qsl[s] for s in seqs])]).astype(np.int32)
    q = np_of(b.q).astype(np.float64)[rows]
    out = oracle.prefill_chunk(q, kp, vp, sub_qsl, b.seq_lens.numpy()[seqs],
                               b.block_tables.numpy()[seqs], b.scale, **kw)
    return rows, out


class Dev:
    """A batch's arrays on the GPU plus a KVPool over them."""

    def __init__(self, b: W.PagedBatch, device="cuda", shared_blocks=None):
        import paged_kv_cache_455_amd as pa
        to = lambda t: None if t is None else t.to(device).contiguous()
        self.b = b
        self.q = to(b.q)
        self.k = to(b.k_pool)
        self.v = to(b.v_pool)
        self.ks = to(b.k_scale)
        self.vs = to(b.v_scale)
        self.bt = to(b.block_tables)
        self.lens = to(b.seq_lens)
        self.qsl = to(b.query_start_loc)
        self.k_new = to(b.k_new)
        self.v_new = to(b.v_new)
        self.pairs = to(b.copy_pairs)
        if shared_blocks is None:
            shared_blocks = b.shares_blocks
        self.pool = pa.KVPool(self.k, self.v, self.ks, self.vs, shared_blocks=shared_blocks)


def max_err(gpu: torch.Tensor, ref: np.ndarray) -> float:
    g = np_of(gpu).astype(np.float64)
    assert np.isfinite(g).all(), "non-finite GPU output"
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0


def err_over_bar(gpu: torch.Tensor, ref: np.ndarray, kv: str) -> float:
    """Largest |gpu - ref| / bar, where each element's bar is the larger of the
    storage type's max-abs tolerance and one ulp of the output type at the
    oracle's value (+1e-6 for fp32 accumulation): on data with |out| ~ 1 a bf16
    output cannot hold the oracle's value to 2e-3.  <= 1 passes."""
    g = np_of(gpu).astype(np.float64)
    assert np.isfinite(g).all(), "non-finite GPU output"
    if ref.size == 0:
        return 0.0
    a = torch.from_numpy(np.abs(ref)).to(gpu.dtype)
    bits = torch.int16 if gpu.element_size() == 2 else torch.int32
    ulp = ((a.view(bits) + 1).view(gpu.dtype).double() - a.double()).numpy()
    bar = np.maximum(TOL[kv], ulp + 1e-6)
    return float(np.max(np.abs(g - ref) / bar))


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)
