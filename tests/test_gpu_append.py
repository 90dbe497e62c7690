"""pa_decode_append: a decode step with the new rows' cache write fused in.

"5688vip" chapter 3, section 3.2: each step computes the new token's K/V, writes it
at the end of the request's last block, then attends over every cached token, the
new one included.  The fused call must equal the three calls it stands for --
pa_slot_mapping, kv_cache_write, pa_decode -- bit for bit (output, both pools,
slots), and match the oracle run after the oracle's own cache write.  The pool
row the new token goes to holds NaN before the call, so a fused decode that read
the pool instead of the new row would show it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_455_amd as pa
from paged_kv_cache_455_amd import workloads as W

from .pa_testlib import TOL, err_over_bar, max_err, np_of, oracle_decode_rows, oracle_slots

pytestmark = pytest.mark.gpu


def say(*a):
    print("[append]", *a, flush=True)


def _poison_new_rows(b):
    """NaN in the pool rows the new tokens go to (before the write)."""
    bt = b.block_tables.numpy()
    kf = b.k_pool.view(-1, b.head_dim)
    vf = b.v_pool.view(-1, b.head_dim)
    for s, n in enumerate(b.seq_lens.tolist()):
        blk, off = divmod(oracle.slot_for_position(bt[s], n - 1, b.block_size), b.block_size)
        for h in range(b.num_kv_heads):
            r = (blk * b.num_kv_heads + h) * b.block_size + off
            kf[r] = float("nan")
            vf[r] = float("nan")


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _run_pair(b, rows_for_oracle=None, peaked=False):
    """Unfused (slot map, write, decode) on one pool copy and fused on another."""
    dev = lambda t: t.clone().cuda()
    kA, vA, kB, vB = dev(b.k_pool), dev(b.v_pool), dev(b.k_pool), dev(b.v_pool)
    poolA, poolB = pa.KVPool(kA, vA), pa.KVPool(kB, vB)
    q, kn, vn, bt, lens = dev(b.q), dev(b.k_new), dev(b.v_new), dev(b.block_tables), dev(b.seq_lens)
    S = b.num_seqs
    qsl = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    slotsA = pa.pa_slot_mapping(bt, qsl, lens, S, block_size=b.block_size)
    pa.kv_cache_write(poolA, kn, vn, slotsA)
    outA = pa.pa_decode(poolA, q, bt, lens, b.max_seq_len, b.scale)
    slotsB = torch.full((S,), -7, dtype=torch.int64, device="cuda")
    outB = pa.pa_decode_append(poolB, q, kn, vn, bt, lens, b.max_seq_len, b.scale,
                               slot_mapping=slotsB)
    torch.cuda.synchronize()
    assert torch.equal(slotsA, slotsB), "slots differ"
    assert torch.equal(_bits(kA), _bits(kB)), "K pools differ"
    assert torch.equal(_bits(vA), _bits(vB)), "V pools differ"
    assert torch.equal(_bits(outA), _bits(outB)), "outputs differ"
    # the oracle: its own slots and cache write, then decode on the sampled rows
    slots = oracle_slots(b)
    assert slotsB.cpu().numpy().tolist() == slots.tolist()
    kp, vp = oracle.cache_write(np_of(b.k_pool), np_of(b.v_pool), np_of(b.k_new), np_of(b.v_new),
                                slots)
    assert np.array_equal(np_of(kB).view(np.uint8), kp.view(np.uint8)), "K pool vs oracle"
    assert np.array_equal(np_of(vB).view(np.uint8), vp.view(np.uint8)), "V pool vs oracle"
    rows = list(range(S)) if rows_for_oracle is None else rows_for_oracle
    ref = oracle.decode(np_of(b.q).astype(np.float64)[rows], kp, vp, b.block_tables.numpy()[rows],
                        b.seq_lens.numpy()[rows], b.scale)
    if peaked:
        return err_over_bar(outB[rows], ref, b.kv_dtype)
    return max_err(outB[rows], ref)


CASES = [  # kv, Hq, Hkv, D, block size, contexts
    ("f32", 4, 2, 64, 16, [5, 16, 17, 40, 1]),
    ("f16", 32, 8, 128, 16, [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 511, 512, 513, 1000,
                             4096]),
    ("bf16", 64, 8, 128, 32, [1, 31, 32, 33, 64, 65, 700, 2048]),
    ("f16", 8, 8, 64, 16, [3, 16, 100, 257]),
    ("bf16", 16, 8, 128, 32, [2, 17, 48, 300, 1025]),
    ("f32", 16, 4, 128, 32, [1, 33, 64, 95]),
    ("f16", 64, 8, 128, 16, [1, 2, 15, 16, 17, 31, 33, 129, 1000, 2049]),  # MFMA tile, f16 P.V
    ("f16", 32, 8, 64, 16, [1, 2, 15, 16, 17, 31, 33, 129, 1000, 2049]),   # MFMA tile, D 64
    ("bf16", 16, 8, 64, 32, [1, 31, 32, 33, 64, 65, 700, 2048]),
]


@pytest.mark.parametrize("kv,hq,hkv,d,bs,ctx", CASES)
def test_fused_equals_unfused_and_oracle(kv, hq, hkv, d, bs, ctx):
    say(kv, f"Hq {hq} Hkv {hkv} D {d} block {bs} ctx {ctx}")
    b = W.decode_batch(77, ctx, hq, hkv, d, kv, kv, div=math.sqrt(d), poison=True,
                       name=f"append-{kv}", block_size=bs)
    _poison_new_rows(b)
    err = _run_pair(b)
    say("max err", err)
    assert err <= TOL[kv]


@pytest.mark.parametrize("kv,hq,hkv,d,bs", [("f16", 32, 8, 128, 16), ("bf16", 16, 8, 64, 32),
                                           ("bf16", 8, 8, 128, 16), ("f16", 64, 8, 64, 32),
                                           ("f16", 64, 8, 128, 16), ("bf16", 64, 8, 128, 32)])
def test_fused_peaked_data(kv, hq, hkv, d, bs):
    """Unscaled N(0,1) data (peaked softmax): the fused step against the unfused
    calls bit for bit, and against the oracle at one ulp of the output type."""
    ctx = [1, 2, 17, 31, 32, 33, 129, 700, 2048, 3000]
    b = W.decode_batch(88, ctx, hq, hkv, d, kv, kv, poison=True, name=f"append-peaked-{kv}",
                       block_size=bs)
    say(b.name, f"Hq {hq} Hkv {hkv} D {d} block {bs}")
    _poison_new_rows(b)
    r = _run_pair(b, peaked=True)
    say("max err/bar", r)
    assert r <= 1.0


@pytest.mark.parametrize("bs", [16, 32])
def test_fused_llama_decode_layer(bs):
    """The 64-sequence Llama-3-8B-shaped decode layer, every row against the oracle."""
    b = W.llama3_8b_decode(block_size=bs)
    say(b.name, "block", bs)
    _poison_new_rows(b)
    err = _run_pair(b)
    say("max err", err)
    assert err <= TOL["f16"]


def _check_fused_quantised(b, kv, oracle_rows=True, large=False):
    """pa_decode_append on a 1-byte pool against pa_slot_mapping +
    kv_cache_write_quant + pa_decode on a copy: codes, scales, slots and output bit
    for bit; then (oracle_rows) the oracle's quantised write and decode, at the
    max-abs bar, or (large: outputs far above 1) at max(bar, one ulp of the output)."""
    bs = b.block_size
    dev = lambda t: t.clone().cuda()
    kA, vA, ksA, vsA = dev(b.k_pool), dev(b.v_pool), dev(b.k_scale), dev(b.v_scale)
    kB, vB, ksB, vsB = dev(b.k_pool), dev(b.v_pool), dev(b.k_scale), dev(b.v_scale)
    poolA, poolB = pa.KVPool(kA, vA, ksA, vsA), pa.KVPool(kB, vB, ksB, vsB)
    q, kn, vn, bt, lens = dev(b.q), dev(b.k_new), dev(b.v_new), dev(b.block_tables), dev(b.seq_lens)
    S = b.num_seqs
    qsl = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    slotsA = pa.pa_slot_mapping(bt, qsl, lens, S, block_size=bs)
    pa.kv_cache_write_quant(poolA, kn, vn, slotsA)
    outA = pa.pa_decode(poolA, q, bt, lens, b.max_seq_len, b.scale)
    slotsB = torch.full((S,), -7, dtype=torch.int64, device="cuda")
    outB = pa.pa_decode_append(poolB, q, kn, vn, bt, lens, b.max_seq_len, b.scale,
                               slot_mapping=slotsB)
    torch.cuda.synchronize()
    assert torch.equal(slotsA, slotsB)
    for x, y in ((kA, kB), (vA, vB), (ksA, ksB), (vsA, vsB)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    assert torch.equal(_bits(outA), _bits(outB))
    if not oracle_rows:
        return
    # the oracle: its quantised write, then decode over the codes it stored
    slots = oracle_slots(b)
    kc, ksc = oracle.quantised_cache_write(b.k_pool.numpy(), b.k_scale.numpy(),
                                           b.k_new.float().numpy(), slots, kv)
    vc, vsc = oracle.quantised_cache_write(b.v_pool.numpy(), b.v_scale.numpy(),
                                           b.v_new.float().numpy(), slots, kv)
    assert np.array_equal(kB.cpu().numpy(), kc) and np.array_equal(vB.cpu().numpy(), vc)
    assert np.array_equal(ksB.cpu().numpy().view(np.uint32), ksc.view(np.uint32))
    assert np.array_equal(vsB.cpu().numpy().view(np.uint32), vsc.view(np.uint32))
    b2 = W.PagedBatch(**{**b.__dict__, "k_pool": torch.from_numpy(kc), "v_pool": torch.from_numpy(vc),
                         "k_scale": torch.from_numpy(ksc), "v_scale": torch.from_numpy(vsc)})
    ref = oracle_decode_rows(b2)
    err = max_err(outB, ref)
    say("max err", err)
    if large:
        assert err_over_bar(outB, ref, kv) <= 1.0
    else:
        assert err <= TOL[kv]


@pytest.mark.parametrize("kv,qd,hq,bs,d", [("fp8", "bf16", 64, 16, 128), ("i8", "f16", 32, 32, 128),
                                           ("fp8", "f16", 16, 32, 128), ("i8", "bf16", 64, 16, 128),
                                           ("fp8", "bf16", 32, 16, 64), ("i8", "f16", 8, 32, 64)])
def test_fused_quantised_equals_separate_and_oracle(kv, qd, hq, bs, d):
    """1-byte pools: the new rows (in q's dtype) are quantised on write with the slots
    taken from the tables; codes, scales, slots and output must equal
    pa_slot_mapping + kv_cache_write_quant + pa_decode bit for bit."""
    ctx = [1, 2, 15, 16, 17, 33, 100, 511, 1000, 1500]
    b = W.decode_batch(91, ctx, hq, 8, d, kv, qd, name=f"append-{kv}", block_size=bs)
    say(b.name, qd, "block", bs, "head_dim", d)
    _check_fused_quantised(b, kv)


@pytest.mark.parametrize("kv,qd", [("fp8", "bf16"), ("i8", "f16"), ("fp8", "f16"), ("i8", "bf16")])
def test_fused_quantised_scale_growth(kv, qd):
    """The fused step's quantised write where it matters most (GQA group 8, head_dim
    128): new rows 8x the cached data's size for half the sequences (the block's
    scale grows and its earlier rows are re-encoded), 1/8 of it for the others (the
    scale stays), and an all-zero new row that starts its block (scale 0, codes 0);
    new rows at every position of a tile, 0 to 15.  The
    8x rows carry the outputs to |out| ~ 10, where one bf16 ulp is 0.06: the
    oracle bar there is one ulp of the output."""
    ctx = [1, 2, 3, 15, 16, 17, 18, 24, 31, 32, 33, 100, 255, 256, 257, 1000, 1500, 1503]
    b = W.decode_batch(97, ctx, 64, 8, 128, kv, qd, name=f"grow-{kv}-{qd}")
    f = torch.tensor([8.0 if s % 2 == 0 else 0.125 for s in range(len(ctx))]).view(-1, 1, 1)
    kn, vn = b.k_new.float() * f, b.v_new.float() * f
    kn[0] = 0.0
    vn[0] = 0.0
    b = W.PagedBatch(**{**b.__dict__, "k_new": kn.to(b.k_new.dtype), "v_new": vn.to(b.v_new.dtype)})
    say(b.name)
    _check_fused_quantised(b, kv, large=True)


@pytest.mark.parametrize("kv", ["fp8", "i8"])
def test_fused_quantised_long_context_full_size(kv):
    """The long-context batch (16 x 32768, 64 q / 8 kv heads, bf16 q) through the
    fused step: bit for bit against the separate write and decode (each of which
    the other tests pin to the oracle)."""
    b = W.long_quantised(kv)
    say(b.name)
    _check_fused_quantised(b, kv, oracle_rows=False)


@pytest.mark.parametrize("bs", [16, 32])
def test_fused_prefix_sharing_cow_step(bs):
    """Prefix sharing + copy-on-write ("uml.org.cn" Prefix Sharing): the copies run
    first, then the fused step writes each row into its (possibly fresh) last block
    and attends, on a pool declared to share blocks (cached loads).  Pools and slots
    must equal the separate calls bit for bit, the output too."""
    b = W.prefix_cow(n_req=24, n_forks=6, suffix_hi=400, block_size=bs)
    say(b.name, "block", bs)
    dev = lambda t: t.clone().cuda()
    kA, vA, kB, vB = dev(b.k_pool), dev(b.v_pool), dev(b.k_pool), dev(b.v_pool)
    poolA = pa.KVPool(kA, vA, shared_blocks=True)
    poolB = pa.KVPool(kB, vB, shared_blocks=True)
    q, kn, vn, bt, lens = dev(b.q), dev(b.k_new), dev(b.v_new), dev(b.block_tables), dev(b.seq_lens)
    pairs = dev(b.copy_pairs)
    S = b.num_seqs
    qsl = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    pa.kv_block_copy(poolA, pairs)
    slotsA = pa.pa_slot_mapping(bt, qsl, lens, S, block_size=bs)
    pa.kv_cache_write(poolA, kn, vn, slotsA)
    outA = pa.pa_decode(poolA, q, bt, lens, b.max_seq_len, b.scale)
    pa.kv_block_copy(poolB, pairs)
    slotsB = torch.empty_like(slotsA)
    outB = pa.pa_decode_append(poolB, q, kn, vn, bt, lens, b.max_seq_len, b.scale,
                               slot_mapping=slotsB)
    torch.cuda.synchronize()
    assert torch.equal(slotsA, slotsB)
    assert torch.equal(_bits(kA), _bits(kB)) and torch.equal(_bits(vA), _bits(vB))
    assert torch.equal(_bits(outA), _bits(outB))
    # and the oracle on a few rows, parents and forks
    kp, vp, _, _ = oracle.block_copy(np_of(b.k_pool), np_of(b.v_pool), b.copy_pairs.numpy())
    kp, vp = oracle.cache_write(kp, vp, np_of(b.k_new), np_of(b.v_new), oracle_slots(b))
    assert np.array_equal(np_of(kB), kp) and np.array_equal(np_of(vB), vp)
    rows = [0, 1, S // 2, S - 2, S - 1]
    ref = oracle.decode(np_of(b.q).astype(np.float64)[rows], kp, vp, b.block_tables.numpy()[rows],
                        b.seq_lens.numpy()[rows], b.scale)
    err = max_err(outB[rows], ref)
    say("max err", err)
    assert err <= TOL["bf16"]
