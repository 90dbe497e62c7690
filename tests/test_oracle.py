"""Pins for the CPU oracle: closed forms, library routines, invariants, brute force.

Each test ties the oracle to something other than itself: the pages' printed
numbers, the OCP FP8 definition checked against torch's float8 type, torch's
scaled_dot_product_attention, or a cache-free recomputation on tiny inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.paged_attention import BLOCK_SIZE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GIB = 1 << 30


# --------------------------------------------------------------------------------------
# KV bytes closed form: "从KV Cache到vLLM" §2.1 / §2.2 printed numbers
# --------------------------------------------------------------------------------------
def test_kv_bytes_matches_printed_numbers():
    with open(os.path.join(GOLDEN, "kv_bytes.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        got = oracle.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["seq_len"],
                                    c["batch"], c["bytes"])
        if "expected_bytes" in c:
            assert got == c["expected_bytes"], c["what"]
        else:
            assert got == c["expected_gib"] * GIB, c["what"]
    for r in fx["ratios"]:
        a = oracle.kv_cache_bytes(32, 8, 128, r["seq_from"], 1, 2)
        b = oracle.kv_cache_bytes(32, 8, 128, r["seq_to"], 1, 2)
        assert b == r["expected_ratio"] * a


# --------------------------------------------------------------------------------------
# FP8 / INT8 codes
# --------------------------------------------------------------------------------------
def test_e4m3fn_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3fn_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF only


def test_e4m3fn_decode_spec_values():
    d = oracle.e4m3fn_decode
    assert d(np.uint8(0x38)) == 1.0
    assert d(np.uint8(0x7E)) == 448.0
    assert d(np.uint8(0xFE)) == -448.0
    assert d(np.uint8(0x01)) == 2.0 ** -9
    assert d(np.uint8(0x08)) == 2.0 ** -6
    assert d(np.uint8(0x07)) == 7 * 2.0 ** -9
    assert np.isnan(d(np.uint8(0x7F)))


def test_e4m3fn_encode_roundtrip_ties_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3fn_decode(codes)
    back = oracle.e4m3fn_encode(vals)
    # +0 and -0 both decode to 0; the encoder keeps the sign bit
    assert np.array_equal(back, codes)
    enc = oracle.e4m3fn_encode
    assert enc(1.0625) == 0x38  # tie between 1.0 (0x38) and 1.125 (0x39): even
    assert enc(1.1875) == 0x3A  # tie between 1.125 (0x39) and 1.25 (0x3A): even
    assert enc(2.0 ** -10) == 0x00  # tie between 0 and the smallest subnormal
    assert enc(3 * 2.0 ** -10) == 0x02
    assert enc(1000.0) == 0x7E and enc(-1000.0) == 0xFE and enc(464.0) == 0x7E
    assert enc(np.nan) == 0x7F


def test_e4m3fn_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 150)])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(x.astype(np.float64)), ref)


def test_int8_codes():
    assert list(oracle.int8_encode([2.5, 3.5, -2.5, 0.49, 200, -200])) == [2, 4, -2, 0, 127, -127]
    assert oracle.int8_decode(np.array([-127, 0, 5], dtype=np.int8)).tolist() == [-127.0, 0.0, 5.0]


# --------------------------------------------------------------------------------------
# Attention: library routine, special cases, invariants
# --------------------------------------------------------------------------------------
def _random_paged(rng, ctx, hq, hkv, d, num_blocks, poison=True):
    """Pools with per-request blocks dealt from a random permutation."""
    k_pool = rng.standard_normal((num_blocks, hkv, BLOCK_SIZE, d))
    v_pool = rng.standard_normal((num_blocks, hkv, BLOCK_SIZE, d))
    perm = rng.permutation(num_blocks)
    nbs = [-(-n // BLOCK_SIZE) for n in ctx]
    mb = max(nbs)
    bt = -np.ones((len(ctx), mb), dtype=np.int32)
    used = np.zeros(num_blocks, bool)
    i = 0
    for s, nb in enumerate(nbs):
        bt[s, :nb] = perm[i:i + nb]
        used[perm[i:i + nb]] = True
        i += nb
    if poison:
        k_pool[~used] = np.nan
        v_pool[~used] = np.nan
        for s, n in enumerate(ctx):  # tail of each partial last block
            if n % BLOCK_SIZE:
                k_pool[bt[s, nbs[s] - 1], :, n % BLOCK_SIZE:, :] = np.nan
                v_pool[bt[s, nbs[s] - 1], :, n % BLOCK_SIZE:, :] = np.nan
    return k_pool, v_pool, bt


def _sdpa(q, K, V, scale, mask=None):
    """torch scaled_dot_product_attention in float64; GQA by repeat_interleave."""
    hq, hkv = q.shape[1], K.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1][Hq][nq][D]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    vt = torch.from_numpy(V).permute(1, 0, 2)[None].repeat_interleave(hq // hkv, dim=1)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (8, 1, 32), (6, 6, 16), (16, 2, 8)])
def test_decode_matches_sdpa(hq, hkv, d):
    rng = np.random.default_rng(hq * 100 + d)
    ctx = [1, 5, 16, 17, 40, 63]
    k_pool, v_pool, bt = _random_paged(rng, ctx, hq, hkv, d, 40)
    q = rng.standard_normal((len(ctx), hq, d))
    scale = 1.0 / np.sqrt(d)
    out = oracle.decode(q, k_pool, v_pool, bt, ctx, scale)
    for s, n in enumerate(ctx):
        K = oracle.gather_sequence(k_pool, bt[s], n)
        V = oracle.gather_sequence(v_pool, bt[s], n)
        ref = _sdpa(q[s][None], K, V, scale)[0]
        np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)
    assert np.isfinite(out).all()


def test_gather_identity_table_is_contiguous_history():
    rng = np.random.default_rng(3)
    hkv, d, n = 2, 8, 37
    history_k = rng.standard_normal((n, hkv, d))
    nb = -(-n // BLOCK_SIZE)
    pool = np.full((nb, hkv, BLOCK_SIZE, d), np.nan)
    for t in range(n):
        pool[t // BLOCK_SIZE, :, t % BLOCK_SIZE, :] = history_k[t]
    got = oracle.gather_sequence(pool, np.arange(nb), n)
    assert np.array_equal(got, history_k)


def test_prefill_matches_sdpa_causal():
    rng = np.random.default_rng(11)
    hq, hkv, d = 8, 2, 32
    seq_lens = [40, 9, 1, 33]
    q_lens = [12, 9, 1, 1]  # chunk over prior context, fresh prompt, two decodes
    k_pool, v_pool, bt = _random_paged(rng, seq_lens, hq, hkv, d, 20)
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    q = rng.standard_normal((qsl[-1], hq, d))
    scale = 0.3
    out = oracle.prefill_chunk(q, k_pool, v_pool, qsl, seq_lens, bt, scale)
    for s, (n, ql) in enumerate(zip(seq_lens, q_lens)):
        K = oracle.gather_sequence(k_pool, bt[s], n)
        V = oracle.gather_sequence(v_pool, bt[s], n)
        pos = n - ql + np.arange(ql)
        mask = np.arange(n)[None, :] <= pos[:, None]
        ref = _sdpa(q[qsl[s]:qsl[s + 1]], K, V, scale, mask[None])
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref, rtol=0, atol=1e-12)


def test_special_cases_closed_form():
    rng = np.random.default_rng(5)
    hq, hkv, d = 4, 2, 16
    # n = 1: the only weight is 1, output is V_0 exactly
    k_pool, v_pool, bt = _random_paged(rng, [1], hq, hkv, d, 4)
    q = rng.standard_normal((1, hq, d))
    out = oracle.decode(q, k_pool, v_pool, bt, [1], 0.7)
    for h in range(hq):
        assert np.array_equal(out[0, h], v_pool[bt[0, 0], h // 2, 0])
    # all keys equal -> uniform weights -> mean of V
    n = 29
    k_pool, v_pool, bt = _random_paged(rng, [n], hq, hkv, d, 4)
    for j in range(2):
        k_pool[bt[0, j]] = k_pool[bt[0, 0], :, :1, :]
    out = oracle.decode(q, k_pool, v_pool, bt, [n], 0.7)
    V = oracle.gather_sequence(v_pool, bt[0], n)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], V[:, h // 2].mean(0), rtol=0, atol=1e-13)
    # scale = 0 -> mean of V regardless of keys
    k_pool, v_pool, bt = _random_paged(rng, [n], hq, hkv, d, 4)
    out = oracle.decode(q, k_pool, v_pool, bt, [n], 0.0)
    V = oracle.gather_sequence(v_pool, bt[0], n)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], V[:, h // 2].mean(0), rtol=0, atol=1e-13)


def test_quantized_single_token_is_decoded_code_times_scale():
    rng = np.random.default_rng(8)
    hq, hkv, d = 2, 1, 16
    k_codes = rng.integers(0, 256, (2, hkv, 16, d)).astype(np.uint8) & 0x77  # finite codes
    v_codes = rng.integers(0, 256, (2, hkv, 16, d)).astype(np.uint8) & 0x77
    ks = np.array([[0.5], [2.0]])
    vs = np.array([[0.25], [3.0]])
    bt = np.array([[1]], dtype=np.int32)
    q = rng.standard_normal((1, hq, d))
    out = oracle.decode(q, k_codes, v_codes, bt, [1], 0.1, ks, vs, codec="e4m3fn")
    expect = oracle.e4m3fn_decode(v_codes[1, 0, 0]) * 3.0
    for h in range(hq):
        assert np.array_equal(out[0, h], expect)
    i8 = rng.integers(-127, 128, (2, hkv, 16, d)).astype(np.int8)
    out = oracle.decode(q, i8, i8, bt, [1], 0.1, ks, vs, codec="int8")
    assert np.array_equal(out[0, 0], i8[1, 0, 0].astype(np.float64) * 3.0)


def test_physical_block_permutation_invariance_bitwise():
    rng = np.random.default_rng(21)
    hq, hkv, d = 8, 2, 32
    ctx = [3, 16, 31, 50, 77]
    nbk = 30
    k_pool, v_pool, bt = _random_paged(rng, ctx, hq, hkv, d, nbk)
    q = rng.standard_normal((len(ctx), hq, d))
    out = oracle.decode(q, k_pool, v_pool, bt, ctx, 0.2)
    relabel = rng.permutation(nbk)  # physical id b moves to relabel[b]
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[relabel] = k_pool
    v2[relabel] = v_pool
    bt2 = np.where(bt >= 0, relabel[np.maximum(bt, 0)], -1)
    out2 = oracle.decode(q, k2, v2, bt2, ctx, 0.2)
    assert np.array_equal(out, out2)


def test_prefix_sharing_equals_private_copies_bitwise():
    rng = np.random.default_rng(4)
    hq, hkv, d = 4, 2, 16
    prefix_blocks, n_req = 3, 4
    suffix = [5, 16, 1, 20]
    nb_total = prefix_blocks + sum(-(-s // 16) for s in suffix)
    k_shared = rng.standard_normal((nb_total, hkv, 16, d))
    v_shared = rng.standard_normal((nb_total, hkv, 16, d))
    bts, ctx, nxt = [], [], prefix_blocks
    for s in suffix:
        nb = -(-s // 16)
        bts.append(list(range(prefix_blocks)) + list(range(nxt, nxt + nb)))
        nxt += nb
        ctx.append(prefix_blocks * 16 + s)
    mb = max(len(r) for r in bts)
    bt = np.array([r + [-1] * (mb - len(r)) for r in bts], dtype=np.int32)
    q = rng.standard_normal((n_req, hq, d))
    out_shared = oracle.decode(q, k_shared, v_shared, bt, ctx, 0.25)
    # private: every request gets its own copy of the prefix blocks
    k_priv = [k_shared]
    v_priv = [v_shared]
    bt_priv = bt.copy()
    base = nb_total
    for r in range(n_req):
        k_priv.append(k_shared[:prefix_blocks])
        v_priv.append(v_shared[:prefix_blocks])
        bt_priv[r, :prefix_blocks] = np.arange(base, base + prefix_blocks)
        base += prefix_blocks
    out_priv = oracle.decode(q, np.concatenate(k_priv), np.concatenate(v_priv), bt_priv, ctx, 0.25)
    assert np.array_equal(out_shared, out_priv)


def test_block_copy_reads_all_sources_first():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((6, 2, 16, 4))
    v = rng.standard_normal((6, 2, 16, 4))
    ks = rng.standard_normal((6, 2))
    pairs = np.array([[1, 4], [2, 5]])
    k2, v2, ks2, vs2 = oracle.block_copy(k, v, pairs, ks, None)
    assert vs2 is None
    assert np.array_equal(k2[4], k[1]) and np.array_equal(k2[5], k[2])
    assert np.array_equal(v2[4], v[1]) and np.array_equal(ks2[5], ks[2])
    untouched = [0, 1, 2, 3]
    assert np.array_equal(k2[untouched], k[untouched])


def test_copy_on_write_leaves_shared_page_untouched():
    """Fork a request whose last block is partial; CoW then diverging writes."""
    rng = np.random.default_rng(9)
    hkv, d, n = 2, 8, 21  # 2 blocks, the second holds 5 tokens
    k = rng.standard_normal((8, hkv, 16, d))
    v = rng.standard_normal((8, hkv, 16, d))
    parent = np.array([3, 6], dtype=np.int32)
    before_k, before_v = k.copy(), v.copy()
    k, v, _, _ = oracle.block_copy(k, v, [[6, 1]])
    child = np.array([3, 1], dtype=np.int32)
    kp, kc = rng.standard_normal((2, hkv, d))
    vp, vc = rng.standard_normal((2, hkv, d))
    slots = [oracle.slot_for_position(parent, n), oracle.slot_for_position(child, n)]
    k, v = oracle.cache_write(k, v, np.stack([kp, kc]), np.stack([vp, vc]), slots)
    assert np.array_equal(k[6, :, 5], kp) and np.array_equal(k[1, :, 5], kc)
    assert np.array_equal(k[6, :, :5], before_k[6, :, :5]) and np.array_equal(k[1, :, :5], before_k[6, :, :5])
    for b in (0, 2, 3, 4, 5, 7):  # the shared full block and all bystanders unchanged
        assert np.array_equal(k[b], before_k[b]) and np.array_equal(v[b], before_v[b])
    Kp = oracle.gather_sequence(k, parent, n + 1)
    Kc = oracle.gather_sequence(k, child, n + 1)
    assert np.array_equal(Kp[:n], Kc[:n]) and np.array_equal(Kp[n], kp) and np.array_equal(Kc[n], kc)


def test_cache_write_skips_negative_slots():
    k = np.zeros((2, 1, 16, 2))
    v = np.zeros((2, 1, 16, 2))
    kn = np.ones((3, 1, 2))
    k2, v2 = oracle.cache_write(k, v, kn, 2 * kn, [17, -1, 0])
    assert k2[1, 0, 1].tolist() == [1, 1] and k2[0, 0, 0].tolist() == [1, 1]
    assert k2.sum() == 4 and v2.sum() == 8


# --------------------------------------------------------------------------------------
# Brute force: the paged cache reproduces cache-free recomputation
# ("从KV Cache到vLLM" §1.2, 5688vip §3.1)
# --------------------------------------------------------------------------------------
class _TinyLayer:
    def __init__(self, seed, n, d_model=32, hq=4, hkv=2, d=16):
        rng = np.random.default_rng(seed)
        self.hq, self.hkv, self.d = hq, hkv, d
        self.x = rng.standard_normal((n, d_model))
        self.wq = rng.standard_normal((d_model, hq * d)) / np.sqrt(d_model)
        self.wk = rng.standard_normal((d_model, hkv * d)) / np.sqrt(d_model)
        self.wv = rng.standard_normal((d_model, hkv * d))

    def qkv(self, idx):
        x = self.x[idx]
        return ((x @ self.wq).reshape(len(idx), self.hq, self.d),
                (x @ self.wk).reshape(len(idx), self.hkv, self.d),
                (x @ self.wv).reshape(len(idx), self.hkv, self.d))

    def full_causal(self, scale):
        n = len(self.x)
        q, k, v = self.qkv(np.arange(n))
        mask = np.tril(np.ones((n, n), bool))
        return _sdpa(q, k, v, scale, mask[None])


class _Allocator:
    """Harness-side block allocation: a shuffled free list, one table row per request."""

    def __init__(self, rng, num_blocks):
        self.free = list(rng.permutation(num_blocks))

    def ensure(self, row, pos):
        if pos % BLOCK_SIZE == 0:  # current block full (or none yet): take a new one
            row.append(int(self.free.pop()))


def test_token_by_token_decode_equals_recompute():
    n = 40
    layer = _TinyLayer(1, n)
    scale = 1 / np.sqrt(layer.d)
    ref = layer.full_causal(scale)
    rng = np.random.default_rng(77)
    nb = 8
    k_pool = np.full((nb, layer.hkv, 16, layer.d), np.nan)
    v_pool = np.full((nb, layer.hkv, 16, layer.d), np.nan)
    alloc, row = _Allocator(rng, nb), []
    for p in range(n):
        q, k, v = layer.qkv([p])
        alloc.ensure(row, p)
        slot = oracle.slot_for_position(row, p)
        k_pool, v_pool = oracle.cache_write(k_pool, v_pool, k, v, [slot])
        bt = np.array([row], dtype=np.int32)
        out = oracle.decode(q, k_pool, v_pool, bt, [p + 1], scale)
        np.testing.assert_allclose(out[0], ref[p], rtol=0, atol=1e-12)


def test_chunked_prefill_mixed_batch_equals_recompute():
    """Two requests advance together: one by prefill chunks, one by decodes."""
    la, lb = _TinyLayer(2, 45), _TinyLayer(3, 30)
    scale = 1 / np.sqrt(la.d)
    ref_a, ref_b = la.full_causal(scale), lb.full_causal(scale)
    rng = np.random.default_rng(5)
    nb = 12
    k_pool = np.full((nb, 2, 16, la.d), np.nan)
    v_pool = np.full((nb, 2, 16, la.d), np.nan)
    alloc = _Allocator(rng, nb)
    rows = [[], []]
    chunks_a = [7, 9, 16, 1, 12]  # sums to 45
    pos_a, pos_b = 0, 0
    for step, ca in enumerate(chunks_a):
        cb = 15 if step == 0 else 1  # request b: prompt of 15, then decodes
        qs, ks, vs, slots, q_lens = [], [], [], [], []
        for layer, row, start, cnt in ((la, rows[0], pos_a, ca), (lb, rows[1], pos_b, cb)):
            idx = np.arange(start, start + cnt)
            q, k, v = layer.qkv(idx)
            for p in idx:
                alloc.ensure(row, p)
                slots.append(oracle.slot_for_position(row, p))
            qs.append(q), ks.append(k), vs.append(v), q_lens.append(cnt)
        k_pool, v_pool = oracle.cache_write(k_pool, v_pool, np.concatenate(ks), np.concatenate(vs), slots)
        pos_a += ca
        pos_b += cb
        mb = max(len(r) for r in rows)
        bt = np.array([r + [-1] * (mb - len(r)) for r in rows], dtype=np.int32)
        qsl = np.array([0, q_lens[0], q_lens[0] + q_lens[1]])
        out = oracle.prefill_chunk(np.concatenate(qs), k_pool, v_pool, qsl, [pos_a, pos_b], bt, scale)
        np.testing.assert_allclose(out[:ca], ref_a[pos_a - ca:pos_a], rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[ca:], ref_b[pos_b - cb:pos_b], rtol=0, atol=1e-12)
