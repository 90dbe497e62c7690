"""Pins for the oracle at 32 tokens per block (CPU only).

5688vip chapter 3, section 3.2 allows blocks of 16 or 32 tokens; the oracle takes
the block size from the pools' third axis.  The pin that does not restate its
code: a request's tokens laid out in 32-token blocks (each the concatenation of
two 16-token blocks of another layout) read back, decode, prefill and take new
tokens exactly as in the 16-token layout.
"""
import numpy as np
import pytest

import oracle

H, D, HQ = 2, 8, 4


def _layouts(rng, n, quant):
    """The same n tokens in a 16-token pool and a 32-token pool, with tables."""
    nb16 = -(-n // 16) + (-(-n // 16)) % 2          # even number of 16-blocks
    perm16 = rng.permutation(40)[:nb16]
    if quant:
        k16 = rng.integers(0, 0x7F, (40, H, 16, D)).astype(np.uint8)
        v16 = rng.integers(0, 0x7F, (40, H, 16, D)).astype(np.uint8)
        ks16 = rng.uniform(0.1, 2, (40, H)).astype(np.float32)
        vs16 = rng.uniform(0.1, 2, (40, H)).astype(np.float32)
        for j in range(0, nb16, 2):                 # a 32-block has one scale per head
            ks16[perm16[j + 1]] = ks16[perm16[j]]
            vs16[perm16[j + 1]] = vs16[perm16[j]]
    else:
        k16, v16 = rng.standard_normal((40, H, 16, D)), rng.standard_normal((40, H, 16, D))
        ks16 = vs16 = None
    perm32 = rng.permutation(25)[:nb16 // 2]
    k32 = np.zeros((25, H, 32, D), dtype=k16.dtype)
    v32 = np.zeros_like(k32)
    ks32 = vs32 = None
    if quant:
        ks32 = np.zeros((25, H), np.float32)
        vs32 = np.zeros((25, H), np.float32)
    for i, b32 in enumerate(perm32):
        a, b = perm16[2 * i], perm16[2 * i + 1]
        k32[b32] = np.concatenate([k16[a], k16[b]], axis=1)
        v32[b32] = np.concatenate([v16[a], v16[b]], axis=1)
        if quant:
            ks32[b32], vs32[b32] = ks16[a], vs16[a]
    return (k16, v16, ks16, vs16, perm16), (k32, v32, ks32, vs32, perm32)


@pytest.mark.parametrize("quant", [False, True])
@pytest.mark.parametrize("n", [1, 16, 17, 32, 33, 95])
def test_32_token_blocks_read_like_two_16_token_blocks(quant, n):
    rng = np.random.default_rng(n + 7 * quant)
    L16, L32 = _layouts(rng, n, quant)
    kw = dict(codec="e4m3fn") if quant else {}
    for a, b in ((0, 2), (1, 3)):
        x16 = oracle.gather_sequence(L16[a], L16[4], n, L16[b], **kw)
        x32 = oracle.gather_sequence(L32[a], L32[4], n, L32[b], **kw)
        assert x16.shape == (n, H, D) and np.array_equal(x16, x32)


@pytest.mark.parametrize("quant", [False, True])
def test_decode_and_prefill_match_across_block_sizes(quant):
    rng = np.random.default_rng(3)
    n = 75
    L16, L32 = _layouts(rng, n, quant)
    kw16 = dict(k_scale=L16[2], v_scale=L16[3], codec="e4m3fn") if quant else {}
    kw32 = dict(k_scale=L32[2], v_scale=L32[3], codec="e4m3fn") if quant else {}
    q = rng.standard_normal((1, HQ, D))
    d16 = oracle.decode(q, L16[0], L16[1], L16[4][None], np.array([n]), 0.3, **kw16)
    d32 = oracle.decode(q, L32[0], L32[1], L32[4][None], np.array([n]), 0.3, **kw32)
    assert np.allclose(d16, d32, rtol=0, atol=1e-12)
    qp = rng.standard_normal((9, HQ, D))
    qsl = np.array([0, 9])
    p16 = oracle.prefill_chunk(qp, L16[0], L16[1], qsl, np.array([n]), L16[4][None], 0.3, **kw16)
    p32 = oracle.prefill_chunk(qp, L32[0], L32[1], qsl, np.array([n]), L32[4][None], 0.3, **kw32)
    assert np.allclose(p16, p32, rtol=0, atol=1e-12)


def test_cache_write_lands_where_the_32_token_table_says():
    rng = np.random.default_rng(4)
    n = 40
    L16, L32 = _layouts(rng, n + 5, False)
    new_k = rng.standard_normal((5, H, D))
    new_v = rng.standard_normal((5, H, D))
    out = {}
    for name, (k, v, _, _, row) in (("16", L16), ("32", L32)):
        bs = k.shape[2]
        slots = [oracle.slot_for_position(row, p, bs) for p in range(n, n + 5)]
        k2, v2 = oracle.cache_write(k, v, new_k, new_v, np.array(slots))
        out[name] = (oracle.gather_sequence(k2, row, n + 5), oracle.gather_sequence(v2, row, n + 5))
    assert np.array_equal(out["16"][0], out["32"][0]) and np.array_equal(out["16"][1], out["32"][1])
    assert np.array_equal(out["32"][0][n:], new_k)
