"""Pins for the oracle's block swap between pools (CPU only).

``oracle.swap_blocks`` moves blocks between a device pool and a host pool
(uml.org.cn "PagedAttention": pages go out to CPU memory under memory pressure
and come back later).  Facts that do not restate its code: a request read
through its host-side table after swapping out gives the same rows (values
decoded with their scales) as through its device table before; swapping out and
back in to other block ids is the identity on the request's rows; blocks outside
the pairs and the source pool do not change.
"""
import numpy as np
import pytest

import oracle

NB, NH, H, D = 12, 6, 2, 8


def _pools(rng, quant):
    if quant:
        k = rng.integers(0, 0x7F, (NB, H, 16, D)).astype(np.uint8)
        v = rng.integers(0, 0x7F, (NB, H, 16, D)).astype(np.uint8)
        return (k, v, rng.uniform(0.1, 2, (NB, H)).astype(np.float32),
                rng.uniform(0.1, 2, (NB, H)).astype(np.float32))
    return (rng.standard_normal((NB, H, 16, D)), rng.standard_normal((NB, H, 16, D)), None, None)


def _host(quant):
    z = np.zeros((NH, H, 16, D), dtype=np.uint8 if quant else np.float64)
    s = np.zeros((NH, H), dtype=np.float32) if quant else None
    return (z.copy(), z.copy(), s if s is None else s.copy(), s if s is None else s.copy())


def _read(pools, row, n, quant):
    kw = dict(codec="e4m3fn") if quant else {}
    k = oracle.gather_sequence(pools[0], row, n, pools[2], **kw)
    v = oracle.gather_sequence(pools[1], row, n, pools[3], **kw)
    return k, v


@pytest.mark.parametrize("quant", [False, True])
def test_request_reads_the_same_through_its_host_table(quant):
    rng = np.random.default_rng(1)
    dev = _pools(rng, quant)
    row, n = np.array([7, 2, 9]), 40
    host_row = np.array([4, 0, 3])
    host = oracle.swap_blocks(_host(quant), dev, np.stack([row, host_row], 1))
    for a, b in zip(_read(dev, row, n, quant), _read(host, host_row, n, quant)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("quant", [False, True])
def test_out_and_back_in_is_the_identity_on_the_rows(quant):
    rng = np.random.default_rng(2)
    dev = _pools(rng, quant)
    row, n = np.array([1, 5, 8, 11]), 57
    host_row = np.array([5, 1, 2, 0])
    new_row = np.array([3, 10, 0, 6])
    host = oracle.swap_blocks(_host(quant), dev, np.stack([row, host_row], 1))
    back = oracle.swap_blocks(dev, host, np.stack([host_row, new_row], 1))
    for a, b in zip(_read(dev, row, n, quant), _read(back, new_row, n, quant)):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("quant", [False, True])
def test_blocks_outside_the_pairs_and_the_source_do_not_change(quant):
    rng = np.random.default_rng(3)
    dev = _pools(rng, quant)
    before = [None if a is None else a.copy() for a in dev]
    host0 = _pools(np.random.default_rng(4), quant)
    host0 = tuple(None if a is None else a[:NH].copy() for a in host0)
    host = oracle.swap_blocks(host0, dev, [[3, 1], [6, 4]])
    for a, b in zip(dev, before):
        assert a is None or np.array_equal(a, b)
    keep = [i for i in range(NH) if i not in (1, 4)]
    for a, b in zip(host, host0):
        assert a is None or np.array_equal(a[keep], b[keep])
