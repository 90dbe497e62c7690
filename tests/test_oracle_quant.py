"""Pins for the oracle's quantise-on-write (CPU only).

The oracle's ``quantised_cache_write`` keeps one fp32 scale per (block, kv head)
of a 1-byte pool ("从KV Cache到vLLM" §2.2-2.3 store K/V as INT8 or FP8).  These
checks tie it to facts that do not restate its code: the scale equals the
running amax over the tile's rows divided by qmax; dequantised values stay
within the rounding error of the encodings they went through; rows written one
at a time equal one write of the block when the scale cannot grow; every stored
code is the nearest code (brute force over all codes) to the scaled value; zero
tiles, skipped slots and untouched tiles behave as defined.
"""
import numpy as np
import pytest

import oracle

QMAX = {"fp8": 448.0, "i8": 127.0}
NB, H, D = 10, 2, 16
BS = 16  # tokens per block; the pins below also run at 32 (5688vip §3.2 allows both)


def _empty_pool(kind):
    dt = np.uint8 if kind == "fp8" else np.int8
    codes = np.zeros((NB, H, BS, D), dtype=dt)
    scales = np.full((NB, H), np.float32(7.0), dtype=np.float32)  # garbage for fresh tiles
    return codes, scales


def _values(kind, codes):
    return oracle.e4m3fn_decode(codes) if kind == "fp8" else oracle.int8_decode(codes)


def _append_schedule(rng, blocks, chunk_sizes):
    """Write calls that append rows to the given blocks in order: list of slot lists."""
    fill = {b: 0 for b in blocks}
    calls = []
    for size in chunk_sizes:
        slots = []
        for b in blocks:
            k = min(size, BS - fill[b])
            slots += [b * BS + fill[b] + i for i in range(k)]
            fill[b] += k
        if slots:
            calls.append(slots)
    return calls, fill


def _run(kind, calls, x_of, rng_scale=None):
    codes, scales = _empty_pool(kind)
    for slots in calls:
        x = np.stack([x_of(s) for s in slots]).astype(np.float32)
        codes, scales = oracle.quantised_cache_write(codes, scales, x, np.array(slots), kind)
    return codes, scales


def _data(seed):
    rng = np.random.default_rng(seed)
    table = (rng.standard_normal((NB * BS, H, D)) * rng.uniform(0.01, 3.0, (NB * BS, 1, 1)))
    return table.astype(np.float32)


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_scale_is_running_amax_over_valid_rows(kind):
    rng = np.random.default_rng(1)
    data = _data(2)
    calls, fill = _append_schedule(rng, [0, 3, 7], [1, 1, 3, 5, 1, 4, 1, 16])
    codes, scales = _run(kind, calls, lambda s: data[s])
    for b in (0, 3, 7):
        for h in range(H):
            rows = data[b * BS:b * BS + fill[b], h]
            expect = np.float32(np.float32(np.max(np.abs(rows))) / np.float32(QMAX[kind]))
            assert scales[b, h] == expect, (b, h, scales[b, h], expect)


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_dequantised_values_within_rounding_bound(kind):
    rng = np.random.default_rng(3)
    data = _data(4)
    blocks = [1, 2, 5]
    calls, fill = _append_schedule(rng, blocks, [1, 2, 1, 1, 3, 2, 6])
    # count, for each row, the encodings it goes through: its own write plus one
    # per later growth of its tile's scale
    codes, scales = _empty_pool(kind)
    encodings = np.zeros((NB, H, BS), dtype=int)
    for slots in calls:
        before = scales.copy()
        x = np.stack([data[s] for s in slots])
        codes, scales = oracle.quantised_cache_write(codes, scales, x, np.array(slots), kind)
        for s in slots:
            encodings[s // BS, :, s % BS] = 1
        for b in {s // BS for s in slots}:
            off0 = min(s % BS for s in slots if s // BS == b)
            for h in range(H):
                if off0 > 0 and scales[b, h] > before[b, h]:
                    encodings[b, h, :off0] += 1
    for b in blocks:
        for h in range(H):
            s = float(scales[b, h])
            for r in range(fill[b]):
                x = data[b * BS + r, h].astype(np.float64)
                v = _values(kind, codes[b, h, r]) * s
                k = encodings[b, h, r]
                if kind == "fp8":  # half an ulp: 2^-4 relative (normal), 2^-10 scaled (subnormal)
                    bound = k * (0.07 * (np.abs(x) + 1e-30) + 2.0 ** -9 * s)
                else:             # half a code unit at a scale no larger than the final one
                    bound = k * 0.5 * s * (1 + 1e-6)
                assert np.all(np.abs(v - x) <= bound), (kind, b, h, r, np.max(np.abs(v - x) - bound))


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_rows_one_at_a_time_equal_one_write_when_scale_cannot_grow(kind):
    data = _data(5)
    b = 4
    rows = data[b * BS:(b + 1) * BS].copy()
    # row 0 holds every head's largest magnitude, so later rows never raise the scale
    for h in range(H):
        rows[0, h, 0] = np.float32(2.0) * np.max(np.abs(rows[:, h]))
    one = _run(kind, [[b * BS + r for r in range(BS)]], lambda s: rows[s - b * BS])
    each = _run(kind, [[b * BS + r] for r in range(BS)], lambda s: rows[s - b * BS])
    assert np.array_equal(one[0], each[0]) and np.array_equal(one[1], each[1])


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_stored_codes_are_the_nearest_codes(kind):
    data = _data(6)
    b = 2
    slots = [b * BS + r for r in range(5)]
    codes, scales = _run(kind, [slots], lambda s: data[s])
    all_codes = np.arange(256, dtype=np.uint8) if kind == "fp8" else np.arange(-127, 128).astype(np.int8)
    grid = _values(kind, all_codes)
    for h in range(H):
        s = scales[b, h]
        for r in range(5):
            for d in range(D):
                y = np.clip(np.float32(data[b * BS + r, h, d] / s), -QMAX[kind], QMAX[kind])
                dist = np.abs(np.where(np.isnan(grid), np.inf, grid) - float(y))
                best = np.flatnonzero(dist == dist.min())
                if len(best) > 1:  # tie: the even code (even mantissa / even integer)
                    best = [c for c in best if int(all_codes[c]) % 2 == 0]
                    if kind == "fp8" and len(best) > 1:  # +0 / -0: the sign of y
                        best = [c for c in best if (all_codes[c] >= 0x80) == bool(np.signbit(y))]
                assert codes[b, h, r, d] == all_codes[best[0]], (h, r, d, y)


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_zero_tile_then_growth(kind):
    codes, scales = _empty_pool(kind)
    zeros = np.zeros((3, H, D), dtype=np.float32)
    codes, scales = oracle.quantised_cache_write(codes, scales, zeros, np.array([BS, BS + 1, BS + 2]), kind)
    assert np.all(scales[1] == 0) and np.all(codes[1, :, :3] == 0)
    x = np.full((1, H, D), np.float32(0.25), dtype=np.float32)
    codes, scales = oracle.quantised_cache_write(codes, scales, x, np.array([BS + 3]), kind)
    assert np.all(scales[1] == np.float32(np.float32(0.25) / np.float32(QMAX[kind])))
    assert np.all(_values(kind, codes[1, :, :3]) == 0)
    assert np.all(_values(kind, codes[1, :, 3]) == QMAX[kind])


@pytest.mark.parametrize("kind", ["fp8", "i8"])
def test_skipped_slots_and_untouched_tiles(kind):
    rng = np.random.default_rng(8)
    codes = rng.integers(0, 0x7E, (NB, H, BS, D)).astype(np.uint8 if kind == "fp8" else np.int8)
    scales = rng.uniform(0.1, 1.0, (NB, H)).astype(np.float32)
    x = _data(9)[:3]
    c2, s2 = oracle.quantised_cache_write(codes, scales, x, np.array([-1, 6 * BS, -5]), kind)
    keep = [b for b in range(NB) if b != 6]
    assert np.array_equal(c2[keep], codes[keep]) and np.array_equal(s2[keep], scales[keep])
    # block 6 row 0 is a fresh tile: its scale comes from the one new row only
    assert np.all(s2[6] == (np.max(np.abs(x[1]), axis=-1) / np.float32(QMAX[kind])).astype(np.float32))


@pytest.fixture(params=[16, 32], autouse=True)
def block_size(request, monkeypatch):
    """Every pin above runs with 16- and with 32-token blocks."""
    monkeypatch.setitem(globals(), "BS", request.param)
    return request.param
