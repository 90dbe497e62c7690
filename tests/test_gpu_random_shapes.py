"""GPU parity over seeded random decode shapes and mixed steps: every KV type,
head_dim 64 and 128, GQA groups 1-8, block sizes 16 and 32, shared-block (cached)
and streamed pools, random batch sizes and context lengths mixed with block and
split edges, NaN past every context.  Unscaled N(0,1) data ("peaked": the scores decide the output),
each element held to the larger of its KV type's max-abs tolerance and one ulp of
the output type at the oracle's value.  The cases cross the decode paths (VALU and
matrix-core tiles, one or two workgroups per CU, the split's two-round skew) in
combinations the shape-by-shape tests do not list one by one.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_455_amd import workloads as W

from .pa_testlib import Dev, err_over_bar, oracle_decode_rows, poison_tails
from .test_gpu_parity import run_decode, say

pytestmark = pytest.mark.gpu

KV_Q = {"f32": ["f32"], "f16": ["f16"], "bf16": ["bf16"], "fp8": ["bf16", "f16"], "i8": ["bf16", "f16"]}
EDGES = [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 511, 513]


def case(i: int):
    rng = np.random.default_rng(1000 + i)
    kv = ["f32", "f16", "bf16", "fp8", "i8"][i % 5]
    qd = KV_Q[kv][int(rng.integers(len(KV_Q[kv])))]
    hd = [64, 128][int(rng.integers(2))]
    g = [1, 2, 4, 8][int(rng.integers(4))]
    hkv = [1, 2, 4, 8][int(rng.integers(4))]
    bs = [16, 32][int(rng.integers(2))]
    n = int(rng.integers(1, 21))
    ctx = [int(c) for c in rng.integers(1, 3001, size=n)]
    ctx[: min(n, 3)] = [int(e) for e in rng.choice(EDGES, size=min(n, 3), replace=False)]
    shared = bool(rng.integers(2))
    return kv, qd, hd, g, hkv, bs, ctx, shared


@pytest.mark.parametrize("i", range(120))
def test_random_decode_shape_peaked(i):
    kv, qd, hd, g, hkv, bs, ctx, shared = case(i)
    b = W.decode_batch(2000 + i, ctx, g * hkv, hkv, hd, kv, qd, poison=True, block_size=bs,
                       name=f"random-{i}-{kv}-{qd}-g{g}-hkv{hkv}-d{hd}-bs{bs}-n{len(ctx)}"
                            f"{'-shared' if shared else ''}")
    b = poison_tails(b)
    say(b.name, "max ctx", max(ctx))
    out = run_decode(Dev(b, shared_blocks=shared))
    torch.cuda.synchronize()
    r = err_over_bar(out, oracle_decode_rows(b), kv)
    say(b.name, "max err/bar", r)
    assert r <= 1.0, (b.name, r)


def mixed_case(i: int):
    rng = np.random.default_rng(5000 + i)
    kv = ["f16", "bf16", "fp8", "i8", "f32"][i % 5]
    qd = KV_Q[kv][int(rng.integers(len(KV_Q[kv])))]
    hd = [64, 128][int(rng.integers(2))]
    g = [1, 2, 4, 8][int(rng.integers(4))]
    hkv = [1, 2, 4][int(rng.integers(3))]
    bs = [16, 32][int(rng.integers(2))]
    n_chunks = int(rng.integers(1, 5))
    chunk_len = int(rng.integers(1, 301))
    priors = [int(p) for p in rng.integers(0, 701, size=n_chunks)]
    priors[0] = int(rng.choice([0, 1, 15, 16, 17, 32]))
    n_dec = int(rng.integers(0, 13))
    return kv, qd, hd, g, hkv, bs, n_chunks, chunk_len, priors, n_dec


@pytest.mark.parametrize("i", range(30))
def test_random_mixed_step_peaked(i):
    """Random mixed steps (chunked prefills over random priors beside decodes) on
    every KV type, head_dim and group, block sizes 16 and 32, peaked data; every
    query row against the oracle."""
    from .pa_testlib import oracle_mixed
    from .test_gpu_parity import run_mixed
    kv, qd, hd, g, hkv, bs, n_chunks, chunk_len, priors, n_dec = mixed_case(i)
    b = W.mixed_batch(6000 + i, n_chunks, chunk_len, 0, 0, n_dec, 300.0, 1.0, 1, 1500, g * hkv,
                      hkv, hd, kv, qd, poison=True, priors=priors, block_size=bs,
                      name=f"random-mixed-{i}-{kv}-{qd}-g{g}-hkv{hkv}-d{hd}-bs{bs}-c{n_chunks}x"
                           f"{chunk_len}-dec{n_dec}")
    b = poison_tails(b)
    say(b.name, "priors", priors)
    out = run_mixed(Dev(b))
    torch.cuda.synchronize()
    rows, ref = oracle_mixed(b)
    assert np.array_equal(rows, np.arange(b.num_tokens))
    r = err_over_bar(out, ref, kv)
    say(b.name, "max err/bar", r)
    assert r <= 1.0, (b.name, r)
