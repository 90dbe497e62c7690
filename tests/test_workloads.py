"""The seeded generators: deterministic, well-formed, and shaped like the workloads."""
import numpy as np
import torch

from paged_kv_cache_455_amd import workloads as W


def _owned_blocks(b):
    bt = b.block_tables.numpy()
    return bt[bt >= 0]


def test_deterministic():
    a, b = W.llama3_8b_decode(batch=4), W.llama3_8b_decode(batch=4)
    assert torch.equal(a.q, b.q) and torch.equal(a.k_pool, b.k_pool)
    assert torch.equal(a.block_tables, b.block_tables)


def test_tiny_shape():
    b = W.tiny_fp32()
    assert b.seq_lens.tolist() == [5, 16, 17, 40]
    assert b.k_pool.shape == (32, 2, 16, 64) and b.q.shape == (4, 4, 64)
    assert abs(b.scale - 1 / 8) < 1e-15
    ids = _owned_blocks(b)
    assert len(ids) == 7 and len(set(ids.tolist())) == 7
    # unused blocks are NaN-poisoned, owned ones are finite
    used = np.zeros(32, bool)
    used[ids] = True
    assert torch.isnan(b.k_pool[torch.from_numpy(~used)]).all()
    assert torch.isfinite(b.k_pool[torch.from_numpy(used)]).all()


def test_llama3_shape_and_pool():
    b = W.llama3_8b_decode()
    ctx = b.seq_lens.numpy()
    assert len(ctx) == 64 and ctx.min() >= 128 and ctx.max() <= 4096
    need = int(sum(-(-int(n) // 16) for n in ctx))
    assert b.num_blocks == int(np.ceil(1.1 * need))
    ids = _owned_blocks(b)
    assert len(ids) == need and len(set(ids.tolist())) == need
    assert b.q.dtype == torch.float16 and b.q.shape == (64, 32, 128)
    assert b.k_pool.shape[1:] == (8, 16, 128)


def test_prefix_cow_structure():
    b = W.prefix_cow()
    n_req = b.extra["n_req"]
    forks = b.extra["forks"]
    assert n_req == 128 and len(forks) == 16 and b.num_seqs == 144
    bt = b.block_tables.numpy()
    shared = b.extra["shared_blocks"]
    assert len(shared) == 64
    assert (bt[:, :64] == shared[None, :]).all()
    ctx = b.seq_lens.numpy()
    pairs = b.copy_pairs.numpy()
    for i, f in enumerate(forks):
        child = n_req + i
        L = ctx[f] - 1
        assert L % 16 != 0 and ctx[child] == ctx[f]
        last = L // 16
        assert pairs[i, 0] == bt[f, last] and pairs[i, 1] == bt[child, last]
        assert (bt[child, :last] == bt[f, :last]).all()
    # private blocks are unique across all rows; destinations are fresh
    private = np.concatenate([bt[r, 64:][bt[r, 64:] >= 0] for r in range(n_req)])
    assert len(set(private.tolist())) == len(private)
    assert not set(pairs[:, 1].tolist()) & set(private.tolist())


def test_mixed_structure():
    b = W.mixed_step()
    qsl = b.query_start_loc.numpy()
    q_len = qsl[1:] - qsl[:-1]
    assert (q_len[:8] == 512).all() and (q_len[8:] == 1).all() and b.num_tokens == 4352
    prior = b.seq_lens.numpy()[:8] - 512
    assert prior.min() >= 0 and prior.max() <= 2048
    dec = b.seq_lens.numpy()[8:]
    assert dec.min() >= 16 and dec.max() <= 8192 and 300 < np.median(dec) < 1200


def test_long_quantised_codes_and_scales():
    f = W.long_quantised("fp8", batch=2, ctx=320)
    i = W.long_quantised("i8", batch=2, ctx=320)
    assert f.k_pool.dtype == torch.uint8 and i.k_pool.dtype == torch.int8
    assert f.k_scale.shape == (f.num_blocks, 8) and (f.k_scale > 0).all()
    # same N(0,1) draws: scales differ exactly by the ratio of the code ranges
    torch.testing.assert_close(f.k_scale * 448.0, i.k_scale * 127.0, rtol=1e-6, atol=0)
    # every tile reaches its largest code
    assert int(i.k_pool.abs().amax()) == 127
    assert torch.equal(f.block_tables, i.block_tables) and torch.equal(f.q, i.q)
