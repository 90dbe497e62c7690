"""A short serving loop: the host block manager drives the device calls.

Each step follows the protocol the manager's arrays are made for (uml.org.cn
"PagedAttention", "Prefix Sharing" and "Continuous Batching"; 5688vip chapter 3,
section 3.2): kv_swap of the step's swap-outs (device -> pinned host pool) and
swap-ins (host -> device), kv_block_copy over its copy-on-write pairs,
pa_slot_mapping, the K/V writes of the query tokens, then pa_decode (all rows
decodes) or pa_prefill_chunk (a mixed step).  Requests are added with shared
prompts (prefix cache hits), forked (parallel sampling, copy-on-write), grown,
swapped out (their device blocks reused meanwhile), swapped back in and released.

Checked every step:
* the device slot mapping equals the oracle's slot of every query position;
* the device and host pools (and scales) equal, bit for bit, an oracle mirror
  that applies the same swaps, copies and writes;
* the attention outputs match the oracle on the mirror, and for 16-bit pools
  also a paging-free recompute: softmax attention over each request's history,
  whose row at position p is a fixed function of the tokens 0..p.  The rows are
  N(0,1), so early prefill outputs reach |out| ~ 3: each element's bar is the
  larger of the dtype's max-abs tolerance and one ulp of the output type.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_455_amd as pa

from .pa_testlib import err_over_bar, max_err, np_of

pytestmark = pytest.mark.gpu

NB, NH, MB = 64, 24, 16
HQ, HKV, D = 16, 2, 128
SCALE = 1.0 / np.sqrt(D)
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)


class History:
    """K/V rows as a function of the token prefix they close."""

    def __init__(self):
        self.rows = {}

    def kv(self, toks, pos):
        key = tuple(toks[:pos + 1])
        if key not in self.rows:
            h = 0
            for t in key:
                h = (h * 1000003 + int(t) + 1) % (1 << 62)
            rng = np.random.default_rng([h, 7])
            self.rows[key] = rng.standard_normal((2, HKV, D)).astype(np.float32)
        return self.rows[key]


def scenario():
    """(adds, forks, appends, releases) per step; tokens drawn from a seeded rng."""
    rng = np.random.default_rng(3)
    P = list(rng.integers(0, 500, 37))
    Q = list(rng.integers(0, 500, 50))
    tok = lambda: int(rng.integers(0, 500))
    steps = [
        dict(add={1: P, 2: Q[:20]}),
        dict(add={3: P + [7, 8, 9, 10, 11]}, append={1: [tok()], 2: [tok()]}),
        dict(fork=[(1, 4), (1, 5)], append={r: [tok()] for r in (1, 2, 3, 4, 5)}),
        dict(append={r: [tok()] for r in (1, 2, 3, 4, 5)}),
        dict(append={r: [tok()] for r in (1, 2, 3, 4, 5)}),
        dict(release=[2], append={r: [tok()] for r in (1, 3, 4, 5)}),
        dict(add={6: Q}, append={r: [tok()] for r in (1, 3, 4, 5)}),
        dict(add={7: P + [1] * 30}, fork=[(3, 8)], append={r: [tok()] for r in (1, 3, 4, 6, 8)}),
        dict(release=[5], append={r: [tok()] for r in (1, 3, 4, 6, 7, 8)}),
        dict(swap_out=[4, 6], append={r: [tok()] for r in (1, 3, 7, 8)}),
        dict(add={9: Q[:5] + [3] * 60}, append={r: [tok()] for r in (1, 3, 7, 8)}),
        dict(swap_in=[4, 6], append={r: [tok()] for r in (1, 3, 4, 6, 7, 8, 9)}),
    ]
    for _ in range(3):
        steps.append(dict(append={r: [tok()] for r in (1, 3, 4, 6, 7, 8, 9)}))
    steps.append(dict(append={1: [tok() for _ in range(21)], 8: [tok()]}))  # a chunk
    return steps


def _pool(kv, bs, n=NB, device="cuda"):
    pin = device == "cpu"
    if kv in TORCH:
        z = lambda: torch.zeros((n, HKV, bs, D), dtype=TORCH[kv], device=device, pin_memory=pin)
        return pa.KVPool(z(), z(), shared_blocks=True), None
    z = lambda: torch.zeros((n, HKV, bs, D), dtype=torch.uint8, device=device, pin_memory=pin)
    s = lambda: torch.zeros((n, HKV), dtype=torch.float32, device=device, pin_memory=pin)
    return pa.KVPool(z(), z(), s(), s(), shared_blocks=True), "e4m3fn"


def _mirror(codec, n, bs):
    mk = np.zeros((n, HKV, bs, D), dtype=np.uint8 if codec else np.float32)
    return dict(k=mk.copy(), v=mk.copy(), ks=np.zeros((n, HKV), np.float32),
                vs=np.zeros((n, HKV), np.float32))


def _tup(m):
    return (m["k"], m["v"], m["ks"], m["vs"])


def _untup(t):
    return dict(k=t[0], v=t[1], ks=t[2], vs=t[3])


@pytest.mark.parametrize("kv,bs", [("f16", 16), ("bf16", 16), ("fp8", 16), ("f16", 32), ("fp8", 32)])
def test_block_manager_drives_the_device_path(kv, bs):
    say(f"[serving] kv={kv} block_size={bs}")
    pool, codec = _pool(kv, bs)
    hpool, _ = _pool(kv, bs, NH, "cpu")
    qdt = TORCH.get(kv, torch.float16)
    mirror, hmirror = _mirror(codec, NB, bs), _mirror(codec, NH, bs)
    bm = pa.BlockManager(NB, NH, block_size=bs)
    hist, live, unwritten = History(), {}, set()
    rng = np.random.default_rng(11)
    ws = None
    for si, ev in enumerate(scenario()):
        for r in ev.get("release", []):
            bm.release(r)
            del live[r]
            unwritten.discard(r)
        for p, c in ev.get("fork", []):
            bm.fork(p, c)
            live[c] = list(live[p])
        for r in ev.get("swap_out", []):
            say(f"  step {si}: swap out {r} ({bm.swap_out(r)} blocks)")
        for r in ev.get("swap_in", []):
            bm.swap_in(r)
        for r, toks in ev.get("add", {}).items():
            cached = bm.add(r, toks)
            live[r] = list(toks)
            unwritten.add(r)
            say(f"  step {si}: add {r} ({len(toks)} tokens, {cached} cached)")
        for r, toks in ev.get("append", {}).items():
            bm.append(r, toks)
            live[r] += toks
            unwritten.add(r)
        out_np, in_np = bm.swaps()
        reqs = sorted(unwritten)
        bt_np, lens_np, qsl_np, pairs_np = bm.step(reqs, MB)
        unwritten.clear()
        T = int(qsl_np[-1])
        q_lens = np.diff(qsl_np)
        say(f"  step {si}: {len(reqs)} requests, {T} query rows, {len(pairs_np)} copies, "
            f"{len(out_np)} out / {len(in_np)} in")

        # device: swaps, copies, slot mapping, writes, attention
        bt = torch.from_numpy(bt_np).cuda()
        lens = torch.from_numpy(lens_np).cuda()
        qsl = torch.from_numpy(qsl_np).cuda()
        if len(out_np):
            pa.kv_swap(hpool, pool, torch.from_numpy(out_np.copy()).cuda())
        if len(in_np):
            pa.kv_swap(pool, hpool, torch.from_numpy(in_np.copy()).cuda())
        if len(pairs_np):
            pa.kv_block_copy(pool, torch.from_numpy(pairs_np.copy()).cuda())
        slots = pa.pa_slot_mapping(bt, qsl, lens, T, block_size=bs)
        pos = [(i, r, int(lens_np[i]) - int(q_lens[i]) + j)
               for i, r in enumerate(reqs) for j in range(int(q_lens[i]))]
        kv_new = np.stack([hist.kv(live[r], p) for _, r, p in pos])       # [T][2][HKV][D]
        knew = torch.from_numpy(kv_new[:, 0]).to(qdt).cuda()
        vnew = torch.from_numpy(kv_new[:, 1]).to(qdt).cuda()
        if codec:
            pa.kv_cache_write_quant(pool, knew, vnew, slots)
        else:
            pa.kv_cache_write(pool, knew, vnew, slots)
        q = torch.from_numpy(rng.standard_normal((T, HQ, D)).astype(np.float32)).to(qdt).cuda()
        if (q_lens == 1).all():
            out = pa.pa_decode(pool, q, bt, lens, int(lens_np.max()), SCALE)
        else:
            need = pa.pa_prefill_workspace_size(len(reqs), T, HQ, HKV, D, int(q_lens.max()),
                                                int(lens_np.max()), pool.k.dtype)
            if ws is None or ws.numel() < need:
                ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
            out = pa.pa_prefill_chunk(pool, q, qsl, lens, bt, int(q_lens.max()),
                                      int(lens_np.max()), SCALE, workspace=ws)
        torch.cuda.synchronize()

        # oracle: slots, mirror pools, attention
        want_slots = [oracle.slot_for_position(bt_np[i], p, bs) for i, _, p in pos]
        assert slots.cpu().tolist() == want_slots
        if len(out_np):
            hmirror = _untup(oracle.swap_blocks(_tup(hmirror), _tup(mirror), out_np))
        if len(in_np):
            mirror = _untup(oracle.swap_blocks(_tup(mirror), _tup(hmirror), in_np))
        if len(pairs_np):
            k2, v2, ks2, vs2 = oracle.block_copy(mirror["k"], mirror["v"], pairs_np,
                                                 mirror["ks"], mirror["vs"])
            mirror.update(k=k2, v=v2, ks=ks2, vs=vs2)
        kn, vn = np_of(knew.cpu()), np_of(vnew.cpu())
        if codec:
            mirror["k"], mirror["ks"] = oracle.quantised_cache_write(mirror["k"], mirror["ks"], kn,
                                                                     np.array(want_slots), "fp8")
            mirror["v"], mirror["vs"] = oracle.quantised_cache_write(mirror["v"], mirror["vs"], vn,
                                                                     np.array(want_slots), "fp8")
            assert np.array_equal(pool.k_scale.cpu().numpy(), mirror["ks"])
            assert np.array_equal(pool.v_scale.cpu().numpy(), mirror["vs"])
        else:
            mirror["k"], mirror["v"] = oracle.cache_write(mirror["k"], mirror["v"], kn, vn,
                                                          np.array(want_slots))
        assert np.array_equal(np_of(pool.k.cpu()), mirror["k"]), f"step {si}: K pool"
        assert np.array_equal(np_of(pool.v.cpu()), mirror["v"]), f"step {si}: V pool"
        assert np.array_equal(np_of(hpool.k), hmirror["k"]), f"step {si}: host K pool"
        assert np.array_equal(np_of(hpool.v), hmirror["v"]), f"step {si}: host V pool"
        if codec:
            assert np.array_equal(hpool.k_scale.numpy(), hmirror["ks"])
        kw = {}
        if codec:
            kw = dict(k_scale=mirror["ks"].astype(np.float64), v_scale=mirror["vs"].astype(np.float64),
                      codec=codec)
        qn = np_of(q.cpu()).astype(np.float64)
        ref = oracle.prefill_chunk(qn, mirror["k"], mirror["v"], qsl_np, lens_np, bt_np, SCALE, **kw)
        ratio = err_over_bar(out, ref, kv)
        say(f"  step {si}: max_err {max_err(out, ref):.2e}, over bar {ratio:.2f}")
        assert ratio <= 1.0
        if not codec:  # paging-free recompute over each request's history
            for i, r in enumerate(reqs):
                n = int(lens_np[i])
                rows = np.stack([hist.kv(live[r], p) for p in range(n)])
                K = np_of(torch.from_numpy(rows[:, 0]).to(qdt)).astype(np.float64)
                V = np_of(torch.from_numpy(rows[:, 1]).to(qdt)).astype(np.float64)
                a, b = int(qsl_np[i]), int(qsl_np[i + 1])
                vis = [n - (b - a) + j + 1 for j in range(b - a)]
                want = oracle.attention_rows(qn[a:b], K, V, SCALE, vis)
                assert err_over_bar(out[a:b], want, kv) <= 1.0, (si, r)
    assert bm.num_free() < NB
