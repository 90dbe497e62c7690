#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the whole path over one synthetic batch already resident
in HBM: slot mapping -> (copy-on-write block copies) -> cache write of this
step's K/V -> paged attention (decode, or the mixed prefill+decode launch).  A
decode step runs slot mapping, write and decode as one pa_decode_append call
(``--unfused``: separate calls); 1-byte pools quantise the new rows on write
inside it.

Default workload: the Llama-3-8B-shaped decode layer (64 sequences, contexts
uniform in [128, 4096], 32 query / 8 KV heads, head_dim 128, fp16 KV, fp32
accumulation).  `value` is the step's algorithmic bytes divided by the step
time (effective GB/s); the roofline object prices the attention launch alone
(its algorithmic bytes over its HIP-event-timed duration) against the 8 TB/s
HBM peak.  The pools are rotated among several copies between steps so that
the 256 MB Infinity Cache cannot serve a step from a previous step's reads.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--rotate R]
"""
import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode effective KV GB/s (% of HBM peak) and tokens/s at Llama-3-8B shape"
HBM_PEAK_GBPS = 8000.0
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "i8": 1}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=600)
    ap.add_argument("--min-warm-ms", type=float, default=100.0,
                    help="untimed steps continue past --warmup until this much time has "
                         "passed: the first tens of ms of steps run slower")
    ap.add_argument("--workload", default="llama3-decode",
                    choices=["llama3-decode", "tiny", "prefix-cow", "mixed", "long-fp8", "long-i8"])
    ap.add_argument("--rotate", type=int, default=4, help="pool copies cycled between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device copy three times (byte-counter calibration)")
    ap.add_argument("--block-size", type=int, default=16, choices=[16, 32],
                    help="tokens per KV block (the pages allow 16 or 32)")
    ap.add_argument("--graph", action="store_true",
                    help="time the decode step eagerly and as a replayed HIP graph")
    ap.add_argument("--unfused", action="store_true",
                    help="decode step as separate slot-mapping, cache-write and decode calls "
                         "instead of pa_decode_append")
    ap.add_argument("--per-step-events", action="store_true",
                    help="bracket every step's timed call with its own event pair")
    ap.add_argument("--swap", action="store_true",
                    help="measure kv_swap (device pool <-> pinned host pool) instead of the step")
    return ap.parse_args()


def make_batch(name, block_size=16):
    from paged_kv_cache_455_amd import workloads as W
    kw = dict(block_size=block_size)
    return {"llama3-decode": lambda: W.llama3_8b_decode(**kw),
            "tiny": lambda: W.tiny_fp32(**kw), "prefix-cow": lambda: W.prefix_cow(**kw),
            "mixed": lambda: W.mixed_step(**kw), "long-fp8": lambda: W.long_quantised("fp8", **kw),
            "long-i8": lambda: W.long_quantised("i8", **kw)}[name]()


# ---------------------------------------------------------------------------------------
# algorithmic work (what the path must move / compute, independent of the kernels)
# ---------------------------------------------------------------------------------------
def attention_bytes(b, seqs=None):
    """KV (+ scales, table entries) read once per (sequence, kv head), q read, out written."""
    e = ELEM[b.kv_dtype]
    eq = ELEM[b.q_dtype]
    qsl = b.query_start_loc.tolist()
    lens = b.seq_lens.tolist()
    seqs = range(b.num_seqs) if seqs is None else seqs
    tot = 0
    for s in seqs:
        n = lens[s]
        q_len = qsl[s + 1] - qsl[s]
        nblk = -(-n // b.block_size)
        tot += 2 * n * b.num_kv_heads * b.head_dim * e
        if b.kv_dtype in ("fp8", "i8"):
            tot += 2 * nblk * b.num_kv_heads * 4
        tot += nblk * 4
        tot += q_len * b.num_q_heads * b.head_dim * 2 * eq
    return tot


def attention_flops(b):
    qsl = b.query_start_loc.tolist()
    tot = 0
    for s, n in enumerate(b.seq_lens.tolist()):
        q_len = qsl[s + 1] - qsl[s]
        c = n - q_len
        tot += 4 * b.num_q_heads * b.head_dim * (q_len * c + q_len * (q_len + 1) // 2)
    return tot


def side_bytes(b):
    """Cache write (read new K/V, write pool rows), slots, and CoW copies (read + write)."""
    e = ELEM[b.kv_dtype]
    tot = b.num_tokens * 8
    if b.k_new is not None:  # read the new rows (their own dtype), write them in the pool's
        tot += 2 * b.num_tokens * b.num_kv_heads * b.head_dim * (b.k_new.element_size() + e)
    if b.copy_pairs is not None:
        tot += 2 * 2 * int(b.copy_pairs.shape[0]) * b.num_kv_heads * b.block_size * b.head_dim * e
    return tot


# ---------------------------------------------------------------------------------------
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvent:
    """A HIP event used only to time work on one stream, created with
    hipEventDisableSystemFence: recording it skips the system-scope cache writeback
    and invalidation of a default event (torch.cuda.Event), which leaves the GPU
    idle for several microseconds at every record and would be counted in the
    bracketed time.  Called on the HIP runtime torch has loaded."""
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = "libamdhip64.so.7"  # the soname: dlopen returns the loaded copy
            for line in open("/proc/self/maps"):
                if "/libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
            h = ctypes.CDLL(path)
            vp, P = ctypes.c_void_p, ctypes.POINTER
            h.hipEventCreateWithFlags.argtypes = [P(vp), ctypes.c_uint]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipEventElapsedTime.argtypes = [P(ctypes.c_float), vp, vp]
            h.hipEventDestroy.argtypes = [vp]
            cls._hip = h
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self._h = self._runtime()
        self._e = ctypes.c_void_p()
        rc = self._h.hipEventCreateWithFlags(ctypes.byref(self._e), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self._h.hipEventRecord(self._e, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to ``end`` (both complete)."""
        ms = self._ct.c_float()
        rc = self._h.hipEventElapsedTime(self._ct.byref(ms), self._e, end._e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if getattr(self, "_e", None) and self._e.value:
            self._h.hipEventDestroy(self._e)


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_455_amd", "csrc")


def _code_tokens(text):
    """C++ source with its comments and whitespace runs removed (string and
    character literals kept whole), so that an edit of comments alone leaves it
    unchanged."""
    import re
    tok = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/|\s+', re.S)
    out, pos, gap = [], 0, False
    for m in tok.finditer(text):
        if m.start() > pos:  # code between the matches
            out.append((" " if gap and out else "") + text[pos:m.start()])
            gap = False
        if m.group(0)[0] in "\"'":
            out.append((" " if gap and out else "") + m.group(0))
            gap = False
        else:  # a comment or whitespace: at most one space in its place
            gap = True
        pos = m.end()
    if pos < len(text):
        out.append((" " if gap and out else "") + text[pos:])
    return "".join(out)


def kernel_source_hash():
    """sha256 over the HIP sources' code (comments and layout ignored); a profiled
    byte count is valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".h", ".hip")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
                h.update(_code_tokens(fh.read()).encode())
    return h.hexdigest()


def profiled_traffic(workload):
    """HBM bytes per attention call from the committed PMC summary, if still current."""
    try:
        with open(os.path.join(PROFILES, "traffic.json")) as f:
            entry = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not entry or entry.get("source_sha256") != kernel_source_hash():
        return None
    return entry.get("bytes_per_call")


def calibrate_copy():
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_each_way": n, "copies": 3}))


PCIE_PEAK_GBPS = 64.0  # PCIe 5.0 x16, per direction


def swap_bench(args):
    """kv_swap at the decode layer's block geometry (8 kv heads x 16 x 128, fp16:
    64 KiB of K+V per block): 4096 scattered blocks (256 MiB) out of a 1 GiB
    device pool into a pinned host pool and back in to other device blocks, one
    launch per direction.  Beside it, one contiguous DMA copy of the same bytes
    each way (torch copy_ into / out of pinned memory), and the same kernel
    between two device pools."""
    import numpy as np
    import torch

    import paged_kv_cache_455_amd as pa
    nb, nh, n, hkv, d = 16384, 8192, 4096, 8, 128
    rng = np.random.default_rng(0)
    shape = lambda m: (m, hkv, 16, d)
    dk = torch.randn(shape(nb), dtype=torch.float16, device="cuda")
    dv = torch.randn(shape(nb), dtype=torch.float16, device="cuda")
    hk = torch.empty(shape(nh), dtype=torch.float16, pin_memory=True)
    hv = torch.empty(shape(nh), dtype=torch.float16, pin_memory=True)
    dev, host = pa.KVPool(dk, dv), pa.KVPool(hk, hv)
    dk2, dv2 = torch.empty_like(dk), torch.empty_like(dv)
    dev2 = pa.KVPool(dk2, dv2)
    blocks = rng.choice(nb, 2 * n, replace=False)   # swap-ins land on other blocks
    src, dst = blocks[:n], blocks[n:]
    slots = rng.choice(nh, n, replace=False)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    out_pairs = to_dev(np.stack([src, slots], 1))
    in_pairs = to_dev(np.stack([slots, dst], 1))
    dd_pairs = to_dev(np.stack([src, dst], 1))
    nbytes = n * 2 * hkv * 16 * d * 2
    flat_d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    flat_h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    stream = torch.cuda.current_stream()
    reps = max(1, args.steps)

    def timed(fn):
        for _ in range(max(1, min(args.warmup, 10))):  # PCIe-bound: a few suffice
            fn()
        torch.cuda.synchronize()
        t0, t1 = TimingEvent(), TimingEvent()
        t0.record(stream)
        for _ in range(reps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / reps
        return {"us": round(ms * 1e3, 1), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2)}

    r_out = timed(lambda: pa.kv_swap(host, dev, out_pairs, stream=stream))
    r_in = timed(lambda: pa.kv_swap(dev, host, in_pairs, stream=stream))
    r_dd = timed(lambda: pa.kv_swap(dev2, dev, dd_pairs, stream=stream))
    r_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True))
    r_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True))
    # the round trip lands the same rows in the destination blocks
    torch.cuda.synchronize()
    ok = bool(torch.equal(dk[torch.from_numpy(src).cuda()], dk[torch.from_numpy(dst).cuda()]))
    print(json.dumps({
        "metric": "kv_swap GB/s, device pool <-> pinned host pool over PCIe",
        "value": round(min(r_out["GBps"], r_in["GBps"]), 2), "unit": "GB/s",
        "higher_is_better": True, "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "kv swap, 4096 scattered blocks of 8x16x128 fp16 K+V (256 MiB)",
                   "device_blocks": nb, "host_blocks": nh},
        "swap_out": r_out, "swap_in": r_in, "device_to_device_same_kernel": r_dd,
        "dma_contiguous_d2h": r_d2h, "dma_contiguous_h2d": r_h2d,
        "roofline": {"bound": "pcie", "achieved": round(min(r_out["GBps"], r_in["GBps"]), 2),
                     "peak": PCIE_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(min(r_out["GBps"], r_in["GBps"]) / PCIE_PEAK_GBPS, 4),
                     "traffic": None, "kernel": "kv_block_copy_kernel (kv_swap)"},
        "round_trip_rows_equal": ok,
    }), flush=True)


def graph_bench(args):
    """The decode step (slot mapping -> K/V write -> decode + merge) of a decode
    workload: the fused call launched directly against the captured HIP graph of
    it replayed on the same buffers (and, for reference, the separate calls).
    All are timed with HIP events over K back-to-back steps on one stream."""
    import torch

    import paged_kv_cache_455_amd as pa
    b = make_batch(args.workload, args.block_size)
    if b.kind != "decode" or b.k_new is None:
        print("--graph takes a decode workload", file=sys.stderr)
        sys.exit(2)
    to = lambda t: None if t is None else t.cuda().contiguous()
    k, v, ks, vs = to(b.k_pool), to(b.v_pool), to(b.k_scale), to(b.v_scale)
    pool = pa.KVPool(k, v, ks, vs, shared_blocks=b.shares_blocks)
    q, kn, vn, bt, lens = to(b.q), to(b.k_new), to(b.v_new), to(b.block_tables), to(b.seq_lens)
    qsl = torch.arange(b.num_seqs + 1, dtype=torch.int32, device="cuda")
    slots = torch.empty(b.num_seqs, dtype=torch.int64, device="cuda")
    out = torch.empty_like(q)
    need = pa.pa_decode_workspace_size(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                       b.max_seq_len)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    write = pa.kv_cache_write_quant if b.kv_dtype in ("fp8", "i8") else pa.kv_cache_write
    stream = torch.cuda.current_stream()

    def separate():
        pa.pa_slot_mapping(bt, qsl, lens, b.num_seqs, out=slots, block_size=b.block_size,
                           stream=stream)
        write(pool, kn, vn, slots, stream=stream)
        pa.pa_decode(pool, q, bt, lens, b.max_seq_len, b.scale, out=out, workspace=ws,
                     stream=stream)

    def eager():  # the calls the graph holds (pa_decode_append), launched directly
        pa.pa_decode_append(pool, q, kn, vn, bt, lens, b.max_seq_len, b.scale, out=out,
                            slot_mapping=slots, workspace=ws, stream=stream)

    g = pa.DecodeStepGraph(pool, q, kn, vn, bt, lens, b.max_seq_len, b.scale)

    def timed(fn):
        for _ in range(max(1, args.warmup)):
            fn()
        torch.cuda.synchronize()
        t0, t1 = TimingEvent(), TimingEvent()
        t0.record(stream)
        for _ in range(args.steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps * 1e3

    us_separate = timed(separate)
    us_eager = timed(eager)
    us_graph = timed(lambda: g.replay(stream=stream))
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16) if out.element_size() == 2 else out,
                            g.out.view(torch.int16) if out.element_size() == 2 else g.out))
    print(json.dumps({
        "metric": "decode step time, eager vs replayed HIP graph",
        "value": round(us_graph, 2), "unit": "us/step", "higher_is_better": False,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": b.kv_dtype,
        "data": "synthetic",
        "config": {"workload": b.name, "block_size": b.block_size, "num_seqs": b.num_seqs},
        "eager_us_per_step": round(us_eager, 2), "graph_us_per_step": round(us_graph, 2),
        "separate_calls_us_per_step": round(us_separate, 2),
        "speedup": round(us_eager / us_graph, 3), "outputs_equal": same,
    }), flush=True)


STREAM_READ_BYTES = 1 << 32  # 4 GiB: far past the 256 MB Infinity Cache


def hbm_read_reference(stream, passes=10):
    """Achievable HBM read rate in this run: pa_stream_read (16-byte nontemporal
    loads, grid-stride) over a 4 GiB buffer, timed with HIP events."""
    import torch

    import paged_kv_cache_455_amd as pa
    buf = torch.empty(STREAM_READ_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.pa_stream_read(buf, sink, stream=stream)
    torch.cuda.synchronize()
    t0, t1 = TimingEvent(), TimingEvent()
    t0.record(stream)
    for _ in range(passes):
        pa.pa_stream_read(buf, sink, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / passes
    del buf
    return {"GBps": round(STREAM_READ_BYTES / (ms * 1e-3) / 1e9, 1), "bytes": STREAM_READ_BYTES,
            "passes": passes, "us_per_pass": round(ms * 1e3, 1),
            "kernel": "pa_stream_read (one read of a 4 GiB buffer, 16-byte nontemporal loads)"}


def cpu_baseline(b, budget_s):
    """The oracle as it stands, timed on this host over a bounded sample of the batch."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    from tests.pa_testlib import np_of, oracle_pools

    kp, vp, kw = oracle_pools(b)
    q = np_of(b.q).astype(np.float64)
    bt = b.block_tables.numpy()
    lens = b.seq_lens.numpy()
    qsl = b.query_start_loc.numpy()
    done, t0 = [], time.perf_counter()
    s = 0
    while time.perf_counter() - t0 < budget_s:
        i = s % b.num_seqs
        a, e = int(qsl[i]), int(qsl[i + 1])
        if b.kind == "decode":
            oracle.decode(q[i:i + 1], kp, vp, bt[i:i + 1], lens[i:i + 1], b.scale, **kw)
        else:
            oracle.prefill_chunk(q[a:e], kp, vp, np.array([0, e - a]), lens[i:i + 1], bt[i:i + 1],
                                 b.scale, **kw)
        done.append(i)
        s += 1
    dt = time.perf_counter() - t0
    nbytes = attention_bytes(b, done)
    uniq = len(set(done))
    return {
        "value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle over {len(done)} sequence passes ({uniq} distinct of "
                   f"{b.num_seqs}) of the same batch in {dt:.1f} s; attention only; "
                   f"tokens/s {len(done) / dt:.2f}"),
        "cpu_model": _cpu_model(), "host_cores": len(os.sched_getaffinity(0)),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


# ---------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the paged-attention path here is a single-GPU build)", file=sys.stderr)
        sys.exit(2)
    import torch

    import paged_kv_cache_455_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.swap:
        swap_bench(args)
        return
    if args.graph:
        graph_bench(args)
        return
    pa.load_library()
    dev = torch.device("cuda:0")
    b = make_batch(args.workload, args.block_size)
    to = lambda t: None if t is None else t.to(dev).contiguous()
    q, bt, lens, qsl = to(b.q), to(b.block_tables), to(b.seq_lens), to(b.query_start_loc)
    k_new, v_new, pairs = to(b.k_new), to(b.v_new), to(b.copy_pairs)
    R = max(1, args.rotate)
    shared = b.shares_blocks
    pools = []
    k0, v0 = to(b.k_pool), to(b.v_pool)
    ks0, vs0 = to(b.k_scale), to(b.v_scale)
    for r in range(R):
        k = k0 if r == 0 else k0.clone()
        v = v0 if r == 0 else v0.clone()
        ks = ks0 if (r == 0 or ks0 is None) else ks0.clone()
        vs = vs0 if (r == 0 or vs0 is None) else vs0.clone()
        pools.append(pa.KVPool(k, v, ks, vs, shared_blocks=shared))
    out = torch.empty_like(q)
    slots = torch.empty(b.num_tokens, dtype=torch.int64, device=dev)
    if b.kind == "decode":
        ws_bytes = pa.pa_decode_workspace_size(b.num_seqs, b.num_q_heads, b.num_kv_heads,
                                               b.head_dim, b.max_seq_len)
    else:
        ws_bytes = pa.pa_prefill_workspace_size(b.num_seqs, b.num_tokens, b.num_q_heads,
                                                b.num_kv_heads, b.head_dim, b.max_query_len,
                                                b.max_seq_len, pools[0].k.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    quantised = b.k_scale is not None
    # decode steps write the new rows inside the decode call (1-byte pools quantise
    # them there, in a launch of their own)
    fused = b.kind == "decode" and k_new is not None and not args.unfused

    def step(i, ev=None, warm=False):
        pool = pools[0] if warm else pools[i % R]
        if pairs is not None:
            pa.kv_block_copy(pool, pairs)
        if fused:
            if ev is not None:
                ev[0].record(stream)
            pa.pa_decode_append(pool, q, k_new, v_new, bt, lens, b.max_seq_len, b.scale, out=out,
                                slot_mapping=slots, workspace=ws)
            if ev is not None:
                ev[1].record(stream)
            return
        pa.pa_slot_mapping(bt, qsl, lens, b.num_tokens, out=slots, block_size=b.block_size)
        if k_new is not None:
            if quantised:  # 1-byte pool: quantise this step's K/V on the way in
                pa.kv_cache_write_quant(pool, k_new, v_new, slots)
            else:
                pa.kv_cache_write(pool, k_new, v_new, slots)
        if ev is not None:
            ev[0].record(stream)
        if b.kind == "decode":
            pa.pa_decode(pool, q, bt, lens, b.max_seq_len, b.scale, out=out, workspace=ws)
        else:
            pa.pa_prefill_chunk(pool, q, qsl, lens, bt, b.max_query_len, b.max_seq_len, b.scale,
                                out=out, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    t_warm = time.perf_counter()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    extra_warm = 0
    while (time.perf_counter() - t_warm) * 1e3 < args.min_warm_ms:
        for _ in range(10):
            step(args.warmup + extra_warm)
            extra_warm += 1
        torch.cuda.synchronize()
    # A step that is the timed call alone (fused decode, no copies) is bracketed once
    # around all K steps: an event record between launches still costs GPU time.
    # Otherwise each step's timed call gets its own pair.
    whole = fused and pairs is None and not args.per_step_events
    evs = [(TimingEvent(), TimingEvent()) for _ in range(1 if whole else args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if whole:
        evs[0][0].record(stream)
    for i in range(args.steps):
        step(i, None if whole else evs[i])
    if whole:
        evs[0][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if whole:
        attn_ms = [evs[0][0].elapsed_time(evs[0][1]) / args.steps]
    else:
        attn_ms = [a.elapsed_time(e) for a, e in evs]
    attn_ms_avg = sum(attn_ms) / len(attn_ms)
    attn_ms_sorted = sorted(attn_ms)
    ms_per_step = wall * 1e3 / args.steps
    spread = None
    if whole:
        # The spread over steps, from a second pass with an event pair around each
        # call: each pair adds its records' GPU time, so these percentiles sit a
        # little above the bracketed average, which stays the reported figure.
        pev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
        for i in range(args.steps):
            step(i, pev[i])
        torch.cuda.synchronize()
        ps = sorted(a.elapsed_time(e) for a, e in pev)
        spread = {"p10": round(ps[len(ps) // 10] * 1e3, 2), "p50": round(ps[len(ps) // 2] * 1e3, 2),
                  "p90": round(ps[(9 * len(ps)) // 10] * 1e3, 2),
                  "bracket": f"second pass: one HIP event pair around each of {args.steps} calls"}

    # Warm figure: the same steps on one pool copy, so the Infinity Cache and the
    # L2s may still hold the previous step's K/V; reported beside the rotated
    # figure, never as it.
    wev = [(TimingEvent(), TimingEvent()) for _ in range(1 if whole else args.steps)]
    for i in range(10):
        step(i, warm=True)
    torch.cuda.synchronize()
    if whole:
        wev[0][0].record(stream)
    for i in range(args.steps):
        step(i, None if whole else wev[i], warm=True)
    if whole:
        wev[0][1].record(stream)
    torch.cuda.synchronize()
    warm_ms = ([wev[0][0].elapsed_time(wev[0][1]) / args.steps] if whole else
               [a.elapsed_time(e) for a, e in wev])
    warm_us = round(sum(warm_ms) / len(warm_ms) * 1e3, 2)

    a_bytes = attention_bytes(b)
    s_bytes = side_bytes(b)
    flops = attention_flops(b)
    step_gbps = (a_bytes + s_bytes) / (ms_per_step * 1e-3) / 1e9
    # the timed call: the attention, plus (fused) the new rows' read, store and slots
    call_bytes = a_bytes + (b.num_tokens * 8 + 2 * b.num_tokens * b.num_kv_heads * b.head_dim *
                            (b.k_new.element_size() + ELEM[b.kv_dtype]) if fused else 0)
    attn_gbps = call_bytes / (attn_ms_avg * 1e-3) / 1e9
    tokens = b.num_seqs if b.kind == "decode" else b.num_tokens
    rec = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "extra_warm_steps": extra_warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.kv_dtype,
        "data": "synthetic (seeded N(0,1) draws; no dataset or weights)",
        "config": {
            "workload": b.name, "num_seqs": b.num_seqs, "num_q_tokens": b.num_tokens,
            "q_heads": b.num_q_heads, "kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
            "block_size": b.block_size, "kv_dtype": b.kv_dtype, "q_dtype": b.q_dtype, "accumulate": "f32",
            "max_context": b.max_seq_len, "pool_copies_rotated": R,
        },
        "tokens_per_s": round(tokens / (ms_per_step * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * step_gbps / HBM_PEAK_GBPS, 2),
        "attention_us": ({"avg": round(attn_ms_avg * 1e3, 2),
                          "bracket": f"one HIP event pair around all {args.steps} back-to-back calls",
                          "per_call": spread}
                         if whole else
                         {"avg": round(attn_ms_avg * 1e3, 2),
                          "p10": round(attn_ms_sorted[len(attn_ms) // 10] * 1e3, 2),
                          "p50": round(attn_ms_sorted[len(attn_ms) // 2] * 1e3, 2),
                          "p90": round(attn_ms_sorted[(9 * len(attn_ms)) // 10] * 1e3, 2),
                          "bracket": "one HIP event pair around each step's timed call"}),
        "algorithmic": {"attention_bytes": a_bytes, "side_bytes": s_bytes, "timed_call_bytes": call_bytes,
                        "attention_flops": flops},
        "roofline": {"bound": "hbm", "achieved": round(attn_gbps, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": (profiled_traffic(args.workload + ("-unfused" if args.unfused else ""))
                                 if b.block_size == 16 else None),
                     "kernel": ("pa_decode_append (balanced-split kernel + piece merge storing the "
                                "new rows)" if fused else
                                "pa_decode (balanced-split kernel + piece merge)" if b.kind == "decode"
                                else "pa_prefill_chunk")},
        "fused_append": fused,
        "warm_us": {"avg": warm_us, "note": "timed call on one pool copy (no rotation): caches may "
                    "hold the previous step's K/V; not the reported value"},
    }
    if b.kind != "decode":
        rec["attention_tflops"] = round(flops / (attn_ms_avg * 1e-3) / 1e12, 2)
    del pools, k0, v0
    torch.cuda.synchronize()
    ref = hbm_read_reference(stream)
    rec["hbm_read_reference"] = ref
    # the timed call's rate against the read rate measured beside it
    rec["pct_measured_peak"] = round(100.0 * attn_gbps / ref["GBps"], 2)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(b, args.cpu_budget_s)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
