"""Benchmark of the AKV hot path on one MI355X: the 64K-token agent trace
(Llama-3.1-8B-shaped layer: 32 q heads / 8 kv heads, head_dim 128, page 16).

One step = one pass of the whole path over a cached 64K-token history:
drop the 32 older tool responses (page-table compaction, compaction check),
repos the 32 surviving runs by their cumulative deltas (one rotation launch),
append the 2,048 new tokens, build the four segments' page lists, and run
segment-batch attention for the 2,048 queries in one launch.  Every step works
on its own copy of the history (appended before timing), so nothing is
reused or undone between steps and each step starts from cold HBM data.

Prints one JSON line.  Kernel durations come from HIP events the library
records on the pool's stream around each of its launches.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PRELUDE_STEPS = 12          # untimed steps before the timed ones (warm-up included)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# HBM byte counters per dispatch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE,
# KiB) of each kernel as built from the source file with the given SHA-1, on
# the 64K step.  A plain 1 GiB device copy reads FETCH_SIZE = 524,302 KiB and
# WRITE_SIZE = 1,048,576 KiB, so fetched KiB are scaled by 2.0 and written KiB
# by 1.0.  When the kernel's source differs, its traffic is reported as null.
_ATTN_SHA1 = "4883d2cf4f9938a8863e15488837c3e251c40763"       # akv_attn_dl.hip
_KERNELS_SHA1 = "28cf8d7a53eb19500e6149ba20c49866ca3a66b4"    # akv_kernels.hip
_COPY_SHA1 = "e0150158ee0d1c27d58bdf5f6e0337b98da28d4d"       # akv_copy.hip
_DECODE_SHA1 = "f1365b8a3e8adaa58c6f7eaa0af19166e1d18e45"     # akv_decode.hip
COUNTERS = {
    "fetch_scale": 1048576 / 524302, "write_scale": 1.0,
    "attention": {"source": "akv_attn_dl.hip", "sha1": _ATTN_SHA1, "fetch_kib": 112697, "write_kib": 17408},
    "rotate": {"source": "akv_kernels.hip", "sha1": _KERNELS_SHA1, "fetch_kib": 39275, "write_kib": 77627},
    "rotate_32_layers": {"source": "akv_kernels.hip", "sha1": _KERNELS_SHA1, "fetch_kib": 1248979,
                         "write_kib": 2484443},
    "compact": {"source": "akv_copy.hip", "sha1": _COPY_SHA1, "fetch_kib": 85360, "write_kib": 165591},
    # the decode steps of 48 requests (seed 0, mean over 8 steps), k_decode_attn<false>
    "decode": {"source": "akv_decode.hip", "sha1": _DECODE_SHA1, "fetch_kib": 611701, "write_kib": 3625},
    # the retrigger clone (seed 0), k_move_tokens with the rotation
    "clone": {"source": "akv_copy.hip", "sha1": _COPY_SHA1, "fetch_kib": 80743, "write_kib": 157375},
}


def counted_traffic(kind: str):
    import hashlib
    c = COUNTERS[kind]
    src = os.path.join(ROOT, "kv_cache_drop_amd", "csrc", c["source"])
    with open(src, "rb") as f:
        if hashlib.sha1(f.read()).hexdigest() != c["sha1"]:
            return None
    return round((c["fetch_kib"] * COUNTERS["fetch_scale"] + c["write_kib"] * COUNTERS["write_scale"]) * 1024)


def attention_kernel_name(layout, max_rows=None) -> str:
    """The attention kernel the library launches for this layout (max_rows:
    the largest q_len x q heads per kv head over the launch's segments)."""
    if layout.d_nope == 0 and layout.d_rope == 128 and layout.d_v == 128 and max_rows is not None and \
            max_rows <= 16:
        return "k_decode_attn"
    if layout.d_nope == 0 and layout.d_rope == 128 and layout.d_v == 128:
        return "k_seg_attn_dl<128,128,0,8,1,4,false>"
    return "k_seg_attn"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(layout, segments, page_lists) -> tuple:
    """2 * Hq * (d_qk + d_v) per visible (query, key) pair of the bottom-right
    causal mask, and the number of such pairs."""
    ex = np.asarray(page_lists).reshape(-1, 3)
    pairs = 0
    for qb, lq, eb, el in np.asarray(segments).reshape(-1, 4).tolist():   # Python ints: no int32 wrap
        if lq == 0:
            continue
        lkv = int((ex[eb:eb + el, 2] - ex[eb:eb + el, 1]).sum())
        pairs += lq * (lkv - lq) + lq * (lq + 1) // 2
    d_qk = layout.d_nope + layout.d_rope
    return 2.0 * layout.n_q_heads * (d_qk + layout.d_v) * pairs, pairs


_CPU_JOB = {}


def _cpu_item(task):
    """One (segment, kv head) item of the oracle's attention, in a worker."""
    from threadpoolctl import threadpool_limits
    from oracle import akv_oracle as AO
    j = _CPU_JOB
    si, g = task
    G = j["pool"].L.n_q_heads // j["pool"].L.n_kv_heads
    qb, ql, _, _ = j["rows"][si]
    only = {i: np.zeros(0, np.int64) for i in range(len(j["rows"])) if i != si}   # the other segments: no rows
    with threadpool_limits(1):
        out = AO.segment_attention(j["pool"], j["q"], j["rows"], j["ex"], 0.0, rows=only,
                                   heads=range(g * G, (g + 1) * G))
    return si, g, out[qb:qb + ql, g * G:(g + 1) * G]


def host_cpu():
    """CPU model and the cores this process may use (at most 16: the host
    share that goes with one GPU)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return model, max(1, min(16, n))


def cpu_baseline(wl):
    """The fp64 oracle as it is, on the host cores, over the whole 64K step:
    drop, repos, append and page lists in this process, then segment-batch
    attention for all 2,048 queries split into (segment, kv head) items over
    worker processes, each with one BLAS thread.  Must run before this
    process touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    import oracle
    from oracle import akv_oracle as AO
    import workloads as W
    model, cores = host_cpu()
    pool = AO.Pool(wl.layout, wl.page_order)
    ops = list(wl.ops)
    i_drop = next(i for i, o in enumerate(ops) if isinstance(o, W.Drop))
    for op in ops[:i_drop]:
        oracle.apply_op(pool, op)
    att = ops[-1]
    t0 = time.perf_counter()
    t_repos, n_repos = 0.0, 0
    for op in ops[i_drop:-1]:
        if isinstance(op, W.Repos):
            n_repos += int(np.count_nonzero(pool.repos_deltas(op.seq, op.spans, op.deltas)))
            t1 = time.perf_counter()
            oracle.apply_op(pool, op)
            t_repos += time.perf_counter() - t1
        else:
            oracle.apply_op(pool, op)
    ex, rows = oracle.segment_lists(pool, att.segments)
    t_ops = time.perf_counter() - t0
    L = wl.layout
    repos_bytes = 2.0 * L.n_rope_heads * L.d_rope * 2 * n_repos      # the bf16 bytes the device rotation moves
    q = W.bf16_to_f64(att.q)
    _CPU_JOB.update(pool=pool, q=q, rows=rows, ex=ex)
    tasks = [(si, g) for si in range(len(rows)) for g in range(wl.layout.n_kv_heads)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as workers:
        done = workers.map(_cpu_item, tasks, chunksize=1)
    t_att = time.perf_counter() - t0
    _CPU_JOB.clear()
    assert len(done) == len(tasks) and all(np.isfinite(o).all() for _, _, o in done)
    flops, _ = attention_flops(wl.layout, rows, ex)
    t_step = t_ops + t_att
    n_q = int(att.q.shape[0])
    return dict(value=round(flops / t_step / 1e12, 6), unit="TFLOP/s", cores=int(cores), kind="oracle",
                cpu=model, ms_per_step=round(t_step * 1e3, 1),
                query_tokens_per_s=round(n_q / t_step, 1),
                repos_ms=round(t_repos * 1e3, 1), repos_gbps_equiv=round(repos_bytes / max(t_repos, 1e-9) / 1e9, 3),
                sample=(f"the whole 64K step once: drop / repos / append / page lists in one process "
                        f"({t_ops:.1f} s), attention for all {n_q} query rows as {len(tasks)} "
                        f"(segment, kv head) items over {cores} worker processes with one BLAS thread each "
                        f"({t_att:.1f} s)"))


def hbm_reference() -> dict:
    """Streaming rates of the chip for the access kinds of the HBM-bound
    kernels, measured with torch's own elementwise kernels on contiguous
    4 GiB buffers (well past the 256 MB Infinity Cache): an in-place
    read-modify-write (x *= 1, what repos does to its keys) and a copy
    (what compaction and clones do).  A reference for the roofline
    fractions, not part of the path."""
    import torch
    n = 4 << 30
    x = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty_like(x)
    out = {}
    for name, fn, nbytes in (("rmw_in_place", lambda: x.mul_(1.0), 2 * n),
                             ("copy", lambda: y.copy_(x), 2 * n)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = float(np.median(ms))
        out[name] = {"bytes": nbytes, "ms": round(t, 4), "GB/s": round(nbytes / (t * 1e-3) / 1e9, 1),
                     "frac_of_8TBps": round(nbytes / (t * 1e-3) / 8e12, 4)}
    return {"hbm_reference": out, "note": "torch elementwise kernels on contiguous 4 GiB bf16 buffers"}


def mfma_reference() -> dict:
    """The chip's dense bf16 rate through the vendor GEMM library (torch.matmul
    of contiguous square bf16 matrices, fp32 accumulation, on hipBLASLt or
    rocBLAS): a reference for the attention kernel's roofline fraction, not
    part of the path.  Median of 5 timed products after 3 warm-ups."""
    import torch
    out = {}
    for n in (4096, 8192, 16384):
        g = torch.Generator(device="cuda:0").manual_seed(n)
        a = torch.randn(n, n, device="cuda:0", generator=g).to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda:0", generator=g).to(torch.bfloat16)
        for _ in range(3):
            c = torch.matmul(a, b)
        torch.cuda.synchronize()
        ms = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            c = torch.matmul(a, b)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = float(np.median(ms))
        flop = 2.0 * n ** 3
        out[f"gemm_{n}"] = {"flop": flop, "ms": round(t, 4), "TFLOP/s": round(flop / (t * 1e-3) / 1e12, 1),
                            "frac_of_2.5PFLOPs": round(flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del a, b, c
    return {"mfma_reference": out, "note": "torch.matmul, contiguous square bf16 operands, fp32 accumulation"}


def compact_extra(pool, seqs, L) -> dict:
    """Extra line: forced compaction (k_move_tokens) of C2 sequences after their
    step, each the only work on its copy since that step (the earliest timed
    copies first, so their pages are long out of every cache)."""
    import torch
    pool.timing_read("compact")
    moved = 0
    for s in seqs:
        moved += pool.info(s)[1]
        pool.compact(s, True)
    torch.cuda.synchronize()
    ms, n = pool.timing_read("compact")
    avg = ms / max(n, 1)
    per_tok = 2 * L.n_kv_heads * (L.d_nope + L.d_rope + L.d_v) * 2     # read + write of K and V
    nbytes = per_tok * moved / max(len(seqs), 1)
    gbps = nbytes / (avg * 1e-3) / 1e9
    return {"extra": True, "what": "forced compaction of the 64K sequence after its step (visible history "
                                   "+ new tokens into fresh pages)",
            "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": counted_traffic("compact"), "kernel": "k_move_tokens",
            "tokens_per_launch": moved / max(len(seqs), 1), "bytes_per_launch": nbytes,
            "avg_launch_ms": round(avg, 5), "launches": n}


def repos_layers_extra(args, L, hist, drop, repos, hk, hv, rep_bytes) -> dict:
    """Extra line (not the headline config): the C2 repos over a model's
    layers in one launch (akv_repos_layers), one pool per layer with the same
    history and drop; alternating +delta / -delta keeps every rep on the same
    data, and 32 layers of rotated keys (5 GB) do not fit any cache."""
    import torch
    import kv_cache_drop_amd as akv
    nl = args.repos_layers
    rng = np.random.default_rng(args.seed + 2)
    order = rng.permutation(L.num_pages).astype(np.int32)
    log(f"[bench] building {nl} layer pools for the batched repos line")
    pools = []
    for _ in range(nl):
        p = akv.Pool(L.n_q_heads, L.n_kv_heads, 0, L.d_rope, L.d_v, L.page_size, L.num_pages,
                     rope_theta=L.rope_theta, page_order=order, scratch_bytes=16 << 20)
        s = p.seq_create()
        p.append(s, hist.pos, hk, None, hv)
        p.drop(s, drop.spans)
        pools.append(p)
    torch.cuda.synchronize()
    neg = -np.asarray(repos.deltas, np.int32)
    for r in range(2):
        akv.repos_layers(pools, 0, repos.spans, repos.deltas if r % 2 == 0 else neg)
    torch.cuda.synchronize()
    pools[0].timing_enable(True)
    pools[0].timing_read("rotate")
    reps = 10
    for r in range(reps):
        akv.repos_layers(pools, 0, repos.spans, repos.deltas if r % 2 == 0 else neg)
    torch.cuda.synchronize()
    ms, n = pools[0].timing_read("rotate")
    pools[0].timing_enable(False)
    for p in pools:
        p.close()
    del pools
    torch.cuda.empty_cache()
    avg = ms / max(n, 1)
    nbytes = rep_bytes * nl
    gbps = nbytes / (avg * 1e-3) / 1e9
    return {"extra": True, "what": f"C2 repos over {nl} layers in one launch (akv_repos_layers)",
            "bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_HBM_GBPS, 4),
            "traffic": counted_traffic("rotate_32_layers") if nl == 32 else None, "kernel": "k_rotate", "layers": nl,
            "bytes_per_launch": nbytes, "avg_launch_ms": round(avg, 5), "launches": n}


def run_config(args) -> dict:
    """One JSON record for a workload other than the headline: replay its op
    script on a fresh device pool per rep (set-up untimed), flush L2 and the
    Infinity Cache by reading 1 GiB (so no dirty lines are left to write back
    inside the timed step), then time the remaining ops (drop / repos /
    splice / clone, the new tokens' append, attention) as one step."""
    import torch
    import device_script as D
    import workloads as W

    def deferred(wl):
        for op in wl.ops:
            if isinstance(op, W.Repos):
                op.deferred = True
        return wl

    gens = {"c1": lambda s: W.c1_tiny(s, "canonical"), "c3": W.c3_mla, "c4": W.c4_batched, "c5": W.c5_128k,
            "decode": W.decode_batch, "decode_fused": lambda s: W.decode_batch(s, deferred=True),
            "retrigger": W.retrigger, "c2_fused": lambda s: deferred(W.c2_64k(s)),
            "decode_compact": W.decode_with_idle, "decode_mass": W.decode_batch,
            "c2_compact": lambda s: W.with_idle_compaction(W.c2_64k(s), s, n_idle=2, idle_ctx=16384)}
    wl = gens[args.config](args.seed)
    L = wl.layout
    ops = list(wl.ops)
    # timed ops: from the first cache operation on (drop / repos / splice /
    # clone, the new tokens, attention), or from where the workload says its
    # step starts (decode: the new tokens and attention after the histories)
    i0 = wl.notes.get("step_from",
                      next(i for i, o in enumerate(ops) if not isinstance(o, (W.SeqCreate, W.Append))))
    n_seq = sum(isinstance(o, W.SeqCreate) for o in ops)
    # device inputs of the timed ops, uploaded once (outside the timed region)
    dev = {}
    for i, op in enumerate(ops[i0:], start=i0):
        if isinstance(op, (W.Append, W.AppendBatch, W.Splice)):
            dev[i] = (D.dev_bf16(op.k), D.dev_bf16(op.kpe) if op.kpe is not None else None, D.dev_bf16(op.v))
        elif isinstance(op, W.Attention):
            q = D.dev_bf16(op.q)
            # the segment descriptions, as a caller keeps them: one int array
            # when no segment hides spans
            if all(len(sg.mask_spans) == 0 for sg in op.segments):
                segs = np.array([(sg.seq, sg.q_begin, sg.q_len) for sg in op.segments], np.int32).reshape(-1, 3)
            else:
                segs = [(sg.seq, sg.q_begin, sg.q_len, sg.mask_spans if len(sg.mask_spans) else None)
                        for sg in op.segments]
            dev[i] = (q, torch.empty((q.shape[0], L.n_q_heads, L.d_v), dtype=torch.bfloat16, device="cuda:0"),
                      segs)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
    rope_heads = L.n_kv_heads if (not L.mla or L.kpe_per_head) else 1
    tot = {k: [0.0, 0] for k in ("attention", "rotate", "append", "compact", "expand", "combine", "clone", "mass")}
    walls, flops, pairs, kv_bytes, n_rot, n_q, clone_bytes = [], 0.0, 0, 0, 0, 0, 0
    idle_moved = 0
    kern = None
    n_dec = args.decode_steps if args.config in ("decode", "decode_fused", "decode_compact", "decode_mass") else 1
    first_walls = []
    # each decode step's positions and the batch's index arrays, made once
    # (int32, contiguous: the binding passes them on as they are)
    step_args = {}
    for i, op in enumerate(ops[i0:], start=i0):
        if isinstance(op, W.AppendBatch):
            rep_counts = np.repeat(op.counts, op.counts).astype(np.int32)
            step_args[i] = (np.ascontiguousarray(op.seqs, np.int32), np.ascontiguousarray(op.counts, np.int32),
                            [np.ascontiguousarray(op.pos + t * rep_counts, np.int32) for t in range(n_dec)])
    # no collector pause inside a timed step, and none right before it (the
    # idle GPU it leaves makes the next launches slower): one collection
    # before the reps, the collector off until they end
    gc.collect()
    gc.disable()
    # reps: warm-up, then args.steps reps timed by the wall clock with the
    # library's per-launch timer events off (they add two marker packets per
    # launch), then args.steps more with the timers on for kernel durations
    walls_timers = []
    for rep in range(args.warmup + 2 * args.steps):
        pool = D.make_pool(wl)
        if args.config == "c2_fused":
            pool.fused_rotation("always")     # keys turned in the attention kernel, not in place
        if args.config == "decode_mass":       # per-page attention mass of every decode launch
            mass_out = torch.zeros(L.num_pages, dtype=torch.float32, device="cuda:0")
            pool.attention_mass(mass_out)
        keep = []
        for op in ops[:i0]:
            D.apply_op(pool, op, keep)
        pre = [pool.tokens(s) for s in range(n_seq)] if rep == 0 else None
        flush_sum = flush.sum(dtype=torch.int64)   # reads 1 GiB: evicts L2 / MALL, dirties nothing
        torch.cuda.synchronize()
        timed = args.warmup <= rep < args.warmup + args.steps
        kernel_rep = rep >= args.warmup + args.steps
        pool.timing_enable(kernel_rep)
        lists = []

        def run_ops(shift):
            # shift > 0: the next decode step (each request's new tokens one
            # step further on; the same query and K/V values)
            for i, op in enumerate(ops[i0:], start=i0):
                if isinstance(op, W.Append):
                    pool.append(op.seq, op.pos, dev[i][0], dev[i][1], dev[i][2])
                elif isinstance(op, W.AppendBatch):
                    seqs, counts, pos = step_args[i]
                    pool.append_batch(seqs, counts, pos[shift], dev[i][0], dev[i][1], dev[i][2])
                elif isinstance(op, W.Splice):
                    pool.splice(op.seq, op.spans, op.stub_lens, dev[i][0], dev[i][1], dev[i][2])
                elif isinstance(op, W.Attention):
                    # lists built inside the library from the sequences' page tables
                    pool.seq_attention(dev[i][0], dev[i][2], op.scale, out=dev[i][1])
                    if shift == 0:
                        lists.append(op)
                else:
                    D.apply_op(pool, op, keep)

        t0 = time.perf_counter()
        run_ops(0)
        if n_dec > 1:
            # the first decode step rebuilds the lists after the histories'
            # drops and repos; the steps after it are the steady state
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for t in range(1, n_dec):
                run_ops(t)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if n_dec > 1:
            first = t1 - t0
            wall = (time.perf_counter() - t1) / (n_dec - 1)
        if timed:
            walls.append(wall)
            if n_dec > 1:
                first_walls.append(first)
        if kernel_rep:
            walls_timers.append(wall)
            for k in tot:
                ms, n = pool.timing_read(k)
                tot[k][0] += ms
                tot[k][1] += n
        if rep == 0:
            idle_moved = sum(pool.info(s)[1] for s in wl.notes.get("idle", []))
            for s in range(n_seq):
                _, pos0, drop0 = pre[s]
                _, pos1, drop1 = pool.tokens(s)
                m = len(pos0)
                n_rot += int(((pos1[:m] != pos0) & ~drop1[:m].astype(bool)).sum())
            for op in lists:
                rows, ex = D.segment_inputs(pool, op)     # the same lists, for the counts
                f, p = attention_flops(L, rows, ex)
                exa = np.asarray(ex).reshape(-1, 3)
                kv = int((exa[:, 2] - exa[:, 1]).sum()) * L.n_kv_heads * (L.d_nope + L.d_rope + L.d_v) * 2
                if n_dec > 1:
                    # these are the lists after the last decode step: step t
                    # attended (n_dec - 1 - t) * q_len fewer keys per segment;
                    # report the mean over the steps
                    f, p, kv = 0.0, 0, 0
                    d_qk = L.d_nope + L.d_rope
                    for t in range(n_dec):
                        for qb, lq, eb, el in np.asarray(rows).reshape(-1, 4).tolist():
                            lkv = int((exa[eb:eb + el, 2] - exa[eb:eb + el, 1]).sum()) - (n_dec - 1 - t) * lq
                            pr = lq * (lkv - lq) + lq * (lq + 1) // 2
                            p += pr
                            f += 2.0 * L.n_q_heads * (d_qk + L.d_v) * pr
                            kv += lkv * L.n_kv_heads * (d_qk + L.d_v) * 2
                    f, p, kv = f / n_dec, p // n_dec, kv // n_dec
                flops += float(f)
                pairs += int(p)
                kv_bytes += int(kv)
                n_q += int(op.q.shape[0])
            # a clone reads and writes every row of each retained source token
            row_bytes = 2 * (rope_heads * L.d_rope + L.n_kv_heads * (L.d_nope + L.d_v))
            for op in ops[i0:]:
                if isinstance(op, W.Clone):
                    dr = pool.tokens(op.src)[2][op.first:op.first + op.n]
                    clone_bytes += 2 * row_bytes * int((dr == 0).sum())
            grp = L.n_q_heads // L.n_kv_heads
            kern = attention_kernel_name(L, max(sg.q_len * grp for op in lists for sg in op.segments))
            if any(isinstance(o, W.Repos) and o.deferred for o in ops):
                kern = "k_decode_attn<rotating>" if kern == "k_decode_attn" else (
                    "k_seg_attn_dl<128,128,0,8,1,4,rotating>" if kern.startswith("k_seg_attn_dl") else kern)
        pool.close()
        del pool, keep
    gc.enable()
    ms_step = float(np.median(walls)) * 1e3
    attn_ms = tot["attention"][0] / max(tot["attention"][1], 1)
    n_launch_steps = max(args.steps, 1) * n_dec     # steps whose kernels the timers saw
    rot_ms = tot["rotate"][0] / max(tot["rotate"][1], 1) if tot["rotate"][1] else None
    rep_bytes = 2.0 * rope_heads * L.d_rope * 2 * n_rot
    # per step: one attention launch; rotate launches per step = tot count / steps
    rot_per_step = tot["rotate"][1] / n_launch_steps
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    rec = {
        "metric": "segment-batch attn TFLOP/s + repos GB/s, % of MI355X roofline",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_timers": round(float(np.median(walls_timers)) * 1e3, 4) if walls_timers else None,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": CONFIG_NAMES[args.config], "seed": args.seed, "query_tokens": n_q,
                   "repositioned_tokens": n_rot, "attention_pairs": pairs},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": kern, "flop_per_launch": flops, "kv_bytes_per_launch": kv_bytes,
                     "avg_launch_ms": round(attn_ms, 5)},
        "kernels_ms_per_step": {k: round(v[0] / n_launch_steps, 5) for k, v in tot.items()},
    }
    if n_dec > 1:
        rec["config"]["decode_steps_per_rep"] = n_dec
        rec["first_step_ms"] = round(float(np.median(first_walls)) * 1e3, 4)
        rec["note"] = (f"ms_per_step: steady decode steps 2..{n_dec} on the same pool (each appends one token "
                       "per request and attends over every list); first_step_ms: the first step after the "
                       "histories' drops and repos, which rebuilds each visible list")
    if args.config in ("decode_compact", "c2_compact") and tot["compact"][1]:
        # the background pass: every visible token of the idle sequences moves
        # (K and V rows read and written), beside the decode step
        cm_ms = tot["compact"][0] / tot["compact"][1]
        cm_per_step = tot["compact"][1] / max(args.steps, 1)    # launches per rep (one pass per rep)
        per_tok = 2 * L.n_kv_heads * (L.d_nope + L.d_rope + L.d_v) * 2
        cm_bytes = per_tok * idle_moved
        cm_gbps = cm_bytes / (cm_ms * cm_per_step * 1e-3) / 1e9
        rec["roofline_compact"] = {"bound": "hbm", "achieved": round(cm_gbps, 1), "peak": PEAK_HBM_GBPS,
                                   "unit": "GB/s", "frac": round(cm_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                                   "kernel": "k_move_tokens (background stream)", "bytes_per_step": cm_bytes,
                                   "launches_per_pass": cm_per_step, "avg_launch_ms": round(cm_ms, 5)}
        rec["note"] = ("the workload's step on the pool stream, then the background compaction pass (its copies on "
                       "the pool's second stream, beside the step's kernels)")
    if tot["mass"][1]:
        # the second pass reads every visible K row once more
        ms_m = tot["mass"][0] / tot["mass"][1]
        k_bytes = kv_bytes * (L.d_nope + L.d_rope) / (L.d_nope + L.d_rope + L.d_v)
        gbps_m = k_bytes / (ms_m * 1e-3) / 1e9
        rec["roofline_mass"] = {"bound": "hbm", "achieved": round(gbps_m, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(gbps_m / PEAK_HBM_GBPS, 4), "traffic": None, "kernel": "k_page_mass",
                                "k_bytes_per_launch": k_bytes, "avg_launch_ms": round(ms_m, 5)}
    if args.config in ("decode", "decode_fused", "decode_compact", "decode_mass"):
        # one query row per kv-head group: the launch streams the visible K/V once
        hbm_gbps = kv_bytes / (attn_ms * 1e-3) / 1e9
        rec["roofline"] = {"bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": round(hbm_gbps / PEAK_HBM_GBPS, 4),
                           "traffic": counted_traffic("decode") if args.config == "decode" and args.seed == 0
                           and kern == "k_decode_attn" else None, "kernel": kern,
                           "kv_bytes_per_launch": kv_bytes, "flop_per_launch": flops,
                           "avg_launch_ms": round(attn_ms, 5)}
    if tot["clone"][1]:
        cl_ms = tot["clone"][0] / tot["clone"][1]
        cl_per_step = tot["clone"][1] / n_launch_steps
        cl_gbps = clone_bytes / (cl_ms * cl_per_step * 1e-3) / 1e9
        rec["roofline_clone"] = {"bound": "hbm", "achieved": round(cl_gbps, 1), "peak": PEAK_HBM_GBPS,
                                 "unit": "GB/s", "frac": round(cl_gbps / PEAK_HBM_GBPS, 4),
                                 "traffic": counted_traffic("clone") if args.config == "retrigger" and args.seed == 0
                                 else None,
                                 "kernel": "k_move_tokens", "bytes_per_step": clone_bytes,
                                 "launches_per_step": cl_per_step, "avg_launch_ms": round(cl_ms, 5)}
    if rot_ms is not None:
        rot_gbps = rep_bytes / (rot_ms * rot_per_step * 1e-3) / 1e9
        rec["roofline_repos"] = {"bound": "hbm", "achieved": round(rot_gbps, 1), "peak": PEAK_HBM_GBPS,
                                 "unit": "GB/s", "frac": round(rot_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                                 "kernel": "k_rotate", "bytes_per_step": rep_bytes,
                                 "launches_per_step": rot_per_step,
                                 "avg_launch_ms": round(rot_ms, 5)}
    return rec


CONFIG_NAMES = {
    "c1": "tiny 2K-token check (8 q / 2 kv heads, head_dim 64, page 16): drop 2 spans, repos the suffix by -640, "
          "2 segments",
    "c3": "MLA 17K context (16 heads, K_nope 128 + shared K_pe 64, V 128, page 64): 1-3 splices, one 512-query "
          "segment",
    "c4": "16 batched requests of 8K-32K tokens on the 64K layer shape (32 q / 8 kv heads, head_dim 128, "
          "page 16), about 40 segments in one launch",
    "c5": "128K-token agent trace, 64 q / 8 kv heads, head_dim 128, page 16: drop 60 spans, repos 60 runs, "
          "4096 queries in 8 segments",
    "retrigger": "64K agent trace re-used at another offset (32 q / 8 kv heads, head_dim 128, page 16): request A "
                 "(512-token preamble, the 64K trace, older tools dropped, survivors repositioned) and request B "
                 "(the same trace after a preamble of another length) cloned from A's state with keys turned by "
                 "the offset change; 512 queries each in one launch",
    "c2_fused": "the 64K step (Llama-3.1-8B-shaped layer, 32 q / 8 kv heads, head_dim 128, page 16) with its repos "
                "deferred: no rotation pass; the attention kernel turns each landed key tile in LDS",
    "decode_compact": "the decode step of 48 requests of 2K-16K tokens (32 q / 8 kv heads, head_dim 128, page 16) "
                      "while 8 idle 32K-token sequences, half their tokens dropped in 8-token blocks, are compacted "
                      "by one background pass (second stream) in the same step",
    "c2_compact": "the 64K step (Llama-3.1-8B-shaped layer, 32 q / 8 kv heads, head_dim 128, page 16), then a "
                  "background compaction pass over 2 idle 16K-token sequences with half their tokens dropped in "
                  "8-token blocks, its copies on the pool's second stream beside the step's attention",
    "decode_fused": "the decode step of 48 requests of 2K-16K tokens whose survivors' repos was deferred: the "
                    "keys stay at their old positions and the decode kernel turns them as it reads them",
    "decode_mass": "the decode step of 48 requests of 2K-16K tokens (32 q / 8 kv heads, head_dim 128, page 16) "
                   "with the per-page attention mass output set (a second pass over each launch's K rows)",
    "decode": "48 requests of 2K-16K tokens on the 64K layer shape (32 q / 8 kv heads, head_dim 128, page 16), "
              "dropped and repositioned at set-up; the step appends one token per request and runs 48 one-query "
              "segments in one launch",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c2_fused", "c3", "c4", "c5", "decode", "decode_fused",
                                                       "decode_compact", "decode_mass", "c2_compact", "retrigger"],
                    help="c2 (default) is the headline 64K step; the others print one record each")
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=8, help="decode steps per rep (decode configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--repos-layers", type=int, default=32,
                    help="layers of the extra batched-repos line (0: skip it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--hbm-reference", action="store_true",
                    help="only time plain streaming kernels (torch's in-place multiply and copy over 4 GiB, "
                         "out of every cache): the chip's rates for in-place read-modify-write and copy")
    ap.add_argument("--mfma-reference", action="store_true",
                    help="only time plain bf16 GEMMs of the vendor library (torch.matmul, 4K-16K squares): "
                         "the chip's dense bf16 rate as a library reaches it")
    args = ap.parse_args()
    if args.mfma_reference:
        print(json.dumps(mfma_reference()), flush=True)
        return
    if args.hbm_reference:
        print(json.dumps(hbm_reference()), flush=True)
        return
    if args.calibrate_copy:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 1 << 30, "copies": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the path is measured on one "
              "MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.config != "c2":
        print(json.dumps(run_config(args)), flush=True)
        return

    import workloads as W

    wl = W.c2_64k(args.seed)
    cpu = None
    if not args.no_cpu_baseline:
        # before any GPU use: the oracle's workers are forked from this process
        log("[bench] timing the fp64 oracle on the host cores (the whole 64K step)")
        cpu = cpu_baseline(wl)
        log(f"[bench] oracle: {cpu['sample']}")

    import torch
    import device_script as D
    import kv_cache_drop_amd as akv

    L = wl.layout
    ops = wl.ops
    hist, drop, repos, new, att = ops[1], ops[2], ops[3], ops[4], ops[5]
    assert isinstance(drop, W.Drop) and isinstance(repos, W.Repos) and isinstance(att, W.Attention)
    # After the GPU has idled (set-up, a Python collection), the first ~10
    # steps run 10-25% slower than the later ones (measured: attention
    # launches of 1.3-1.48 ms against 1.12-1.15 ms, settling over ~30 ms of
    # load); untimed prelude steps on their own copies keep that transient
    # out of the timed steps.
    prelude = max(0, PRELUDE_STEPS - args.warmup) if args.warmup > 0 else 0
    # the timed steps run without the library's per-launch timer events (two
    # marker packets around every launch: about 35 us per step); the kernel
    # durations come from as many steps again with the timers on
    n_copies = prelude + args.warmup + 2 * args.steps
    per_copy = L.num_pages                      # 4,224 pages: history + new tokens
    rng = np.random.default_rng(args.seed + 1)
    order = rng.permutation(per_copy * n_copies).astype(np.int32)
    log(f"[bench] building {n_copies} copies of the 64K history ({per_copy * n_copies} pages)")
    pool = akv.Pool(L.n_q_heads, L.n_kv_heads, 0, L.d_rope, L.d_v, L.page_size, per_copy * n_copies,
                    rope_theta=L.rope_theta, page_order=order, scratch_bytes=256 << 20)
    hk, hv = D.dev_bf16(hist.k), D.dev_bf16(hist.v)
    nk, nv = D.dev_bf16(new.k), D.dev_bf16(new.v)
    q = D.dev_bf16(att.q)
    out = torch.empty((q.shape[0], L.n_q_heads, L.d_v), dtype=torch.bfloat16, device="cuda:0")
    seqs = []
    for c in range(n_copies):
        s = pool.seq_create()
        pool.append(s, hist.pos, hk, None, hv)
        seqs.append(s)
    torch.cuda.synchronize()

    masks = [sg.mask_spans if len(sg.mask_spans) else None for sg in att.segments]

    def step(s):
        pool.drop(s, drop.spans)
        pool.repos(s, repos.spans, repos.deltas)
        pool.append(s, new.pos, nk, None, nv)
        # the attention call reads each segment's visible list from the pool
        pool.seq_attention(q, [(s, sg.q_begin, sg.q_len, m) for sg, m in zip(att.segments, masks)], 0.0, out=out)

    def page_lists_of(s):
        exts, segs, eb = [], [], 0
        for sg, m in zip(att.segments, masks):
            ex = pool.visible(s, m)
            exts.append(ex)
            segs.append((sg.q_begin, sg.q_len, eb, len(ex)))
            eb += len(ex)
        return segs, np.concatenate(exts)

    # A collector pause (tens of ms) would land in the timed steps, and the
    # idle GPU it leaves behind restarts the slow-clock transient above: the
    # collection runs before the untimed steps.
    gc.collect()
    gc.disable()
    w0 = prelude + args.warmup
    for c in range(w0):
        step(seqs[c])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for c in range(w0, w0 + args.steps):
        step(seqs[c])
    t_host = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # kernel durations: the same steps on the next copies, timers on
    pool.timing_enable(True)
    for k in akv.KERNEL_KINDS:
        pool.timing_read(k)
    t1 = time.perf_counter()
    for c in range(w0 + args.steps, n_copies):
        step(seqs[c])
    torch.cuda.synchronize()
    wall_timers = time.perf_counter() - t1
    gc.enable()
    segs, page_lists = page_lists_of(seqs[-1])
    pct = {k: [round(float(x), 5) for x in np.percentile(pool.timing_samples(k), [10, 50, 90])]
           for k in ("attention", "rotate")}
    kt = {k: pool.timing_read(k) for k in akv.KERNEL_KINDS}

    flops, pairs = attention_flops(L, segs, page_lists)
    ex_all = np.asarray(page_lists).reshape(-1, 3)
    kv_bytes = int((ex_all[:, 2] - ex_all[:, 1]).sum()) * L.n_kv_heads * (L.d_rope + L.d_v) * 2
    n_rep = int(sum(e - b for b, e in repos.spans))
    rep_bytes = 2.0 * L.n_kv_heads * L.d_rope * 2 * n_rep      # read + write of the rotated keys
    ms_step = wall / args.steps * 1e3
    attn_ms = kt["attention"][0] / max(kt["attention"][1], 1)
    rot_ms = kt["rotate"][0] / max(kt["rotate"][1], 1)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    rot_gbps = rep_bytes / (rot_ms * 1e-3) / 1e9
    value = flops / (ms_step * 1e-3) / 1e12

    t0c = prelude + args.warmup
    comp_rec = compact_extra(pool, seqs[t0c:t0c + min(10, args.steps)], L)
    pool.timing_enable(False)
    layers_rec = None
    if args.repos_layers > 0:
        layers_rec = repos_layers_extra(args, L, hist, drop, repos, hk, hv, rep_bytes)

    rec = {
        "metric": "segment-batch attn TFLOP/s + repos GB/s at 64K ctx, % of MI355X roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prelude_steps": prelude,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_with_kernel_timers": round(wall_timers / max(args.steps, 1) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "64K-token agent trace, Llama-3.1-8B-shaped layer (32 q / 8 kv heads, "
                               "head_dim 128, page 16): drop 32 older tool spans, repos 32 runs, "
                               "segment-batch attention for 2048 queries in 4 segments",
                   "history_tokens": 65536, "visible_after_drop": int(wl.notes["history"]),
                   "repositioned_tokens": n_rep, "query_tokens": int(att.q.shape[0]), "segments": 4,
                   "seed": args.seed},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": counted_traffic("attention"),
                     "kernel": attention_kernel_name(L), "flop_per_launch": flops,
                     "kv_bytes_per_launch": kv_bytes,
                     "avg_launch_ms": round(attn_ms, 5), "launch_ms_p10_p50_p90": pct["attention"]},
        "roofline_repos": {"bound": "hbm", "achieved": round(rot_gbps, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(rot_gbps / PEAK_HBM_GBPS, 4),
                           "traffic": counted_traffic("rotate"),
                           "kernel": "k_rotate", "bytes_per_launch": rep_bytes,
                           "avg_launch_ms": round(rot_ms, 5), "launch_ms_p10_p50_p90": pct["rotate"]},
        "roofline_repos_layers": layers_rec,
        "roofline_compact": comp_rec,
        "kernels_ms_per_step": {k: round(v[0] / max(args.steps, 1), 5) for k, v in kt.items()},
        "host_ms_per_step": round(t_host / args.steps * 1e3, 4),
        "attention_pairs": int(pairs),
        "query_tokens_per_s": round(att.q.shape[0] / (ms_step * 1e-3), 1),
        "repositioned_tokens_per_s": round(n_rep / (rot_ms * 1e-3), 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    pool.close()


if __name__ == "__main__":
    main()
