"""Run a `workloads` script on the HIP path through the C ABI binding.

Only marshalling: every operation is a call of kv_cache_drop_amd.Pool (the
library's kernels and host runtime).  Used by the GPU parity tests, smoke()
and bench.py."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_drop_amd as akv
import workloads as W


def dev_bf16(u16: np.ndarray, device="cuda:0") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def make_pool(wl: W.Workload, scratch_bytes: int = 256 << 20, **kw) -> akv.Pool:
    L = wl.layout
    return akv.Pool(L.n_q_heads, L.n_kv_heads, L.d_nope, L.d_rope, L.d_v, L.page_size, L.num_pages,
                    kpe_per_head=L.kpe_per_head, pairing=L.pairing, rope_theta=L.rope_theta,
                    page_order=wl.page_order, device=True, scratch_bytes=scratch_bytes, **kw)


def segment_inputs(pool: akv.Pool, att: W.Attention):
    exts, rows, eb = [], [], 0
    for sg in att.segments:
        ex = pool.visible(sg.seq, sg.mask_spans if len(sg.mask_spans) else None)
        exts.append(ex)
        rows.append((sg.q_begin, sg.q_len, eb, len(ex)))
        eb += len(ex)
    ex = np.concatenate(exts) if exts else np.zeros((0, 3), np.int32)
    return np.asarray(rows, np.int32).reshape(-1, 4), ex


def apply_op(pool: akv.Pool, op, keep=None):
    """Apply one script op; device inputs are kept alive in `keep`."""
    keep = keep if keep is not None else []
    if isinstance(op, W.SeqCreate):
        pool.seq_create()
    elif isinstance(op, W.Append):
        k, v = dev_bf16(op.k), dev_bf16(op.v)
        kpe = dev_bf16(op.kpe) if op.kpe is not None else None
        keep += [k, v, kpe]
        pool.append(op.seq, op.pos, k, kpe, v)
    elif isinstance(op, W.AppendBatch):
        k, v = dev_bf16(op.k), dev_bf16(op.v)
        kpe = dev_bf16(op.kpe) if op.kpe is not None else None
        keep += [k, v, kpe]
        pool.append_batch(op.seqs, op.counts, op.pos, k, kpe, v)
    elif isinstance(op, W.Drop):
        pool.drop(op.seq, op.spans)
    elif isinstance(op, W.Repos):
        if op.deferred:
            pool.repos_deferred(op.seq, op.spans, op.deltas)
        else:
            pool.repos(op.seq, op.spans, op.deltas)
    elif isinstance(op, W.Splice):
        k, v = dev_bf16(op.k), dev_bf16(op.v)
        kpe = dev_bf16(op.kpe) if op.kpe is not None else None
        keep += [k, v, kpe]
        return pool.splice(op.seq, op.spans, op.stub_lens, k, kpe, v)
    elif isinstance(op, W.Compact):
        pool.compact(op.seq, bool(op.force))
    elif isinstance(op, W.Clone):
        pool.clone(op.src, op.first, op.n, op.dst, op.delta)
    elif isinstance(op, W.Freeze):
        pool.freeze(op.seq)
    elif isinstance(op, W.Share):
        pool.share(op.src, op.first, op.n, op.dst, op.delta)
    elif isinstance(op, W.Materialize):
        pool.materialize(op.seq)
    elif isinstance(op, W.ReposBatch):
        pool.repos_batch(list(op.entries()))
    elif isinstance(op, W.CompactMode):
        pool.compaction_mode(op.deferred)
    elif isinstance(op, W.CompactPending):
        return pool.compact_pending(op.max_tokens, op.max_seqs)
    elif isinstance(op, W.Release):
        pool.seq_release(op.seq)
    else:
        raise TypeError(op)
    return None


def run(wl: W.Workload, pool: akv.Pool | None = None, **kw):
    pool = pool if pool is not None else make_pool(wl, **kw)
    keep, outs = [], []
    # keys that owe a rotation (deferred repos, shared rows): attention over
    # sequence ids, which applies what each key owes
    deferred = any((isinstance(o, W.Repos) and o.deferred) or isinstance(o, W.Share) for o in wl.ops)
    for op in wl.ops:
        if isinstance(op, W.Attention):
            q = dev_bf16(op.q)
            keep.append(q)
            if deferred:   # keys owe rotations: the library applies them
                out = pool.seq_attention(q, [(sg.seq, sg.q_begin, sg.q_len,
                                              sg.mask_spans if len(sg.mask_spans) else None)
                                             for sg in op.segments], op.scale)
                # the lists the launch read (a launch that materializes first
                # can move rows of shared pages)
                rows, ex = segment_inputs(pool, op)
            else:
                rows, ex = segment_inputs(pool, op)
                out = pool.segment_attention(q, rows, ex, op.scale)
            outs.append(dict(segments=rows, extents=ex, out=out))
        else:
            apply_op(pool, op, keep)
    torch.cuda.synchronize()
    return pool, outs
