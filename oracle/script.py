"""Execute a `workloads` script on the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see akv_oracle's header).  Every operation is the
oracle's own; this file only walks the script and records what the tests
compare: the page-table image of every segment list, the per-token positions,
and the attention outputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

import workloads as W
from . import akv_oracle as AO
from .akv_oracle import Pool


@dataclass
class OracleRun:
    pool: Pool
    attention: List[dict] = field(default_factory=list)   # one record per Attention op
    splice_positions: List[np.ndarray] = field(default_factory=list)


def _f64(u):
    return None if u is None else W.bf16_to_f64(u)


def apply_op(pool: Pool, op) -> Optional[np.ndarray]:
    if isinstance(op, W.SeqCreate):
        pool.seq_create()
    elif isinstance(op, W.Append):
        pool.append(op.seq, op.pos, _f64(op.k), _f64(op.kpe), _f64(op.v))
    elif isinstance(op, W.AppendBatch):
        # the same as one append per entry, in entry order
        off = 0
        for s, n in zip(op.seqs, op.counts):
            sl = slice(off, off + int(n))
            pool.append(int(s), op.pos[sl], _f64(op.k[sl]), _f64(op.kpe[sl]) if op.kpe is not None else None,
                        _f64(op.v[sl]))
            off += int(n)
    elif isinstance(op, W.Drop):
        pool.drop(op.seq, op.spans)
    elif isinstance(op, W.Repos):
        # a deferred repos means the same positions and the same attention;
        # only where the device rotates the keys differs
        pool.repos(op.seq, op.spans, op.deltas)
    elif isinstance(op, W.Splice):
        return pool.splice(op.seq, op.spans, op.stub_lens, _f64(op.k), _f64(op.kpe), _f64(op.v))
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
        # the same as one repos per entry, in entry order
        for seq, spans, deltas in op.entries():
            pool.repos(int(seq), spans, deltas)
    elif isinstance(op, W.CompactMode):
        pool.compaction_mode(op.deferred)
    elif isinstance(op, W.CompactPending):
        return pool.compact_pending(op.max_tokens, op.max_seqs)
    elif isinstance(op, W.Release):
        pool.seq_release(op.seq)
    else:
        raise TypeError(op)
    return None


def segment_lists(pool: Pool, segments, with_lags: bool = False):
    """Concatenated extents and (q_begin, q_len, ext_begin, ext_len) rows
    (and, with_lags, every list entry's owed rotation)."""
    exts, rows, lags, eb = [], [], [], 0
    for sg in segments:
        m = sg.mask_spans if len(sg.mask_spans) else None
        ex = pool.extents(sg.seq, m)
        exts.append(ex)
        lags.append(pool.visible_lag(sg.seq, m))
        rows.append((sg.q_begin, sg.q_len, eb, len(ex)))
        eb += len(ex)
    ex = np.concatenate(exts) if exts else np.zeros((0, 3), np.int64)
    if with_lags:
        return ex, rows, (np.concatenate(lags) if lags else np.zeros(0, np.int64))
    return ex, rows


def run_workload(wl: W.Workload, keep_log: bool = False, attention: bool = True,
        sample_rows: Optional[Dict[int, np.ndarray]] = None, stop_before_attention: bool = False,
        key_store: str = "fp64", materialize_at: Optional[Callable[[W.Attention], bool]] = None) -> OracleRun:
    """materialize_at(op) True: every segment's sequence is materialized
    before that attention (the launch that rotates owed keys in place first)."""
    pool = Pool(wl.layout, wl.page_order, keep_log=keep_log, key_store=key_store)
    res = OracleRun(pool)
    for op in wl.ops:
        if isinstance(op, W.Attention):
            if stop_before_attention:
                break
            if materialize_at is not None and materialize_at(op):
                for sg in op.segments:
                    pool.materialize(sg.seq)
            ex, rows, lags = segment_lists(pool, op.segments, with_lags=True)
            rec = dict(extents=ex, segments=rows)
            if attention:
                rec["out"] = AO.segment_attention(pool, W.bf16_to_f64(op.q), rows, ex, op.scale, rows=sample_rows,
                                                  lags=lags)
            res.attention.append(rec)
        else:
            sp = apply_op(pool, op)
            if sp is not None:
                res.splice_positions.append(sp)
    return res
