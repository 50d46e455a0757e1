"""Seeded synthetic workloads for AKV cache engineering (drop / repos / splice /
segment-batch attention).

This module is shared by both sides of every parity check: the fp64 oracle
(`oracle/`) and the HIP path (`kv_cache_drop_amd`).  It therefore holds none of
the method's arithmetic: no rotation, no attention, no visibility logic.  It
only draws seeded random numbers, lays out token spans, and encodes float32
values as bfloat16 bit patterns through torch's round-to-nearest-even cast.

Every workload is a *script*: a layout, an initial free-page order, and a list
of operations (create a sequence, append tokens, drop spans, reposition spans,
splice, compact, run segment-batch attention).  Each side executes the same
script with its own code.

The shapes follow the agent traces described on the source pages:

* "AKV: Cache Engineering for Autonomous Agents and State-Preserving Prefix
  Invalidation Bypass" (A. Akhunji), section 1 (a 40-step agent trajectory
  grows past 64K tokens) and section 2 (block-paged KV, 16-token blocks in the
  drop/repos figure).
* "Cache Engineering for Agents" (reading notes on Fu et al.), section 2
  (keep all reasoning and recent tool responses, drop older tool responses).
* "Leyline: KV Cache Directives for Agentic Inference" (paper digest), Method
  and Results (span-replacement directives on ~17K-token MLA prompts).

Raw keys are drawn N(0, 1) and stored without applying RoPE: a RoPE rotation
of an isotropic Gaussian pair is again an isotropic Gaussian pair, so these
values are distributed exactly like keys already rotated to their positions.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Layout", "SeqCreate", "Append", "AppendBatch", "Drop", "Repos", "Splice", "Compact", "Clone",
    "Freeze", "Share", "Materialize",
    "Segment", "Attention", "Workload", "to_bf16", "bf16_to_f64",
    "c1_tiny", "c2_64k", "c3_mla", "c4_batched", "c5_128k", "decode_batch", "decode_with_idle", "retrigger",
    "with_idle_compaction", "share_fuzz", "share_background",
    "fuzz_small",
    "CONFIGS", "make", "query_variant",
]


# --------------------------------------------------------------------------
# bf16 encoding (torch's RNE cast; uint16 bit patterns in numpy)
# --------------------------------------------------------------------------
def to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_to_f64(u: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact)."""
    u32 = np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# script types
# --------------------------------------------------------------------------
@dataclass
class Layout:
    n_q_heads: int
    n_kv_heads: int
    d_nope: int          # 0 for GQA; per-head position-free key part for MLA
    d_rope: int          # rotated key dims (all of K for GQA, K_pe for MLA)
    d_v: int
    page_size: int
    num_pages: int
    kpe_per_head: int = 0   # MLA: 0 = one K_pe row per token shared by all heads
    pairing: int = 0        # 0 = interleaved pairs (2i, 2i+1); 1 = half-split (i, i+d/2)
    rope_theta: float = 10000.0

    @property
    def d_qk(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def mla(self) -> bool:
        return self.d_nope > 0

    @property
    def n_rope_heads(self) -> int:
        """Heads stored in the rotated-key array."""
        if self.mla and not self.kpe_per_head:
            return 1
        return self.n_kv_heads


@dataclass
class SeqCreate:
    pass                 # sequence ids are 0, 1, 2, ... in creation order


@dataclass
class Append:
    seq: int
    pos: np.ndarray      # int32 [n]
    k: np.ndarray        # uint16 bf16: GQA full K [n,Hkv,d_rope]; MLA K_nope [n,Hkv,d_nope]
    kpe: Optional[np.ndarray]  # MLA only: [n, n_rope_heads, d_rope]
    v: np.ndarray        # uint16 bf16 [n, Hkv, d_v]


@dataclass
class AppendBatch:
    seqs: np.ndarray     # int32 [m]: entry i appends counts[i] tokens to seqs[i]
    counts: np.ndarray   # int32 [m]
    pos: np.ndarray      # int32 [sum(counts)], entries concatenated in order
    k: np.ndarray        # as Append, rows of all entries concatenated
    kpe: Optional[np.ndarray]
    v: np.ndarray


@dataclass
class Drop:
    seq: int
    spans: np.ndarray    # int32 [m, 2], half-open logical-index spans


@dataclass
class Repos:
    seq: int
    spans: np.ndarray    # int32 [m, 2]
    deltas: np.ndarray   # int32 [m]
    deferred: bool = False   # keys keep their rotation until read (same positions, same attention)


@dataclass
class ReposBatch:
    seqs: np.ndarray         # int32 [m], distinct
    span_counts: np.ndarray  # int32 [m]
    spans: np.ndarray        # int32 [sum(span_counts), 2], entries concatenated in order
    deltas: np.ndarray       # int32 [sum(span_counts)]

    def entries(self):
        off = 0
        for s, c in zip(self.seqs.tolist(), self.span_counts.tolist()):
            yield s, self.spans[off:off + c], self.deltas[off:off + c]
            off += c


@dataclass
class Splice:
    seq: int
    spans: np.ndarray    # int32 [m, 2] in visible-list coordinates, sorted, disjoint
    stub_lens: np.ndarray  # int32 [m]
    k: np.ndarray        # stub keys, concatenated over splices (same layout as Append.k)
    kpe: Optional[np.ndarray]
    v: np.ndarray


@dataclass
class Compact:
    seq: int
    force: int = 1


@dataclass
class CompactMode:
    deferred: bool           # True: drops and splices queue fragmented sequences


@dataclass
class CompactPending:
    max_tokens: int          # budget of moved tokens for this pass
    max_seqs: int = 1 << 30


@dataclass
class Release:
    seq: int


@dataclass
class Clone:
    src: int             # retained tokens [first, first+n) of src ...
    first: int
    n: int
    dst: int             # ... appended to dst at pos + delta (positional version)
    delta: int


@dataclass
class Freeze:
    seq: int             # the sequence becomes a checkpoint (rows never change)


@dataclass
class Share:
    src: int             # retained tokens [first, first+n) of frozen src ...
    first: int
    n: int
    dst: int             # ... appended to dst by reference, at pos + delta (they owe the rotation)
    delta: int


@dataclass
class Materialize:
    seq: int             # every key turned by what it owes (shared rows: copy on write)


@dataclass
class Segment:
    seq: int
    q_begin: int
    q_len: int
    mask_spans: np.ndarray   # int32 [m, 2] logical spans hidden from this segment only


@dataclass
class Attention:
    q: np.ndarray            # uint16 bf16 [Nq, Hq, d_qk]
    segments: List[Segment]
    scale: float = 0.0       # 0 => 1/sqrt(d_qk)


@dataclass
class Workload:
    name: str
    layout: Layout
    page_order: np.ndarray   # int32 [num_pages], initial free-list order
    ops: list = field(default_factory=list)
    notes: dict = field(default_factory=dict)


# --------------------------------------------------------------------------
# helpers
# --------------------------------------------------------------------------
def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal_bf16(rng, shape, scale=1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_bf16(x)


def _append_op(rng, lay: Layout, seq: int, pos: np.ndarray) -> Append:
    n = int(len(pos))
    if lay.mla:
        k = _normal_bf16(rng, (n, lay.n_kv_heads, lay.d_nope))
        kpe = _normal_bf16(rng, (n, lay.n_rope_heads, lay.d_rope))
    else:
        k = _normal_bf16(rng, (n, lay.n_kv_heads, lay.d_rope))
        kpe = None
    v = _normal_bf16(rng, (n, lay.n_kv_heads, lay.d_v))
    return Append(seq, np.asarray(pos, dtype=np.int32), k, kpe, v)


def _loguniform(rng, lo, hi, n) -> np.ndarray:
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n))


def _rescale_int(weights: np.ndarray, total: int) -> np.ndarray:
    """Integer lengths proportional to `weights` that sum exactly to `total`
    (largest-remainder rounding)."""
    x = weights / weights.sum() * total
    out = np.floor(x).astype(np.int64)
    rem = int(total - out.sum())
    order = np.argsort(-(x - out), kind="stable")
    out[order[:rem]] += 1
    return out


def _spans(pairs) -> np.ndarray:
    a = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
    return a


def _survivor_runs(n: int, dropped: Sequence[Tuple[int, int]]):
    """For sorted disjoint dropped spans, return (spans, deltas) of the kept
    runs that follow each dropped span, with delta = -(tokens dropped before
    the run).  Runs before the first dropped span keep delta 0 and are not
    listed."""
    spans, deltas = [], []
    gone = 0
    for j, (b, e) in enumerate(dropped):
        gone += e - b
        nxt = dropped[j + 1][0] if j + 1 < len(dropped) else n
        if nxt > e:
            spans.append((e, nxt))
            deltas.append(-gone)
    return _spans(spans), np.asarray(deltas, dtype=np.int32)


def _query_segments(seq, hist_end_logical, q_row0, seg_lens, masks_per_seg):
    """Segments over freshly appended query tokens.  Segment k sees the history
    minus its own mask spans plus the new tokens of segments 0..k; the new
    tokens of later segments are hidden with one more mask span."""
    segs = []
    total = int(sum(seg_lens))
    off = 0
    for k, L in enumerate(seg_lens):
        m = list(masks_per_seg[k])
        later_b = hist_end_logical + off + L
        later_e = hist_end_logical + total
        if later_e > later_b:
            m.append((later_b, later_e))
        segs.append(Segment(seq, q_row0 + off, int(L), _spans(m) if m else np.zeros((0, 2), np.int32)))
        off += L
    return segs


# --------------------------------------------------------------------------
# config 1: tiny single request (GQA 8/2, d 64)
# --------------------------------------------------------------------------
def c1_tiny(seed: int = 0, variant: str = "canonical") -> Workload:
    """2048 cached tokens; drop 256 + 384 tokens, reposition the suffix by a
    total of -640, append 256 query tokens as two 128-token segments.

    variant "canonical":  drop [1024,1280) and [1280,1664); repos [1664,2048) by -640.
    variant "cumulative": drop [512,768) and [1280,1664); repos [768,1280) by -256
                          and [1664,2048) by -640.
    variant "unaligned":  the canonical spans shifted by +5 tokens.
    """
    rng = _rng(seed)
    lay = Layout(8, 2, 0, 64, 64, 16, 144, rope_theta=10000.0)
    n = 2048
    if variant == "canonical":
        drop = [(1024, 1280), (1280, 1664)]
        rep_s, rep_d = _spans([(1664, 2048)]), np.array([-640], np.int32)
    elif variant == "cumulative":
        drop = [(512, 768), (1280, 1664)]
        rep_s, rep_d = _spans([(768, 1280), (1664, 2048)]), np.array([-256, -640], np.int32)
    elif variant == "unaligned":
        drop = [(1029, 1285), (1285, 1669)]
        rep_s, rep_d = _spans([(1669, 2048)]), np.array([-640], np.int32)
    else:
        raise ValueError(variant)
    h = n - sum(e - b for b, e in drop)           # 1408 visible
    wl = Workload(f"c1_tiny_{variant}", lay, rng.permutation(lay.num_pages).astype(np.int32))
    wl.ops.append(SeqCreate())
    wl.ops.append(_append_op(rng, lay, 0, np.arange(n, dtype=np.int32)))
    wl.ops.append(Drop(0, _spans(drop)))
    wl.ops.append(Repos(0, rep_s, rep_d))
    wl.ops.append(_append_op(rng, lay, 0, np.arange(h, h + 256, dtype=np.int32)))
    q = _normal_bf16(rng, (256, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    segs = _query_segments(0, n, 0, [128, 128], [[], [(250, 390)]])
    wl.ops.append(Attention(q, segs))
    wl.notes.update(history=h, repositioned=int(sum(e - b for b, e in rep_s)))
    return wl


# --------------------------------------------------------------------------
# config 2: Llama-3.1-8B-shaped layer, 64K tokens in 40 agent turns
# --------------------------------------------------------------------------
def _c2_like_history(rng, n_turns=40, n_recent=8, total=65536, drop_frac=0.40, reasoning=512):
    """Turn lengths for a 40-turn trace of exactly `total` tokens: each turn is
    `reasoning` tokens then a tool response.  Log-uniform[256, 8192] tool
    lengths are rescaled per group so the older tools hold drop_frac of the
    tokens (they are the ones dropped) and the recent tools hold the rest."""
    old = n_turns - n_recent
    old_total = int(round(drop_frac * total))
    recent_total = total - n_turns * reasoning - old_total
    t_old = _rescale_int(_loguniform(rng, 256, 8192, old), old_total)
    t_new = _rescale_int(_loguniform(rng, 256, 8192, n_recent), recent_total)
    tools = np.concatenate([t_old, t_new])
    spans_tool, cur = [], 0
    for t in tools:
        cur += reasoning
        spans_tool.append((cur, cur + int(t)))
        cur += int(t)
    assert cur == total
    return spans_tool


def c2_64k(seed: int = 0, num_pages: Optional[int] = None) -> Workload:
    rng = _rng(seed)
    n = 65536
    nq = 2048
    pages = num_pages if num_pages is not None else (n + nq) // 16
    lay = Layout(32, 8, 0, 128, 128, 16, pages, rope_theta=500000.0)
    tools = _c2_like_history(rng)
    dropped = tools[:32]
    rep_s, rep_d = _survivor_runs(n, dropped)
    h = n - sum(e - b for b, e in dropped)
    wl = Workload("c2_64k", lay, rng.permutation(lay.num_pages).astype(np.int32))
    wl.ops.append(SeqCreate())
    wl.ops.append(_append_op(rng, lay, 0, np.arange(n, dtype=np.int32)))
    wl.ops.append(Drop(0, _spans(dropped)))
    wl.ops.append(Repos(0, rep_s, rep_d))
    wl.ops.append(_append_op(rng, lay, 0, np.arange(h, h + nq, dtype=np.int32)))
    q = _normal_bf16(rng, (nq, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    masks = [[tools[32 + j] for j in range(k)] for k in range(4)]
    wl.ops.append(Attention(q, _query_segments(0, n, 0, [512] * 4, masks)))
    wl.notes.update(history=h, repositioned=int(sum(e - b for b, e in rep_s)),
                    tool_spans=tools, dropped_spans=dropped)
    return wl


# --------------------------------------------------------------------------
# config 3: MLA-shaped layer (DeepSeek-V2-Lite-like), Leyline splices
# --------------------------------------------------------------------------
def _place_disjoint(rng, n, lens, max_tries=10000):
    """Uniform placement of spans with the given lengths inside [0, n) without
    overlap (rejection sampling); returned sorted by start."""
    for _ in range(max_tries):
        starts = [int(rng.integers(0, n - L + 1)) for L in lens]
        sp = sorted(zip(starts, [s + L for s, L in zip(starts, lens)]))
        if all(sp[i][1] <= sp[i + 1][0] for i in range(len(sp) - 1)):
            return sp
    raise RuntimeError("could not place spans")


def c3_mla(seed: int = 0) -> Workload:
    rng = _rng(seed)
    n = 17408
    nq = 512
    lay = Layout(16, 16, 128, 64, 128, 64, 288, kpe_per_head=0, rope_theta=10000.0)
    m = int(rng.integers(1, 4))
    lens = [int(rng.integers(500, 4001)) for _ in range(m)]
    spans = _place_disjoint(rng, n, lens)
    stub = np.array([int(rng.integers(8, 33)) for _ in range(m)], np.int32)
    wl = Workload("c3_mla", lay, rng.permutation(lay.num_pages).astype(np.int32))
    wl.ops.append(SeqCreate())
    wl.ops.append(_append_op(rng, lay, 0, np.arange(n, dtype=np.int32)))
    ns = int(stub.sum())
    a = _append_op(rng, lay, 0, np.zeros(ns, np.int32))
    wl.ops.append(Splice(0, _spans(spans), stub, a.k, a.kpe, a.v))
    h = n - sum(e - b for b, e in spans) + ns
    wl.ops.append(_append_op(rng, lay, 0, np.arange(h, h + nq, dtype=np.int32)))
    q = _normal_bf16(rng, (nq, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    wl.ops.append(Attention(q, _query_segments(0, n + ns, 0, [nq], [[]])))
    wl.notes.update(history=h, splices=spans, stub_lens=stub.tolist())
    return wl


# --------------------------------------------------------------------------
# config 4: 16 concurrent requests on the config-2 layer shape
# --------------------------------------------------------------------------
def c4_batched(seed: int = 0, n_req: int = 16, ctx_lo: int = 8192, ctx_hi: int = 32768,
               batched: bool = True) -> Workload:
    """batched: the requests' repos go in one ReposBatch (one rotation launch)
    and their new tokens in one AppendBatch; otherwise one call per request.
    The two forms give the same state (ops on different sequences commute and
    the appends keep their order)."""
    rng = _rng(seed)
    reqs = []
    for r in range(n_req):
        ctx = int(rng.integers(ctx_lo, ctx_hi + 1))
        tools, cur = [], 0
        while cur < ctx:
            cur = min(cur + 512, ctx)
            if cur >= ctx:
                break
            t = int(_loguniform(rng, 256, 8192, 1)[0])
            tools.append((cur, min(cur + t, ctx)))
            cur = min(cur + t, ctx)
        f = float(rng.uniform(0.10, 0.60))
        cand = list(range(max(0, len(tools) - 2)))      # the last two tool spans are recent
        rng.shuffle(cand)
        gone, chosen = 0, []
        for i in cand:
            if gone >= f * ctx:
                break
            chosen.append(i)
            gone += tools[i][1] - tools[i][0]
        chosen.sort()
        dropped = [tools[i] for i in chosen]
        keep_tools = [tools[i] for i in range(len(tools)) if i not in set(chosen)]
        n_seg = int(rng.integers(1, 5))
        qtot = int(rng.integers(256, 1025))
        cuts = np.sort(rng.choice(np.arange(1, qtot), size=n_seg - 1, replace=False)) if n_seg > 1 else np.array([], int)
        bounds = [0] + [int(c) for c in cuts] + [qtot]
        seg_lens = [bounds[i + 1] - bounds[i] for i in range(n_seg)]
        reqs.append(dict(ctx=ctx, tools=tools, dropped=dropped, keep_tools=keep_tools,
                         seg_lens=seg_lens, qtot=qtot))
    pages = sum((q["ctx"] + q["qtot"] + 15) // 16 for q in reqs) + 16
    lay = Layout(32, 8, 0, 128, 128, 16, pages, rope_theta=500000.0)
    wl = Workload("c4_batched", lay, rng.permutation(pages).astype(np.int32))
    for r in range(n_req):
        wl.ops.append(SeqCreate())
    for r, q in enumerate(reqs):            # histories, interleaved in the shared pool
        wl.ops.append(_append_op(rng, lay, r, np.arange(q["ctx"], dtype=np.int32)))
    rep = []
    for r, q in enumerate(reqs):
        if q["dropped"]:
            wl.ops.append(Drop(r, _spans(q["dropped"])))
            rs, rd = _survivor_runs(q["ctx"], q["dropped"])
            if len(rs):
                rep.append(Repos(r, rs, rd))
    if batched and rep:
        wl.ops.append(ReposBatch(np.asarray([o.seq for o in rep], np.int32),
                                 np.asarray([len(o.spans) for o in rep], np.int32),
                                 np.concatenate([o.spans for o in rep]).astype(np.int32),
                                 np.concatenate([o.deltas for o in rep]).astype(np.int32)))
    else:
        wl.ops += rep
    segs, row = [], 0
    new = []
    for r, q in enumerate(reqs):
        h = q["ctx"] - sum(e - b for b, e in q["dropped"])
        new.append(_append_op(rng, lay, r, np.arange(h, h + q["qtot"], dtype=np.int32)))
        kt = q["keep_tools"]
        masks = [[kt[j] for j in range(min(k, len(kt)))] for k in range(len(q["seg_lens"]))]
        segs += _query_segments(r, q["ctx"], row, q["seg_lens"], masks)
        row += q["qtot"]
    if batched:
        wl.ops.append(AppendBatch(np.asarray([a.seq for a in new], np.int32),
                                  np.asarray([len(a.pos) for a in new], np.int32),
                                  np.concatenate([a.pos for a in new]), np.concatenate([a.k for a in new]),
                                  None, np.concatenate([a.v for a in new])))
    else:
        wl.ops += new
    qarr = _normal_bf16(rng, (row, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    wl.ops.append(Attention(qarr, segs))
    wl.notes.update(requests=reqs)
    return wl


# --------------------------------------------------------------------------
# retrigger: a cached state re-used at other positions (positional version)
# --------------------------------------------------------------------------
def retrigger(seed: int = 0, ctx: int = 65536, pre_a: int = 512, nq: int = 512, n_turns: int = 40,
              n_recent: int = 8, pre_b: Optional[int] = None, mla: bool = False) -> Workload:
    """Request A: a pre_a-token preamble, then a ctx-token agent trace (the
    64K recipe: reasoning turns and log-uniform tool outputs, the older tools
    holding 40% of the tokens, all dropped, the survivors repositioned).
    Request B holds the same trace after a preamble of pre_b tokens (random in
    [0, 2 pre_a] unless given): its cached state is A's, re-used at positions
    shifted by pre_b - pre_a through one clone.  Both then append nq new
    tokens and attend in one launch (one segment each)."""
    rng = _rng(seed)
    if pre_b is None:
        pre_b = int(rng.integers(0, 2 * pre_a + 1))
    if mla:
        S = 64
        lay = Layout(16, 16, 128, 64, 128, S, 1, kpe_per_head=0, rope_theta=10000.0)
    else:
        S = 16
        lay = Layout(32, 8, 0, 128, 128, S, 1, rope_theta=500000.0)
    reasoning = max(32, min(512, ctx // (2 * n_turns)))
    tools = _c2_like_history(rng, n_turns, n_recent, ctx, 0.40, reasoning)
    dropped = [(pre_a + b, pre_a + e) for b, e in tools[:n_turns - n_recent]]
    n_a = pre_a + ctx
    rep_s, rep_d = _survivor_runs(n_a, dropped)
    kept = ctx - sum(e - b for b, e in dropped)
    pages = (n_a + nq) // S + (pre_b + kept + nq) // S + 8
    lay.num_pages = pages
    wl = Workload("retrigger", lay, rng.permutation(pages).astype(np.int32))
    wl.ops.append(SeqCreate())
    wl.ops.append(SeqCreate())
    wl.ops.append(_append_op(rng, lay, 0, np.arange(n_a, dtype=np.int32)))
    wl.ops.append(_append_op(rng, lay, 1, np.arange(pre_b, dtype=np.int32)))
    wl.ops.append(Drop(0, _spans(dropped)))
    if len(rep_s):
        wl.ops.append(Repos(0, rep_s, rep_d))
    wl.ops.append(Clone(0, pre_a, ctx, 1, pre_b - pre_a))
    h_a, h_b = pre_a + kept, pre_b + kept
    wl.ops.append(_append_op(rng, lay, 0, np.arange(h_a, h_a + nq, dtype=np.int32)))
    wl.ops.append(_append_op(rng, lay, 1, np.arange(h_b, h_b + nq, dtype=np.int32)))
    q = _normal_bf16(rng, (2 * nq, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    none = np.zeros((0, 2), np.int32)
    wl.ops.append(Attention(q, [Segment(0, 0, nq, none), Segment(1, nq, nq, none)]))
    wl.notes.update(pre_a=pre_a, pre_b=pre_b, delta=pre_b - pre_a, kept=kept, dropped_spans=dropped)
    return wl


# --------------------------------------------------------------------------
# decode: one new token per request at high batch (the inter-token side)
# --------------------------------------------------------------------------
def decode_batch(seed: int = 0, n_req: int = 48, ctx_lo: int = 2048, ctx_hi: int = 16384,
                 n_q_heads: int = 32, q_len: int = 1, deferred: bool = False, pairing: int = 0,
                 page_size: int = 16) -> Workload:
    """n_req agent histories in one pool, each built with the batched recipe
    (512-token reasoning turns, log-uniform tool spans, 10-60% of the older
    tools dropped, survivors repositioned); then every request appends q_len
    tokens (1: plain decode; a few: speculative or multi-token steps) at its
    next positions and runs one segment over its whole visible list, all in
    one attention launch.  deferred: the survivors' repos leaves the keys
    where they are (the decode kernel turns them as it reads them)."""
    rng = _rng(seed)
    reqs = []
    for r in range(n_req):
        ctx = int(rng.integers(ctx_lo, ctx_hi + 1))
        tools, cur = [], 0
        while cur < ctx:
            cur = min(cur + 512, ctx)
            if cur >= ctx:
                break
            t = int(_loguniform(rng, 256, 8192, 1)[0])
            tools.append((cur, min(cur + t, ctx)))
            cur = min(cur + t, ctx)
        f = float(rng.uniform(0.10, 0.60))
        cand = list(range(max(0, len(tools) - 2)))
        rng.shuffle(cand)
        gone, chosen = 0, []
        for i in cand:
            if gone >= f * ctx:
                break
            chosen.append(i)
            gone += tools[i][1] - tools[i][0]
        dropped = [tools[i] for i in sorted(chosen)]
        reqs.append(dict(ctx=ctx, dropped=dropped))
    pages = sum((q["ctx"] + q_len + page_size - 1) // page_size for q in reqs) + 16
    lay = Layout(n_q_heads, 8, 0, 128, 128, page_size, pages, pairing=pairing, rope_theta=500000.0)
    wl = Workload("decode_batch", lay, rng.permutation(pages).astype(np.int32))
    for r in range(n_req):
        wl.ops.append(SeqCreate())
    for r, q in enumerate(reqs):
        wl.ops.append(_append_op(rng, lay, r, np.arange(q["ctx"], dtype=np.int32)))
    for r, q in enumerate(reqs):
        if q["dropped"]:
            wl.ops.append(Drop(r, _spans(q["dropped"])))
            rs, rd = _survivor_runs(q["ctx"], q["dropped"])
            if len(rs):
                wl.ops.append(Repos(r, rs, rd, deferred))
    segs, news = [], []
    wl.notes["step_from"] = len(wl.ops)     # one decode step: the new tokens and attention
    for r, q in enumerate(reqs):
        h = q["ctx"] - sum(e - b for b, e in q["dropped"])
        news.append(_append_op(rng, lay, r, np.arange(h, h + q_len, dtype=np.int32)))
        segs.append(Segment(r, r * q_len, q_len, np.zeros((0, 2), np.int32)))
    wl.ops.append(AppendBatch(np.arange(n_req, dtype=np.int32), np.full(n_req, q_len, np.int32),
                              np.concatenate([a.pos for a in news]), np.concatenate([a.k for a in news]),
                              None, np.concatenate([a.v for a in news])))
    qarr = _normal_bf16(rng, (n_req * q_len, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    wl.ops.append(Attention(qarr, segs))
    wl.notes.update(requests=reqs)
    return wl


def with_idle_compaction(wl: Workload, seed: int = 0, n_idle: int = 8, idle_ctx: int = 32768, block: int = 8,
                         attend_idle: bool = False) -> Workload:
    """`wl` while other agents wait on tools: n_idle idle sequences of
    idle_ctx tokens (created after wl's own sequences) lose every other
    block of `block` tokens (half a 16-token page: fragmentation 0.5, above
    the 0.4 threshold) in deferred compaction mode, so they wait in the
    compaction queue.  The step runs wl's own step (its operations from
    notes["step_from"], else from its first operation other than a sequence
    creation or an append), then the background compaction pass over the
    queue (its copies read and write none of the pages wl's step reads, so
    they run beside it).  attend_idle appends one more launch with a
    one-query segment over each idle sequence (its last token)."""
    rng = _rng(seed + 7919)
    lay = wl.layout
    S = lay.page_size
    i0 = wl.notes.get("step_from",
                      next(i for i, o in enumerate(wl.ops) if not isinstance(o, (SeqCreate, Append))))
    head, step = wl.ops[:i0], wl.ops[i0:]
    n_own = sum(isinstance(o, SeqCreate) for o in wl.ops)
    idle = list(range(n_own, n_own + n_idle))
    last_create = max(i for i, o in enumerate(head) if isinstance(o, SeqCreate))
    ops = head[:last_create + 1] + [SeqCreate() for _ in idle] + head[last_create + 1:]
    for s in idle:
        ops.append(_append_op(rng, lay, s, np.arange(idle_ctx, dtype=np.int32)))
    ops.append(CompactMode(True))
    for s in idle:
        ops.append(Drop(s, _spans([(b, min(b + block, idle_ctx)) for b in range(block, idle_ctx, 2 * block)])))
    out = Workload(f"{wl.name}_idle", lay, wl.page_order, ops, dict(wl.notes))
    out.notes["step_from"] = len(ops)
    ops += step
    ops.append(CompactPending(1 << 40))
    if attend_idle:
        q = _normal_bf16(rng, (n_idle, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
        none = np.zeros((0, 2), np.int32)
        ops.append(Attention(q, [Segment(s, i, 1, none) for i, s in enumerate(idle)]))
    # pages: the idle sequences and their compacted copies
    extra = n_idle * (2 * ((idle_ctx + S - 1) // S) + 2)
    lay.num_pages += extra
    order = np.concatenate([wl.page_order, np.arange(lay.num_pages - extra, lay.num_pages, dtype=np.int32)])
    out.page_order = rng.permutation(order).astype(np.int32)
    out.notes["idle"] = idle
    return out


def decode_with_idle(seed: int = 0, n_req: int = 48, n_idle: int = 8, idle_ctx: int = 32768,
                     attend_idle: bool = False, **kw) -> Workload:
    """The decode step of decode_batch, then a background compaction pass
    over n_idle fragmented idle sequences (with_idle_compaction)."""
    return with_idle_compaction(decode_batch(seed, n_req=n_req, **kw), seed, n_idle, idle_ctx,
                                attend_idle=attend_idle)


def share_fuzz(seed: int, mla: bool = False, page_size: int = 16, d: int = 64, pairing: int = 0,
               n_hist: int = 600, n_q: int = 24, group: int = 4, materialize: Optional[bool] = None) -> Workload:
    """Checkpoints and sharers: sequence 0 (a history with a drop and a
    repos) is frozen; sequences 1 and 2 share all or a suffix of it at other
    positions (one delta each, either sign, or 0); sequence 1 appends, drops
    shared and own tokens, repositions across both, then compacts or
    materializes (copy on write); sequence 0 is released while shared;
    sequence 2 drops shared tokens and splices over shared rows; sequence 3
    clones half of sequence 1.
    Then sequences 1, 2 and 3 append n_q query tokens each (positions past
    every earlier one, so they are each list's last entries) and attend in
    one launch."""
    rng = _rng(seed)
    if mla:
        lay = Layout(4, 4, 32, 32, 32, page_size, 0, pairing=pairing, rope_theta=10000.0)
    else:
        lay = Layout(2 * group, 2, 0, d, d, page_size, 0, pairing=pairing, rope_theta=10000.0)
    n0 = n_hist
    ops: list = [SeqCreate() for _ in range(4)]
    ops.append(_append_op(rng, lay, 0, np.arange(n0, dtype=np.int32)))
    b = int(rng.integers(50, n0 // 2))
    e = b + int(rng.integers(10, 80))
    ops.append(Drop(0, _spans([(b, e)])))
    ops.append(Repos(0, _spans([(e, n0)]), np.array([-(e - b)], np.int32)))
    ops.append(Freeze(0))
    vis0 = n0 - (e - b)
    d1 = int(rng.choice([0, 333, -40, 1000]))
    d2 = int(rng.choice([77, -30, 0]))
    first2 = int(rng.integers(0, b))
    ops.append(Share(0, 0, n0, 1, d1 + 60))
    ops.append(Share(0, first2, n0 - first2, 2, d2 + 60))
    ops.append(_append_op(rng, lay, 1, np.arange(500_000, 500_030, dtype=np.int32)))
    n1 = vis0 + 30
    s1 = int(rng.integers(20, vis0 - 60))
    ops.append(Drop(1, _spans([(s1, s1 + 25), (vis0 + 5, vis0 + 9)])))
    ops.append(Repos(1, _spans([(s1 + 25, n1)]), np.array([-25], np.int32)))
    mat = bool(rng.random() < 0.5) if materialize is None else materialize
    ops.append(Materialize(1) if mat else Compact(1, 1))
    ops.append(Release(0))                     # still shared: its pages stay
    ops.append(Drop(2, _spans([(3, 11)])))
    # a splice over shared rows: the span's shared tokens give their slots
    # up, the stub goes to sequence 2's own pages, the shared tokens
    # downstream owe the shift
    stub = _append_op(rng, lay, 2, np.zeros(5, np.int32))
    ops.append(Splice(2, _spans([(20, 60)]), np.array([5], np.int32), stub.k, stub.kpe, stub.v))
    ops.append(Clone(1, 0, n1 // 2, 3, int(rng.choice([0, 55]))))
    segs = []
    for i, sq in enumerate((1, 2, 3)):
        ops.append(_append_op(rng, lay, sq, np.arange(1_000_000, 1_000_000 + n_q, dtype=np.int32)))
        segs.append(Segment(sq, i * n_q, n_q, np.zeros((0, 2), np.int32)))
    ops.append(Attention(_normal_bf16(rng, (3 * n_q, lay.n_q_heads, lay.d_qk), scale=0.5), segs))
    lay.num_pages = 4 * ((n0 + 3 * n_q + 64) // page_size + 8)
    wl = Workload(f"share_fuzz_{seed}", lay, rng.permutation(lay.num_pages).astype(np.int32), ops)
    wl.notes.update(materialize=mat)
    return wl


def share_background(seed: int, page_size: int = 8, n_src: int = 400, n_q: int = 16) -> Workload:
    """Shared rows through a background compaction pass: sequence 0 is
    frozen and shared (at +50) by sequence 1, which appends its own tokens;
    sequence 0 is released while shared; in deferred compaction mode
    sequence 1 drops every other block of 4 shared tokens (fragmented), and
    the background pass moves its rows, shared ones included, into its own
    pages, so the source's last holder lets go and the source's pages return
    to the queue while the copies that read them may still run; a new
    sequence then appends into pages the queue hands out, and sequences 1
    and 2 attend in one launch."""
    rng = _rng(seed)
    lay = Layout(8, 2, 0, 64, 64, page_size, 0, rope_theta=10000.0)
    ops: list = [SeqCreate(), SeqCreate()]
    ops.append(_append_op(rng, lay, 0, np.arange(n_src, dtype=np.int32)))
    ops.append(Freeze(0))
    ops.append(Share(0, 0, n_src, 1, 50))
    ops.append(_append_op(rng, lay, 1, np.arange(n_src + 50, n_src + 90, dtype=np.int32)))
    ops.append(Release(0))
    ops.append(CompactMode(True))
    ops.append(Drop(1, _spans([(b, b + 4) for b in range(4, n_src - 8, 8)])))
    ops.append(CompactPending(1 << 30))
    ops.append(SeqCreate())
    ops.append(_append_op(rng, lay, 2, np.arange(0, n_src, dtype=np.int32)))
    segs = []
    for i, (sq, p0) in enumerate([(1, 1_000_000), (2, 2_000_000)]):
        ops.append(_append_op(rng, lay, sq, np.arange(p0, p0 + n_q, dtype=np.int32)))
        segs.append(Segment(sq, i * n_q, n_q, np.zeros((0, 2), np.int32)))
    ops.append(Attention(_normal_bf16(rng, (2 * n_q, lay.n_q_heads, lay.d_qk), scale=0.5), segs))
    # tight: the new sequence's pages must include the source's, given back
    # during the pass
    lay.num_pages = (n_src + 90 + n_src // 2 + 60) // page_size + 12
    return Workload(f"share_background_{seed}", lay, rng.permutation(lay.num_pages).astype(np.int32), ops)


# --------------------------------------------------------------------------
# config 5: Llama-3.1-70B-shaped layer on one GPU, 128K tokens
# --------------------------------------------------------------------------
def c5_128k(seed: int = 0) -> Workload:
    rng = _rng(seed)
    n = 131072
    nq = 4096
    lay = Layout(64, 8, 0, 128, 128, 16, (n + nq) // 16, rope_theta=500000.0)
    keep = _rescale_int(_loguniform(rng, 256, 8192, 61), 39322)
    drop = _rescale_int(_loguniform(rng, 256, 8192, 60), n - 39322)
    runs_keep, dropped, cur = [], [], 0
    for j in range(61):
        runs_keep.append((cur, cur + int(keep[j])))
        cur += int(keep[j])
        if j < 60:
            dropped.append((cur, cur + int(drop[j])))
            cur += int(drop[j])
    assert cur == n
    rep_s, rep_d = _survivor_runs(n, dropped)
    h = 39322
    wl = Workload("c5_128k", lay, rng.permutation(lay.num_pages).astype(np.int32))
    wl.ops.append(SeqCreate())
    wl.ops.append(_append_op(rng, lay, 0, np.arange(n, dtype=np.int32)))
    wl.ops.append(Drop(0, _spans(dropped)))
    wl.ops.append(Repos(0, rep_s, rep_d))
    wl.ops.append(_append_op(rng, lay, 0, np.arange(h, h + nq, dtype=np.int32)))
    q = _normal_bf16(rng, (nq, lay.n_q_heads, lay.d_qk), scale=1.0 / 8.0)
    masks = [[runs_keep[1 + j] for j in range(k)] for k in range(8)]
    wl.ops.append(Attention(q, _query_segments(0, n, 0, [512] * 8, masks)))
    wl.notes.update(history=h, repositioned=int(sum(e - b for b, e in rep_s)))
    return wl


# --------------------------------------------------------------------------
# small random scripts (fuzz): overlapping spans, either sign of delta,
# splices, forced compaction, several sequences, ragged pages
# --------------------------------------------------------------------------
def fuzz_small(seed: int, mla: bool = False, pairing: int = 0, n_seqs: int = 2,
               max_tokens: int = 300, page_size: int = 16, n_rounds: int = 3,
               compact: bool = True, kpe_per_head: int = 0,
               head_dims: Sequence[int] = (16, 32, 64), mla_dims: Tuple[int, int, int] = (32, 16, 32),
               groups: Sequence[int] = (1, 2, 4)) -> Workload:
    """head_dims: GQA head sizes to draw from; mla_dims: (d_nope, d_rope, d_v)."""
    rng = _rng(seed)
    if mla:
        dn, dr, dv = mla_dims
        lay = Layout(4, 4, dn, dr, dv, page_size, 0, kpe_per_head=kpe_per_head,
                     pairing=pairing, rope_theta=10000.0)
    else:
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice(list(groups)))
        d = int(rng.choice(list(head_dims)))
        lay = Layout(hkv * g, hkv, 0, d, d, page_size, 0, pairing=pairing, rope_theta=10000.0)
    ops = []
    ntok = [0] * n_seqs
    npos = [200] * n_seqs          # room below: repos deltas here never push a position under 0
    total_tokens = 0
    for s in range(n_seqs):
        ops.append(SeqCreate())
    for rnd in range(n_rounds):
        for s in range(n_seqs):
            n = int(rng.integers(1, max_tokens // n_rounds + 2))
            ops.append(_append_op(rng, lay, s, np.arange(npos[s], npos[s] + n, dtype=np.int32)))
            ntok[s] += n
            npos[s] += n
            total_tokens += n
            k = int(rng.integers(0, 3))
            sp = []
            for _ in range(k):
                b = int(rng.integers(0, ntok[s]))
                e = int(rng.integers(b, min(ntok[s], b + 40) + 1))
                sp.append((b, e))
            if sp:
                ops.append(Drop(s, _spans(sp)))
            k = int(rng.integers(0, 3))
            sp, dl = [], []
            for _ in range(k):
                b = int(rng.integers(0, ntok[s]))
                e = int(rng.integers(b, ntok[s] + 1))
                sp.append((b, e))
                dl.append(int(rng.integers(-30, 31)))
            if sp:
                ops.append(Repos(s, _spans(sp), np.asarray(dl, np.int32)))
            if compact and rng.random() < 0.3:
                ops.append(Compact(s, 1))
    # a fresh sequence per segment tail: query tokens appended last
    segs, row = [], 0
    for s in range(n_seqs):
        nq = int(rng.integers(1, 24))
        p0 = npos[s] + 1000            # positions of the new tokens exceed every cached one
        ops.append(_append_op(rng, lay, s, np.arange(p0, p0 + nq, dtype=np.int32)))
        total_tokens += nq
        hist = ntok[s]
        ntok[s] += nq
        nseg = int(rng.integers(1, 3)) if nq > 1 else 1
        lens = [nq] if nseg == 1 else [nq // 2, nq - nq // 2]
        masks = []
        for k in range(nseg):
            if k and hist > 4:
                b = int(rng.integers(0, hist - 2))
                masks.append([(b, b + int(rng.integers(1, 4)))])
            else:
                masks.append([])
        segs += _query_segments(s, hist, row, lens, masks)
        row += nq
    lay.num_pages = 2 * ((total_tokens + page_size - 1) // page_size) + 4 * n_seqs + 8
    q = _normal_bf16(rng, (row, lay.n_q_heads, lay.d_qk), scale=0.5)
    ops.append(Attention(q, segs))
    wl = Workload(f"fuzz_{seed}", lay, rng.permutation(lay.num_pages).astype(np.int32), ops)
    return wl


def deferred_compaction(seed: int, n_seqs: int = 4, n_rounds: int = 5, page_size: int = 8,
                        pages_factor: float = 3.0) -> Workload:
    """Sequences whose drops leave them fragmented, in deferred-compaction
    mode: the compactions wait in the queue and run in later passes under
    token budgets (some too small for the queue's head, some limited to one
    sequence), some queued sequences are brought back under the threshold by
    appends before their turn, one queued sequence is released, and attention
    runs between passes and at the end ([AKV-blog] section 7, Dilemma 2)."""
    rng = _rng(seed)
    lay = Layout(8, 2, 0, 64, 64, page_size, 0, rope_theta=10000.0)
    ops = [CompactMode(True)]
    n_all = n_seqs + 1                   # the last sequence is released while queued
    ntok, npos = [0] * n_all, [64] * n_all
    total = 0
    for _ in range(n_all):
        ops.append(SeqCreate())

    def append(s, n):
        nonlocal total
        ops.append(_append_op(rng, lay, s, np.arange(npos[s], npos[s] + n, dtype=np.int32)))
        ntok[s] += n
        npos[s] += n
        total += n

    def shred(s):
        # drop every other block of 4..12 tokens over a random range: most
        # pages keep some visible token, so fragmentation passes 0.4
        b = int(rng.integers(0, max(1, ntok[s] // 4)))
        sp, t = [], b
        while t < ntok[s]:
            w = int(rng.integers(4, 13))
            sp.append((t, min(t + w, ntok[s])))
            t += 2 * w
        ops.append(Drop(s, _spans(sp)))

    for rnd in range(n_rounds):
        for s in range(n_all):
            if s == n_seqs and rnd > 1:
                continue
            append(s, int(rng.integers(24, 96)))
            if rng.random() < 0.6:
                shred(s)
            if rng.random() < 0.3:
                b = int(rng.integers(0, ntok[s]))
                ops.append(Repos(s, _spans([(b, ntok[s])]), np.asarray([int(rng.integers(-20, 21))], np.int32)))
        if rnd == 1:
            shred(n_seqs)
            ops.append(Release(n_seqs))
        budget = [0, 40, 150, 1 << 20][int(rng.integers(0, 4))]
        ops.append(CompactPending(budget, [1, 2, 1 << 30][int(rng.integers(0, 3))]))
        if rnd == 2:                     # appends after queuing can bring one under the threshold
            append(int(rng.integers(0, n_seqs)), 200)
    segs, row = [], 0
    for s in range(n_seqs):
        nq = int(rng.integers(4, 20))
        hist = ntok[s]
        append(s, nq)
        segs += _query_segments(s, hist, row, [nq], [[]])
        row += nq
    ops.append(CompactPending(1 << 20))
    q = _normal_bf16(rng, (row, lay.n_q_heads, lay.d_qk), scale=0.5)
    ops.append(Attention(q, segs))
    # pages_factor near 1: compactions must take pages back from the evictable queue
    lay.num_pages = int(pages_factor * ((total + page_size - 1) // page_size)) + 8 * n_all + 16
    return Workload(f"deferred_compaction_{seed}", lay, rng.permutation(lay.num_pages).astype(np.int32), ops,
                    notes={"deferred_compaction": True})


# --------------------------------------------------------------------------
# query variants: stress (Q ~ N(0,1)) and focused attention
# --------------------------------------------------------------------------
FOCUS_GAIN = 20.0     # a focused query adds FOCUS_GAIN x a unit vector: score ~ 20 above the rest
FOCUS_V_CLIP = 3.5    # focused workloads keep |V| <= 3.5 (exact in bf16), see query_variant


def _low_freq_dims(lay: Layout, n: int = 8) -> np.ndarray:
    """Key dims whose rotation angle per position is smallest: the last n/2
    rotation pairs (MLA: the first n position-free K_nope dims, which are
    never rotated).  A needle key put there stays aligned with its query
    direction after a repos by tens of thousands of positions."""
    if lay.mla:
        return np.arange(n)
    d = lay.d_rope
    pairs = np.arange(d // 2 - n // 2, d // 2)
    if lay.pairing == 0:
        return np.sort(np.concatenate([2 * pairs, 2 * pairs + 1]))
    return np.sort(np.concatenate([pairs, pairs + d // 2]))


def _bf16_f32(u: np.ndarray) -> np.ndarray:
    return bf16_to_f64(u).astype(np.float32)


def query_variant(wl: Workload, mode: str, seed: int = 0, n_dirs: int = 4, needles_per_dir: int = 2) -> Workload:
    """A copy of `wl` with other queries.

    "stress": every query row is drawn N(0,1) in fp32 (the base workloads
    draw N(0,1)/8, which leaves the softmax nearly uniform over long lists).

    "focus": stress queries, then row i of each segment, q head h, gets one
    target by (i + h) % 4:
      0  its own key (the segment's i-th own token, the last entry it sees),
      1  the key of the next token (hidden from it by causality or by the
         segment's mask of later tokens),
      2  a needle direction u: n_dirs directions per sequence, each added
         (times sqrt(d_qk)) to the keys of needles_per_dir random history
         tokens, some of which later drops or masks hide (GQA: only tokens
         no repos moves, see below),
      3  nothing;
    the target's unit vector times FOCUS_GAIN is added to the row, so the
    target's score stands about 20 above the others and a handful of keys
    carry almost all of the softmax mass.  Values are clipped to
    |v| <= FOCUS_V_CLIP so an output dominated by one key stays within the
    range where bf16 output rounding leaves room under a 2e-2 error bar.

    The targets are keys whose stored bits are exact inputs on every side:
    own and next tokens are appended after the history's repos, and GQA
    needles sit on tokens no repos span covers (MLA needles live in K_nope,
    which no repos touches).  A repositioned key is stored rounded to bf16
    (its 1e-2 relative bar), and a softmax this sharp would turn that
    rounding into output differences of a few 1e-2 between two competing
    keys; the stress queries cover repositioned keys with a soft softmax.

    Own tokens of a segment are its sequence's last q_len appended tokens
    outside its mask spans (the generators append the query tokens last);
    workloads whose query tokens are rewritten later (repos, splice or clone
    after their append) or that clone tokens are refused in focus mode.
    Input construction only: no rotation, attention or visibility rule."""
    if mode not in ("stress", "focus"):
        raise ValueError(mode)
    rng = _rng(1_000_003 + seed)
    lay = wl.layout
    ops = list(wl.ops)
    out = Workload(f"{wl.name}_{mode}", lay, wl.page_order, ops, dict(wl.notes, query_variant=mode))
    if mode == "stress":
        for i, op in enumerate(ops):
            if isinstance(op, Attention):
                ops[i] = Attention(_normal_bf16(rng, op.q.shape), op.segments, op.scale)
        return out

    G = lay.n_q_heads // lay.n_kv_heads
    moved = {}   # seq -> logical spans any repos of the script covers
    for op in ops:
        if isinstance(op, Repos):
            moved.setdefault(op.seq, []).extend(np.asarray(op.spans).reshape(-1, 2).tolist())
        elif isinstance(op, ReposBatch):
            for s_, sp, _ in op.entries():
                moved.setdefault(s_, []).extend(np.asarray(sp).reshape(-1, 2).tolist())

    def unmoved(seq, n):
        keep = np.ones(n, bool)
        if not lay.mla:
            for b, e in moved.get(seq, []):
                keep[b:e] = False
        return keep

    # copies of every op array this variant changes
    for i, op in enumerate(ops):
        if isinstance(op, (Append, AppendBatch, Splice)):
            vf = np.clip(_bf16_f32(op.v), -FOCUS_V_CLIP, FOCUS_V_CLIP)
            kw = dict(op.__dict__)
            kw["v"] = to_bf16(vf)
            kw["k"] = op.k.copy()
            ops[i] = type(op)(**kw)
    # logical index -> (op index, row) per sequence, as the ops append tokens
    src = {}          # seq -> list of (op index, row)
    hist_ops = {}     # seq -> set of op indices that appended plain (non-stub) tokens
    last_rewrite = {} # seq -> op index of its last repos / splice
    n_seqs = 0
    dims = _low_freq_dims(lay)
    dirs = {}         # seq -> [n_dirs, len(dims)] unit vectors
    beta = float(np.sqrt(lay.d_qk))

    def key_row(seq, t):
        oi, r = src[seq][t]
        op = ops[oi]
        if lay.mla:
            kpe = op.kpe[r]
            kn = _bf16_f32(op.k[r])                       # [Hkv, d_nope]
            kp = _bf16_f32(kpe)                           # [H_pe, d_rope]
            kp = np.broadcast_to(kp, (lay.n_kv_heads, lay.d_rope)) if kp.shape[0] == 1 else kp
            return np.concatenate([kn, kp], axis=-1)
        return _bf16_f32(op.k[r])                         # [Hkv, d]

    for i, op in enumerate(ops):
        if isinstance(op, SeqCreate):
            src[n_seqs] = []
            hist_ops[n_seqs] = set()
            n_seqs += 1
        elif isinstance(op, Append):
            src[op.seq] += [(i, r) for r in range(len(op.pos))]
            hist_ops[op.seq].add(i)
        elif isinstance(op, AppendBatch):
            off = 0
            for s_, c in zip(op.seqs.tolist(), op.counts.tolist()):
                src[s_] += [(i, off + r) for r in range(c)]
                hist_ops[s_].add(i)
                off += c
        elif isinstance(op, Splice):
            src[op.seq] += [(i, r) for r in range(int(np.sum(op.stub_lens)))]
            last_rewrite[op.seq] = i
        elif isinstance(op, (Repos,)):
            last_rewrite[op.seq] = i
        elif isinstance(op, ReposBatch):
            for s_ in op.seqs.tolist():
                last_rewrite[s_] = i
        elif isinstance(op, Clone):
            raise ValueError("focus queries: workloads with clones are not supported")
        elif isinstance(op, Attention):
            q = rng.standard_normal(op.q.shape, dtype=np.float32)
            for sg in op.segments:
                if sg.q_len == 0:
                    continue
                n = len(src[sg.seq])
                hidden = np.zeros(n, bool)
                for b, e in np.asarray(sg.mask_spans).reshape(-1, 2):
                    hidden[b:e] = True
                shown = np.flatnonzero(~hidden)
                own = shown[-sg.q_len:]
                if len(own) < sg.q_len:
                    raise ValueError("focus queries: segment has fewer tokens than rows")
                if any(src[sg.seq][t][0] <= last_rewrite.get(sg.seq, -1) for t in own):
                    raise ValueError("focus queries: query tokens rewritten after their append")
                if sg.seq not in dirs:
                    # needle directions and tokens among the history before the query tokens
                    u = np.zeros((n_dirs, lay.d_qk), np.float32)
                    u[:, dims] = rng.standard_normal((n_dirs, len(dims)), dtype=np.float32)
                    u /= np.linalg.norm(u, axis=1, keepdims=True)
                    dirs[sg.seq] = u
                    keep = unmoved(sg.seq, n)
                    cand = [t for t in range(int(own[0])) if keep[t] and src[sg.seq][t][0] in hist_ops[sg.seq]]
                    m = min(len(cand), n_dirs * needles_per_dir)
                    pick = rng.choice(len(cand), size=m, replace=False) if m else []
                    for j, c in enumerate(pick):
                        oi, r = src[sg.seq][cand[c]]
                        o = ops[oi]
                        add = beta * u[j % n_dirs]
                        if lay.mla:
                            o.k[r] = to_bf16(_bf16_f32(o.k[r]) + add[None, :lay.d_nope])
                        else:
                            o.k[r] = to_bf16(_bf16_f32(o.k[r]) + add[None, :])
                u = dirs[sg.seq]
                for li, t in enumerate(own):
                    row = sg.q_begin + li
                    k_own = key_row(sg.seq, int(t))
                    k_next = key_row(sg.seq, int(t) + 1) if int(t) + 1 < n else None
                    for h in range(lay.n_q_heads):
                        g = h // G
                        sel = (li + h) % 4
                        if sel == 0:
                            tgt = k_own[g]
                        elif sel == 1 and k_next is not None:
                            tgt = k_next[g]
                        elif sel == 2:
                            tgt = u[(li // 4 + h) % n_dirs]
                        else:
                            continue
                        q[row, h] += FOCUS_GAIN * tgt / max(float(np.linalg.norm(tgt)), 1e-6)
            ops[i] = Attention(to_bf16(q), op.segments, op.scale)
    return out


CONFIGS = {
    "c1": c1_tiny, "c2": c2_64k, "c3": c3_mla, "c4": c4_batched, "c5": c5_128k, "decode": decode_batch,
    "retrigger": retrigger,
}


def make(name: str, seed: int = 0, **kw) -> Workload:
    return CONFIGS[name](seed, **kw)
