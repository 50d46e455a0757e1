"""fp64 CPU oracle for AKV cache engineering over a paged KV pool.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this module.  The product package
(`kv_cache_drop_amd`) never imports it, and the two share no code: no kernels,
headers, helpers, tables or constant generators.  The only module both sides
use is `workloads`, which holds seeded input generators and no arithmetic of
the method.

Sources, cited by page title and section:

  [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and State-Preserving
              Prefix Invalidation Bypass" (A. Akhunji, technical breakdown)
  [AKV-notes] "Cache Engineering for Agents" (reading notes on Fu et al.,
              arXiv:2610.28577)
  [Leyline]   "Leyline: KV Cache Directives for Agentic Inference" (paper digest)

What is computed, and where the pages fix it:

* append / drop / repos are the three cache operations of [AKV-notes] section 1
  (Problem & Solution).  Drop marks a token span inactive without freeing or
  rewriting it; attention then skips those entries ([AKV-blog] section 2,
  "The Drop Primitive").
* repos rotates retained keys by the RoPE closure R(a)R(b) = R(a+b)
  ([AKV-blog] section 2, "The Repos Primitive and Rotary Position Embeddings";
  [Leyline] Method).  Reading adopted: signed delta, new position = pos + delta,
  new key = R(delta) key, with R(phi) = [[cos, -sin], [sin, cos]] acting on the
  pair (k_2i, k_2i+1) at angle phi = delta * theta_i and
  theta_i = base^(-2i/d_rot).  Deltas from several spans covering one token add
  ([Leyline] Method, composition of directives of either sign).
* MLA layouts rotate only K_pe; K_nope and V are left as they are ([Leyline]
  Method).
* splice is the [Leyline] AMORTIZE directive: a span is replaced by a stub and
  every downstream token moves by delta = |R| - (s_end - s_start).
* compaction copies the visible tokens into fresh dense pages when the
  fraction of wasted slots in a sequence's referenced pages exceeds 40%
  ([AKV-blog] section 7, Dilemma 2).
* segment-batch attention: the queries are split into segments; each segment
  gathers its own list of visible KV entries and runs ordinary causal attention
  over it, with no dense mask ([AKV-notes] section 3, Segment-Batch Attention;
  [AKV-blog] section 4).  The mask is bottom-right causal over list order.
* dense_masked_attention is the masked-softmax definition of [AKV-blog]
  section 2 taken literally (additive 0 / -inf mask over every token ever
  appended), used only to pin the segment oracle.

Page allocation (not described on the pages; a stated rule both sides follow):
the pool holds a FIFO free queue initialised to a caller-given page order and
a FIFO evictable queue.  Pages are taken from the free queue first, then from
the evictable queue (dropped cache is evicted first, [AKV-notes] section 3,
Cache Management).  A page enters the evictable queue when its last visible
token is dropped or moved away, unless it is the sequence's open tail page.
"""
from __future__ import annotations

from collections import deque
from typing import List, Optional, Sequence

import numpy as np

INT32_MAX = 2 ** 31 - 1
DEFAULT_COMPACT_THRESHOLD = 0.40


class OracleError(Exception):
    code = 0


class EInval(OracleError):
    code = -1


class ERange(OracleError):
    code = -2


class ENoMem(OracleError):
    code = -3


class EState(OracleError):
    code = -4


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------
def rope_inv_freq(d_rot: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_rot), i < d_rot/2 (reading of the RoPE angle
    m*theta in [AKV-blog] section 2; no frequency scaling)."""
    i = np.arange(d_rot // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d_rot)


def rotate(x: np.ndarray, delta: np.ndarray, inv_freq: np.ndarray, pairing: int) -> np.ndarray:
    """R(delta) applied to every rotation pair on the last axis of x, in fp64.

    x: [..., d_rot]; delta: shape x.shape[:-1] (or broadcastable to it).
    Pair i is (2i, 2i+1) for interleaved pairing ([AKV-blog] section 2 writes
    the update on (k_2i, k_2i+1)) or (i, i + d_rot/2) for half-split pairing.
    Each pair (a, b) becomes (a cos phi - b sin phi, a sin phi + b cos phi)
    with phi = delta * theta_i."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    phi = np.asarray(delta, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty_like(x)
    if pairing == 0:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
    else:
        h = d // 2
        a, b = x[..., :h], x[..., h:]
        out[..., :h] = a * c - b * s
        out[..., h:] = a * s + b * c
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 precision (8 significant bits, the
    exponent range of fp32), to nearest with ties to even: x = m 2^e with
    0.5 <= |m| < 1, and m 2^8 is rounded to an integer, half to even."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


# ---------------------------------------------------------------------------
# pool
# ---------------------------------------------------------------------------
class _Seq:
    def __init__(self):
        self.slot = np.zeros(0, np.int64)       # page * S + offset, -1 once its page is evicted
        self.pos = np.zeros(0, np.int64)
        self.dropped = np.zeros(0, bool)
        self.pages: List[int] = []              # owned pages in allocation order
        self.tail = -1                          # open (not yet full) page, or -1
        self.alive = True
        # shared pages: the rotation each token's stored key still owes (a
        # token reading another sequence's row owes the share's delta), and the
        # reference bookkeeping of checkpoints and their sharers
        self.lag = np.zeros(0, np.int64)
        self.id = -1
        self.frozen = False
        self.refs = 0                           # sequences holding slots in this sequence's pages
        self.zombie = False                     # released while referenced
        self.owners: dict = {}                  # owner sequence -> this sequence's tokens in its pages
        self.fvis: dict = {}                    # foreign page -> this sequence's visible tokens in it
        # token log for the dense brute force (only when keep_log)
        self.log_k: List[np.ndarray] = []
        self.log_kpe: List[np.ndarray] = []
        self.log_v: List[np.ndarray] = []
        self.log_pos: List[np.ndarray] = []

    @property
    def n(self) -> int:
        return len(self.slot)


class Pool:
    """Paged KV pool with per-sequence token tables, in fp64.

    Storage mirrors a paged layout: the rotated key part `kr[page, h, off, d_rope]`
    (all of K for GQA; K_pe for MLA, with one head when K_pe is shared),
    `kn[page, h, off, d_nope]` (MLA only) and `v[page, h, off, d_v]`.

    key_store: "fp64" keeps a rotated key exactly (the method's own values);
    "bf16" stores each key a repos, splice or clone rotates as its bfloat16
    rounding, once per call, as a pool held in bf16 does (the device pool
    holds bf16 pages; [Leyline] Limitations: the rotation is done in
    higher precision and stored)."""

    def __init__(self, layout, page_order: Optional[Sequence[int]] = None,
                 keep_log: bool = False, compact_threshold: float = DEFAULT_COMPACT_THRESHOLD,
                 inv_freq: Optional[np.ndarray] = None, key_store: str = "fp64"):
        L = layout
        self.L = L
        if key_store not in ("fp64", "bf16"):
            raise EInval("key_store must be fp64 or bf16")
        self.key_store = key_store
        S, P = L.page_size, L.num_pages
        self.S = S
        self.kr = np.zeros((P, L.n_rope_heads, S, L.d_rope))
        self.kn = np.zeros((P, L.n_kv_heads, S, L.d_nope)) if L.mla else None
        self.v = np.zeros((P, L.n_kv_heads, S, L.d_v))
        order = list(range(P)) if page_order is None else [int(p) for p in page_order]
        if sorted(order) != list(range(P)):
            raise EInval("page_order must be a permutation of the pages")
        self.free = deque(order)
        self.evictable = deque()
        self.owner = np.full(P, -1, np.int64)
        self.nvis = np.zeros(P, np.int64)
        self.filled = np.zeros(P, np.int64)
        self.in_evict = np.zeros(P, bool)
        self.seqs: List[_Seq] = []
        self.keep_log = keep_log
        self.compact_threshold = compact_threshold
        self.deferred = False           # deferred compaction: fragmented sequences wait in `queue`
        self.queue: deque = deque()
        self.inv_freq = rope_inv_freq(L.d_rope, L.rope_theta) if inv_freq is None else np.asarray(inv_freq, np.float64)

    # -- sequences -----------------------------------------------------------
    def seq_create(self) -> int:
        self.seqs.append(_Seq())
        self.seqs[-1].id = len(self.seqs) - 1
        return len(self.seqs) - 1

    def _live(self, s: int) -> _Seq:
        """A sequence a call changes: alive and not frozen."""
        q = self._seq(s)
        if q.frozen:
            raise EState(f"sequence {s} is frozen")
        return q

    def _foreign(self, q: _Seq, slot: int) -> bool:
        """The slot lies in a page another sequence allocated (a shared page)."""
        return slot >= 0 and self.owner[slot // self.S] != q.id

    def _unref(self, q: _Seq, slot: int) -> None:
        o = int(self.owner[slot // self.S])
        q.owners[o] -= 1
        if q.owners[o] == 0:
            del q.owners[o]
            so = self.seqs[o]
            so.refs -= 1
            if so.refs == 0 and so.zombie:
                self._finish_release(o)

    def _fvis_dec(self, q: _Seq, page: int) -> None:
        q.fvis[page] -= 1
        if q.fvis[page] == 0:
            del q.fvis[page]

    def _seq(self, s: int) -> _Seq:
        if not (0 <= s < len(self.seqs)):
            raise EInval(f"no sequence {s}")
        q = self.seqs[s]
        if not q.alive:
            raise EState(f"sequence {s} was released")
        return q

    def seq_release(self, s: int) -> None:
        """Return every page the sequence still owns to the back of the free
        queue, in allocation order (pages waiting in the evictable queue are
        taken out of it).  Slots it holds in other sequences' pages are given
        up; while other sequences still hold slots in its pages, those pages
        stay until the last of them lets go."""
        q = self._seq(s)
        for t in range(q.n):
            if self._foreign(q, int(q.slot[t])):
                q.slot[t] = -1
        held = list(q.owners.items())
        q.owners, q.fvis = {}, {}
        q.alive = False
        if s in self.queue:
            self.queue.remove(s)
        for o, _ in held:
            so = self.seqs[o]
            so.refs -= 1
            if so.refs == 0 and so.zombie:
                self._finish_release(o)
        if q.refs > 0:
            q.zombie = True
        else:
            self._finish_release(s)

    def _finish_release(self, s: int) -> None:
        q = self.seqs[s]
        for p in q.pages:
            if self.in_evict[p]:
                self.evictable.remove(p)
                self.in_evict[p] = False
            self.owner[p] = -1
            self.nvis[p] = 0
            self.filled[p] = 0
            self.free.append(p)
        q.pages = []
        q.tail = -1
        q.zombie = False

    # -- shared pages ([AKV-blog] section 3: copy-on-write page-table references;
    # [AKV-notes] section 3, Cache Management: re-use by key rotation) ---------------
    def freeze(self, s: int) -> None:
        """Make s a checkpoint whose rows never change (keys owing a rotation
        are turned first)."""
        q = self._seq(s)
        if q.frozen:
            return
        self.materialize(s)
        q.frozen = True
        if s in self.queue:
            self.queue.remove(s)

    def share(self, src: int, first: int, n: int, dst: int, delta: int) -> None:
        """Append the retained tokens of frozen src in [first, first+n) to dst
        at pos + delta, each holding the source token's slot and owing the
        rotation by delta; nothing is written."""
        qs = self._seq(src)
        qd = self._live(dst)
        if not qs.frozen:
            raise EState("the source of a share must be frozen")
        if n < 0:
            raise EInval("negative token count")
        if first < 0 or first + n > qs.n:
            raise ERange("share range outside the source sequence")
        t = np.arange(first, first + n, dtype=np.int64)
        t = t[~qs.dropped[t]]
        if len(t) == 0:
            return
        newpos = qs.pos[t] + int(delta)
        if np.any(newpos < 0) or np.any(newpos > INT32_MAX):
            raise ERange("shared position out of range")
        for k in t:
            slot = int(qs.slot[k])
            o = int(self.owner[slot // self.S])
            if qd.owners.get(o, 0) == 0:
                self.seqs[o].refs += 1
            qd.owners[o] = qd.owners.get(o, 0) + 1
            qd.fvis[slot // self.S] = qd.fvis.get(slot // self.S, 0) + 1
        qd.slot = np.concatenate([qd.slot, qs.slot[t]])
        qd.pos = np.concatenate([qd.pos, newpos])
        qd.dropped = np.concatenate([qd.dropped, np.zeros(len(t), bool)])
        qd.lag = np.concatenate([qd.lag, qs.lag[t] + int(delta)])

    def materialize(self, s: int) -> None:
        """Turn every visible key by what it owes: rows of s's own pages in
        place; rows in shared pages are copied, turned, into slots of s's own
        (copy on write)."""
        q = self._seq(s)
        vis = np.nonzero(~q.dropped & (q.lag != 0))[0]
        own = [int(t) for t in vis if not self._foreign(q, int(q.slot[t]))]
        cow = [int(t) for t in vis if self._foreign(q, int(q.slot[t]))]
        if cow and self._pages_needed(q, len(cow)) > self._available():
            raise ENoMem("pool exhausted")
        if own:
            self._rotate_tokens(q, np.asarray(own, np.int64), q.lag[own].astype(np.float64))
        if cow:
            S = self.S
            old = q.slot[cow].copy()
            new = self._place_existing(s, cow)
            sp, so_ = old // S, old % S
            dp, do = new // S, new % S
            rot = self.kr[sp, :, so_, :]
            self.kr[dp, :, do, :] = self._store(rotate(rot, np.broadcast_to(q.lag[cow].astype(np.float64)[:, None],
                                                                            rot.shape[:2]),
                                                       self.inv_freq, self.L.pairing))
            if self.kn is not None:
                self.kn[dp, :, do, :] = self.kn[sp, :, so_, :]
            self.v[dp, :, do, :] = self.v[sp, :, so_, :]
            for sl in old:
                self._fvis_dec(q, int(sl) // S)
                self._unref(q, int(sl))
        q.lag[vis] = 0

    def _place_existing(self, s: int, toks) -> np.ndarray:
        """New slots of s's own for existing tokens (tail page first, then
        fresh pages, as for an append)."""
        q = self.seqs[s]
        S = self.S
        out = []
        for t in toks:
            if q.tail < 0:
                q.tail = self._take_page(s)
            p = q.tail
            slot = p * S + int(self.filled[p])
            self.filled[p] += 1
            self.nvis[p] += 1
            if self.filled[p] == S:
                q.tail = -1
            q.slot[t] = slot
            out.append(slot)
        return np.asarray(out, np.int64)

    # -- allocation ------------------------------------------------------------
    def _available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _evict(self, p: int) -> None:
        o = self.seqs[self.owner[p]]
        S = self.S
        hit = (o.slot >= 0) & (o.slot // S == p)
        assert not np.any(hit & ~o.dropped), "evicting a page with visible tokens"
        o.slot[hit] = -1
        o.pages.remove(p)
        self.in_evict[p] = False

    def _take_page(self, s: int) -> int:
        if self.free:
            p = self.free.popleft()
        else:
            p = self.evictable.popleft()
            self._evict(p)
        self.owner[p] = s
        self.nvis[p] = 0
        self.filled[p] = 0
        self.seqs[s].pages.append(p)
        return p

    def _pages_needed(self, q: _Seq, n: int) -> int:
        room = self.S - self.filled[q.tail] if q.tail >= 0 else 0
        extra = max(0, n - room)
        return (extra + self.S - 1) // self.S

    def _place(self, s: int, n: int) -> np.ndarray:
        """Slots for n new tokens: fill the open tail page, then fresh pages."""
        q = self.seqs[s]
        S = self.S
        slots = np.empty(n, np.int64)
        for i in range(n):
            if q.tail < 0:
                q.tail = self._take_page(s)
            p = q.tail
            slots[i] = p * S + self.filled[p]
            self.filled[p] += 1
            self.nvis[p] += 1
            if self.filled[p] == S:
                q.tail = -1
        return slots

    # -- append (a cache operation of [AKV-notes] section 1) ---------------------
    def _check_kv(self, n: int, k, kpe, v):
        L = self.L
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        if L.mla:
            if kpe is None or k.shape != (n, L.n_kv_heads, L.d_nope):
                raise EInval("bad K_nope / K_pe")
            kpe = np.asarray(kpe, np.float64)
            if kpe.shape != (n, L.n_rope_heads, L.d_rope):
                raise EInval("bad K_pe shape")
        else:
            if kpe is not None or k.shape != (n, L.n_kv_heads, L.d_rope):
                raise EInval("bad K shape")
        if v.shape != (n, L.n_kv_heads, L.d_v):
            raise EInval("bad V shape")
        return k, kpe, v

    def append(self, s: int, pos, k, kpe, v) -> None:
        q = self._live(s)
        L = self.L
        pos = np.asarray(pos, np.int64)
        n = len(pos)
        if n == 0:
            return
        if np.any(pos < 0) or np.any(pos > INT32_MAX):
            raise ERange("position out of range")
        k, kpe, v = self._check_kv(n, k, kpe, v)
        if self._pages_needed(q, n) > self._available():
            raise ENoMem("pool exhausted")
        slots = self._place(s, n)
        pg, off = slots // self.S, slots % self.S
        if L.mla:
            self.kn[pg, :, off, :] = k
            self.kr[pg, :, off, :] = kpe
        else:
            self.kr[pg, :, off, :] = k
        self.v[pg, :, off, :] = v
        q.slot = np.concatenate([q.slot, slots])
        q.pos = np.concatenate([q.pos, pos])
        q.dropped = np.concatenate([q.dropped, np.zeros(n, bool)])
        q.lag = np.concatenate([q.lag, np.zeros(n, np.int64)])
        if self.keep_log:
            q.log_k.append(k.copy())
            q.log_kpe.append(None if kpe is None else np.asarray(kpe, np.float64).copy())
            q.log_v.append(v.copy())
            q.log_pos.append(pos.copy())

    # -- drop ([AKV-blog] section 2, The Drop Primitive) -----------------------------
    @staticmethod
    def _check_spans(spans, n) -> np.ndarray:
        sp = np.asarray(spans, np.int64).reshape(-1, 2)
        for b, e in sp:
            if b > e:
                raise EInval("span with end before begin")
            if b < 0 or e > n:
                raise ERange("span outside the sequence")
        return sp

    def _drop_tokens(self, q: _Seq, tokens) -> None:
        S = self.S
        for t in tokens:
            if q.dropped[t]:
                continue
            q.dropped[t] = True
            p = q.slot[t] // S
            if self._foreign(q, int(q.slot[t])):     # a shared token gives its slot up at once
                self._fvis_dec(q, int(p))
                self._unref(q, int(q.slot[t]))
                q.slot[t] = -1
                continue
            self.nvis[p] -= 1
            if self.nvis[p] == 0 and p != q.tail and not self.in_evict[p]:
                self.evictable.append(p)
                self.in_evict[p] = True

    def drop(self, s: int, spans, auto_compact: bool = True) -> None:
        """Mark logical spans [b, e) inactive.  Nothing is freed or rewritten;
        pages left without a visible token join the evictable queue (in the
        order their last visible token is dropped)."""
        q = self._live(s)
        sp = self._check_spans(spans, q.n)
        for b, e in sp:
            self._drop_tokens(q, range(int(b), int(e)))
        if auto_compact:
            self._auto_compact(s)

    # -- fragmentation and compaction ([AKV-blog] section 7, Dilemma 2) -----------------
    def fragmentation(self, s: int) -> float:
        """1 - visible tokens / written slots of the pages holding a visible token."""
        q = self._seq(s)
        ref = [p for p in q.pages if self.nvis[p] > 0] + list(q.fvis)
        cap = int(sum(self.filled[p] for p in ref))
        if cap == 0:
            return 0.0
        return 1.0 - int(np.count_nonzero(~q.dropped)) / cap

    def _auto_compact(self, s: int) -> None:
        """Automatic compaction is opportunistic: above the threshold it runs
        when the allocator can supply the fresh pages, else it is skipped.  In
        deferred mode the sequence joins the queue instead (once)."""
        if self.fragmentation(s) > self.compact_threshold and self.deferred:
            if s not in self.queue:
                self.queue.append(s)
            return
        if self.fragmentation(s) > self.compact_threshold:
            nv = int(np.count_nonzero(~self.seqs[s].dropped))
            if (nv + self.S - 1) // self.S <= self._available():
                self.compact(s, force=True)

    def compact(self, s: int, force: bool = True) -> None:
        """Copy every visible token, in visible-list order, into fresh pages
        taken from the allocator; the old pages join the evictable queue in
        allocation order.  Values are copied unchanged."""
        q = self._live(s)
        if not force and self.fragmentation(s) <= self.compact_threshold:
            return
        order = self.visible(s)
        nv = len(order)
        need = (nv + self.S - 1) // self.S
        if need > self._available():
            raise ENoMem("pool exhausted")
        old_pages = list(q.pages)
        dest = [self._take_page(s) for _ in range(need)]
        S = self.S
        src = q.slot[order]
        sp, so = src // S, src % S
        new = np.array([dest[i // S] * S + i % S for i in range(nv)], np.int64)
        dp, do = new // S, new % S
        self.kr[dp, :, do, :] = self.kr[sp, :, so, :]
        if self.kn is not None:
            self.kn[dp, :, do, :] = self.kn[sp, :, so, :]
        self.v[dp, :, do, :] = self.v[sp, :, so, :]
        shared = [int(x) for x in src if self._foreign(q, int(x))]
        q.slot[order] = new
        q.fvis = {}
        for x in shared:
            self._unref(q, x)
        for i, p in enumerate(dest):
            c = min(S, nv - i * S)
            self.filled[p] = c
            self.nvis[p] = c
        q.tail = dest[-1] if (need and nv % S) else -1
        for p in old_pages:
            if p in dest or self.owner[p] != s:
                continue
            self.nvis[p] = 0
            if not self.in_evict[p]:
                self.evictable.append(p)
                self.in_evict[p] = True

    # -- deferred compaction ([AKV-blog] section 7, Dilemma 2: the pass runs
    # asynchronously, in decode bubbles) ---------------------------------------
    def compaction_mode(self, deferred: bool) -> None:
        self.deferred = bool(deferred)

    def compact_pending(self, max_tokens: int, max_seqs: int = 1 << 30) -> list:
        """Walk the queue front to back: a sequence no longer above the
        threshold leaves it without a copy; the walk stops at the first one
        whose visible tokens would take the moved total past max_tokens or
        that the allocator cannot supply pages for, and after max_seqs
        compactions.  Returns the compacted sequences."""
        done, used = [], 0
        while self.queue and len(done) < max_seqs:
            s = self.queue[0]
            if self.fragmentation(s) <= self.compact_threshold:
                self.queue.popleft()
                continue
            nv = int(np.count_nonzero(~self.seqs[s].dropped))
            if used + nv > max_tokens or (nv + self.S - 1) // self.S > self._available():
                break
            self.compact(s, force=True)
            used += nv
            self.queue.popleft()
            done.append(s)
        return done

    # -- repos ([AKV-blog] section 2, The Repos Primitive; [Leyline] Method) -----
    def repos_deltas(self, s: int, spans, deltas) -> np.ndarray:
        """Per-token total delta: deltas of every span covering a retained
        token add up; dropped tokens get 0 (they are never rotated)."""
        q = self._seq(s)
        sp = self._check_spans(spans, q.n)
        dl = np.asarray(deltas, np.int64).reshape(-1)
        if len(dl) != len(sp):
            raise EInval("one delta per span")
        tot = np.zeros(q.n, np.int64)
        for (b, e), d in zip(sp, dl):
            tot[b:e] += d
        tot[q.dropped] = 0
        newpos = q.pos + tot
        if np.any(newpos < 0) or np.any(newpos > INT32_MAX):
            raise ERange("repositioned position out of range")
        return tot

    def _rotate_tokens(self, q: _Seq, tokens: np.ndarray, delta: np.ndarray) -> None:
        S = self.S
        pg, off = q.slot[tokens] // S, q.slot[tokens] % S
        cur = self.kr[pg, :, off, :]                        # [m, Hr, d_rope]
        self.kr[pg, :, off, :] = self._store(rotate(cur, np.broadcast_to(delta[:, None], cur.shape[:2]),
                                                    self.inv_freq, self.L.pairing))

    def _store(self, k: np.ndarray) -> np.ndarray:
        return round_bf16(k) if self.key_store == "bf16" else k

    def repos(self, s: int, spans, deltas) -> None:
        q = self._live(s)
        tot = self.repos_deltas(s, spans, deltas)
        t = np.nonzero(tot)[0]
        if len(t):
            shared = np.array([self._foreign(q, int(q.slot[k])) for k in t], bool)
            if np.any(~shared):
                self._rotate_tokens(q, t[~shared], tot[t[~shared]])
            q.lag[t[shared]] += tot[t[shared]]     # a shared row is not written: the token owes it
            q.pos[t] += tot[t]

    def rotated_in_place(self, s: int, tokens) -> np.ndarray:
        """Which of the tokens a repos rotates in place (not shared rows)."""
        q = self.seqs[s]
        return np.array([not self._foreign(q, int(q.slot[k])) for k in tokens], bool)

    # -- positional version ([AKV-notes] section 3, Cache Management) ------------------
    def clone(self, src: int, first: int, n: int, dst: int, delta: int) -> None:
        """Re-use a cached state at other positions (re-use by key rotation; the
        retrigger match of the cache reuse matching rules): the retained tokens
        of src with logical index in [first, first+n) are appended to dst, in
        logical order, at positions pos + delta, with their rotated key part
        turned by R(delta) and every other row copied.  src is left as it is."""
        qs = self._seq(src)
        self._live(dst)
        if n < 0:
            raise EInval("negative token count")
        if first < 0 or first + n > qs.n:
            raise ERange("clone range outside the source sequence")
        t = np.arange(first, first + n, dtype=np.int64)
        t = t[~qs.dropped[t]]
        if len(t) == 0:
            return
        newpos = qs.pos[t] + int(delta)
        if np.any(newpos < 0) or np.any(newpos > INT32_MAX):
            raise ERange("cloned position out of range")
        S = self.S
        pg, off = qs.slot[t] // S, qs.slot[t] % S
        kr = self.kr[pg, :, off, :]
        kr = self._store(rotate(kr, np.full(kr.shape[:2], float(delta)), self.inv_freq, self.L.pairing))
        v = self.v[pg, :, off, :].copy()
        lag = qs.lag[t].copy()
        if self.L.mla:
            self.append(dst, newpos, self.kn[pg, :, off, :].copy(), kr, v)
        else:
            self.append(dst, newpos, kr, None, v)
        qd = self.seqs[dst]
        qd.lag[qd.n - len(t):] = lag      # the copies owe what their sources owe

    # -- splice ([Leyline] Method, AMORTIZE mode) ---------------------------------------
    def splice_plan(self, s: int, spans, stub_lens):
        """Validate a batch of splices given in visible-list coordinates and
        return (visible list, per-splice delta, stub positions, per-visible-
        entry downstream delta)."""
        q = self._seq(s)
        vis = self.visible(s)
        H = len(vis)
        sp = np.asarray(spans, np.int64).reshape(-1, 2)
        st = np.asarray(stub_lens, np.int64).reshape(-1)
        if len(st) != len(sp):
            raise EInval("one stub length per splice")
        prev_e = 0
        for j, (b, e) in enumerate(sp):
            if b >= e or st[j] < 0:
                raise EInval("empty splice span or negative stub")
            if b < 0 or e > H:
                raise ERange("splice span outside the visible list")
            if j and b < prev_e:
                raise EInval("splice spans must be sorted and disjoint")
            prev_e = e
        dj = st - (sp[:, 1] - sp[:, 0])                     # delta = |R| - (s_end - s_start)
        down = np.zeros(H, np.int64)
        for (b, e), d in zip(sp, dj):
            down[e:] += d
        stub_pos = []
        for j, (b, e) in enumerate(sp):
            p0 = q.pos[vis[b]] + int(dj[:j].sum())
            stub_pos.append(np.arange(p0, p0 + st[j], dtype=np.int64))
        stub_pos = np.concatenate(stub_pos) if stub_pos else np.zeros(0, np.int64)
        newpos = q.pos[vis] + down
        if np.any(newpos < 0) or np.any(newpos > INT32_MAX) or np.any(stub_pos < 0) or np.any(stub_pos > INT32_MAX):
            raise ERange("splice moves a position out of range")
        return vis, dj, stub_pos, down

    def splice(self, s: int, spans, stub_lens, k, kpe, v) -> np.ndarray:
        """Drop each span, append its stub at the span's start position, and
        move every downstream visible token by the summed deltas of the
        splices before it (one rotation per token).  Returns stub positions."""
        q = self._live(s)
        vis, dj, stub_pos, down = self.splice_plan(s, spans, stub_lens)
        sp = np.asarray(spans, np.int64).reshape(-1, 2)
        n_stub = len(stub_pos)
        self._check_kv(n_stub, k, kpe, v)
        # stub pages must be available once the spans are dropped (dropped pages
        # may be evicted for the stub): count before mutating anything
        drop_tokens = np.concatenate([vis[b:e] for b, e in sp]) if len(sp) else np.zeros(0, np.int64)
        freed = self._evictable_after_drop(q, drop_tokens)
        if self._pages_needed(q, n_stub) > self._available() + freed:
            raise ENoMem("pool exhausted")
        self._drop_tokens(q, drop_tokens)
        if n_stub:
            self.append(s, stub_pos, k, kpe, v)
        moved = np.nonzero(down)[0]
        keep = np.ones(len(vis), bool)
        keep[np.isin(vis, drop_tokens)] = False
        moved = moved[keep[moved]]
        if len(moved):
            t = vis[moved]
            d = down[moved]
            shared = np.array([self._foreign(q, int(q.slot[k])) for k in t], bool)
            if np.any(~shared):
                self._rotate_tokens(q, t[~shared], d[~shared])
            q.lag[t[shared]] += d[shared]
            q.pos[t] += d
        self._auto_compact(s)
        return stub_pos

    def _evictable_after_drop(self, q: _Seq, tokens) -> int:
        nv = self.nvis.copy()
        cnt = 0
        seen = set()
        for t in tokens:
            if q.dropped[t] or t in seen:
                continue
            seen.add(t)
            p = q.slot[t] // self.S
            nv[p] -= 1
            if nv[p] == 0 and p != q.tail and not self.in_evict[p]:
                cnt += 1
        return cnt

    # -- visibility ------------------------------------------------------------------
    def visible(self, s: int, mask_spans=None) -> np.ndarray:
        """Retained tokens (minus optional per-segment mask spans), ordered by
        (position, logical index)."""
        q = self._seq(s)
        keep = ~q.dropped.copy()
        if mask_spans is not None:
            for b, e in self._check_spans(mask_spans, q.n):
                keep[b:e] = False
        t = np.nonzero(keep)[0]
        order = np.lexsort((t, q.pos[t]))
        return t[order]

    def extents(self, s: int, mask_spans=None) -> np.ndarray:
        """Page-table image of the visible list: maximal runs (page, lo, hi) of
        consecutive offsets of one page, in list order."""
        q = self.seqs[s]
        vis = self.visible(s, mask_spans)
        out = []
        S = self.S
        for t in vis:
            p, o = int(q.slot[t] // S), int(q.slot[t] % S)
            if out and out[-1][0] == p and out[-1][2] == o:
                out[-1][2] = o + 1
            else:
                out.append([p, o, o + 1])
        return np.asarray(out, np.int64).reshape(-1, 3)

    # -- gathers -----------------------------------------------------------------------
    def visible_lag(self, s: int, mask_spans=None) -> np.ndarray:
        """The rotation each entry of the visible list still owes, in list order."""
        return self.seqs[s].lag[self.visible(s, mask_spans)]

    def gather(self, extents, lag=None):
        """K (d_qk = d_nope + d_rope per head) and V rows of an extent list,
        in list order: K [L, Hkv, d_qk], V [L, Hkv, d_v].  lag (optional, one
        per entry): the rotation each stored key still owes, applied here (the
        key as attention sees it; stored once in bf16 with key_store bf16)."""
        L = self.L
        ex = np.asarray(extents, np.int64).reshape(-1, 3)
        pg = np.concatenate([np.full(h - l, p) for p, l, h in ex]) if len(ex) else np.zeros(0, np.int64)
        of = np.concatenate([np.arange(l, h) for p, l, h in ex]) if len(ex) else np.zeros(0, np.int64)
        kr = self.kr[pg, :, of, :]
        if lag is not None and np.any(np.asarray(lag) != 0):
            lag = np.asarray(lag, np.float64)
            turned = self._store(rotate(kr, np.broadcast_to(lag[:, None], kr.shape[:2]), self.inv_freq, L.pairing))
            kr = np.where((lag != 0)[:, None, None], turned, kr)
        if L.mla:
            kn = self.kn[pg, :, of, :]
            kr = np.broadcast_to(kr, (len(pg), L.n_kv_heads, L.d_rope))
            k = np.concatenate([kn, kr], axis=-1)
        else:
            k = kr
        return k, self.v[pg, :, of, :]


# ---------------------------------------------------------------------------
# segment-batch attention ([AKV-notes] section 3; [AKV-blog] section 4)
# ---------------------------------------------------------------------------
def check_extents(pool: Pool, extents) -> np.ndarray:
    ex = np.asarray(extents, np.int64).reshape(-1, 3)
    for p, lo, hi in ex:
        if not (0 <= p < pool.L.num_pages) or not (0 <= lo < hi <= pool.S):
            raise ERange("extent outside the pool")
    return ex


def last_visible(lkv: int, lq: int, i: np.ndarray) -> np.ndarray:
    """Last list index query i may attend to: the segment's own Lq entries are
    the tail of its list, so causality is bottom-right over list order."""
    return lkv - lq + i


def segment_attention(pool: Pool, q: np.ndarray, segments, page_lists, scale: float = 0.0,
                      rows: Optional[dict] = None, heads=None, lags=None) -> np.ndarray:
    """Causal attention of each query segment over its own KV list.

    q: [Nq, Hq, d_qk] fp64.  segments: iterable of (q_begin, q_len, ext_begin,
    ext_len).  page_lists: [n_ext, 3] extents.  Query i of a segment with Lq
    queries and Lkv list entries sees list entries 0 .. Lkv - Lq + i.  Query
    head h reads kv head floor(h * Hkv / Hq).  Returns [Nq, Hq, d_v] with NaN
    in rows no segment covers.  `rows` optionally maps a segment index to the
    local query rows to evaluate (sampling); `heads` optionally lists the q
    heads to evaluate (the others stay NaN); `lags` optionally gives every
    list entry's owed rotation (concatenated over segments in list order)."""
    L = pool.L
    q = np.asarray(q, np.float64)
    nq = q.shape[0]
    if scale == 0.0:
        scale = 1.0 / np.sqrt(L.d_qk)
    ex_all = check_extents(pool, page_lists)
    out = np.full((nq, L.n_q_heads, L.d_v), np.nan)
    grp = L.n_q_heads // L.n_kv_heads
    for si, (qb, ql, eb, el) in enumerate(segments):
        if ql == 0:
            continue
        seg_lag = None
        if lags is not None:
            off = int(sum((ex_all[:eb, 2] - ex_all[:eb, 1]).tolist()))
            n_e = int((ex_all[eb:eb + el, 2] - ex_all[eb:eb + el, 1]).sum())
            seg_lag = np.asarray(lags)[off:off + n_e]
        k, v = pool.gather(ex_all[eb:eb + el], seg_lag)
        lkv = k.shape[0]
        if lkv < ql:
            raise EInval("segment has fewer KV entries than queries")
        loc = np.arange(ql) if rows is None or si not in rows else np.asarray(rows[si])
        lim = last_visible(lkv, ql, loc)
        for h in (range(L.n_q_heads) if heads is None else heads):
            g = h // grp
            s = (q[qb + loc, h, :] @ k[:, g, :].T) * scale
            s[np.arange(lkv)[None, :] > lim[:, None]] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[qb + loc, h, :] = p @ v[:, g, :]
    return out


def page_mass(pool: Pool, q: np.ndarray, segments, page_lists, scale: float = 0.0, lags=None) -> np.ndarray:
    """Attention weight per page: the statistic the server-side drop policy
    of [AKV-blog] section 7 (Dilemma 1) watches, the cumulative attention
    weight of each block of the history.  For every segment, query row and
    q head, the softmax weights over the segment's list (as in
    segment_attention) are added to the page of each list entry; the result
    is summed over rows, heads and segments ([num_pages], fp64)."""
    L = pool.L
    q = np.asarray(q, np.float64)
    if scale == 0.0:
        scale = 1.0 / np.sqrt(L.d_qk)
    ex_all = check_extents(pool, page_lists)
    mass = np.zeros(L.num_pages)
    grp = L.n_q_heads // L.n_kv_heads
    for qb, ql, eb, el in segments:
        if ql == 0:
            continue
        ex = ex_all[eb:eb + el]
        seg_lag = None
        if lags is not None:
            off = int(sum((ex_all[:eb, 2] - ex_all[:eb, 1]).tolist()))
            n_e = int((ex[:, 2] - ex[:, 1]).sum())
            seg_lag = np.asarray(lags)[off:off + n_e]
        k, _ = pool.gather(ex, seg_lag)
        lkv = k.shape[0]
        if lkv < ql:
            raise EInval("segment has fewer KV entries than queries")
        page_of = np.repeat(ex[:, 0], ex[:, 2] - ex[:, 1])      # the page of every list entry
        lim = last_visible(lkv, ql, np.arange(ql))
        w = np.zeros(lkv)
        for h in range(L.n_q_heads):
            s = (q[qb:qb + ql, h, :] @ k[:, h // grp, :].T) * scale
            s[np.arange(lkv)[None, :] > lim[:, None]] = -np.inf
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            w += p.sum(axis=0)
        np.add.at(mass, page_of, w)
    return mass


# ---------------------------------------------------------------------------
# dense brute force: the masked-softmax definition of [AKV-blog] section 2
# ---------------------------------------------------------------------------
def _rope_complex(x: np.ndarray, delta: np.ndarray, inv_freq: np.ndarray, pairing: int) -> np.ndarray:
    """Rotation written as complex multiplication: pair (a, b) -> a + ib,
    times exp(i * delta * theta_i).  A second formulation of the rotation, so
    the brute force does not reuse `rotate`."""
    d = x.shape[-1]
    if pairing == 0:
        z = x[..., 0::2] + 1j * x[..., 1::2]
    else:
        z = x[..., : d // 2] + 1j * x[..., d // 2:]
    z = z * np.exp(1j * np.asarray(delta, np.float64)[..., None] * inv_freq)
    out = np.empty_like(x)
    if pairing == 0:
        out[..., 0::2], out[..., 1::2] = z.real, z.imag
    else:
        out[..., : d // 2], out[..., d // 2:] = z.real, z.imag
    return out


def dense_masked_attention(pool: Pool, q: np.ndarray, seg_seq: int, q_rows, q_pos,
                           mask_spans=None, scale: float = 0.0) -> np.ndarray:
    """softmax(Q K^T * scale + M) V over every token ever appended to any
    sequence of the pool, with M = 0 where the key belongs to the query's
    sequence, is not dropped, is not hidden by the segment's mask spans and
    has position <= the query's position, and M = -inf elsewhere.

    Key values come from the append log and are moved to their current
    position by complex rotation by (current position - appended position);
    the pool's pages, extents and repos code are not used.  Needs keep_log."""
    L = pool.L
    assert pool.keep_log, "dense_masked_attention needs Pool(keep_log=True)"
    if scale == 0.0:
        scale = 1.0 / np.sqrt(L.d_qk)
    ks, vs, allowed_parts = [], [], []
    for si, sq in enumerate(pool.seqs):
        if not sq.log_pos:
            continue
        pos0 = np.concatenate(sq.log_pos)
        shift = sq.pos - pos0
        if L.mla:
            kn = np.concatenate(sq.log_k)
            kpe = _rope_complex(np.concatenate(sq.log_kpe), shift[:, None], pool.inv_freq, L.pairing)
            kpe = np.broadcast_to(kpe, (len(pos0), L.n_kv_heads, L.d_rope))
            k = np.concatenate([kn, kpe], axis=-1)
        else:
            k = _rope_complex(np.concatenate(sq.log_k), shift[:, None], pool.inv_freq, L.pairing)
        ks.append(k)
        vs.append(np.concatenate(sq.log_v))
        ok = np.zeros(len(pos0), bool)
        if si == seg_seq and sq.alive:
            ok = ~sq.dropped.copy()
            if mask_spans is not None:
                for b, e in np.asarray(mask_spans, np.int64).reshape(-1, 2):
                    ok[b:e] = False
        allowed_parts.append((ok, sq.pos.copy()))
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    ok = np.concatenate([a for a, _ in allowed_parts])
    kpos = np.concatenate([p for _, p in allowed_parts])
    q = np.asarray(q, np.float64)
    q_rows = np.asarray(q_rows)
    q_pos = np.asarray(q_pos, np.int64)
    grp = L.n_q_heads // L.n_kv_heads
    out = np.zeros((len(q_rows), L.n_q_heads, L.d_v))
    M = np.where(ok[None, :] & (kpos[None, :] <= q_pos[:, None]), 0.0, -np.inf)
    for h in range(L.n_q_heads):
        g = h // grp
        s = (q[q_rows, h, :] @ K[:, g, :].T) * scale + M
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, h, :] = (p / p.sum(axis=1, keepdims=True)) @ V[:, g, :]
    return out
