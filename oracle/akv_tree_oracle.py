"""Brute-force cache reuse matching (the extended radix tree's rules).

TEST INFRASTRUCTURE ONLY.  Only `tests/` may import this module; the product
(`kv_cache_drop_amd`, whose tree is C++) shares no code with it.

Sources, cited by page title and section:

  [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and State-Preserving
              Prefix Invalidation Bypass", section 3: each edge carries the
              token sequence and the ordered cache operations applied to it; a
              request matches tokens and operations together and diverges where
              the operation histories differ.
  [AKV-notes] "Cache Engineering for Agents", section 3, Cache Management and
              Cache Reuse Matching Rules: a cached node is T(x, p) (token x, the
              position p its key encodes); exact match = same tokens, same
              positions, same operation records along the path (reuse as is);
              retrigger match = same tokens and operation history, positions
              may differ (reuse after a key transform); lookup takes the longest
              exact prefix first and replaces it with a history-compatible one
              only when strictly longer; the walk stops at the first token or
              operation that differs.  Versions no running request uses are
              evicted on their own.

Readings (stated, the pages leave them open):
  * a history is a list of events (kind, a, b, c): token (id a, position b),
    drop span [a, b), repos span [a, b) by c, in the order applied;
  * a checkpoint (a registered state) can serve the prefix of its history of
    length d only when every event after d is a token: an operation after the
    prefix would have changed the prefix's tokens;
  * the retrigger transform is one shift of every position (one key rotation);
  * among candidates of equal length the checkpoint registered last wins;
    eviction takes unpinned checkpoints by least recent use (insert or match),
    then registration order.

Everything here is a direct scan over all checkpoints; no trie.
"""
from __future__ import annotations

import numpy as np

TOKEN, DROP, REPOS = 0, 1, 2


class TreeOracle:
    def __init__(self):
        self.checks = []          # dicts: hist, seq, order, stamp, pins, live
        self.clock = 0
        self.inserted = 0

    def insert(self, hist, seq: int) -> None:
        hist = np.asarray(hist, np.int64).reshape(-1, 4)
        if len(hist) == 0 or seq < 0 or any(c["live"] and c["seq"] == seq for c in self.checks):
            raise ValueError("bad checkpoint")
        self.clock += 1
        self.inserted += 1
        self.checks.append(dict(hist=hist, seq=seq, order=self.inserted, stamp=self.clock, pins=0, live=True))

    @staticmethod
    def _first_servable(hist) -> int:
        """Smallest prefix length this checkpoint serves: after its last operation."""
        ops = np.nonzero(hist[:, 0] != TOKEN)[0]
        return int(ops[-1]) + 1 if len(ops) else 1

    def match(self, req) -> dict:
        req = np.asarray(req, np.int64).reshape(-1, 4)
        ex_best, rt_best = None, None          # (depth, order, check, delta)
        for c in self.checks:
            if not c["live"]:
                continue
            h = c["hist"]
            lo = max(1, self._first_servable(h))
            # exact: events equal
            p = 0
            while p < min(len(h), len(req)) and np.array_equal(h[p], req[p]):
                p += 1
            if p >= lo:
                cand = (p, c["order"], c, 0)
                if ex_best is None or cand[:2] > ex_best[:2]:
                    ex_best = cand
            # retrigger: token ids equal under one shift, operations equal
            q, shift = 0, None
            while q < min(len(h), len(req)):
                a, b = h[q], req[q]
                if a[0] != b[0]:
                    break
                if a[0] == TOKEN:
                    if a[1] != b[1]:
                        break
                    d = int(b[2] - a[2])
                    if shift is not None and d != shift:
                        break
                    shift = d
                elif not np.array_equal(a, b):
                    break
                q += 1
            if q >= lo:
                cand = (q, c["order"], c, shift if shift is not None else 0)
                if rt_best is None or cand[:2] > rt_best[:2]:
                    rt_best = cand
        if rt_best is not None and (ex_best is None or rt_best[0] > ex_best[0]):
            best, exact = rt_best, 0
        elif ex_best is not None:
            best, exact = ex_best, 1
        else:
            return dict(seq=-1, n_events=0, n_tokens=0, exact=0, delta=0)
        depth, _, c, delta = best
        self.clock += 1
        c["stamp"] = self.clock
        n_tok = int(np.count_nonzero(c["hist"][:depth, 0] == TOKEN))
        return dict(seq=c["seq"], n_events=int(depth), n_tokens=n_tok, exact=exact, delta=int(delta) if not exact else 0)

    def pin(self, seq: int, add: int) -> None:
        for c in self.checks:
            if c["live"] and c["seq"] == seq:
                if c["pins"] + add < 0:
                    raise ValueError("unpinned more than pinned")
                c["pins"] += add
                return
        raise ValueError("not registered")

    def evict(self, max_n: int) -> list:
        cand = [c for c in self.checks if c["live"] and c["pins"] == 0]
        cand.sort(key=lambda c: (c["stamp"], c["order"]))
        out = []
        for c in cand[:max_n]:
            c["live"] = False
            out.append(c["seq"])
        return out
