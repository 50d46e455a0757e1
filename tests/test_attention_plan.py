"""The attention planner's work list covers every visible (query row, key)
pair exactly once ([AKV-notes] section 3: one launch over all segments, each
over its own list), checked on the CPU through the dry run
akv_attention_plan on page-table-only pools.

Semantics of an item, as the kernels run it: block i takes packed rows
row0 .. row0 + rows_per_block - 1 of its segment (q_len x group rows,
token-major) and kv head, over list entries k_begin .. k_end - 1, each row
clipped to its causal limit Lkv - Lq + token.  Checked for the workload
shapes at full size, decode batches and random scripts, for 1 to 300
compute units:
  * the row tiles of every (segment, kv head) tile its rows, and the key
    ranges of each row tile tile its list, so every visible pair is covered
    once (small shapes: also by explicit enumeration of every pair);
  * a tile with one key range writes its rows directly; a split tile writes
    fp32 partials whose rows are disjoint and inside the partial buffer, and
    one combine entry merges them, split j at part0 + j * rows;
  * splits per tile stay within what the merge kernel holds (16 prefill, 64
    decode), and the row tiles of one key range share an XCD (index % 8).
"""
import numpy as np
import pytest

import workloads as W

akv = pytest.importorskip("kv_cache_drop_amd")
import os  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(akv.LIB_PATH), reason="libakv.so not built")


def _host_pool(lay):
    return akv.Pool(lay.n_q_heads, lay.n_kv_heads, lay.d_nope, lay.d_rope, lay.d_v, lay.page_size,
                    lay.num_pages, kpe_per_head=lay.kpe_per_head, pairing=lay.pairing,
                    rope_theta=lay.rope_theta, device=False)


def _host_lists(wl):
    """Replay the script on a page-table-only pool; the lists of each attention."""
    lay = wl.layout
    hp = akv.Pool(lay.n_q_heads, lay.n_kv_heads, lay.d_nope, lay.d_rope, lay.d_v, lay.page_size,
                  lay.num_pages, kpe_per_head=lay.kpe_per_head, pairing=lay.pairing,
                  rope_theta=lay.rope_theta, page_order=wl.page_order, device=False)
    launches = []
    for op in wl.ops:
        if isinstance(op, W.SeqCreate):
            hp.seq_create()
        elif isinstance(op, W.Append):
            hp.append(op.seq, op.pos)
        elif isinstance(op, W.AppendBatch):
            hp.append_batch(op.seqs, op.counts, op.pos)
        elif isinstance(op, W.Drop):
            hp.drop(op.seq, op.spans)
        elif isinstance(op, W.Repos):
            hp.repos(op.seq, op.spans, op.deltas)
        elif isinstance(op, W.ReposBatch):
            hp.repos_batch(list(op.entries()))
        elif isinstance(op, W.Splice):
            hp.splice(op.seq, op.spans, op.stub_lens)
        elif isinstance(op, W.Compact):
            hp.compact(op.seq, bool(op.force))
        elif isinstance(op, W.Clone):
            hp.clone(op.src, op.first, op.n, op.dst, op.delta)
        elif isinstance(op, W.CompactMode):
            hp.compaction_mode(op.deferred)
        elif isinstance(op, W.CompactPending):
            hp.compact_pending(op.max_tokens, op.max_seqs)
        elif isinstance(op, W.Release):
            hp.seq_release(op.seq)
        elif isinstance(op, W.Attention):
            exts, rows, eb = [], [], 0
            for sg in op.segments:
                ex = hp.visible(sg.seq, sg.mask_spans if len(sg.mask_spans) else None)
                exts.append(ex)
                rows.append((sg.q_begin, sg.q_len, eb, len(ex)))
                eb += len(ex)
            launches.append((op.q.shape[0], np.asarray(rows, np.int64).reshape(-1, 4), np.concatenate(exts)))
    return hp, launches


def _check_plan(lay, nq, rows, ex, items, comb, rb, part_rows, enumerate_pairs=False):
    G = lay.n_q_heads // lay.n_kv_heads
    Hkv = lay.n_kv_heads
    lkv = [int((ex[b:b + e, 2] - ex[b:b + e, 1]).sum()) for _, _, b, e in rows]
    decode = (lay.d_nope == 0 and lay.d_rope == 128 and lay.d_v == 128 and
              max(int(r[1]) * G for r in rows) <= 16)
    assert rb == (16 if decode else 256)
    assert len(items) % 8 == 0, "grid padded to whole XCD rounds"
    real = items[items[:, 0] >= 0]
    pad = items[items[:, 0] < 0]
    assert np.all(pad[:, 5] == -1)
    # row tiles and their key ranges
    tiles = {}
    for i, (sg, h, r0, kb, ke, part) in enumerate(items.tolist()):
        if sg < 0:
            continue
        tiles.setdefault((sg, h, r0), []).append((kb, ke, part, i))
    want_tiles = {(s, h, r0) for s, (qb, ql, _, _) in enumerate(rows.tolist()) if ql > 0
                  for h in range(Hkv) for r0 in range(0, ql * G, rb)}
    assert set(tiles) == want_tiles, "row tiles do not tile the segments' rows"
    comb_of = {}
    for c in comb.tolist():
        key = tuple(c[:3])
        assert key not in comb_of, "two combine entries for one row tile"
        comb_of[key] = c
    used = np.zeros(max(part_rows, 1), np.int32)
    groups = {}
    for (sg, h, r0), lst in tiles.items():
        lst.sort()
        n_rows = min(rb, int(rows[sg][1]) * G - r0)
        # key ranges: contiguous, from 0 to the list end
        assert lst[0][0] == 0 and lst[-1][1] == lkv[sg], (sg, h, r0, lst[0], lst[-1], lkv[sg])
        for a, b in zip(lst, lst[1:]):
            assert a[1] == b[0] and a[0] < a[1], "key ranges overlap or leave a gap"
        assert len(lst) <= (64 if decode else 16)
        if len(lst) == 1:
            assert lst[0][2] == -1 and (sg, h, r0) not in comb_of
        else:
            c = comb_of[(sg, h, r0)]
            assert c[4] == len(lst) and c[5] == n_rows
            for j, (kb, ke, part, _) in enumerate(lst):
                assert part == c[3] + j * n_rows
                assert 0 <= part and part + n_rows <= part_rows
                used[part:part + n_rows] += 1
        for kb, ke, part, i in lst:
            groups.setdefault((sg, h, kb), set()).add(i % 8)
    assert set(comb_of) <= set(tiles)
    assert np.all(used[:part_rows] <= 1), "partial rows written twice"
    assert int(used.sum()) == part_rows, "partial rows left unwritten"
    for g, xcds in groups.items():
        assert len(xcds) == 1, f"row tiles of one key range on several XCDs: {g}"
    if enumerate_pairs:
        for s, (qb, ql, _, _) in enumerate(rows.tolist()):
            if ql == 0:
                continue
            R = ql * G
            for h in range(Hkv):
                cnt = np.zeros((R, lkv[s]), np.int32)
                for r0 in range(0, R, rb):
                    for kb, ke, _, _ in tiles[(s, h, r0)]:
                        for r in range(r0, min(r0 + rb, R)):
                            lim = lkv[s] - ql + r // G
                            cnt[r, kb:min(ke, lim + 1)] += 1
                vis = np.arange(lkv[s])[None, :] <= (lkv[s] - ql + np.arange(R) // G)[:, None]
                np.testing.assert_array_equal(cnt, vis.astype(np.int32))


CASES = {
    "c1": lambda: W.c1_tiny(0, "unaligned"),
    "c2": lambda: W.c2_64k(0),
    "c3": lambda: W.c3_mla(0),
    "c4": lambda: W.c4_batched(0),
    "c5": lambda: W.c5_128k(0),
    "decode48": lambda: W.decode_batch(0),
    "decode_q2_64h": lambda: W.decode_batch(2, n_req=24, ctx_lo=1, ctx_hi=700, n_q_heads=64, q_len=2),
    "decode_long": lambda: W.decode_batch(4, n_req=3, ctx_lo=60000, ctx_hi=90000),
    "retrigger": lambda: W.retrigger(0),
}


@pytest.fixture(scope="module")
def launches():
    return {}


@pytest.mark.parametrize("name", list(CASES))
def test_plan_covers_every_pair_once(name, launches):
    wl = CASES[name]()
    hp, ls = _host_lists(wl)
    for nq, rows, ex in ls:
        for n_cu in (1, 7, 64, 256, 300):
            items, comb, rb, pr = hp.attention_plan(nq, rows, ex, n_cu)
            _check_plan(wl.layout, nq, rows, ex, items, comb, rb, pr, enumerate_pairs=(name == "c1"))


@pytest.mark.parametrize("seed", range(12))
def test_plan_random_scripts_enumerated(seed):
    """Random scripts (GQA and MLA, several sequences, masks, pages of 1 to
    256 tokens): every (row, key) pair of every segment counted."""
    mla = seed % 4 == 3
    wl = W.fuzz_small(700 + seed, mla=mla, n_seqs=3, page_size=[16, 1, 4, 64, 256, 8][seed % 6],
                      head_dims=(32, 64, 128), groups=(1, 2, 4, 8), mla_dims=(32, 32, 32))
    hp, ls = _host_lists(wl)
    assert ls
    for nq, rows, ex in ls:
        for n_cu in (1, 3, 256, 300):
            items, comb, rb, pr = hp.attention_plan(nq, rows, ex, n_cu)
            _check_plan(wl.layout, nq, rows, ex, items, comb, rb, pr, enumerate_pairs=True)


def test_plan_refuses_what_attention_refuses():
    lay = W.Layout(8, 2, 0, 64, 64, 16, 8)
    hp = _host_pool(lay)
    s = hp.seq_create()
    hp.append(s, np.arange(20))
    ex = hp.visible(s)
    for segs, lists, code in [([(0, 30, 0, len(ex))], ex, akv.AKV_EINVAL),        # Lkv < Lq
                              ([(0, 5, 0, 1)], [[99, 0, 3]], akv.AKV_ERANGE),      # page out of range
                              ([(28, 5, 0, len(ex))], ex, akv.AKV_ERANGE),         # rows beyond Q
                              ([(0, 5, 0, len(ex)), (3, 5, 0, len(ex))], ex, akv.AKV_EINVAL)]:
        with pytest.raises(akv.AkvError) as ei:
            hp.attention_plan(30, segs, lists)
        assert ei.value.status == code
    items, comb, rb, pr = hp.attention_plan(30, [(0, 0, 0, len(ex))], ex)     # no rows: nothing to run
    assert len(items) == 0 and len(comb) == 0 and pr == 0
