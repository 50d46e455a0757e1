"""The attention checks of the GPU parity tests can fail: mistakes planted in
the oracle's own output (on the CPU) must exceed the bars at full size.

Planted mistakes, each a plausible kernel bug:
  * one 64-key tile missing from a 64K segment's list (stress queries, and
    the base queries of N(0,1)/8 where the absolute bar alone is blind);
  * the causal limit moved by one key in either direction (focused queries);
  * one 1,536-key decode split missing from a request's list.
The planted outputs come from the oracle itself with a changed list or a
shifted query row; nothing here runs the HIP path.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle import akv_oracle as AO
from parity_check import ATOL_ATTN, RTOL_L2_ATTN, attention_errors, check_attention_rows


def _entries(ex):
    return [(int(p), o) for p, lo, hi in np.asarray(ex).reshape(-1, 3) for o in range(lo, hi)]


def _extents(entries):
    out = []
    for p, o in entries:
        if out and out[-1][0] == p and out[-1][2] == o:
            out[-1][2] = o + 1
        else:
            out.append([p, o, o + 1])
    return np.asarray(out, np.int64).reshape(-1, 3)


def _cut_list(ex, rows, seg, k0, n):
    """The page lists with entries k0 .. k0+n-1 of segment `seg` removed."""
    ex = np.asarray(ex).reshape(-1, 3)
    parts, new_rows, eb = [], [], 0
    for i, (qb, ql, b, e) in enumerate(rows):
        part = ex[b:b + e]
        if i == seg:
            ent = _entries(part)
            part = _extents(ent[:k0] + ent[k0 + n:])
        parts.append(part)
        new_rows.append((qb, ql, eb, len(part)))
        eb += len(part)
    return new_rows, np.concatenate(parts)


def _sample(att, n, seed=0):
    rng = np.random.default_rng(seed)
    return {i: np.unique(np.concatenate([rng.choice(sg.q_len, min(n, sg.q_len), replace=False),
                                         [0, sg.q_len - 1]]))
            for i, sg in enumerate(att.segments) if sg.q_len}


def _oracle_rows(wl, n_rows):
    att = [o for o in wl.ops if isinstance(o, W.Attention)][0]
    sample = _sample(att, n_rows)
    res = oracle.run_workload(wl, sample_rows=sample)
    rec = res.attention[0]
    return res.pool, att, rec, sample


@pytest.fixture(scope="module")
def c2_base():
    return _oracle_rows(W.c2_64k(0), 6)


@pytest.fixture(scope="module")
def c2_stress():
    return _oracle_rows(W.query_variant(W.c2_64k(0), "stress"), 6)


@pytest.mark.parametrize("which", ["base", "stress"])
def test_missing_tile_fails_the_check(which, c2_base, c2_stress):
    pool, att, rec, sample = c2_base if which == "base" else c2_stress
    want = rec["out"]
    q = W.bf16_to_f64(att.q)
    seg = 1
    lkv = int(sum(hi - lo for _, lo, hi in rec["extents"][rec["segments"][seg][2]:][:rec["segments"][seg][3]]))
    k0 = (lkv // 2) // 64 * 64                    # a tile in the middle of the history
    rows, ex = _cut_list(rec["extents"], rec["segments"], seg, k0, 64)
    only = {i: (sample[seg] if i == seg else np.zeros(0, np.int64)) for i in range(len(rows))}
    planted = AO.segment_attention(pool, q, rows, ex, 0.0, rows=only)
    ref = np.full_like(want, np.nan)
    r = att.segments[seg].q_begin + sample[seg]
    ref[r] = want[r]
    ea, er, _ = attention_errors(planted, ref)
    print(f"[{which}] one tile of {lkv} keys missing: max abs {ea:.2e}, max rel L2 {er:.2e}")
    assert er > 3 * RTOL_L2_ATTN
    with pytest.raises(AssertionError):
        check_attention_rows(planted, ref)
    if which == "base":
        # the absolute bar alone would not have seen it
        assert ea < ATOL_ATTN


def test_correct_rows_pass_the_check(c2_stress):
    """The oracle's output rounded to bf16 (the kernel's last rounding) passes."""
    _, _, rec, _ = c2_stress
    want = rec["out"]
    got = W.bf16_to_f64(W.to_bf16(np.nan_to_num(want).astype(np.float32)))
    got[np.isnan(want)] = np.nan
    check_attention_rows(np.nan_to_num(got), want)


@pytest.mark.parametrize("shift", [1, -1])
def test_causal_limit_off_by_one_fails_the_check(shift):
    """Focused queries: row i, head h aims at its own key ((i + h) % 4 == 0)
    or at the next, hidden one (== 1).  A kernel whose causal limit is one
    key late (or early) turns the output of those rows."""
    wl = W.query_variant(W.c2_64k(0), "focus")
    att = [o for o in wl.ops if isinstance(o, W.Attention)][0]
    seg = 2
    rows_local = np.arange(100, 140)
    only = {i: (rows_local if i == seg else np.zeros(0, np.int64)) for i in range(len(att.segments))}
    res = oracle.run_workload(wl, sample_rows=only)
    pool, rec = res.pool, res.attention[0]
    want = rec["out"]
    q = W.bf16_to_f64(att.q)
    qb = att.segments[seg].q_begin
    # row i with limit moved by `shift` = the oracle's row i + shift fed row i's query
    q2 = q.copy()
    q2[qb + rows_local + shift] = q[qb + rows_local]
    only[seg] = rows_local + shift
    moved = AO.segment_attention(pool, q2, rec["segments"], rec["extents"], 0.0, rows=only)
    planted = np.full_like(want, np.nan)
    planted[qb + rows_local] = moved[qb + rows_local + shift]
    ea, er, _ = attention_errors(planted, want)
    print(f"causal limit {shift:+d}: max abs {ea:.2e}, max rel L2 {er:.2e}")
    assert ea > 10 * ATOL_ATTN and er > 10 * RTOL_L2_ATTN
    with pytest.raises(AssertionError):
        check_attention_rows(planted, want)


def test_focused_rows_concentrate():
    """The focus variant really concentrates the softmax: a row aimed at its
    own key returns nearly that key's value row."""
    wl = W.query_variant(W.c1_tiny(0, "canonical"), "focus")
    res = oracle.run_workload(wl)
    att = [o for o in wl.ops if isinstance(o, W.Attention)][0]
    out = res.attention[0]["out"]
    rec = res.attention[0]
    ex = rec["extents"]
    qb, ql, eb, el = rec["segments"][0]
    _, v = res.pool.gather(ex[eb:eb + el])
    lkv = v.shape[0]
    G = wl.layout.n_q_heads // wl.layout.n_kv_heads
    close = []
    for i in range(0, ql, 7):
        for h in range(wl.layout.n_q_heads):
            if (i + h) % 4 == 0:
                own = v[lkv - ql + i, h // G]
                close.append(np.linalg.norm(out[qb + i, h] - own) / np.linalg.norm(own))
    assert np.median(close) < 0.05, np.median(close)
    assert np.all(np.abs(out[~np.isnan(out)]) <= W.FOCUS_V_CLIP + 1e-12)


def test_missing_decode_split_fails_the_check():
    wl = W.query_variant(W.decode_batch(3, n_req=4, ctx_lo=6000, ctx_hi=9000), "stress")
    res = oracle.run_workload(wl)
    rec = res.attention[0]
    att = [o for o in wl.ops if isinstance(o, W.Attention)][0]
    want = rec["out"]
    rows, ex = _cut_list(rec["extents"], rec["segments"], 0, 1536, 1536)
    planted = AO.segment_attention(res.pool, W.bf16_to_f64(att.q), rows, ex, 0.0)
    ea, er, _ = attention_errors(planted, want)
    print(f"decode split missing: max abs {ea:.2e}, max rel L2 {er:.2e}")
    with pytest.raises(AssertionError):
        check_attention_rows(planted, want)
