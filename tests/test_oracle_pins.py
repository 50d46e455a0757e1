"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: worked
examples printed on the pages (tests/golden/), the rotation matrix as printed,
closed forms of the rotation group, a literal dense masked-softmax brute force,
and torch's scaled_dot_product_attention for the cases that reduce to it.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import akv_oracle as AO

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _lay(**kw):
    base = dict(n_q_heads=4, n_kv_heads=2, d_nope=0, d_rope=16, d_v=16, page_size=16, num_pages=64)
    base.update(kw)
    return W.Layout(**base)


def _fill(pool, seq, n, rng, pos0=0):
    L = pool.L
    pos = np.arange(pos0, pos0 + n)
    if L.mla:
        k = rng.standard_normal((n, L.n_kv_heads, L.d_nope))
        kpe = rng.standard_normal((n, L.n_rope_heads, L.d_rope))
    else:
        k = rng.standard_normal((n, L.n_kv_heads, L.d_rope))
        kpe = None
    v = rng.standard_normal((n, L.n_kv_heads, L.d_v))
    pool.append(seq, pos, k, kpe, v)
    return k, kpe, v


# ---------------------------------------------------------------------------
# rotation matrix exactly as printed: R_{Theta,m} = [[cos m t, -sin m t], [sin m t, cos m t]]
# ("AKV: Cache Engineering for Autonomous Agents ...", section 2, The Repos Primitive)
# ---------------------------------------------------------------------------
def _rope_by_matrix(x, m, base, pairing):
    """Apply R_{Theta,m} built as explicit 2x2 matrices, one per pair."""
    d = x.shape[-1]
    th = np.array([base ** (-2.0 * i / d) for i in range(d // 2)])
    out = np.empty_like(x)
    for i in range(d // 2):
        a = m * th[i]
        R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
        ia, ib = (2 * i, 2 * i + 1) if pairing == 0 else (i, i + d // 2)
        pair = np.stack([x[..., ia], x[..., ib]], axis=-1)          # [..., 2]
        rot = pair @ R.T
        out[..., ia], out[..., ib] = rot[..., 0], rot[..., 1]
    return out


@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_repos_equals_fresh_rope_at_new_position(pairing, base):
    """Keys RoPE'd at m, then repositioned by delta, equal raw keys RoPE'd at
    m + delta (closure R(m+delta) = R(delta) R(m))."""
    rng = np.random.default_rng(1)
    d, n = 32, 200
    lay = _lay(d_rope=d, d_v=8, n_q_heads=2, n_kv_heads=1, pairing=pairing, rope_theta=base, num_pages=32)
    raw = rng.standard_normal((n, 1, d))
    m = np.arange(n, dtype=np.float64) * 37.0 + 2000.0
    pool = AO.Pool(lay)
    s = pool.seq_create()
    pool.append(s, m.astype(np.int64), _rope_by_matrix(raw, m[:, None], base, pairing), None,
                rng.standard_normal((n, 1, 8)))
    spans = np.array([[0, 120], [50, 200]])
    deltas = np.array([-1234, 60001])
    pool.repos(s, spans, deltas)
    tot = np.zeros(n)
    tot[0:120] += -1234
    tot[50:200] += 60001
    want = _rope_by_matrix(raw, (m + tot)[:, None], base, pairing)
    got, _ = pool.gather(pool.extents(s))
    order = pool.visible(s)
    np.testing.assert_allclose(got, want[order], rtol=0, atol=1e-9)
    np.testing.assert_array_equal(pool.seqs[s].pos, (m + tot).astype(np.int64))


def test_rotation_closure_either_sign_and_inverse():
    rng = np.random.default_rng(2)
    th = AO.rope_inv_freq(64, 10000.0)
    x = rng.standard_normal((500, 3, 64))
    a = rng.integers(-2 ** 17, 2 ** 17, size=(500, 3))
    b = rng.integers(-2 ** 17, 2 ** 17, size=(500, 3))
    for pairing in (0, 1):
        ab = AO.rotate(AO.rotate(x, a, th, pairing), b, th, pairing)
        np.testing.assert_allclose(ab, AO.rotate(x, a + b, th, pairing), atol=1e-9, rtol=0)
        back = AO.rotate(AO.rotate(x, a, th, pairing), -a, th, pairing)
        np.testing.assert_allclose(back, x, atol=1e-12, rtol=0)
        # orthogonal: every pair keeps its norm
        y = AO.rotate(x, a, th, pairing)
        if pairing == 0:
            n0, n1 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2, y[..., 0::2] ** 2 + y[..., 1::2] ** 2
        else:
            n0, n1 = x[..., :32] ** 2 + x[..., 32:] ** 2, y[..., :32] ** 2 + y[..., 32:] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # delta 0 is the identity, bit for bit
    np.testing.assert_array_equal(AO.rotate(x, np.zeros((500, 3)), th, 0), x)


def test_repos_sequential_equals_summed_and_skips_dropped():
    rng = np.random.default_rng(3)
    lay = _lay(num_pages=40)
    p1, p2 = AO.Pool(lay), AO.Pool(lay)
    for p in (p1, p2):
        p.seq_create()
    r1, r2 = np.random.default_rng(9), np.random.default_rng(9)
    _fill(p1, 0, 300, r1, pos0=100000)
    _fill(p2, 0, 300, r2, pos0=100000)
    for p in (p1, p2):
        p.drop(0, [[10, 30]], auto_compact=False)
    p1.repos(0, [[0, 200]], [-777])
    p1.repos(0, [[100, 300]], [4000])
    p2.repos(0, [[0, 200], [100, 300]], [-777, 4000])
    np.testing.assert_array_equal(p1.seqs[0].pos, p2.seqs[0].pos)
    np.testing.assert_allclose(p1.kr, p2.kr, atol=1e-9, rtol=0)
    # dropped tokens keep their position and are not rotated
    assert np.all(p2.seqs[0].pos[10:30] == 100000 + np.arange(10, 30))


# ---------------------------------------------------------------------------
# bf16 storage of rotated keys (the pool is bf16): round to nearest, ties to even
# ---------------------------------------------------------------------------
def _bf16_by_bits(x):
    """Nearest bfloat16 by enumeration: the bf16 numbers are the float32
    numbers whose low 16 bits are zero; take the three such numbers around
    float32(x) (its upper 16 bits, one step below, one above), keep the
    nearest to x in fp64, and on a tie the one whose last kept bit is 0."""
    x = np.asarray(x, np.float64)
    hi = (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.int64)
    best = np.full(x.shape, np.nan)
    bd = np.full(x.shape, np.inf)
    bodd = np.ones(x.shape, bool)
    for k in (-1, 0, 1):
        c = ((hi + k) & 0xFFFF).astype(np.uint32) << 16
        v = c.view(np.float32).astype(np.float64)
        d = np.abs(v - x)
        odd = ((hi + k) & 1).astype(bool)
        take = (d < bd) | ((d == bd) & bodd & ~odd)
        best = np.where(take, v, best)
        bd = np.where(take, d, bd)
        bodd = np.where(take, odd, bodd)
    return best


def test_round_bf16_nearest_even():
    rng = np.random.default_rng(12)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))
    np.testing.assert_array_equal(AO.round_bf16(x), _bf16_by_bits(x))
    # exact ties go to the even neighbour
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), (1.5 + 2.0 ** -8) * 2.0 ** -9])
    np.testing.assert_array_equal(AO.round_bf16(ties), [1.0, 1 + 2.0 ** -6, -1.0, 1.5 * 2.0 ** -9])
    np.testing.assert_array_equal(AO.round_bf16(np.array([0.0, -0.0, 1.0, 2.0 ** -100])), [0.0, 0.0, 1.0, 2.0 ** -100])


def test_bf16_key_store_rounds_each_call():
    """A bf16 pool stores each rotated key as the bf16 rounding of its exact
    rotation, once per repos or clone call, from the key as stored before the
    call; values and unrotated keys are kept as appended."""
    rng = np.random.default_rng(13)
    d, n, base = 32, 120, 10000.0
    lay = _lay(d_rope=d, d_v=8, n_q_heads=2, n_kv_heads=1, rope_theta=base, num_pages=40)
    raw = AO.round_bf16(rng.standard_normal((n, 1, d)))
    v = AO.round_bf16(rng.standard_normal((n, 1, 8)))
    m = np.arange(n) + 500
    pool = AO.Pool(lay, key_store="bf16")
    s = pool.seq_create()
    pool.append(s, m, raw, None, v)
    pool.repos(s, [[20, 120]], [-333])
    pool.repos(s, [[60, 120]], [71])
    t = pool.seqs[s]
    d1 = np.zeros(n); d1[20:] = -333
    d2 = np.zeros(n); d2[60:] = 71
    step1 = np.where((d1 != 0)[:, None, None], _bf16_by_bits(_rope_by_matrix(raw, d1[:, None], base, 0)), raw)
    want = np.where((d2 != 0)[:, None, None], _bf16_by_bits(_rope_by_matrix(step1, d2[:, None], base, 0)), step1)
    got = pool.kr[t.slot // 16, :, t.slot % 16, :]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * np.abs(want).max())
    np.testing.assert_array_equal(got[:20], raw[:20])
    np.testing.assert_array_equal(pool.v[t.slot // 16, :, t.slot % 16, :], v)
    # clone: one rounding of R(delta) applied to the stored source key
    s2 = pool.seq_create()
    pool.clone(s, 0, n, s2, 1000)
    t2 = pool.seqs[s2]
    np.testing.assert_allclose(pool.kr[t2.slot // 16, :, t2.slot % 16, :],
                               _bf16_by_bits(_rope_by_matrix(want, np.full((n, 1), 1000.0), base, 0)),
                               rtol=0, atol=1e-12 * np.abs(want).max())
    # the exact store keeps the exact rotation
    exact = AO.Pool(lay)
    exact.seq_create()
    exact.append(0, m, raw, None, v)
    exact.repos(0, [[20, 120]], [-333])
    te = exact.seqs[0]
    np.testing.assert_allclose(exact.kr[te.slot // 16, :, te.slot % 16, :],
                               np.where((d1 != 0)[:, None, None], _rope_by_matrix(raw, d1[:, None], base, 0), raw),
                               rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# positional versions ("Cache Engineering for Agents", section 3, Cache
# Management: re-use by key rotation; the retrigger match rule)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("base", [10000.0, 500000.0])
def test_clone_equals_fresh_rope_at_shifted_position(pairing, base):
    """Keys RoPE'd at m, cloned with delta, equal the raw keys RoPE'd at
    m + delta (explicit 2x2 matrices); V is copied, dropped tokens are
    skipped, and the source keeps its own version unchanged."""
    rng = np.random.default_rng(11)
    d, n = 32, 150
    lay = _lay(d_rope=d, d_v=8, n_q_heads=4, n_kv_heads=2, pairing=pairing, rope_theta=base, num_pages=40)
    raw = rng.standard_normal((n, 2, d))
    m = np.arange(n, dtype=np.float64) * 11.0 + 900.0
    v = rng.standard_normal((n, 2, 8))
    pool = AO.Pool(lay)
    a, b = pool.seq_create(), pool.seq_create()
    pool.append(a, m.astype(np.int64), _rope_by_matrix(raw, m[:, None, None], base, pairing), None, v)
    pool.drop(a, [[20, 35], [90, 91]], auto_compact=False)
    kr0, v0 = pool.kr.copy(), pool.v.copy()
    delta = -777
    pool.clone(a, 10, 120, b, delta)
    keep = np.array([t for t in range(10, 130) if not (20 <= t < 35 or t == 90)])
    qb = pool.seqs[b]
    np.testing.assert_array_equal(qb.pos, (m[keep] + delta).astype(np.int64))
    S = lay.page_size
    pg, off = qb.slot // S, qb.slot % S
    want = _rope_by_matrix(raw[keep], (m[keep] + delta)[:, None, None], base, pairing)
    np.testing.assert_allclose(pool.kr[pg, :, off, :], want, rtol=0, atol=1e-9)
    np.testing.assert_array_equal(pool.v[pg, :, off, :], v[keep])
    qa = pool.seqs[a]
    pa, oa = qa.slot // S, qa.slot % S
    np.testing.assert_array_equal(pool.kr[pa, :, oa, :], kr0[pa, :, oa, :])
    np.testing.assert_array_equal(pool.v[pa, :, oa, :], v0[pa, :, oa, :])


def test_clone_round_trip_zero_delta_and_mla_parts():
    rng = np.random.default_rng(12)
    lay = _lay(d_nope=16, d_rope=16, d_v=16, n_q_heads=4, n_kv_heads=4, page_size=8, num_pages=80)
    pool = AO.Pool(lay)
    a, b, c, z = (pool.seq_create() for _ in range(4))
    k, kpe, v = _fill(pool, a, 100, rng, pos0=5000)
    pool.clone(a, 0, 100, b, 4321)
    pool.clone(b, 0, 100, c, -4321)                  # R(-d) R(d) = I
    pool.clone(a, 0, 100, z, 0)                      # delta 0: a copy
    S = lay.page_size
    def rows(s):
        q = pool.seqs[s]
        return pool.kr[q.slot // S, :, q.slot % S, :], pool.kn[q.slot // S, :, q.slot % S, :], \
            pool.v[q.slot // S, :, q.slot % S, :]
    ra, rc, rz = rows(a), rows(c), rows(z)
    np.testing.assert_allclose(rc[0], ra[0], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(rz[0], ra[0])
    for r in (rc, rz, rows(b)):
        np.testing.assert_array_equal(r[1], kn := ra[1])       # K_nope carries no position
        np.testing.assert_array_equal(r[2], ra[2])
    assert kn.shape == (100, 4, 16)
    # the shared K_pe head of b is turned: pair norms are kept, values are not
    rb = rows(b)
    assert rb[0].shape == (100, 1, 16)
    nb = rb[0][..., 0::2] ** 2 + rb[0][..., 1::2] ** 2
    na = ra[0][..., 0::2] ** 2 + ra[0][..., 1::2] ** 2
    np.testing.assert_allclose(nb, na, rtol=1e-12)
    assert np.abs(rb[0] - ra[0]).max() > 0.1
    np.testing.assert_array_equal(pool.seqs[c].pos, pool.seqs[a].pos)


def test_clone_places_like_append_and_refusals_are_atomic():
    rng = np.random.default_rng(13)
    lay = _lay(num_pages=21, page_size=4)
    order = rng.permutation(21)
    p1, p2 = AO.Pool(lay, order), AO.Pool(lay, order)
    for p in (p1, p2):
        p.seq_create(), p.seq_create()
    r1, r2 = np.random.default_rng(3), np.random.default_rng(3)
    _fill(p1, 0, 40, r1)
    _fill(p2, 0, 40, r2)
    _fill(p1, 1, 3, r1, pos0=7)
    _fill(p2, 1, 3, r2, pos0=7)
    for p in (p1, p2):
        p.drop(0, [[0, 12]], auto_compact=False)      # pages 0..2 of seq 0 become evictable
    p1.clone(0, 0, 40, 1, 100)
    z = np.zeros((28, 2, 16))
    p2.append(1, np.arange(12, 40) + 100, z, None, z)
    np.testing.assert_array_equal(p1.seqs[1].slot, p2.seqs[1].slot)
    assert list(p1.free) == list(p2.free) and list(p1.evictable) == list(p2.evictable)
    snap = (p1.seqs[1].slot.copy(), list(p1.free), list(p1.evictable), p1.kr.copy())
    for args, exc in [((0, 0, 41, 1, 0), AO.ERange), ((0, 0, 40, 1, -113), AO.ERange),
                      ((0, 5, -1, 1, 0), AO.EInval), ((0, 0, 40, 1, 0), AO.ENoMem)]:
        with pytest.raises(exc):
            p1.clone(*args)
        assert np.array_equal(p1.seqs[1].slot, snap[0]) and list(p1.free) == snap[1]
        assert list(p1.evictable) == snap[2] and np.array_equal(p1.kr, snap[3])


# ---------------------------------------------------------------------------
# shared pages ("Cache Engineering for Agents", section 3: copy-on-write
# page-table references; "Cache Engineering for Autonomous Agents", section 3,
# Cache Management: re-use by key rotation)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("pairing", [0, 1])
def test_share_reads_as_fresh_rope_and_copy_on_write(pairing):
    """A frozen checkpoint shared at delta, then repositioned in part, reads
    (gathered keys, attention) as the raw keys RoPE'd at the new positions
    (explicit 2x2 matrices); nothing is written until materialize, which
    copies into the sharer's own pages and leaves the source's rows as they
    were."""
    rng = np.random.default_rng(21)
    base, d, n = 10000.0, 32, 120
    lay = _lay(d_rope=d, d_v=8, n_q_heads=4, n_kv_heads=2, pairing=pairing, rope_theta=base, num_pages=40, page_size=8)
    raw = rng.standard_normal((n, 2, d))
    m = np.arange(n, dtype=np.float64) * 3.0 + 50.0
    v = rng.standard_normal((n, 2, 8))
    pool = AO.Pool(lay)
    a, b = pool.seq_create(), pool.seq_create()
    pool.append(a, m.astype(np.int64), _rope_by_matrix(raw, m[:, None, None], base, pairing), None, v)
    pool.drop(a, [[40, 50]], auto_compact=False)
    pool.freeze(a)
    kr0, v0, free0 = pool.kr.copy(), pool.v.copy(), list(pool.free)
    pool.share(a, 20, 100, b, 999)
    assert np.array_equal(pool.kr, kr0) and list(pool.free) == free0, "share wrote or allocated"
    keep = np.array([t for t in range(20, 120) if not 40 <= t < 50])
    qb = pool.seqs[b]
    np.testing.assert_array_equal(qb.slot, pool.seqs[a].slot[keep])
    pool.repos(b, [[30, 90]], [-12])
    newpos = m[keep] + 999
    newpos[30:90] -= 12
    np.testing.assert_array_equal(qb.pos, newpos.astype(np.int64))
    assert np.array_equal(pool.kr, kr0), "repos wrote a shared row"
    want = _rope_by_matrix(raw[keep], newpos[:, None, None], base, pairing)
    got, gv = pool.gather(pool.extents(b), lag=pool.visible_lag(b))
    order = pool.visible(b)                          # the list is in position order
    np.testing.assert_allclose(got, want[order], rtol=0, atol=1e-9)
    np.testing.assert_array_equal(gv, v[keep][order])
    # attention over the shared, owed keys equals attention over the fresh keys
    qry = rng.standard_normal((5, 4, d))
    out = AO.segment_attention(pool, qry, [(0, 5, 0, len(pool.extents(b)))], pool.extents(b), 1 / np.sqrt(d),
                               lags=pool.visible_lag(b))
    fresh = AO.Pool(lay)
    f = fresh.seq_create()
    fresh.append(f, newpos.astype(np.int64), want, None, v[keep])
    out2 = AO.segment_attention(fresh, qry, [(0, 5, 0, len(fresh.extents(f)))], fresh.extents(f), 1 / np.sqrt(d))
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    pool.materialize(b)
    assert not np.isin(qb.slot, pool.seqs[a].slot).any() and not qb.lag.any()
    S = lay.page_size
    np.testing.assert_allclose(pool.kr[qb.slot // S, :, qb.slot % S, :], want, rtol=0, atol=1e-9)
    qa = pool.seqs[a]
    np.testing.assert_array_equal(pool.kr[qa.slot // S, :, qa.slot % S, :], kr0[qa.slot // S, :, qa.slot % S, :])
    np.testing.assert_array_equal(pool.v[qa.slot // S, :, qa.slot % S, :], v0[qa.slot // S, :, qa.slot % S, :])
    assert pool.seqs[a].refs == 0 and not qb.owners


def test_shared_pages_outlive_their_source():
    """Pages of a released source stay while a sharer holds slots in them
    and return, in allocation order, when the last one lets go (by release,
    by dropping every shared token, or by materialize); frozen sequences
    refuse every change."""
    rng = np.random.default_rng(22)
    lay = _lay(page_size=4, num_pages=30)
    pool = AO.Pool(lay)
    a, b, c = (pool.seq_create() for _ in range(3))
    _fill(pool, a, 16, rng)
    pages_a = list(pool.seqs[a].pages)
    with pytest.raises(AO.EState):
        pool.share(a, 0, 16, b, 0)                   # not frozen
    pool.freeze(a)
    z = np.zeros((1, 2, 16))
    for call in (lambda: pool.drop(a, [[0, 1]]), lambda: pool.repos(a, [[0, 1]], [1]),
                 lambda: pool.append(a, [99], z, None, z), lambda: pool.compact(a, True),
                 lambda: pool.clone(b, 0, 0, a, 0)):
        with pytest.raises(AO.EState):
            call()
    pool.share(a, 0, 8, b, 10)                       # pages 0, 1 of a
    pool.share(a, 8, 8, c, 10)                       # pages 2, 3 of a
    assert pool.seqs[a].refs == 2
    pool.seq_release(a)
    assert pool.seqs[a].zombie and not any(p in pool.free for p in pages_a)
    pool.drop(b, [[0, 8]], auto_compact=False)       # b lets go of every shared token
    assert pool.seqs[a].refs == 1 and pool.seqs[a].zombie
    pool.seq_release(c)                              # the last holder
    assert not pool.seqs[a].zombie
    assert list(pool.free)[-4:] == pages_a


# ---------------------------------------------------------------------------
# attention mass per page ("AKV: Cache Engineering for Autonomous Agents ...",
# section 7, Dilemma 1: the cumulative attention weight of each block)
# ---------------------------------------------------------------------------
def _mass_pool(rng, page_size=4):
    lay = _lay(page_size=page_size, num_pages=40, n_q_heads=4, n_kv_heads=2)
    pool = AO.Pool(lay, rng.permutation(40))
    a, b = pool.seq_create(), pool.seq_create()
    _fill(pool, a, 50, rng)
    _fill(pool, b, 23, rng)
    pool.drop(a, [[5, 17], [30, 31]], auto_compact=False)
    ex_a, ex_b = pool.extents(a), pool.extents(b)
    ex = np.concatenate([ex_a, ex_b])
    segs = [(0, 3, 0, len(ex_a)), (3, 2, len(ex_a), len(ex_b))]
    return pool, lay, ex, segs


def test_page_mass_uniform_queries_closed_form():
    """Zero queries make every visible weight 1 / (limit + 1): the mass of a
    page is heads x sum over rows of (its entries up to the row's causal
    limit) / (limit + 1), counted here from the extents alone."""
    rng = np.random.default_rng(31)
    pool, lay, ex, segs = _mass_pool(rng)
    q = np.zeros((5, lay.n_q_heads, lay.d_qk))
    got = AO.page_mass(pool, q, segs, ex)
    want = np.zeros(lay.num_pages)
    for qb, ql, eb, el in segs:
        pages = np.concatenate([[p] * (hi - lo) for p, lo, hi in ex[eb:eb + el]])
        lkv = len(pages)
        for i in range(ql):
            lim = lkv - ql + i
            for idx in range(lim + 1):
                want[pages[idx]] += lay.n_q_heads / (lim + 1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert abs(got.sum() - 5 * lay.n_q_heads) < 1e-9


def test_page_mass_sums_to_rows_and_follows_a_sharp_key():
    """Random queries: the mass of a launch sums to (query rows x q heads);
    a query aimed hard at one key puts almost all of its row's weight on
    that key's page; pages of dropped tokens get nothing."""
    rng = np.random.default_rng(32)
    pool, lay, ex, segs = _mass_pool(rng)
    q = rng.standard_normal((5, lay.n_q_heads, lay.d_qk))
    m = AO.page_mass(pool, q, segs, ex)
    assert abs(m.sum() - 5 * lay.n_q_heads) < 1e-9
    used = set(ex[:, 0].tolist())
    assert np.all(m[[p for p in range(lay.num_pages) if p not in used]] == 0)
    # row 0 of segment 0, every head aimed at list entry 2 of its own list
    k, _ = pool.gather(ex[:segs[0][3]])
    q2 = q.copy()
    grp = lay.n_q_heads // lay.n_kv_heads
    for h in range(lay.n_q_heads):
        q2[0, h] = 200.0 * k[2, h // grp] / np.linalg.norm(k[2, h // grp])
    m2 = AO.page_mass(pool, q2, [segs[0]], ex[:segs[0][3]])
    page2 = np.repeat(ex[:segs[0][3], 0], ex[:segs[0][3], 2] - ex[:segs[0][3], 1])[2]
    # the aimed row's heads each give nearly 1 to page2; the two other rows at most 2 x heads in total
    assert m2[page2] >= lay.n_q_heads * (1 - 1e-6)
    assert abs(m2.sum() - 3 * lay.n_q_heads) < 1e-9


def test_repos_position_range_is_atomic():
    rng = np.random.default_rng(4)
    pool = AO.Pool(_lay())
    pool.seq_create()
    _fill(pool, 0, 50, rng)
    kr0, pos0 = pool.kr.copy(), pool.seqs[0].pos.copy()
    with pytest.raises(AO.ERange):
        pool.repos(0, [[0, 10], [5, 50]], [3, -60])      # tokens 5..56 would go below 0
    np.testing.assert_array_equal(pool.kr, kr0)
    np.testing.assert_array_equal(pool.seqs[0].pos, pos0)
    with pytest.raises(AO.EInval):
        pool.repos(0, [[10, 5]], [1])
    with pytest.raises(AO.ERange):
        pool.repos(0, [[0, 51]], [1])


# ---------------------------------------------------------------------------
# worked examples printed on the pages
# ---------------------------------------------------------------------------
def test_golden_blog_figure_blocks():
    g = _gold("akv_blog_drop_repos_figure.json")
    B, nb = g["block_size"], g["n_blocks"]
    lay = _lay(page_size=B, num_pages=nb)
    pool = AO.Pool(lay)                            # identity page order: block i -> page i
    pool.seq_create()
    _fill(pool, 0, B * nb, np.random.default_rng(5))
    drop = [[g["drop_blocks"][0] * B, (g["drop_blocks"][-1] + 1) * B]]
    rep = [[g["repos_blocks"][0] * B, (g["repos_blocks"][-1] + 1) * B]]
    pool.drop(0, drop, auto_compact=False)
    pool.repos(0, rep, [g["delta"]])
    ex = pool.extents(0)
    assert [int(p) for p in ex[:, 0]] == g["expected_active_blocks"]
    assert np.all(ex[:, 1] == 0) and np.all(ex[:, 2] == B)
    sq = pool.seqs[0]
    moved = sq.pos[rep[0][0]:rep[0][1]]
    assert [int(moved.min()), int(moved.max())] == g["expected_positions_of_repos_blocks"]
    # the visible list is now position-compact 0..63
    assert list(sq.pos[pool.visible(0)]) == list(range(len(g["expected_active_blocks"]) * B))


def test_golden_blog_history_dependence():
    g = _gold("akv_blog_history_dependence.json")
    n = g["n_tokens"]
    lay = _lay(num_pages=2 * ((n + 15) // 16))
    pool = AO.Pool(lay)
    a, b = pool.seq_create(), pool.seq_create()
    _fill(pool, a, n, np.random.default_rng(6))
    _fill(pool, b, n, np.random.default_rng(6))
    pool.drop(a, [g["drop"]], auto_compact=False)
    pool.repos(a, [[g["drop"][1], n]], [g["delta"]])
    vis = pool.visible(a)
    kept = np.concatenate([np.arange(x, y) for x, y in g["state_a_kept_logical"]])
    np.testing.assert_array_equal(vis, kept)
    want_pos = np.concatenate([np.arange(x, y) for x, y in g["state_a_positions"]])
    np.testing.assert_array_equal(pool.seqs[a].pos[vis], want_pos)
    np.testing.assert_array_equal(pool.seqs[b].pos[pool.visible(b)], np.arange(*g["state_b_positions"][0]))
    # state B's keys are untouched by session 1's ops; the two sessions started from equal keys
    kb, _ = pool.gather(pool.extents(b))
    ka, _ = pool.gather(pool.extents(a))
    np.testing.assert_array_equal(ka[:1000], kb[:1000])


@pytest.mark.parametrize("case", range(3))
def test_golden_leyline_amortize(case):
    g = _gold("leyline_amortize_directive.json")
    c = g["cases"][case]
    rng = np.random.default_rng(7 + case)
    lay = _lay(d_nope=8, d_rope=8, d_v=8, n_q_heads=2, n_kv_heads=2, page_size=16, num_pages=96)
    pool = AO.Pool(lay)
    pool.seq_create()
    n = c["n_tokens"]
    raw_pe = rng.standard_normal((n, 1, 8))
    pos = np.arange(n, dtype=np.float64)
    kn = rng.standard_normal((n, 2, 8))
    v = rng.standard_normal((n, 2, 8))
    pool.append(0, np.arange(n), kn, _rope_by_matrix(raw_pe, pos[:, None], 10000.0, 0), v)
    st = c["stub_len"]
    stub_kn, stub_pe, stub_v = (rng.standard_normal((st, 2, 8)), rng.standard_normal((st, 1, 8)),
                                rng.standard_normal((st, 2, 8)))
    kr0, kn0, v0 = pool.kr.copy(), pool.kn.copy(), pool.v.copy()
    sp = pool.splice(0, [[c["s_start"], c["s_end"]]], [st], stub_kn, stub_pe, stub_v)
    d = st - (c["s_end"] - c["s_start"])
    assert d == c["expected_delta"]
    sq = pool.seqs[0]
    # downstream positions shifted by delta, keys K_pe rotated as fresh RoPE at i + delta
    down = np.arange(c["s_end"], n)
    np.testing.assert_array_equal(sq.pos[down], down + d)
    slot = sq.slot[down]
    got = pool.kr[slot // 16, :, slot % 16, :]
    np.testing.assert_allclose(got, _rope_by_matrix(raw_pe[down], (down + d)[:, None].astype(float), 10000.0, 0),
                               atol=1e-9, rtol=0)
    # K_nope and V of every old slot untouched; prefix K_pe untouched
    old = sq.slot[:n]
    live = old >= 0
    np.testing.assert_array_equal(pool.kn[old[live] // 16, :, old[live] % 16], kn0[old[live] // 16, :, old[live] % 16])
    np.testing.assert_array_equal(pool.v[old[live] // 16, :, old[live] % 16], v0[old[live] // 16, :, old[live] % 16])
    pre = sq.slot[: c["s_start"]]
    np.testing.assert_array_equal(pool.kr[pre // 16, :, pre % 16], kr0[pre // 16, :, pre % 16])
    np.testing.assert_array_equal(sp, np.arange(c["s_start"], c["s_start"] + st))
    # visible positions are compact again: prefix, stub, shifted suffix
    np.testing.assert_array_equal(sq.pos[pool.visible(0)], np.arange(n + d))


def test_splice_composition_of_several_directives():
    """Several disjoint directives at once equal applying them one by one from
    the back (so earlier coordinates stay valid), with per-slot deltas summed."""
    rng = np.random.default_rng(8)
    lay = _lay(d_nope=8, d_rope=8, d_v=8, n_q_heads=2, n_kv_heads=2, num_pages=200)
    spans = [[40, 300], [500, 520], [700, 1500]]
    stubs = [10, 35, 3]
    tot = sum(stubs)
    kn, pe, vv = rng.standard_normal((tot, 2, 8)), rng.standard_normal((tot, 1, 8)), rng.standard_normal((tot, 2, 8))
    pa, pb = AO.Pool(lay), AO.Pool(lay)
    for p in (pa, pb):
        p.seq_create()
        _fill(p, 0, 2000, np.random.default_rng(11))
    pa.splice(0, spans, stubs, kn, pe, vv)
    offs = np.cumsum([0] + stubs)
    dj = [st - (e - b) for (b, e), st in zip(spans, stubs)]
    for j in reversed(range(3)):
        sl = slice(offs[j], offs[j + 1])
        # applied one at a time, stub j is placed before the earlier splices move it
        # by sum(dj[:j]); hand it in rotated back by that amount
        pe_j = _rope_by_matrix(pe[sl], np.full((stubs[j], 1), -float(sum(dj[:j]))), 10000.0, 0)
        pb.splice(0, [spans[j]], [stubs[j]], kn[sl], pe_j, vv[sl])
    ka, va = pa.gather(pa.extents(0))
    kb, vb = pb.gather(pb.extents(0))
    np.testing.assert_allclose(ka, kb, atol=1e-9, rtol=0)
    np.testing.assert_array_equal(va, vb)
    assert sorted(pa.seqs[0].pos[pa.visible(0)]) == list(range(2000 - 260 - 20 - 800 + tot))


# ---------------------------------------------------------------------------
# drop: page-table image
# ---------------------------------------------------------------------------
def _rle_extents(pool, s):
    """Independent run-length encoding of the visible list into extents."""
    q = pool.seqs[s]
    vis = [t for t in range(q.n) if not q.dropped[t]]
    vis.sort(key=lambda t: (q.pos[t], t))
    out = []
    for t in vis:
        p, o = divmod(int(q.slot[t]), pool.S)
        if out and out[-1][0] == p and out[-1][2] == o:
            out[-1][2] += 1
        else:
            out.append([p, o, o + 1])
    return out


@pytest.mark.parametrize("seed", range(6))
def test_extent_invariants_fuzz(seed):
    wl = W.fuzz_small(seed, compact=True)
    res = oracle.run_workload(wl, attention=False)
    pool = res.pool
    for s in range(len(pool.seqs)):
        ex = pool.extents(s)
        assert ex.tolist() == _rle_extents(pool, s)
        q = pool.seqs[s]
        vis = pool.visible(s)
        assert int((ex[:, 2] - ex[:, 1]).sum()) == len(vis) == int(np.count_nonzero(~q.dropped))
        slots = np.concatenate([p * pool.S + np.arange(l, h) for p, l, h in ex]) if len(ex) else []
        assert len(set(slots)) == len(slots)
        assert set(slots) == set(q.slot[~q.dropped].tolist())
        key = list(zip(q.pos[vis], vis))
        assert key == sorted(key)


def test_drop_edge_cases_and_atomicity():
    rng = np.random.default_rng(12)
    pool = AO.Pool(_lay(num_pages=8))
    pool.seq_create()
    _fill(pool, 0, 40, rng)
    pool.drop(0, [[5, 5]])                         # empty span: no-op
    pool.drop(0, [[0, 3], [1, 3]], auto_compact=False)   # overlapping / repeated: idempotent
    assert int(np.count_nonzero(pool.seqs[0].dropped)) == 3
    before = pool.seqs[0].dropped.copy()
    with pytest.raises(AO.ERange):
        pool.drop(0, [[10, 12], [30, 41]])
    np.testing.assert_array_equal(pool.seqs[0].dropped, before)
    with pytest.raises(AO.EInval):
        pool.drop(0, [[12, 10]])
    with pytest.raises(AO.EInval):
        pool.drop(5, [[0, 1]])


def test_allocation_rule_and_eviction_order():
    """Free queue in the given order, then dropped-first eviction."""
    lay = _lay(page_size=4, num_pages=6)
    pool = AO.Pool(lay, page_order=[3, 1, 5, 0, 2, 4])
    pool.seq_create()
    rng = np.random.default_rng(13)
    _fill(pool, 0, 14, rng)                        # pages 3, 1, 5, 0 (0 is the open tail, 2 used)
    assert pool.seqs[0].pages == [3, 1, 5, 0]
    pool.drop(0, [[4, 8], [0, 2]], auto_compact=False)   # page 1 empties first; page 3 keeps 2
    assert list(pool.evictable) == [1]
    pool.drop(0, [[12, 14]], auto_compact=False)   # open tail page 0 emptied: stays held
    assert list(pool.evictable) == [1]
    _fill(pool, 0, 2 + 4 + 4 + 4, rng, pos0=100)   # fills page 0, then pages 2, 4, then evicts 1
    assert pool.seqs[0].pages == [3, 5, 0, 2, 4, 1]
    with pytest.raises(AO.ENoMem):
        _fill(pool, 0, 5, rng, pos0=200)
    assert pool.seqs[0].pages == [3, 5, 0, 2, 4, 1]


# ---------------------------------------------------------------------------
# compaction ("AKV: Cache Engineering ...", section 7, Dilemma 2)
# ---------------------------------------------------------------------------
def test_compaction_moves_values_unchanged_and_triggers_above_threshold():
    rng = np.random.default_rng(14)
    lay = _lay(page_size=8, num_pages=64)
    pool = AO.Pool(lay, page_order=rng.permutation(64))
    pool.seq_create()
    _fill(pool, 0, 160, rng)
    # every other 8-token block -> 50% waste... but those pages become unreferenced;
    # drop half of every page instead: fragmentation 0.5 > 0.40 triggers compaction
    spans = [[8 * i, 8 * i + 4] for i in range(20)]
    k0, v0 = pool.gather(pool.extents(0))
    keep = np.concatenate([np.arange(8 * i + 4, 8 * i + 8) for i in range(20)])
    pool.drop(0, spans[:2], auto_compact=False)
    assert pool.fragmentation(0) == pytest.approx(1 - 152 / 160)
    pool.drop(0, spans[2:])                        # auto-compaction runs here
    assert pool.fragmentation(0) == 0.0
    ex = pool.extents(0)
    assert len(ex) == 10 and np.all(ex[:, 1] == 0) and np.all(ex[:, 2] == 8)
    k1, v1 = pool.gather(ex)
    np.testing.assert_array_equal(k1, k0[keep])
    np.testing.assert_array_equal(v1, v0[keep])


# ---------------------------------------------------------------------------
# segment-batch attention
# ---------------------------------------------------------------------------
def _fuzz_cases():
    out = []
    for seed in range(8):
        out.append(dict(seed=seed))
    out.append(dict(seed=100, mla=True))
    out.append(dict(seed=101, mla=True, kpe_per_head=1))
    out.append(dict(seed=102, pairing=1))
    out.append(dict(seed=103, mla=True, pairing=1, page_size=4))
    return out


@pytest.mark.parametrize("kw", _fuzz_cases(), ids=lambda k: "-".join(f"{a}{b}" for a, b in k.items()))
def test_segment_oracle_equals_dense_masked_bruteforce(kw):
    """Drop equals masking, repos equals fresh RoPE, and list order equals
    position order: the segment oracle over its page lists matches the literal
    masked softmax over every appended token."""
    wl = W.fuzz_small(**kw)
    res = oracle.run_workload(wl, keep_log=True)
    pool = res.pool
    att = [o for o in wl.ops if isinstance(o, W.Attention)][0]
    got = res.attention[0]["out"]
    q = W.bf16_to_f64(att.q)
    appends = [o for o in wl.ops if isinstance(o, W.Append)]
    for sg in att.segments:
        # the query tokens are the last appended tokens of the sequence
        last = [a for a in appends if a.seq == sg.seq][-1]
        mine = [s for s in att.segments if s.seq == sg.seq]
        off = sum(s.q_len for s in mine[: mine.index(sg)])
        qpos = last.pos[off: off + sg.q_len]
        rows = np.arange(sg.q_begin, sg.q_begin + sg.q_len)
        want = oracle.dense_masked_attention(pool, q, sg.seq, rows, qpos,
                                             sg.mask_spans if len(sg.mask_spans) else None)
        np.testing.assert_allclose(got[rows], want, atol=1e-12, rtol=0)


def _sdpa_ref(q, k, v, grp, scale, bottom_right_causal=True):
    """torch SDPA in fp64 with an explicit bottom-right boolean mask."""
    Lq, Lk = q.shape[0], k.shape[0]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]           # [1, Hq, Lq, d]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    mask = None
    if bottom_right_causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        mask = j <= (Lk - Lq + i)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                                         enable_gqa=grp > 1)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("lq", [1, 7, 40])
def test_single_segment_contiguous_equals_sdpa(lq):
    """One segment over an undropped cache is ordinary causal attention (and
    with one query it is decode attention)."""
    rng = np.random.default_rng(15)
    lay = _lay(n_q_heads=8, n_kv_heads=2, d_rope=32, d_v=24, page_size=16, num_pages=32)
    pool = AO.Pool(lay, page_order=rng.permutation(32))
    pool.seq_create()
    n = 300
    k, _, v = _fill(pool, 0, n, rng)
    q = rng.standard_normal((lq, 8, 32))
    ex = pool.extents(0)
    out = AO.segment_attention(pool, q, [(0, lq, 0, len(ex))], ex, 0.0)
    ref = _sdpa_ref(q, k, v, 4, 1 / np.sqrt(32))
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)


def test_attention_relative_position_invariance():
    """q_n . k_m depends on m - n only ("AKV: Cache Engineering ...", section 2):
    shifting every query and key position by c leaves the output unchanged."""
    rng = np.random.default_rng(16)
    lay = _lay(n_q_heads=2, n_kv_heads=1, d_rope=32, d_v=8, num_pages=24)
    n, lq = 200, 10
    kraw, vv, qraw = rng.standard_normal((n, 1, 32)), rng.standard_normal((n, 1, 8)), rng.standard_normal((lq, 2, 32))
    outs = []
    for c in (0, 12345):
        pool = AO.Pool(lay)
        pool.seq_create()
        m = np.arange(n, dtype=np.float64) + c
        pool.append(0, m.astype(np.int64), _rope_by_matrix(kraw, m[:, None], 10000.0, 0), None, vv)
        qp = (np.arange(n - lq, n) + c).astype(float)
        q = _rope_by_matrix(qraw, qp[:, None], 10000.0, 0)
        ex = pool.extents(0)
        outs.append(AO.segment_attention(pool, q, [(0, lq, 0, len(ex))], ex))
    np.testing.assert_allclose(outs[0], outs[1], atol=1e-10, rtol=0)


def test_attention_history_extent_permutation_invariance():
    """Entries every query sees may be listed in any order."""
    rng = np.random.default_rng(17)
    lay = _lay(n_q_heads=4, n_kv_heads=2, d_rope=16, d_v=16, num_pages=32)
    pool = AO.Pool(lay, page_order=rng.permutation(32))
    pool.seq_create()
    _fill(pool, 0, 250, rng)
    ex = pool.extents(0)
    q = rng.standard_normal((20, 4, 16))
    hist, tail = ex[:-3], ex[-3:]                # the last 3 extents hold the causal window
    assert (tail[:, 2] - tail[:, 1]).sum() >= 20
    perm = np.concatenate([hist[rng.permutation(len(hist))], tail])
    a = AO.segment_attention(pool, q, [(0, 20, 0, len(ex))], ex)
    b = AO.segment_attention(pool, q, [(0, 20, 0, len(perm))], perm)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_attention_rejects_short_lists_and_bad_extents():
    rng = np.random.default_rng(18)
    pool = AO.Pool(_lay())
    pool.seq_create()
    _fill(pool, 0, 20, rng)
    ex = pool.extents(0)
    q = rng.standard_normal((30, 4, 16))
    with pytest.raises(AO.EInval):
        AO.segment_attention(pool, q, [(0, 30, 0, len(ex))], ex)
    with pytest.raises(AO.ERange):
        AO.segment_attention(pool, q, [(0, 1, 0, 1)], [[0, 3, 17]])


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin above
# ---------------------------------------------------------------------------
def test_planted_sign_error_is_caught(monkeypatch):
    real = AO.rotate
    monkeypatch.setattr(AO, "rotate", lambda x, d, f, p: real(x, -np.asarray(d), f, p))
    with pytest.raises(AssertionError):
        test_repos_equals_fresh_rope_at_new_position(0, 10000.0)


def test_planted_pairing_error_is_caught(monkeypatch):
    real = AO.rotate
    monkeypatch.setattr(AO, "rotate", lambda x, d, f, p: real(x, d, f, 1 - p))
    with pytest.raises(AssertionError):
        test_repos_equals_fresh_rope_at_new_position(0, 10000.0)


def test_planted_causal_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(AO, "last_visible", lambda lkv, lq, i: lkv - lq + i + 1)
    with pytest.raises(AssertionError):
        test_segment_oracle_equals_dense_masked_bruteforce(dict(seed=0))
    with pytest.raises(AssertionError):
        test_single_segment_contiguous_equals_sdpa(7)


def test_planted_gqa_mapping_error_is_caught(monkeypatch):
    real = AO.segment_attention

    def wrong(pool, q, segments, page_lists, scale=0.0, rows=None):
        # interleaved head groups instead of contiguous ones
        L = pool.L
        perm = np.arange(L.n_q_heads).reshape(-1, L.n_kv_heads).T.reshape(-1)
        return real(pool, q[:, perm], segments, page_lists, scale, rows)[:, np.argsort(perm)]
    monkeypatch.setattr(AO, "segment_attention", wrong)
    with pytest.raises(AssertionError):
        test_single_segment_contiguous_equals_sdpa(7)
