"""Extended radix tree (host, through the C ABI) against the brute-force
matcher of the cache reuse rules (oracle/akv_tree_oracle.py): every match,
pin and eviction result equal, on random families of related histories and on
the two-agent example of "AKV: Cache Engineering for Autonomous Agents ...",
section 3."""
import os

import numpy as np
import pytest

from oracle.akv_tree_oracle import DROP, REPOS, TOKEN, TreeOracle

akv = pytest.importorskip("kv_cache_drop_amd")
pytestmark = pytest.mark.skipif(not os.path.exists(akv.LIB_PATH), reason="libakv.so not built")


def _tokens(ids, pos0):
    return [(TOKEN, int(t), int(pos0 + i), 0) for i, t in enumerate(ids)]


def _family(rng, n_base=40):
    """A base history and variants: prefixes, shifted replays, divergent
    operations, extensions."""
    ids = rng.integers(0, 5, n_base)
    base = _tokens(ids[:20], 0) + [(DROP, 3, 9, 0), (REPOS, 9, 20, -6)] + _tokens(ids[20:], 14)
    out = [base]
    for _ in range(6):
        kind = rng.integers(0, 5)
        h = list(out[rng.integers(0, len(out))])
        cut = int(rng.integers(1, len(h) + 1))
        if kind == 0:                      # prefix
            out.append(h[:cut])
        elif kind == 1:                    # the same history at shifted positions
            s = int(rng.integers(-5, 30))
            out.append([(k, a, b + s, c) if k == TOKEN else (k, a, b, c) for k, a, b, c in h if k != TOKEN or b + s >= 0])
        elif kind == 2:                    # divergent operation
            out.append(h[:cut] + [(DROP, 0, 2, 0)] + _tokens(rng.integers(0, 5, 5), 100))
        elif kind == 3:                    # extension
            out.append(h + _tokens(rng.integers(0, 5, int(rng.integers(1, 8))), 200))
        else:                              # different tokens after a cut
            out.append(h[:cut] + _tokens(rng.integers(5, 9, 4), 50))
    return [np.asarray(h, np.int32).reshape(-1, 4) for h in out if len(h)]


@pytest.mark.parametrize("seed", range(20))
def test_tree_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    fam = _family(rng)
    tree, ref = akv.Tree(), TreeOracle()
    seq = 0
    for h in fam[: len(fam) // 2 + 1]:
        tree.insert(h, seq)
        ref.insert(h, seq)
        seq += 1
    for step in range(40):
        h = fam[rng.integers(0, len(fam))]
        r = h[: int(rng.integers(0, len(h) + 1))]
        if rng.random() < 0.3 and len(r):      # perturb one event
            r = r.copy()
            i = int(rng.integers(0, len(r)))
            r[i, 1 if r[i, 0] == TOKEN else 2] += 1
        got, want = tree.match(r), ref.match(r)
        assert got == want, (step, got, want)
        act = rng.random()
        if act < 0.15 and got["seq"] >= 0:
            tree.pin(got["seq"], 1)
            ref.pin(got["seq"], 1)
        elif act < 0.25:
            n = int(rng.integers(0, 3))
            assert tree.evict(n) == ref.evict(n)
        elif act < 0.4:
            h = fam[rng.integers(0, len(fam))]
            try:
                ref.insert(h, seq)
            except ValueError:
                continue
            tree.insert(h, seq)
            seq += 1
    assert tree.stats()[1] == sum(c["live"] for c in ref.checks)
    tree.close()


@pytest.mark.parametrize("impl", ["library", "oracle"])
def test_two_agents_fork_on_operation_history(impl):
    """Agent 1 dropped a tool span and repositioned the rest; agent 2 kept
    everything.  Same tokens, different operations: each request is served
    only by the state with its own operation history.  Expected hits are
    worked out by hand from the rules (pins the brute force too)."""
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 1000, 40)
    trace = _tokens(ids, 0)
    agent1 = trace + [(DROP, 10, 35, 0), (REPOS, 35, 40, -25)]
    agent2 = trace + _tokens(rng.integers(0, 1000, 3), 40)
    tree = akv.Tree() if impl == "library" else TreeOracle()
    tree.insert(agent1, 1)
    tree.insert(agent2, 2)
    hit = tree.match(agent1 + _tokens([7, 8], 15))
    assert hit == dict(seq=1, n_events=42, n_tokens=40, exact=1, delta=0)
    hit = tree.match(agent2)
    assert hit == dict(seq=2, n_events=43, n_tokens=43, exact=1, delta=0)
    # the raw trace prefix: agent 2 serves it (only tokens follow); agent 1
    # cannot (its drop changed those tokens)
    assert tree.match(trace)["seq"] == 2
    # agent 1's tokens with another drop: diverges at the operation, and
    # agent 1's state cannot serve the shared token prefix
    hit = tree.match(trace + [(DROP, 0, 5, 0)])
    assert hit["seq"] == 2 and hit["n_events"] == 40
    # the same two histories replayed 300 positions later: retrigger matches
    shifted = [(k, a, b + 300, c) if k == TOKEN else (k, a, b, c) for k, a, b, c in agent1]
    hit = tree.match(shifted)
    assert hit == dict(seq=1, n_events=42, n_tokens=40, exact=0, delta=300)
    # positions shifted unevenly: one rotation covers only the first 20
    # tokens, and only agent 2 (tokens only after them) can serve that prefix
    uneven = [(k, a, b + (300 if b < 20 else 301), c) if k == TOKEN else (k, a, b, c) for k, a, b, c in agent1]
    assert tree.match(uneven) == dict(seq=2, n_events=20, n_tokens=20, exact=0, delta=300)
    if impl == "library":
        tree.close()


def test_retrigger_hit_rebuilds_the_state_through_clone():
    """A retrigger hit reused through akv_seq_clone gives the same positions,
    flags and visible order as replaying the shifted history."""
    lay_args = (4, 2, 0, 16, 16, 8, 64)
    hp = akv.Pool(*lay_args, device=False)
    ref = akv.Pool(*lay_args, device=False)
    a = hp.seq_create()
    hp.append(a, np.arange(60))
    hp.drop(a, [[10, 25]])
    hp.repos(a, [[25, 60]], [-15])
    hist = [(TOKEN, i % 7, i, 0) for i in range(60)] + [(DROP, 10, 25, 0), (REPOS, 25, 60, -15)]
    tree = akv.Tree()
    tree.insert(hist, a)
    req = [(k, x, y + 33, z) if k == TOKEN else (k, x, y, z) for k, x, y, z in hist]
    hit = tree.match(req)
    assert hit == dict(seq=a, n_events=62, n_tokens=60, exact=0, delta=33)
    b = hp.seq_create()
    hp.clone(a, 0, hit["n_tokens"], b, hit["delta"])
    r = ref.seq_create()
    ref.append(r, np.arange(60) + 33)
    ref.drop(r, [[10, 25]])
    ref.repos(r, [[25, 60]], [-15])
    _, pos_r, drop_r = ref.tokens(r)
    _, pos_b, drop_b = hp.tokens(b)
    np.testing.assert_array_equal(pos_b, pos_r[~drop_r])
    assert not drop_b.any()
    tree.close()


def test_tree_errors():
    tree = akv.Tree()
    with pytest.raises(akv.AkvError):
        tree.insert(np.zeros((0, 4)), 1)
    with pytest.raises(akv.AkvError):
        tree.insert([(TOKEN, 1, -1, 0)], 1)
    with pytest.raises(akv.AkvError):
        tree.insert([(9, 1, 1, 0)], 1)
    tree.insert([(TOKEN, 1, 0, 0)], 1)
    with pytest.raises(akv.AkvError):
        tree.insert([(TOKEN, 2, 0, 0)], 1)
    with pytest.raises(akv.AkvError):
        tree.pin(5, 1)
    with pytest.raises(akv.AkvError):
        tree.pin(1, -1)
    assert tree.match([])["seq"] == -1
    tree.pin(1, 1)
    assert tree.evict(3) == []
    tree.pin(1, -1)
    assert tree.evict(3) == [1]
    assert tree.match([(TOKEN, 1, 0, 0)])["seq"] == -1
    tree.close()
