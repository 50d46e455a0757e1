"""Debug switches and kernel timers of libakv.so.  The switches are read from the
environment once per process:
AKV_CHECKS (host checks of every device work list before its launch),
AKV_TRACE (planning decisions on stderr), AKV_COMPACT_THRESHOLD (default
fragmentation threshold) and AKV_FAULT_INJECT=launch (every launch reports
failure, so each call's error path runs).  Every case runs in a child process
with the switch set; the GPU cases drive device pools.
"""
import os
import subprocess
import sys
import textwrap

import pytest

akv = pytest.importorskip("kv_cache_drop_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")


def _child(code: str, timeout: int = 300, **env):
    e = dict(os.environ)
    for k in ("AKV_CHECKS", "AKV_TRACE", "AKV_COMPACT_THRESHOLD", "AKV_FAULT_INJECT"):
        e.pop(k, None)
    e.update({k: str(v) for k, v in env.items()})
    pre = f"import sys; sys.path[:0] = [{ROOT!r}, {TESTS!r}]\n"
    r = subprocess.run([sys.executable, "-c", pre + textwrap.dedent(code)], env=e, capture_output=True,
                       text=True, timeout=timeout)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r.stdout, r.stderr


def _need_lib():
    if not os.path.exists(akv.LIB_PATH):
        pytest.skip("libakv.so not built")


# A page-table-only pool: 64 tokens fill 4 pages of 16; dropping the second
# half of every page leaves half of the written slots of pages holding a
# visible token dead (fragmentation 0.5).
_FRAG_SCRIPT = """
import numpy as np
import kv_cache_drop_amd as akv
p = akv.Pool(8, 2, 0, 64, 64, 16, 64, device=False)
s = p.seq_create()
p.append(s, np.arange(64))
slots0 = p.tokens(s)[0].copy()
p.drop(s, [[8, 16], [24, 32], [40, 48], [56, 64]])
slots1 = p.tokens(s)[0]
n, v, frag = p.info(s)
print("MOVED", int((slots0 != slots1).sum()), "FRAG", frag)
"""


def test_compact_threshold_from_the_environment():
    """Fragmentation 0.5 is above the default 0.40, so the sequence is
    compacted at once (its 32 visible rows move); with
    AKV_COMPACT_THRESHOLD=0.9 it is not, and an out-of-range value leaves the
    default in force."""
    _need_lib()
    out, _ = _child(_FRAG_SCRIPT)
    moved = int(out.split()[1])
    assert moved == 32, out
    out, _ = _child(_FRAG_SCRIPT, AKV_COMPACT_THRESHOLD="0.9")
    assert int(out.split()[1]) == 0 and abs(float(out.split()[3]) - 0.5) < 1e-12, out
    out, _ = _child(_FRAG_SCRIPT, AKV_COMPACT_THRESHOLD="1.7")
    assert int(out.split()[1]) == moved, out


def test_trace_names_each_planning_decision():
    _need_lib()
    code = """
    import numpy as np
    import kv_cache_drop_amd as akv
    p = akv.Pool(8, 2, 0, 64, 64, 16, 64, device=False)
    halves = [[8, 16], [24, 32], [40, 48], [56, 64]]
    s = p.seq_create()
    p.append(s, np.arange(64))
    p.drop(s, halves)                      # fragmentation 0.5: compacted at once
    p.repos(s, [[48, 56]], [-8])           # 8 rows of one page
    p.compaction_mode(True)
    t = p.seq_create()
    p.append(t, np.arange(64))
    p.drop(t, halves)                      # queued
    p.compact_pending(1 << 20)
    print("DONE")
    """
    out, err = _child(code, AKV_TRACE="1")
    assert "DONE" in out
    lines = [l for l in err.splitlines() if l.startswith("akv: ")]
    text = "\n".join(lines)
    assert "fragmentation 0.500 above 0.40, compacting" in text, text
    assert "compact seq 0: 32 visible tokens into 2 fresh pages" in text, text
    assert "rotate: 1 items, 1 distinct deltas, 1 layer(s)" in text, text
    assert "seq 1: fragmentation 0.500 above 0.40, queued for compaction" in text, text
    assert "compact seq 1: 32 visible tokens into 2 fresh pages" in text, text
    assert "background compaction: 32 row copies" in text, text
    # without the switch the library prints nothing
    _, err = _child(code)
    assert "akv: " not in err


def test_checks_pass_on_every_host_script():
    """With AKV_CHECKS=1 the library checks every work list it builds
    (append slots, rotate items, compaction and clone copies, attention
    plans) before its launch; page-table-only pools build the same lists.
    The host-runtime scripts and the planner cases still match the oracle
    bit for bit, so no check fires on correct lists."""
    _need_lib()
    code = """
    import test_host_runtime as T
    import test_attention_plan as P
    for s in range(4):
        T.test_fuzz_scripts_bit_exact(s)
    T.test_fuzz_scripts_page_size_extremes(1)
    T.test_fuzz_mla_splice_scripts_bit_exact(0)
    for s in range(3):
        T.test_share_scripts_bit_exact(s)
    T.test_share_through_background_compaction_bit_exact(0)
    T.test_deferred_compaction_scripts_bit_exact(0, 0.7)
    T.test_c1_page_tables_bit_exact("canonical")
    T.test_c3_splices_bit_exact()
    T.test_retrigger_clone_page_tables_bit_exact(3, True, 700)
    T.test_decode_batch_page_tables_bit_exact(2, 1, True)
    T.test_repos_layers_host()
    T.test_repos_batch_equals_sequential_and_is_atomic()
    for s in range(4):
        P.test_plan_random_scripts_enumerated(s)
    print("CHECKED")
    """
    out, err = _child(code, timeout=600, AKV_CHECKS="1")
    assert "CHECKED" in out and "AKV_CHECKS" not in err, err[-2000:]


@pytest.mark.gpu
def test_injected_launch_failure_reports_ehip():
    """AKV_FAULT_INJECT=launch: the kernels still run, every launch reports
    failure, and each call returns AKV_EHIP with the launch named in the
    error text (append, repos, attention, compaction)."""
    _need_lib()
    code = """
    import numpy as np, torch
    import kv_cache_drop_amd as akv
    p = akv.Pool(8, 2, 0, 128, 128, 16, 64)
    s = p.seq_create()
    k = torch.randn(64, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    v = torch.randn(64, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    q = torch.randn(4, 8, 128, dtype=torch.bfloat16, device="cuda:0")
    def status(f):
        try:
            f()
        except akv.AkvError as e:
            return e.status, str(e)
        return 0, ""
    print("APPEND", *status(lambda: p.append(s, np.arange(64), k, None, v)))
    print("REPOS", *status(lambda: p.repos(s, [[0, 64]], [5])))
    print("ATTN", *status(lambda: p.seq_attention(q, [(s, 0, 4, None)])))
    print("COMPACT", *status(lambda: p.compact(s, True)))
    torch.cuda.synchronize()
    print("DONE")
    """
    out, _ = _child(code, AKV_FAULT_INJECT="launch")
    assert "DONE" in out, out
    for tag, what in [("APPEND", "append kernel launch"), ("REPOS", "rotate kernel launch"),
                      ("ATTN", "expand kernel launch"), ("COMPACT", "compaction kernel launch")]:
        line = next(l for l in out.splitlines() if l.startswith(tag + " "))
        assert line.split()[1] == "-5" and what in line and "injected" in line, line


@pytest.mark.gpu
def test_checks_on_device_scripts():
    """AKV_CHECKS=1 with device pools: shared pages, deferred rotations fused
    into attention, background compaction and split-KV decode all pass their
    host checks and still match the oracle."""
    _need_lib()
    code = """
    import test_gpu_parity as G
    G.test_share_scripts_full(0, "auto")
    G.test_share_through_background_compaction_full(0)
    G.test_deferred_compaction_full(2, 0.7)
    G.test_page_mass_decode_full(1, 1, 1, True, 32, "stress")
    print("CHECKED")
    """
    out, err = _child(code, timeout=600, AKV_CHECKS="1", AKV_TRACE="1")
    assert "CHECKED" in out and "AKV_CHECKS failed" not in err, err[-2000:]
    assert "akv: attention:" in err


@pytest.mark.gpu
def test_kernel_timers_count_each_launch():
    """With the pool's timers on, every kernel launch carries its own start and
    stop events: one duration per launch and kind (append, rotate, expand,
    attention, compaction), each positive and below the wall time of the
    synchronised call sequence; with the timers off nothing is recorded."""
    _need_lib()
    import time

    import numpy as np
    import torch

    p = akv.Pool(8, 2, 0, 128, 128, 16, 256)
    s = p.seq_create()
    n = 1024
    k = torch.randn(n, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    v = torch.randn(n, 2, 128, dtype=torch.bfloat16, device="cuda:0")
    q = torch.randn(64, 8, 128, dtype=torch.bfloat16, device="cuda:0")
    p.append(s, np.arange(n), k, None, v)        # untimed
    torch.cuda.synchronize()
    p.timing_enable(True)
    for kind in akv.KERNEL_KINDS:
        p.timing_read(kind)
    t0 = time.perf_counter()
    p.drop(s, [[100, 500]])
    p.repos(s, [[500, n]], [-400])
    p.seq_attention(q, [(s, 0, 64, None)])
    p.compact(s, True)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    got = {kind: p.timing_read(kind) for kind in ("append", "rotate", "expand", "attention", "compact")}
    assert got["append"] == (0.0, 0), got
    for kind in ("rotate", "expand", "attention", "compact"):
        ms, cnt = got[kind]
        assert cnt == 1 and 0.0 < ms < wall_ms, (kind, got)
    p.timing_enable(False)
    p.seq_attention(q, [(s, 0, 64, None)])
    torch.cuda.synchronize()
    assert p.timing_read("attention") == (0.0, 0)
    p.close()
