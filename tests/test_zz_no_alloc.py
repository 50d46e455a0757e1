"""The no-allocation attention entry point (akv_segment_attention_static)
against akv_segment_attention: the same kernels and plan over a static device
workspace, so the outputs must be equal bit for bit; two calls in a row, the
second smaller, and a call too large for the workspace refused before
anything runs."""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

akv = pytest.importorskip("kv_cache_drop_amd")
import device_script as D  # noqa: E402


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    akv.lib()
    yield
    torch.cuda.synchronize()


def _inputs(wl):
    """Replay a workload up to its attention; the device pool, Q and lists."""
    att_i = max(i for i, o in enumerate(wl.ops) if isinstance(o, W.Attention))
    head = W.Workload(wl.name, wl.layout, wl.page_order, wl.ops[:att_i], wl.notes)
    pool, _ = D.run(head)
    att = wl.ops[att_i]
    rows, ex = D.segment_inputs(pool, att)
    return pool, D.dev_bf16(att.q), rows, ex


@pytest.mark.parametrize("make", [lambda: W.c2_64k(0), lambda: W.c3_mla(0)])
def test_static_workspace_attention_equals_pool_scratch(make):
    wl = make()
    _say(f"[gpu] static workspace attention: {wl.name}")
    pool, q, rows, ex = _inputs(wl)
    L = wl.layout
    shape = (q.shape[0], L.n_q_heads, L.d_v)
    # call 1: every segment; call 2: a smaller launch (the last segment only,
    # its rows and list), into a fresh output
    small = rows[-1:].copy()
    small_ex = ex[small[0, 2]:small[0, 2] + small[0, 3]]
    small[0, 2] = 0
    for segs, lists in ((rows, ex), (small, small_ex)):
        want = torch.full(shape, 3.0, dtype=torch.bfloat16, device="cuda:0")
        got = torch.full(shape, 3.0, dtype=torch.bfloat16, device="cuda:0")
        pool.segment_attention(q, segs, lists, 0.0, out=want)
        pool.segment_attention_static(q, segs, lists, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{wl.name}: {len(segs)} segments"
    pool.close()


def test_static_workspace_back_to_back_without_sync():
    """Several calls queued on the pool stream with no sync between them:
    each call's table copy lands after the earlier calls' kernels."""
    wl = W.decode_batch(1, n_req=24, ctx_lo=2000, ctx_hi=8000)
    _say("[gpu] static workspace: back-to-back decode launches")
    pool, q, rows, ex = _inputs(wl)
    L = wl.layout
    shape = (q.shape[0], L.n_q_heads, L.d_v)
    cuts = [len(rows), len(rows) // 2, 3]
    outs, refs = [], []
    for n in cuts:
        segs = rows[:n].copy()
        lists = ex[:segs[-1, 2] + segs[-1, 3]]
        o = torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
        pool.segment_attention_static(q, segs, lists, o)
        outs.append((o, segs, lists))
    torch.cuda.synchronize()
    for o, segs, lists in outs:
        r = torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
        pool.segment_attention(q, segs, lists, 0.0, out=r)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), r.view(torch.int16))
    pool.close()


def test_static_workspace_refuses_oversized_calls():
    """A launch whose lists need more than the 128 MiB workspace is refused
    with AKV_ENOMEM and writes nothing."""
    lay = W.Layout(8, 2, 0, 64, 64, 16, 300000 // 16 + 8)
    pool = akv.Pool(8, 2, 0, 64, 64, 16, lay.num_pages, scratch_bytes=64 << 20)
    s = pool.seq_create()
    n = 300000
    z = torch.zeros((n, 2, 64), dtype=torch.bfloat16, device="cuda:0")
    pool.append(s, np.arange(n), z, None, z)
    ex = pool.visible(s)
    # 128 segments of one query each over the whole list: 128 x 300K slots = 154 MB
    segs = np.array([(i, 1, 0, len(ex)) for i in range(128)], np.int32)
    q = torch.zeros((128, 8, 64), dtype=torch.bfloat16, device="cuda:0")
    out = torch.full((128, 8, 64), 5.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(akv.AkvError) as ei:
        pool.segment_attention_static(q, segs, ex, out)
    assert ei.value.status == akv.AKV_ENOMEM and "static workspace" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)
    pool.close()
