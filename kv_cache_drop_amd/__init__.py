"""AKV cache engineering on AMD MI355X (gfx950): a paged bf16 KV pool with
append / drop / repos / splice / compaction and segment-batch attention.

This module is a thin ctypes binding over the C ABI in include/akv.h
(libakv.so, built in-tree by `kv_cache_drop_amd.build`).  It only marshals
arguments: every step of the path runs in the library's host runtime and HIP
kernels.  torch supplies device memory and the stream.  When the library is
missing, every call raises; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = ["AkvError", "Pool", "Tree", "lib", "LIB_PATH", "SYMBOLS", "KERNEL_KINDS", "attention_supported",
           "repos_layers", "EV_TOKEN", "EV_DROP", "EV_REPOS"]

# The built library; AKV_LIB_PATH may name another build of the same sources
# (the host-sanitized one of `python -m kv_cache_drop_amd.build --sanitize`).
LIB_PATH = os.environ.get("AKV_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libakv.so")

AKV_OK, AKV_EINVAL, AKV_ERANGE, AKV_ENOMEM, AKV_ESTATE, AKV_EHIP = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "AKV_OK", -1: "AKV_EINVAL", -2: "AKV_ERANGE", -3: "AKV_ENOMEM",
                -4: "AKV_ESTATE", -5: "AKV_EHIP"}
EV_TOKEN, EV_DROP, EV_REPOS = 0, 1, 2
KERNEL_KINDS = {"append": 0, "rotate": 1, "compact": 2, "expand": 3, "attention": 4, "combine": 5,
                "clone": 6, "mass": 7}


class AkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("kpe_per_head", ctypes.c_int32), ("pairing", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("inv_freq", ctypes.POINTER(ctypes.c_double)),
                ("compact_threshold", ctypes.c_double)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_IP = ctypes.POINTER(ctypes.c_int32)

# name -> argtypes (restype is akv_status = int32 unless noted)
SYMBOLS = {
    "akv_pool_create": [ctypes.POINTER(Layout), _IP, _P, _P, _P, _P, ctypes.c_size_t, _P,
                        ctypes.POINTER(_P)],
    "akv_pool_destroy": [_P],
    "akv_seq_create": [_P, _IP],
    "akv_seq_release": [_P, _I],
    "akv_append": [_P, _I, _P, _P, _P, _IP, _I],
    "akv_drop": [_P, _I, _IP, _I],
    "akv_compact": [_P, _I, _I],
    "akv_compaction_mode": [_P, _I],
    "akv_fused_rotation": [_P, _I],
    "akv_compact_pending": [_P, ctypes.c_int64, _I, _IP, _IP],
    "akv_compact_queue": [_P, _IP, _I, _IP],
    "akv_repos": [_P, _I, _IP, _IP, _I],
    "akv_repos_batch": [_P, _I, _IP, _IP, _IP, _IP],
    "akv_repos_layers": [ctypes.POINTER(_P), _I, _I, _IP, _IP, _I],
    "akv_repos_deferred": [_P, _I, _IP, _IP, _I],
    "akv_materialize": [_P, _I],
    "akv_seq_lag": [_P, _I, _I, _I, _IP],
    "akv_splice": [_P, _I, _IP, _IP, _I, _P, _P, _P, _IP],
    "akv_seq_clone": [_P, _I, _I, _I, _I, _I],
    "akv_seq_freeze": [_P, _I],
    "akv_seq_share": [_P, _I, _I, _I, _I, _I],
    "akv_append_batch": [_P, _I, _IP, _IP, _P, _P, _P, _IP],
    "akv_seq_attention": [_P, _P, _I, _IP, _I, _IP, _I, ctypes.c_float, _P],
    "akv_seq_visible": [_P, _I, _IP, _I, _IP, _I, _IP],
    "akv_segment_attention": [_P, _P, _I, _IP, _I, _IP, _I, ctypes.c_float, _P],
    "akv_segment_attention_static": [_P, _P, _I, _IP, _I, _IP, _I, ctypes.c_float, _P],
    "akv_attention_mass": [_P, _P, _I],
    "akv_seq_tokens": [_P, _I, _I, _I, _IP, _IP, ctypes.POINTER(ctypes.c_uint8)],
    "akv_seq_info": [_P, _I, _IP, _IP, ctypes.POINTER(ctypes.c_double)],
    "akv_pool_queues": [_P, _IP, _I, _IP, _IP, _I, _IP],
    "akv_repos_plan": [_P, _I, _IP, _IP, _I, _IP, _IP, _I, _IP],
    "akv_attention_plan": [_P, _I, _IP, _I, _IP, _I, _I, _IP, _I, _IP, _IP, _I, _IP, _IP,
                           ctypes.POINTER(ctypes.c_int64)],
    "akv_tree_create": [ctypes.POINTER(_P)],
    "akv_tree_destroy": [_P],
    "akv_tree_insert": [_P, _IP, _I, _I],
    "akv_tree_match": [_P, _IP, _I, _IP],
    "akv_tree_pin": [_P, _I, _I],
    "akv_tree_evict": [_P, _I, _IP, _IP],
    "akv_tree_stats": [_P, _IP, _IP],
    "akv_timing_enable": [_P, _I],
    "akv_timing_read": [_P, _I, ctypes.POINTER(ctypes.c_double), _IP],
    "akv_timing_samples": [_P, _I, ctypes.POINTER(ctypes.c_float), _I, _IP],
    "akv_sync": [_P],
    "akv_last_error": [],
}

_LIB = None


def lib() -> ctypes.CDLL:
    """Load libakv.so (raises when it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m kv_cache_drop_amd.build` "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SYMBOLS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "akv_last_error" else ctypes.c_int32
        _LIB = L
    return _LIB


def _check(st: int) -> None:
    if st != AKV_OK:
        raise AkvError(st, lib().akv_last_error().decode(errors="replace"))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


_NO_SPANS = np.zeros((0, 2), np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_IP) if a.size else None


def _dptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def attention_supported(d_nope: int, d_rope: int, d_v: int) -> bool:
    if d_nope == 0:
        return d_rope in (32, 64, 128) and d_v == d_rope
    return (d_nope, d_rope, d_v) in ((128, 64, 128), (32, 32, 32))


class Pool:
    """A paged KV pool.  With device=True the page arrays and the scratch
    buffer are torch tensors on `device` (attributes k_pages, kpe_pages,
    v_pages, scratch; the page arrays start zero-filled, so unused slots never
    hold stale bits); with device=False the pool is page-table-only."""

    def __init__(self, n_q_heads: int, n_kv_heads: int, d_nope: int, d_rope: int, d_v: int,
                 page_size: int, num_pages: int, kpe_per_head: int = 0, pairing: int = 0,
                 rope_theta: float = 10000.0, inv_freq: Optional[Sequence[float]] = None,
                 compact_threshold: float = 0.0, page_order=None, device: bool = True,
                 scratch_bytes: int = 64 << 20, torch_device: str = "cuda:0", stream=None):
        L = lib()
        self.layout = dict(n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, d_nope=d_nope, d_rope=d_rope,
                           d_v=d_v, page_size=page_size, num_pages=num_pages,
                           kpe_per_head=kpe_per_head, pairing=pairing)
        self._inv = None
        lay = Layout(n_q_heads, n_kv_heads, d_nope, d_rope, d_v, page_size, num_pages, kpe_per_head,
                     pairing, float(rope_theta), None, float(compact_threshold))
        if inv_freq is not None:
            self._inv = np.ascontiguousarray(np.asarray(inv_freq, np.float64))
            lay.inv_freq = self._inv.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
        order = None if page_order is None else _i32(page_order)
        self.k_pages = self.kpe_pages = self.v_pages = self.scratch = None
        self.stream = None
        h = ctypes.c_void_p()
        if device:
            import torch
            dev = torch.device(torch_device)
            bf = torch.bfloat16
            if d_nope > 0:
                hpe = n_kv_heads if kpe_per_head else 1
                self.k_pages = torch.zeros((num_pages, n_kv_heads, page_size, d_nope), dtype=bf, device=dev)
                self.kpe_pages = torch.zeros((num_pages, hpe, page_size, d_rope), dtype=bf, device=dev)
            else:
                self.k_pages = torch.zeros((num_pages, n_kv_heads, page_size, d_rope), dtype=bf, device=dev)
            self.v_pages = torch.zeros((num_pages, n_kv_heads, page_size, d_v), dtype=bf, device=dev)
            self.scratch = torch.empty(scratch_bytes, dtype=torch.uint8, device=dev)
            self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
            st = L.akv_pool_create(ctypes.byref(lay), _ptr(order) if order is not None else None,
                                   _dptr(self.k_pages), _dptr(self.kpe_pages), _dptr(self.v_pages),
                                   _dptr(self.scratch), scratch_bytes, self.stream.cuda_stream,
                                   ctypes.byref(h))
        else:
            st = L.akv_pool_create(ctypes.byref(lay), _ptr(order) if order is not None else None,
                                   None, None, None, None, 0, None, ctypes.byref(h))
        _check(st)
        self._h = h

    # -- lifetime -------------------------------------------------------------
    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().akv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- sequences -------------------------------------------------------------
    def seq_create(self) -> int:
        s = ctypes.c_int32()
        _check(lib().akv_seq_create(self._h, ctypes.byref(s)))
        return s.value

    def seq_release(self, seq: int) -> None:
        _check(lib().akv_seq_release(self._h, seq))

    # -- shape checks of device tensors (the C ABI cannot see buffer sizes) -------
    def _check_kv(self, n: int, k, kpe, v) -> None:
        L = self.layout
        if k is None and kpe is None and v is None:
            return
        import torch
        hpe = (L["n_kv_heads"] if L["kpe_per_head"] else 1) if L["d_nope"] else 0
        want_k = (n, L["n_kv_heads"], L["d_nope"] if L["d_nope"] else L["d_rope"])
        for name, t, shape in (("K", k, want_k), ("V", v, (n, L["n_kv_heads"], L["d_v"])),
                               ("K_pe", kpe, (n, hpe, L["d_rope"]) if L["d_nope"] else None)):
            if shape is None:
                if t is not None:
                    raise ValueError("K_pe is only taken by MLA layouts")
                continue
            if t is None or tuple(t.shape) != shape or t.dtype != torch.bfloat16 or not t.is_cuda:
                raise ValueError(f"{name} must be a bf16 device tensor of shape {shape}")

    # -- cache ops ---------------------------------------------------------------
    def append(self, seq: int, pos, k=None, kpe=None, v=None) -> None:
        pos = _i32(pos)
        self._check_kv(len(pos), k, kpe, v)
        _check(lib().akv_append(self._h, seq, _dptr(k), _dptr(kpe), _dptr(v), _ptr(pos), len(pos)))

    def append_batch(self, seqs, counts, pos, k=None, kpe=None, v=None) -> None:
        """counts[i] tokens to seqs[i] for every entry, rows concatenated in
        entry order (akv_append_batch: one kernel launch)."""
        sq, cn, pos = _i32(seqs).reshape(-1), _i32(counts).reshape(-1), _i32(pos).reshape(-1)
        if len(sq) != len(cn) or int(cn.astype(np.int64).sum()) != len(pos):
            raise ValueError("one count per sequence entry, and one position per token")
        self._check_kv(len(pos), k, kpe, v)
        _check(lib().akv_append_batch(self._h, len(sq), _ptr(sq), _ptr(cn), _dptr(k), _dptr(kpe), _dptr(v),
                                      _ptr(pos)))

    def drop(self, seq: int, spans) -> None:
        sp = _i32(spans).reshape(-1, 2)
        _check(lib().akv_drop(self._h, seq, _ptr(sp), len(sp)))

    def compact(self, seq: int, force: bool = True) -> None:
        _check(lib().akv_compact(self._h, seq, int(bool(force))))

    def fused_rotation(self, mode: str) -> None:
        """Where akv_seq_attention applies owed rotations: "auto", "always" or "never"."""
        _check(lib().akv_fused_rotation(self._h, {"auto": 0, "always": 1, "never": 2}[mode]))

    def compaction_mode(self, deferred: bool) -> None:
        """Deferred: drops and splices queue fragmented sequences instead of
        compacting them (akv_compaction_mode)."""
        _check(lib().akv_compaction_mode(self._h, int(bool(deferred))))

    def compact_pending(self, max_tokens: int, max_seqs: int = 1 << 30) -> list:
        """Compact queued sequences within the budget; returns their ids."""
        n = ctypes.c_int32()
        out = np.zeros(max(min(max_seqs, len(self.compact_queue())), 1), np.int32)
        _check(lib().akv_compact_pending(self._h, int(max_tokens), min(max_seqs, len(out)), _ptr(out),
                                         ctypes.byref(n)))
        return out[: n.value].tolist()

    def compact_queue(self) -> list:
        n = ctypes.c_int32()
        _check(lib().akv_compact_queue(self._h, None, 0, ctypes.byref(n)))
        out = np.zeros(max(n.value, 1), np.int32)
        _check(lib().akv_compact_queue(self._h, _ptr(out), n.value, ctypes.byref(n)))
        return out[: n.value].tolist()

    def repos(self, seq: int, spans, deltas) -> None:
        sp = _i32(spans).reshape(-1, 2)
        dl = _i32(deltas).reshape(-1)
        _check(lib().akv_repos(self._h, seq, _ptr(sp), _ptr(dl), len(sp)))

    def repos_batch(self, entries) -> None:
        """entries: (seq, spans [m, 2], deltas [m]) per distinct sequence; one
        call and one rotation launch (akv_repos_batch)."""
        sq, cnt, sps, dls = [], [], [], []
        for seq, spans, deltas in entries:
            sp = _i32(spans).reshape(-1, 2)
            dl = _i32(deltas).reshape(-1)
            if len(sp) != len(dl):
                raise ValueError("one delta per span")
            sq.append(seq)
            cnt.append(len(sp))
            sps.append(sp)
            dls.append(dl)
        sq, cnt = _i32(sq), _i32(cnt)
        sp = np.concatenate(sps) if sps else np.zeros((0, 2), np.int32)
        dl = np.concatenate(dls) if dls else np.zeros(0, np.int32)
        _check(lib().akv_repos_batch(self._h, len(sq), _ptr(sq), _ptr(cnt), _ptr(sp), _ptr(dl)))

    def repos_deferred(self, seq: int, spans, deltas) -> None:
        """repos without rewriting keys: positions move, keys owe the rotation
        (akv_repos_deferred)."""
        sp = _i32(spans).reshape(-1, 2)
        dl = _i32(deltas).reshape(-1)
        _check(lib().akv_repos_deferred(self._h, seq, _ptr(sp), _ptr(dl), len(sp)))

    def materialize(self, seq: int) -> None:
        _check(lib().akv_materialize(self._h, seq))

    def lag(self, seq: int) -> np.ndarray:
        n, _, _ = self.info(seq)
        out = np.zeros(max(n, 1), np.int32)
        _check(lib().akv_seq_lag(self._h, seq, 0, n, _ptr(out)))
        return out[:n]

    def freeze(self, seq: int) -> None:
        _check(lib().akv_seq_freeze(self._h, seq))

    def share(self, src: int, first: int, n: int, dst: int, delta: int = 0) -> None:
        _check(lib().akv_seq_share(self._h, src, first, n, dst, delta))

    def attention_mass(self, mass) -> None:
        """Per-page attention mass of decode launches added to `mass` (a
        device float32 tensor of num_pages entries), or None to stop
        (akv_attention_mass).  The tensor must outlive its use."""
        if mass is None:
            _check(lib().akv_attention_mass(self._h, None, 0))
            self._mass = None
            return
        import torch
        if mass.dtype != torch.float32 or mass.numel() != self.layout["num_pages"]:
            raise ValueError("mass must be float32 with one entry per page")
        _check(lib().akv_attention_mass(self._h, _dptr(mass), mass.numel()))
        self._mass = mass

    def clone(self, src: int, first: int, n: int, dst: int, delta: int) -> None:
        """Positional version: append src's retained tokens [first, first+n)
        to dst at pos + delta, keys turned by R(delta) (akv_seq_clone)."""
        _check(lib().akv_seq_clone(self._h, src, first, n, dst, delta))

    def repos_plan(self, seq: int, spans, deltas):
        sp = _i32(spans).reshape(-1, 2)
        dl = _i32(deltas).reshape(-1)
        n = ctypes.c_int32()
        st = lib().akv_repos_plan(self._h, seq, _ptr(sp), _ptr(dl), len(sp), None, None, 0, ctypes.byref(n))
        if st not in (AKV_OK, AKV_ERANGE):
            _check(st)
        slot = np.zeros(max(n.value, 1), np.int32)
        delta = np.zeros(max(n.value, 1), np.int32)
        _check(lib().akv_repos_plan(self._h, seq, _ptr(sp), _ptr(dl), len(sp), _ptr(slot), _ptr(delta),
                                    n.value, ctypes.byref(n)))
        return slot[: n.value], delta[: n.value]

    def attention_plan(self, n_q_tokens: int, segments, page_lists, n_cu: int = 0):
        """Dry run of the attention planner (akv_attention_plan): returns
        (items [n, 6] = seg, kv_head, row0, k_begin, k_end, part in grid order;
        combine [m, 6] = seg, kv_head, row0, part0, n_split, rows;
        rows_per_block, partial rows)."""
        sg = _i32(segments).reshape(-1, 4)
        ex = _i32(page_lists).reshape(-1, 3)
        ni, nc, rb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        pr = ctypes.c_int64()
        args = (self._h, int(n_q_tokens), _ptr(sg), len(sg), _ptr(ex), len(ex), int(n_cu))
        _check(lib().akv_attention_plan(*args, None, 0, ctypes.byref(ni), None, 0, ctypes.byref(nc),
                                        ctypes.byref(rb), ctypes.byref(pr)))
        items = np.zeros((max(ni.value, 1), 6), np.int32)
        comb = np.zeros((max(nc.value, 1), 6), np.int32)
        _check(lib().akv_attention_plan(*args, _ptr(items), ni.value, ctypes.byref(ni), _ptr(comb), nc.value,
                                        ctypes.byref(nc), ctypes.byref(rb), ctypes.byref(pr)))
        return items[: ni.value], comb[: nc.value], rb.value, pr.value

    def splice(self, seq: int, spans, stub_lens, k=None, kpe=None, v=None) -> np.ndarray:
        sp = _i32(spans).reshape(-1, 2)
        sl = _i32(stub_lens).reshape(-1)
        out = np.zeros(max(int(sl.sum()), 1), np.int32)
        if len(sl) and (sl < 0).any():
            raise ValueError("negative stub length")
        self._check_kv(int(sl.sum()), k, kpe, v)
        _check(lib().akv_splice(self._h, seq, _ptr(sp), _ptr(sl), len(sp), _dptr(k), _dptr(kpe), _dptr(v),
                                _ptr(out)))
        return out[: int(sl.sum())]

    # -- visibility --------------------------------------------------------------
    def visible(self, seq: int, mask=None) -> np.ndarray:
        """Extents (page, lo, hi) of the visible list, optionally minus mask spans."""
        m = _i32(mask if mask is not None else np.zeros((0, 2))).reshape(-1, 2)
        n = ctypes.c_int32()
        cap = getattr(self, "_vis_cap", 4096)    # the largest list seen so far: one call as a rule
        while True:
            out = np.empty((cap, 3), np.int32)
            st = lib().akv_seq_visible(self._h, seq, _ptr(m), len(m), _ptr(out), cap, ctypes.byref(n))
            if st == AKV_ERANGE and n.value > cap:
                cap = self._vis_cap = n.value
                continue
            _check(st)
            return out[: n.value]

    def tokens(self, seq: int):
        n, _, _ = self.info(seq)
        slot, pos = np.zeros(max(n, 1), np.int32), np.zeros(max(n, 1), np.int32)
        dropped = np.zeros(max(n, 1), np.uint8)
        _check(lib().akv_seq_tokens(self._h, seq, 0, n, _ptr(slot), _ptr(pos),
                                    dropped.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))))
        return slot[:n], pos[:n], dropped[:n].astype(bool)

    def info(self, seq: int):
        n, v, f = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_double()
        _check(lib().akv_seq_info(self._h, seq, ctypes.byref(n), ctypes.byref(v), ctypes.byref(f)))
        return n.value, v.value, f.value

    def queues(self):
        nf, ne = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().akv_pool_queues(self._h, None, 0, ctypes.byref(nf), None, 0, ctypes.byref(ne)))
        fr = np.zeros(max(nf.value, 1), np.int32)
        ev = np.zeros(max(ne.value, 1), np.int32)
        _check(lib().akv_pool_queues(self._h, _ptr(fr), nf.value, ctypes.byref(nf), _ptr(ev), ne.value,
                                     ctypes.byref(ne)))
        return fr[: nf.value], ev[: ne.value]

    # -- segment-batch attention -------------------------------------------------
    def segment_attention(self, q, segments, page_lists, scale: float = 0.0, out=None):
        """q: bf16 device tensor [Nq, Hq, d_nope + d_rope]; segments: rows of
        (q_begin, q_len, ext_begin, ext_len); page_lists: [n_ext, 3] extents.
        Returns out [Nq, Hq, d_v] (bf16; rows no segment covers are left as is)."""
        import torch
        sg = _i32(segments).reshape(-1, 4)
        ex = _i32(page_lists).reshape(-1, 3)
        L = self.layout
        if q.dim() != 3 or q.shape[1] != L["n_q_heads"] or q.shape[2] != L["d_nope"] + L["d_rope"] \
                or q.dtype != torch.bfloat16:
            raise ValueError("q must be bf16 [Nq, n_q_heads, d_nope + d_rope]")
        if out is None:
            out = torch.zeros((q.shape[0], q.shape[1], L["d_v"]), dtype=torch.bfloat16, device=q.device)
        if tuple(out.shape) != (q.shape[0], L["n_q_heads"], L["d_v"]) or out.dtype != torch.bfloat16:
            raise ValueError("out must be bf16 [Nq, n_q_heads, d_v]")
        _check(lib().akv_segment_attention(self._h, _dptr(q), q.shape[0], _ptr(sg), len(sg), _ptr(ex),
                                           len(ex), float(scale), _dptr(out)))
        return out

    def segment_attention_static(self, q, segments, page_lists, out, scale: float = 0.0):
        """akv_segment_attention_static: segment_attention with the call's
        tables in the library's static device workspace (no allocation); out
        is the caller's bf16 tensor [Nq, Hq, d_v]."""
        import torch
        sg = _i32(segments).reshape(-1, 4)
        ex = _i32(page_lists).reshape(-1, 3)
        L = self.layout
        if q.dim() != 3 or q.shape[1] != L["n_q_heads"] or q.shape[2] != L["d_nope"] + L["d_rope"] \
                or q.dtype != torch.bfloat16:
            raise ValueError("q must be bf16 [Nq, n_q_heads, d_nope + d_rope]")
        if tuple(out.shape) != (q.shape[0], L["n_q_heads"], L["d_v"]) or out.dtype != torch.bfloat16:
            raise ValueError("out must be bf16 [Nq, n_q_heads, d_v]")
        _check(lib().akv_segment_attention_static(self._h, _dptr(q), q.shape[0], _ptr(sg), len(sg), _ptr(ex),
                                                  len(ex), float(scale), _dptr(out)))
        return out

    def seq_attention(self, q, segments, scale: float = 0.0, out=None):
        """Attention over sequences' own visible lists (akv_seq_attention):
        segments are (seq, q_begin, q_len, mask_spans) with mask_spans an
        [m, 2] array of logical spans hidden from that segment (or None), or,
        when no segment hides spans, an int [n, 3] array of (seq, q_begin,
        q_len) rows."""
        import torch
        if isinstance(segments, np.ndarray):
            a = np.asarray(segments).reshape(-1, 3)
            sg = np.zeros((len(a), 5), np.int32)
            sg[:, :3] = a
            ms = _NO_SPANS
        else:
            rows, spans = [], []
            for seq, qb, ql, m in segments:
                if m is None or len(m) == 0:
                    rows.append((seq, qb, ql, len(spans), 0))
                    continue
                m = _i32(m).reshape(-1, 2)
                rows.append((seq, qb, ql, len(spans), len(m)))
                spans.extend(m.tolist())
            sg = np.asarray(rows, np.int32).reshape(-1, 5)
            ms = np.asarray(spans, np.int32).reshape(-1, 2)
        L = self.layout
        if q.dim() != 3 or q.shape[1] != L["n_q_heads"] or q.shape[2] != L["d_nope"] + L["d_rope"] \
                or q.dtype != torch.bfloat16:
            raise ValueError("q must be bf16 [Nq, n_q_heads, d_nope + d_rope]")
        if out is None:
            out = torch.zeros((q.shape[0], q.shape[1], L["d_v"]), dtype=torch.bfloat16, device=q.device)
        if tuple(out.shape) != (q.shape[0], L["n_q_heads"], L["d_v"]) or out.dtype != torch.bfloat16:
            raise ValueError("out must be bf16 [Nq, n_q_heads, d_v]")
        _check(lib().akv_seq_attention(self._h, _dptr(q), q.shape[0], _ptr(sg), len(sg), _ptr(ms), len(ms),
                                       float(scale), _dptr(out)))
        return out

    # -- timing / sync -------------------------------------------------------------
    def timing_enable(self, on: bool = True) -> None:
        _check(lib().akv_timing_enable(self._h, int(on)))

    def timing_samples(self, kind: str) -> np.ndarray:
        """Each launch's milliseconds since the last timing_read of this kind."""
        n = ctypes.c_int32()
        st = lib().akv_timing_samples(self._h, KERNEL_KINDS[kind], None, 0, ctypes.byref(n))
        if st not in (AKV_OK, AKV_ERANGE):
            _check(st)
        out = np.zeros(max(n.value, 1), np.float32)
        _check(lib().akv_timing_samples(self._h, KERNEL_KINDS[kind],
                                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), len(out),
                                        ctypes.byref(n)))
        return out[: n.value]

    def timing_read(self, kind: str):
        ms, cnt = ctypes.c_double(), ctypes.c_int32()
        _check(lib().akv_timing_read(self._h, KERNEL_KINDS[kind], ctypes.byref(ms), ctypes.byref(cnt)))
        return ms.value, cnt.value

    def sync(self) -> None:
        _check(lib().akv_sync(self._h))


def repos_layers(pools, seq: int, spans, deltas) -> None:
    """akv_repos_layers: the same repos on every pool (one pool per model
    layer, same op history and stream), rotated in one kernel launch."""
    pools = list(pools)
    hs = (_P * len(pools))(*[p._h.value for p in pools])
    sp = _i32(spans).reshape(-1, 2)
    dl = _i32(deltas).reshape(-1)
    _check(lib().akv_repos_layers(hs, len(pools), seq, _ptr(sp), _ptr(dl), len(sp)))


class Tree:
    """Extended radix tree of cached states (akv_tree_*): histories are
    [n, 4] int32 event rows (kind, a, b, c): EV_TOKEN (id, position),
    EV_DROP [a, b), EV_REPOS [a, b) by c."""

    def __init__(self):
        h = _P()
        _check(lib().akv_tree_create(ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if self._h:
            lib().akv_tree_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _events(ev) -> np.ndarray:
        return _i32(ev).reshape(-1, 4)

    def insert(self, events, seq: int) -> None:
        ev = self._events(events)
        _check(lib().akv_tree_insert(self._h, _ptr(ev), len(ev), seq))

    def match(self, events) -> dict:
        ev = self._events(events)
        out = np.zeros(5, np.int32)
        _check(lib().akv_tree_match(self._h, _ptr(ev), len(ev), _ptr(out)))
        return dict(seq=int(out[0]), n_events=int(out[1]), n_tokens=int(out[2]), exact=int(out[3]),
                    delta=int(out[4]))

    def pin(self, seq: int, add: int = 1) -> None:
        _check(lib().akv_tree_pin(self._h, seq, add))

    def evict(self, max_n: int) -> list:
        out = np.zeros(max(max_n, 1), np.int32)
        n = ctypes.c_int32()
        _check(lib().akv_tree_evict(self._h, max_n, _ptr(out), ctypes.byref(n)))
        return out[: n.value].tolist()

    def stats(self):
        a, b = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().akv_tree_stats(self._h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value
