// Host runtime and C ABI of the AKV hot path (include/akv.h).
//
// Holds the page allocator, per-sequence token tables (slot, position, drop
// flag), the visible-list / page-table builder, the repos and attention
// planners, a pinned staging ring for host->device metadata, and the launches
// of the HIP kernels in akv_kernels.hip and akv_copy.hip.
//
// Sources, cited by page title and section:
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and State-Preserving
//               Prefix Invalidation Bypass" (A. Akhunji)
//   [AKV-notes] "Cache Engineering for Agents" (reading notes on Fu et al.)
//   [Leyline]   "Leyline: KV Cache Directives for Agentic Inference" (digest)
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <initializer_list>
#include <utility>
#include <vector>

#include "../../include/akv.h"
#include "akv_internal.h"

namespace {

thread_local std::string g_err;

akv_status fail(akv_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

void akv::set_error(const char* msg) { g_err = msg; }

akv::LaunchEvents& akv::launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

namespace {

akv_status hip_fail(hipError_t e, const char* what) {
  return fail(AKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr double kDefaultCompactThreshold = 0.40;
constexpr int64_t kInt32Max = 2147483647LL;

// Debug switches, read from the environment once per process:
//   AKV_TRACE=1             one line on stderr per planning decision
//                           (attention plans, rotations, copies, compaction)
//   AKV_CHECKS=1            every device work list is checked on the host
//                           before its launch (also in page-table-only pools,
//                           which build the lists without launching them):
//                           slots inside the pool and in pages in use, rows
//                           inside their page, rotate items disjoint, copy
//                           destinations distinct and apart from the sources,
//                           attention items inside their segment and list and
//                           covering each row tile's keys exactly once.  A
//                           failed check is a library bug: the call returns
//                           AKV_ESTATE and the pool's state is undefined.
//   AKV_FAULT_INJECT=launch every kernel launch reports failure once it is
//                           enqueued (the kernel itself runs normally), so each
//                           call takes its AKV_EHIP error path: for tests of
//                           error handling.
//   AKV_COMPACT_THRESHOLD=x fragmentation threshold (0 < x <= 1) of pools
//                           whose layout leaves compact_threshold at 0.
struct DebugFlags {
  bool trace = false, checks = false, inject_launch = false;
  double thr = kDefaultCompactThreshold;
};

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && *v && std::strcmp(v, "0") != 0;
}

const DebugFlags& dbg() {
  static const DebugFlags flags = [] {
    DebugFlags f;
    f.trace = env_on("AKV_TRACE");
    f.checks = env_on("AKV_CHECKS");
    const char* fi = std::getenv("AKV_FAULT_INJECT");
    f.inject_launch = fi && std::strcmp(fi, "launch") == 0;
    if (const char* t = std::getenv("AKV_COMPACT_THRESHOLD")) {
      char* end = nullptr;
      const double x = std::strtod(t, &end);
      if (end != t && x > 0.0 && x <= 1.0) f.thr = x;
    }
    return f;
  }();
  return flags;
}

void trace(const char* fmt, ...) {
  if (!dbg().trace) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "akv: %s\n", buf);
}

akv_status check_fail(const char* fmt, ...) {
  char buf[448];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  trace("AKV_CHECKS failed: %s", buf);
  return fail(AKV_ESTATE, "AKV_CHECKS: %s", buf);
}

struct PageRec {
  int32_t owner = -1;   // sequence id, -1 when free
  int32_t nvis = 0;     // visible tokens held
  int32_t filled = 0;   // slots written
  bool in_evict = false;
  uint32_t evict_gen = 0;
  uint32_t take_gen = 0;   // bumped each time the page is taken by a sequence
  std::vector<int32_t> toks;   // tokens of the owner whose slot is in this page
};

struct SeqRec {
  std::vector<int32_t> slot, pos;
  std::vector<uint8_t> dropped;
  // rotation each stored key still owes (position minus the position its key
  // encodes): nonzero only after a deferred repos, until it is materialized
  std::vector<int32_t> lag;
  bool lagging = false;        // some token may have lag != 0
  // owned pages in allocation order; an entry (page, take_gen) is live while
  // the page still carries that generation (evicted pages leave stale
  // entries behind, dropped in bulk once they are half of the list)
  std::vector<std::pair<int32_t, uint32_t>> pages;
  size_t stale_pages = 0;
  int32_t tail = -1;           // open page, or -1
  bool alive = true;
  int64_t n_vis = 0;
  std::vector<int32_t> vis;    // cached visible order
  bool vis_ok = false;
  bool vis_logical = false;    // vis is in logical order (positions never decrease along it)
  std::vector<akv_extent> ext; // cached page-table image of vis (valid with ext_ok)
  bool ext_ok = false;
  // the same image with runs also cut where the owed rotation changes, and
  // each extent's owed rotation (valid with lg_ok)
  std::vector<akv_extent> ext_lg;
  std::vector<int32_t> ext_lg_lag;
  bool lg_ok = false;
  bool queued = false;         // waiting in the deferred-compaction queue
  // Shared pages (akv_seq_share): a frozen sequence is a checkpoint whose
  // rows never change; other sequences hold tokens whose slots lie in its
  // pages (foreign slots: the page's owner is another sequence).
  int32_t id = -1;
  bool frozen = false;
  int32_t refs = 0;             // sequences holding slots in this sequence's pages
  bool zombie = false;          // released while referenced: pages kept until refs reach 0
  std::unordered_map<int32_t, int32_t> owners;  // owner sequence -> this sequence's tokens in its pages
  std::unordered_map<int32_t, int32_t> fvis;    // foreign page -> this sequence's visible tokens in it
  void stale() { vis_ok = ext_ok = lg_ok = false; }
};

// Pinned host ring for metadata uploads (coherent and mapped: small tables
// are also read by kernels straight from it).  A region may be rewritten once
// the copy or the kernels that read it have finished (its event completed).
struct Staging {
  char* base = nullptr;
  char* dbase = nullptr;   // the same memory as the device addresses it (mapped), or NULL
  size_t cap = 0, head = 0;
  struct Region {
    size_t b, e;
    hipEvent_t ev;
  };
  std::deque<Region> pending;
  std::vector<hipEvent_t> spare;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

// Host lists of an attention call, kept by the pool so their capacity
// persists from call to call (calls on one pool are not re-entrant).
// Launch plan of one attention call, and the planner's working space (kept
// in the pool between calls, so a steady decode loop allocates nothing).
struct AttnPlan {
  std::vector<akv::AttnSeg> segs;
  std::vector<akv::AttnItem> items;  // grid order (XCD interleaved, padded)
  std::vector<akv::CombItem> comb;
  int64_t part_rows = 0;  // rows of split-KV partials
  // Items of one group (same segment, kv head and key split: the row tiles
  // that read the same K/V) are contiguous in `all`; a group is its range.
  struct Group {
    int64_t cost;
    int32_t begin, end;
  };
  std::vector<akv::AttnItem> all;
  std::vector<int64_t> cost;
  std::vector<Group> groups, gtmp;
  std::vector<int32_t> nsplit;                          // key splits of each segment
  std::vector<int32_t> split_kb, split_ke;              // one segment's key splits
  std::vector<int64_t> tile_base, tile_rows, tile_lim;  // one segment's row tiles
  std::vector<int32_t> gbin, order;
  std::vector<uint32_t> cnt;
};

struct AttnHostBufs {
  std::vector<char> static_up;   // tables of a static-workspace call, before their copy
  std::vector<akv_extent> lists, masked;
  std::vector<int32_t> lags, mlag, ex_off, ex_didx;
  std::vector<akv::Extent> ex_used;
  std::vector<akv::MassItem> mass_items;
  AttnPlan plan;
};

struct akv_pool {
  akv_layout L{};
  std::vector<double> inv_freq;
  int log2S = 0;
  bool device = false;
  uint16_t* k = nullptr;    // GQA K / MLA K_nope
  uint16_t* kpe = nullptr;  // MLA K_pe
  uint16_t* v = nullptr;
  char* scratch = nullptr;
  size_t scratch_bytes = 0;
  size_t scratch_base = 0;  // first byte available to a call
  hipStream_t stream = nullptr;
  // While the pool stream is busy, metadata uploads run on their own stream,
  // so a call's tables arrive while the kernels of earlier calls still run;
  // the pool stream waits for each such upload.  Per-call scratch is taken
  // round-robin from [scratch_base, scratch_bytes), and an upload into a
  // range waits (on the copy stream) for the last call that used the range.
  hipStream_t cstream = nullptr;
  size_t ring_head = 0;
  struct RingUse {
    size_t b0, e0, b1, e1;   // at most two ranges (a call may wrap once)
    bool bg;                 // read by a background-compaction launch (kstream)
  };
  std::deque<RingUse> ring_uses;
  // Background compaction ([AKV-blog] section 7, Dilemma 2: defragmentation
  // runs asynchronously, without pausing inference): akv_compact_pending
  // launches its copies on kstream (default priority), ordered after the pool
  // stream's earlier work; bg_done follows the last of them.  Until the pool
  // stream waits for bg_done, the pages those copies read or write are
  // flagged, and pool-stream work touching a flagged page waits first; other
  // work runs beside the copies.
  hipStream_t kstream = nullptr;
  hipEvent_t bg_done = nullptr;
  bool bg_pending = false;
  // Points of the pool stream the background copies are ordered after: the
  // end of the last launch that wrote pool rows, and the end of the work
  // enqueued before the last call that gave pages back to the queues (work
  // that may still read those pages).  Later pool-stream work is not waited
  // for, so the copies run beside it.
  hipEvent_t write_ev = nullptr, free_ev = nullptr;
  bool write_set = false, free_set = false;
  std::vector<uint8_t> page_bg;
  std::vector<int32_t> bg_pages;
  int n_cu = 256;
  double thr = kDefaultCompactThreshold;
  int compact_mode = AKV_COMPACT_IMMEDIATE;
  int fuse_mode = AKV_FUSE_AUTO;   // where owed rotations are applied (akv_fused_rotation)
  float* mass = nullptr;           // per-page attention mass of decode launches (akv_attention_mass)
  std::deque<int32_t> compact_q;   // deferred compactions, in the order queued

  std::deque<int32_t> free_q;
  std::deque<std::pair<int32_t, uint32_t>> evict_q;
  int64_t n_evict = 0;
  std::vector<PageRec> pages;
  std::vector<SeqRec> seqs;

  Staging stg;
  AttnHostBufs hb;

  bool timing = false;
  struct TEv {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<TEv> tev;
  std::vector<hipEvent_t> ev_spare;
  double t_ms[AKV_K_KINDS] = {};
  int t_cnt[AKV_K_KINDS] = {};
  std::vector<float> t_each[AKV_K_KINDS];   // each launch's milliseconds since the last read

  // cos / sin rows of recently used deltas (rotation tables are formed on the
  // host and uploaded with each call's work list)
  std::unordered_map<int32_t, std::vector<float>> rot_cache;
  std::vector<float> rot_tab;

  int rope_heads() const { return (L.d_nope > 0 && !L.kpe_per_head) ? 1 : L.n_kv_heads; }
  uint16_t* rope_array() const { return L.d_nope > 0 ? kpe : k; }
};

namespace {

// ---------------------------------------------------------------------------
// staging + upload
// ---------------------------------------------------------------------------
hipError_t stg_event(akv_pool* p, hipEvent_t* ev) {
  if (!p->stg.spare.empty()) {
    *ev = p->stg.spare.back();
    p->stg.spare.pop_back();
    return hipSuccess;
  }
  return hipEventCreateWithFlags(ev, hipEventDisableTiming);
}

// Reserve n bytes of pinned staging (16-byte aligned).
akv_status stg_reserve(akv_pool* p, size_t n, char** out) {
  Staging& s = p->stg;
  n = align_up(std::max<size_t>(n, 16), 256);
  if (n > s.cap) {
    hipError_t e = hipStreamSynchronize(p->cstream);
    if (e == hipSuccess) e = hipStreamSynchronize(p->stream);
    if (e == hipSuccess && p->kstream) e = hipStreamSynchronize(p->kstream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    for (auto& r : s.pending) s.spare.push_back(r.ev);
    s.pending.clear();
    if (s.base) (void)hipHostFree(s.base);
    s.base = nullptr;
    // room for several calls in flight, so refills rarely wait on the GPU
    size_t cap = std::max<size_t>({4 * n, 2 * s.cap, (size_t)8 << 20});
    e = hipHostMalloc((void**)&s.base, cap, hipHostMallocMapped | hipHostMallocCoherent);
    if (e != hipSuccess) {
      s.cap = 0;
      return hip_fail(e, "hipHostMalloc(staging)");
    }
    s.dbase = nullptr;
    if (hipHostGetDevicePointer((void**)&s.dbase, s.base, 0) != hipSuccess) s.dbase = nullptr;
    (void)hipGetLastError();
    s.cap = cap;
    s.head = 0;
  }
  if (s.head + n > s.cap) s.head = 0;
  const size_t b = s.head, e_ = s.head + n;
  // Wait for the newest pending region overlapping [b, e_) and every region
  // before it.  Their events come from two streams, so a newer one having
  // completed says nothing of an older one: each is synchronized (at no cost
  // once it has completed).
  int last = -1;
  for (int i = 0; i < (int)s.pending.size(); ++i)
    if (s.pending[i].b < e_ && b < s.pending[i].e) last = i;
  for (int i = 0; i <= last; ++i) {
    hipError_t e = hipEventSynchronize(s.pending.front().ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(staging)");
    s.spare.push_back(s.pending.front().ev);
    s.pending.pop_front();
  }
  s.head = e_;
  *out = s.base + b;
  return AKV_OK;
}

// Copy a filled staging region to device memory on the pool stream.
// While the pool stream still has work queued, the copy runs on the copy
// stream and the pool stream waits for it: the copy then overlaps the
// earlier kernels.  On an idle pool stream the copy is enqueued there
// directly (fewer calls, no cross-queue wait).  Either way the call's
// kernels, enqueued after this, see the data.
akv_status stg_upload(akv_pool* p, const char* host, void* dev, size_t n) {
  if (n == 0) return AKV_OK;
  const bool overlap = hipStreamQuery(p->stream) == hipErrorNotReady;
  (void)hipGetLastError();   // "not ready" is a status, not an error for the launch checks that follow
  hipStream_t cs = overlap ? p->cstream : p->stream;
  hipError_t e = hipMemcpyAsync(dev, host, n, hipMemcpyHostToDevice, cs);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(H2D)");
  hipEvent_t ev;
  e = stg_event(p, &ev);
  if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
  e = hipEventRecord(ev, cs);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  const size_t off = (size_t)(host - p->stg.base);
  p->stg.pending.push_back({off, off + align_up(std::max<size_t>(n, 16), 256), ev});
  if (overlap) {
    e = hipStreamWaitEvent(p->stream, ev, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  return AKV_OK;
}

// Before a range is written by an upload (which may run on the copy
// stream), the copy stream waits until every earlier call that used bytes of
// [b, e) has finished on the pool stream; those calls are then forgotten.
// The calls' ranges carry no event: one recorded now on the pool stream
// follows all of their kernels (the pool stream is in order).
void ring_wait(akv_pool* p, size_t b, size_t e, bool bg_upload = false) {
  auto& u = p->ring_uses;
  int last = -1;
  for (int i = 0; i < (int)u.size(); ++i)
    if ((u[i].b0 < e && b < u[i].e0) || (u[i].b1 < e && b < u[i].e1)) last = i;
  // keep the list short: also retire the oldest calls once it grows long
  if (last < 0 && u.size() > 256) last = 127;
  if (last < 0) return;
  hipEvent_t ev;
  if (stg_event(p, &ev) == hipSuccess) {
    if (hipEventRecord(ev, p->stream) == hipSuccess) {
      (void)hipStreamWaitEvent(p->cstream, ev, 0);
      if (bg_upload) (void)hipStreamWaitEvent(p->kstream, ev, 0);   // the upload runs on kstream
    }
    p->stg.spare.push_back(ev);
  }
  // a range a background copy reads: the upload (on either stream) waits for
  // the background stream's last launch
  for (int i = 0; i <= last; ++i)
    if (u[i].bg) {
      (void)hipStreamWaitEvent(p->cstream, p->bg_done, 0);
      (void)hipStreamWaitEvent(p->stream, p->bg_done, 0);
      break;
    }
  u.erase(u.begin(), u.begin() + last + 1);
}

// Per-call scratch, taken round-robin from [scratch_base, scratch_bytes):
// `need` (the call's bound, when known) starts the call at the ring's start
// if it does not fit before the end.  On destruction the call's ranges are
// recorded (ring_wait orders later uploads into them after its kernels).
struct ScratchCursor {
  akv_pool* p;
  size_t off;            // next byte
  size_t first = 0;      // the call's first byte
  bool bad = false, wrapped = false, any = false, bg = false;
  size_t r0b = 0, r0e = 0, r1b = 0, r1e = 0;
  explicit ScratchCursor(akv_pool* pp, size_t need = 0) : p(pp), off(pp->ring_head) {
    if (off < p->scratch_base || off + align_up(need, 256) > p->scratch_bytes) off = p->scratch_base;
    first = off;
  }
  ScratchCursor(const ScratchCursor&) = delete;
  ScratchCursor& operator=(const ScratchCursor&) = delete;
  char* take(size_t n) {
    const size_t m = align_up(std::max<size_t>(n, 1), 256);
    off = align_up(off, 256);
    if (off + m > p->scratch_bytes) {
      // wrap once; the new range must stay clear of this call's own bytes
      if (wrapped || p->scratch_base + m > first) {
        bad = true;
        return p->scratch + p->scratch_base;
      }
      wrapped = true;
      off = p->scratch_base;
    }
    if (!bad && p->device) ring_wait(p, off, off + m, bg);
    if (!wrapped) {
      if (!any) r0b = off;
      r0e = off + m;
    } else {
      if (r1e == 0) r1b = off;
      r1e = off + m;
    }
    any = true;
    char* r = p->scratch + off;
    off += m;
    return r;
  }
  bool ok() const { return !bad; }
  size_t needed() const { return bad ? p->scratch_bytes + 1 : off; }
  ~ScratchCursor() {
    if (!any || bad || !p->device) return;
    p->ring_uses.push_back({r0b, r0e, r1b, r1e, bg});
    p->ring_head = off;
  }
};

// ---------------------------------------------------------------------------
// timing
// ---------------------------------------------------------------------------
hipError_t tev_get(akv_pool* p, hipEvent_t* ev) {
  if (!p->ev_spare.empty()) {
    *ev = p->ev_spare.back();
    p->ev_spare.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(ev);
}

// Times the one launch made between construction and done(): the two events
// are armed for that launch, which carries them (stamped by the dispatch at
// the kernel's start and end; no packets of their own on the stream).
struct KTimer {
  akv_pool* p;
  int kind;
  hipEvent_t a = nullptr, b = nullptr;
  KTimer(akv_pool* pp, int k, hipStream_t = nullptr) : p(pp), kind(k) {
    if (p->timing && tev_get(p, &a) == hipSuccess && tev_get(p, &b) == hipSuccess) {
      akv::LaunchEvents& ev = akv::launch_events();
      ev.start = a;
      ev.stop = b;
      ev.used = false;
    } else {
      a = b = nullptr;
    }
  }
  void done() {
    if (!a || !b) return;
    akv::LaunchEvents& ev = akv::launch_events();
    if (ev.used) {
      p->tev.push_back({kind, a, b});
    } else {   // no launch took them (nothing to do)
      p->ev_spare.push_back(a);
      p->ev_spare.push_back(b);
    }
    ev = akv::LaunchEvents{};
    a = b = nullptr;
  }
  ~KTimer() { done(); }   // a path that returns early leaves no events armed
};

akv_status timing_collect(akv_pool* p) {
  if (p->tev.empty()) return AKV_OK;
  for (auto& t : p->tev) {   // launches of two streams: each end event on its own
    hipError_t e = hipEventSynchronize(t.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(timing)");
  }
  for (auto& t : p->tev) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.a, t.b) == hipSuccess) {
      p->t_ms[t.kind] += ms;
      p->t_cnt[t.kind] += 1;
      p->t_each[t.kind].push_back(ms);
    }
    p->ev_spare.push_back(t.a);
    p->ev_spare.push_back(t.b);
  }
  p->tev.clear();
  return AKV_OK;
}

// ---------------------------------------------------------------------------
// allocator
// ---------------------------------------------------------------------------
int64_t available(const akv_pool* p) { return (int64_t)p->free_q.size() + p->n_evict; }

void evict_push(akv_pool* p, int32_t pg) {
  PageRec& r = p->pages[pg];
  r.in_evict = true;
  r.evict_gen += 1;
  p->evict_q.emplace_back(pg, r.evict_gen);
  p->n_evict += 1;
}

void evict_unlink(akv_pool* p, int32_t pg) {  // entry becomes stale in the queue
  p->pages[pg].in_evict = false;
  p->n_evict -= 1;
}

int32_t evict_pop(akv_pool* p) {
  while (!p->evict_q.empty()) {
    auto [pg, gen] = p->evict_q.front();
    p->evict_q.pop_front();
    const PageRec& r = p->pages[pg];
    if (r.in_evict && r.evict_gen == gen) {
      evict_unlink(p, pg);
      return pg;
    }
  }
  return -1;
}

// A live entry of q's page list: the page was taken by q and not since.
inline bool page_live(const akv_pool* p, const std::pair<int32_t, uint32_t>& e);

// The page leaves q's list (its entry goes stale; the list drops stale
// entries, keeping the live ones in order, once they are half of it).
void remove_page_from_seq(akv_pool* p, SeqRec& q) {
  q.stale_pages += 1;
  if (2 * q.stale_pages < q.pages.size()) return;
  size_t w = 0;
  for (const auto& e : q.pages)
    if (page_live(p, e)) q.pages[w++] = e;
  q.pages.resize(w);
  q.stale_pages = 0;
}

// Reclaim an evictable page: its tokens (all dropped) lose their slot.
void evict_page(akv_pool* p, int32_t pg) {
  PageRec& r = p->pages[pg];
  SeqRec& o = p->seqs[r.owner];
  for (int32_t t : r.toks) o.slot[t] = -1;
  r.toks.clear();
  r.take_gen += 1;   // o's entry for the page goes stale
  remove_page_from_seq(p, o);
}

int32_t take_page(akv_pool* p, int32_t s) {
  int32_t pg;
  if (!p->free_q.empty()) {
    pg = p->free_q.front();
    p->free_q.pop_front();
  } else {
    pg = evict_pop(p);
    evict_page(p, pg);
  }
  PageRec& r = p->pages[pg];
  r.owner = s;
  r.nvis = 0;
  r.filled = 0;
  r.toks.clear();
  r.toks.reserve(p->L.page_size);   // one allocation per page record, kept across reuse
  r.take_gen += 1;
  p->seqs[s].pages.emplace_back(pg, r.take_gen);
  return pg;
}

inline bool page_live(const akv_pool* p, const std::pair<int32_t, uint32_t>& e) {
  return p->pages[e.first].take_gen == e.second;
}

int64_t pages_needed(const akv_pool* p, const SeqRec& q, int64_t n) {
  const int64_t S = p->L.page_size;
  const int64_t room = q.tail >= 0 ? S - p->pages[q.tail].filled : 0;
  const int64_t extra = std::max<int64_t>(0, n - room);
  return (extra + S - 1) / S;
}

// Slots for n new tokens of sequence s (tail page first, then fresh pages).
void place_tokens(akv_pool* p, int32_t s, int32_t n, const int32_t* pos, int32_t* slots_out) {
  SeqRec& q = p->seqs[s];
  const int32_t S = p->L.page_size;
  const int32_t t0 = (int32_t)q.slot.size();
  for (int32_t i = 0; i < n; ++i) {
    if (q.tail < 0) q.tail = take_page(p, s);
    const int32_t pg = q.tail;
    PageRec& r = p->pages[pg];
    const int32_t slot = pg * S + r.filled;
    r.filled += 1;
    r.nvis += 1;
    r.toks.push_back(t0 + i);
    if (r.filled == S) q.tail = -1;
    slots_out[i] = slot;
    q.slot.push_back(slot);
    q.pos.push_back(pos[i]);
    q.dropped.push_back(0);
    q.lag.push_back(0);
    // a token placed at or after the last visible position extends the
    // cached visible order (and its extents) at the end
    if (q.vis_ok) {
      if (q.vis.empty() || pos[i] >= q.pos[q.vis.back()]) {
        q.vis.push_back(t0 + i);
        const int32_t off = slot - pg * S;
        if (q.ext_ok) {
          if (!q.ext.empty() && q.ext.back().page == pg && q.ext.back().hi == off)
            q.ext.back().hi = off + 1;
          else
            q.ext.push_back({pg, off, off + 1});
        }
        if (q.lg_ok) {   // a new token owes nothing
          if (!q.ext_lg.empty() && q.ext_lg.back().page == pg && q.ext_lg.back().hi == off &&
              q.ext_lg_lag.back() == 0) {
            q.ext_lg.back().hi = off + 1;
          } else {
            q.ext_lg.push_back({pg, off, off + 1});
            q.ext_lg_lag.push_back(0);
          }
        }
      } else {
        q.stale();
      }
    }
  }
  q.n_vis += n;
}

akv_status get_seq(akv_pool* p, int32_t s, SeqRec** out) {
  if (s < 0 || s >= (int32_t)p->seqs.size()) return fail(AKV_EINVAL, "no sequence %d", s);
  if (!p->seqs[s].alive) return fail(AKV_ESTATE, "sequence %d was released", s);
  *out = &p->seqs[s];
  return AKV_OK;
}

// A sequence whose tokens or rows a call changes: alive and not frozen.
akv_status get_live_seq(akv_pool* p, int32_t s, SeqRec** out) {
  akv_status st = get_seq(p, s, out);
  if (st != AKV_OK) return st;
  if ((*out)->frozen) return fail(AKV_ESTATE, "sequence %d is frozen (a shared checkpoint)", s);
  return AKV_OK;
}

// The slot lies in a page another sequence allocated (a shared page).
inline bool foreign_slot(const akv_pool* p, int32_t s, int32_t slot) {
  return slot >= 0 && p->pages[slot >> p->log2S].owner != s;
}

void note_free(akv_pool* p);

// The pages of a released sequence go back to the free queue, in allocation
// order (pages waiting in the evictable queue are taken out of it).
void finish_release(akv_pool* p, int32_t s) {
  SeqRec& q = p->seqs[s];
  for (const auto& e : q.pages) {
    if (!page_live(p, e)) continue;
    const int32_t pg = e.first;
    PageRec& r = p->pages[pg];
    if (r.in_evict) evict_unlink(p, pg);
    r.owner = -1;
    r.nvis = 0;
    r.filled = 0;
    r.toks.clear();
    p->free_q.push_back(pg);
  }
  q.pages.clear();
  q.stale_pages = 0;
  q.tail = -1;
  q.zombie = false;
  note_free(p);
}

// A token of q stops holding a slot in another sequence's page.
void unref(akv_pool* p, SeqRec& q, int32_t slot) {
  const int32_t o = p->pages[slot >> p->log2S].owner;
  auto it = q.owners.find(o);
  if (it == q.owners.end()) return;
  if (--it->second == 0) {
    q.owners.erase(it);
    SeqRec& so = p->seqs[o];
    if (--so.refs == 0 && so.zombie) finish_release(p, o);
  }
}

// q's visible token in foreign page pg stops being visible there.
void fvis_dec(SeqRec& q, int32_t pg) {
  auto f = q.fvis.find(pg);
  if (f != q.fvis.end() && --f->second == 0) q.fvis.erase(f);
}

akv_status check_spans(const akv_span* sp, int32_t n, int32_t len) {
  if (n < 0) return fail(AKV_EINVAL, "negative span count");
  if (n > 0 && !sp) return fail(AKV_EINVAL, "spans is NULL");
  for (int32_t i = 0; i < n; ++i) {
    if (sp[i].begin > sp[i].end) return fail(AKV_EINVAL, "span %d has end < begin", i);
    if (sp[i].begin < 0 || sp[i].end > len)
      return fail(AKV_ERANGE, "span %d [%d,%d) outside 0..%d", i, sp[i].begin, sp[i].end, len);
  }
  return AKV_OK;
}

// ---------------------------------------------------------------------------
// visibility
// ---------------------------------------------------------------------------
const std::vector<int32_t>& visible(SeqRec& q) {
  if (q.vis_ok) return q.vis;
  q.vis.clear();
  q.vis.reserve(q.n_vis);
  bool sorted = true;
  int64_t last = -1;
  for (int32_t t = 0; t < (int32_t)q.slot.size(); ++t) {
    if (q.dropped[t]) continue;
    if (q.pos[t] < last) sorted = false;
    last = q.pos[t];
    q.vis.push_back(t);
  }
  if (!sorted)
    std::stable_sort(q.vis.begin(), q.vis.end(),
                     [&](int32_t a, int32_t b) { return q.pos[a] < q.pos[b]; });
  q.vis_ok = true;
  q.vis_logical = sorted;
  return q.vis;
}

// The page-table image of vis minus the tokens of the mask spans, cut from
// the cached image: with vis in logical order a span is one range of it, so
// only the extents it meets are trimmed, and pieces that become adjacent
// merge as build_extents would merge them (the result is the same list).
// The ranges of vis (in logical order) that the logical spans cover, sorted
// and merged.
std::vector<std::pair<int64_t, int64_t>> vis_ranges(const SeqRec& q, const akv_span* m, int32_t nm) {
  std::vector<std::pair<int64_t, int64_t>> cut;
  for (int32_t k = 0; k < nm; ++k) {
    const int64_t i0 = std::lower_bound(q.vis.begin(), q.vis.end(), m[k].begin) - q.vis.begin();
    const int64_t i1 = std::lower_bound(q.vis.begin(), q.vis.end(), m[k].end) - q.vis.begin();
    if (i0 < i1) cut.emplace_back(i0, i1);
  }
  std::sort(cut.begin(), cut.end());
  size_t w = 0;   // coalesce overlapping ranges
  for (size_t k = 0; k < cut.size(); ++k) {
    if (w && cut[k].first <= cut[w - 1].second)
      cut[w - 1].second = std::max(cut[w - 1].second, cut[k].second);
    else
      cut[w++] = cut[k];
  }
  cut.resize(w);
  return cut;
}

void masked_from_image(const SeqRec& q, const akv_span* m, int32_t nm, std::vector<akv_extent>& out) {
  const std::vector<std::pair<int64_t, int64_t>> cut = vis_ranges(q, m, nm);
  out.clear();
  auto emit = [&](int32_t pg, int32_t lo, int32_t hi) {
    if (!out.empty() && out.back().page == pg && out.back().hi == lo)
      out.back().hi = hi;
    else
      out.push_back({pg, lo, hi});
  };
  int64_t off = 0;
  size_t c = 0;
  for (const akv_extent& x : q.ext) {
    const int64_t a = off, b = off + (x.hi - x.lo);
    while (c < cut.size() && cut[c].second <= a) ++c;
    int64_t cur = a;
    for (size_t k = c; k < cut.size() && cut[k].first < b; ++k) {
      if (cut[k].first > cur) emit(x.page, x.lo + (int32_t)(cur - a), x.lo + (int32_t)(cut[k].first - a));
      cur = std::max(cur, cut[k].second);
    }
    if (cur < b) emit(x.page, x.lo + (int32_t)(cur - a), x.hi);
    off = b;
  }
}

// After a drop of logical spans: with vis in logical order the dropped
// tokens are whole ranges of it, so the cached order loses those ranges and
// the cached image is trimmed like a masked list (the same lists a rebuild
// gives); otherwise the caches are rebuilt on next use.
void cache_after_drop(SeqRec& q, const akv_span* sp, int32_t n) {
  if (!q.vis_ok || !q.vis_logical) {
    q.stale();
    return;
  }
  if (q.ext_ok) {
    std::vector<akv_extent> trimmed;
    masked_from_image(q, sp, n, trimmed);
    q.ext.swap(trimmed);
  }
  const std::vector<std::pair<int64_t, int64_t>> cut = vis_ranges(q, sp, n);
  size_t w = 0, c = 0;
  for (size_t i = 0; i < q.vis.size(); ++i) {
    while (c < cut.size() && (int64_t)i >= cut[c].second) ++c;
    if (c < cut.size() && (int64_t)i >= cut[c].first) continue;
    q.vis[w++] = q.vis[i];
  }
  q.vis.resize(w);
  q.lg_ok = false;
}

// After positions moved (repos) with slots unchanged: the cached order and
// image stay valid while positions still never decrease along vis.
void cache_after_move(SeqRec& q) {
  if (!q.vis_ok || !q.vis_logical) {
    q.stale();
    return;
  }
  for (size_t i = 1; i < q.vis.size(); ++i)
    if (q.pos[q.vis[i]] < q.pos[q.vis[i - 1]]) {
      q.stale();
      return;
    }
}

void build_extents(const akv_pool* p, const SeqRec& q, const std::vector<int32_t>& order,
                   const std::vector<uint8_t>* hide, std::vector<akv_extent>& out) {
  const int32_t lg = p->log2S, mask = p->L.page_size - 1;
  out.clear();
  for (int32_t t : order) {
    if (hide && (*hide)[t]) continue;
    const int32_t slot = q.slot[t];
    const int32_t pg = slot >> lg, off = slot & mask;
    if (!out.empty() && out.back().page == pg && out.back().hi == off)
      out.back().hi = off + 1;
    else
      out.push_back({pg, off, off + 1});
  }
}

// The same image with runs also cut where the owed rotation changes; lag_out
// gets each extent's owed rotation.
void build_extents_lag(const akv_pool* p, const SeqRec& q, const std::vector<int32_t>& order,
                       const std::vector<uint8_t>* hide, std::vector<akv_extent>& out,
                       std::vector<int32_t>& lag_out) {
  const int32_t lg = p->log2S, mask = p->L.page_size - 1;
  out.clear();
  lag_out.clear();
  for (int32_t t : order) {
    if (hide && (*hide)[t]) continue;
    const int32_t slot = q.slot[t];
    const int32_t pg = slot >> lg, off = slot & mask;
    if (!out.empty() && out.back().page == pg && out.back().hi == off && lag_out.back() == q.lag[t]) {
      out.back().hi = off + 1;
    } else {
      out.push_back({pg, off, off + 1});
      lag_out.push_back(q.lag[t]);
    }
  }
}

double fragmentation(const akv_pool* p, const SeqRec& q) {
  // the sequence's page records are scattered: fetch a few ahead
  constexpr size_t kAhead = 16;
  const size_t np = q.pages.size();
  int64_t cap = 0;
  for (size_t i = 0; i < np; ++i) {
    if (i + kAhead < np) __builtin_prefetch(p->pages.data() + q.pages[i + kAhead].first);
    const PageRec& r = p->pages[q.pages[i].first];
    if (r.take_gen == q.pages[i].second && r.nvis > 0) cap += r.filled;
  }
  for (const auto& f : q.fvis) cap += p->pages[f.first].filled;   // shared pages holding a visible token
  if (cap == 0) return 0.0;
  return 1.0 - (double)q.n_vis / (double)cap;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
akv_status upload_array(akv_pool* p, ScratchCursor& sc, const void* src, size_t n, void** dev) {
  char* h;
  akv_status st = stg_reserve(p, n, &h);
  if (st != AKV_OK) return st;
  std::memcpy(h, src, n);
  *dev = sc.take(n);
  if (!sc.ok())
    return fail(AKV_ENOMEM, "scratch too small for this call (%zu bytes per call)",
                                 p->scratch_bytes - p->scratch_base);
  return stg_upload(p, h, *dev, n);
}

// Several host arrays through one staging region and one copy; dev[i]
// receives array i's device address (each 256-byte aligned).
akv_status upload_arrays(akv_pool* p, ScratchCursor& sc, std::initializer_list<std::pair<const void*, size_t>> parts,
                         void** dev) {
  size_t total = 0;
  for (const auto& pr : parts) total += align_up(std::max<size_t>(pr.second, 1), 256);
  char* h;
  akv_status st = stg_reserve(p, total, &h);
  if (st != AKV_OK) return st;
  char* d = sc.take(total);
  if (!sc.ok()) return fail(AKV_ENOMEM, "scratch too small for this call (%zu bytes per call)",
                                 p->scratch_bytes - p->scratch_base);
  size_t off = 0;
  int i = 0;
  for (const auto& pr : parts) {
    if (pr.second) std::memcpy(h + off, pr.first, pr.second);
    dev[i++] = d + off;
    off += align_up(std::max<size_t>(pr.second, 1), 256);
  }
  return stg_upload(p, h, d, total);
}

// Small tables that a kernel reads once, off its critical path, go through
// the staging ring without a copy: the kernel reads them from the mapped
// pinned memory (no copy and no wait ahead of the launch; the append's slot
// list).  stg_direct fills a region and gives each array's
// device address (256-byte aligned); stg_release, called after the launches
// that read it, records when the region may be rewritten.  Returns false
// when the staging memory is not mapped (the caller uploads instead).
struct DirectRegion {
  size_t b = 0, e = 0;
  bool used = false;
};

bool stg_direct(akv_pool* p, std::initializer_list<std::pair<const void*, size_t>> parts, void** dev,
                DirectRegion& r, akv_status* st) {
  *st = AKV_OK;
  size_t total = 0;
  for (const auto& pr : parts) total += align_up(std::max<size_t>(pr.second, 1), 256);
  char* h;
  *st = stg_reserve(p, total, &h);
  if (*st != AKV_OK || !p->stg.dbase) return false;
  size_t off = 0;
  int i = 0;
  for (const auto& pr : parts) {
    if (pr.second) std::memcpy(h + off, pr.first, pr.second);
    dev[i++] = p->stg.dbase + (h - p->stg.base) + off;
    off += align_up(std::max<size_t>(pr.second, 1), 256);
  }
  r.b = (size_t)(h - p->stg.base);
  r.e = r.b + align_up(std::max<size_t>(total, 16), 256);
  r.used = true;
  return true;
}

void stg_release(akv_pool* p, const DirectRegion& r) {
  if (!r.used) return;
  hipEvent_t ev;
  if (stg_event(p, &ev) != hipSuccess) return;
  if (hipEventRecord(ev, p->stream) != hipSuccess) {
    // the region cannot be tracked: wait here so it is never rewritten early
    (void)hipStreamSynchronize(p->stream);
    p->stg.spare.push_back(ev);
    return;
  }
  p->stg.pending.push_back({r.b, r.e, ev});
}

// Rotation table of the given deltas into p->rot_tab: row i holds cos of the
// d_rope/2 pairs at angle deltas[i] * theta_j, then their sin, as fp32
// ([AKV-blog] section 2, The Repos Primitive; [Leyline] Method and
// Limitations, fp32 rotation).  The angle is formed in fp64 and reduced mod
// 2 pi before sincos, so large deltas keep full accuracy.  Rows of recent
// deltas are kept in the pool (the same deltas recur over layers and steps).
const std::vector<float>& rot_table_rows(akv_pool* p, const int32_t* deltas, size_t n) {
  const int d = p->L.d_rope, half = d / 2;
  p->rot_tab.resize(n * (size_t)d);
  if (p->rot_cache.size() > 8192) p->rot_cache.clear();
  for (size_t i = 0; i < n; ++i) {
    std::vector<float>& row = p->rot_cache[deltas[i]];
    if (row.empty()) {
      row.resize(d);
      for (int j = 0; j < half; ++j) {
        const double ang = (double)deltas[i] * p->inv_freq[j];
        const double red = ang - 6.283185307179586476925 * std::rint(ang * 0.15915494309189533577);
        row[j] = (float)std::cos(red);
        row[half + j] = (float)std::sin(red);
      }
    }
    std::copy(row.begin(), row.end(), p->rot_tab.begin() + i * (size_t)d);
  }
  return p->rot_tab;
}

// Per-call scratch bytes left after the persistent tables (a conservative
// bound checked before any state changes, so a short buffer leaves no trace).
// Scratch bytes of one rotation: items, the cos/sin table, the layer pointer
// table, and the alignment of each upload.
size_t rotate_scratch_bytes(const akv_pool* p, size_t n_items, size_t n_deltas, size_t n_layers) {
  return n_items * sizeof(akv::RotItem) + n_deltas * (size_t)p->L.d_rope * 4 + n_layers * sizeof(void*) +
         3 * 256;
}

akv_status scratch_fits(const akv_pool* p, size_t bytes) {
  if (!p->device) return AKV_OK;
  const size_t need = p->scratch_base + bytes + 4096;
  if (need > p->scratch_bytes)
    return fail(AKV_ENOMEM, "scratch too small: need at least %zu bytes", need);
  return AKV_OK;
}

akv_status check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return hip_fail(e, what);
  if (dbg().inject_launch) return fail(AKV_EHIP, "%s: injected failure (AKV_FAULT_INJECT=launch)", what);
  return AKV_OK;
}

// ---- AKV_CHECKS: host checks of device work lists ---------------------------
bool slot_in_pool(const akv_pool* p, int32_t slot) {
  return slot >= 0 && (int64_t)slot < (int64_t)p->L.num_pages * p->L.page_size;
}

// Slots written by one launch: inside the pool, in pages in use, distinct.
akv_status check_slots(const akv_pool* p, const int32_t* slots, size_t n, const char* what) {
  std::vector<int32_t> s(slots, slots + n);
  for (int32_t x : s) {
    if (!slot_in_pool(p, x)) return check_fail("%s: slot %d outside the pool", what, x);
    if (p->pages[x >> p->log2S].owner < 0) return check_fail("%s: slot %d lies in a free page", what, x);
  }
  std::sort(s.begin(), s.end());
  for (size_t i = 1; i < s.size(); ++i)
    if (s[i] == s[i - 1]) return check_fail("%s: slot %d written twice", what, s[i]);
  return AKV_OK;
}

// Rotate items: rows inside pages in use, a valid table row, and no row
// turned by two items (the kernel works in place).
akv_status check_rot_items(const akv_pool* p, const std::vector<akv::RotItem>& items, size_t n_deltas) {
  const akv_layout& L = p->L;
  for (const akv::RotItem& it : items) {
    if (it.page < 0 || it.page >= L.num_pages || it.lo < 0 || it.lo >= it.hi || it.hi > L.page_size)
      return check_fail("rotate item (%d, %d, %d) outside the pool", it.page, it.lo, it.hi);
    if (p->pages[it.page].owner < 0) return check_fail("rotate item in free page %d", it.page);
    if (it.didx < 0 || (size_t)it.didx >= n_deltas)
      return check_fail("rotate item of page %d: table row %d of %zu", it.page, it.didx, n_deltas);
  }
  std::vector<akv::RotItem> s(items);
  std::sort(s.begin(), s.end(), [](const akv::RotItem& a, const akv::RotItem& b) {
    return a.page != b.page ? a.page < b.page : a.lo < b.lo;
  });
  for (size_t i = 1; i < s.size(); ++i)
    if (s[i].page == s[i - 1].page && s[i].lo < s[i - 1].hi)
      return check_fail("rows %d..%d of page %d rotated twice", s[i].lo, s[i - 1].hi, s[i].page);
  return AKV_OK;
}

// Row copies: slots inside the pool, destinations in pages in use, distinct,
// and none of them a source (copies of one launch run in any order).
akv_status check_moves(const akv_pool* p, const akv::MovePair* mv, size_t n, const char* what) {
  std::vector<int32_t> src(n), dst(n);
  for (size_t i = 0; i < n; ++i) {
    if (!slot_in_pool(p, mv[i].src) || !slot_in_pool(p, mv[i].dst))
      return check_fail("%s: copy %d -> %d outside the pool", what, mv[i].src, mv[i].dst);
    src[i] = mv[i].src;
    dst[i] = mv[i].dst;
  }
  akv_status st = check_slots(p, dst.data(), n, what);
  if (st != AKV_OK) return st;
  std::sort(src.begin(), src.end());
  std::sort(dst.begin(), dst.end());
  for (size_t i = 0, j = 0; i < n && j < n;) {
    if (src[i] == dst[j]) return check_fail("%s: slot %d is both a source and a destination", what, src[i]);
    if (src[i] < dst[j]) ++i;
    else ++j;
  }
  return AKV_OK;
}

// Marks the pool stream's current end as the last write of pool rows.
void note_write(akv_pool* p) {
  if (p->device && hipEventRecord(p->write_ev, p->stream) == hipSuccess) p->write_set = true;
}
// Marks the pool stream's current end: pages just given back to the queues
// are read by no pool-stream work enqueued later.
void note_free(akv_pool* p) {
  if (p->device && hipEventRecord(p->free_ev, p->stream) == hipSuccess) p->free_set = true;
}

// The pool stream waits for the background compaction copies; their pages
// are no longer flagged.
akv_status bg_wait(akv_pool* p) {
  if (!p->bg_pending) return AKV_OK;
  hipError_t e = hipStreamWaitEvent(p->stream, p->bg_done, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent(background compaction)");
  p->bg_pending = false;
  for (int32_t pg : p->bg_pages) p->page_bg[pg] = 0;
  p->bg_pages.clear();
  return AKV_OK;
}

// bg_wait when any of the slots lies in a page a background copy touches.
akv_status bg_wait_slots(akv_pool* p, const int32_t* slots, size_t n) {
  if (!p->bg_pending) return AKV_OK;
  for (size_t i = 0; i < n; ++i)
    if (slots[i] >= 0 && p->page_bg[slots[i] >> p->log2S]) return bg_wait(p);
  return AKV_OK;
}

// scatter appended rows of one token batch into the pool arrays
akv_status device_append(akv_pool* p, const std::vector<int32_t>& slots, const void* K,
                         const void* Kpe, const void* V) {
  if (dbg().checks) {
    akv_status cst = check_slots(p, slots.data(), slots.size(), "append");
    if (cst != AKV_OK) return cst;
  }
  if (!p->device || !K) return AKV_OK;
  akv_status bst = bg_wait_slots(p, slots.data(), slots.size());
  if (bst != AKV_OK) return bst;
  ScratchCursor sc(p, slots.size() * 4 + 256);
  void* dslots;
  DirectRegion dr;
  akv_status st;
  if (!stg_direct(p, {{slots.data(), slots.size() * 4}}, &dslots, dr, &st)) {
    if (st != AKV_OK) return st;
    st = upload_array(p, sc, slots.data(), slots.size() * 4, &dslots);
    if (st != AKV_OK) return st;
  }
  const akv_layout& L = p->L;
  const int n = (int)slots.size();
  akv::TokenRows rows[3];
  int nr = 0;
  if (L.d_nope > 0) {
    rows[nr++] = {(const uint16_t*)K, p->k, L.n_kv_heads, L.d_nope};
    rows[nr++] = {(const uint16_t*)Kpe, p->kpe, p->rope_heads(), L.d_rope};
  } else {
    rows[nr++] = {(const uint16_t*)K, p->k, L.n_kv_heads, L.d_rope};
  }
  rows[nr++] = {(const uint16_t*)V, p->v, L.n_kv_heads, L.d_v};
  KTimer tm(p, AKV_K_APPEND);
  hipError_t e = akv::launch_scatter_tokens(p->stream, rows, nr, (const int32_t*)dslots, n, L.page_size, p->log2S);
  tm.done();
  stg_release(p, dr);
  note_write(p);
  return check_launch(e, "append kernel launch");
}

// rotate the listed (slot, delta) runs in the rotated-key arrays of `layers`
// (pools sharing p's page table; p itself when empty) with one launch
akv_status device_rotate(akv_pool* p, const std::vector<akv::RotItem>& items,
                         const std::vector<int32_t>& deltas,
                         const std::vector<akv_pool*>& layers = {}) {
  if (dbg().checks) {
    akv_status cst = check_rot_items(p, items, deltas.size());
    if (cst != AKV_OK) return cst;
  }
  if (!items.empty())
    trace("rotate: %zu items, %zu distinct deltas, %zu layer(s)", items.size(), deltas.size(),
          std::max<size_t>(layers.size(), 1));
  if (!p->device || items.empty()) return AKV_OK;
  akv_status bst = bg_wait(p);
  for (akv_pool* l : layers)
    if (bst == AKV_OK && l != p) bst = bg_wait(l);
  if (bst != AKV_OK) return bst;
  std::vector<uint16_t*> krs;
  if (layers.empty()) krs.push_back(p->rope_array());
  for (akv_pool* l : layers) krs.push_back(l->rope_array());
  // The work list is copied to device memory: every rotate block reads its
  // item before it can address its keys, and reading it across PCIe would
  // add that latency to each block (measured: 30 -> 35 us at the 64K step).
  ScratchCursor sc(p, rotate_scratch_bytes(p, items.size(), deltas.size(), krs.size()));
  const std::vector<float>& tab = rot_table_rows(p, deltas.data(), deltas.size());
  void* dv[3];
  akv_status st = upload_arrays(p, sc,
                                {{items.data(), items.size() * sizeof(akv::RotItem)},
                                 {tab.data(), tab.size() * 4},
                                 {krs.data(), krs.size() * sizeof(uint16_t*)}},
                                dv);
  if (st != AKV_OK) return st;
  void *ditems = dv[0], *dkrs = dv[2];
  const float* dtab = (const float*)dv[1];
  hipError_t e;
  KTimer tm(p, AKV_K_ROTATE);
  e = akv::launch_rotate(p->stream, (uint16_t* const*)dkrs, (int)krs.size(), p->rope_heads(), p->L.page_size,
                         p->L.d_rope, p->L.pairing, (const akv::RotItem*)ditems, (int)items.size(), dtab);
  tm.done();
  note_write(p);
  for (akv_pool* l : layers)
    if (l != p) note_write(l);
  return check_launch(e, "rotate kernel launch");
}

// One launch moving every paged array of n tokens (pairs on the device); the
// rotated-key rows are turned by `table` when it is given.
hipError_t move_tokens(akv_pool* p, const akv::MovePair* pairs, int n, const float* table) {
  const akv_layout& L = p->L;
  akv::TokenRows plain[2];
  int np = 0;
  plain[np++] = {p->v, p->v, L.n_kv_heads, L.d_v};
  if (L.d_nope > 0) plain[np++] = {p->k, p->k, L.n_kv_heads, L.d_nope};
  return akv::launch_move_tokens(p->stream, p->rope_array(), p->rope_heads(), L.d_rope, L.pairing, plain, np,
                                 pairs, n, L.page_size, p->log2S, table);
}

akv_status device_move(akv_pool* p, const std::vector<akv::MovePair>& mv) {
  if (dbg().checks) {
    akv_status cst = check_moves(p, mv.data(), mv.size(), "compaction");
    if (cst != AKV_OK) return cst;
  }
  if (!p->device || mv.empty()) return AKV_OK;
  akv_status bst = bg_wait(p);
  if (bst != AKV_OK) return bst;
  ScratchCursor sc(p, mv.size() * sizeof(akv::MovePair) + 256);
  void* dmv;
  akv_status st = upload_array(p, sc, mv.data(), mv.size() * sizeof(akv::MovePair), &dmv);
  if (st != AKV_OK) return st;
  const int n = (int)mv.size();
  KTimer tm(p, AKV_K_COMPACT);
  hipError_t e = move_tokens(p, (const akv::MovePair*)dmv, n, nullptr);
  tm.done();
  note_write(p);
  note_free(p);   // compaction gave the old pages back
  return check_launch(e, "compaction kernel launch");
}

// The same copies as a background launch on kstream: after the pool
// stream's work so far (which wrote the rows read and last read the pages
// written), beside the pool stream's later work; every page the copies read
// or write is flagged until the pool stream waits for them.
akv_status device_move_bg(akv_pool* p, const std::vector<akv::MovePair>& mv, bool after_all) {
  if (dbg().checks) {
    akv_status cst = check_moves(p, mv.data(), mv.size(), "background compaction");
    if (cst != AKV_OK) return cst;
  }
  if (!mv.empty()) trace("background compaction: %zu row copies on the second stream", mv.size());
  if (!p->device || mv.empty()) return AKV_OK;
  // ordered after the last write of pool rows and after the work that may
  // still read pages given back to the queues, not after later work; when
  // fresh pages come from the evictable queue (pages an earlier background
  // pass gave back may still be read by work enqueued before it), after all
  // of the pool stream's work so far
  hipError_t e = hipSuccess;
  if (after_all) {
    e = hipEventRecord(p->free_ev, p->stream);
    if (e == hipSuccess) p->free_set = true;
  }
  if (e == hipSuccess && p->write_set) e = hipStreamWaitEvent(p->kstream, p->write_ev, 0);
  if (e == hipSuccess && p->free_set) e = hipStreamWaitEvent(p->kstream, p->free_ev, 0);
  if (e != hipSuccess) return hip_fail(e, "ordering the background copies");
  // the copy list goes up on kstream itself
  const size_t nb = mv.size() * sizeof(akv::MovePair);
  ScratchCursor sc(p, nb + 256);
  sc.bg = true;
  char* h;
  akv_status st = stg_reserve(p, nb, &h);
  if (st != AKV_OK) return st;
  std::memcpy(h, mv.data(), nb);
  void* dmv = sc.take(nb);
  if (!sc.ok()) return fail(AKV_ENOMEM, "scratch too small for this call (%zu bytes per call)",
                            p->scratch_bytes - p->scratch_base);
  e = hipMemcpyAsync(dmv, h, nb, hipMemcpyHostToDevice, p->kstream);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(H2D, background)");
  hipEvent_t uev;
  e = stg_event(p, &uev);
  if (e == hipSuccess) e = hipEventRecord(uev, p->kstream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(background upload)");
  const size_t off = (size_t)(h - p->stg.base);
  p->stg.pending.push_back({off, off + align_up(std::max<size_t>(nb, 16), 256), uev});
  const akv_layout& L = p->L;
  akv::TokenRows plain[2];
  int np = 0;
  plain[np++] = {p->v, p->v, L.n_kv_heads, L.d_v};
  if (L.d_nope > 0) plain[np++] = {p->k, p->k, L.n_kv_heads, L.d_nope};
  KTimer tm(p, AKV_K_COMPACT, p->kstream);
  e = akv::launch_move_tokens(p->kstream, p->rope_array(), p->rope_heads(), L.d_rope, L.pairing, plain, np,
                              (const akv::MovePair*)dmv, (int)mv.size(), L.page_size, p->log2S, nullptr);
  tm.done();
  if (e != hipSuccess) return hip_fail(e, "background compaction kernel launch");
  e = hipEventRecord(p->bg_done, p->kstream);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord(background compaction)");
  p->bg_pending = true;
  for (const akv::MovePair& m : mv)
    for (int32_t slot : {m.src, m.dst}) {
      const int32_t pg = slot >> p->log2S;
      if (!p->page_bg[pg]) {
        p->page_bg[pg] = 1;
        p->bg_pages.push_back(pg);
      }
    }
  return check_launch(e, "background compaction kernel launch");
}

// ---------------------------------------------------------------------------
// compaction ([AKV-blog] section 7, Dilemma 2)
// ---------------------------------------------------------------------------
// Host side of compacting s: fresh pages, new slots, old pages to the
// evictable queue; the copies are appended to mv for the caller to launch.
akv_status compact_plan(akv_pool* p, int32_t s, std::vector<akv::MovePair>& mv) {
  SeqRec& q = p->seqs[s];
  const std::vector<int32_t> order = visible(q);  // copy: q.vis is rebuilt below
  const int32_t S = p->L.page_size;
  const int64_t nv = (int64_t)order.size();
  const int64_t need = (nv + S - 1) / S;
  if (need > available(p)) return fail(AKV_ENOMEM, "compaction needs %lld free pages", (long long)need);
  std::vector<int32_t> old_pages;
  old_pages.reserve(q.pages.size());
  for (const auto& e : q.pages)
    if (page_live(p, e)) old_pages.push_back(e.first);
  std::vector<int32_t> dest;
  dest.reserve(need);
  for (int64_t i = 0; i < need; ++i) dest.push_back(take_page(p, s));
  trace("compact seq %d: %lld visible tokens into %lld fresh pages", s, (long long)nv, (long long)need);
  mv.reserve(mv.size() + nv);
  std::vector<int32_t> shared_src;   // slots given up in other sequences' pages
  const bool shares = !q.owners.empty();
  for (int64_t i = 0; i < nv; ++i) {
    const int32_t t = order[i];
    const int32_t dst = dest[i / S] * S + (int32_t)(i % S);
    mv.push_back({q.slot[t], dst});
    if (shares && foreign_slot(p, s, q.slot[t])) shared_src.push_back(q.slot[t]);
    q.slot[t] = dst;
    p->pages[dest[i / S]].toks.push_back(t);
  }
  q.fvis.clear();
  for (int32_t sl : shared_src) unref(p, q, sl);
  for (int64_t i = 0; i < need; ++i) {
    PageRec& r = p->pages[dest[i]];
    const int32_t c = (int32_t)std::min<int64_t>(S, nv - i * S);
    r.filled = c;
    r.nvis = c;
  }
  q.tail = (need > 0 && nv % S) ? dest.back() : -1;
  // an old page may come back as a fresh one (from the evictable queue)
  std::vector<int32_t> dest_sorted(dest);
  std::sort(dest_sorted.begin(), dest_sorted.end());
  for (int32_t pg : old_pages) {
    if (std::binary_search(dest_sorted.begin(), dest_sorted.end(), pg)) continue;
    PageRec& r = p->pages[pg];
    if (r.owner != s) continue;
    r.nvis = 0;
    // keep only tokens that still point into this page (the dropped ones)
    r.toks.erase(std::remove_if(r.toks.begin(), r.toks.end(),
                                [&](int32_t t) { return !(q.slot[t] >= 0 && q.slot[t] / S == pg); }),
                 r.toks.end());
    if (!r.in_evict) evict_push(p, pg);
  }
  q.stale();
  return AKV_OK;
}

akv_status compact_seq(akv_pool* p, int32_t s) {
  std::vector<akv::MovePair> mv;
  akv_status st = compact_plan(p, s, mv);
  if (st != AKV_OK) return st;
  return device_move(p, mv);
}

void drop_tokens(akv_pool* p, SeqRec& q, int32_t b, int32_t e, bool keep_cache = false) {
  // page records lie in allocation order, not in the sequence's: fetch the
  // record a few pages ahead (tokens of evicted pages have no slot).  Tokens
  // dropped from one of q's own pages in a row are counted together: the
  // page's record is updated once per run (a page empties at the last token
  // of its run, so the evictable queue gets pages in the same order).
  constexpr int32_t kAhead = 64;
  const int32_t lg = p->log2S;
  uint8_t* const dropped = q.dropped.data();
  int32_t* const slot = q.slot.data();
  const PageRec* const recs = p->pages.data();
  int64_t n_drop = 0;
  int32_t run_pg = -1, run_n = 0;
  auto flush = [&]() {
    if (run_n == 0) return;
    PageRec& r = p->pages[run_pg];
    r.nvis -= run_n;
    if (r.nvis == 0 && run_pg != q.tail && !r.in_evict) evict_push(p, run_pg);
    run_n = 0;
  };
  for (int32_t t = b; t < e; ++t) {
    if (t + kAhead < e && slot[t + kAhead] >= 0) __builtin_prefetch(recs + (slot[t + kAhead] >> lg));
    if (dropped[t]) continue;
    dropped[t] = 1;
    n_drop += 1;
    const int32_t pg = slot[t] >> lg;
    if (pg == run_pg) {   // the run's page is one of q's own
      run_n += 1;
      continue;
    }
    flush();
    run_pg = -1;
    if (foreign_slot(p, q.id, slot[t])) {   // a shared token gives its slot up at once
      fvis_dec(q, pg);
      unref(p, q, slot[t]);
      slot[t] = -1;
      continue;
    }
    run_pg = pg;
    run_n = 1;
  }
  flush();
  q.n_vis -= n_drop;
  if (!keep_cache) q.stale();
}

// Above the threshold: compact now when the allocator can supply the pages
// (skipped otherwise), or, in deferred mode, queue the sequence for
// akv_compact_pending.
akv_status auto_compact(akv_pool* p, int32_t s) {
  SeqRec& q = p->seqs[s];
  const double frag = fragmentation(p, q);
  if (frag > p->thr) {
    if (p->compact_mode == AKV_COMPACT_DEFERRED) {
      if (!q.queued) {
        q.queued = true;
        p->compact_q.push_back(s);
        trace("seq %d: fragmentation %.3f above %.2f, queued for compaction", s, frag, p->thr);
      }
      return AKV_OK;
    }
    const int64_t need = (q.n_vis + p->L.page_size - 1) / p->L.page_size;
    if (need <= available(p)) {
      trace("seq %d: fragmentation %.3f above %.2f, compacting", s, frag, p->thr);
      return compact_seq(p, s);
    }
    trace("seq %d: fragmentation %.3f above %.2f, compaction skipped (%lld pages needed, %lld available)", s,
          frag, p->thr, (long long)need, (long long)available(p));
  }
  return AKV_OK;
}

// ---------------------------------------------------------------------------
// repos planning ([AKV-blog] section 2; [Leyline] Method)
// ---------------------------------------------------------------------------
// Runs of logical tokens [b, e) that move by one total delta d != 0 (the sum
// over the spans covering them); dropped tokens inside a run do not move.
struct Run {
  int32_t b, e;
  int64_t d;
};

// Spans and deltas to runs in ascending token order (a sweep over the span
// ends), then the range check of every moved position.
akv_status repos_runs(const SeqRec& q, const akv_span* sp, const int32_t* d, int32_t n, std::vector<Run>& runs) {
  const int32_t len = (int32_t)q.slot.size();
  akv_status st = check_spans(sp, n, len);
  if (st != AKV_OK) return st;
  if (n > 0 && !d) return fail(AKV_EINVAL, "delta is NULL");
  std::vector<std::pair<int32_t, int64_t>> ev;
  ev.reserve(2 * (size_t)n);
  for (int32_t i = 0; i < n; ++i)
    if (sp[i].begin < sp[i].end && d[i] != 0) {
      ev.emplace_back(sp[i].begin, (int64_t)d[i]);
      ev.emplace_back(sp[i].end, -(int64_t)d[i]);
    }
  std::sort(ev.begin(), ev.end(), [](const auto& a, const auto& b) { return a.first < b.first; });
  runs.clear();
  int64_t cur = 0;
  int32_t x0 = 0;
  for (size_t i = 0; i < ev.size();) {
    const int32_t x = ev[i].first;
    if (cur != 0 && x0 < x) runs.push_back({x0, x, cur});
    for (; i < ev.size() && ev[i].first == x; ++i) cur += ev[i].second;
    x0 = x;
  }
  for (const Run& r : runs)
    for (int32_t t = r.b; t < r.e; ++t) {
      if (q.dropped[t]) continue;
      const int64_t np = (int64_t)q.pos[t] + r.d;
      if (np < 0 || np > kInt32Max)
        return fail(AKV_ERANGE, "token %d would move to position %lld", t, (long long)np);
    }
  return AKV_OK;
}

// Sort rotation items by page * S + lo (LSD radix, 11-bit digits, as many
// passes as the largest key needs).
void sort_by_first_slot(std::vector<akv::RotItem>& items, int32_t S) {
  const size_t n = items.size();
  if (n < 2) return;
  uint32_t kmax = 0;
  std::vector<uint32_t> key(n), key2(n);
  for (size_t i = 0; i < n; ++i) {
    key[i] = (uint32_t)items[i].page * (uint32_t)S + (uint32_t)items[i].lo;
    kmax = std::max(kmax, key[i]);
  }
  std::vector<akv::RotItem> tmp(n);
  uint32_t cnt[2048];
  for (int shift = 0; shift < 32 && (kmax >> shift) != 0; shift += 11) {
    std::fill(cnt, cnt + 2048, 0u);
    for (size_t i = 0; i < n; ++i) cnt[(key[i] >> shift) & 2047] += 1;
    uint32_t sum = 0;
    for (uint32_t& c : cnt) {
      const uint32_t c0 = c;
      c = sum;
      sum += c0;
    }
    for (size_t i = 0; i < n; ++i) {
      const uint32_t j = cnt[(key[i] >> shift) & 2047]++;
      tmp[j] = items[i];
      key2[j] = key[i];
    }
    items.swap(tmp);
    key.swap(key2);
  }
}

// Work items: runs of consecutive slots of one page with one delta, in the
// runs' token order, cut to about 16 KiB of rotated keys each (half a 16-token
// page of 8 heads x 128 dims) so the blocks spread evenly over the CUs.
// The items of one sequence's runs, appended to `items`; their deltas are
// appended to `deltas` once each (didx maps a delta to its index).  The
// caller sorts the items into page order.
void repos_items_append(const akv_pool* p, const SeqRec& q, const std::vector<Run>& runs,
                        std::vector<akv::RotItem>& items, std::vector<int32_t>& deltas,
                        std::unordered_map<int64_t, int32_t>& didx) {
  const int32_t S = p->L.page_size, lg = p->log2S;
  const int32_t row_bytes = p->rope_heads() * p->L.d_rope * 2;
  const int32_t max_rows = std::max<int32_t>(1, 16384 / row_bytes);
  size_t span_tokens = 0;
  for (const Run& r : runs) span_tokens += (size_t)(r.e - r.b);
  // grow geometrically: a batched repos calls this once per sequence
  const size_t want = items.size() + span_tokens / (size_t)std::min(max_rows, S) + 2 * runs.size() + 16;
  if (want > items.capacity()) items.reserve(std::max(want, 2 * items.capacity()));
  const bool shares = !q.owners.empty();   // the sequence holds slots in other sequences' pages
  // the open item is kept in registers and stored when the next one starts
  // (it may continue the last item of the list)
  akv::RotItem cur{-1, 0, 0, -1};
  if (!items.empty()) {
    cur = items.back();
    items.pop_back();
  }
  for (const Run& r : runs) {
    int32_t di = -1;   // looked up at the run's first moved token
    for (int32_t t = r.b; t < r.e; ++t) {
      if (q.dropped[t]) continue;
      if (shares && foreign_slot(p, q.id, q.slot[t])) continue;   // a shared row is not written: the token owes it
      if (di < 0) {
        auto f = didx.find(r.d);
        if (f == didx.end()) {
          di = (int32_t)deltas.size();
          deltas.push_back((int32_t)r.d);
          didx.emplace(r.d, di);
        } else {
          di = f->second;
        }
      }
      const int32_t slot = q.slot[t];
      const int32_t pg = slot >> lg, off = slot & (S - 1);
      if (cur.page == pg && cur.hi == off && cur.didx == di && cur.hi - cur.lo < max_rows) {
        cur.hi += 1;
      } else {
        if (cur.page >= 0) items.push_back(cur);
        cur = {pg, off, off + 1, di};
      }
    }
  }
  if (cur.page >= 0) items.push_back(cur);
}

void repos_items(const akv_pool* p, const SeqRec& q, const std::vector<Run>& runs,
                 std::vector<akv::RotItem>& items, std::vector<int32_t>& deltas) {
  std::unordered_map<int64_t, int32_t> didx;
  items.clear();
  deltas.clear();
  repos_items_append(p, q, runs, items, deltas, didx);
  // Physical page order, then slot order in a page: neighbouring blocks then
  // touch neighbouring memory.  Items never overlap, so an item's first slot
  // is a unique key for that order: LSD radix sort on it.
  sort_by_first_slot(items, p->L.page_size);
}

// Positions after a repos; tokens whose rows are shared pages (not rotated in
// place) owe the rotation instead, as after a deferred repos.
void repos_commit(const akv_pool* p, SeqRec& q, const std::vector<Run>& runs, bool owe_shared = true) {
  owe_shared = owe_shared && !q.owners.empty();
  for (const Run& r : runs)
    for (int32_t t = r.b; t < r.e; ++t)
      if (!q.dropped[t]) {
        q.pos[t] = (int32_t)(q.pos[t] + r.d);
        if (owe_shared && foreign_slot(p, q.id, q.slot[t])) {
          q.lag[t] = (int32_t)(q.lag[t] + r.d);
          q.lagging = true;
          q.lg_ok = false;
        }
      }
  if (!runs.empty()) cache_after_move(q);
}

// Rotate every visible key by the rotation it still owes (one launch) and
// clear the debt.
// Slots for existing tokens of s that leave shared pages (tail page first,
// then fresh pages, as place_tokens).
void place_existing(akv_pool* p, int32_t s, const std::vector<int32_t>& toks, std::vector<int32_t>& slots_out) {
  SeqRec& q = p->seqs[s];
  const int32_t S = p->L.page_size;
  for (int32_t t : toks) {
    if (q.tail < 0) q.tail = take_page(p, s);
    const int32_t pg = q.tail;
    PageRec& r = p->pages[pg];
    const int32_t slot = pg * S + r.filled;
    r.filled += 1;
    r.nvis += 1;
    r.toks.push_back(t);
    if (r.filled == S) q.tail = -1;
    slots_out.push_back(slot);
    q.slot[t] = slot;
  }
}

// One launch copying rows (all paged arrays) from src to dst slots, the
// rotated-key part turned by R(delta) (the table row and fp32 formula of an
// in-place repos; delta 0 copies).
akv_status device_copy_rows(akv_pool* p, const std::vector<akv::MovePair>& mv, int32_t delta) {
  if (dbg().checks) {
    akv_status cst = check_moves(p, mv.data(), mv.size(), "row copy");
    if (cst != AKV_OK) return cst;
  }
  if (!mv.empty()) trace("copy on write: %zu rows turned by %d", mv.size(), delta);
  if (!p->device || mv.empty()) return AKV_OK;
  ScratchCursor sc(p, mv.size() * sizeof(akv::MovePair) + (size_t)p->L.d_rope * 4 + 3 * 256);
  const std::vector<float>& tab = rot_table_rows(p, &delta, 1);
  void* dv[2];
  akv_status st = upload_arrays(p, sc, {{mv.data(), mv.size() * sizeof(akv::MovePair)},
                                        {tab.data(), delta != 0 ? tab.size() * 4 : 0}}, dv);
  if (st != AKV_OK) return st;
  st = bg_wait(p);
  if (st != AKV_OK) return st;
  KTimer tm(p, AKV_K_CLONE);
  hipError_t e = move_tokens(p, (const akv::MovePair*)dv[0], (int)mv.size(), delta != 0 ? (const float*)dv[1] : nullptr);
  tm.done();
  note_write(p);
  return check_launch(e, "row copy kernel launch");
}

// Every visible key of q turned by what it owes: rows of q's own pages in
// place; rows in shared pages (which other sequences read as they are) are
// copied with the rotation into slots of q's own (copy on write).
akv_status materialize_seq(akv_pool* p, SeqRec& q) {
  if (!q.lagging) return AKV_OK;
  std::vector<Run> runs;
  std::vector<int32_t> cow;
  const int32_t len = (int32_t)q.slot.size();
  for (int32_t t = 0; t < len; ++t) {
    if (q.dropped[t] || q.lag[t] == 0) continue;
    if (foreign_slot(p, q.id, q.slot[t])) {
      cow.push_back(t);
      continue;
    }
    if (!runs.empty() && runs.back().e == t && runs.back().d == q.lag[t])
      runs.back().e = t + 1;
    else
      runs.push_back({t, t + 1, q.lag[t]});
  }
  if (!cow.empty() && pages_needed(p, q, (int64_t)cow.size()) > available(p))
    return fail(AKV_ENOMEM, "copy on write of %zu shared rows: pool exhausted", cow.size());
  trace("materialize seq %d: %zu runs in place, %zu shared rows copied", q.id, runs.size(), cow.size());
  std::vector<akv::RotItem> items;
  std::vector<int32_t> deltas;
  repos_items(p, q, runs, items, deltas);
  akv_status st = scratch_fits(p, std::max(rotate_scratch_bytes(p, items.size(), deltas.size(), 1),
                                           cow.size() * sizeof(akv::MovePair) + (size_t)p->L.d_rope * 4 + 1024));
  if (st != AKV_OK) return st;
  st = device_rotate(p, items, deltas);
  if (st != AKV_OK) return st;
  if (!cow.empty()) {
    std::vector<int32_t> old_slots, new_slots;
    for (int32_t t : cow) old_slots.push_back(q.slot[t]);
    place_existing(p, q.id, cow, new_slots);
    // one copy launch per distinct owed rotation
    std::unordered_map<int32_t, std::vector<akv::MovePair>> by_lag;
    for (size_t i = 0; i < cow.size(); ++i) by_lag[q.lag[cow[i]]].push_back({old_slots[i], new_slots[i]});
    for (const auto& kv : by_lag) {
      st = device_copy_rows(p, kv.second, kv.first);
      if (st != AKV_OK) return st;
    }
    for (size_t i = 0; i < cow.size(); ++i) {
      fvis_dec(q, old_slots[i] >> p->log2S);
      unref(p, q, old_slots[i]);
    }
    q.stale();
  }
  for (const Run& r : runs)
    for (int32_t t = r.b; t < r.e; ++t) q.lag[t] = 0;
  for (int32_t t : cow) q.lag[t] = 0;
  q.lagging = false;
  q.lg_ok = false;
  return AKV_OK;
}

// ---------------------------------------------------------------------------
// attention planning ([AKV-notes] section 3; [AKV-blog] section 4)
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int64_t kDecodeChunk = 1536;

void plan_attention(const akv_pool* p, const akv_segment* segs, int32_t n_segs,
                    const std::vector<int64_t>& lkv, const std::vector<int64_t>& list_off, int RB, int n_cu,
                    AttnPlan& plan) {
  const akv_layout& L = p->L;
  const int G = L.n_q_heads / L.n_kv_heads;
  const int KT = akv::ATTN_KTILE;
  plan.segs.clear();
  for (int32_t i = 0; i < n_segs; ++i)
    plan.segs.push_back({segs[i].q_begin, segs[i].q_len, (int32_t)lkv[i], (int32_t)list_off[i]});
  // base work: row tiles per (segment, kv head)
  int64_t base = 0;
  for (int32_t i = 0; i < n_segs; ++i)
    if (segs[i].q_len > 0) base += (int64_t)L.n_kv_heads * ((segs[i].q_len * (int64_t)G + RB - 1) / RB);
  int target = 1;
  // split the key range only when the row tiles alone cannot fill the CUs,
  // into about one work item per CU (a prefill block holds its CU's LDS, so
  // a second round of blocks would pay its pipeline fill again); at most 16
  // here, 64 for decode items: the combine kernel holds one split per lane of
  // a wave
  if (base > 0 && base < n_cu) target = (int)std::min<int64_t>(16, ((int64_t)n_cu + base - 1) / base);
  // ... or when one row tile alone would hold a CU well past the even share
  // of the launch (few query rows over long lists: decode): such a segment's
  // key range is cut into blocks of at most half a CU's share.
  int64_t total_cost = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    const int32_t lq = segs[i].q_len;
    if (lq <= 0) continue;
    const int64_t rows = (int64_t)lq * G;
    for (int64_t row0 = 0; row0 < rows; row0 += RB) {
      const int64_t last_row = std::min<int64_t>(row0 + RB, rows) - 1;
      total_cost += (int64_t)L.n_kv_heads * (std::min<int64_t>(lkv[i], lkv[i] - lq + last_row / G + 1) + 64);
    }
  }
  const int64_t cu_share = total_cost / n_cu;
  const int64_t block_cap = std::max<int64_t>(2048, cu_share / 2);

  // key splits of each segment
  std::vector<int32_t>& nsplit = plan.nsplit;
  nsplit.assign(n_segs, 0);
  size_t n_items = 0, n_groups = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    const int32_t lq = segs[i].q_len;
    if (lq <= 0) continue;
    const int64_t key_tiles = (lkv[i] + KT - 1) / KT;
    int ns = target;
    if (4 * (lkv[i] + 64) > 5 * cu_share)
      ns = (int)std::max<int64_t>(ns, std::min<int64_t>(16, (lkv[i] + 64 + block_cap - 1) / block_cap));
    // decode items stream their keys at the HBM rate: cut every list into
    // chunks of about kDecodeChunk keys so that many blocks share the CUs
    if (RB == akv::DECODE_ROWS)
      ns = (int)std::max<int64_t>(ns, std::min<int64_t>(64, (lkv[i] + kDecodeChunk - 1) / kDecodeChunk));
    ns = (int)std::min<int64_t>(ns, std::max<int64_t>(1, lkv[i] / 512));
    ns = (int)std::min<int64_t>(ns, key_tiles);
    if (ns < 1) ns = 1;
    nsplit[i] = ns;
    n_groups += (size_t)L.n_kv_heads * ns;
    n_items += (size_t)L.n_kv_heads * ns * ((lq * (int64_t)G + RB - 1) / RB);
  }
  std::vector<akv::AttnItem>& all = plan.all;
  std::vector<int64_t>& cost = plan.cost;
  std::vector<AttnPlan::Group>& groups = plan.groups;
  all.resize(n_items);
  cost.resize(n_items);
  groups.resize(n_groups);
  plan.comb.clear();
  int64_t part = 0;
  int32_t at = 0, gat = 0;
  for (int32_t i = 0; i < n_segs; ++i) {
    const int32_t lq = segs[i].q_len;
    if (lq <= 0) continue;
    const int64_t rows = (int64_t)lq * G;
    const int64_t ntile_rows = (rows + RB - 1) / RB;
    const int64_t key_tiles = (lkv[i] + KT - 1) / KT;
    const int ns = nsplit[i];
    // key range of each split: whole key tiles, as even as they divide
    plan.split_kb.resize(ns);
    plan.split_ke.resize(ns);
    for (int sp = 0; sp < ns; ++sp) {
      plan.split_kb[sp] = (int32_t)(key_tiles * sp / ns * KT);
      plan.split_ke[sp] = (int32_t)std::min<int64_t>(key_tiles * (sp + 1) / ns * KT, lkv[i]);
    }
    // each row tile: its rows, one past the last key its last row sees, and
    // (split) the first partial row of its splits within one kv head
    plan.tile_rows.resize(ntile_rows);
    plan.tile_lim.resize(ntile_rows);
    plan.tile_base.resize(ntile_rows);
    int64_t head_part_rows = 0;
    for (int64_t m = 0; m < ntile_rows; ++m) {
      const int64_t nr = std::min<int64_t>(RB, rows - m * RB);
      plan.tile_rows[m] = nr;
      plan.tile_lim[m] = lkv[i] - lq + (m * RB + nr - 1) / G + 1;
      plan.tile_base[m] = head_part_rows;
      if (ns > 1) head_part_rows += ns * nr;
    }
    for (int32_t h = 0; h < L.n_kv_heads; ++h) {
      for (int sp = 0; sp < ns; ++sp) {
        const int32_t kb = plan.split_kb[sp], ke = plan.split_ke[sp];
        AttnPlan::Group gr{0, at, 0};
        for (int64_t m = 0; m < ntile_rows; ++m, ++at) {
          const int64_t keys = std::max<int64_t>(0, std::min<int64_t>(ke, plan.tile_lim[m]) - kb);
          const int32_t pidx = ns > 1 ? (int32_t)(part + plan.tile_base[m] + sp * plan.tile_rows[m]) : -1;
          all[at] = {i, h, (int32_t)(m * RB), kb, ke, pidx};
          cost[at] = keys + 64;  // + fixed cost of a block
          gr.cost += keys + 64;
        }
        gr.end = at;
        groups[gat++] = gr;
      }
      if (ns > 1) {
        for (int64_t m = 0; m < ntile_rows; ++m)
          plan.comb.push_back({i, h, (int32_t)(m * RB), (int32_t)(part + plan.tile_base[m]), ns,
                               (int32_t)plan.tile_rows[m]});
        part += head_part_rows;
      }
    }
  }
  plan.part_rows = part;
  // Longest groups first, each to the least loaded XCD, so row tiles reading
  // the same K/V share that XCD's L2; then each XCD's items are dispatched
  // longest first, so the CUs of an XCD finish together.
  // Longest first, ties in build order: a stable counting sort on the cost
  // counted down from the largest, in one pass when the costs span at most
  // 4096 values (decode plans: thousands of groups of nearly equal cost),
  // else in 11-bit digits.  The order equals a comparison sort's with
  // `begin` as tie-break.
  if (!groups.empty()) {
    int64_t cmin = groups[0].cost, cmax = 0;
    for (const AttnPlan::Group& g : groups) {
      cmax = std::max(cmax, g.cost);
      cmin = std::min(cmin, g.cost);
    }
    std::vector<AttnPlan::Group>& tmp = plan.gtmp;
    tmp.resize(groups.size());
    std::vector<uint32_t>& cnt = plan.cnt;
    auto pass = [&](int shift, int64_t mask) {
      cnt.assign((size_t)mask + 1, 0u);
      for (const AttnPlan::Group& g : groups) cnt[((cmax - g.cost) >> shift) & mask] += 1;
      uint32_t sum = 0;
      for (uint32_t& c : cnt) {
        const uint32_t c0 = c;
        c = sum;
        sum += c0;
      }
      for (const AttnPlan::Group& g : groups) tmp[cnt[((cmax - g.cost) >> shift) & mask]++] = g;
      groups.swap(tmp);
    };
    if (cmax - cmin < 4096)
      pass(0, 4095);
    else
      for (int shift = 0; shift < 63 && (cmax >> shift) != 0; shift += 11) pass(shift, 2047);
  }
  // XCD of each group, then every XCD's items in a range of `order`
  std::vector<int32_t>& gbin = plan.gbin;
  gbin.resize(groups.size());
  int64_t load[kXcds] = {};
  size_t bin_n[kXcds] = {};
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best]) best = x;
    load[best] += groups[gi].cost;
    gbin[gi] = best;
    bin_n[best] += groups[gi].end - groups[gi].begin;
  }
  size_t bin_at[kXcds + 1] = {};
  for (int x = 0; x < kXcds; ++x) bin_at[x + 1] = bin_at[x] + bin_n[x];
  std::vector<int32_t>& order = plan.order;
  order.resize(all.size());
  {
    size_t fill[kXcds];
    std::copy(bin_at, bin_at + kXcds, fill);
    for (size_t gi = 0; gi < groups.size(); ++gi)
      for (int32_t k = groups[gi].begin; k < groups[gi].end; ++k) order[fill[gbin[gi]]++] = k;
  }
  size_t depth = 0;
  auto longer = [&](int32_t a, int32_t b) { return cost[a] > cost[b]; };
  for (int x = 0; x < kXcds; ++x) {
    auto b0 = order.begin() + bin_at[x], b1 = order.begin() + bin_at[x + 1];
    // one-item groups (decode) arrive already in this order
    if (!std::is_sorted(b0, b1, longer)) std::stable_sort(b0, b1, longer);
    depth = std::max(depth, bin_n[x]);
  }
  plan.items.assign(depth * kXcds, akv::AttnItem{-1, 0, 0, 0, 0, -1});
  for (int x = 0; x < kXcds; ++x)
    for (size_t i = 0; i < bin_n[x]; ++i) plan.items[i * kXcds + x] = all[order[bin_at[x] + i]];
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* akv_last_error(void) { return g_err.c_str(); }

akv_status akv_pool_create(const akv_layout* layout, const int32_t* page_order, void* k_pages,
                           void* kpe_pages, void* v_pages, void* scratch, size_t scratch_bytes,
                           void* hip_stream, akv_pool** out) {
  try {
    if (!layout || !out) return fail(AKV_EINVAL, "layout and out must be non-NULL");
    const akv_layout& L = *layout;
    if (L.n_kv_heads <= 0 || L.n_q_heads <= 0 || L.n_q_heads % L.n_kv_heads)
      return fail(AKV_EINVAL, "n_q_heads must be a positive multiple of n_kv_heads");
    if (L.d_rope <= 0 || L.d_rope % 16 || L.d_rope > 256)
      return fail(AKV_EINVAL, "d_rope must be a multiple of 16 in 16..256");
    if (L.d_nope < 0 || L.d_nope % 8 || L.d_v <= 0 || L.d_v % 8)
      return fail(AKV_EINVAL, "d_nope and d_v must be multiples of 8");
    if (L.page_size < 1 || L.page_size > 256 || (L.page_size & (L.page_size - 1)))
      return fail(AKV_EINVAL, "page_size must be a power of two in 1..256");
    if (L.num_pages <= 0 || (int64_t)L.num_pages * L.page_size > kInt32Max)
      return fail(AKV_EINVAL, "num_pages out of range");
    // the kernels form row indices with 24-bit multiplies (page * heads *
    // page_size) and keep them in 32 bits
    if (L.num_pages >= (1 << 24)) return fail(AKV_EINVAL, "num_pages must be below 2^24");
    if ((int64_t)L.num_pages * L.n_kv_heads * L.page_size >= (int64_t(1) << 32) ||
        (int64_t)L.n_kv_heads * L.page_size >= (1 << 24))
      return fail(AKV_EINVAL, "num_pages x n_kv_heads x page_size must be below 2^32");
    if (L.pairing != 0 && L.pairing != 1) return fail(AKV_EINVAL, "pairing must be 0 or 1");
    if (L.d_nope == 0 && L.kpe_per_head) return fail(AKV_EINVAL, "kpe_per_head needs an MLA layout");
    const bool any_dev = k_pages || kpe_pages || v_pages || scratch;
    if (any_dev) {
      if (!k_pages || !v_pages) return fail(AKV_EINVAL, "k_pages and v_pages are required");
      if ((L.d_nope > 0) != (kpe_pages != nullptr))
        return fail(AKV_EINVAL, "kpe_pages is required exactly for MLA layouts (d_nope > 0)");
      if (!scratch) return fail(AKV_EINVAL, "scratch is required for a device pool");
    }
    if (!L.inv_freq && !(L.rope_theta > 0)) return fail(AKV_EINVAL, "rope_theta must be > 0");
    std::vector<int32_t> order(L.num_pages);
    if (page_order) {
      std::vector<uint8_t> seen(L.num_pages, 0);
      for (int32_t i = 0; i < L.num_pages; ++i) {
        const int32_t pg = page_order[i];
        if (pg < 0 || pg >= L.num_pages || seen[pg])
          return fail(AKV_EINVAL, "page_order is not a permutation of 0..num_pages-1");
        seen[pg] = 1;
        order[i] = pg;
      }
    } else {
      for (int32_t i = 0; i < L.num_pages; ++i) order[i] = i;
    }
    akv_pool* p = new akv_pool();
    p->L = L;
    p->L.inv_freq = nullptr;
    p->inv_freq.resize(L.d_rope / 2);
    for (int i = 0; i < L.d_rope / 2; ++i)
      p->inv_freq[i] = L.inv_freq ? L.inv_freq[i] : std::pow(L.rope_theta, -2.0 * i / L.d_rope);
    p->log2S = 0;
    while ((1 << p->log2S) < L.page_size) ++p->log2S;
    p->thr = L.compact_threshold > 0 ? L.compact_threshold : dbg().thr;
    p->free_q.assign(order.begin(), order.end());
    p->pages.resize(L.num_pages);
    p->device = any_dev;
    if (p->device) {
      p->k = (uint16_t*)k_pages;
      p->kpe = (uint16_t*)kpe_pages;
      p->v = (uint16_t*)v_pages;
      p->scratch = (char*)scratch;
      p->scratch_bytes = scratch_bytes;
      p->stream = (hipStream_t)hip_stream;
      if (scratch_bytes < 65536) {
        delete p;
        return fail(AKV_ENOMEM, "scratch must hold at least 65536 bytes");
      }
      hipError_t ce = hipStreamCreateWithFlags(&p->cstream, hipStreamNonBlocking);
      if (ce != hipSuccess) {
        p->cstream = nullptr;
        delete p;
        return hip_fail(ce, "hipStreamCreateWithFlags(copy stream)");
      }
      ce = hipStreamCreateWithFlags(&p->kstream, hipStreamNonBlocking);
      if (ce == hipSuccess) ce = hipEventCreateWithFlags(&p->bg_done, hipEventDisableTiming);
      if (ce == hipSuccess) ce = hipEventCreateWithFlags(&p->write_ev, hipEventDisableTiming);
      if (ce == hipSuccess) ce = hipEventCreateWithFlags(&p->free_ev, hipEventDisableTiming);
      if (ce != hipSuccess) {
        akv_pool_destroy(p);
        return hip_fail(ce, "background compaction stream");
      }
      p->page_bg.assign(L.num_pages, 0);
      int dev = 0;
      hipDeviceProp_t prop;
      if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
        p->n_cu = prop.multiProcessorCount;
      p->scratch_base = 0;
      p->ring_head = 0;
    }
    *out = p;
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_pool_destroy(akv_pool* p) {
  if (!p) return AKV_OK;
  if (p->device) (void)hipStreamSynchronize(p->stream);
  if (p->cstream) {
    (void)hipStreamSynchronize(p->cstream);
    (void)hipStreamDestroy(p->cstream);
  }
  if (p->kstream) {
    (void)hipStreamSynchronize(p->kstream);
    (void)hipStreamDestroy(p->kstream);
  }
  if (p->bg_done) (void)hipEventDestroy(p->bg_done);
  if (p->write_ev) (void)hipEventDestroy(p->write_ev);
  if (p->free_ev) (void)hipEventDestroy(p->free_ev);
  for (auto& r : p->stg.pending) (void)hipEventDestroy(r.ev);
  for (auto e : p->stg.spare) (void)hipEventDestroy(e);
  if (p->stg.base) (void)hipHostFree(p->stg.base);
  for (auto& t : p->tev) {
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  for (auto e : p->ev_spare) (void)hipEventDestroy(e);
  delete p;
  return AKV_OK;
}

akv_status akv_seq_create(akv_pool* p, int32_t* seq) {
  if (!p || !seq) return fail(AKV_EINVAL, "NULL argument");
  try {
    p->seqs.emplace_back();
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
  *seq = (int32_t)p->seqs.size() - 1;
  p->seqs.back().id = *seq;
  return AKV_OK;
}

akv_status akv_seq_release(akv_pool* p, int32_t s) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  SeqRec* q;
  akv_status st = get_seq(p, s, &q);
  if (st != AKV_OK) return st;
  // slots this sequence holds in other sequences' pages are given up
  const int32_t len = (int32_t)q->slot.size();
  for (int32_t t = 0; t < len; ++t)
    if (foreign_slot(p, s, q->slot[t])) q->slot[t] = -1;
  const std::vector<std::pair<int32_t, int32_t>> held(q->owners.begin(), q->owners.end());
  q->owners.clear();
  q->fvis.clear();
  q->alive = false;
  if (q->queued) {
    p->compact_q.erase(std::find(p->compact_q.begin(), p->compact_q.end(), s));
    q->queued = false;
  }
  q->vis.clear();
  q->stale();
  for (const auto& h : held) {
    SeqRec& so = p->seqs[h.first];
    if (--so.refs == 0 && so.zombie) finish_release(p, h.first);
  }
  // pages other sequences still read stay until the last of them lets go
  if (q->refs > 0)
    q->zombie = true;
  else
    finish_release(p, s);
  return AKV_OK;
}

akv_status akv_append(akv_pool* p, int32_t s, const void* K, const void* K_pe, const void* V,
                      const int32_t* pos, int32_t n) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    if (n < 0) return fail(AKV_EINVAL, "negative token count");
    if (n == 0) return AKV_OK;
    if (!pos) return fail(AKV_EINVAL, "pos is NULL");
    const bool mla = p->L.d_nope > 0;
    const bool none = !K && !K_pe && !V;
    if (!none) {
      if (!p->device) return fail(AKV_EINVAL, "a page-table-only pool takes no K/V data");
      if (!K || !V || (mla != (K_pe != nullptr)))
        return fail(AKV_EINVAL, "K and V (and K_pe exactly for MLA) must be given together");
    }
    for (int32_t i = 0; i < n; ++i)
      if (pos[i] < 0) return fail(AKV_ERANGE, "position %d of token %d is negative", pos[i], i);
    if ((int64_t)q->slot.size() + n > kInt32Max) return fail(AKV_ERANGE, "sequence too long");
    if (pages_needed(p, *q, n) > available(p))
      return fail(AKV_ENOMEM, "pool exhausted: %lld pages needed, %lld available",
                  (long long)pages_needed(p, *q, n), (long long)available(p));
    if (!none) {
      st = scratch_fits(p, (size_t)n * 4 + 256);
      if (st != AKV_OK) return st;
    }
    std::vector<int32_t> slots(n);
    place_tokens(p, s, n, pos, slots.data());
    return device_append(p, slots, K, K_pe, V);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_clone(akv_pool* p, int32_t src, int32_t first, int32_t n, int32_t dst,
                         int32_t delta) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* qs;
    SeqRec* qd;
    akv_status st = get_seq(p, src, &qs);
    if (st == AKV_OK) st = get_live_seq(p, dst, &qd);
    if (st != AKV_OK) return st;
    if (n < 0) return fail(AKV_EINVAL, "negative token count");
    if (first < 0 || (int64_t)first + n > (int64_t)qs->slot.size())
      return fail(AKV_ERANGE, "tokens [%d,%lld) outside sequence %d of %zu tokens", first,
                  (long long)first + n, src, qs->slot.size());
    std::vector<int32_t> pos;
    std::vector<akv::MovePair> mv;
    for (int32_t t = first; t < first + n; ++t) {
      if (qs->dropped[t]) continue;
      const int64_t np = (int64_t)qs->pos[t] + delta;
      if (np < 0 || np > kInt32Max)
        return fail(AKV_ERANGE, "token %d would move to position %lld", t, (long long)np);
      pos.push_back((int32_t)np);
      mv.push_back({qs->slot[t], -1});
    }
    const int32_t m = (int32_t)pos.size();
    if (m == 0) return AKV_OK;
    if ((int64_t)qd->slot.size() + m > kInt32Max) return fail(AKV_ERANGE, "sequence too long");
    if (pages_needed(p, *qd, m) > available(p))
      return fail(AKV_ENOMEM, "pool exhausted: %lld pages needed, %lld available",
                  (long long)pages_needed(p, *qd, m), (long long)available(p));
    st = scratch_fits(p, (size_t)m * sizeof(akv::MovePair) + 4 + (size_t)p->L.d_rope * 4 + 3 * 256);
    if (st != AKV_OK) return st;
    std::vector<int32_t> lags;
    lags.reserve(m);
    for (int32_t t = first; t < first + n; ++t)
      if (!qs->dropped[t]) lags.push_back(qs->lag[t]);
    std::vector<int32_t> slots(m);
    place_tokens(p, dst, m, pos.data(), slots.data());
    SeqRec& qd2 = p->seqs[dst];   // the copies owe what their sources owe
    for (int32_t i = 0; i < m; ++i) {
      mv[i].dst = slots[i];
      const size_t t = qd2.slot.size() - m + i;
      qd2.lag[t] = lags[i];
      if (lags[i]) {
        qd2.lagging = true;
        qd2.lg_ok = false;
      }
    }
    if (dbg().checks) {
      akv_status cst = check_moves(p, mv.data(), mv.size(), "clone");
      if (cst != AKV_OK) return cst;
    }
    trace("clone: %d rows of seq %d into seq %d turned by %d", m, src, dst, delta);
    if (!p->device) return AKV_OK;
    ScratchCursor sc(p, mv.size() * sizeof(akv::MovePair) + (size_t)p->L.d_rope * 4 + 3 * 256);
    const std::vector<float>& tab = rot_table_rows(p, &delta, 1);
    void* dv[2];
    st = upload_arrays(p, sc, {{mv.data(), mv.size() * sizeof(akv::MovePair)},
                               {tab.data(), delta != 0 ? tab.size() * 4 : 0}}, dv);
    if (st != AKV_OK) return st;
    const void* dmv = dv[0];
    const float* dtab = (const float*)dv[1];
    hipError_t e;
    st = bg_wait(p);
    if (st != AKV_OK) return st;
    KTimer tm(p, AKV_K_CLONE);
    e = move_tokens(p, (const akv::MovePair*)dmv, m, delta != 0 ? dtab : nullptr);
    tm.done();
    note_write(p);
    return check_launch(e, "clone kernel launch");
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_freeze(akv_pool* p, int32_t s) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_seq(p, s, &q);
    if (st != AKV_OK) return st;
    if (q->frozen) return AKV_OK;
    // sharers read the rows as stored: keys owing a rotation are turned first
    st = materialize_seq(p, *q);
    if (st != AKV_OK) return st;
    q->frozen = true;
    if (q->queued) {
      p->compact_q.erase(std::find(p->compact_q.begin(), p->compact_q.end(), s));
      q->queued = false;
    }
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_share(akv_pool* p, int32_t src, int32_t first, int32_t n, int32_t dst, int32_t delta) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* qs;
    SeqRec* qd;
    akv_status st = get_seq(p, src, &qs);
    if (st == AKV_OK) st = get_live_seq(p, dst, &qd);
    if (st != AKV_OK) return st;
    if (!qs->frozen) return fail(AKV_ESTATE, "sequence %d is not frozen (akv_seq_freeze)", src);
    if (n < 0) return fail(AKV_EINVAL, "negative token count");
    if (first < 0 || (int64_t)first + n > (int64_t)qs->slot.size())
      return fail(AKV_ERANGE, "tokens [%d,%lld) outside sequence %d of %zu tokens", first,
                  (long long)first + n, src, qs->slot.size());
    int64_t m = 0;
    for (int32_t t = first; t < first + n; ++t) {
      if (qs->dropped[t]) continue;
      const int64_t np = (int64_t)qs->pos[t] + delta;
      if (np < 0 || np > kInt32Max)
        return fail(AKV_ERANGE, "token %d would move to position %lld", t, (long long)np);
      ++m;
    }
    if (m == 0) return AKV_OK;
    if ((int64_t)qd->slot.size() + m > kInt32Max) return fail(AKV_ERANGE, "sequence too long");
    // the new tokens hold the source's slots: nothing is written
    for (int32_t t = first; t < first + n; ++t) {
      if (qs->dropped[t]) continue;
      const int32_t slot = qs->slot[t];
      const int32_t pg = slot >> p->log2S;
      const int32_t o = p->pages[pg].owner;
      if (qd->owners[o]++ == 0) p->seqs[o].refs += 1;
      qd->fvis[pg] += 1;
      qd->slot.push_back(slot);
      qd->pos.push_back((int32_t)(qs->pos[t] + delta));
      qd->dropped.push_back(0);
      qd->lag.push_back((int32_t)(qs->lag[t] + delta));
    }
    qd->n_vis += m;
    if (delta != 0) {
      qd->lagging = true;
      qd->lg_ok = false;
    }
    qd->stale();
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_append_batch(akv_pool* p, int32_t n_seqs, const int32_t* seqs, const int32_t* counts,
                            const void* K, const void* K_pe, const void* V, const int32_t* pos) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    if (n_seqs < 0) return fail(AKV_EINVAL, "negative sequence count");
    if (n_seqs == 0) return AKV_OK;
    if (!seqs || !counts) return fail(AKV_EINVAL, "seqs and counts must be non-NULL");
    const bool mla = p->L.d_nope > 0;
    const bool none = !K && !K_pe && !V;
    if (!none) {
      if (!p->device) return fail(AKV_EINVAL, "a page-table-only pool takes no K/V data");
      if (!K || !V || (mla != (K_pe != nullptr)))
        return fail(AKV_EINVAL, "K and V (and K_pe exactly for MLA) must be given together");
    }
    // validate every entry; count pages with each sequence's tail room as the
    // entries before it leave it
    const int64_t S = p->L.page_size;
    std::unordered_map<int32_t, std::pair<int64_t, int64_t>> st_of;   // seq -> (room, tokens)
    int64_t total = 0, pages = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
      SeqRec* q;
      akv_status st = get_live_seq(p, seqs[i], &q);
      if (st != AKV_OK) return st;
      if (counts[i] < 0) return fail(AKV_EINVAL, "entry %d: negative token count", i);
      auto it = st_of.find(seqs[i]);
      if (it == st_of.end())
        it = st_of.emplace(seqs[i], std::make_pair(q->tail >= 0 ? S - p->pages[q->tail].filled : 0,
                                                   (int64_t)q->slot.size())).first;
      int64_t& room = it->second.first;
      int64_t& len = it->second.second;
      const int64_t n = counts[i];
      const int64_t extra = std::max<int64_t>(0, n - room);
      pages += (extra + S - 1) / S;
      room = n <= room ? room - n : (S - extra % S) % S;
      len += n;
      if (len > kInt32Max) return fail(AKV_ERANGE, "sequence %d too long", seqs[i]);
      total += n;
      if (total > kInt32Max) return fail(AKV_ERANGE, "too many tokens in one call");
    }
    if (total == 0) return AKV_OK;
    if (!pos) return fail(AKV_EINVAL, "pos is NULL");
    for (int64_t t = 0; t < total; ++t)
      if (pos[t] < 0) return fail(AKV_ERANGE, "position %d of token %lld is negative", pos[t], (long long)t);
    if (pages > available(p))
      return fail(AKV_ENOMEM, "pool exhausted: %lld pages needed, %lld available", (long long)pages,
                  (long long)available(p));
    if (!none) {
      akv_status st = scratch_fits(p, (size_t)total * 4 + 256);
      if (st != AKV_OK) return st;
    }
    std::vector<int32_t> slots((size_t)total);
    int64_t off = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
      place_tokens(p, seqs[i], counts[i], pos + off, slots.data() + off);
      off += counts[i];
    }
    return device_append(p, slots, K, K_pe, V);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_drop(akv_pool* p, int32_t s, const akv_span* spans, int32_t n) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    st = check_spans(spans, n, (int32_t)q->slot.size());
    if (st != AKV_OK) return st;
    st = scratch_fits(p, (size_t)q->n_vis * sizeof(akv::MovePair) + 256);
    if (st != AKV_OK) return st;
    for (int32_t i = 0; i < n; ++i) drop_tokens(p, *q, spans[i].begin, spans[i].end, true);
    cache_after_drop(*q, spans, n);
    note_free(p);
    return auto_compact(p, s);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_compact(akv_pool* p, int32_t s, int32_t force) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    if (!force && fragmentation(p, *q) <= p->thr) return AKV_OK;
    st = scratch_fits(p, (size_t)q->n_vis * sizeof(akv::MovePair) + 256);
    if (st != AKV_OK) return st;
    return compact_seq(p, s);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_compaction_mode(akv_pool* p, int32_t mode) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  if (mode != AKV_COMPACT_IMMEDIATE && mode != AKV_COMPACT_DEFERRED)
    return fail(AKV_EINVAL, "unknown compaction mode %d", mode);
  p->compact_mode = mode;
  return AKV_OK;
}

akv_status akv_fused_rotation(akv_pool* p, int32_t mode) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  if (mode != AKV_FUSE_AUTO && mode != AKV_FUSE_ALWAYS && mode != AKV_FUSE_NEVER)
    return fail(AKV_EINVAL, "unknown fused-rotation mode %d", mode);
  p->fuse_mode = mode;
  return AKV_OK;
}

akv_status akv_compact_queue(akv_pool* p, int32_t* seqs_out, int32_t cap, int32_t* n_out) {
  if (!p || !n_out) return fail(AKV_EINVAL, "NULL argument");
  if (cap < 0 || (cap > 0 && !seqs_out)) return fail(AKV_EINVAL, "bad output");
  *n_out = (int32_t)p->compact_q.size();
  for (int32_t i = 0; i < cap && i < *n_out; ++i) seqs_out[i] = p->compact_q[i];
  return AKV_OK;
}

akv_status akv_compact_pending(akv_pool* p, int64_t max_tokens, int32_t max_seqs, int32_t* seqs_out,
                               int32_t* n_out) {
  try {
    if (!p || !n_out) return fail(AKV_EINVAL, "NULL argument");
    if (max_tokens < 0 || max_seqs < 0) return fail(AKV_EINVAL, "negative budget");
    *n_out = 0;
    const int32_t S = p->L.page_size;
    std::vector<akv::MovePair> mv;
    bool from_evict = false;   // this batch takes fresh pages from the evictable queue
    // Copies of one batch run in one launch.  A sequence whose fresh pages
    // would come from the evictable queue (possibly pages this batch still
    // reads) starts a new batch, so its copies run after the earlier ones.
    auto flush = [&]() -> akv_status {
      if (mv.empty()) return AKV_OK;
      akv_status st = device_move_bg(p, mv, from_evict);
      mv.clear();
      from_evict = false;
      return st;
    };
    int64_t used = 0;
    int32_t k = 0;
    while (!p->compact_q.empty() && k < max_seqs) {
      const int32_t s = p->compact_q.front();
      SeqRec& q = p->seqs[s];
      if (fragmentation(p, q) <= p->thr) {   // appends since queuing brought it under
        q.queued = false;
        p->compact_q.pop_front();
        continue;
      }
      const int64_t need = (q.n_vis + S - 1) / S;
      if (used + q.n_vis > max_tokens || need > available(p)) break;
      if ((int64_t)p->free_q.size() < need) {
        akv_status st = flush();
        if (st != AKV_OK) return st;
        from_evict = true;
      }
      auto fits = [&](size_t n) { return !p->device || p->scratch_base + n * sizeof(akv::MovePair) + 4352 <= p->scratch_bytes; };
      if (!fits(mv.size() + q.n_vis)) {
        akv_status st = flush();
        if (st != AKV_OK) return st;
        if (!fits(q.n_vis)) break;   // stays queued; akv_compact reports the shortage
      }
      akv_status st = compact_plan(p, s, mv);
      if (st != AKV_OK) return st;
      used += q.n_vis;
      q.queued = false;
      p->compact_q.pop_front();
      if (seqs_out) seqs_out[k] = s;
      ++k;
      *n_out = k;
    }
    return flush();
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_repos_deferred(akv_pool* p, int32_t s, const akv_span* spans, const int32_t* delta,
                              int32_t n) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    std::vector<Run> runs;
    st = repos_runs(*q, spans, delta, n, runs);
    if (st != AKV_OK) return st;
    for (const Run& r : runs)
      for (int32_t t = r.b; t < r.e; ++t)
        if (!q->dropped[t]) {
          q->lag[t] = (int32_t)(q->lag[t] + r.d);
          q->lagging = true;
        }
    q->lg_ok = false;
    repos_commit(p, *q, runs, false);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_materialize(akv_pool* p, int32_t s) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_seq(p, s, &q);
    if (st != AKV_OK) return st;
    return materialize_seq(p, *q);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_lag(akv_pool* p, int32_t s, int32_t first, int32_t n, int32_t* lag) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  SeqRec* q;
  akv_status st = get_seq(p, s, &q);
  if (st != AKV_OK) return st;
  if (first < 0 || n < 0 || (int64_t)first + n > (int64_t)q->slot.size())
    return fail(AKV_ERANGE, "tokens %d..%d outside 0..%zu", first, first + n, q->slot.size());
  if (n > 0 && !lag) return fail(AKV_EINVAL, "lag is NULL");
  for (int32_t i = 0; i < n; ++i) lag[i] = q->lag[first + i];
  return AKV_OK;
}

akv_status akv_repos(akv_pool* p, int32_t s, const akv_span* spans, const int32_t* delta,
                     int32_t n) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    std::vector<Run> runs;
    st = repos_runs(*q, spans, delta, n, runs);
    if (st != AKV_OK) return st;
    std::vector<akv::RotItem> items;
    std::vector<int32_t> deltas;
    repos_items(p, *q, runs, items, deltas);
    st = scratch_fits(p, rotate_scratch_bytes(p, items.size(), deltas.size(), 1));
    if (st != AKV_OK) return st;
    st = device_rotate(p, items, deltas);
    if (st != AKV_OK) return st;
    repos_commit(p, *q, runs);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_repos_batch(akv_pool* p, int32_t n_seqs, const int32_t* seqs, const int32_t* span_counts,
                           const akv_span* spans, const int32_t* delta) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    if (n_seqs < 0) return fail(AKV_EINVAL, "negative sequence count");
    if (n_seqs == 0) return AKV_OK;
    if (!seqs || !span_counts) return fail(AKV_EINVAL, "seqs and span_counts must be non-NULL");
    // validate every entry before any change: sequences distinct (two
    // entries on one sequence would put two items on one slot in a launch)
    std::vector<std::vector<Run>> runs((size_t)n_seqs);
    std::unordered_map<int32_t, int32_t> seen;
    int64_t off = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
      SeqRec* q;
      akv_status st = get_live_seq(p, seqs[i], &q);
      if (st != AKV_OK) return st;
      if (!seen.emplace(seqs[i], i).second)
        return fail(AKV_EINVAL, "entries %d and %d name the same sequence %d", seen[seqs[i]], i, seqs[i]);
      if (span_counts[i] < 0) return fail(AKV_EINVAL, "entry %d: negative span count", i);
      st = repos_runs(*q, spans ? spans + off : nullptr, delta ? delta + off : nullptr, span_counts[i], runs[i]);
      if (st != AKV_OK) return st;
      off += span_counts[i];
    }
    std::vector<akv::RotItem> items;
    std::vector<int32_t> deltas;
    std::unordered_map<int64_t, int32_t> didx;
    for (int32_t i = 0; i < n_seqs; ++i) repos_items_append(p, p->seqs[seqs[i]], runs[i], items, deltas, didx);
    sort_by_first_slot(items, p->L.page_size);
    akv_status st = scratch_fits(p, rotate_scratch_bytes(p, items.size(), deltas.size(), 1));
    if (st != AKV_OK) return st;
    st = device_rotate(p, items, deltas);
    if (st != AKV_OK) return st;
    for (int32_t i = 0; i < n_seqs; ++i) repos_commit(p, p->seqs[seqs[i]], runs[i]);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_repos_layers(akv_pool* const* pools, int32_t n_pools, int32_t s, const akv_span* spans,
                            const int32_t* delta, int32_t n) {
  try {
    if (!pools || n_pools <= 0) return fail(AKV_EINVAL, "no pools");
    akv_pool* p = pools[0];
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    std::vector<SeqRec*> qs{q};
    std::vector<akv_pool*> layers{p};
    for (int32_t i = 1; i < n_pools; ++i) {
      akv_pool* o = pools[i];
      if (!o) return fail(AKV_EINVAL, "pool %d is NULL", i);
      for (int32_t k = 0; k < i; ++k)
        if (pools[k] == o) return fail(AKV_EINVAL, "pool %d is listed twice", i);
      const akv_layout &A = p->L, &B = o->L;
      if (A.n_kv_heads != B.n_kv_heads || A.d_nope != B.d_nope || A.d_rope != B.d_rope ||
          A.page_size != B.page_size || A.num_pages != B.num_pages || A.kpe_per_head != B.kpe_per_head ||
          A.pairing != B.pairing || p->inv_freq != o->inv_freq)
        return fail(AKV_EINVAL, "pool %d has another layout or frequency table", i);
      if (o->device != p->device || o->stream != p->stream)
        return fail(AKV_EINVAL, "pool %d runs on another stream", i);
      SeqRec* oq;
      st = get_seq(o, s, &oq);
      if (st != AKV_OK) return st;
      if (oq->slot != q->slot || oq->pos != q->pos || oq->dropped != q->dropped)
        return fail(AKV_EINVAL, "pool %d: sequence %d differs from pool 0's", i, s);
      qs.push_back(oq);
      layers.push_back(o);
    }
    std::vector<Run> runs;
    st = repos_runs(*q, spans, delta, n, runs);
    if (st != AKV_OK) return st;
    std::vector<akv::RotItem> items;
    std::vector<int32_t> deltas;
    repos_items(p, *q, runs, items, deltas);
    st = scratch_fits(p, rotate_scratch_bytes(p, items.size(), deltas.size(), n_pools));
    if (st != AKV_OK) return st;
    st = device_rotate(p, items, deltas, layers);
    if (st != AKV_OK) return st;
    for (size_t i = 0; i < qs.size(); ++i) repos_commit(layers[i], *qs[i], runs);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_repos_plan(akv_pool* p, int32_t s, const akv_span* spans, const int32_t* delta,
                          int32_t n, int32_t* slot_out, int32_t* delta_out, int32_t cap,
                          int32_t* n_out) {
  try {
    if (!p || !n_out) return fail(AKV_EINVAL, "NULL argument");
    SeqRec* q;
    akv_status st = get_seq(p, s, &q);
    if (st != AKV_OK) return st;
    std::vector<Run> runs;
    st = repos_runs(*q, spans, delta, n, runs);
    if (st != AKV_OK) return st;
    std::vector<akv::RotItem> items;
    std::vector<int32_t> deltas;
    repos_items(p, *q, runs, items, deltas);
    int32_t k = 0;
    const int32_t S = p->L.page_size;
    for (auto& it : items)
      for (int32_t o = it.lo; o < it.hi; ++o) {
        if (k < cap) {
          if (slot_out) slot_out[k] = it.page * S + o;
          if (delta_out) delta_out[k] = deltas[it.didx];
        }
        ++k;
      }
    *n_out = k;
    if (k > cap) return fail(AKV_ERANGE, "plan has %d entries, cap %d", k, cap);
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_splice(akv_pool* p, int32_t s, const akv_span* spans, const int32_t* stub_len,
                      int32_t n, const void* sK, const void* sKpe, const void* sV,
                      int32_t* stub_pos_out) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    SeqRec* q;
    akv_status st = get_live_seq(p, s, &q);
    if (st != AKV_OK) return st;
    if (n < 0) return fail(AKV_EINVAL, "negative splice count");
    if (n == 0) return AKV_OK;
    if (!spans || !stub_len) return fail(AKV_EINVAL, "spans and stub_len are required");
    const std::vector<int32_t> vis = visible(*q);
    const int32_t H = (int32_t)vis.size();
    int64_t n_stub = 0;
    for (int32_t j = 0; j < n; ++j) {
      if (spans[j].begin >= spans[j].end || stub_len[j] < 0)
        return fail(AKV_EINVAL, "splice %d: empty span or negative stub", j);
      if (spans[j].begin < 0 || spans[j].end > H)
        return fail(AKV_ERANGE, "splice %d outside the visible list of %d entries", j, H);
      if (j && spans[j].begin < spans[j - 1].end)
        return fail(AKV_EINVAL, "splice spans must be sorted and disjoint");
      n_stub += stub_len[j];
    }
    const bool mla = p->L.d_nope > 0;
    const bool none = !sK && !sKpe && !sV;
    if (n_stub > 0 && !none) {
      if (!p->device) return fail(AKV_EINVAL, "a page-table-only pool takes no K/V data");
      if (!sK || !sV || (mla != (sKpe != nullptr)))
        return fail(AKV_EINVAL, "stub K and V (and K_pe exactly for MLA) must be given together");
    }
    // per-splice delta |R| - (end - begin), downstream sums, stub positions
    std::vector<int64_t> dj(n);
    for (int32_t j = 0; j < n; ++j) dj[j] = (int64_t)stub_len[j] - (spans[j].end - spans[j].begin);
    std::vector<int64_t> down(H, 0);
    {
      int64_t run = 0;
      int32_t j = 0;
      for (int32_t i = 0; i < H; ++i) {
        while (j < n && spans[j].end <= i) run += dj[j++];
        down[i] = run;
      }
    }
    std::vector<int32_t> stub_pos;
    stub_pos.reserve(n_stub);
    {
      int64_t before = 0;
      for (int32_t j = 0; j < n; ++j) {
        const int64_t p0 = (int64_t)q->pos[vis[spans[j].begin]] + before;
        for (int32_t k = 0; k < stub_len[j]; ++k) {
          const int64_t ps = p0 + k;
          if (ps < 0 || ps > kInt32Max) return fail(AKV_ERANGE, "stub position out of range");
          stub_pos.push_back((int32_t)ps);
        }
        before += dj[j];
      }
    }
    std::vector<uint8_t> in_span(H, 0);
    for (int32_t j = 0; j < n; ++j)
      for (int32_t i = spans[j].begin; i < spans[j].end; ++i) in_span[i] = 1;
    std::vector<Run> runs;
    for (int32_t i = 0; i < H; ++i) {
      if (in_span[i] || down[i] == 0) continue;
      const int64_t np = (int64_t)q->pos[vis[i]] + down[i];
      if (np < 0 || np > kInt32Max) return fail(AKV_ERANGE, "splice moves a position out of range");
      if (!runs.empty() && runs.back().e == vis[i] && runs.back().d == down[i])
        runs.back().e = vis[i] + 1;
      else
        runs.push_back({vis[i], vis[i] + 1, down[i]});
    }
    // pages for the stubs, counting those the drop will make evictable
    {
      std::vector<int32_t> nv_left;
      int64_t freed = 0;
      std::unordered_map<int32_t, int32_t> dec;
      for (int32_t i = 0; i < H; ++i)
        if (in_span[i]) dec[q->slot[vis[i]] / p->L.page_size] += 1;
      for (auto& kv : dec) {
        const PageRec& r = p->pages[kv.first];
        if (r.nvis - kv.second == 0 && kv.first != q->tail && !r.in_evict) ++freed;
      }
      if (pages_needed(p, *q, n_stub) > available(p) + freed)
        return fail(AKV_ENOMEM, "pool exhausted for the splice stubs");
    }
    // worst-case scratch of the stub copy, the rotation list and a compaction
    st = scratch_fits(p, std::max<size_t>((size_t)n_stub * 4 + (size_t)H * (sizeof(akv::RotItem) + 4) + 1024,
                                          (size_t)(q->n_vis + n_stub) * sizeof(akv::MovePair) + 256));
    if (st != AKV_OK) return st;
    // apply: drop, append stubs, rotate downstream (one launch), positions
    for (int32_t i = 0; i < H; ++i)
      if (in_span[i]) drop_tokens(p, *q, vis[i], vis[i] + 1);
    note_free(p);
    if (n_stub > 0) {
      std::vector<int32_t> slots(n_stub);
      place_tokens(p, s, (int32_t)n_stub, stub_pos.data(), slots.data());
      st = device_append(p, slots, sK, sKpe, sV);
      if (st != AKV_OK) return st;
    }
    std::vector<akv::RotItem> items;
    std::vector<int32_t> deltas;
    repos_items(p, *q, runs, items, deltas);
    st = device_rotate(p, items, deltas);
    if (st != AKV_OK) return st;
    repos_commit(p, *q, runs);
    if (stub_pos_out) std::copy(stub_pos.begin(), stub_pos.end(), stub_pos_out);
    return auto_compact(p, s);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_visible(akv_pool* p, int32_t s, const akv_span* mask, int32_t n_mask,
                           akv_extent* out, int32_t cap, int32_t* n_out) {
  try {
    if (!p || !n_out) return fail(AKV_EINVAL, "NULL argument");
    SeqRec* q;
    akv_status st = get_seq(p, s, &q);
    if (st != AKV_OK) return st;
    st = check_spans(mask, n_mask, (int32_t)q->slot.size());
    if (st != AKV_OK) return st;
    const std::vector<int32_t>& vis = visible(*q);
    std::vector<akv_extent> masked;
    if (n_mask > 0 && q->vis_logical) {
      if (!q->ext_ok) {
        build_extents(p, *q, vis, nullptr, q->ext);
        q->ext_ok = true;
      }
      masked_from_image(*q, mask, n_mask, masked);
    } else if (n_mask > 0) {
      std::vector<uint8_t> hide(q->slot.size(), 0);
      for (int32_t i = 0; i < n_mask; ++i)
        std::fill(hide.begin() + mask[i].begin, hide.begin() + mask[i].end, 1);
      build_extents(p, *q, vis, &hide, masked);
    } else if (!q->ext_ok) {
      build_extents(p, *q, vis, nullptr, q->ext);
      q->ext_ok = true;
    }
    const std::vector<akv_extent>& ex = n_mask > 0 ? masked : q->ext;
    *n_out = (int32_t)ex.size();
    if ((int32_t)ex.size() > cap) return fail(AKV_ERANGE, "%zu extents, cap %d", ex.size(), cap);
    if (!ex.empty()) {
      if (!out) return fail(AKV_EINVAL, "out is NULL");
      std::memcpy(out, ex.data(), ex.size() * sizeof(akv_extent));
    }
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

static bool decode_launch(const akv_pool* p, const int64_t* q_len, int32_t n, int32_t stride);
// The prefill kernel that turns owed keys in LDS: the 128-dim GQA layout.
static bool rotating_prefill(const akv_pool* p) {
  return p->L.d_nope == 0 && p->L.d_rope == 128 && p->L.d_v == 128;
}
static akv_status attention_impl(akv_pool* p, const void* Q, int32_t n_q_tokens, const akv_segment* segs,
                                 int32_t n_segs, const akv_extent* page_lists, int32_t n_ext,
                                 const int32_t* ext_lag, float scale, void* out, bool ws_static = false);

akv_status akv_seq_attention(akv_pool* p, const void* Q, int32_t n_q_tokens, const akv_seq_segment* segs,
                             int32_t n_segs, const akv_span* masks, int32_t n_masks, float scale, void* out) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    if (n_segs < 0 || n_masks < 0) return fail(AKV_EINVAL, "negative count");
    if ((n_segs > 0 && !segs) || (n_masks > 0 && !masks)) return fail(AKV_EINVAL, "segments / masks are NULL");
    bool lagging = false;
    std::vector<int64_t> qlens(n_segs);
    for (int32_t i = 0; i < n_segs; ++i) {
      const akv_seq_segment& sg = segs[i];
      SeqRec* q;
      akv_status st = get_seq(p, sg.seq, &q);
      if (st != AKV_OK) return st;
      if (sg.mask_len < 0 || sg.mask_begin < 0 || (int64_t)sg.mask_begin + sg.mask_len > n_masks)
        return fail(AKV_EINVAL, "segment %d: mask spans outside 0..%d", i, n_masks);
      st = check_spans(masks ? masks + sg.mask_begin : nullptr, sg.mask_len, (int32_t)q->slot.size());
      if (st != AKV_OK) return st;
      lagging = lagging || q->lagging;
      qlens[i] = sg.q_len;
    }
    // Owed rotations (deferred repos) are applied inside the attention
    // kernels that turn keys where they read them (the decode kernel, and the
    // direct-to-LDS prefill kernel of the 128-dim GQA layout), or the keys are
    // first rotated in place (akv_fused_rotation picks; by default a prefill
    // launch fuses only when it turns each owed key at most once per kv head:
    // one row tile per segment and one segment per sequence; a prefill block
    // turns every tile it reads, so keys read by many row tiles are cheaper
    // to rotate once in place).
    bool fused = false;
    if (lagging && p->device && p->fuse_mode != AKV_FUSE_NEVER) {
      if (decode_launch(p, qlens.data(), n_segs, 1)) {
        fused = true;
      } else if (rotating_prefill(p)) {
        fused = p->fuse_mode == AKV_FUSE_ALWAYS;
        if (!fused) {
          const akv_layout& L = p->L;
          const int64_t G = L.n_q_heads / L.n_kv_heads;
          std::unordered_map<int32_t, int> uses;
          bool once = true;
          for (int32_t i = 0; i < n_segs && once; ++i)
            once = segs[i].q_len * G <= akv::attn_rows_per_block(L.d_nope) && ++uses[segs[i].seq] == 1;
          fused = once;
        }
      }
    }
    if (lagging && !fused && p->device)
      for (int32_t i = 0; i < n_segs; ++i) {
        akv_status st = materialize_seq(p, p->seqs[segs[i].seq]);
        if (st != AKV_OK) return st;
      }
    std::vector<akv_segment> rows((size_t)n_segs);
    std::vector<akv_extent>& lists = p->hb.lists;
    std::vector<akv_extent>& masked = p->hb.masked;
    std::vector<int32_t>& lags = p->hb.lags;
    std::vector<int32_t>& mlag = p->hb.mlag;
    lists.clear();
    lags.clear();
    for (int32_t i = 0; i < n_segs; ++i) {
      const akv_seq_segment& sg = segs[i];
      SeqRec* q = &p->seqs[sg.seq];
      const akv_span* m = masks ? masks + sg.mask_begin : nullptr;
      const std::vector<int32_t>& vis = visible(*q);
      std::vector<uint8_t> hide;
      const bool from_image = sg.mask_len > 0 && !fused && q->vis_logical;
      if (sg.mask_len > 0 && !from_image) {
        hide.assign(q->slot.size(), 0);
        for (int32_t k = 0; k < sg.mask_len; ++k) std::fill(hide.begin() + m[k].begin, hide.begin() + m[k].end, 1);
      }
      const std::vector<akv_extent>* ex;
      if (fused && sg.mask_len > 0) {
        build_extents_lag(p, *q, vis, &hide, masked, mlag);
        lags.insert(lags.end(), mlag.begin(), mlag.end());
        ex = &masked;
      } else if (fused) {
        if (!q->lg_ok) {
          build_extents_lag(p, *q, vis, nullptr, q->ext_lg, q->ext_lg_lag);
          q->lg_ok = true;
        }
        lags.insert(lags.end(), q->ext_lg_lag.begin(), q->ext_lg_lag.end());
        ex = &q->ext_lg;
      } else if (from_image) {
        if (!q->ext_ok) {
          build_extents(p, *q, vis, nullptr, q->ext);
          q->ext_ok = true;
        }
        masked_from_image(*q, m, sg.mask_len, masked);
        ex = &masked;
      } else if (sg.mask_len > 0) {
        build_extents(p, *q, vis, &hide, masked);
        ex = &masked;
      } else {
        if (!q->ext_ok) {
          build_extents(p, *q, vis, nullptr, q->ext);
          q->ext_ok = true;
        }
        ex = &q->ext;
      }
      if (lists.size() + ex->size() > (size_t)kInt32Max) return fail(AKV_ERANGE, "page lists too long");
      rows[i] = {sg.q_begin, sg.q_len, (int32_t)lists.size(), (int32_t)ex->size()};
      lists.insert(lists.end(), ex->begin(), ex->end());
    }
    if (dbg().checks)
      for (const akv_extent& x : lists)
        if (x.page < 0 || x.page >= p->L.num_pages || p->pages[x.page].owner < 0)
          return check_fail("a visible list reads page %d, which is not in use", x.page);
    return attention_impl(p, Q, n_q_tokens, rows.data(), n_segs, lists.data(), (int32_t)lists.size(),
                          fused ? lags.data() : nullptr, scale, out);
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

// Launches whose every segment packs at most 16 rows per kv head (decode)
// run the decode kernel on 16-row items; the others the prefill kernels.
static bool decode_launch(const akv_pool* p, const int64_t* q_len, int32_t n, int32_t stride) {
  const akv_layout& L = p->L;
  const int G = L.n_q_heads / L.n_kv_heads;
  int64_t max_rows = 0;
  for (int32_t i = 0; i < n; ++i) max_rows = std::max<int64_t>(max_rows, q_len[(size_t)i * stride] * G);
  return L.d_nope == 0 && L.d_rope == 128 && L.d_v == 128 &&
         max_rows <= akv::DECODE_ROWS;
}

// Checks the segments and page lists of an attention launch; fills each
// segment's list length and offset in the expanded slot list.  *any_rows is
// false when no segment has a query row.
static akv_status attn_validate(akv_pool* p, int32_t n_q_tokens, const akv_segment* segs, int32_t n_segs,
                                const akv_extent* page_lists, int32_t n_ext, std::vector<int64_t>& lkv,
                                std::vector<int64_t>& list_off, int64_t* total_out, bool* any_rows) {
  const akv_layout& L = p->L;
  if (!akv::attn_dims_supported(L.d_nope, L.d_rope, L.d_v))
    return fail(AKV_EINVAL, "no attention kernel for d_nope=%d d_rope=%d d_v=%d", L.d_nope,
                L.d_rope, L.d_v);
  if (n_segs < 0 || n_ext < 0 || n_q_tokens < 0) return fail(AKV_EINVAL, "negative count");
  if ((n_segs > 0 && !segs) || (n_ext > 0 && !page_lists))
    return fail(AKV_EINVAL, "segments / page lists are NULL");
  lkv.assign(n_segs, 0);
  list_off.assign(n_segs, 0);
  int64_t total = 0;
  std::vector<std::pair<int32_t, int32_t>> rows;
  for (int32_t i = 0; i < n_segs; ++i) {
    const akv_segment& sg = segs[i];
    if (sg.q_len < 0 || sg.ext_len < 0) return fail(AKV_EINVAL, "segment %d: negative length", i);
    if (sg.q_begin < 0 || (int64_t)sg.q_begin + sg.q_len > n_q_tokens)
      return fail(AKV_ERANGE, "segment %d: query rows outside 0..%d", i, n_q_tokens);
    if (sg.ext_begin < 0 || (int64_t)sg.ext_begin + sg.ext_len > n_ext)
      return fail(AKV_ERANGE, "segment %d: extents outside 0..%d", i, n_ext);
    int64_t n_keys = 0;
    for (int32_t e = sg.ext_begin; e < sg.ext_begin + sg.ext_len; ++e) {
      const akv_extent& x = page_lists[e];
      if (x.page < 0 || x.page >= L.num_pages || x.lo < 0 || x.lo >= x.hi || x.hi > L.page_size)
        return fail(AKV_ERANGE, "extent %d (%d, %d, %d) outside the pool", e, x.page, x.lo, x.hi);
      n_keys += x.hi - x.lo;
    }
    if (sg.q_len > 0 && n_keys < sg.q_len)
      return fail(AKV_EINVAL, "segment %d has %lld list entries for %d queries", i,
                  (long long)n_keys, sg.q_len);
    if (n_keys > kInt32Max) return fail(AKV_ERANGE, "segment %d list too long", i);
    lkv[i] = n_keys;
    list_off[i] = total;
    total += n_keys;
    if (sg.q_len > 0) rows.emplace_back(sg.q_begin, sg.q_begin + sg.q_len);
  }
  std::sort(rows.begin(), rows.end());
  for (size_t i = 1; i < rows.size(); ++i)
    if (rows[i].first < rows[i - 1].second) return fail(AKV_EINVAL, "segments overlap in Q rows");
  if (total > kInt32Max) return fail(AKV_ERANGE, "page lists too long");
  *total_out = total;
  *any_rows = !rows.empty();
  return AKV_OK;
}

// AKV_CHECKS: the plan's items lie inside their segment's rows and list, and
// the key splits of every row tile cover its list exactly once; combine items
// and partial rows stay inside the partial buffer.
static akv_status check_plan(const akv_pool* p, const AttnPlan& plan, const akv_segment* segs, int32_t n_segs,
                             const std::vector<int64_t>& lkv, int RB) {
  const akv_layout& L = p->L;
  const int64_t G = L.n_q_heads / L.n_kv_heads;
  struct Key {
    int32_t seg, kvh, row0, kb, ke;
  };
  std::vector<Key> keys;
  keys.reserve(plan.items.size());
  for (const akv::AttnItem& it : plan.items) {
    if (it.seg < 0) continue;
    if (it.seg >= n_segs || segs[it.seg].q_len <= 0) return check_fail("attention item of segment %d", it.seg);
    const int64_t rows = segs[it.seg].q_len * G;
    if (it.kvh < 0 || it.kvh >= L.n_kv_heads) return check_fail("attention item of kv head %d", it.kvh);
    if (it.row0 < 0 || it.row0 >= rows || it.row0 % RB)
      return check_fail("attention item rows from %d in a segment of %lld rows", it.row0, (long long)rows);
    if (it.k_begin < 0 || it.k_begin >= it.k_end || it.k_end > lkv[it.seg])
      return check_fail("attention item keys %d..%d of a list of %lld", it.k_begin, it.k_end,
                        (long long)lkv[it.seg]);
    const int64_t nr = std::min<int64_t>(RB, rows - it.row0);
    if (it.part >= 0 && it.part + nr > plan.part_rows)
      return check_fail("attention item partial rows %d..%lld of %lld", it.part, (long long)(it.part + nr),
                        (long long)plan.part_rows);
    keys.push_back({it.seg, it.kvh, it.row0, it.k_begin, it.k_end});
  }
  std::sort(keys.begin(), keys.end(), [](const Key& a, const Key& b) {
    if (a.seg != b.seg) return a.seg < b.seg;
    if (a.kvh != b.kvh) return a.kvh < b.kvh;
    if (a.row0 != b.row0) return a.row0 < b.row0;
    return a.kb < b.kb;
  });
  int64_t tiles = 0, want = 0;
  for (int32_t i = 0; i < n_segs; ++i)
    if (segs[i].q_len > 0) want += (int64_t)L.n_kv_heads * ((segs[i].q_len * G + RB - 1) / RB);
  for (size_t i = 0; i < keys.size();) {
    size_t j = i;
    int32_t at = 0;
    for (; j < keys.size() && keys[j].seg == keys[i].seg && keys[j].kvh == keys[i].kvh &&
           keys[j].row0 == keys[i].row0;
         ++j) {
      if (keys[j].kb != at) break;
      at = keys[j].ke;
    }
    const bool same = j < keys.size() && keys[j].seg == keys[i].seg && keys[j].kvh == keys[i].kvh &&
                      keys[j].row0 == keys[i].row0;
    if (same || at != lkv[keys[i].seg])
      return check_fail("row tile (segment %d, kv head %d, row %d): key splits do not cover its list once",
                        keys[i].seg, keys[i].kvh, keys[i].row0);
    ++tiles;
    i = j;
  }
  if (tiles != want) return check_fail("%lld row tiles planned, %lld expected", (long long)tiles, (long long)want);
  for (const akv::CombItem& c : plan.comb)
    if (c.seg < 0 || c.seg >= n_segs || c.nsplit < 2 || c.nsplit > 64 || c.rows < 1 || c.rows > RB ||
        c.part0 < 0 || c.part0 + (int64_t)c.nsplit * c.rows > plan.part_rows)
      return check_fail("combine item (segment %d, %d splits of %d rows from %d) outside %lld partial rows", c.seg,
                        c.nsplit, c.rows, c.part0, (long long)plan.part_rows);
  return AKV_OK;
}

// Segment-batch attention over caller lists; ext_lag (optional, one per
// extent) is the rotation each extent's keys still owe, applied inside the
// kernel that reads them (the decode kernel and the 128-dim GQA prefill
// kernel take it).  ws_static: tables and partials in the static workspace.
static akv_status attention_impl(akv_pool* p, const void* Q, int32_t n_q_tokens, const akv_segment* segs,
                                 int32_t n_segs, const akv_extent* page_lists, int32_t n_ext,
                                 const int32_t* ext_lag, float scale, void* out, bool ws_static) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    if (!p->device) return fail(AKV_ESTATE, "attention needs a device pool");
    const akv_layout& L = p->L;
    if (!(scale >= 0.f) || !std::isfinite(scale)) return fail(AKV_EINVAL, "bad scale");
    std::vector<int64_t> lkv, list_off;
    int64_t total = 0;
    bool any_rows = false;
    akv_status vst = attn_validate(p, n_q_tokens, segs, n_segs, page_lists, n_ext, lkv, list_off, &total,
                                   &any_rows);
    if (vst != AKV_OK) return vst;
    if (!any_rows) return AKV_OK;
    if (!Q || !out) return fail(AKV_EINVAL, "Q and out are required");
    if (p->bg_pending) {   // lists reading pages a background copy touches wait for it
      bool touch = false;
      for (int32_t e = 0; e < n_ext && !touch; ++e) touch = p->page_bg[page_lists[e].page] != 0;
      if (touch) {
        akv_status bst = bg_wait(p);
        if (bst != AKV_OK) return bst;
      }
    }

    std::vector<int64_t> qlens(n_segs);
    for (int32_t i = 0; i < n_segs; ++i) qlens[i] = segs[i].q_len;
    const bool decode = decode_launch(p, qlens.data(), n_segs, 1);
    // distinct owed rotations of the lists (fused into the decode kernel)
    std::vector<int32_t> rot_deltas;
    std::vector<int32_t>& ex_didx = p->hb.ex_didx;
    ex_didx.clear();
    std::unordered_map<int32_t, int32_t> di;   // owed rotation -> its table row
    if (ext_lag) {
      for (int32_t i = 0; i < n_segs; ++i)
        for (int32_t e = segs[i].ext_begin; e < segs[i].ext_begin + segs[i].ext_len; ++e)
          if (ext_lag[e] && !di.count(ext_lag[e])) {
            di.emplace(ext_lag[e], (int32_t)rot_deltas.size());
            rot_deltas.push_back(ext_lag[e]);
          }
      if (!rot_deltas.empty() && !decode && !rotating_prefill(p))
        return fail(AKV_EINVAL, "owed rotations are applied only by the decode and 128-dim GQA prefill kernels");
    }
    const int rb = decode ? akv::DECODE_ROWS : akv::attn_rows_per_block(L.d_nope);
    AttnPlan& plan = p->hb.plan;
    plan_attention(p, segs, n_segs, lkv, list_off, rb, p->n_cu, plan);
    if (plan.part_rows > kInt32Max) return fail(AKV_ERANGE, "too many split-KV partial rows");
    if (dbg().checks) {
      akv_status cst = check_plan(p, plan, segs, n_segs, lkv, rb);
      if (cst != AKV_OK) return cst;
    }
    // extent offsets for the slot expansion (over all segments' ranges, in order)
    const bool fused = !rot_deltas.empty();
    // The segments' ranges usually tile the page lists in order: then the
    // lists are uploaded as they are (akv_extent and akv::Extent share
    // their layout); otherwise the ranges are gathered.
    bool in_order = true;
    int64_t covered = 0;
    for (int32_t i = 0; i < n_segs && in_order; ++i) {
      in_order = segs[i].ext_begin == covered;
      covered += segs[i].ext_len;
    }
    in_order = in_order && covered == n_ext;
    static_assert(sizeof(akv::Extent) == sizeof(akv_extent), "extent layouts");
    std::vector<akv::Extent>& ex_used = p->hb.ex_used;
    std::vector<int32_t>& ex_off = p->hb.ex_off;
    ex_used.clear();
    ex_off.clear();
    for (int32_t i = 0; i < n_segs; ++i) {
      int64_t o = list_off[i];
      for (int32_t e = segs[i].ext_begin; e < segs[i].ext_begin + segs[i].ext_len; ++e) {
        const akv_extent& x = page_lists[e];
        if (!in_order) ex_used.push_back({x.page, x.lo, x.hi});
        ex_off.push_back((int32_t)o);
        if (fused) {
          ex_didx.push_back(ext_lag[e] ? di.find(ext_lag[e])->second : -1);
        }
        o += x.hi - x.lo;
      }
    }
    const size_t keys4 = (size_t)std::max<int64_t>(total, 1) * 4;
    // attention mass per page (decode launches): chunks of each segment's list
    const bool want_mass = decode && p->mass && !ws_static;
    std::vector<akv::MassItem>& mass_items = p->hb.mass_items;
    mass_items.clear();
    if (want_mass)
      for (int32_t i = 0; i < n_segs; ++i)
        if (segs[i].q_len > 0)
          for (int64_t k0 = 0; k0 < lkv[i]; k0 += akv::MASS_CHUNK) mass_items.push_back({i, (int32_t)k0});
    const size_t lse_bytes = want_mass ? (size_t)n_q_tokens * L.n_q_heads * 4 : 0;
    if (dbg().trace) {
      int64_t pad = 0;
      for (const akv::AttnItem& it : plan.items) pad += it.seg < 0;
      int max_split = 1;
      for (int32_t ns : plan.nsplit) max_split = std::max(max_split, (int)ns);
      trace("attention: %d segments, %lld keys, %s kernel, %zu items (%lld padding), up to %d key splits, "
            "%zu combine items, %lld partial rows, %zu owed rotations applied in the kernel, %zu mass items",
            n_segs, (long long)total, decode ? "decode" : (L.d_nope > 0 ? "MLA prefill" : "prefill"),
            plan.items.size(), (long long)pad, max_split, plan.comb.size(), (long long)plan.part_rows,
            rot_deltas.size(), mass_items.size());
    }
    const size_t need = plan.segs.size() * sizeof(akv::AttnSeg) + plan.items.size() * sizeof(akv::AttnItem) +
                        plan.comb.size() * sizeof(akv::CombItem) + ex_off.size() * sizeof(akv::Extent) +
                        (ex_off.size() + ex_didx.size()) * 4 + keys4 * (fused ? 2 : 1) +
                        rot_deltas.size() * (size_t)L.d_rope * 4 + (size_t)plan.part_rows * (L.d_v + 2) * 4 +
                        mass_items.size() * sizeof(akv::MassItem) + lse_bytes + 14 * 256;
    static const std::vector<float> no_rows;
    const std::vector<float>& rot_rows = fused ? rot_table_rows(p, rot_deltas.data(), rot_deltas.size()) : no_rows;
    const std::pair<const void*, size_t> up_parts[7] = {
        {plan.segs.data(), plan.segs.size() * sizeof(akv::AttnSeg)},
        {plan.items.data(), plan.items.size() * sizeof(akv::AttnItem)},
        {plan.comb.data(), plan.comb.size() * sizeof(akv::CombItem)},
        {in_order ? (const void*)page_lists : (const void*)ex_used.data(), ex_off.size() * sizeof(akv::Extent)},
        {ex_off.data(), ex_off.size() * 4},
        {ex_didx.data(), ex_didx.size() * 4},
        {rot_rows.data(), rot_rows.size() * 4}};
    void* dv[7];
    int32_t* dslots = nullptr;
    int32_t* dkey_didx = nullptr;
    float* part_o = nullptr;
    float* part_ml = nullptr;
    float* dlse = nullptr;
    void* dmass_items = nullptr;
    if (ws_static) {
      // The call's tables, slot list and partials in the library's static
      // device workspace: one copy of the tables on the pool stream (after
      // the kernels of earlier calls, which may still read the workspace),
      // no allocation of any kind.
      char* base = nullptr;
      hipError_t we = akv::static_workspace((void**)&base);
      if (we != hipSuccess) return hip_fail(we, "static workspace address (hipGetSymbolAddress)");
      size_t up = 0;
      for (const auto& pr : up_parts) up += align_up(std::max<size_t>(pr.second, 1), 256);
      const size_t slots_at = up, didx_at = slots_at + align_up(keys4, 256);
      const size_t po_at = didx_at + (fused ? align_up(keys4, 256) : 0);
      const size_t pml_at = po_at + align_up((size_t)plan.part_rows * L.d_v * 4, 256);
      const size_t end = pml_at + align_up((size_t)plan.part_rows * 2 * 4, 256);
      if (end > akv::STATIC_WORKSPACE_BYTES)
        return fail(AKV_ENOMEM, "this call needs %zu bytes of workspace; the static workspace holds %zu",
                    end, akv::STATIC_WORKSPACE_BYTES);
      std::vector<char>& hst = p->hb.static_up;
      hst.assign(up, 0);
      size_t off = 0;
      int i = 0;
      for (const auto& pr : up_parts) {
        if (pr.second) std::memcpy(hst.data() + off, pr.first, pr.second);
        dv[i++] = base + off;
        off += align_up(std::max<size_t>(pr.second, 1), 256);
      }
      // pageable source: the runtime has read it when the call returns
      we = hipMemcpyAsync(base, hst.data(), up, hipMemcpyHostToDevice, p->stream);
      if (we != hipSuccess) return hip_fail(we, "hipMemcpyAsync(static workspace)");
      dslots = (int32_t*)(base + slots_at);
      if (fused) dkey_didx = (int32_t*)(base + didx_at);
      if (plan.part_rows > 0) {
        part_o = (float*)(base + po_at);
        part_ml = (float*)(base + pml_at);
      }
    } else {
      ScratchCursor sc(p, need);
      void* dv8[8];
      akv_status st = upload_arrays(p, sc, {up_parts[0], up_parts[1], up_parts[2], up_parts[3], up_parts[4],
                                            up_parts[5], up_parts[6],
                                            {mass_items.data(), mass_items.size() * sizeof(akv::MassItem)}}, dv8);
      if (st != AKV_OK) return st;
      for (int i = 0; i < 7; ++i) dv[i] = dv8[i];
      dmass_items = dv8[7];
      dslots = (int32_t*)sc.take((size_t)std::max<int64_t>(total, 1) * 4);
      dkey_didx = fused ? (int32_t*)sc.take((size_t)std::max<int64_t>(total, 1) * 4) : nullptr;
      if (plan.part_rows > 0) {
        part_o = (float*)sc.take((size_t)plan.part_rows * L.d_v * 4);
        part_ml = (float*)sc.take((size_t)plan.part_rows * 2 * 4);
      }
      if (want_mass) dlse = (float*)sc.take(lse_bytes);
      if (!sc.ok()) return fail(AKV_ENOMEM, "scratch too small for this call (%zu bytes per call)",
                                   p->scratch_bytes - p->scratch_base);
    }
    void *dsegs = dv[0], *ditems = dv[1], *dcomb = plan.comb.empty() ? nullptr : dv[2], *dex = dv[3],
         *doff = dv[4];
    const float* drot = fused ? (const float*)dv[6] : nullptr;

    hipError_t e;
    {
      KTimer tm(p, AKV_K_EXPAND);
      e = akv::launch_expand(p->stream, (const akv::Extent*)dex, (const int32_t*)doff,
                             (int)ex_off.size(), L.page_size, dslots);
      tm.done();
    }
    if (akv_status lst = check_launch(e, "expand kernel launch")) return lst;
    if (fused) {
      KTimer tm(p, AKV_K_EXPAND);
      e = akv::launch_expand_didx(p->stream, (const akv::Extent*)dex, (const int32_t*)doff,
                                    (const int32_t*)dv[5], (int)ex_off.size(), dkey_didx);
      tm.done();
      if (akv_status lst = check_launch(e, "owed-rotation table launch")) return lst;
    }
    akv::AttnArgs a{};
    a.q = (const uint16_t*)Q;
    a.n_q_heads = L.n_q_heads;
    a.group = L.n_q_heads / L.n_kv_heads;
    a.k_a = p->k;
    a.k_b = p->kpe;
    a.kpe_heads = p->rope_heads();
    a.v = p->v;
    a.n_kv_heads = L.n_kv_heads;
    a.page_size = L.page_size;
    a.log2_page = p->log2S;
    a.segs = (const akv::AttnSeg*)dsegs;
    a.items = (const akv::AttnItem*)ditems;
    a.n_items = (int)plan.items.size();
    a.slots = dslots;
    const float sc_ = scale > 0.f ? scale : 1.f / std::sqrt((float)(L.d_nope + L.d_rope));
    a.scale_log2e = sc_ * 1.4426950408889634f;
    a.out = (uint16_t*)out;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.rows_per_block = rb;
    a.key_didx = dkey_didx;
    a.rot_table = drot;
    a.rot_pairing = L.pairing;
    a.lse = dlse;
    {
      KTimer tm(p, AKV_K_ATTN);
      e = decode ? akv::launch_decode_attn(p->stream, a) : akv::launch_seg_attn(p->stream, a, L.d_nope, L.d_rope, L.d_v);
      tm.done();
    }
    if (akv_status lst = check_launch(e, "attention kernel launch")) return lst;
    if (!plan.comb.empty()) {
      KTimer tm(p, AKV_K_COMBINE);
      e = akv::launch_combine(p->stream, a, (const akv::CombItem*)dcomb, (int)plan.comb.size(), L.d_v);
      tm.done();
      if (akv_status lst = check_launch(e, "combine kernel launch")) return lst;
    }
    if (want_mass && !mass_items.empty()) {
      KTimer tm(p, AKV_K_MASS);
      int64_t max_rows = 0;
      for (int32_t i = 0; i < n_segs; ++i)
        max_rows = std::max<int64_t>(max_rows, (int64_t)segs[i].q_len * (L.n_q_heads / L.n_kv_heads));
      e = akv::launch_page_mass(p->stream, a, (const akv::MassItem*)dmass_items, (int)mass_items.size(),
                                (int)max_rows, p->mass);
      tm.done();
      if (akv_status lst = check_launch(e, "attention mass kernel launch")) return lst;
    }
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_attention_mass(akv_pool* p, float* mass, int32_t n_pages) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  if (!p->device) return fail(AKV_ESTATE, "attention mass needs a device pool");
  if (mass && n_pages != p->L.num_pages)
    return fail(AKV_EINVAL, "mass holds %d pages, the pool %d", n_pages, p->L.num_pages);
  p->mass = mass;
  return AKV_OK;
}

akv_status akv_segment_attention(akv_pool* p, const void* Q, int32_t n_q_tokens, const akv_segment* segs,
                                 int32_t n_segs, const akv_extent* page_lists, int32_t n_ext, float scale,
                                 void* out) {
  return attention_impl(p, Q, n_q_tokens, segs, n_segs, page_lists, n_ext, nullptr, scale, out);
}

akv_status akv_segment_attention_static(akv_pool* p, const void* Q, int32_t n_q_tokens, const akv_segment* segs,
                                        int32_t n_segs, const akv_extent* page_lists, int32_t n_ext, float scale,
                                        void* out) {
  return attention_impl(p, Q, n_q_tokens, segs, n_segs, page_lists, n_ext, nullptr, scale, out, true);
}

akv_status akv_attention_plan(akv_pool* p, int32_t n_q_tokens, const akv_segment* segs, int32_t n_segs,
                              const akv_extent* page_lists, int32_t n_ext, int32_t n_cu, akv_attn_item* items,
                              int32_t items_cap, int32_t* n_items, akv_attn_combine* comb, int32_t comb_cap,
                              int32_t* n_comb, int32_t* rows_per_block, int64_t* part_rows) {
  try {
    if (!p) return fail(AKV_EINVAL, "NULL pool");
    if (!n_items || !n_comb || !rows_per_block || !part_rows) return fail(AKV_EINVAL, "NULL output count");
    if (n_cu < 0 || items_cap < 0 || comb_cap < 0) return fail(AKV_EINVAL, "negative count");
    std::vector<int64_t> lkv, list_off;
    int64_t total = 0;
    bool any_rows = false;
    akv_status st = attn_validate(p, n_q_tokens, segs, n_segs, page_lists, n_ext, lkv, list_off, &total,
                                  &any_rows);
    if (st != AKV_OK) return st;
    *n_items = 0;
    *n_comb = 0;
    *part_rows = 0;
    std::vector<int64_t> qlens(n_segs);
    for (int32_t i = 0; i < n_segs; ++i) qlens[i] = segs[i].q_len;
    const bool decode = decode_launch(p, qlens.data(), n_segs, 1);
    const int rb = decode ? akv::DECODE_ROWS : akv::attn_rows_per_block(p->L.d_nope);
    *rows_per_block = rb;
    if (!any_rows) return AKV_OK;
    AttnPlan plan;
    plan_attention(p, segs, n_segs, lkv, list_off, rb, n_cu > 0 ? n_cu : p->n_cu, plan);
    if (dbg().checks) {
      akv_status cst = check_plan(p, plan, segs, n_segs, lkv, rb);
      if (cst != AKV_OK) return cst;
    }
    *n_items = (int32_t)plan.items.size();
    *n_comb = (int32_t)plan.comb.size();
    *part_rows = plan.part_rows;
    static_assert(sizeof(akv_attn_item) == sizeof(akv::AttnItem), "item layouts");
    static_assert(sizeof(akv_attn_combine) == sizeof(akv::CombItem), "combine layouts");
    if ((items && items_cap < *n_items) || (comb && comb_cap < *n_comb))
      return fail(AKV_ERANGE, "plan needs %d items and %d combine entries", *n_items, *n_comb);
    if (items && !plan.items.empty())
      std::memcpy(items, plan.items.data(), plan.items.size() * sizeof(akv::AttnItem));
    if (comb && !plan.comb.empty())
      std::memcpy(comb, plan.comb.data(), plan.comb.size() * sizeof(akv::CombItem));
    return AKV_OK;
  } catch (const std::bad_alloc&) {
    return fail(AKV_ENOMEM, "host allocation failed");
  }
}

akv_status akv_seq_tokens(akv_pool* p, int32_t s, int32_t first, int32_t n, int32_t* slot,
                          int32_t* pos, uint8_t* dropped) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  SeqRec* q;
  akv_status st = get_seq(p, s, &q);
  if (st != AKV_OK) return st;
  if (first < 0 || n < 0 || (int64_t)first + n > (int64_t)q->slot.size())
    return fail(AKV_ERANGE, "tokens %d..%d outside 0..%zu", first, first + n, q->slot.size());
  for (int32_t i = 0; i < n; ++i) {
    if (slot) slot[i] = q->slot[first + i];
    if (pos) pos[i] = q->pos[first + i];
    if (dropped) dropped[i] = q->dropped[first + i];
  }
  return AKV_OK;
}

akv_status akv_seq_info(akv_pool* p, int32_t s, int32_t* n_tokens, int32_t* n_visible,
                        double* frag) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  SeqRec* q;
  akv_status st = get_seq(p, s, &q);
  if (st != AKV_OK) return st;
  if (n_tokens) *n_tokens = (int32_t)q->slot.size();
  if (n_visible) *n_visible = (int32_t)q->n_vis;
  if (frag) *frag = fragmentation(p, *q);
  return AKV_OK;
}

akv_status akv_pool_queues(akv_pool* p, int32_t* free_out, int32_t free_cap, int32_t* n_free,
                           int32_t* evict_out, int32_t evict_cap, int32_t* n_evict) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  int32_t k = 0;
  for (int32_t pg : p->free_q) {
    if (free_out && k < free_cap) free_out[k] = pg;
    ++k;
  }
  if (n_free) *n_free = k;
  k = 0;
  for (auto& e : p->evict_q) {
    const PageRec& r = p->pages[e.first];
    if (!(r.in_evict && r.evict_gen == e.second)) continue;
    if (evict_out && k < evict_cap) evict_out[k] = e.first;
    ++k;
  }
  if (n_evict) *n_evict = k;
  return AKV_OK;
}

akv_status akv_timing_enable(akv_pool* p, int32_t enable) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  p->timing = enable != 0;
  return AKV_OK;
}

akv_status akv_timing_read(akv_pool* p, int32_t kind, double* total_ms, int32_t* count) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  if (kind < 0 || kind >= AKV_K_KINDS) return fail(AKV_EINVAL, "bad kernel kind %d", kind);
  akv_status st = timing_collect(p);
  if (st != AKV_OK) return st;
  if (total_ms) *total_ms = p->t_ms[kind];
  if (count) *count = p->t_cnt[kind];
  p->t_ms[kind] = 0;
  p->t_cnt[kind] = 0;
  p->t_each[kind].clear();
  return AKV_OK;
}

akv_status akv_timing_samples(akv_pool* p, int32_t kind, float* ms, int32_t cap, int32_t* n_out) {
  if (!p || !n_out) return fail(AKV_EINVAL, "NULL argument");
  if (kind < 0 || kind >= AKV_K_KINDS) return fail(AKV_EINVAL, "bad kernel kind %d", kind);
  akv_status st = timing_collect(p);
  if (st != AKV_OK) return st;
  const std::vector<float>& v = p->t_each[kind];
  *n_out = (int32_t)v.size();
  if ((int32_t)v.size() > cap) return fail(AKV_ERANGE, "%zu samples, cap %d", v.size(), cap);
  if (!v.empty()) {
    if (!ms) return fail(AKV_EINVAL, "ms is NULL");
    std::memcpy(ms, v.data(), v.size() * sizeof(float));
  }
  return AKV_OK;
}

akv_status akv_sync(akv_pool* p) {
  if (!p) return fail(AKV_EINVAL, "NULL pool");
  if (!p->device) return AKV_OK;
  hipError_t e = hipStreamSynchronize(p->stream);
  if (e == hipSuccess && p->kstream) e = hipStreamSynchronize(p->kstream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return AKV_OK;
}

}  // extern "C"
