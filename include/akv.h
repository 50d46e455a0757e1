/*
 * akv.h -- C ABI of the AKV cache-engineering hot path for AMD MI355X (gfx950).
 *
 * Operations on a paged bf16 KV pool: append, drop, repos (RoPE delta
 * rotation of retained keys), splice, compaction, and segment-batch
 * attention.  Sources, cited by page title and section:
 *
 *   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and
 *               State-Preserving Prefix Invalidation Bypass" (A. Akhunji)
 *   [AKV-notes] "Cache Engineering for Agents" (reading notes on Fu et al.,
 *               arXiv:2610.28577)
 *   [Leyline]   "Leyline: KV Cache Directives for Agentic Inference"
 *               (paper digest)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Device memory (page arrays, Q, K, V, outputs, scratch) belongs to the
 *   caller.  The library never allocates or frees device memory; it keeps raw
 *   pointers.  It owns all host metadata and a pinned host staging ring.
 * - Host arrays passed in (spans, positions, segments, extents) are copied
 *   before the call returns.  Device inputs (K, V, Q) must stay valid until the
 *   work is done (akv_sync or a sync of the pool's stream).
 * - Kernels are enqueued on the pool's HIP stream; calls return once they
 *   are enqueued, with the host metadata already updated.  A device pool also
 *   owns two streams of its own (default priority): one for metadata copies
 *   into scratch while the pool's stream is busy (the pool's stream waits for
 *   each such copy), and one for the background compaction copies of
 *   akv_compact_pending, which run beside later work on the pool's stream.
 *   The pool's stream waits for those copies before any later library launch
 *   that reads or writes a page they touch; akv_sync waits for every stream of
 *   the pool (a caller's own kernels that read the page arrays order
 *   themselves after akv_sync or after such a launch).
 * - Calls on one pool are not re-entrant; separate pools are independent.
 * - Every call validates all arguments before changing any state: a call that
 *   fails leaves the pool as it was.  akv_last_error() gives the reason.  The
 *   exception is AKV_EHIP: a HIP call that fails is seen after the host
 *   metadata has changed, and the rows the call was to write are then
 *   undefined (release the pool).
 * - Debug switches, read from the environment once per process:
 *   AKV_CHECKS=1 checks every device work list on the host before its launch
 *   (slots and pages inside the pool and in use, rows inside their page,
 *   rotate items disjoint, copy destinations distinct and apart from the
 *   sources, attention items covering each row tile's keys once); a failed
 *   check is a library bug, returned as AKV_ESTATE with "AKV_CHECKS" in the
 *   error text.  AKV_TRACE=1 prints one line per planning decision to stderr.
 *   AKV_COMPACT_THRESHOLD=x (0 < x <= 1) replaces the 0.40 default
 *   threshold.  AKV_FAULT_INJECT=launch makes every kernel launch report
 *   failure once enqueued (AKV_EHIP), for tests of error handling.
 * - Spans are half-open [begin, end) over a sequence's logical token indices,
 *   which never change: the n-th token appended to a sequence has index n.
 * - Page slots are numbered page * page_size + offset.
 *
 * Pool memory layout (all bf16, caller-allocated, row-major):
 *   GQA  (d_nope == 0): k_pages [num_pages][n_kv_heads][page_size][d_rope]
 *                       v_pages [num_pages][n_kv_heads][page_size][d_v]
 *                       kpe_pages must be NULL.
 *   MLA  (d_nope  > 0): k_pages   = K_nope [num_pages][n_kv_heads][page_size][d_nope]
 *                       kpe_pages = K_pe   [num_pages][H_pe][page_size][d_rope]
 *                       with H_pe = 1 (shared by all heads) or n_kv_heads
 *                       (kpe_per_head = 1);
 *                       v_pages   [num_pages][n_kv_heads][page_size][d_v].
 *
 * Page allocation rule: a FIFO free queue initialised to page_order (or
 * 0..num_pages-1), then a FIFO evictable queue of pages without any visible
 * token (dropped cache is evicted first, [AKV-notes] section 3, Cache
 * Management).  A sequence fills its open tail page before taking a new one.
 * A page joins the evictable queue when its last visible token is dropped or
 * moved away by compaction, unless it is the sequence's open tail page.
 */
#ifndef AKV_H
#define AKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct akv_pool akv_pool;

typedef enum {
  AKV_OK = 0,
  AKV_EINVAL = -1, /* malformed argument (NULL, bad shape, end < begin, ...) */
  AKV_ERANGE = -2, /* index, span, page or position out of range            */
  AKV_ENOMEM = -3, /* pool pages or scratch bytes exhausted                  */
  AKV_ESTATE = -4, /* released sequence, or a device op on a page-table-only pool */
  AKV_EHIP = -5    /* a HIP runtime call failed                              */
} akv_status;

typedef struct { int32_t begin, end; } akv_span;          /* [begin, end)             */
typedef struct { int32_t page, lo, hi; } akv_extent;      /* slots lo..hi-1 of a page */
typedef struct { int32_t q_begin, q_len, ext_begin, ext_len; } akv_segment;
typedef struct { int32_t seq, q_begin, q_len, mask_begin, mask_len; } akv_seq_segment;

typedef struct {
  int32_t n_q_heads;     /* multiple of n_kv_heads; q head h reads kv head h / (n_q_heads/n_kv_heads) */
  int32_t n_kv_heads;
  int32_t d_nope;        /* 0 for GQA; MLA position-free key dims per head          */
  int32_t d_rope;        /* rotated key dims: all of K (GQA) or K_pe (MLA); even   */
  int32_t d_v;
  int32_t page_size;     /* power of two, 1..256                                    */
  int32_t num_pages;
  int32_t kpe_per_head;  /* MLA: 0 = one K_pe row per token shared by all heads     */
  int32_t pairing;       /* 0 = interleaved pairs (2i, 2i+1); 1 = half-split (i, i + d_rope/2) */
  double rope_theta;     /* theta_i = rope_theta^(-2i/d_rope) unless inv_freq is given */
  const double* inv_freq;/* optional d_rope/2 angular frequencies (copied)          */
  double compact_threshold; /* automatic compaction above this fragmentation;
                               <= 0 selects 0.40 (or AKV_COMPACT_THRESHOLD),
                               >= 1 disables it                                  */
} akv_layout;

/* ---- pool ---------------------------------------------------------------- */

/* Create a pool over caller-owned device page arrays (layout above).
 * page_order: optional permutation of 0..num_pages-1 (initial free queue).
 * scratch / scratch_bytes: caller-owned device memory for work lists, slot maps
 * and split-KV partials; attention needs about
 *   64 KiB + 16 B * n_ext + 4 B * total list length + 16 B * work items
 *   + split partials (4 B * n_split * rows * (d_v + 2)).
 * hip_stream: the stream all device work goes to (NULL = the null stream).
 * A pool with k_pages == v_pages == kpe_pages == NULL and scratch == NULL is
 * page-table-only: it tracks slots, positions, visibility and allocation
 * exactly like a device pool but holds no KV values, so attention on it
 * returns AKV_ESTATE.
 * Limits: num_pages < 2^24 and num_pages * n_kv_heads * page_size < 2^32
 * (row indices in the kernels), num_pages * page_size < 2^31 (slots).
 * Errors: AKV_EINVAL (bad layout or a limit exceeded, page_order not a
 * permutation), AKV_EHIP (device query or pinned allocation failed). */
akv_status akv_pool_create(const akv_layout* layout, const int32_t* page_order,
                           void* k_pages, void* kpe_pages, void* v_pages,
                           void* scratch, size_t scratch_bytes, void* hip_stream,
                           akv_pool** out);
akv_status akv_pool_destroy(akv_pool* pool);   /* waits for the pool's stream */

/* Sequences get ids 0, 1, 2, ... in creation order; ids are not reused.
 * Releasing returns every page the sequence still owns to the back of the
 * free queue in allocation order.  Errors: AKV_EINVAL (unknown id),
 * AKV_ESTATE (already released). */
akv_status akv_seq_create(akv_pool* pool, int32_t* seq);
akv_status akv_seq_release(akv_pool* pool, int32_t seq);

/* ---- cache operations ([AKV-notes] section 1: append, drop, repos) ---------- */

/* append: add n tokens with positions pos[0..n) (host array, each in
 * [0, 2^31)).  K, K_pe, V are device arrays, token-major:
 *   GQA: K [n][n_kv_heads][d_rope], K_pe NULL, V [n][n_kv_heads][d_v]
 *   MLA: K = K_nope [n][n_kv_heads][d_nope], K_pe [n][H_pe][d_rope], V as above.
 * Keys arrive already rotated to their positions.  Passing K == K_pe == V ==
 * NULL reserves the slots only (a caller's own kernel writes them; see
 * akv_seq_tokens).  Errors: AKV_EINVAL, AKV_ERANGE (position), AKV_ENOMEM
 * (no page left in the free and evictable queues). */
akv_status akv_append(akv_pool* pool, int32_t seq, const void* K, const void* K_pe,
                      const void* V, const int32_t* pos, int32_t n);

/* append to several sequences in one call (a decode step: a few new tokens
 * for each of many requests).  Entry i appends counts[i] tokens to seqs[i];
 * K, K_pe, V and pos hold all entries' tokens concatenated in entry order,
 * laid out as for akv_append.  The result, slots and page order included,
 * is that of calling akv_append for each entry in order (a sequence may
 * appear more than once); every entry is validated and the pages for all of
 * them are counted before anything changes, and all rows are written by one
 * kernel launch.  Errors: as akv_append (AKV_EINVAL also for n_seqs < 0 or
 * a negative count). */
akv_status akv_append_batch(akv_pool* pool, int32_t n_seqs, const int32_t* seqs, const int32_t* counts,
                            const void* K, const void* K_pe, const void* V, const int32_t* pos);

/* drop ([AKV-blog] section 2, The Drop Primitive): mark the tokens of every
 * span inactive.  Nothing is freed or rewritten; later attention lists skip
 * them.  Dropping a token twice is a no-op; an empty span is a no-op.  When
 * the sequence's fragmentation (1 - visible tokens / written slots of the pages
 * holding a visible token) then exceeds the threshold, compaction runs if the
 * allocator can supply the fresh pages (it is skipped otherwise).
 * Errors: AKV_EINVAL (end < begin), AKV_ERANGE (span outside 0..n). */
akv_status akv_drop(akv_pool* pool, int32_t seq, const akv_span* spans, int32_t n_spans);

/* compaction ([AKV-blog] section 7, Dilemma 2): copy every visible token, in
 * visible-list order, into fresh pages (one device copy kernel), then move the
 * old pages to the evictable queue.  Values are copied bit for bit.  Without
 * force it runs only above the fragmentation threshold. */
akv_status akv_compact(akv_pool* pool, int32_t seq, int32_t force);

/* Deferred compaction ([AKV-blog] section 7, Dilemma 2: the defragmentation
 * pass runs asynchronously, in decode bubbles, without pausing inference).  AKV_COMPACT_IMMEDIATE (the default):
 * akv_drop and akv_splice compact a sequence as soon as it exceeds the
 * threshold.  AKV_COMPACT_DEFERRED: they only append it to a FIFO queue (once;
 * releasing the sequence removes it), and the caller runs the copies when the
 * GPU has room, with akv_compact_pending.  Errors: AKV_EINVAL (unknown mode). */
enum { AKV_COMPACT_IMMEDIATE = 0, AKV_COMPACT_DEFERRED = 1 };
akv_status akv_compaction_mode(akv_pool* pool, int32_t mode);

/* Compact queued sequences in queue order, as a background pass: the copies
 * run on the pool's background stream, after the pool stream's work so far
 * and beside its later work (a later launch touching a page the copies read
 * or write waits for them first).  A sequence no longer above the
 * threshold leaves the queue without a copy; the walk stops at the first one
 * whose visible tokens would take the moved total past max_tokens, that the
 * allocator cannot supply pages for, or whose copy list does not fit the
 * scratch buffer, and after max_seqs compactions.  Each compaction is the same
 * as akv_compact's; the copies of consecutive compactions share one kernel
 * launch unless a sequence takes its fresh pages from the evictable queue (it
 * then starts a new launch, ordered after the copies that read those pages).
 * seqs_out (max_seqs entries, may be NULL) receives the compacted sequences,
 * n_out their number.  Errors: AKV_EINVAL (negative budget, NULL n_out). */
akv_status akv_compact_pending(akv_pool* pool, int64_t max_tokens, int32_t max_seqs, int32_t* seqs_out,
                               int32_t* n_out);

/* The queued sequences in queue order (the first cap of them; n_out = all). */
akv_status akv_compact_queue(akv_pool* pool, int32_t* seqs_out, int32_t cap, int32_t* n_out);

/* repos ([AKV-blog] section 2, The Repos Primitive; [Leyline] Method): every
 * retained token covered by spans gets the sum of their deltas d (signed);
 * its position becomes pos + d and its rotated key part becomes R(d) k, with
 * R(phi) = [[cos, -sin], [sin, cos]] on each pair at angle d * theta_i.  The
 * angle is formed in fp64 and reduced mod 2*pi, the rotation is done in fp32
 * and rounded once to bf16 (round to nearest even).  GQA rotates all of K;
 * MLA rotates K_pe only (K_nope and V are untouched).  Dropped tokens and
 * tokens with total delta 0 are not touched.  One kernel launch covers all
 * spans.  Errors: AKV_EINVAL, AKV_ERANGE (span, or a new position outside
 * [0, 2^31)). */
akv_status akv_repos(akv_pool* pool, int32_t seq, const akv_span* spans, const int32_t* delta,
                     int32_t n_spans);

/* repos of many sequences in one call: entry i applies span_counts[i] spans
 * (and as many deltas) to seqs[i]; spans and deltas are concatenated in entry
 * order.  The result equals akv_repos on each entry in turn; all entries are
 * validated first (any error leaves every sequence as it was), and one
 * rotation launch covers every entry.  The sequences must be distinct.
 * Errors: AKV_EINVAL (a sequence named twice, negative counts), AKV_ERANGE
 * (as akv_repos), AKV_ESTATE (released sequence). */
akv_status akv_repos_batch(akv_pool* pool, int32_t n_seqs, const int32_t* seqs, const int32_t* span_counts,
                           const akv_span* spans, const int32_t* delta);

/* deferred repos (the fused rotation of [AKV-blog] section 4 and rule of
 * thumb 2: keys stay where they are and are turned where they are read):
 * the same validation, positions and errors as akv_repos, but no key is
 * rewritten; each token records the rotation its stored key still owes.
 * akv_seq_attention applies owed rotations where the kernels read the keys:
 * the decode kernel in registers, the 128-dim GQA prefill kernel in LDS
 * (each landed key tile turned once per block), both with the rotation table
 * and fp32 formula of akv_repos, so the results equal repos-then-attention
 * bit for bit; other launches first materialize each sequence they read
 * (as akv_materialize: own rows rotated in place, rows in shared pages copied
 * into the sequence's own pages, which can fail with AKV_ENOMEM before the
 * launch; see akv_fused_rotation).  akv_segment_attention reads keys as
 * stored.  Later repos calls, compaction, splices and clones keep each
 * token's debt. */
akv_status akv_repos_deferred(akv_pool* pool, int32_t seq, const akv_span* spans, const int32_t* delta,
                              int32_t n_spans);
/* Where akv_seq_attention applies owed rotations.  AKV_FUSE_AUTO (the
 * default): decode launches turn keys in the kernel; a prefill launch on the
 * 128-dim GQA layout does so when it turns each owed key at most once per kv
 * head (every segment one row tile of 256 packed rows, every sequence in one
 * segment), and otherwise materializes the sequences first (a prefill block
 * turns every tile it reads, so keys read by many row tiles are cheaper to
 * rotate once in HBM).  AKV_FUSE_ALWAYS: every launch whose kernel can turn
 * keys does.  AKV_FUSE_NEVER: the sequences are always materialized first.
 * Outputs are the same bits in every mode (materializing copies rows of
 * shared pages, so page tables can differ).  Errors: AKV_EINVAL. */
enum { AKV_FUSE_AUTO = 0, AKV_FUSE_ALWAYS = 1, AKV_FUSE_NEVER = 2 };
akv_status akv_fused_rotation(akv_pool* pool, int32_t mode);
/* Rotate the sequence's visible keys by what they owe, as akv_repos would
 * have; the debt is then 0.  Rows of its own pages are turned in place (one
 * launch); rows in shared pages (akv_seq_share) are copied, turned, into new
 * slots of its own pages, placed as an append places tokens (one copy launch
 * per distinct owed rotation).  Errors: AKV_EINVAL, AKV_ESTATE, AKV_ENOMEM
 * (scratch, or no pages for the copies: then nothing changed). */
akv_status akv_materialize(akv_pool* pool, int32_t seq);
/* Owed rotation of tokens first .. first+n-1 (position minus the position
 * their stored key encodes). */
akv_status akv_seq_lag(akv_pool* pool, int32_t seq, int32_t first, int32_t n, int32_t* lag);

/* repos over the layers of a model in one launch (the same operation as
 * akv_repos, applied to every pool in pools[0..n_pools)).  A model keeps one
 * pool per layer with the same op history, so the layers' page tables and
 * positions agree and one plan serves them all; the rotation of every
 * layer's keys is a single kernel launch (grid rows = layers).  Requirements,
 * checked before anything changes: the pools are distinct, share pool 0's
 * layout, frequency table and HIP stream, and sequence seq has the same
 * slots, positions and dropped flags in each.  Metadata is committed in every
 * pool on success.  Device work goes on the shared stream; the pointer table
 * lives in pool 0's scratch.  Errors: AKV_EINVAL (mismatch, NULL), AKV_ERANGE
 * (as akv_repos), AKV_ENOMEM (pool 0's scratch). */
akv_status akv_repos_layers(akv_pool* const* pools, int32_t n_pools, int32_t seq, const akv_span* spans,
                            const int32_t* delta, int32_t n_spans);

/* splice ([Leyline] Method, AMORTIZE mode): spans are given in coordinates of
 * the current visible list (entry i is the i-th visible token in position
 * order), sorted and disjoint, each non-empty.  Splice j drops its span,
 * appends stub_len[j] stub tokens at positions p_j + sum_{i<j} delta_i + 0..,
 * where p_j is the position of the span's first entry, and moves every visible
 * entry after the span by delta_j = stub_len[j] - (end_j - begin_j).  Per-token
 * deltas of several splices are summed and applied in one rotation launch.
 * Stub K/K_pe/V: device arrays as for akv_append, concatenated over splices,
 * already rotated to their stub positions.  stub_pos_out (optional host array
 * of sum(stub_len) entries) receives the stub positions. */
akv_status akv_splice(akv_pool* pool, int32_t seq, const akv_span* spans, const int32_t* stub_len,
                      int32_t n_splices, const void* stub_K, const void* stub_Kpe,
                      const void* stub_V, int32_t* stub_pos_out);

/* positional version ([AKV-notes] section 3, Cache Management: re-use by key
 * rotation, and the retrigger match of the cache reuse matching rules): the
 * retained tokens of src with logical index in [first, first+n), in logical
 * order, are appended to dst at positions pos + delta.  Their keys are copied
 * with the rotated part turned by R(delta) (GQA: all of K; MLA: K_pe, with
 * K_nope copied as is) and their V rows are copied; the source rows are not
 * touched, so src keeps its own version.  The new tokens take dst's next
 * logical indices and slots exactly as akv_append would place them (src ==
 * dst is allowed: the copies are read from the state before the call).
 * Rotation arithmetic as akv_repos; delta 0 is a bit-exact copy.  Dropped
 * tokens are skipped; when no token qualifies nothing changes.  All rows move
 * in one kernel launch (after the cos/sin table launch).  Errors, checked before
 * anything changes: AKV_EINVAL (bad sequence, n < 0), AKV_ERANGE ([first,
 * first+n) outside src, a new position outside [0, 2^31), dst too long),
 * AKV_ENOMEM (pages or scratch), AKV_ESTATE (released sequence). */
akv_status akv_seq_clone(akv_pool* pool, int32_t src, int32_t first, int32_t n, int32_t dst,
                         int32_t delta);

/* Shared pages for cached states ([AKV-blog] section 3, branching on
 * divergence with copy-on-write page-table references; [AKV-notes] section 3,
 * Cache Management: a positional version re-uses a cached state through a
 * key rotation, and versions are evicted once nothing uses them).
 *
 * akv_seq_freeze makes a sequence a checkpoint: keys owing a rotation are
 * turned in place first, then its rows never change; calls that would change
 * it (append, drop, repos, splice, compaction, clone into it) return
 * AKV_ESTATE.  Releasing it while other sequences still hold slots in its
 * pages keeps those pages until the last of them lets go (release, drop of
 * the shared tokens, compaction or copy on write).
 *
 * akv_seq_share appends the retained tokens of frozen sequence src with
 * logical index in [first, first+n), in logical order, to dst at positions
 * pos + delta without writing anything: each new token holds the source
 * token's slot (a reference into src's page) and owes the rotation by delta
 * (akv_seq_lag), which the attention kernels apply where they read the key
 * (akv_fused_rotation).  On dst, tokens in shared pages are never written in
 * place: a repos makes them owe the rotation, akv_materialize gives them
 * private rows (copy on write: K turned by what it owes, V and K_nope
 * copied), compaction copies them like any visible token, and a drop gives
 * their slot up at once (akv_seq_tokens then reports -1).  dst's appends go to
 * its own pages.  Errors: AKV_EINVAL (bad sequence, n < 0), AKV_ESTATE (src not
 * frozen, dst frozen or released), AKV_ERANGE ([first, first+n) outside src, a
 * new position outside [0, 2^31), dst too long). */
akv_status akv_seq_freeze(akv_pool* pool, int32_t seq);
akv_status akv_seq_share(akv_pool* pool, int32_t src, int32_t first, int32_t n, int32_t dst, int32_t delta);

/* ---- visibility -------------------------------------------------------------- */

/* Page-table image of the sequence's visible list: retained tokens minus the
 * optional mask spans (hidden from this list only, not dropped), ordered by
 * (position, logical index), encoded as maximal runs of consecutive slots of
 * one page.  Writes up to cap extents; *n_out gets the full count (call again
 * with a larger cap when *n_out > cap; AKV_ERANGE is returned then). */
akv_status akv_seq_visible(akv_pool* pool, int32_t seq, const akv_span* mask, int32_t n_mask,
                           akv_extent* out, int32_t cap, int32_t* n_out);

/* ---- segment-batch attention ([AKV-notes] section 3; [AKV-blog] section 4) -------- */

/* Q: device bf16 [n_q_tokens][n_q_heads][d_nope + d_rope] (MLA rows are
 * [q_nope | q_pe]); out: device bf16 [n_q_tokens][n_q_heads][d_v].
 * Segment s covers query rows q_begin .. q_begin+q_len-1 and reads the list
 * page_lists[ext_begin .. ext_begin+ext_len) (host array of extents) of
 * Lkv >= q_len entries.  Query i of the segment attends to list entries
 * 0 .. Lkv - q_len + i (the segment's own tokens are the last q_len entries):
 * out = softmax(scale * q K^T) V with fp32 accumulation; scale 0 selects
 * 1/sqrt(d_nope + d_rope).  All segments run in one launch.  Segments must not
 * overlap in Q rows; rows no segment covers are not written.  q_len == 0
 * segments are skipped.  Errors: AKV_EINVAL (Lkv < q_len, overlapping rows),
 * AKV_ERANGE (row or extent out of range), AKV_ENOMEM (scratch too small),
 * AKV_ESTATE (page-table-only pool). */
akv_status akv_segment_attention(akv_pool* pool, const void* Q, int32_t n_q_tokens,
                                 const akv_segment* segs, int32_t n_segs,
                                 const akv_extent* page_lists, int32_t n_ext, float scale,
                                 void* out);

/* akv_segment_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same validation, plan, kernels and results (bit for bit),
 * but the call's work tables, expanded slot list and split-KV partials live
 * in a static device workspace of the library (128 MiB per GPU, held from
 * the library's first use on that GPU until the process ends) instead of
 * the pool's scratch buffer.  The call allocates nothing: no hipMalloc,
 * hipHostMalloc or hipFree (the tables are copied from host memory the pool
 * already holds, on the pool's stream, after the kernels of earlier calls).
 * Every call on one GPU shares that GPU's workspace, which keeps the last
 * call's contents (nothing in it needs clearing): calls on one stream are
 * ordered, but calls that overlap on one GPU (other streams, other pools,
 * other threads) race.  Errors: those of akv_segment_attention, and
 * AKV_ENOMEM when the call needs more than 128 MiB of workspace (about 4 B per
 * list entry + 16 B per extent + 24 B per work item + split partials of
 * 4 B * (d_v + 2) per row and split), before anything is enqueued. */
akv_status akv_segment_attention_static(akv_pool* pool, const void* Q, int32_t n_q_tokens,
                                        const akv_segment* segs, int32_t n_segs,
                                        const akv_extent* page_lists, int32_t n_ext, float scale,
                                        void* out);

/* segment-batch attention over sequences' own lists: segment i reads the
 * visible list of sequence segs[i].seq minus the spans masks[mask_begin ..
 * mask_begin+mask_len) (logical-index spans, hidden from this segment only),
 * i.e. the list akv_seq_visible returns for that mask, and runs exactly as
 * akv_segment_attention with those lists (same kernels, same results).  The
 * lists are built inside the library from each sequence's cached page-table
 * image, so a decode step hands over no extents.  Errors: AKV_EINVAL (bad
 * sequence, negative count, mask range outside masks[]), AKV_ESTATE (released
 * sequence), AKV_ERANGE (mask span outside its sequence), and those of
 * akv_segment_attention. */
akv_status akv_seq_attention(akv_pool* pool, const void* Q, int32_t n_q_tokens, const akv_seq_segment* segs,
                             int32_t n_segs, const akv_span* masks, int32_t n_masks, float scale, void* out);

/* Attention mass per page, the statistic a server-side drop policy watches
 * ([AKV-blog] section 7, Dilemma 1: blocks whose cumulative attention weight
 * stays below a threshold over consecutive decode turns are dropped).
 * mass: device float array of num_pages entries (caller-owned, not cleared
 * by the library), or NULL to stop.  While set, every decode launch of
 * akv_segment_attention or akv_seq_attention on the pool (128-dim GQA,
 * segments of at most 16 packed rows per kv head) also adds, to mass[page],
 * the softmax weight its rows put on the page's keys: summed over the
 * segments' query tokens and q heads, so the pages of one launch receive
 * (query tokens x q heads) in total (divide by that for the mean weight).
 * Keys owing a rotation count at their position.  It is a second pass over
 * the launch's K rows (one more read of K) after the attention, which also
 * writes each row's log-sum-exp to the pool's scratch buffer; other launches
 * (prefill, other layouts, akv_segment_attention_static) leave mass alone.
 * Errors: AKV_EINVAL (n_pages differs from the pool's page count),
 * AKV_ESTATE (page-table-only pool). */
akv_status akv_attention_mass(akv_pool* pool, float* mass, int32_t n_pages);

/* ---- extended radix tree of cached states ([AKV-blog] section 3; [AKV-notes]
 * section 3, Cache Management and Cache Reuse Matching Rules) -------------------- */

/* A history is a sequence of events: a token (a = id, b = position), or one
 * span of a cache operation (drop: [a, b); repos: [a, b) by c), in the order
 * they were applied.  A checkpoint registers a pool sequence whose current
 * state is the state of a history.  A node of the tree is served by a
 * checkpoint below it when only token events lie between them (operations
 * would have changed the node's tokens; appended tokens do not): the first
 * n_tokens logical tokens of the checkpoint's sequence are then that node's
 * state.  The tree is host metadata only; it holds sequence ids, not pages. */
enum { AKV_EV_TOKEN = 0, AKV_EV_DROP = 1, AKV_EV_REPOS = 2 };
typedef struct { int32_t kind, a, b, c; } akv_event;
typedef struct akv_tree akv_tree;
/* Result of a match: seq = -1 when nothing matched.  n_events of the request
 * history matched; reuse the first n_tokens logical tokens of seq; exact = 1
 * (tokens, positions and operations equal: reuse as is) or 0 (retrigger:
 * tokens and operations equal, positions all shifted by delta: reuse through
 * akv_seq_clone with that delta). */
typedef struct { int32_t seq, n_events, n_tokens, exact, delta; } akv_tree_hit;

akv_status akv_tree_create(akv_tree** out);
akv_status akv_tree_destroy(akv_tree* tree);
/* Register seq as the state of history ev[0..n) (n >= 1; a sequence is
 * registered once).  Errors: AKV_EINVAL (bad event, empty history, seq
 * registered), AKV_ENOMEM. */
akv_status akv_tree_insert(akv_tree* tree, const akv_event* ev, int32_t n, int32_t seq);
/* Longest reusable prefix of a request history: the walk stops at the
 * first event that does not match; the longest exact prefix is taken first
 * and a retrigger prefix replaces it only when strictly longer; among the
 * checkpoints serving one node, the one registered last.  The hit's
 * checkpoint counts as used now (eviction order). */
akv_status akv_tree_match(akv_tree* tree, const akv_event* ev, int32_t n, akv_tree_hit* out);
/* Pin (add > 0) or unpin (add < 0) a checkpoint in use by a running request;
 * pinned checkpoints are not evicted. */
akv_status akv_tree_pin(akv_tree* tree, int32_t seq, int32_t add);
/* Remove up to max_n unpinned checkpoints, least recently used first (each
 * positional version on its own); their sequence ids go to seqs_out for the
 * caller to release.  Dropped tokens' pages are already the pool's first
 * eviction candidates. */
akv_status akv_tree_evict(akv_tree* tree, int32_t max_n, int32_t* seqs_out, int32_t* n_out);
akv_status akv_tree_stats(akv_tree* tree, int32_t* n_nodes, int32_t* n_checkpoints);

/* ---- inspection, sync, errors ---------------------------------------------------- */

/* Per-token metadata of tokens first .. first+n-1 (any output may be NULL);
 * slot is -1 for a dropped token whose page was evicted. */
akv_status akv_seq_tokens(akv_pool* pool, int32_t seq, int32_t first, int32_t n,
                          int32_t* slot, int32_t* pos, uint8_t* dropped);
/* Token count, visible count and fragmentation of a sequence. */
akv_status akv_seq_info(akv_pool* pool, int32_t seq, int32_t* n_tokens, int32_t* n_visible,
                        double* fragmentation);
/* Current free and evictable queues, front first (outputs may be NULL). */
akv_status akv_pool_queues(akv_pool* pool, int32_t* free_out, int32_t free_cap, int32_t* n_free,
                           int32_t* evict_out, int32_t evict_cap, int32_t* n_evict);
/* Dry run of akv_repos: the rotation work list it would launch, as (slot, delta)
 * pairs of every token it would rotate, in launch order; *n_out gets the count.
 * Changes nothing. */
akv_status akv_repos_plan(akv_pool* pool, int32_t seq, const akv_span* spans, const int32_t* delta,
                          int32_t n_spans, int32_t* slot_out, int32_t* delta_out, int32_t cap,
                          int32_t* n_out);

/* Dry run of the segment planner of akv_segment_attention ([AKV-notes]
 * section 3: one launch over every segment; [AKV-blog] section 4): the same
 * validation and errors (a page-table-only pool is accepted), then the work
 * list the call would launch, in grid order.  Item i runs as block i: rows
 * row0 .. row0 + rows_per_block - 1 (clipped to the segment's q_len x group
 * packed rows, token-major) of kv head kv_head, over list entries k_begin ..
 * k_end - 1 clipped to each row's causal limit; seg = -1 marks a padding
 * block.  part >= 0: the item writes fp32 partials of its rows from partial
 * row `part` on, and combine entry (seg, kv_head, row0, part0, n_split, rows)
 * merges split j's partial rows part0 + j * rows + r.  n_cu: compute units to
 * plan for (0 = the pool's device, or 256).  Outputs may be NULL (counts
 * only); AKV_ERANGE when a capacity is too small.  Changes nothing. */
typedef struct { int32_t seg, kv_head, row0, k_begin, k_end, part; } akv_attn_item;
typedef struct { int32_t seg, kv_head, row0, part0, n_split, rows; } akv_attn_combine;
akv_status akv_attention_plan(akv_pool* pool, int32_t n_q_tokens, const akv_segment* segs, int32_t n_segs,
                              const akv_extent* page_lists, int32_t n_ext, int32_t n_cu, akv_attn_item* items,
                              int32_t items_cap, int32_t* n_items, akv_attn_combine* comb, int32_t comb_cap,
                              int32_t* n_comb, int32_t* rows_per_block, int64_t* part_rows);

/* Kernel timing: when enabled, each kernel launch of the library carries a
 * start and a stop HIP event, stamped by the dispatch at the kernel's start and
 * end (the launch's duration, without the gap before it).  akv_timing_read
 * waits for the events, returns the summed milliseconds and launch count of one
 * kernel kind since the last read of that kind, and clears them. */
enum { AKV_K_APPEND = 0, AKV_K_ROTATE = 1, AKV_K_COMPACT = 2, AKV_K_EXPAND = 3,
       AKV_K_ATTN = 4, AKV_K_COMBINE = 5, AKV_K_CLONE = 6, AKV_K_MASS = 7, AKV_K_KINDS = 8 };
akv_status akv_timing_enable(akv_pool* pool, int32_t enable);
akv_status akv_timing_read(akv_pool* pool, int32_t kind, double* total_ms, int32_t* count);
/* The individual launch durations (ms) behind the next akv_timing_read of
 * the same kind, in launch order; *n_out gets their count (AKV_ERANGE when it
 * exceeds cap).  Does not clear them. */
akv_status akv_timing_samples(akv_pool* pool, int32_t kind, float* ms, int32_t cap, int32_t* n_out);

akv_status akv_sync(akv_pool* pool);       /* wait for the pool's streams */
const char* akv_last_error(void);          /* thread-local text of the last failure */

#ifdef __cplusplus
}
#endif
#endif /* AKV_H */
