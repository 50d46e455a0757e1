// Internal interface between the host runtime (akv_runtime.cpp) and the HIP
// kernels (akv_kernels.hip).  Plain structs that both the host planner and the
// device code read; every launcher enqueues on the given stream and returns the
// hipError_t of the launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace akv {

// One repos work item: rows lo..hi-1 of one page, rotated by deltas[didx].
struct RotItem {
  int32_t page, lo, hi, didx;
};

// One row copy of the compaction kernel: token moves from src slot to dst slot.
struct MovePair {
  int32_t src, dst;
};

// A page-table extent (same layout as akv_extent).
struct Extent {
  int32_t page, lo, hi;
};

// Segment as the attention kernel sees it: query rows, list length, and the
// offset of its slot list inside the expanded slot map.
struct AttnSeg {
  int32_t q_begin, q_len, lkv, list_off;
};

// One attention work item: a tile of attn_rows_per_block(d_nope) packed rows (token, q head in
// group) of one segment and kv head, over list entries k_begin..k_end-1.
// part >= 0: write an unnormalised fp32 partial (split-KV): the tile's row r
// goes to partial row part + r.
// seg < 0: padding block, exits at once.
struct AttnItem {
  int32_t seg, kvh, row0, k_begin, k_end, part;
};

// Split-KV merge for one row tile of `rows` rows: split j's partial of tile
// row r sits at partial row part0 + j * rows + r.
struct CombItem {
  int32_t seg, kvh, row0, part0, nsplit, rows;
};

constexpr int ATTN_KTILE = 64;       // keys per pipeline stage

// Packed rows per block of the prefill attention kernels (256 for every layout).
int attn_rows_per_block(int d_nope);

// ---- launchers --------------------------------------------------------------
// Rotates the items in place with the fp32 cos/sin table's rows (RotItem::didx;
// row = cos of the d_rope/2 pairs, then sin), in each
// of the n_layers page arrays listed in krs (a device array of pointers).
hipError_t launch_rotate(hipStream_t st, uint16_t* const* krs, int n_layers, int n_heads, int page_size,
                         int d_rope, int pairing, const RotItem* items, int n_items, const float* table);

// Rows of one paged array in a copy launch (akv_copy.hip): src is token-major
// [n][heads][d] for an append, the paged array itself for a move; dst is the
// paged array [pages][heads][page_size][d].
struct TokenRows {
  const uint16_t* src;
  uint16_t* dst;
  int heads, d;
};

// append: token t's rows of every listed array (at most 3) go to slots[t].
hipError_t launch_scatter_tokens(hipStream_t st, const TokenRows* rows, int n_rows, const int32_t* slots,
                                 int n, int page_size, int log2_page);

// slot -> slot moves of n tokens (compaction, positional versions): the
// rotated-key array kr (rope_heads x d_rope) moves with each pair turned by
// the delta whose cos / sin row is `table` (d_rope floats: cos of the d_rope/2
// pairs, then sin; nullptr = plain copy); the plain arrays (V, MLA K_nope; at
// most 2) are copied.  Source and destination slots are disjoint.
hipError_t launch_move_tokens(hipStream_t st, uint16_t* kr, int rope_heads, int d_rope, int pairing,
                              const TokenRows* plain, int n_plain, const MovePair* pairs, int n,
                              int page_size, int log2_page, const float* table);

hipError_t launch_expand(hipStream_t st, const Extent* ex, const int32_t* ex_off, int n_ext,
                         int page_size, int32_t* slots);

struct AttnArgs {
  const uint16_t* q;
  int n_q_heads, group;          // group = n_q_heads / n_kv_heads
  const uint16_t* k_a;           // GQA: K pages; MLA: K_nope pages
  const uint16_t* k_b;           // MLA: K_pe pages (else nullptr)
  int kpe_heads;                 // MLA: heads stored in K_pe pages (1 = shared)
  const uint16_t* v;
  int n_kv_heads, page_size, log2_page;
  const AttnSeg* segs;
  const AttnItem* items;
  int n_items;
  const int32_t* slots;
  float scale_log2e;             // softmax scale * log2(e)
  uint16_t* out;
  float* part_o;                 // [partial rows][d_v]
  float* part_ml;                // [partial rows][2]: (running max, sum)
  int rows_per_block;
  // decode kernel only: per list entry the row of rot_table (cos of the
  // d_rope/2 pairs, then sin) that turns its stored key to its position, or
  // -1 (key already there); nullptr when no key owes a rotation
  const int32_t* key_didx;
  const float* rot_table;
  int rot_pairing;
  // optional: per output row (token, q head) its log-sum-exp in base 2,
  // lse = m + log2(l) in the units of scale * log2(e) (so a key's weight for
  // the row is 2^(s * scale_log2e - lse)); +inf for a row with no key.
  // Written by the decode kernel for rows it finishes and by the combine
  // kernel; nullptr when not wanted
  float* lse;
};

// Returns hipErrorInvalidValue when no kernel is instantiated for the dims.
hipError_t launch_seg_attn(hipStream_t st, const AttnArgs& a, int d_nope, int d_rope, int d_v);
// The 128-dim GQA prefill kernel (akv_attn_dl.hip), called by launch_seg_attn.
hipError_t launch_seg_attn_dl(hipStream_t st, const AttnArgs& a);

hipError_t launch_combine(hipStream_t st, const AttnArgs& a, const CombItem* items, int n_items,
                          int d_v);

// Decode attention (akv_decode.hip): 128-dim GQA work items of at most
// DECODE_ROWS packed rows, the block's waves splitting the key range.
constexpr int DECODE_ROWS = 16;
hipError_t launch_decode_attn(hipStream_t st, const AttnArgs& a);
// Attention mass per page of a decode launch (second pass with a.lse): work
// item = (segment, first list entry of a chunk of MASS_CHUNK entries), grid
// rows = kv heads; mass[page] += the weight of the page's keys, summed over
// the segment's rows and q heads.
constexpr int MASS_CHUNK = 256;
struct MassItem {
  int32_t seg, k0;
};
hipError_t launch_page_mass(hipStream_t st, const AttnArgs& a, const MassItem* items, int n_items, int max_rows,
                            float* mass);
// Per list entry of each extent e (entries ex_off[e] .. + hi - lo): ex_didx[e].
hipError_t launch_expand_didx(hipStream_t st, const Extent* ex, const int32_t* ex_off, const int32_t* ex_didx,
                              int n_ext, int32_t* out);

bool attn_dims_supported(int d_nope, int d_rope, int d_v);

// Static device workspace of the no-allocation attention entry point: its
// size, and its device address on the current device (looked up once per
// device with hipGetSymbolAddress).
constexpr size_t STATIC_WORKSPACE_BYTES = (size_t)128 << 20;
hipError_t static_workspace(void** ptr);

// Text returned by akv_last_error (thread-local; host code of the library).
void set_error(const char* msg);

// Timer events armed for the next kernel launch of this thread (both null:
// none); a launch that carries them sets used (akv_launch.h).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchEvents& launch_events();

}  // namespace akv
