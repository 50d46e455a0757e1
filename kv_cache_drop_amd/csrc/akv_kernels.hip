// HIP kernels of the AKV hot path for MI355X (gfx950, wave64, MFMA).
//
// Sources, cited by page title and section:
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and State-Preserving
//               Prefix Invalidation Bypass" (A. Akhunji)
//   [AKV-notes] "Cache Engineering for Agents" (reading notes on Fu et al.)
//   [Leyline]   "Leyline: KV Cache Directives for Agentic Inference" (digest)
//
// Kernels:
//   k_rotate       repos delta rotation, in place on the paged pool (HBM-bound)
//   k_expand       extents -> per-entry slot list for the attention gather
//   k_seg_attn     segment-batch attention, bf16 MFMA 32x32x16 (MFMA-bound),
//                  register-staged gather (head sizes 32 and 64)
//   k_seg_attn_mla the same for the MLA row, direct-to-LDS
//   k_combine      split-KV merge of (m, l, O) partials
// (the 128-dim GQA attention kernel is in akv_attn_dl.hip)
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "akv_device.h"
#include "akv_internal.h"
#include "akv_launch.h"

namespace akv {

// ---------------------------------------------------------------------------
// repos rotation ([AKV-blog] section 2, The Repos Primitive; [Leyline] Method)
//
// The host forms each distinct delta's row of cos and sin (fp64 angle
// delta * theta_i reduced mod 2*pi, stored as fp32: table[di][0..half) = cos,
// table[di][half..d) = sin) and uploads it with the work list.
// k_rotate: one block per (work item, layer) — items are (page, rows lo..hi-1,
// delta), the grid's second dimension picks one of n_layers page arrays that
// share the page table; the block
// stages its delta's row of the table in LDS and every head and row of the
// item reuses it.  A "unit" is 8 rotation pairs held in two 16-byte loads;
// pair (x, y) becomes (x cos - y sin, x sin + y cos) in fp32 and is rounded
// once to bf16.  The first pass issues its loads before the table is staged.
// ---------------------------------------------------------------------------
constexpr int ROT_THREADS = 256;
constexpr int ROT_UPT = 2;   // 512 units (one 16 KiB item) per pass

__global__ __launch_bounds__(ROT_THREADS, 8) void k_rotate(uint16_t* const* __restrict__ krs, int n_heads,
                                                            int S, int d, int pairing,
                                                            const RotItem* __restrict__ items,
                                                            const float* __restrict__ table) {
  __shared__ float s_c[128], s_s[128];
  const RotItem it = items[blockIdx.x];
  uint16_t* __restrict__ kr = krs[blockIdx.y];   // one layer's rotated-key pages per grid row
  const int half = d >> 1;
  const int upr = d >> 4;
  const int rows = it.hi - it.lo;
  const int per_head = rows * upr;
  const int n_units = n_heads * per_head;
  const int n_pass = (n_units + ROT_UPT * ROT_THREADS - 1) / (ROT_UPT * ROT_THREADS);

  u32x4 ra[ROT_UPT], rb[ROT_UPT];
  uint16_t* pa[ROT_UPT];
  uint16_t* pb[ROT_UPT];
  int cu[ROT_UPT];

  auto locate = [&](int u, int i) {
    const int h = u / per_head;
    const int rem = u - h * per_head;
    const int row = it.lo + rem / upr;
    const int c = rem - (rem / upr) * upr;
    uint16_t* base = kr + (((size_t)it.page * n_heads + h) * S + row) * d;
    cu[i] = c;
    if (pairing == 0) {
      pa[i] = base + 16 * c;
      pb[i] = pa[i] + 8;
    } else {
      pa[i] = base + 8 * c;
      pb[i] = base + half + 8 * c;
    }
  };

#pragma unroll
  for (int i = 0; i < ROT_UPT; ++i) {
    const int u = threadIdx.x + i * ROT_THREADS;
    if (u < n_units) {
      locate(u, i);
      ra[i] = *(const u32x4*)pa[i];
      rb[i] = *(const u32x4*)pb[i];
    }
  }
  if ((int)threadIdx.x < half) {
    s_c[threadIdx.x] = table[(size_t)it.didx * d + threadIdx.x];
    s_s[threadIdx.x] = table[(size_t)it.didx * d + half + threadIdx.x];
  }
  __syncthreads();

  for (int pass = 0; pass < n_pass; ++pass) {
#pragma unroll
    for (int i = 0; i < ROT_UPT; ++i) {
      const int u = threadIdx.x + (pass * ROT_UPT + i) * ROT_THREADS;
      if (u >= n_units) continue;
      if (pass > 0) {
        locate(u, i);
        ra[i] = *(const u32x4*)pa[i];
        rb[i] = *(const u32x4*)pb[i];
      }
      const int p0 = 8 * cu[i];  // first pair of the unit
      u32x4 oa, ob;
      if (pairing == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          oa[k] = rot_pair_word(ra[i][k], s_c[p0 + k], s_s[p0 + k]);
          ob[k] = rot_pair_word(rb[i][k], s_c[p0 + 4 + k], s_s[p0 + 4 + k]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float c0 = s_c[p0 + 2 * k], s0 = s_s[p0 + 2 * k];
          const float c1 = s_c[p0 + 2 * k + 1], s1 = s_s[p0 + 2 * k + 1];
          const float x0 = bf_lo(ra[i][k]), x1 = bf_hi(ra[i][k]);
          const float y0 = bf_lo(rb[i][k]), y1 = bf_hi(rb[i][k]);
          oa[k] = pack_bf2(fmaf(x0, c0, -y0 * s0), fmaf(x1, c1, -y1 * s1));
          ob[k] = pack_bf2(fmaf(x0, s0, y0 * c0), fmaf(x1, s1, y1 * c1));
        }
      }
      *(u32x4*)pa[i] = oa;
      *(u32x4*)pb[i] = ob;
    }
  }
}

hipError_t launch_rotate(hipStream_t st, uint16_t* const* krs, int n_layers, int n_heads, int page_size,
                         int d_rope, int pairing, const RotItem* items, int n_items, const float* table) {
  if (n_items <= 0 || n_layers <= 0) return hipSuccess;
  launch_k(k_rotate, dim3(n_items, n_layers), dim3(ROT_THREADS), st, krs, n_heads, page_size, d_rope, pairing,
           items, table);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// extents -> slot list (one thread per extent)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_expand(const Extent* __restrict__ ex,
                                                const int32_t* __restrict__ ex_off, int n_ext, int S,
                                                int32_t* __restrict__ slots) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n_ext) return;
  const Extent x = ex[e];
  int32_t* o = slots + ex_off[e];
  for (int i = x.lo; i < x.hi; ++i) o[i - x.lo] = x.page * S + i;
}

hipError_t launch_expand(hipStream_t st, const Extent* ex, const int32_t* ex_off, int n_ext,
                         int page_size, int32_t* slots) {
  if (n_ext <= 0) return hipSuccess;
  launch_k(k_expand, dim3((n_ext + 255) / 256), dim3(256), st, ex, ex_off, n_ext, page_size, slots);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// segment-batch attention ([AKV-notes] section 3, Segment-Batch Attention;
// [AKV-blog] section 4)
//
// One block = NW waves = 32*NW packed rows (token-major, the q heads of one
// kv head side by side) of one segment, over list entries k_begin..k_end-1,
// in tiles of 64 keys gathered from pages through the segment's slot list.
// Two waves share each SIMD (NW = 8: one block per CU; NW = 4: two blocks per
// CU that run out of step), so one wave's softmax overlaps another's matrix
// work.
//
// Per wave: 32 query rows.  S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K
// tile from LDS, B = Q in registers), so every lane owns one query row
// (lane % 32) and half of the keys of each 32-key block; the row max and sum
// need one exchange with lane ^ 32.  O^T = V^T P^T takes the S^T accumulators
// (as bf16 P) directly as the B operand: V is stored transposed in LDS with
// the keys of every 16-key group permuted into the accumulator's key order, so
// no register shuffles are needed.  Causality is bottom-right over list order:
// query i sees entries 0 .. Lkv - Lq + i.
//
// Softmax runs in base 2 with a lazily updated running max: O and l are
// rescaled only when a row's max grows by more than 2^RESCALE_LOG2 over the
// reference (so P <= 2^8 in between), which takes the accumulator rescale off
// almost every tile.
//
// Loads: the tile j+1 loads are in flight in registers while tile j is
// computed, then written to the other LDS buffer (one barrier per tile); V is
// transposed on the way into LDS.
// ---------------------------------------------------------------------------

template <int DQK, int DV, int DNOPE, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_seg_attn(AttnArgs a) {
  constexpr int NT = 64 * NW;          // threads per block
  constexpr int RB = 32 * NW;          // packed rows per block
  constexpr int KT = ATTN_KTILE;
  constexpr int KPAD = DQK + 8;        // LDS K row stride (elements)
  constexpr int VPAD = KT + 8;         // LDS V^T row stride (elements)
  constexpr int NKS = DQK / 16;        // k-steps of S^T
  constexpr int NCB = DV / 32;         // 32-wide column blocks of O^T
  constexpr int KCH = DQK / 8;         // 16-byte chunks per K row
  constexpr int VCH = DV / 8;          // 16-byte chunks per V row
  constexpr int VTASKS = VCH * (KT / 2);  // V tasks: 2 keys x 8 columns each
  constexpr int NVL = (VTASKS + NT - 1) / NT;
  static_assert(DQK % 32 == 0 && DV % 32 == 0, "dims");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][DV * VPAD];

  const AttnItem it = a.items[blockIdx.x];
  if (it.seg < 0) return;
  const AttnSeg sg = a.segs[it.seg];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const int G = a.group;
  const int lq = sg.q_len, lkv = sg.lkv;
  const int rows_total = lq * G;
  const int brow_last = min(it.row0 + RB, rows_total) - 1;
  const int lim_first = lkv - lq + it.row0 / G;
  const int lim_last = lkv - lq + brow_last / G;
  const int k_end = it.k_end;
  const int k_stop = min(k_end, lim_last + 1);
  const int n_tiles = k_stop > it.k_begin ? (k_stop - it.k_begin + KT - 1) / KT : 0;
  const int Hkv = a.n_kv_heads, S = a.page_size, lg = a.log2_page;
  const int kvh = it.kvh;
  const int32_t* __restrict__ slots = a.slots + sg.list_off;

  // the lane's query row
  const int r = it.row0 + 32 * w + l32;
  const bool valid = r < rows_total;
  const int tok = valid ? r / G : 0;
  const int hq = kvh * G + (valid ? r - tok * G : 0);
  const int lim = valid ? min(lkv - lq + tok, k_end - 1) : k_stop - 1;
  bf16x8 qf[NKS];
  {
    const uint16_t* qp = a.q + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (valid) {
        qf[ks] = *(const bf16x8*)(qp + 16 * ks);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // Loaders.  K: TPK threads per key row, each staging CPT consecutive 16-byte
  // chunks, so a thread resolves one slot per pass.  V: tasks of 2 keys x 8
  // columns, transposed on the way into LDS.  Every thread issues the same
  // loads (surplus threads repeat a task and write identical values), so the
  // compiler can count outstanding loads exactly instead of draining them.
  // Page offsets use 24-bit multiplies (pools hold fewer than 2^24 pages).
  //
  // The gather is a chain of two dependent global loads (slot index, then the
  // row), each mostly an L2 miss, so it runs ahead of the compute: slot indices
  // are fetched three tiles ahead and K/V rows two tiles ahead, into one of two
  // register staging sets.  Indices past the list end are clamped to its last
  // entry, so tail loads stay in bounds.
  constexpr int TPK = KCH < 8 ? KCH : 8;
  constexpr int CPT = KCH / TPK;
  constexpr int KPP = NT / TPK;                 // key rows per pass
  constexpr int NKP = (KT + KPP - 1) / KPP;     // passes
  struct Slots {
    int k[NKP];
    int v[NVL][2];
  };
  struct Stage {
    u32x4 k[NKP][CPT];
    u32x4 v[NVL][2];
  };
  const int HS = Hkv * S;
  const int hoff = kvh * S;
  const int kpe_hoff = (a.kpe_heads == 1 ? 0 : kvh) * S;
  const int kpe_hs = a.kpe_heads * S;
  auto k_key = [&](int ps) { return (tid / TPK + KPP * ps) % KT; };
  auto v_task = [&](int j) { return (tid + NT * j) % VTASKS; };

  auto fetch_slots = [&](int k0, Slots& sl) {
#pragma unroll
    for (int ps = 0; ps < NKP; ++ps) sl.k[ps] = slots[min(k0 + k_key(ps), lkv - 1)];
#pragma unroll
    for (int j = 0; j < NVL; ++j) {
      const int pair = v_task(j) % (KT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) sl.v[j][e] = slots[min(k0 + 2 * pair + e, lkv - 1)];
    }
  };

  auto fetch_rows = [&](const Slots& sl, Stage& st) {
#pragma unroll
    for (int ps = 0; ps < NKP; ++ps) {
      const int slot = sl.k[ps];
      const int page = slot >> lg, off = slot & (S - 1);
      const int c0 = (tid % TPK) * CPT;
      const uint32_t row = __umul24(page, HS) + hoff + off;
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int c = c0 + q;
        const uint16_t* src;
        if (DNOPE == 0) {
          src = a.k_a + (size_t)row * DQK + 8 * c;
        } else {
          const uint32_t prow = __umul24(page, kpe_hs) + kpe_hoff + off;
          const uint16_t* pn = a.k_a + (size_t)row * DNOPE + 8 * c;
          const uint16_t* pp = a.k_b + (size_t)prow * (DQK - DNOPE) + 8 * (c - DNOPE / 8);
          src = c < DNOPE / 8 ? pn : pp;
        }
        st.k[ps][q] = *(const u32x4*)src;
      }
    }
#pragma unroll
    for (int j = 0; j < NVL; ++j) {
      const int vp = v_task(j) / (KT / 2);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int slot = sl.v[j][e];
        const uint32_t row = __umul24(slot >> lg, HS) + hoff + (slot & (S - 1));
        st.v[j][e] = *(const u32x4*)(a.v + (size_t)row * DV + 8 * vp);
      }
    }
  };

  auto store_tile = [&](const Stage& st, int buf) {
#pragma unroll
    for (int ps = 0; ps < NKP; ++ps) {
      const int c0 = (tid % TPK) * CPT;
#pragma unroll
      for (int q = 0; q < CPT; ++q)
        *(u32x4*)&sK[buf][k_key(ps) * KPAD + 8 * (c0 + q)] = st.k[ps][q];
    }
#pragma unroll
    for (int j = 0; j < NVL; ++j) {
      // keys 2*pair, 2*pair+1 go to LDS positions with quads 1 and 2 of every
      // 16-key group swapped (the accumulator's key order)
      const int vt = v_task(j);
      const int pair = vt % (KT / 2), vp = vt / (KT / 2);
      const int key = 2 * pair, quad = key >> 2, qg = quad & 3;
      const int pos = (quad & ~3) * 4 + (qg == 1 ? 2 : (qg == 2 ? 1 : qg)) * 4 + (key & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        const unsigned w2 = (e & 1) == 0 ? (st.v[j][0][dw] & 0xffffu) | (st.v[j][1][dw] << 16)
                                          : (st.v[j][0][dw] >> 16) | (st.v[j][1][dw] & 0xffff0000u);
        *(unsigned*)&sV[buf][(8 * vp + e) * VPAD + pos] = w2;
      }
    }
  };

  f32x16 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
  float m_run = -INFINITY;  // reference max (base-2 units) of O and l
  float l_run = 0.f;
  const float c2 = a.scale_log2e;

  Slots slA, slB;
  Stage stA, stB;
  const int k_begin = it.k_begin;
  fetch_slots(k_begin, slA);
  fetch_rows(slA, stA);
  fetch_slots(k_begin + KT, slB);
  fetch_rows(slB, stB);
  fetch_slots(k_begin + 2 * KT, slA);
  store_tile(stA, 0);
  __syncthreads();

  // Tile j: rows of tile j+2 are requested into the staging set tile j used,
  // slots of tile j+3 into the slot set tile j+1 used, the tile is computed,
  // and tile j+1 (requested one iteration earlier) is written to LDS.  The
  // loop runs an even number of tiles: a tile past the range is fully masked
  // and adds nothing.
  auto step = [&](int j, Slots& sl_cur, Stage& st_cur, Slots& sl_nxt, Stage& st_nxt) {
    const int buf = j & 1;
    const int k0 = k_begin + j * KT;
    fetch_rows(sl_cur, st_cur);      // sl_cur holds tile j+2's slots
    fetch_slots(k0 + 3 * KT, sl_nxt);

    // S^T = K Q^T: two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    const uint16_t* kbase = &sK[buf][0];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 af = *(const bf16x8*)(kbase + (32 * kb + l32) * KPAD + 16 * ks + 8 * g);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[ks], sacc[kb], 0, 0, 0);
      }
    }

    if ((k0 + KT > k_end) || (k0 + KT - 1 > lim_first)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key > lim) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_xor32(mx);
    const float m_cand = fmaxf(m_run, mx * c2);
    if (__ballot(m_cand > m_run + RESCALE_LOG2)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
      l_run *= alpha;
      if (j > 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
      }
      m_run = m_cand;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
    bf16x8 pf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, r0 = 8 * (t & 1);
      u32x4 pk;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r0 + 2 * k], c2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r0 + 2 * k + 1], c2, -m_use));
        pk[k] = pack_bf2(p0, p1);
        rs += p0 + p1;
      }
      pf[t] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += rs;   // per-lane partial; the two halves of a row are added at the end

    // O^T += V^T P^T
    const uint16_t* vbase = &sV[buf][0];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const bf16x8 vf = *(const bf16x8*)(vbase + (32 * cb + l32) * VPAD + 16 * t + 8 * g);
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[cb], 0, 0, 0);
      }
    }

    store_tile(st_nxt, buf ^ 1);
    __syncthreads();
  };
  for (int j = 0; j < n_tiles; j += 2) {
    step(j, slA, stA, slB, stB);
    step(j + 1, slB, stB, slA, stA);
  }

  // the two lanes of a row hold disjoint key halves of l
  l_run = sum_xor32(l_run);
  // epilogue: lane holds O^T columns c = 32cb + 8m + 4g + 0..3 of its row
  if (!valid) return;
  if (it.part < 0) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* op = a.out + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x2 v2 = {pack_bf2(oacc[cb][4 * m] * inv, oacc[cb][4 * m + 1] * inv),
                    pack_bf2(oacc[cb][4 * m + 2] * inv, oacc[cb][4 * m + 3] * inv)};
        *(u32x2*)(op + 32 * cb + 8 * m + 4 * g) = v2;
      }
  } else {
    const int prow = it.part + 32 * w + l32;
    float* po = a.part_o + (size_t)prow * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 v4 = {oacc[cb][4 * m], oacc[cb][4 * m + 1], oacc[cb][4 * m + 2], oacc[cb][4 * m + 3]};
        *(f32x4*)(po + 32 * cb + 8 * m + 4 * g) = v4;
      }
    if (g == 0) {
      a.part_ml[2 * (size_t)prow] = m_run;
      a.part_ml[2 * (size_t)prow + 1] = l_run;
    }
  }
}

// ---------------------------------------------------------------------------
// Segment-batch attention for the MLA row, direct-to-LDS (gfx950): K_nope
// (per head, DNOPE), K_pe (shared by the heads or per head, DPE) and V (per
// head, DV).  The math, lane layout and row DMA are those of k_seg_attn_dl
// (akv_attn_dl.hip);
// the K tile is held in two LDS parts (K_nope, then K_pe) and the S^T k-steps
// walk K_nope then K_pe, so Q rows are [q_nope | q_pe].  A 64-key stage holds
// 40 KiB of K and V, so three stages fit in LDS: tile t goes to stage t % 3
// and its slots to ring entry t % 3.  With three stages the scores are not
// computed a tile ahead (that would leave one iteration to land each tile):
// iteration j waits for tile j's rows (issued at iteration j - 2; iteration
// j - 1's loads stay in flight), barrier, issues tile j + 2's rows into tile
// j - 1's stage and tile j + 4's slots into tile j + 1's ring entry, then
// runs S, softmax and PV of tile j; the two waves of a SIMD overlap each
// other's matrix and vector work.
// ---------------------------------------------------------------------------
template <int DNOPE, int DPE, int DV>
__global__ __launch_bounds__(512, 1) void k_seg_attn_mla(AttnArgs a) {
  constexpr int NW = 8;
  constexpr int DQK = DNOPE + DPE;
  constexpr int RB = 32 * NW;
  constexpr int KT = ATTN_KTILE;
  constexpr int NKS = DQK / 16, NKN = DNOPE / 16;
  constexpr int NCB = DV / 32;
  constexpr int CHN = DNOPE / 8, CHP = DPE / 8, CHV = DV / 8;
  using PN = LdsPart<CHN, 16>;
  using PP = LdsPart<CHP, 16>;
  using PV = LdsPart<CHV, 64>;
  constexpr int OP = PN::BYTES, OV = PN::BYTES + PP::BYTES;
  constexpr int SSTAGE = OV + PV::BYTES;
  static_assert(KT == 64 && CHN % NW == 0 && CHP % NW == 0 && CHV % NW == 0 && 64 % CHP == 0,
                "blocks per wave");
  constexpr int NIW = (CHN + CHP + CHV) / NW;          // row loads per wave per tile
  static_assert(NIW + 1 <= 15, "vmcnt");
  __shared__ __attribute__((aligned(16))) unsigned char st0[SSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[SSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[SSTAGE];
  __shared__ __attribute__((aligned(16))) int32_t sr0[NW * 64];
  __shared__ __attribute__((aligned(16))) int32_t sr1[NW * 64];
  __shared__ __attribute__((aligned(16))) int32_t sr2[NW * 64];

  const AttnItem it = a.items[blockIdx.x];
  if (it.seg < 0) return;
  const AttnSeg sg = a.segs[it.seg];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), g = lane >> 5, l32 = lane & 31;
  const int G = a.group;
  const int lq = sg.q_len, lkv = sg.lkv;
  const int rows_total = lq * G;
  const int brow_last = min(it.row0 + RB, rows_total) - 1;
  const int lim_first = lkv - lq + it.row0 / G;
  const int lim_last = lkv - lq + brow_last / G;
  const int k_end = it.k_end;
  const int k_stop = min(k_end, lim_last + 1);
  const int n_tiles = k_stop > it.k_begin ? (k_stop - it.k_begin + KT - 1) / KT : 0;
  const int Hkv = a.n_kv_heads, S = a.page_size, lg = a.log2_page;
  const int kvh = it.kvh;
  const int32_t* __restrict__ slots = a.slots + sg.list_off;
  const int HS = Hkv * S, hoff = kvh * S;
  const int HP = a.kpe_heads * S, hpoff = (a.kpe_heads > 1 ? kvh : 0) * S;

  const int r0 = it.row0 + 32 * w + l32;
  const bool valid = r0 < rows_total;
  const int tok = valid ? r0 / G : 0;
  const int hq = kvh * G + (valid ? r0 - tok * G : 0);
  const int lim = valid ? min(lkv - lq + tok, k_end - 1) : k_stop - 1;
  bf16x8 qf[NKS];
  {
    const uint16_t* qp = a.q + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (valid) {
        qf[ks] = *(const bf16x8*)(qp + 16 * ks);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qf[ks] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  auto stage_ptr = [&](int s) __attribute__((always_inline)) -> unsigned char AKV_LDS* {
    return (unsigned char AKV_LDS*)(s == 0 ? st0 : (s == 1 ? st1 : st2));
  };
  auto ring_ptr = [&](int e) __attribute__((always_inline)) -> int32_t AKV_LDS* {
    int32_t* r = e == 0 ? sr0 : (e == 1 ? sr1 : sr2);
    return (int32_t AKV_LDS*)r + 64 * w;
  };
  auto slot_load = [&](int e, int t) __attribute__((always_inline)) {
    const int idx = min(it.k_begin + t * KT + lane, lkv - 1);
    __builtin_amdgcn_global_load_lds(slots + idx, (void AKV_LDS*)ring_ptr(e), 4, 0, 0);
  };
  // Row loads of one tile: this wave's blocks b = w + NW m of each part;
  // lane holds key b + CH (lane / CH), chunk lane % CH of the part.
  auto issue_tile = [&](unsigned char AKV_LDS* stg, int e) __attribute__((always_inline)) {
    const int32_t AKV_LDS* ring = ring_ptr(e);
#pragma unroll
    for (int m = 0; m < CHN / NW; ++m) {
      const int b = w + NW * m, c = lane % CHN;
      const int slot = ring[b + CHN * (lane / CHN)];
      const uint32_t row = __umul24(slot >> lg, HS) + hoff + (slot & (S - 1));
      __builtin_amdgcn_global_load_lds(a.k_a + (size_t)row * DNOPE + 8 * c, (void AKV_LDS*)(stg + b * PN::BLK),
                                       16, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < CHP / NW; ++m) {
      const int b = w + NW * m, c = lane % CHP;
      const int slot = ring[b + CHP * (lane / CHP)];
      const uint32_t row = __umul24(slot >> lg, HP) + hpoff + (slot & (S - 1));
      __builtin_amdgcn_global_load_lds(a.k_b + (size_t)row * DPE + 8 * c, (void AKV_LDS*)(stg + OP + b * PP::BLK),
                                       16, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < CHV / NW; ++m) {
      const int b = w + NW * m, c = lane % CHV;
      const int slot = ring[b + CHV * (lane / CHV)];
      const uint32_t row = __umul24(slot >> lg, HS) + hoff + (slot & (S - 1));
      __builtin_amdgcn_global_load_lds(a.v + (size_t)row * DV + 8 * c, (void AKV_LDS*)(stg + OV + b * PV::BLK),
                                       16, 0, 0);
    }
  };

  f32x16 oacc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2e;
  int koffN[2], koffP[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    koffN[kb] = PN::off(32 * kb + l32, g);
    koffP[kb] = OP + PP::off(32 * kb + l32, g);
  }
  const int qq = lane >> 4, ii = lane & 15;
  const int voff0 = OV + PV::off(4 * g + (ii >> 2), 0) + 2 * (16 * (qq & 1) + 4 * (ii & 3));

  auto qk = [&](const unsigned char AKV_LDS* stg, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        af[kb] = ks < NKN ? *(const bf16x8 AKV_LDS*)(stg + koffN[kb] + 32 * ks)
                          : *(const bf16x8 AKV_LDS*)(stg + koffP[kb] + 32 * (ks - NKN));
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], qf[ks], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], qf[ks], sacc[1], 0, 0, 0);
    }
  };
  auto sm_mask = [&](f32x16 (&sacc)[2], int j) __attribute__((always_inline)) {
    const int k0 = it.k_begin + j * KT;
    if ((k0 + KT > k_end) || (k0 + KT - 1 > lim_first)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key > lim) sacc[kb][i] = -INFINITY;
        }
    }
  };
  auto sm_max = [&](const f32x16 (&sacc)[2]) __attribute__((always_inline)) -> float {
    float m = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, sacc[kb][i]);
    return max_xor32(m);
  };
  auto sm_rescale = [&](float mx, int j) __attribute__((always_inline)) -> float {
    const float m_cand = fmaxf(m_run, mx * c2);
    if (__ballot(m_cand > m_run + RESCALE_LOG2)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
      l_run *= alpha;
      if (j > 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[cb][i] *= alpha;
      }
      m_run = m_cand;
    }
    return (m_run == -INFINITY) ? 0.f : m_run;
  };
  auto sm_exp = [&](const f32x16 (&sacc)[2], float m_use, bf16x8 (&pf)[4]) __attribute__((always_inline)) {
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb = t >> 1, q0 = 8 * (t & 1);
      u32x4 pk;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][q0 + 2 * k], c2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][q0 + 2 * k + 1], c2, -m_use));
        rs += p0 + p1;
        pk[k] = pack_bf2(p0, p1);
      }
      pf[t] = __builtin_bit_cast(bf16x8, pk);
    }
    l_run += rs;
  };
  auto pv = [&](const unsigned char AKV_LDS* stg, const bf16x8 (&pf)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const unsigned char AKV_LDS* vp = stg + voff0 + 2 * 32 * cb;
        const int kA = 16 * t, kB = 16 * t + 8;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 AKV_LDS*)(vp + (kA % CHV) * PV::BLK + (kA / CHV) * (CHV * 16)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 AKV_LDS*)(vp + (kB % CHV) * PV::BLK + (kB / CHV) * (CHV * 16)));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[t], oacc[cb], 0, 0, 0);
      }
    }
  };

#pragma unroll
  for (int t = 0; t < 3; ++t) slot_load(t, t);
  __builtin_amdgcn_s_waitcnt(0);
  issue_tile(stage_ptr(0), 0);
  issue_tile(stage_ptr(1), 1);
  slot_load(0, 3);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool idle = it.row0 + 32 * w >= rows_total;
  // iteration j: tile j landed at iteration j - 2; iteration j - 1's loads
  // (NIW rows + 1 slot load) may still be in flight
  constexpr int WAITV = NIW + 1;
  constexpr int WAIT_SYNC = (WAITV & 0xF) | ((WAITV >> 4) << 14) | (0x7 << 4);
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(WAIT_SYNC);
    __builtin_amdgcn_s_barrier();
  };
  const int lmask = min(k_end, lim_first + 1) - it.k_begin;
  const int jm = lmask > 0 ? lmask / KT : 0;
  auto iter = [&](int j, auto c, auto masked) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    sync();
    issue_tile(stage_ptr((C + 2) % 3), (C + 2) % 3);
    slot_load((C + 1) % 3, j + 4);
    f32x16 sc[2];
    qk(stage_ptr(C), sc);
    if constexpr (decltype(masked)::value) sm_mask(sc, j);
    const float m_use = sm_rescale(sm_max(sc), j);
    bf16x8 pf[4];
    sm_exp(sc, m_use, pf);
    pv(stage_ptr(C), pf);
  };
  auto idle_iter = [&](int j, auto c) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    sync();
    issue_tile(stage_ptr((C + 2) % 3), (C + 2) % 3);
    slot_load((C + 1) % 3, j + 4);
  };
  using J0 = std::integral_constant<int, 0>;
  using J1 = std::integral_constant<int, 1>;
  using J2 = std::integral_constant<int, 2>;
  using TF = std::false_type;
  using TT = std::true_type;
  int j = 0;
  if (idle) {
    for (; j < n_tiles; j += 3) {
      idle_iter(j, J0{});
      idle_iter(j + 1, J1{});
      idle_iter(j + 2, J2{});
    }
  } else {
    for (; j + 3 <= jm; j += 3) {
      iter(j, J0{}, TF{});
      iter(j + 1, J1{}, TF{});
      iter(j + 2, J2{}, TF{});
    }
    for (; j < n_tiles; j += 3) {
      iter(j, J0{}, TT{});
      iter(j + 1, J1{}, TT{});
      iter(j + 2, J2{}, TT{});
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

  const float l = sum_xor32(l_run);
  if (!valid) return;
  if (it.part < 0) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = a.out + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u32x2 v2 = {pack_bf2(oacc[cb][4 * m] * inv, oacc[cb][4 * m + 1] * inv),
                    pack_bf2(oacc[cb][4 * m + 2] * inv, oacc[cb][4 * m + 3] * inv)};
        *(u32x2*)(op + 32 * cb + 8 * m + 4 * g) = v2;
      }
  } else {
    const int prow = it.part + 32 * w + l32;
    float* po = a.part_o + (size_t)prow * DV;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 v4 = {oacc[cb][4 * m], oacc[cb][4 * m + 1], oacc[cb][4 * m + 2], oacc[cb][4 * m + 3]};
        *(f32x4*)(po + 32 * cb + 8 * m + 4 * g) = v4;
      }
    if (g == 0) {
      a.part_ml[2 * (size_t)prow] = m_run;
      a.part_ml[2 * (size_t)prow + 1] = l;
    }
  }
}

// Split-KV merge: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j (m in log2
// units).  One wave per row, four rows per block, so every row of every item
// is its own wave: lane j holds split j's (m, l) (the planner splits at most
// 64 ways), the row max and the weighted l come from wave reductions, and the
// lanes split the d_v columns with all splits' loads in flight together.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int DV>
__global__ __launch_bounds__(256) void k_combine(AttnArgs a, const CombItem* __restrict__ items,
                                                  int blocks_per_item) {
  constexpr int PER = DV / 64 > 0 ? DV / 64 : 1;
  const CombItem it = items[blockIdx.x / blocks_per_item];
  const int lane = threadIdx.x & 63;
  const int rl = (blockIdx.x % blocks_per_item) * 4 + (threadIdx.x >> 6);
  const AttnSeg sg = a.segs[it.seg];
  const int G = a.group;
  const int r = it.row0 + rl;
  if (rl >= a.rows_per_block || r >= sg.q_len * G) return;
  const int ns = it.nsplit;
  float mj = -INFINITY, lj = 0.f;
  if (lane < ns) {
    const size_t prow = (size_t)it.part0 + (size_t)lane * it.rows + rl;
    mj = a.part_ml[2 * prow];
    lj = a.part_ml[2 * prow + 1];
  }
  const float M = wave_max(mj);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float wj = lane < ns ? __builtin_amdgcn_exp2f(mj - Mu) : 0.f;
  const float L = wave_sum(wj * lj);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  // eight splits per round, their loads issued together (splits past ns
  // re-read the last one with weight 0)
  for (int j0 = 0; j0 < ns; j0 += 8) {
    float x[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, ns - 1);
      const float* po = a.part_o + ((size_t)it.part0 + (size_t)j * it.rows + rl) * DV;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int c = lane + 64 * e;
        x[u][e] = c < DV ? po[c] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wb = j0 + u < ns ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j0 + u)) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += wb * x[u][e];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  const int tok = r / G, hq = it.kvh * G + (r - tok * G);
  if (a.lse && lane == 0)
    a.lse[(size_t)(sg.q_begin + tok) * a.n_q_heads + hq] = L > 0.f ? Mu + __log2f(L) : INFINITY;
  uint16_t* op = a.out + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DV;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int c = lane + 64 * e;
    if (c < DV) {
      const __bf16 bv = (__bf16)(acc[e] * inv);
      op[c] = __builtin_bit_cast(uint16_t, bv);
    }
  }
}

// ---------------------------------------------------------------------------
// Static workspace for callers that cannot allocate (akv_segment_attention_static):
// a file-scope device array of fixed size.  Each GPU holds its own copy from
// the moment the library's code object is loaded on it until the process
// ends.  On the host the array's name is only a stand-in for the symbol, so
// its device address is looked up once per device (with that device
// current) and every kernel argument, copy or fill uses that address.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[STATIC_WORKSPACE_BYTES];

hipError_t static_workspace(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

bool attn_dims_supported(int d_nope, int d_rope, int d_v) {
  if (d_nope == 0) return (d_rope == 32 || d_rope == 64 || d_rope == 128) && d_v == d_rope;
  return (d_nope == 128 && d_rope == 64 && d_v == 128) || (d_nope == 32 && d_rope == 32 && d_v == 32);
}

// Every attention block holds 8 waves (256 packed rows, one block per CU, two
// waves per SIMD).
int attn_rows_per_block(int) { return 256; }

template <int DQK, int DV, int DNOPE>
static hipError_t launch_attn_t(hipStream_t st, const AttnArgs& a) {
  if constexpr (DQK == 128 && DV == 128 && DNOPE == 0) {
    // the 128-dim GQA layout: direct-to-LDS pipeline (akv_attn_dl.hip)
    return launch_seg_attn_dl(st, a);
  } else if constexpr (DNOPE == 128 && DQK == 192 && DV == 128) {
    // the MLA row (K_nope 128, K_pe 64, V 128): direct-to-LDS, three stages
    launch_k(k_seg_attn_mla<128, 64, 128>, dim3(a.n_items), dim3(512), st, a);
  } else {
    launch_k(k_seg_attn<DQK, DV, DNOPE, 8>, dim3(a.n_items), dim3(512), st, a);
  }
  return hipGetLastError();
}

hipError_t launch_seg_attn(hipStream_t st, const AttnArgs& a, int d_nope, int d_rope, int d_v) {
  if (a.n_items <= 0) return hipSuccess;
  if (d_nope == 0) {
    if (d_rope == 128 && d_v == 128) return launch_attn_t<128, 128, 0>(st, a);
    if (d_rope == 64 && d_v == 64) return launch_attn_t<64, 64, 0>(st, a);
    if (d_rope == 32 && d_v == 32) return launch_attn_t<32, 32, 0>(st, a);
  } else {
    if (d_nope == 128 && d_rope == 64 && d_v == 128) return launch_attn_t<192, 128, 128>(st, a);
    if (d_nope == 32 && d_rope == 32 && d_v == 32) return launch_attn_t<64, 32, 32>(st, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(hipStream_t st, const AttnArgs& a, const CombItem* items, int n_items,
                          int d_v) {
  if (n_items <= 0) return hipSuccess;
  const int bpi = (a.rows_per_block + 3) / 4;
  const dim3 grid((unsigned)(n_items * bpi));
  switch (d_v) {
    case 128: launch_k(k_combine<128>, grid, dim3(256), st, a, items, bpi); break;
    case 64: launch_k(k_combine<64>, grid, dim3(256), st, a, items, bpi); break;
    case 32: launch_k(k_combine<32>, grid, dim3(256), st, a, items, bpi); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace akv
