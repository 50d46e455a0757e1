// Segment-batch attention for the 128-dim GQA layout, direct-to-LDS (gfx950).
//
// Sources, cited by page title and section:
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents and State-Preserving
//               Prefix Invalidation Bypass" (A. Akhunji)
//   [AKV-notes] "Cache Engineering for Agents" (reading notes on Fu et al.)
//
// Built on its own with the compiler's max-ILP machine scheduler (see the
// build script): the main loop's MFMA, LDS and vector work interleave better
// under it, while the MLA kernel runs slower with it.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "akv_device.h"
#include "akv_internal.h"
#include "akv_launch.h"

namespace akv {

// ---------------------------------------------------------------------------
// Segment-batch attention, direct-to-LDS variant (gfx950).
//
// Same math and lane layout as k_seg_attn; the K/V gather goes straight from
// global memory into LDS with global_load_lds_dwordx4 (16 bytes per lane, lane
// l lands at base + 16 l), NST tiles deep, so no registers stage the tiles and
// no vector instructions write LDS.  Each tile stage is its own LDS array so
// the compiler keeps reads of one stage independent of loads into another.
// The slot indices of a tile's 64 keys reach LDS the same way (4 bytes per
// lane, into a per-wave ring), so every vector-memory instruction of the main
// loop is an LDS load of fixed count and the waits below can be counted.
//
// LDS layout of a part with CH 16-byte chunks per key row (K, K_pe or V): the
// 64 keys of a tile form CH blocks of 1 KiB (one load instruction each); block
// b holds keys r = b + CH*i (i = 0 .. 64/CH-1), row after row, and blocks are
// padded (16 B for K, 64 B for V) so the fragment reads below spread over the
// banks.  K fragments are plain 16-byte reads; V^T fragments come from two
// ds_read_b64_tr_b16 per fragment: within each 16-lane group the transposing
// read hands lane i the elements V[K0 + k][C0 + i], k = 0..3, when lane
// 4k + j points at V[K0 + k][C0 + 4j .. 4j + 3].
// ---------------------------------------------------------------------------

// ROT: keys may owe a rotation (deferred repos, [AKV-blog] section 4 and rule
// of thumb 2: turn the key where it is read).  Every list entry carries the
// row of the cos / sin table that turns its stored key to its position, or
// -1.  Each landed K tile is turned once, in LDS, by the whole block before
// any wave reads it: wave w takes rotation pairs 8w .. 8w + 7 of every key
// (lane = key), with the table row read through the scalar cache, one
// distinct row at a time, and the formula of the in-place repos, so the
// scores equal those of keys rotated in place bit for bit.
template <int DQK, int DV, int DNOPE, int NW, int QB, int NST, bool ROT>
__global__ __launch_bounds__(64 * NW, 1) void k_seg_attn_dl(AttnArgs a) {
  constexpr int RB = 32 * QB * NW;
  constexpr int KT = ATTN_KTILE;
  constexpr int NKS = DQK / 16;
  constexpr int NCB = DV / 32;
  constexpr int CH = DQK / 8;                           // 16-byte chunks per K (and V) row
  using PA = LdsPart<CH, 16>;
  using PV = LdsPart<CH, 64>;
  constexpr int SA = PA::BYTES, SV = PV::BYTES;
  constexpr int SSTAGE = SA + SV;
  constexpr int NBW = CH / NW;                          // K/V blocks loaded by each wave
  constexpr int NIW = 2 * NBW;                          // row loads per wave per tile
  static_assert(DNOPE == 0 && DQK == DV, "one K part with V's row size");
  static_assert(KT == 64 && 64 % CH == 0 && CH % NW == 0, "tile");
  static_assert(NST == 4, "the unrolled pipeline below is written for four stages");
  static_assert(!ROT || (NW == 8 && DQK == 128), "the in-LDS rotation maps wave w to pairs 8w .. 8w + 7");
  constexpr int WAIT_LDS = 0xF | (0x3 << 14) | (0x7 << 4);                        // lgkmcnt(0) only

  __shared__ __attribute__((aligned(16))) unsigned char st0[SSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st1[SSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st2[SSTAGE];
  __shared__ __attribute__((aligned(16))) unsigned char st3[SSTAGE];
  // per-wave slot ring: entry e holds the 64 slots of tile t, t % 4 == e
  // (ROT: then the tile's 64 rotation-table rows, in the same array, so the
  // compiler's wait tracking still sees eight LDS targets of the DMA)
  constexpr int RING = (ROT ? 2 : 1) * NW * 64;
  __shared__ __attribute__((aligned(16))) int32_t sr0[RING];
  __shared__ __attribute__((aligned(16))) int32_t sr1[RING];
  __shared__ __attribute__((aligned(16))) int32_t sr2[RING];
  __shared__ __attribute__((aligned(16))) int32_t sr3[RING];

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
  const int HS = Hkv * S;
  const int hoff = kvh * S;

  bool valid[QB];
  int tok[QB], hq[QB], lim[QB];
  bf16x8 qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = it.row0 + 32 * (QB * w + qb) + l32;
    valid[qb] = r < rows_total;
    tok[qb] = valid[qb] ? r / G : 0;
    hq[qb] = kvh * G + (valid[qb] ? r - tok[qb] * G : 0);
    lim[qb] = valid[qb] ? min(lkv - lq + tok[qb], k_end - 1) : k_stop - 1;
    const uint16_t* qp = a.q + ((size_t)(sg.q_begin + tok[qb]) * a.n_q_heads + hq[qb]) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (valid[qb]) {
        qf[qb][ks] = *(const bf16x8*)(qp + 16 * ks);
      } else {
        u32x4 z = {0u, 0u, 0u, 0u};
        qf[qb][ks] = __builtin_bit_cast(bf16x8, z);
      }
    }
  }

  // Slots of tile t (list entries k_begin + 64 t ..) into this wave's part of
  // a ring entry; entries past the list end repeat its last slot.
  auto ring_ptr = [&](int e) __attribute__((always_inline)) -> int32_t AKV_LDS* {
    int32_t* r = e == 0 ? sr0 : (e == 1 ? sr1 : (e == 2 ? sr2 : sr3));
    return (int32_t AKV_LDS*)r + 64 * w;
  };
  auto dring_ptr = [&](int e) __attribute__((always_inline)) -> int32_t AKV_LDS* {
    int32_t* r = e == 0 ? sr0 : (e == 1 ? sr1 : (e == 2 ? sr2 : sr3));
    return (int32_t AKV_LDS*)r + NW * 64 + 64 * w;
  };
  auto slot_load = [&](int e, int t) __attribute__((always_inline)) {
    const int idx = min(it.k_begin + t * KT + lane, lkv - 1);
    __builtin_amdgcn_global_load_lds(slots + idx, (void AKV_LDS*)ring_ptr(e), 4, 0, 0);
    if constexpr (ROT)
      __builtin_amdgcn_global_load_lds(a.key_didx + sg.list_off + idx, (void AKV_LDS*)dring_ptr(e), 4, 0, 0);
  };
  // Turn the owed keys of the K tile in stage stg (di: this lane's key's
  // table row, read from the ring before the ring entry is reloaded).  With
  // with_barrier, a barrier follows so every wave reads turned keys; in the
  // loop the next iteration's barrier publishes them instead.  Skipped when
  // no key of the tile owes a rotation (the same decision in every wave:
  // each holds the tile's 64 rows).
  auto rotate_tile = [&](unsigned char AKV_LDS* stg, int di, auto with_barrier) __attribute__((always_inline)) {
    if constexpr (ROT) {
      uint64_t todo = __ballot(di >= 0);
      if (todo == 0) return;
      const int c0 = a.rot_pairing == 0 ? 2 * w : w;
      const int c1 = a.rot_pairing == 0 ? 2 * w + 1 : w + 8;
      u32x4 AKV_LDS* p0 = (u32x4 AKV_LDS*)(stg + PA::off(lane, c0));
      u32x4 AKV_LDS* p1 = (u32x4 AKV_LDS*)(stg + PA::off(lane, c1));
      const u32x4 x0 = *p0, x1 = *p1;
      u32x4 o0 = x0, o1 = x1;
      while (todo) {
        const int d0 = __builtin_amdgcn_readlane(di, __builtin_ctzll(todo));
        const float* row = a.rot_table + (size_t)d0 * DQK + 8 * w;
        const f32x8 cs = scalar_load8(row);
        const f32x8 sn = scalar_load8(row + DQK / 2);
        const bool mine = di == d0;
        if (mine) {
          if (a.rot_pairing == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              o0[k] = rot_pair_word(x0[k], cs[k], sn[k]);
              o1[k] = rot_pair_word(x1[k], cs[4 + k], sn[4 + k]);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float xa = bf_lo(x0[k]), xb = bf_hi(x0[k]);
              const float ya = bf_lo(x1[k]), yb = bf_hi(x1[k]);
              o0[k] = pack_bf2(fmaf(xa, cs[2 * k], -ya * sn[2 * k]), fmaf(xb, cs[2 * k + 1], -yb * sn[2 * k + 1]));
              o1[k] = pack_bf2(fmaf(xa, sn[2 * k], ya * cs[2 * k]), fmaf(xb, sn[2 * k + 1], yb * cs[2 * k + 1]));
            }
          }
        }
        todo &= ~__ballot(mine);
      }
      *p0 = o0;
      *p1 = o1;
      if constexpr (decltype(with_barrier)::value) {
        __builtin_amdgcn_s_waitcnt(WAIT_LDS);
        __builtin_amdgcn_s_barrier();
      }
    }
  };
  auto ring_didx = [&](int e) __attribute__((always_inline)) -> int {
    if constexpr (ROT) {
      const int d = dring_ptr(e)[lane];
      // read before this wave's next slot load rewrites the entry
      __builtin_amdgcn_s_waitcnt(WAIT_LDS);
      return d;
    }
    return -1;
  };
  // Row loads of one tile: this wave's blocks b = w + NW m; lane holds key
  // b + CH (lane / CH), chunk lane % CH, of both K and V.
  auto issue_tile = [&](unsigned char AKV_LDS* stg, int e) __attribute__((always_inline)) {
    const int32_t AKV_LDS* ring = ring_ptr(e);
#pragma unroll
    for (int m = 0; m < NBW; ++m) {
      const int b = w + NW * m, c = lane % CH;
      const int slot = ring[b + CH * (lane / CH)];
      const int page = slot >> lg, off = slot & (S - 1);
      const uint32_t row = __umul24(page, HS) + hoff + off;
      __builtin_amdgcn_global_load_lds(a.k_a + (size_t)row * DQK + 8 * c,
                                       (void AKV_LDS*)(stg + b * PA::BLK), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.v + (size_t)row * DV + 8 * c,
                                       (void AKV_LDS*)(stg + SA + b * PV::BLK), 16, 0, 0);
    }
  };

  f32x16 oacc[QB][NCB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[qb][cb][i] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float c2 = a.scale_log2e;

  // per-lane fragment offsets
  int koffA[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) koffA[kb] = PA::off(32 * kb + l32, g);
  const int qq = lane >> 4, ii = lane & 15;
  // V^T reads: lane points at key 4g + ii/4 (+ 8h + 16t), column 16(qq&1) + 4(ii&3) (+ 32cb)
  const int voff0 = SA + PV::off(4 * g + (ii >> 2), 0) + 2 * (16 * (qq & 1) + 4 * (ii & 3));

  // S^T = K Q^T for one tile (raw scores, fp32).
  auto qk = [&](const unsigned char AKV_LDS* stg, f32x16 (&sacc)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[qb][kb][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 af[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        af[kb] = *(const bf16x8 AKV_LDS*)(stg + koffA[kb] + 32 * ks);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        sacc[qb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], qf[qb][ks], sacc[qb][0], 0, 0, 0);
        sacc[qb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[1], qf[qb][ks], sacc[qb][1], 0, 0, 0);
      }
    }
  };

  // Causal / range mask of tile j (taken only on tiles that reach past a
  // row's limit or the item's key range).
  auto sm_mask = [&](f32x16 (&sacc)[QB][2], int j) __attribute__((always_inline)) {
    const int k0 = it.k_begin + j * KT;
    if ((k0 + KT > k_end) || (k0 + KT - 1 > lim_first)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > lim[qb]) sacc[qb][kb][i] = -INFINITY;
          }
    }
  };
  // Row max of tile j's scores (both lane halves of a row agree).
  auto sm_max = [&](const f32x16 (&sacc)[QB][2], float (&mx)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, sacc[qb][kb][i]);
      mx[qb] = max_xor32(m);
    }
  };
  // Lazy rescale: move the running offset only when the max grew by more
  // than 2^RESCALE_LOG2; returns the exponent offset of each row block.
  auto sm_rescale = [&](const float (&mx)[QB], int j, float (&m_use)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_cand = fmaxf(m_run[qb], mx[qb] * c2);
      if (__ballot(m_cand > m_run[qb] + RESCALE_LOG2)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_cand);
        l_run[qb] *= alpha;
        if (j > 0) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[qb][cb][i] *= alpha;
        }
        m_run[qb] = m_cand;
      }
      m_use[qb] = (m_run[qb] == -INFINITY) ? 0.f : m_run[qb];
    }
  };

  // P = 2^(S c2 - m) in bf16 and the row sums (branch free).
  auto sm_exp = [&](const f32x16 (&sacc)[QB][2], const float (&m_use)[QB], bf16x8 (&pf)[QB][4])
      __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float rs = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kb = t >> 1, r0 = 8 * (t & 1);
        u32x4 pk;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][r0 + 2 * k], c2, -m_use[qb]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[qb][kb][r0 + 2 * k + 1], c2, -m_use[qb]));
          rs += p0 + p1;
          pk[k] = pack_bf2(p0, p1);
        }
        pf[qb][t] = __builtin_bit_cast(bf16x8, pk);
      }
      l_run[qb] += rs;
    }
  };

  // O^T += V^T P^T for the tile in stage stg.
  auto pv = [&](const unsigned char AKV_LDS* stg, const bf16x8 (&pf)[QB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const unsigned char AKV_LDS* vp = stg + voff0 + 2 * 32 * cb;
        const int kA = 16 * t, kB = 16 * t + 8;   // key offsets of the two halves
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 AKV_LDS*)(vp + (kA % CH) * PV::BLK + (kA / CH) * (CH * 16)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (s16x4 AKV_LDS*)(vp + (kB % CH) * PV::BLK + (kB / CH) * (CH * 16)));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, v8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][t], oacc[qb][cb], 0, 0, 0);
      }
    }
  };

  // Pipeline.  Tile t's rows go to stage t % 4, its slots to ring entry
  // t % 4.  The scores of tile j + 1 are computed before the softmax of tile
  // j, so the matrix cores work on them while the vector units run the
  // softmax.  Iteration j: wait for this wave's loads of iteration j - 2 and
  // earlier, barrier (every wave's rows of tile j + 1 are in LDS, and every
  // wave is done with tile j - 1), issue the rows of tile j + 3 into tile
  // j - 1's stage (their slots came in at iteration j - 2) and the slots of
  // tile j + 5 into tile j + 1's ring entry (read at iteration j - 2), then
  // S(j + 1) and softmax / PV of tile j.  Loads past the list end are
  // clamped (in bounds); extra tiles past the range are fully masked.
  // ROT: iteration j also turns tile j + 2 (issued at iteration j - 1, so the
  // wait covers every row load but the last iteration's slot loads); the
  // barrier of iteration j + 1 publishes the turned keys before S(j + 2).
  auto stage_ptr = [&](int s) __attribute__((always_inline)) -> unsigned char AKV_LDS* {
    return (unsigned char AKV_LDS*)(s == 0 ? st0 : (s == 1 ? st1 : (s == 2 ? st2 : st3)));
  };
#pragma unroll
  for (int t = 0; t < 4; ++t) slot_load(t, t);
  __builtin_amdgcn_s_waitcnt(0);
  const int di0 = ring_didx(0);
#pragma unroll
  for (int t = 0; t < 3; ++t) issue_tile(stage_ptr(t), t);
  slot_load(0, 4);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int di1 = ring_didx(1);
  rotate_tile(stage_ptr(0), di0, std::false_type{});
  rotate_tile(stage_ptr(1), di1, std::true_type{});
  // A wave whose rows all lie past the segment's last row (a short segment's
  // padding) computes nothing: it keeps its share of the tile loads and every
  // barrier, and leaves its SIMD's matrix core to the other wave there.
  const bool idle = it.row0 + 32 * QB * w >= rows_total;
  f32x16 sa[QB][2], sb[QB][2];
  if (!idle) qk(stage_ptr(0), sa);

  // All of iteration j - 2's loads have landed once at most one iteration's
  // worth (NIW rows + 1 slot load) is outstanding (ROT: iteration j - 1's
  // rows too, once only its two slot loads are).  The barrier carries no
  // memory fence: a workgroup fence would wait for every LDS load in flight,
  // tiles j + 2 and j + 3 included.  lgkmcnt(0) makes this wave's reads of
  // tile j - 1's stage complete before any wave reloads it.
  constexpr int WAITV = ROT ? 2 : NIW + 1;
  // s_waitcnt operands (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
  // 6:4, lgkmcnt 11:8), given through the builtin so the compiler's own wait
  // tracking knows them and adds no stricter wait of its own
  constexpr int WAIT_SYNC = (WAITV & 0xF) | ((WAITV >> 4) << 14) | (0x7 << 4);   // vmcnt(WAITV) lgkmcnt(0)
  static_assert(WAITV <= 15, "vmcnt");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(WAIT_SYNC);
    __builtin_amdgcn_s_barrier();
  };
  // Tiles j < jm need no mask (they end before every row's limit and before
  // the item's key range end).  The main loop runs while tiles j .. j + 4 are
  // all such tiles: its iteration is one basic block apart from the rare
  // rescale branch at the top (the row max of tile j + 1 is taken at the end
  // of iteration j).  The remaining tiles run in the masked loop.
  const int lmask = min(k_end, lim_first + 1) - it.k_begin;
  const int jm = lmask > 0 ? lmask / KT : 0;
  float mx[QB];
  auto main_iter = [&](int j, auto c, f32x16 (&s_cur)[QB][2], f32x16 (&s_nxt)[QB][2])
      __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;   // j % 4
    sync();
    float m_use[QB];
    sm_rescale(mx, j, m_use);
    const int di = ring_didx((C + 2) & 3);
    issue_tile(stage_ptr((C + 3) & 3), (C + 3) & 3);
    slot_load((C + 1) & 3, j + 5);
    rotate_tile(stage_ptr((C + 2) & 3), di, std::false_type{});
    qk(stage_ptr((C + 1) & 3), s_nxt);
    bf16x8 pf[QB][4];
    sm_exp(s_cur, m_use, pf);
    pv(stage_ptr(C), pf);
    sm_max(s_nxt, mx);
    // the compiler's small-GEMM interleave (two LDS reads per MFMA, the
    // vector work left free): fragment reads run ahead of the MFMAs that
    // take them (measured: 2% faster at the 64K step)
    __builtin_amdgcn_iglp_opt(0);
  };
  auto tail_iter = [&](int j, auto c, f32x16 (&s_cur)[QB][2], f32x16 (&s_nxt)[QB][2])
      __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    sync();
    const int di = ring_didx((C + 2) & 3);
    issue_tile(stage_ptr((C + 3) & 3), (C + 3) & 3);
    slot_load((C + 1) & 3, j + 5);
    rotate_tile(stage_ptr((C + 2) & 3), di, std::false_type{});
    float m_use[QB];
    bf16x8 pf[QB][4];
    sm_mask(s_cur, j);
    qk(stage_ptr((C + 1) & 3), s_nxt);
    sm_max(s_cur, mx);
    sm_rescale(mx, j, m_use);
    sm_exp(s_cur, m_use, pf);
    pv(stage_ptr(C), pf);
  };
  auto idle_iter = [&](int j, auto c) __attribute__((always_inline)) {
    constexpr int C = decltype(c)::value;
    sync();
    const int di = ring_didx((C + 2) & 3);
    issue_tile(stage_ptr((C + 3) & 3), (C + 3) & 3);
    slot_load((C + 1) & 3, j + 5);
    rotate_tile(stage_ptr((C + 2) & 3), di, std::false_type{});
  };
  int j = 0;
  if (idle) {
    // same number of iterations (and barriers) as the two loops below
    for (; j < n_tiles; j += 4) {
      idle_iter(j, I0{});
      idle_iter(j + 1, I1{});
      idle_iter(j + 2, I2{});
      idle_iter(j + 3, I3{});
    }
  } else {
    if (jm > 4) {
      sm_max(sa, mx);
      for (; j + 4 < jm; j += 4) {
        main_iter(j, I0{}, sa, sb);
        main_iter(j + 1, I1{}, sb, sa);
        main_iter(j + 2, I2{}, sa, sb);
        main_iter(j + 3, I3{}, sb, sa);
      }
    }
    for (; j < n_tiles; j += 4) {
      tail_iter(j, I0{}, sa, sb);
      tail_iter(j + 1, I1{}, sb, sa);
      tail_iter(j + 2, I2{}, sa, sb);
      tail_iter(j + 3, I3{}, sb, sa);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = sum_xor32(l_run[qb]);
    if (!valid[qb]) continue;
    if (it.part < 0) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* op = a.out + ((size_t)(sg.q_begin + tok[qb]) * a.n_q_heads + hq[qb]) * DV;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          u32x2 v2 = {pack_bf2(oacc[qb][cb][4 * m] * inv, oacc[qb][cb][4 * m + 1] * inv),
                      pack_bf2(oacc[qb][cb][4 * m + 2] * inv, oacc[qb][cb][4 * m + 3] * inv)};
          *(u32x2*)(op + 32 * cb + 8 * m + 4 * g) = v2;
        }
    } else {
      const int prow = it.part + 32 * (QB * w + qb) + l32;
      float* po = a.part_o + (size_t)prow * DV;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 v4 = {oacc[qb][cb][4 * m], oacc[qb][cb][4 * m + 1], oacc[qb][cb][4 * m + 2],
                      oacc[qb][cb][4 * m + 3]};
          *(f32x4*)(po + 32 * cb + 8 * m + 4 * g) = v4;
        }
      if (g == 0) {
        a.part_ml[2 * (size_t)prow] = m_run[qb];
        a.part_ml[2 * (size_t)prow + 1] = l;
      }
    }
  }
}

hipError_t launch_seg_attn_dl(hipStream_t st, const AttnArgs& a) {
  // keys owing a rotation are turned in LDS when the launch carries a
  // rotation table
  if (a.key_didx)
    launch_k(k_seg_attn_dl<128, 128, 0, 8, 1, 4, true>, dim3(a.n_items), dim3(512), st, a);
  else
    launch_k(k_seg_attn_dl<128, 128, 0, 8, 1, 4, false>, dim3(a.n_items), dim3(512), st, a);
  return hipGetLastError();
}

}  // namespace akv
