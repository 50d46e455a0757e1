// Decode attention (gfx950): segment-batch attention for work items of at most
// 16 packed rows (query tokens x q heads of one kv head), the decode side of
// the method ("Cache Engineering for Agents", section 3, Segment-Batch
// Attention: every segment runs causal attention over its own page list).
//
// Such an item reads its keys and values once and does 2 x 16 x 256 FLOP per
// key: the launch is bound by HBM, not by the matrix cores.  The block's four
// waves therefore split the item's key range (tile t goes to wave t % 4), each
// with its own online softmax, and merge through LDS at the end; a block holds
// no barrier in its key loop.  Each wave keeps up to two 32-key tiles of K
// and V in flight in its registers (issued two tiles ahead, from slot indices
// loaded two tiles before that), so a CU running two blocks has up to 256 KiB
// of loads in flight.
//
// Per tile and wave, with v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16):
//   S^T = K Q^T : A = K (lane: key l % 16 of a 16-key block, d 8g .. 8g+7 of a
//                 32-wide d step), B = Q^T (lane: row l % 16, same d slots);
//                 lane l receives row l % 16, keys 4g .. 4g+3 of the block.
//   O^T += V^T P^T : B = P^T is the lane's own scores (row l % 16; keys 4g+e
//                 of block 0 for e < 4, of block 1 for e >= 4); A = V^T comes
//                 from two ds_read_b64_tr_b16 of the tile staged in LDS (lane
//                 i of a 16-lane group receives V[K0 + k][C0 + i], k = 0..3,
//                 when lane 4k + j points at V[K0 + k][C0 + 4j]).
// The softmax is base 2 with a lazily moved reference max, as in the
// prefill kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "akv_device.h"
#include "akv_internal.h"
#include "akv_launch.h"

namespace akv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
#define DEC_LDS __attribute__((address_space(3)))

constexpr int DEC_WAVES = 4;
constexpr int DEC_KT = 32;                 // keys per tile
constexpr int DEC_D = 128;                 // d_qk = d_v
constexpr int DEC_KROW = 256 + 16;        // LDS K row (+ pad: 8 lanes' 16-byte reads span the banks)
constexpr int DEC_VBLK = 512 + 32;         // LDS V block: keys b, b+16 of a tile (2 x 256 B) + pad
constexpr int DEC_KTILE = DEC_KT * DEC_KROW;
constexpr int DEC_VTILE = 16 * DEC_VBLK;
constexpr int DEC_WTILE = DEC_KTILE + DEC_VTILE;   // one wave's staged K and V tile
constexpr float DEC_RESCALE_LOG2 = 8.f;

__device__ __forceinline__ unsigned pk_bf2(float a, float b) {
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(unsigned, v);
}

// Key rotation in registers, with the fp32 formula of the in-place repos:
// pair (x, y) -> (x cos - y sin, x sin + y cos), rounded once to bf16.
// Interleaved pairing: word e of w holds pair (x, y) with cos / sin cs[e],
// sn[e].
__device__ __forceinline__ void turn_interleaved(u32x4_t& w, const f32x4_t& cs, const f32x4_t& sn) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = __uint_as_float(w[e] << 16), y = __uint_as_float(w[e] & 0xffff0000u);
    w[e] = pk_bf2(fmaf(x, cs[e], -y * sn[e]), fmaf(x, sn[e], y * cs[e]));
  }
}

// Half-split pairing: xw holds the first elements of 8 pairs, yw their
// second elements; cos / sin of the 8 pairs in (c0, c1), (s0, s1).
__device__ __forceinline__ void turn_half(u32x4_t& xw, u32x4_t& yw, const f32x4_t& c0, const f32x4_t& c1,
                                          const f32x4_t& s0, const f32x4_t& s1) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float cA = e < 2 ? c0[2 * e] : c1[2 * e - 4], cB = e < 2 ? c0[2 * e + 1] : c1[2 * e - 3];
    const float sA = e < 2 ? s0[2 * e] : s1[2 * e - 4], sB = e < 2 ? s0[2 * e + 1] : s1[2 * e - 3];
    const float x0 = __uint_as_float(xw[e] << 16), x1 = __uint_as_float(xw[e] & 0xffff0000u);
    const float y0 = __uint_as_float(yw[e] << 16), y1 = __uint_as_float(yw[e] & 0xffff0000u);
    xw[e] = pk_bf2(fmaf(x0, cA, -y0 * sA), fmaf(x1, cB, -y1 * sB));
    yw[e] = pk_bf2(fmaf(x0, sA, y0 * cA), fmaf(x1, sB, y1 * cB));
  }
}

template <bool ROT>
__global__ __launch_bounds__(64 * DEC_WAVES, 2) void k_decode_attn(AttnArgs a) {
  // per wave: its staged V tile; after the key loop the same space holds the
  // waves' (m, l, O) for the merge
  __shared__ __attribute__((aligned(16))) unsigned char s_v[DEC_WAVES * DEC_WTILE];
  __shared__ float s_ml[DEC_WAVES][16][2];

  const AttnItem it = a.items[blockIdx.x];
  if (it.seg < 0) return;
  const AttnSeg sg = a.segs[it.seg];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, i16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.group, lq = sg.q_len, lkv = sg.lkv;
  const int rows_total = min(lq * G - it.row0, 16);
  const int k_end = it.k_end;
  const int lim_last = lkv - lq + (it.row0 + rows_total - 1) / G;
  const int lim_first = lkv - lq + it.row0 / G;
  const int k_stop = min(k_end, lim_last + 1);
  const int n_tiles = k_stop > it.k_begin ? (k_stop - it.k_begin + DEC_KT - 1) / DEC_KT : 0;
  const int n_loc = n_tiles > w ? (n_tiles - w + DEC_WAVES - 1) / DEC_WAVES : 0;
  const int S = a.page_size, lg = a.log2_page;
  const int HS = a.n_kv_heads * S, hoff = it.kvh * S;
  const int32_t* __restrict__ slots = a.slots + sg.list_off;

  // this lane's query row (row = lane % 16 of the item)
  const int row = i16;
  const bool valid = row < rows_total;
  const int tok = valid ? (it.row0 + row) / G : 0;
  const int hq = it.kvh * G + (valid ? (it.row0 + row) - tok * G : 0);
  const int lim = valid ? min(lkv - lq + tok, k_end - 1) : k_stop - 1;
  bf16x8_t qf[4];
  {
    const uint16_t* qp = a.q + ((size_t)(sg.q_begin + tok) * a.n_q_heads + hq) * DEC_D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t z = {0u, 0u, 0u, 0u};
      qf[ks] = __builtin_bit_cast(bf16x8_t, valid ? *(const u32x4_t*)(qp + 32 * ks) : z);
    }
  }

  unsigned char DEC_LDS* kl = (unsigned char DEC_LDS*)s_v + w * DEC_WTILE;
  unsigned char DEC_LDS* vl = kl + DEC_KTILE;
  // V^T fragment reads: lane i of group g points at key 4g + i/4 (+16 for the
  // second half), columns 4(i % 4) .. (+16 per 16-column block)
  const int tr_off = (4 * g + (i16 >> 2)) * DEC_VBLK + 8 * (i16 & 3);

  // slot of key `lane` of local tile j, clamped to the item's last key: the
  // tiles a wave loads past its range (the pipeline always runs two ahead)
  // read one row, which the caches serve
  const int k_clamp = max(k_stop - 1, 0);
  auto slot_of = [&](int j) __attribute__((always_inline)) -> int {
    const int k = it.k_begin + (w + DEC_WAVES * j) * DEC_KT + (lane & 31);
    return slots[min(k, k_clamp)];
  };
  // owed rotation (table row, or -1) of key `lane` of local tile j
  const int32_t* __restrict__ kdidx = ROT ? a.key_didx + sg.list_off : nullptr;
  auto didx_of = [&](int j) __attribute__((always_inline)) -> int {
    if constexpr (ROT) {
      const int k = it.k_begin + (w + DEC_WAVES * j) * DEC_KT + (lane & 31);
      return kdidx[min(k, k_clamp)];
    } else {
      return -1;
    }
  };
  // K and V rows of the tile whose slots `sv` holds: load b covers keys
  // 4b .. 4b+3, lane l taking chunk l % 16 of key 4b + l / 16, so each load
  // instruction reads whole 256-byte rows
  auto load_tile = [&](int sv, u32x4_t (&kr)[8], u32x4_t (&vr)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int s = __shfl(sv, 4 * b + g);
      const size_t base = ((size_t)(uint32_t)(__umul24(s >> lg, HS) + hoff + (s & (S - 1)))) * DEC_D + 8 * i16;
      kr[b] = *(const u32x4_t*)(a.k_a + base);
      vr[b] = *(const u32x4_t*)(a.v + base);
    }
  };

  f32x4_t oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2e;

  // first half of a tile: K and V rows into this wave's LDS tile (the
  // tile's registers are free afterwards), then S^T of the two 16-key blocks
  // from K fragments (lane: key 16kb + l%16, chunk 4c + g)
  // A key stored at an earlier position (deferred repos) is turned to its
  // own position in the lane's fragments, with the table row and the fp32
  // formula of the in-place repos, so the scores equal those of keys that
  // repos had rotated.  Fragment c of key 16kb + l%16 holds d = 32c + 8g ..
  // +7: interleaved pairs 16c + 4g .. +3; half-split pairs 32c + 8g .. +7 for
  // c < 2, whose second elements are fragment c + 2 of the same lane.
  auto turn_frags = [&](u32x4_t (&kf)[4], int dk) __attribute__((always_inline)) {
    if (dk < 0) return;
    const float* row = a.rot_table + (size_t)dk * DEC_D;
    if (a.rot_pairing == 0) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        turn_interleaved(kf[c], *(const f32x4_t*)(row + 16 * c + 4 * g),
                         *(const f32x4_t*)(row + DEC_D / 2 + 16 * c + 4 * g));
    } else {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float* hr = row + 32 * c + 8 * g;
        turn_half(kf[c], kf[c + 2], *(const f32x4_t*)hr, *(const f32x4_t*)(hr + 4),
                  *(const f32x4_t*)(hr + DEC_D / 2), *(const f32x4_t*)(hr + DEC_D / 2 + 4));
      }
    }
  };
  auto tile_front = [&](const u32x4_t (&kr)[8], const u32x4_t (&vr)[8], f32x4_t (&s)[2], int dv)
      __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int r = 4 * b + g;
      *(u32x4_t DEC_LDS*)(kl + r * DEC_KROW + 16 * i16) = kr[b];
      *(u32x4_t DEC_LDS*)(vl + (r & 15) * DEC_VBLK + (r >> 4) * 256 + 16 * i16) = vr[b];
    }
    // the rows written above are read back by other lanes of this wave
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4_t kf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kf[c] = *(const u32x4_t DEC_LDS*)(kl + (16 * kb + i16) * DEC_KROW + 16 * (4 * c + g));
      if constexpr (ROT) turn_frags(kf, __shfl(dv, 16 * kb + i16));
      s[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[c]), qf[c], s[kb], 0, 0, 0);
    }
  };
  // second half: mask, softmax, O^T += V^T P^T
  auto tile_back = [&](int j, f32x4_t (&s)[2]) __attribute__((always_inline)) {
    const int k0 = it.k_begin + (w + DEC_WAVES * j) * DEC_KT;
    if (k0 + DEC_KT - 1 > lim_first || k0 + DEC_KT > k_end) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (k0 + 16 * kb + 4 * g + r > lim) s[kb][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = max_xor32(max_xor16(mx));
    const float m_cand = fmaxf(m_run, mx * c2);
    if (__ballot(m_cand > m_run + DEC_RESCALE_LOG2)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
      l_run *= alpha;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) oacc[nb] *= alpha;
      m_run = m_cand;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    u32x4_t pk;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * h], c2, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * h + 1], c2, -m_use));
        rs += p0 + p1;
        pk[2 * kb + h] = pk_bf2(p0, p1);
      }
    l_run += rs;
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pk);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const unsigned char DEC_LDS* vp = vl + tr_off + 32 * nb;
      const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t DEC_LDS*)vp);
      const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t DEC_LDS*)(vp + 256));
      const s16x8_t v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v8), pf, oacc[nb], 0, 0, 0);
    }
    // the next tile's V writes must not pass these reads
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Pipeline: tile j + 2's rows are issued as soon as tile j's registers are
  // consumed (after its scores), from slots loaded two tiles earlier, so two
  // tiles are in flight through tile j's softmax and PV.  Every iteration
  // issues the same loads (tiles past the range are clamped reads, and a
  // wave with an odd tile count runs one fully masked tile), so the load
  // waits are exact counts.
  u32x4_t kA[8], vA[8], kB[8], vB[8];
  int sA = slot_of(0), sB = slot_of(1);
  int dA = didx_of(0), dB = didx_of(1);
  load_tile(sA, kA, vA);
  sA = slot_of(2);
  load_tile(sB, kB, vB);
  sB = slot_of(3);
  f32x4_t s[2];
  const int n_pairs = (n_loc + 1) / 2;
  for (int pj = 0; pj < n_pairs; ++pj) {
    const int j = 2 * pj;
    tile_front(kA, vA, s, dA);
    load_tile(sA, kA, vA);
    dA = didx_of(j + 2);
    sA = slot_of(j + 4);
    tile_back(j, s);
    tile_front(kB, vB, s, dB);
    load_tile(sB, kB, vB);
    dB = didx_of(j + 3);
    sB = slot_of(j + 5);
    tile_back(j + 1, s);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // merge the waves: (m, l) per row, O^T rows through LDS
  l_run = sum_xor32(sum_xor16(l_run));
  __syncthreads();
  float* s_o = (float*)s_v;   // [wave][row 16][d 128] (32 KiB of the staging space)
  if (g == 0) {
    s_ml[w][row][0] = m_run;
    s_ml[w][row][1] = l_run;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[(w * 16 + row) * DEC_D + 16 * nb + 4 * g + r] = oacc[nb][r];
  __syncthreads();
  // thread: row tid / 16, columns 8 (tid % 16) .. + 8
  const int orow = tid >> 4, oc = 8 * (tid & 15);
  if (orow >= rows_total) return;
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < DEC_WAVES; ++v) M = fmaxf(M, s_ml[v][orow][0]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
  for (int v = 0; v < DEC_WAVES; ++v) {
    const float wv = __builtin_amdgcn_exp2f(s_ml[v][orow][0] - Mu);
    L += wv * s_ml[v][orow][1];
    const float* src = s_o + (v * 16 + orow) * DEC_D + oc;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += wv * src[e];
  }
  const int otok = (it.row0 + orow) / G, ohq = it.kvh * G + (it.row0 + orow) - otok * G;
  if (it.part < 0) {
    const float inv = L > 0.f ? 1.f / L : 0.f;
    u32x4_t ov;
#pragma unroll
    for (int e = 0; e < 4; ++e) ov[e] = pk_bf2(o[2 * e] * inv, o[2 * e + 1] * inv);
    *(u32x4_t*)(a.out + ((size_t)(sg.q_begin + otok) * a.n_q_heads + ohq) * DEC_D + oc) = ov;
    if (a.lse && (tid & 15) == 0)
      a.lse[(size_t)(sg.q_begin + otok) * a.n_q_heads + ohq] = L > 0.f ? Mu + __log2f(L) : INFINITY;
  } else {
    const size_t prow = (size_t)it.part + orow;
    float* po = a.part_o + prow * DEC_D + oc;
    *(f32x4_t*)po = f32x4_t{o[0], o[1], o[2], o[3]};
    *(f32x4_t*)(po + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
    if ((tid & 15) == 0) {
      a.part_ml[2 * prow] = M;
      a.part_ml[2 * prow + 1] = L;
    }
  }
}

// Attention mass per page ("AKV: Cache Engineering for Autonomous Agents",
// section 7, Dilemma 1: a server-side drop policy watches the cumulative
// attention weight of each block of the history over decode turns).  Second
// pass over a decode launch's lists: with each row's log-sum-exp from the
// attention, key k's weight for row r (token, q head) is 2^(s_rk c - lse_r)
// for keys within the row's causal limit; the weights of the segment's rows
// are summed per key and added to mass[page].
//
// Block: MASS_CHUNK consecutive list entries of one segment, one kv head
// (blockIdx.y); 16 groups of 16 lanes, group g takes entries g*16 .. +15 in
// order, lane j of a group holds d 8j .. 8j+7 of the key (one 16-byte load
// per lane, so a key row is one load of the group).  The group's lanes (one
// DPP row) reduce each row's dot product with DPP moves, lane 0 adds the weights and
// flushes one atomic add per run of entries in one page.  Keys owing a
// rotation are turned as the attention turned them (same table row, fp32
// formula and bf16 rounding).
constexpr int MASS_GROUPS = 16;
constexpr int MASS_PER_GROUP = MASS_CHUNK / MASS_GROUPS;
constexpr int MASS_BATCH = 8;
static_assert(MASS_PER_GROUP % MASS_BATCH == 0, "the group walk takes MASS_BATCH keys at a time");

// Sum over the 16 lanes of a DPP row (every lane gets it): quad xor 1, quad
// xor 2, half-row mirror, row mirror.
__device__ __forceinline__ float row_sum16(float s) {
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0xB1, 0xF, 0xF, false));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x4E, 0xF, 0xF, false));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x141, 0xF, 0xF, false));
  s += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(s), 0x140, 0xF, 0xF, false));
  return s;
}

// dot product of 8 bf16 pairs-of-words: key w, query qw (both packed bf16)
__device__ __forceinline__ float dot8(const u32x4_t& w, const u32x4_t& qw) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = fmaf(__uint_as_float(w[e] << 16), __uint_as_float(qw[e] << 16), s);
    s = fmaf(__uint_as_float(w[e] & 0xffff0000u), __uint_as_float(qw[e] & 0xffff0000u), s);
  }
  return s;
}

// R: rows per (segment, kv head) the launch holds at most (4, 8 or 16);
// ROT: list entries may owe a rotation (a.key_didx set).
template <int R, bool ROT>
__global__ __launch_bounds__(256) void k_page_mass(AttnArgs a, const MassItem* __restrict__ items,
                                                   float* __restrict__ mass) {
  const MassItem it = items[blockIdx.x];
  const int kvh = blockIdx.y;
  const AttnSeg sg = a.segs[it.seg];
  const int G = a.group, rows = sg.q_len * G;
  const int tid = threadIdx.x;
  const int grp = tid >> 4, j = tid & 15;
  // this lane's eight d of every row's query (packed bf16), the rows'
  // log-sum-exp and causal limits
  u32x4_t qw[R];
  float lse[R];
  int lim[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rr = r < rows ? r : 0;
    const int tok = rr / G, hq = kvh * G + (rr - tok * G);
    const size_t qrow = (size_t)(sg.q_begin + tok) * a.n_q_heads + hq;
    qw[r] = *(const u32x4_t*)(a.q + qrow * DEC_D + 8 * j);
    lse[r] = a.lse[qrow];
    lim[r] = r < rows ? sg.lkv - sg.q_len + tok : -1;
  }
  const int Hkv = a.n_kv_heads, S = a.page_size, lg = a.log2_page;
  const float c2 = a.scale_log2e;
  const int kb = it.k0 + grp * MASS_PER_GROUP;
  const int32_t* __restrict__ slots = a.slots + sg.list_off;
  int cur_page = -1;
  float acc = 0.f;
  int slot_n[MASS_BATCH];
#pragma unroll
  for (int u = 0; u < MASS_BATCH; ++u) slot_n[u] = slots[min(kb + u, sg.lkv - 1)];
  for (int k4 = 0; k4 < MASS_PER_GROUP; k4 += MASS_BATCH) {
    // this batch's rows in flight (entries past the list end re-read its
    // last), the next batch's slots behind them
    u32x4_t w[MASS_BATCH];
    int page[MASS_BATCH], didx[MASS_BATCH];
#pragma unroll
    for (int u = 0; u < MASS_BATCH; ++u) {
      const int e = min(kb + k4 + u, sg.lkv - 1);
      page[u] = slot_n[u] >> lg;
      const size_t row = ((size_t)page[u] * Hkv + kvh) * S + (slot_n[u] & (S - 1));
      w[u] = *(const u32x4_t*)(a.k_a + row * DEC_D + 8 * j);
      didx[u] = ROT ? a.key_didx[sg.list_off + e] : -1;
    }
    if (k4 + MASS_BATCH < MASS_PER_GROUP) {
#pragma unroll
      for (int u = 0; u < MASS_BATCH; ++u) slot_n[u] = slots[min(kb + k4 + MASS_BATCH + u, sg.lkv - 1)];
    }
#pragma unroll
    for (int u = 0; u < MASS_BATCH; ++u) {
      const int e = kb + k4 + u;
      if (e < sg.lkv) {
        if (ROT && didx[u] >= 0) {   // the same for all 16 lanes of the group
          const float* row = a.rot_table + (size_t)didx[u] * DEC_D;
          if (a.rot_pairing == 0) {
            const f32x4_t cs = *(const f32x4_t*)(row + 4 * j), sn = *(const f32x4_t*)(row + DEC_D / 2 + 4 * j);
            turn_interleaved(w[u], cs, sn);
          } else {
            // lanes j < 8 hold the first elements of pairs 8j .. 8j+7, lane
            // j + 8 their second elements
            const int p0 = 8 * (j & 7);
            u32x4_t o;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) o[e2] = (unsigned)__shfl_xor((int)w[u][e2], 8, 16);
            u32x4_t xw = j < 8 ? w[u] : o, yw = j < 8 ? o : w[u];
            const f32x4_t c0 = *(const f32x4_t*)(row + p0), c1 = *(const f32x4_t*)(row + p0 + 4);
            const f32x4_t s0 = *(const f32x4_t*)(row + DEC_D / 2 + p0);
            const f32x4_t s1 = *(const f32x4_t*)(row + DEC_D / 2 + p0 + 4);
            turn_half(xw, yw, c0, c1, s0, s1);
            w[u] = j < 8 ? xw : yw;
          }
        }
        float km = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float s = row_sum16(dot8(w[u], qw[r]));
          if (e <= lim[r]) km += __builtin_amdgcn_exp2f(fmaf(s, c2, -lse[r]));
        }
        if (page[u] != cur_page) {
          if (cur_page >= 0 && j == 0) atomicAdd(mass + cur_page, acc);
          cur_page = page[u];
          acc = 0.f;
        }
        acc += km;
      }
    }
  }
  if (cur_page >= 0 && j == 0) atomicAdd(mass + cur_page, acc);
}

}  // namespace

__global__ __launch_bounds__(256) void k_expand_didx(const Extent* __restrict__ ex, const int32_t* __restrict__ ex_off,
                                                     const int32_t* __restrict__ ex_didx, int n_ext,
                                                     int32_t* __restrict__ out) {
  for (int e = blockIdx.x * 256 + threadIdx.x; e < n_ext; e += gridDim.x * 256) {
    const int n = ex[e].hi - ex[e].lo, o = ex_off[e], d = ex_didx[e];
    for (int i = 0; i < n; ++i) out[o + i] = d;
  }
}

hipError_t launch_expand_didx(hipStream_t st, const Extent* ex, const int32_t* ex_off, const int32_t* ex_didx,
                              int n_ext, int32_t* out) {
  if (n_ext <= 0) return hipSuccess;
  const int blocks = std::min(4096, (n_ext + 255) / 256);
  launch_k(k_expand_didx, dim3(blocks), dim3(256), st, ex, ex_off, ex_didx, n_ext, out);
  return hipGetLastError();
}

hipError_t launch_page_mass(hipStream_t st, const AttnArgs& a, const MassItem* items, int n_items, int max_rows,
                            float* mass) {
  if (n_items <= 0) return hipSuccess;
  if (a.n_kv_heads > 65535 || !a.lse || max_rows > DECODE_ROWS) return hipErrorInvalidValue;
  const dim3 grid(n_items, a.n_kv_heads);
  const bool rot = a.key_didx != nullptr;
  if (max_rows <= 4) {
    if (rot) launch_k(k_page_mass<4, true>, grid, dim3(256), st, a, items, mass);
    else launch_k(k_page_mass<4, false>, grid, dim3(256), st, a, items, mass);
  } else if (max_rows <= 8) {
    if (rot) launch_k(k_page_mass<8, true>, grid, dim3(256), st, a, items, mass);
    else launch_k(k_page_mass<8, false>, grid, dim3(256), st, a, items, mass);
  } else {
    if (rot) launch_k(k_page_mass<16, true>, grid, dim3(256), st, a, items, mass);
    else launch_k(k_page_mass<16, false>, grid, dim3(256), st, a, items, mass);
  }
  return hipGetLastError();
}

hipError_t launch_decode_attn(hipStream_t st, const AttnArgs& a) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.key_didx)
    launch_k(k_decode_attn<true>, dim3(a.n_items), dim3(64 * DEC_WAVES), st, a);
  else
    launch_k(k_decode_attn<false>, dim3(a.n_items), dim3(64 * DEC_WAVES), st, a);
  return hipGetLastError();
}

}  // namespace akv
