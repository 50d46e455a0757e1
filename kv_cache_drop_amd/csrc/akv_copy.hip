// Token-row copies of the paged pool (gfx950): append, compaction and
// positional versions.  All three are HBM-bound streams of 16-byte chunks.
//
// Sources, cited by page title and section:
//   [AKV-notes] "Cache Engineering for Agents", section 1 (append) and
//               section 3 (Cache Management: re-use by key rotation; the
//               retrigger match of the cache reuse matching rules)
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents ...", section 2
//               (The Repos Primitive: R(a)R(b) = R(a+b)) and section 7
//               (Dilemma 2: compaction when fragmentation passes 40%)
//
// One launch moves every paged array of the listed tokens: the rotated-key
// array (GQA K, MLA K_pe), V and, for MLA, K_nope.  Each thread keeps four
// 16-byte chunks (64 bytes) in flight: it issues all its loads, then all its
// stores, so a CU holds enough bytes in flight to cover HBM latency.  The
// grid strides over the chunks; consecutive lanes take consecutive chunks of a
// row.  Moves order the rows head-major (head, token), so a wave's rows are
// neighbouring slots of one head: runs of consecutive slots become contiguous
// reads and writes of a page's head block.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "akv_internal.h"
#include "akv_launch.h"

namespace akv {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kChunks = 4;   // 16-byte chunks in flight per thread (rotated-key units: 2)

__device__ __forceinline__ float lo_bf(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned bf2(float a, float b) {
  // round to nearest even on the float -> bf16 conversion
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ size_t page_row(int slot, int h, int H, int S, int log2S, int d) {
  return (((size_t)(slot >> log2S) * H + h) * S + (slot & (S - 1))) * d;
}

// Rows of one array, addressed per chunk: chunk c of (token t, head h).
struct Part {
  const uint16_t* src;   // token-major [n][H][d] (append) or a paged array (moves)
  uint16_t* dst;         // paged array
  int H, d;
};

// ---------------------------------------------------------------------------
// append: token-major rows -> page slots
// ---------------------------------------------------------------------------
struct ScatterArgs {
  Part part[3];
  int n_parts;
  const int32_t* slots;
  int n, S, log2S;
};

__global__ __launch_bounds__(kThreads) void k_scatter_tokens(ScatterArgs a) {
  const long T = (long)gridDim.x * kThreads;
  for (int pi = 0; pi < a.n_parts; ++pi) {
    const Part p = a.part[pi];
    const int cpr = p.d >> 3;
    const long total = (long)a.n * p.H * cpr;
    for (long i0 = (long)blockIdx.x * kThreads + threadIdx.x; i0 < total; i0 += T * kChunks) {
      u32x4_t r[kChunks];
      uint16_t* dp[kChunks];
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        const long i = i0 + k * T;
        if (i < total) {
          const int c = (int)(i % cpr);
          const long row = i / cpr;               // token * H + head
          const int h = (int)(row % p.H);
          const int t = (int)(row / p.H);
          r[k] = *(const u32x4_t*)(p.src + row * p.d + 8 * c);
          dp[k] = p.dst + page_row(a.slots[t], h, p.H, a.S, a.log2S, p.d) + 8 * c;
        }
      }
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
        if (i0 + k * T < total) *(u32x4_t*)dp[k] = r[k];
    }
  }
}

// ---------------------------------------------------------------------------
// slot -> slot moves (compaction; positional versions with key rotation)
// ---------------------------------------------------------------------------
// The rotated-key array moves in "units" of 8 rotation pairs held in two
// 16-byte words (interleaved pairing: 16 consecutive elements; half-split
// pairing: 8 elements of each half).  With a table, pair (x, y) becomes
// (x cos - y sin, x sin + y cos) in fp32, rounded once to bf16: the formula
// and table of the in-place repos, so both write the same keys.  The other
// arrays (V, MLA K_nope) move in plain 16-byte chunks.
struct MoveArgs {
  uint16_t* kr;          // rotated-key pages (GQA K, MLA K_pe)
  Part plain[2];         // V, then K_nope (src == dst array)
  int n_plain;
  const MovePair* pairs;
  const float* table;    // cos[d_rope/2], sin[d_rope/2], or nullptr (copy)
  int n, rope_heads, S, log2S, d_rope, pairing;
};

__global__ __launch_bounds__(kThreads) void k_move_tokens(MoveArgs a) {
  __shared__ float s_c[128], s_s[128];
  const int half = a.d_rope >> 1;
  const bool rot = a.table != nullptr;
  if (rot && (int)threadIdx.x < half) {
    s_c[threadIdx.x] = a.table[threadIdx.x];
    s_s[threadIdx.x] = a.table[half + threadIdx.x];
  }
  __syncthreads();
  const long T = (long)gridDim.x * kThreads;

  // rotated-key units, two per thread in flight
  {
    constexpr int U = kChunks / 2;
    const int upr = a.d_rope >> 4;
    const long total = (long)a.n * a.rope_heads * upr;
    for (long i0 = (long)blockIdx.x * kThreads + threadIdx.x; i0 < total; i0 += T * U) {
      u32x4_t ra[U], rb[U];
      uint16_t* dp[U];
      int cu[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const long i = i0 + k * T;
        if (i < total) {
          const int c = (int)(i % upr);
          const long r = i / upr;                 // head * n + pair
          const int h = (int)(r / a.n);
          const MovePair mp = a.pairs[r - (long)h * a.n];
          const int oa = a.pairing == 0 ? 16 * c : 8 * c;
          const uint16_t* sp = a.kr + page_row(mp.src, h, a.rope_heads, a.S, a.log2S, a.d_rope) + oa;
          const int ob = a.pairing == 0 ? 8 : half;      // second word, relative to the first
          ra[k] = *(const u32x4_t*)sp;
          rb[k] = *(const u32x4_t*)(sp + ob);
          dp[k] = a.kr + page_row(mp.dst, h, a.rope_heads, a.S, a.log2S, a.d_rope) + oa;
          cu[k] = c;
        }
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (i0 + k * T >= total) continue;
        u32x4_t wa = ra[k], wb = rb[k];
        const int p0 = 8 * cu[k];
        if (rot && a.pairing == 0) {
          // word j of ra holds pair p0 + j, word j of rb pair p0 + 4 + j
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x = lo_bf(ra[k][j]), y = hi_bf(ra[k][j]);
            float cs = s_c[p0 + j], sn = s_s[p0 + j];
            wa[j] = bf2(fmaf(x, cs, -y * sn), fmaf(x, sn, y * cs));
            x = lo_bf(rb[k][j]);
            y = hi_bf(rb[k][j]);
            cs = s_c[p0 + 4 + j];
            sn = s_s[p0 + 4 + j];
            wb[j] = bf2(fmaf(x, cs, -y * sn), fmaf(x, sn, y * cs));
          }
        } else if (rot) {
          // word j of ra holds the first elements of pairs p0 + 2j, p0 + 2j + 1,
          // word j of rb their second elements
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float c0 = s_c[p0 + 2 * j], s0 = s_s[p0 + 2 * j];
            const float c1 = s_c[p0 + 2 * j + 1], s1 = s_s[p0 + 2 * j + 1];
            const float x0 = lo_bf(ra[k][j]), x1 = hi_bf(ra[k][j]);
            const float y0 = lo_bf(rb[k][j]), y1 = hi_bf(rb[k][j]);
            wa[j] = bf2(fmaf(x0, c0, -y0 * s0), fmaf(x1, c1, -y1 * s1));
            wb[j] = bf2(fmaf(x0, s0, y0 * c0), fmaf(x1, s1, y1 * c1));
          }
        }
        *(u32x4_t*)dp[k] = wa;
        *(u32x4_t*)(dp[k] + (a.pairing == 0 ? 8 : half)) = wb;
      }
    }
  }

  // plain arrays, four chunks per thread in flight
  for (int pi = 0; pi < a.n_plain; ++pi) {
    const Part p = a.plain[pi];
    const int cpr = p.d >> 3;
    const long total = (long)a.n * p.H * cpr;
    for (long i0 = (long)blockIdx.x * kThreads + threadIdx.x; i0 < total; i0 += T * kChunks) {
      u32x4_t r[kChunks];
      uint16_t* dp[kChunks];
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        const long i = i0 + k * T;
        if (i < total) {
          const int c = (int)(i % cpr);
          const long row = i / cpr;               // head * n + pair
          const int h = (int)(row / a.n);
          const MovePair mp = a.pairs[row - (long)h * a.n];
          r[k] = *(const u32x4_t*)(p.src + page_row(mp.src, h, p.H, a.S, a.log2S, p.d) + 8 * c);
          dp[k] = p.dst + page_row(mp.dst, h, p.H, a.S, a.log2S, p.d) + 8 * c;
        }
      }
#pragma unroll
      for (int k = 0; k < kChunks; ++k)
        if (i0 + k * T < total) *(u32x4_t*)dp[k] = r[k];
    }
  }
}

int blocks_for(long chunks) {
  long b = (chunks + (long)kThreads * kChunks - 1) / ((long)kThreads * kChunks);
  if (b > 65536) b = 65536;
  return (int)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_scatter_tokens(hipStream_t st, const TokenRows* rows, int n_rows, const int32_t* slots,
                                 int n, int page_size, int log2_page) {
  if (n <= 0 || n_rows <= 0) return hipSuccess;
  if (n_rows > 3) return hipErrorInvalidValue;
  ScatterArgs a{};
  long most = 0;
  for (int i = 0; i < n_rows; ++i) {
    a.part[i] = Part{rows[i].src, rows[i].dst, rows[i].heads, rows[i].d};
    most = std::max(most, (long)n * rows[i].heads * (rows[i].d >> 3));
  }
  a.n_parts = n_rows;
  a.slots = slots;
  a.n = n;
  a.S = page_size;
  a.log2S = log2_page;
  launch_k(k_scatter_tokens, dim3(blocks_for(most)), dim3(kThreads), st, a);
  return hipGetLastError();
}

hipError_t launch_move_tokens(hipStream_t st, uint16_t* kr, int rope_heads, int d_rope, int pairing,
                              const TokenRows* plain, int n_plain, const MovePair* pairs, int n,
                              int page_size, int log2_page, const float* table) {
  if (n <= 0) return hipSuccess;
  if (n_plain > 2) return hipErrorInvalidValue;
  MoveArgs a{};
  a.kr = kr;
  long most = (long)n * rope_heads * (d_rope >> 3);
  for (int i = 0; i < n_plain; ++i) {
    a.plain[i] = Part{plain[i].src, plain[i].dst, plain[i].heads, plain[i].d};
    most = std::max(most, (long)n * plain[i].heads * (plain[i].d >> 3));
  }
  a.n_plain = n_plain;
  a.pairs = pairs;
  a.table = table;
  a.n = n;
  a.rope_heads = rope_heads;
  a.S = page_size;
  a.log2S = log2_page;
  a.d_rope = d_rope;
  a.pairing = pairing;
  launch_k(k_move_tokens, dim3(blocks_for(most)), dim3(kThreads), st, a);
  return hipGetLastError();
}

}  // namespace akv
