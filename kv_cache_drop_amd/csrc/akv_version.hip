// Positional versions: out-of-place repos of token rows (gfx950).
//
// Sources, cited by page title and section:
//   [AKV-notes] "Cache Engineering for Agents", section 3 (Cache Management:
//               reuse through key rotation; cache reuse matching rules, the
//               retrigger match that re-uses a cached state at other positions)
//   [AKV-blog]  "AKV: Cache Engineering for Autonomous Agents ...", section 2
//               (The Repos Primitive: R(a)R(b) = R(a+b))
//
// A cached token state is re-used at new positions by copying its rows into
// fresh slots and turning the rotated key part by the position change on the
// way; the source rows stay as they are, so the old positional version keeps
// serving its own sequence.  The rows that carry no position (V, MLA K_nope)
// are copied as they are, in the same launch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "akv_internal.h"

namespace akv {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

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

// One launch moves every row of the listed tokens.  The index space is the
// rotated-key "units" first (8 rotation pairs held in two 16-byte words:
// interleaved pairing, 16 consecutive elements; half-split pairing, 8
// elements of each half), then the 16-byte chunks of the V rows, then those
// of the K_nope rows (MLA).  A unit's pair (x, y) becomes (x cos - y sin,
// x sin + y cos) in fp32, rounded once to bf16; with rotate == 0 the unit is
// copied.  The block stages the delta's cos / sin row in LDS; the grid
// strides over the index space.
struct CloneArgs {
  uint16_t* kr;          // rotated-key pages (GQA K, MLA K_pe)
  uint16_t* v;
  uint16_t* kn;          // MLA K_nope pages, else nullptr
  const MovePair* pairs;
  const float* table;    // cos[d_rope/2], sin[d_rope/2]
  int n, rope_heads, heads, S, log2S, d_rope, d_v, d_nope, pairing, rotate;
};

__device__ __forceinline__ size_t row_off(int slot, int h, int H, int S, int log2S, int d) {
  return (((size_t)(slot >> log2S) * H + h) * S + (slot & (S - 1))) * d;
}

__global__ __launch_bounds__(256) void k_clone_rows(CloneArgs a) {
  __shared__ float s_c[128], s_s[128];
  const int half = a.d_rope >> 1;
  if (a.rotate && (int)threadIdx.x < half) {
    s_c[threadIdx.x] = a.table[threadIdx.x];
    s_s[threadIdx.x] = a.table[half + threadIdx.x];
  }
  __syncthreads();
  const int upr = a.d_rope >> 4, vpr = a.d_v >> 3, npr = a.d_nope >> 3;
  const long n_k = (long)a.n * a.rope_heads * upr;
  const long n_v = (long)a.n * a.heads * vpr;
  const long total = n_k + n_v + (long)a.n * a.heads * npr;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    if (i < n_k) {
      const int c = (int)(i % upr);
      const long r = i / upr;
      const int h = (int)(r % a.rope_heads);
      const MovePair mp = a.pairs[r / a.rope_heads];
      const uint16_t* src = a.kr + row_off(mp.src, h, a.rope_heads, a.S, a.log2S, a.d_rope);
      uint16_t* dst = a.kr + row_off(mp.dst, h, a.rope_heads, a.S, a.log2S, a.d_rope);
      const int oa = a.pairing == 0 ? 16 * c : 8 * c;
      const int ob = a.pairing == 0 ? 16 * c + 8 : half + 8 * c;
      const u32x4_t ra = *(const u32x4_t*)(src + oa);
      const u32x4_t rb = *(const u32x4_t*)(src + ob);
      u32x4_t wa = ra, wb = rb;
      const int p0 = 8 * c;
      if (a.rotate && a.pairing == 0) {
        // word k of ra holds pair p0 + k, word k of rb pair p0 + 4 + k
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float x = lo_bf(ra[k]), y = hi_bf(ra[k]);
          float cs = s_c[p0 + k], sn = s_s[p0 + k];
          wa[k] = bf2(fmaf(x, cs, -y * sn), fmaf(x, sn, y * cs));
          x = lo_bf(rb[k]);
          y = hi_bf(rb[k]);
          cs = s_c[p0 + 4 + k];
          sn = s_s[p0 + 4 + k];
          wb[k] = bf2(fmaf(x, cs, -y * sn), fmaf(x, sn, y * cs));
        }
      } else if (a.rotate) {
        // word k of ra holds the first elements of pairs p0 + 2k, p0 + 2k + 1,
        // word k of rb their second elements
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float c0 = s_c[p0 + 2 * k], s0 = s_s[p0 + 2 * k];
          const float c1 = s_c[p0 + 2 * k + 1], s1 = s_s[p0 + 2 * k + 1];
          const float x0 = lo_bf(ra[k]), x1 = hi_bf(ra[k]);
          const float y0 = lo_bf(rb[k]), y1 = hi_bf(rb[k]);
          wa[k] = bf2(fmaf(x0, c0, -y0 * s0), fmaf(x1, c1, -y1 * s1));
          wb[k] = bf2(fmaf(x0, s0, y0 * c0), fmaf(x1, s1, y1 * c1));
        }
      }
      *(u32x4_t*)(dst + oa) = wa;
      *(u32x4_t*)(dst + ob) = wb;
    } else {
      long j = i - n_k;
      uint16_t* base = a.v;
      int cpr = vpr, d = a.d_v;
      if (j >= n_v) {
        j -= n_v;
        base = a.kn;
        cpr = npr;
        d = a.d_nope;
      }
      const int c = (int)(j % cpr);
      const long r = j / cpr;
      const int h = (int)(r % a.heads);
      const MovePair mp = a.pairs[r / a.heads];
      *(u32x4_t*)(base + row_off(mp.dst, h, a.heads, a.S, a.log2S, d) + 8 * c) =
          *(const u32x4_t*)(base + row_off(mp.src, h, a.heads, a.S, a.log2S, d) + 8 * c);
    }
  }
}

}  // namespace

hipError_t launch_clone_rows(hipStream_t st, uint16_t* kr, uint16_t* v, uint16_t* kn, const MovePair* pairs,
                             int n, int rope_heads, int n_heads, int page_size, int log2_page, int d_rope,
                             int d_v, int d_nope, int pairing, const float* table) {
  if (n <= 0) return hipSuccess;
  CloneArgs a{kr, v, kn, pairs, table, n, rope_heads, n_heads, page_size, log2_page, d_rope, d_v, d_nope,
              pairing, table != nullptr};
  const long total = (long)n * (rope_heads * (d_rope >> 4) + n_heads * ((d_v + d_nope) >> 3));
  long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_clone_rows, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace akv
