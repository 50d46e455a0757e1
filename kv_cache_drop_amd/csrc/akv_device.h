// Device-side helpers shared by the attention and rotation kernels (gfx950):
// vector types, bf16 packing, the rotation of one interleaved pair, the LDS
// tile-part layout of the direct-to-LDS attention kernels, and scalar-cache
// loads.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace akv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

#define AKV_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf2(float a, float b) {
  bf16x2 v;
  v.x = (__bf16)a;
  v.y = (__bf16)b;
  return __builtin_bit_cast(unsigned, v);
}

// Turns one 32-bit word holding a rotation pair by (cos c, sin s): fp32
// arithmetic, one rounding to bf16 per element.
__device__ __forceinline__ unsigned rot_pair_word(unsigned w, float c, float s) {
  // word holds an interleaved pair (x = low half, y = high half)
  float x = bf_lo(w), y = bf_hi(w);
  return pack_bf2(fmaf(x, c, -y * s), fmaf(x, s, y * c));
}

// Online softmax: O and l are rescaled only when a row's max grows by more
// than 2^RESCALE_LOG2 over the running reference (base-2 units).
constexpr float RESCALE_LOG2 = 8.f;

// LDS layout of one part of a 64-key tile with CH 16-byte chunks per key row:
// CH blocks of 1 KiB plus PAD bytes; block b holds keys b, b + CH, ...
template <int CH, int PAD>
struct LdsPart {
  static constexpr int BLK = 1024 + PAD;
  static constexpr int BYTES = CH * BLK;
  // byte offset of (key r, chunk c)
  static __device__ __forceinline__ int off(int r, int c) {
    return (r % CH) * BLK + (r / CH) * (CH * 16) + 16 * c;
  }
};

// Reductions over lane pairs of a wave without LDS traffic.  On gfx950,
// v_permlane32_swap (v_permlane16_swap) with one register as both operands
// leaves each lane the two values of its pair, lane l and lane l ^ 32 (within
// each half of 32 lanes, l ^ 16), in two registers, in the same order for both
// lanes of the pair, which therefore agree bit for bit.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight floats from a wave-uniform address through the scalar data cache
// (a load: counted by lgkmcnt, so waiting for it never drains the tile DMAs
// that vmcnt counts).
__device__ __forceinline__ f32x8 scalar_load8(const float* p) {
  return *(const __attribute__((address_space(4))) f32x8*)(size_t)p;
}

}  // namespace akv
