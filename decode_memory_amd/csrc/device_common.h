// Device-side helpers for gfx950 (CDNA4, 64-wide wavefronts).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pagedkv {

constexpr int kWave = 64;

// ---- 16-bit float conversions ---------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return __half2float(__ushort_as_half(static_cast<unsigned short>(w >> 16)));
}

// ---- global-memory access through table pointers ----------------------------
// Slab tables hold generic pointers, so a plain access through one compiles
// to a FLAT instruction, which also counts against the LDS wait counter and
// so holds up unrelated LDS waits; these cast the pointer to the global
// address space first (every slab lives in device global memory).

typedef unsigned int gw2 __attribute__((ext_vector_type(2)));
typedef unsigned int gw4 __attribute__((ext_vector_type(4)));
template <int N> struct GlobalWords;
template <> struct GlobalWords<4> { typedef unsigned int type; };
template <> struct GlobalWords<8> { typedef gw2 type; };
template <> struct GlobalWords<16> { typedef gw4 type; };

template <class T>
__device__ __forceinline__ void store_global(void* p, const T& v) {
  typedef typename GlobalWords<sizeof(T)>::type W;
  *(__attribute__((address_space(1))) W*)p = __builtin_bit_cast(W, v);
}

template <class T>
__device__ __forceinline__ T load_global(const void* p) {
  typedef typename GlobalWords<sizeof(T)>::type W;
  return __builtin_bit_cast(T, *(const __attribute__((address_space(1))) W*)p);
}

// Widen 8 packed 16-bit values (one 16-byte vector) to fp32.
template <bool BF16>
__device__ __forceinline__ void widen8(const uint4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    } else {
      x[2 * i] = f16_lo(w[i]);
      x[2 * i + 1] = f16_hi(w[i]);
    }
  }
}

// Dot product of 8 packed 16-bit values (one 16-byte vector each) added to
// acc, with the gfx950 packed dot instructions (two products per
// instruction, exact products, fp32 accumulation).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <bool BF16>
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b, float acc) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (BF16)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x[i]),
                                            __builtin_bit_cast(bf16x2_t, y[i]), acc, false);
    else
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x[i]),
                                   __builtin_bit_cast(f16x2_t, y[i]), acc, false);
  }
  return acc;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

template <bool BF16>
__device__ __forceinline__ uint16_t f32_to_out(float f) {
  if constexpr (BF16) return f32_to_bf16_rne(f);
  else return f32_to_f16_rne(f);
}

// ---- cross-lane reductions ---------------------------------------------------
// DPP row operations keep the reduction inside the VALU (no LDS crossbar):
// quad_perm swaps neighbours and pairs, row_half_mirror pairs the two quads of
// an 8-lane half row, row_mirror pairs the two halves of a 16-lane row.  After
// each step every lane holds the combined value of its partner set, so all
// lanes of the group end with the full result.

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Sum over aligned groups of W lanes (W in 1..64); every lane gets its group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W >= 2) v += dpp<kDppXor1>(v);
  if constexpr (W >= 4) v += dpp<kDppXor2>(v);
  if constexpr (W >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (W >= 16) v += dpp<kDppMirror>(v);
  if constexpr (W >= 32) v += xor_lane(v, 16);
  if constexpr (W >= 64) v += xor_lane(v, 32);
  return v;
}

// Max / sum across the lane groups of a wave: lanes that differ only in the
// bits >= log2(W) are combined (W = lanes per group).
template <int W>
__device__ __forceinline__ float across_groups_max(float v) {
#pragma unroll
  for (int m = W; m < kWave; m <<= 1) v = fmaxf(v, xor_lane(v, m));
  return v;
}
template <int W>
__device__ __forceinline__ float across_groups_sum(float v) {
#pragma unroll
  for (int m = W; m < kWave; m <<= 1) v += xor_lane(v, m);
  return v;
}

// ---- launch geometry --------------------------------------------------------
// Workgroup k of a launch is dispatched to XCD k % 8 and each XCD has its own
// L2.  This maps hardware workgroup ids to work ids so that consecutive work
// ids (which share a sequence and kv head) run on the same XCD.  The grid must
// be a multiple of 8; work ids >= the real count are idle.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_work_id(int hw_id, int grid) {
  const int per_xcd = grid / kXcds;
  return (hw_id % kXcds) * per_xcd + hw_id / kXcds;
}

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }

__device__ __forceinline__ void set_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace pagedkv
