// Packing one token-head vector of a packed pool: the signed Hadamard
// rotation of K and the affine group quantisation (mlx-swift-lm PR #142, "Add
// packed paged KV formats with bounded workspace admission", section
// "Summary": K is rotated by a fixed signed Hadamard basis, then each group of
// 32 or 64 values gets unsigned codes with an fp32 (scale, offset) pair).
// A lane holds 8 consecutive values of the vector and D/8 lanes, aligned to a
// multiple of D/8, hold the vector.  Every lane of the wave must call these
// functions (they exchange values across lanes); lanes whose vector is not
// stored still compute.
#pragma once

#include "device_common.h"

namespace pagedkv {

// Every rounding below is the one the packed format's definition states, in
// fp32.  Each function turns contraction off and uses plain operators (HIP's
// __fmul_rn and the like are plain operators in a header that allows
// contraction), so no product is fused into a following sum unless the code
// says so with an fma whose product is exact.

// The Sylvester Hadamard butterfly network over a D-value vector held 8
// values per lane by D/8 lanes (lane c of the group: values 8c .. 8c+7):
// stages h = 1, 2, ..., D/2, each pair (a, b) -> (a + b, a - b) in fp32 (the
// lower index gets a + b).  Stages h < 8 pair values inside a lane, the
// others pair lanes c and c ^ (h / 8) of the vector's lane group.  The values
// are first multiplied by the signs sg (exact), and that product is fused
// into the first stage: fma(s, x, b) = RN(s x + b).  With ODD_SIGNED the odd
// values x[1], x[3], ... carry their signs already.
template <int D, bool ODD_SIGNED = false>
__device__ __forceinline__ void signed_fwht8(float (&x)[8], int c, const float (&sg)[8]) {
  #pragma clang fp contract(off)
  constexpr int LPT = D / 8;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float a = x[e];
    const float b = ODD_SIGNED ? x[e + 1] : x[e + 1] * sg[e + 1];
    x[e] = __builtin_fmaf(sg[e], a, b);
    x[e + 1] = __builtin_fmaf(sg[e], a, -b);
  }
#pragma unroll
  for (int h = 2; h < 8; h <<= 1) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (e & h) ? x[e ^ h] - x[e] : x[e] + x[e ^ h];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = y[e];
  }
  const int lane = static_cast<int>(__lane_id());
#pragma unroll
  for (int hl = 1; hl < LPT; hl <<= 1) {
    // the lower lane keeps x + other, the upper other - x: one fma with a
    // +-1 factor (exact product, one rounding) gives both
    const float sgn = (c & hl) ? -1.f : 1.f;
    const int from = (lane ^ hl) * 4;  // byte address of the partner lane
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float other = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(x[e])));
      x[e] = __builtin_fmaf(sgn, x[e], other);
    }
  }
}

// x' = H diag(sigma) x / sqrt(D): the sign flips (exact), the butterfly
// network above, then one multiply by 1/sqrt(D).  sg holds the lane's signs
// sigma[8c .. 8c+7].
template <int D>
__device__ __forceinline__ void fwht_rotate8_held(float (&x)[8], const float (&sg)[8], int c, float inv_sqrt_d) {
  #pragma clang fp contract(off)
  signed_fwht8<D>(x, c, sg);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] * inv_sqrt_d;
}

// The same with the signs read from the D-value sign vector.
template <int D>
__device__ __forceinline__ void fwht_rotate8(float (&x)[8], const float* signs, int c, float inv_sqrt_d) {
  float sg[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sg[e] = signs[8 * c + e];
  fwht_rotate8_held<D>(x, sg, c, inv_sqrt_d);
}

// The rotation straight from the lane's 16 bytes of bf16 values: each odd
// value's sign flip is folded into the mask that widens it (an exact flip of
// the sign bit, odd_sign[i] = sign bit of sigma[8c + 2i + 1]).
template <int D>
__device__ __forceinline__ void widen_rotate8(const uint4& u, const uint32_t (&odd_sign)[4], const float (&sg)[8],
                                              int c, float inv_sqrt_d, float (&x)[8]) {
  #pragma clang fp contract(off)
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float((w[i] & 0xffff0000u) ^ odd_sign[i]);
  }
  signed_fwht8<D, true>(x, c, sg);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] * inv_sqrt_d;
}

// RN(a / b) for b = 15 or 255 and every finite a >= 0: q0 = RN(a * RN(1/b)),
// then one correction with the exact remainder a - q0 * b (an fma).  For
// these two divisors this equals the correctly rounded quotient for all 2^31
// - 2^23 finite non-negative fp32 a (checked exhaustively against IEEE
// division on the host); a = inf gives inf.
__device__ __forceinline__ float div_levels_rn(float a, float levels, float inv_levels) {
  #pragma clang fp contract(off)
  const float q0 = a * inv_levels;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, levels, a), inv_levels, q0);
  return a < __builtin_inff() ? q1 : a;
}

// Quantise the lane's 8 values (values 8c .. 8c+7 of the vector) with the
// (scale, offset) of their group of GS values, all in fp32: mn = min, mx =
// max, scale = (mx - mn) / (2^bits - 1), offset = mn, code = clamp(rint((x -
// mn) / scale)) with round-half-even, and a constant group gets code 0.  The
// codes are packed as a record holds them (8-bit: one byte per value; 4-bit:
// value 2i in the low nibble of byte i).
// The lane's codes packed as they are stored (8-bit: bytes 0-3 in lo, 4-7 in
// hi; 4-bit: the nibble pairs in lo), and its group's (scale, offset).
struct Codes8 {
  uint32_t lo, hi;
  float scale, offset;
};

template <int D, int GS>
__device__ __forceinline__ Codes8 quantise8(const float (&x)[8], int c, int bits) {
  #pragma clang fp contract(off)
  static_assert(GS == 32 || GS == 64, "groups of 32 or 64 values");
  constexpr int LPG = GS / 8;  // lanes per group
  // min and max in the lane, then across the lane quad, then (groups of 64)
  // across the two quads of the 8-lane half row
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  // Each step is one DPP min and one DPP max: the lane exchange rides in the
  // instruction, where a separate DPP move would also need the compiler's
  // canonicalising max of the moved value (both inputs here are results of
  // min/max, so the plain IEEE min/max is the same operation).  s_nop 4 gives
  // the wait states a DPP instruction needs after a VALU write of its source
  // register (2) or of EXEC (5), whatever the compiler placed before it.
  // Records unchanged; the packed write measured 1-6% faster.
#define PD_DPP_MINMAX(CTRL)                                                                      \
  asm("s_nop 4\n\tv_min_f32_dpp %0, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t" \
      "v_max_f32_dpp %1, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"                 \
      : "=&v"(mn), "=&v"(mx)                                                                    \
      : "v"(mn), "v"(mx))
  PD_DPP_MINMAX("quad_perm:[1,0,3,2]");  // lanes c ^ 1
  PD_DPP_MINMAX("quad_perm:[2,3,0,1]");  // lanes c ^ 2
  if constexpr (LPG == 8) PD_DPP_MINMAX("row_half_mirror");  // the other quad of the 8
#undef PD_DPP_MINMAX
  const bool eight = bits == 8;
  const float levels = eight ? 255.f : 15.f;
  const float scale = div_levels_rn(mx - mn, levels, eight ? 1.f / 255.f : 1.f / 15.f);
  // a constant group (scale 0) divides by 1 instead: every x - mn is then
  // below half the smallest subnormal times 2^bits, so its code is 0
  const float div = scale == 0.f ? 1.f : scale;
  // The code is rint(q), q = RN(d / div), d = RN(x - mn) >= 0.  With div
  // normal, the hardware reciprocal estimate and one Newton step give r with
  // relative error below 2^-24 + 2^-40, so q' = RN(d * r) lies within 2.01
  // ulp(q) of q (below 2^-14.9 at 8 bits, q < 256; below 2^-18.9 at 4 bits,
  // q < 16), and t = rint(q') is rint(q) unless q' lies within 2^-14 (4 bits:
  // 2^-18) of a half-integer, about 1 value in 8000 (4 bits: 1 in 130000).
  // Such a value takes the correctly rounded division, clamped (a subnormal
  // scale can give q > 2^bits - 1): for each of the lane's 8 positions, the
  // wave divides at that position when any of its lanes has a value there in
  // the band.  Bf16 data put values exactly at a code midpoint often (the
  // middle of a group's range is q = 7.5 at 4 bits), so about 1 position in
  // 8 of a wave needs it, while a whole-wave fallback would divide all 8 in
  // most wave tasks.  A divisor below 2^-125 or not finite sends every
  // position through the division.  The fast path needs no clamp: q' <=
  // (2^bits - 1)(1 + 2^-21) for a normal scale.  A NaN value gets an
  // unspecified code.
  const float r0 = __builtin_amdgcn_rcpf(div);
  const float r = __builtin_fmaf(__builtin_fmaf(-div, r0, 1.f), r0, r0);
  // (a divisor out of range makes the threshold -1, which every position
  // fails; so does a NaN quotient)
  const float band = eight ? 0.49993896484375f : 0.4999961853027344f;
  const float thr = (div >= 0x1p-125f && div <= 0x1.fffffep127f) ? band : -1.f;
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float d = x[e] - mn;
    const float q = d * r;
    t[e] = rintf(q);
    if (__ballot(!(fabsf(q - t[e]) < thr))) t[e] = fminf(rintf(d / div), levels);
  }
  // codes to bytes (each t is an integer in 0 .. 255: the conversion is exact)
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo = __builtin_amdgcn_cvt_pk_u8_f32(t[e], e, lo);
    hi = __builtin_amdgcn_cvt_pk_u8_f32(t[4 + e], e, hi);
  }
  if (!eight) {
    // nibbles: byte 0 of w | w >> 4 is v0 | v1 << 4, byte 2 is v2 | v3 << 4
    const uint32_t lw = lo | (lo >> 4), hw = hi | (hi >> 4);
    lo = __builtin_amdgcn_perm(hw, lw, 0x06040200u);
  }
  return Codes8{lo, hi, scale, mn};
}

// Store the lane's codes, and from the group's first lane the (scale, offset)
// pair, into the record rec of a D-value vector.
template <int D, int GS>
__device__ __forceinline__ void store_codes8(const Codes8& q, int c, int bits, char* rec) {
  constexpr int LPG = GS / 8;  // lanes per group
  if (bits == 8)
    store_global(rec + 8 * c, make_uint2(q.lo, q.hi));
  else
    store_global(rec + 4 * c, q.lo);
  if (c % LPG == 0) store_global(rec + D * bits / 8 + 8 * (c / LPG), make_float2(q.scale, q.offset));
}

// Quantise the lane's 8 values and, when rec is not null, store them (see
// quantise8 and store_codes8).
template <int D, int GS>
__device__ __forceinline__ void quantise_store8(const float (&x)[8], int c, int bits, char* rec) {
  const Codes8 q = quantise8<D, GS>(x, c, bits);
  if (rec) store_codes8<D, GS>(q, c, bits, rec);
}

}  // namespace pagedkv
