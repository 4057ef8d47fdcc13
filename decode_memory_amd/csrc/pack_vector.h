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

// The Sylvester Hadamard butterfly network over a D-value vector held 8
// values per lane by D/8 lanes (lane c of the group: values 8c .. 8c+7):
// stages h = 1, 2, ..., D/2, each pair (a, b) -> (a + b, a - b) in fp32 (the
// lower index gets a + b).  Stages h < 8 pair values inside a lane, the
// others pair lanes c and c ^ (h / 8) of the vector's lane group.
template <int D>
__device__ __forceinline__ void fwht8(float (&x)[8], int c) {
  constexpr int LPT = D / 8;
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (e & h) ? __fsub_rn(x[e ^ h], x[e]) : __fadd_rn(x[e], x[e ^ h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = y[e];
  }
#pragma unroll
  for (int hl = 1; hl < LPT; hl <<= 1) {
    // the lower lane keeps x + other, the upper other - x: one fma with a
    // +-1 factor (exact product, one rounding) gives both
    const float sgn = (c & hl) ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float other = __shfl_xor(x[e], hl, kWave);
      x[e] = __fmaf_rn(sgn, x[e], other);
    }
  }
}

// x' = H diag(sigma) x / sqrt(D): the sign flips (exact), the butterfly
// network above, then one multiply by 1/sqrt(D).
template <int D>
__device__ __forceinline__ void fwht_rotate8(float (&x)[8], const float* signs, int c,
                                             float inv_sqrt_d) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= signs[8 * c + e];  // exact sign flips
  fwht8<D>(x, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __fmul_rn(x[e], inv_sqrt_d);
}

// The same with the lane's 8 signs already in registers.
template <int D>
__device__ __forceinline__ void fwht_rotate8(float (&x)[8], const float (&sg)[8], int c, float inv_sqrt_d) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= sg[e];  // exact sign flips
  fwht8<D>(x, c);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __fmul_rn(x[e], inv_sqrt_d);
}

// Quantise the lane's 8 values (values 8c .. 8c+7 of the vector) with the
// (scale, offset) of their group of GS values, all in fp32: mn = min, mx =
// max, scale = (mx - mn) / (2^bits - 1), offset = mn, code = clamp(rint((x -
// mn) / scale)) with round-half-even, and a constant group gets code 0.  When
// rec is not null the codes (8-bit: one byte per value; 4-bit: value 2i in
// the low nibble of byte i) and, from the group's first lane, the (scale,
// offset) pair are stored into the record rec of a D-value vector.
template <int D, int GS>
__device__ __forceinline__ void quantise_store8(const float (&x)[8], int c, int bits, char* rec) {
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
  mn = fminf(mn, dpp<kDppXor1>(mn));
  mx = fmaxf(mx, dpp<kDppXor1>(mx));
  mn = fminf(mn, dpp<kDppXor2>(mn));
  mx = fmaxf(mx, dpp<kDppXor2>(mx));
  if constexpr (LPG == 8) {
    mn = fminf(mn, dpp<kDppHalfMirror>(mn));
    mx = fmaxf(mx, dpp<kDppHalfMirror>(mx));
  }
  const float levels = static_cast<float>((1 << bits) - 1);
  const float scale = __fdiv_rn(__fsub_rn(mx, mn), levels);
  // a constant group (scale 0) gets code 0; it divides by 1 instead, so that
  // no lane branches
  const bool flat = scale == 0.f;
  const float div = flat ? 1.f : scale;
  // The code is rint of the correctly rounded quotient q = RN(d / div), d =
  // RN(x - mn) >= 0.  One correctly rounded reciprocal r = RN(1 / div) per
  // lane and a product q' = RN(d * r) give q' within 2.5 ulp(q) of q, and for
  // q < 256 that is below 2^-14.6, so rint(q') = rint(q) unless q' lies
  // within 2^-14 of a half-integer.  Such a value (about 1 in 8000) sends the
  // whole wave through the correctly rounded divisions.
  const float r = __fdiv_rn(1.f, div);
  float t[8];
  bool near = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = __fmul_rn(__fsub_rn(x[e], mn), r);
    near |= fabsf(__fsub_rn(q, floorf(q)) - 0.5f) <= 6.103515625e-05f;  // 2^-14
    t[e] = rintf(q);
  }
  if (__ballot(near)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = rintf(__fdiv_rn(__fsub_rn(x[e], mn), div));
  }
  uint32_t code[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = fminf(fmaxf(t[e], 0.f), levels);
    code[e] = flat ? 0u : static_cast<uint32_t>(c);
  }
  if (!rec) return;
  if (bits == 8) {
    *reinterpret_cast<uint2*>(rec + 8 * c) =
        make_uint2(code[0] | (code[1] << 8) | (code[2] << 16) | (code[3] << 24),
                   code[4] | (code[5] << 8) | (code[6] << 16) | (code[7] << 24));
  } else {
    *reinterpret_cast<uint32_t*>(rec + 4 * c) =
        (code[0] | (code[1] << 4)) | ((code[2] | (code[3] << 4)) << 8) |
        ((code[4] | (code[5] << 4)) << 16) | ((code[6] | (code[7] << 4)) << 24);
  }
  if (c % LPG == 0) {
    float* meta = reinterpret_cast<float*>(rec + D * bits / 8) + 2 * (c / LPG);
    *reinterpret_cast<float2*>(meta) = make_float2(scale, mn);
  }
}

}  // namespace pagedkv
