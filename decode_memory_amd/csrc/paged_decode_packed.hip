// paged_decode for packed pools (K8/V8, K8/V4, K4/V4): attention that reads
// the packed pages directly and dequantises values as it reads them.
//
// mlx-swift-lm PR #142 ("Add packed paged KV formats with bounded workspace
// admission"), section "Summary" and the "After" flowchart: direct attention
// consumes packed pages without expanding the history; keys were rotated by a
// fixed signed Hadamard basis before they were quantised, so the query gets
// the same rotation (q'.k' = q.k) and values, stored unrotated, need no
// inverse.  Record of one token-head: codes (8-bit bytes, or 4-bit nibbles
// with value 2i in the low nibble of byte i), then (fp32 scale, fp32 offset)
// per group of 32 values; a value is code * scale + offset.
//
// Decomposition.  A workgroup (4 waves) owns (sequence, split of the token
// axis) and every kv head; split s takes logical blocks s, s + n_split, ...
// Packed records are short (48..320 bytes), so a tile of T tokens x n_kv
// heads is first copied into LDS with 16-byte coalesced loads of whole token
// rows (the rows of a block are contiguous in the slab; the next tile's loads
// are in flight while the current one is computed), and the waves then
// read codes and group metadata from LDS in the layout the arithmetic wants:
// a lane group of D/8 lanes owns one kv head, each lane 8 consecutive values
// (one group of 32 spans 4 lanes).  The affine terms are folded so that each
// value costs one unpack/convert plus one FMA per query head:
//   q'.k  = sum_lanes [ scale_g * (q'_lane . c_lane) + offset_g * sum(q'_lane) ]
//   acc  += (p * scale_g) * c   and a per-lane bias   sum_t p_t * offset_g
// The query is rotated in the prologue with an fp32 fast Walsh-Hadamard
// transform (within-lane stages for h < 8, DPP/shuffle stages above).
// Partials go to the same workspace layout as the 16-bit kernels and the same
// combine kernel merges them.
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

namespace {

constexpr int kPThreads = 256;
constexpr int kPWaves = kPThreads / kWave;
constexpr int kPBS = 32;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ const char* lane_ptr(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), j);
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Byte k of a dword as a float (one v_cvt_f32_ubyte<k> after instruction
// selection).
template <int K>
__device__ __forceinline__ float ubyte(uint32_t w) {
  return static_cast<float>((w >> (8 * K)) & 0xffu);
}

// 8 codes of a lane as floats.  BITS 8: two dwords of bytes; BITS 4: one dword
// of nibbles, element 2i in the low nibble of byte i.
template <int BITS>
__device__ __forceinline__ void codes8(const uint32_t* w, float (&c)[8]) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c[4 * i + 0] = ubyte<0>(w[i]);
      c[4 * i + 1] = ubyte<1>(w[i]);
      c[4 * i + 2] = ubyte<2>(w[i]);
      c[4 * i + 3] = ubyte<3>(w[i]);
    }
  } else {
    const uint32_t lo = w[0] & 0x0f0f0f0fu, hi = (w[0] >> 4) & 0x0f0f0f0fu;
    c[0] = ubyte<0>(lo);
    c[1] = ubyte<0>(hi);
    c[2] = ubyte<1>(lo);
    c[3] = ubyte<1>(hi);
    c[4] = ubyte<2>(lo);
    c[5] = ubyte<2>(hi);
    c[6] = ubyte<3>(lo);
    c[7] = ubyte<3>(hi);
  }
}

template <int D, int KB, int VB, int G>
__global__ __launch_bounds__(kPThreads) void paged_decode_packed_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;           // lanes per head (8 values each)
  constexpr int HPW = kWave / LPT;     // heads per wave
  constexpr int KREC = D * KB / 8 + (D / 32) * 8;
  constexpr int VREC = D * VB / 8 + (D / 32) * 8;
  constexpr int T = D == 64 ? 16 : (D == 128 ? 8 : 4);  // tokens per tile
  constexpr int NKV = 8;               // kv heads (the packed kernels take 8)
  constexpr int NHS = NKV / HPW;       // head slots
  constexpr int SLICES = kPWaves / NHS;  // waves per head slot (token slices)
  constexpr int KTILE = T * NKV * KREC;  // bytes of a K tile (whole token rows)
  constexpr int VTILE = T * NKV * VREC;
  static_assert(kPWaves % NHS == 0 && T % SLICES == 0, "tile shape");
  static_assert(KTILE % 16 == 0 && VTILE % 16 == 0, "tile must be whole 16-byte units");

  constexpr int KU = (KTILE / 16 + kPThreads - 1) / kPThreads;  // 16-byte units per thread
  constexpr int VU = (VTILE / 16 + kPThreads - 1) / kPThreads;
  __shared__ __attribute__((aligned(16))) unsigned char s_kbuf[2][KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char s_vbuf[2][VTILE];
  __shared__ float s_m[kPWaves][HPW * G];
  __shared__ float s_l[kPWaves][HPW * G];
  __shared__ float s_acc[kPWaves][HPW * G][D];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hs = wave % NHS;       // head slot of this wave
  const int slice = wave / NHS;    // token slice of this wave
  const int c = lane % LPT;        // 8-value chunk
  const int lg = lane / LPT;
  const int head = hs * HPW + lg;  // kv head of this lane
  const int grp = c / 4;           // group of 32 values

  const LayerView& lv = a.lv;
  const int n_split = a.n_split;
  const int w = xcd_work_id(blockIdx.x, gridDim.x);
  if (w >= a.B * n_split) return;
  const int s = w % n_split;
  const int b = w / n_split;
  const int32_t* trow = a.table + static_cast<size_t>(b) * a.max_blocks;

  int len = a.lens[b];
  int row = -1;
  {
    const int blk = s + lane * n_split;
    if (lane < a.blocks_per_split && blk < a.max_blocks) row = trow[blk];
  }

  // Query: widen, apply the signs, rotate (fp32 FWHT over the D/8 lanes of
  // the head), normalise; keep q' and the per-lane sums of q' (offset term).
  float qr[G][8], qpart[G];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<size_t>(b) * a.n_q + head * G) * D + c * 8;
    float sg[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sg[e] = a.signs[c * 8 + e];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      widen8<true>(*reinterpret_cast<const uint4*>(q + j * D), qr[j]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[j][e] *= sg[e];
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {  // within the lane
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (e & h) ? qr[j][e ^ h] - qr[j][e] : qr[j][e] + qr[j][e ^ h];
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[j][e] = y[e];
      }
#pragma unroll
      for (int hl = 1; hl < LPT; hl <<= 1) {  // across lanes of the head
        const bool upper = (c & hl) != 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o = __shfl_xor(qr[j][e], hl, kWave);
          qr[j][e] = upper ? o - qr[j][e] : qr[j][e] + o;
        }
      }
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qr[j][e] *= a.inv_sqrt_d * a.scale_log2;  // scores in the exp2 domain
        sum += qr[j][e];
      }
      qpart[j] = sum;
    }
  }

  const size_t k_row_bytes = static_cast<size_t>(kPBS) * NKV * KREC;
  const size_t v_row_bytes = static_cast<size_t>(kPBS) * NKV * VREC;
  const bool row_ok = row >= 0 && row < lv.capacity_rows;
  uint64_t kaddr = 0, vaddr = 0;
  if (lv.capacity_rows > 0) {
    const int r = row_ok ? row : 0;  // rows outside the pool read row 0 and are masked
    const int slab = r / lv.slab_blocks;
    kaddr = reinterpret_cast<uint64_t>(lv.k_tab[slab]) + (r - slab * lv.slab_blocks) * k_row_bytes;
    vaddr = reinterpret_cast<uint64_t>(lv.v_tab[slab]) + (r - slab * lv.slab_blocks) * v_row_bytes;
  }

  const int cap_len = min(a.max_blocks, n_split * a.blocks_per_split) * kPBS;
  if (len < 0 || len > cap_len) {
    if (threadIdx.x == 0 && s == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + kPBS - 1) / kPBS;
  if (s >= nb) return;
  const int nblk = (nb - s + n_split - 1) / n_split;
  const uint64_t ok_mask = __ballot(row_ok);
  if (wave == 0 && lane < nblk && !row_ok) set_error(lv.err, PD_DEVERR_TABLE_ROW);
  const int n_tiles = lv.capacity_rows > 0 ? nblk * (kPBS / T) : 0;

  float m[G], l[G], acc[G][8], bias[G];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
    bias[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  }

  // Tile i+1 is loaded into registers (non-temporal: read once) while tile i
  // is computed from LDS; two LDS buffers, one barrier per tile.
  u32x4 rk[KU], rv[VU];
  auto fetch = [&](int i) {
    const int jb = i / (kPBS / T);
    const int t0 = (i % (kPBS / T)) * T;
    const gu32x4* kb = (const gu32x4*)(lane_ptr(kaddr, jb) + static_cast<size_t>(t0) * NKV * KREC);
    const gu32x4* vb = (const gu32x4*)(lane_ptr(vaddr, jb) + static_cast<size_t>(t0) * NKV * VREC);
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = threadIdx.x + j * kPThreads;
      if (u < KTILE / 16) rk[j] = __builtin_nontemporal_load(kb + u);
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = threadIdx.x + j * kPThreads;
      if (u < VTILE / 16) rv[j] = __builtin_nontemporal_load(vb + u);
    }
  };
  if (n_tiles > 0) fetch(0);
  for (int i = 0; i < n_tiles; ++i) {
    const int jb = i / (kPBS / T);
    const int t0 = (i % (kPBS / T)) * T;  // first token of the tile in the block
    const int nt = ((ok_mask >> jb) & 1) ? min(kPBS, len - (s + jb * n_split) * kPBS) : 0;
    unsigned char* s_k = s_kbuf[i & 1];
    unsigned char* s_v = s_vbuf[i & 1];
    // buffer i&1 was last read in iteration i-2, before every wave passed
    // the barrier of iteration i-1
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const int u = threadIdx.x + j * kPThreads;
      if (u < KTILE / 16) reinterpret_cast<u32x4*>(s_k)[u] = rk[j];
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = threadIdx.x + j * kPThreads;
      if (u < VTILE / 16) reinterpret_cast<u32x4*>(s_v)[u] = rv[j];
    }
    if (i + 1 < n_tiles) fetch(i + 1);
    __syncthreads();
    if (t0 >= nt) continue;  // uniform: the whole tile is past the length

    // this wave's tokens of the tile: slice, slice + SLICES, ...
    constexpr int TW = T / SLICES;
    float sc[G][TW];
    float voff[TW], vscale[TW];
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = slice + u * SLICES;
      const unsigned char* kr = s_k + (t * NKV + head) * KREC;
      uint32_t kw[2];
      if constexpr (KB == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(kr + c * 8);
        kw[0] = x.x;
        kw[1] = x.y;
      } else {
        kw[0] = *reinterpret_cast<const uint32_t*>(kr + c * 4);
        kw[1] = 0;
      }
      const float2 km = *reinterpret_cast<const float2*>(kr + D * KB / 8 + grp * 8);
      float cf[8];
      codes8<KB>(kw, cf);
      const unsigned char* vr = s_v + (t * NKV + head) * VREC;
      const float2 vm = *reinterpret_cast<const float2*>(vr + D * VB / 8 + grp * 8);
      vscale[u] = vm.x;
      voff[u] = vm.y;
      const bool vis = t0 + t < nt;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d = fmaf(qr[j][e], cf[e], d);
        d = fmaf(km.x, d, km.y * qpart[j]);
        d = group_sum<LPT>(d);
        sc[j][u] = vis ? d : -INFINITY;
      }
    }
    float p[G][TW];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float mx = sc[j][0];
#pragma unroll
      for (int u = 1; u < TW; ++u) mx = fmaxf(mx, sc[j][u]);
      const float m_new = fmaxf(m[j], mx);  // -inf while nothing this wave saw is visible
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m[j] - m_new);
      m[j] = m_new;
      l[j] *= alpha;
      bias[j] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= alpha;
#pragma unroll
      for (int u = 0; u < TW; ++u) {
        p[j][u] = (sc[j][u] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[j][u] - m_new);
        l[j] += p[j][u];
      }
    }
#pragma unroll
    for (int u = 0; u < TW; ++u) {
      const int t = slice + u * SLICES;
      const unsigned char* vr = s_v + (t * NKV + head) * VREC;
      uint32_t vw[2];
      if constexpr (VB == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(vr + c * 8);
        vw[0] = x.x;
        vw[1] = x.y;
      } else {
        vw[0] = *reinterpret_cast<const uint32_t*>(vr + c * 4);
        vw[1] = 0;
      }
      float cf[8];
      codes8<VB>(vw, cf);
      const bool vis = t0 + t < nt;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        // invisible tokens contribute nothing even if their metadata is garbage
        const float as = vis ? p[j][u] * vscale[u] : 0.f;
        bias[j] += vis ? p[j][u] * voff[u] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = fmaf(as, cf[e], acc[j][e]);
      }
    }
  }

  // Stage per-wave state (with the offset bias folded in), merge the slices.
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const int hq = lg * G + j;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[wave][hq][c * 8 + e] = acc[j][e] + bias[j];
    if (c == 0) {
      s_m[wave][hq] = m[j];
      s_l[wave][hq] = l[j];
    }
  }
  __syncthreads();
  float* part_acc = a.partials;
  float* part_ml = a.partials + a.ml_offset;
  for (int idx = threadIdx.x; idx < NKV * G * D; idx += kPThreads) {
    const int d = idx % D;
    const int hq = (idx / D) % (HPW * G);
    const int slot = idx / (D * HPW * G);
    float M = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < SLICES; ++sl) M = fmaxf(M, s_m[sl * NHS + slot][hq]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int sl = 0; sl < SLICES; ++sl) {
      const int wv = sl * NHS + slot;
      const float mw = s_m[wv][hq];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = fmaf(s_l[wv][hq], f, L);
      A = fmaf(s_acc[wv][hq][d], f, A);
    }
    const size_t hsplit = (static_cast<size_t>(b) * a.n_q + slot * HPW * G + hq) * n_split + s;
    part_acc[hsplit * D + d] = A;
    if (d == 0) {
      part_ml[hsplit * 2] = M;
      part_ml[hsplit * 2 + 1] = L;
    }
  }
}

template <int D, int KB, int VB, int G>
hipError_t launch_packed(const DecodeArgs& a, hipStream_t s) {
  const int grid = round_up(a.B * a.n_split, kXcds);
  hipLaunchKernelGGL((paged_decode_packed_kernel<D, KB, VB, G>), dim3(grid), dim3(kPThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int KB, int VB>
hipError_t packed_by_group(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_packed<D, KB, VB, 1>(a, s);
    case 2: return launch_packed<D, KB, VB, 2>(a, s);
    case 4: return launch_packed<D, KB, VB, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KB, int VB>
hipError_t packed_by_dim(const DecodeArgs& a, int head_dim, int group, hipStream_t s) {
  switch (head_dim) {
    case 64: return packed_by_group<64, KB, VB>(a, group, s);
    case 128: return packed_by_group<128, KB, VB>(a, group, s);
    case 256: return packed_by_group<256, KB, VB>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool packed_decode_supported(int32_t n_kv, int32_t head_dim, int32_t group, int32_t block_size) {
  return n_kv == 8 && block_size == kPBS && (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4);
}

hipError_t launch_paged_decode_packed(const DecodeArgs& a, int32_t head_dim, int32_t group,
                                      hipStream_t s) {
  if (a.k_bits == 8 && a.v_bits == 8) return packed_by_dim<8, 8>(a, head_dim, group, s);
  if (a.k_bits == 8 && a.v_bits == 4) return packed_by_dim<8, 4>(a, head_dim, group, s);
  if (a.k_bits == 4 && a.v_bits == 4) return packed_by_dim<4, 4>(a, head_dim, group, s);
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
