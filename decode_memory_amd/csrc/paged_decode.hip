// paged_decode for 16-bit pools, column kernel (one kv head per workgroup; the
// general shape fallback of the row kernel) and the split-K combine kernel.
//
// Operation (mlxcel issue #2171, "refactor: one KV storage abstraction with
// dense and paged backends", section "Proposed Solution": attend(q, k, v,
// scale, mask) with one query token and no mask; mlxcel issue #235, section
// "Proposed solution: chunked slabs", touch point 4: the fused kernel reads
// the pool through per-slab base pointers):
//   o[b, h] = sum_t softmax_t(scale * q[b,h] . K_b[t, h/G]) V_b[t, h/G]
//
// Work decomposition (flash-decoding): the token axis of every (sequence,
// kv head) pair is cut into n_split ranges of blocks_per_split blocks.  One
// workgroup (4 waves) owns one (sequence, kv head, split) and all G query
// heads of that kv head, so every K/V byte is read from HBM exactly once.
// Inside the workgroup the waves take the split's blocks round-robin.  For a
// block a wave resolves row -> (slab, row_in_slab) -> slab base pointer and
// streams the block's K and V token-head vectors straight from HBM into
// registers, 16 bytes per lane (D/8 lanes per token, so every token-head
// vector is one contiguous 2*D-byte segment).  q.k is a per-lane partial dot
// product finished with DPP row reductions; the softmax is online (running
// max and sum in the exp2 domain).  The four waves merge through LDS and the
// workgroup writes one (max, sum, acc[D]) partial per query head.
//
// A second kernel combines the splits of each (sequence, kv head) in split
// order, so the result does not depend on timing.  (Merging inside the split
// kernel through an arrival counter needs the partials to cross XCDs within
// the launch: with an agent-scope release fence per workgroup, which writes
// back the XCD's whole L2, or with device-scope write-through stores; the
// latter works but the last workgroup of a sequence then pulls every split's
// partial through one CU, which costs as much as this launch.)
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Register budget: waves per SIMD the split kernel must fit (3 -> up to 168
// VGPRs, 3 workgroups of 4 waves per CU, 768 resident on 256 CUs).
#ifndef PAGEDKV_DECODE_WAVES_PER_SIMD
#define PAGEDKV_DECODE_WAVES_PER_SIMD 3
#endif
// Loads of 16 bytes per lane in flight per sub-tile (K and V each).
#ifndef PAGEDKV_DECODE_LOADS
#define PAGEDKV_DECODE_LOADS 8
#endif
constexpr int kMinWavesPerSimd = PAGEDKV_DECODE_WAVES_PER_SIMD;
constexpr int kLoads = PAGEDKV_DECODE_LOADS;

// 16-byte load from global memory at a uniform base plus a per-lane offset;
// non-temporal, since each K/V byte is read once per call.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(const char* base, uint32_t off) {
  const u32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Lane j's 64-bit value as a wave-uniform pointer (j must be uniform).
__device__ __forceinline__ const char* lane_ptr(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), j);
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int D, int G, bool BF16, int BS>
__global__ __launch_bounds__(kThreads, kMinWavesPerSimd) void paged_decode_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;                       // lanes per token (16 B each)
  constexpr int TPW = kWave / LPT;                 // tokens per wave-wide load
  constexpr int U = (BS / TPW) < kLoads ? (BS / TPW) : kLoads;  // loads per sub-tile
  constexpr int SUB = TPW * U;                     // tokens per sub-tile
  constexpr int NSUB = BS / SUB;
  static_assert(BS % SUB == 0 && U >= 1, "block size must be a multiple of the tile");

  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ float s_acc[kWaves][G][D];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c = lane % LPT;   // which 16-byte chunk of the head vector
  const int ts = lane / LPT;  // which token of a wave-wide load

  const LayerView& lv = a.lv;
  const int n_kv = lv.n_kv;
  const int total = a.B * n_kv * a.n_split;
  const int w = xcd_work_id(blockIdx.x, gridDim.x);
  if (w >= total) return;
  const int s = w % a.n_split;
  const int bg = w / a.n_split;  // b * n_kv + g
  const int g = bg % n_kv;
  const int b = bg / n_kv;
  const int n_split = a.n_split;
  const int32_t* trow = a.table + static_cast<size_t>(b) * a.max_blocks;

  // Issue the independent loads together: the sequence length, the rows of
  // this split's blocks (split s takes logical blocks s, s + n_split, ...;
  // one per lane; in bounds of the table whatever the length turns out to
  // be) and the query.
  int len = a.lens[b];
  int row = -1;
  {
    const int blk = s + lane * n_split;
    if (lane < a.blocks_per_split && blk < a.max_blocks) row = trow[blk];
  }
  uint4 qv[G];  // this lane's 8 query values of each head, raw 16-bit
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<size_t>(b) * a.n_q + g * G) * D + c * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const uint4*>(q + h * D);
  }

  // Resolve each lane's row through its slab's base pointer (rows outside the
  // pool resolve to null and are reported below if they are visible).
  const size_t tok_stride = static_cast<size_t>(n_kv) * D * 2;  // bytes between tokens
  const size_t row_bytes = static_cast<size_t>(BS) * tok_stride;
  uint64_t kaddr = 0, vaddr = 0;
  if (row >= 0 && row < lv.capacity_rows) {
    const int slab = row / lv.slab_blocks;
    const size_t off = (row - slab * lv.slab_blocks) * row_bytes + static_cast<size_t>(g) * D * 2;
    kaddr = reinterpret_cast<uint64_t>(lv.k_tab[slab]) + off;
    vaddr = reinterpret_cast<uint64_t>(lv.v_tab[slab]) + off;
  }

  // A length beyond what the block table or the split plan can hold (the
  // caller's max_len was too small) is clamped and flagged; the workspace is
  // sized for the plan, so nothing is written outside it.
  const int cap_len = min(a.max_blocks, n_split * a.blocks_per_split) * BS;
  if (len < 0 || len > cap_len) {
    if (threadIdx.x == 0 && s == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + BS - 1) / BS;
  if (s >= nb) return;  // inactive split
  const int nblk = (nb - s + n_split - 1) / n_split;  // blocks of this split

  const float scale_log2 = a.scale_log2;
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  // per-lane byte offset of load u of sub-tile 0 inside a token-head column
  const uint32_t lane_off = static_cast<uint32_t>(ts * tok_stride + c * 16);
  const uint32_t load_step = static_cast<uint32_t>(TPW * tok_stride);

  for (int j = wave; j < nblk; j += kWaves) {
    const char* kb = lane_ptr(kaddr, j);
    const char* vb = lane_ptr(vaddr, j);
    if (kb == nullptr) {  // a visible block whose row is outside the pool
      if (lane == 0) set_error(lv.err, PD_DEVERR_TABLE_ROW);
      continue;
    }
    const int nt = min(BS, len - (s + j * n_split) * BS);  // visible tokens in this block

#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      if (sub * SUB >= nt) break;
      const uint32_t sub_off = lane_off + static_cast<uint32_t>(sub * SUB * tok_stride);
      uint4 kr[U], vr[U];
      if (nt == BS) {
#pragma unroll
        for (int u = 0; u < U; ++u) kr[u] = gload16(kb, sub_off + u * load_step);
#pragma unroll
        for (int u = 0; u < U; ++u) vr[u] = gload16(vb, sub_off + u * load_step);
      } else {
        // ragged last block: invisible tokens are neither loaded nor used
#pragma unroll
        for (int u = 0; u < U; ++u) {
          kr[u] = make_uint4(0, 0, 0, 0);
          vr[u] = make_uint4(0, 0, 0, 0);
          if (sub * SUB + u * TPW + ts < nt) {
            kr[u] = gload16(kb, sub_off + u * load_step);
            vr[u] = gload16(vb, sub_off + u * load_step);
          }
        }
      }

      // scores of this lane's tokens for the G heads (log2 domain)
      float sc[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool visible = sub * SUB + u * TPW + ts < nt;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float d = group_sum<LPT>(dot8<BF16>(qv[h], kr[u], 0.f));
          sc[u][h] = visible ? d * scale_log2 : -INFINITY;
        }
      }

#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = sc[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][h]);
        mx = across_groups_max<LPT>(mx);
        const float m_new = fmaxf(m[h], mx);       // finite: token sub*SUB is visible
        const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);  // 0 on the first tile
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = __builtin_amdgcn_exp2f(sc[u][h] - m_new);
          l[h] += p;
          float vf[8];
          widen8<BF16>(vr[u], vf);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    }
  }

  // Merge the token groups of the wave: every lane of a group holds the same
  // l (its tokens' weights) and its own chunk of acc.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = across_groups_sum<LPT>(l[h]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = across_groups_sum<LPT>(acc[h][e]);
  }
  if (ts == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][c * 8 + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // Merge the waves and write this split's partial for each query head
  // (partials are laid out [B * n_q][n_split][D + 4]).
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, s_m[wv][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) {
      const float mw = s_m[wv][h];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = fmaf(s_l[wv][h], f, L);
      A = fmaf(s_acc[wv][h][d], f, A);
    }
    const size_t hs = (static_cast<size_t>(b) * a.n_q + g * G + h) * n_split + s;
    a.partials[hs * D + d] = A;
    if (d == 0) {
      a.partials[a.ml_offset + hs * 2] = M;
      a.partials[a.ml_offset + hs * 2 + 1] = L;
    }
  }
}

// Split-K combine.  One wave owns 64 output columns of one (sequence, query
// head): lane j holds column j of the chunk.  Everything it needs is
// requested at once -- the (max, sum) of every active split (one per lane,
// coalesced) and its column of the first kCChunk splits' weighted V -- so the
// pass costs about one memory round trip and has no LDS or barrier.  The
// maxima are reduced across the wave (a fixed butterfly), each split's weight
// exp2(m_s - M) is broadcast from the lane that holds it, and every lane sums
// its column in split order -- the result does not depend on timing -- and
// rounds once to the q dtype.  Empty sequences get zeros.
constexpr int kCChunk = 32;                 // splits whose values a lane holds at once
constexpr int kCWaves = 4;                  // waves per combine workgroup

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = kWave / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// KM: (max, sum) pairs a lane holds, splits / 64 rounded up (the launch
// picks the smallest that covers the call's splits)
template <int D, bool BF16, int KM>
__global__ __launch_bounds__(kCWaves * kWave) void combine_kernel(DecodeArgs a) {
  constexpr int CH = D / kWave;  // 64-column chunks per query head
  const int lane = threadIdx.x % kWave;
  // the split kernel's work ids are (sequence, head set, split) in order and
  // XCD x runs a contiguous range of them; the same mapping here gives XCD x
  // the combine of those sequences, whose partials are still in its L2
  const int wg = xcd_work_id(blockIdx.x, gridDim.x);
  const int item = wg * kCWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int total = a.B * a.n_q;
  if (item >= total * CH) return;
  const int hq = item / CH;                 // (sequence, query head) index
  const int col = (item % CH) * kWave + lane;
  const int n_split = a.n_split;
  const int BS = a.lv.block_size;
  const int cap_len = min(a.max_blocks, n_split * a.blocks_per_split) * BS;
  int len = a.lens[hq / a.n_q];
  len = len < 0 ? 0 : (len > cap_len ? cap_len : len);
  const int n_act = min(n_split, (len + BS - 1) / BS);
  uint16_t* out = static_cast<uint16_t*>(a.out) + static_cast<size_t>(hq) * D + col;

  const float* acc = a.partials + static_cast<size_t>(hq) * n_split * D + col;
  const float2* ml = reinterpret_cast<const float2*>(a.partials + a.ml_offset) +
                     static_cast<size_t>(hq) * n_split;
  // requests first: the first kCChunk splits' values (in bounds of the
  // workspace whatever the length is; inactive splits are never used) and
  // the (max, sum) pairs, one split per lane
  float v[kCChunk];
#pragma unroll
  for (int k = 0; k < kCChunk; ++k) v[k] = k < n_split ? acc[static_cast<size_t>(k) * D] : 0.f;
  float mm[KM], ll[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int sp = lane + k * kWave;
    const float2 x = sp < n_act ? ml[sp] : make_float2(-INFINITY, 0.f);
    mm[k] = x.x;
    ll[k] = x.y;
  }
  if (n_act == 0) {
    *out = 0;
    return;
  }
  float M = mm[0];
#pragma unroll
  for (int k = 1; k < KM; ++k) M = fmaxf(M, mm[k]);
  M = wave_max(M);
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    // a split whose rows were all rejected carries (-inf, 0, 0)
    mm[k] = (mm[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mm[k] - M);
    L = fmaf(ll[k], mm[k], L);
  }
  L = wave_sum(L);
  // weight of split sp: mm[sp / 64] of lane sp % 64
  auto weight = [&](int sp) {
    float w = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (sp / kWave == k) w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mm[k]), sp % kWave));
    return w;
  };
  float A = 0.f;
#pragma unroll
  for (int k = 0; k < kCChunk; ++k)
    if (k < n_act) A = fmaf(v[k], weight(k), A);
  for (int sp = kCChunk; sp < n_act; ++sp) A = fmaf(acc[static_cast<size_t>(sp) * D], weight(sp), A);
  *out = f32_to_out<BF16>(A * (L > 0.f ? 1.f / L : 0.f));
}

template <int D, int G, bool BF16, int BS>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
  const int total = a.B * a.lv.n_kv * a.n_split;
  const int grid = round_up(total, kXcds);
  hipLaunchKernelGGL((paged_decode_kernel<D, G, BF16, BS>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_combine_typed(const DecodeArgs& a, hipStream_t s) {
  const long long waves = static_cast<long long>(a.B) * a.n_q * (D / kWave);
  const int grid = round_up(static_cast<int>((waves + kCWaves - 1) / kCWaves), kXcds);
  static_assert(kMaxSplits <= 16 * kWave, "combine holds at most 16 (max, sum) pairs per lane");
  const int km = (a.n_split + kWave - 1) / kWave;
  if (km <= 1)
    hipLaunchKernelGGL((combine_kernel<D, BF16, 1>), dim3(grid), dim3(kCWaves * kWave), 0, s, a);
  else if (km <= 2)
    hipLaunchKernelGGL((combine_kernel<D, BF16, 2>), dim3(grid), dim3(kCWaves * kWave), 0, s, a);
  else if (km <= 4)
    hipLaunchKernelGGL((combine_kernel<D, BF16, 4>), dim3(grid), dim3(kCWaves * kWave), 0, s, a);
  else if (km <= 8)
    hipLaunchKernelGGL((combine_kernel<D, BF16, 8>), dim3(grid), dim3(kCWaves * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((combine_kernel<D, BF16, 16>), dim3(grid), dim3(kCWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int D, int G, bool BF16>
hipError_t by_block(const DecodeArgs& a, hipStream_t s) {
  switch (a.lv.block_size) {
    case 16: return launch_typed<D, G, BF16, 16>(a, s);
    case 32: return launch_typed<D, G, BF16, 32>(a, s);
    case 64: return launch_typed<D, G, BF16, 64>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool BF16>
hipError_t by_group(const DecodeArgs& a, int32_t group, hipStream_t s) {
  switch (group) {
    case 1: return by_block<D, 1, BF16>(a, s);
    case 2: return by_block<D, 2, BF16>(a, s);
    case 4: return by_block<D, 4, BF16>(a, s);
    case 8: return by_block<D, 8, BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
hipError_t by_dim(const DecodeArgs& a, int32_t head_dim, int32_t group, hipStream_t s) {
  switch (head_dim) {
    case 64: return by_group<64, BF16>(a, group, s);
    case 128: return by_group<128, BF16>(a, group, s);
    case 256: return by_group<256, BF16>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool BF16>
hipError_t combine_by_dim(const DecodeArgs& a, int32_t head_dim, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_combine_typed<64, BF16>(a, s);
    case 128: return launch_combine_typed<128, BF16>(a, s);
    case 256: return launch_combine_typed<256, BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_paged_decode_column(const DecodeArgs& a, bool bf16, int32_t head_dim,
                                      int32_t group, hipStream_t s) {
  return bf16 ? by_dim<true>(a, head_dim, group, s) : by_dim<false>(a, head_dim, group, s);
}

hipError_t launch_decode_combine(const DecodeArgs& a, bool bf16, int32_t head_dim, hipStream_t s) {
  return bf16 ? combine_by_dim<true>(a, head_dim, s) : combine_by_dim<false>(a, head_dim, s);
}

}  // namespace pagedkv
