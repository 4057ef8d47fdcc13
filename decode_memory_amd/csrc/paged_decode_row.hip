// paged_decode, row-streaming kernel for 16-bit pools whose token row spans
// whole 1 KiB wave loads (n_kv * head_dim * 2 bytes a multiple of 1 KiB).
//
// Operation (mlxcel issue #2171, "refactor: one KV storage abstraction with
// dense and paged backends", section "Proposed Solution": attend(q, k, v,
// scale, mask) with one query token and no mask; mlxcel issue #235, section
// "Proposed solution: chunked slabs", touch point 4: the fused kernel reads
// the pool through per-slab base pointers):
//   o[b, h] = sum_t softmax_t(scale * q[b,h] . K_b[t, h/G]) V_b[t, h/G]
//
// Memory layout drives the decomposition.  A block row of a slab is
// [block_size, n_kv, head_dim]: the n_kv head vectors of one token are one
// contiguous n_kv*head_dim*2-byte run.  A workgroup (8 waves) owns
// (sequence, set of kv heads, split of the token axis) -- for the
// qwen3-shaped pools every kv head -- so it streams whole token rows: a
// wave-wide 16-byte-per-lane load covers 1 KiB (one head group) of one
// token, the waves of a head group take consecutive token slices of each
// block, and the head groups' waves read the other parts of the same rows at
// the same time.  A lane group (head_dim/8 lanes) owns one kv head for the
// whole split, so the online softmax state (running max, sum and the lane's 8
// output columns per query head) stays in the lane group: the only
// cross-lane operation per token is the DPP reduction that finishes each dot
// product.  Each wave keeps PAGEDKV_ROW_TILES_IN_FLIGHT tiles of K/V loads in
// flight (tile i + 1 is requested before tile i is consumed); with one
// 8-wave workgroup per CU that is 64-128 KiB of reads outstanding per CU.
// Deeper queues measured slower: with every CU streaming at once, more
// requests in flight only add contention.
//
// A block's address costs two dependent global reads: its row in the block
// table, then its slab's base pointer.  At the end each wave stages its state in LDS and, after one
// workgroup barrier, the waves of each head group merge the group's slices
// together, each wave a share of the columns, in slice order, and write one
// partial (max, sum, weighted V) per query head and split; a combine kernel
// merges the splits.
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

namespace {

#ifndef PAGEDKV_ROW_TILES_IN_FLIGHT
#define PAGEDKV_ROW_TILES_IN_FLIGHT 2
#endif
#ifndef PAGEDKV_ROW_WAVES
#define PAGEDKV_ROW_WAVES 8
#endif
// Most head groups (1 KiB of a token row each) one workgroup covers.
#ifndef PAGEDKV_ROW_MAX_HEAD_GROUPS
#define PAGEDKV_ROW_MAX_HEAD_GROUPS 4
#endif
#ifndef PAGEDKV_ROW_WAVES_PER_SIMD
#define PAGEDKV_ROW_WAVES_PER_SIMD 2
#endif
#ifndef PAGEDKV_ROW_TILE_TOKENS
#define PAGEDKV_ROW_TILE_TOKENS 4
#endif

constexpr int kRowWaves = PAGEDKV_ROW_WAVES;  // waves per workgroup
constexpr int kRowThreads = kRowWaves * kWave;
constexpr int kTile = PAGEDKV_ROW_TILE_TOKENS;  // tokens per wave per tile
constexpr int kBuf = PAGEDKV_ROW_TILES_IN_FLIGHT;  // tiles a wave keeps in flight
constexpr int kBS = 32;                      // tokens per block

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// K/V bytes are read once per call: non-temporal loads keep them from
// displacing the block tables, slab pointers and partials in L2.
__device__ __forceinline__ uint4 gload16(const char* base, uint32_t off) {
  const u32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ const char* lane_ptr(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), j);
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// One tile: kTile tokens of one block, the HPL kv heads of one head group,
// K and V (16 bytes per lane and token each).
struct Tile {
  uint4 k[kTile];
  uint4 v[kTile];
};

// D: head_dim, G: query heads per kv head, HGW: head groups (of HPL =
// 64/(D/8) kv heads, one 1 KiB wave load per token) per workgroup.
template <int D, int G, bool BF16, int HGW>
__global__ __launch_bounds__(kRowThreads, PAGEDKV_ROW_WAVES_PER_SIMD) void paged_decode_row_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;              // lanes per head vector (16 B each)
  constexpr int HPL = kWave / LPT;        // kv heads per wave load
  constexpr int HG = HPL * HGW;           // kv heads per workgroup
  constexpr int SLICES = kRowWaves / HGW; // waves sharing one head group
  constexpr int NT = kBS / (SLICES * kTile);  // tiles per block per wave
  static_assert(kRowWaves % HGW == 0 && NT >= 1 && NT * SLICES * kTile == kBS, "tile shape");

  __shared__ float s_m[kRowWaves][HPL * G];
  __shared__ float s_l[kRowWaves][HPL * G];
  __shared__ float s_acc[kRowWaves][HPL * G][D];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hgw = wave % HGW;     // this wave's head group inside the workgroup
  const int slice = wave / HGW;   // this wave's share of every block's tiles
  const int c = lane % LPT;       // 16-byte chunk of the head vector
  const int lg = lane / LPT;      // kv head inside the head group

  const LayerView& lv = a.lv;
  const int n_kv = lv.n_kv;
  const int n_sets = n_kv / HG;
  const int n_split = a.n_split;
  const int w = xcd_work_id(blockIdx.x, gridDim.x);
  if (w >= a.B * n_sets * n_split) return;
  const int s = w % n_split;
  const int bh = w / n_split;
  const int hset = bh % n_sets;
  const int b = bh / n_sets;
  const int kvh = hset * HG + hgw * HPL + lg;  // this lane group's kv head
  // without a block table (dense sequences) block j of sequence b is row
  // b * slab_blocks + j
  const int32_t* trow = a.table ? a.table + static_cast<size_t>(b) * a.max_blocks : nullptr;

  // Independent loads first: the length, the rows of this split's blocks
  // (split s takes logical blocks s, s + n_split, ...; one per lane), the
  // query.
  int len = a.lens[b];
  int row = -1;
  {
    const int blk = s + lane * n_split;
    if (lane < a.blocks_per_split && blk < a.max_blocks) row = trow ? trow[blk] : b * lv.slab_blocks + blk;
  }
  uint4 qv[G];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) +
                        (static_cast<size_t>(b) * a.n_q + kvh * G) * D + c * 8;
#pragma unroll
    for (int j = 0; j < G; ++j) qv[j] = *reinterpret_cast<const uint4*>(q + j * D);
  }

  const uint32_t tok_bytes = static_cast<uint32_t>(n_kv) * D * 2;
  const size_t row_bytes = static_cast<size_t>(kBS) * tok_bytes;
  const bool row_ok = row >= 0 && row < lv.capacity_rows;

  // The block's address: its slab's base pointer, read from the layer's
  // table as soon as the row is known (each lane its own block), plus the
  // row's offset in the slab.  Reading the pointers straight from global
  // memory beat staging the whole table in LDS behind a workgroup barrier.
  uint64_t kaddr = 0, vaddr = 0;
  if (lv.capacity_rows > 0) {
    // a row outside the pool is read as row 0 of slab 0 and masked below
    const int r = row_ok ? row : 0;
    const int slab = r / lv.slab_blocks;
    const size_t off = (r - slab * lv.slab_blocks) * row_bytes;
    kaddr = reinterpret_cast<uint64_t>(lv.k_tab[slab]) + off;
    vaddr = reinterpret_cast<uint64_t>(lv.v_tab[slab]) + off;
  }

  const int cap_len = min(a.max_blocks, n_split * a.blocks_per_split) * kBS;
  const bool len_ok = len >= 0 && len <= cap_len;
  if (!len_ok) {
    if (threadIdx.x == 0 && s == 0 && hset == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + kBS - 1) / kBS;
  if (s >= nb) return;  // inactive split
  const int nblk = (nb - s + n_split - 1) / n_split;  // blocks of this split
  const uint64_t ok_mask = __ballot(row_ok);
  if (wave == 0 && lane < nblk && !row_ok) set_error(lv.err, PD_DEVERR_TABLE_ROW);
  const int n_tiles = lv.capacity_rows > 0 ? nblk * NT : 0;

  const float scale_log2 = a.scale_log2;
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }
  const uint32_t lane_off = static_cast<uint32_t>(kvh * D * 2 + c * 16);

  // Fused append (pd_paged_decode_append): token len - 1 of the sequence is
  // new.  The workgroup whose split owns its block -- the only one that reads
  // those bytes -- stores this workgroup's kv heads of it (each head group's
  // slice-0 wave, 16 bytes per lane of K and of V, laid out [n_kv, D] as in
  // a token row) before any tile is requested; the stores are waited for
  // and a barrier orders them before every wave's loads.  A rejected length
  // or row appends nothing.
  if (a.k_new && len_ok && len > 0) {
    const int p = len - 1;
    const int jb = p / kBS;
    if (jb % n_split == s) {  // uniform over the workgroup
      const int jj = jb / n_split;  // this split's jj-th block
      if (slice == 0 && ((ok_mask >> jj) & 1)) {
        const size_t src = static_cast<size_t>(b) * tok_bytes + lane_off;
        const uint32_t off = lane_off + static_cast<uint32_t>(p % kBS) * tok_bytes;
        const uint4 kn = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src);
        const uint4 vn = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src);
        store_global(const_cast<char*>(lane_ptr(kaddr, jj)) + off, kn);
        store_global(const_cast<char*>(lane_ptr(vaddr, jj)) + off, vn);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have reached L2
      __syncthreads();
    }
  }

  // Tile i: block j = i / NT of the split, tokens (k*SLICES + slice)*kTile +
  // [0, kTile) with k = i % NT -- at any moment the slices of a head group
  // read one contiguous run of tokens.  Tokens past the visible length are
  // clamped to the last visible token (in bounds) and masked.
  // A tile past the last one (i >= n_tiles) is still requested -- see the
  // pipeline below -- but every lane reads the same 16 bytes at the start of
  // the query (valid memory of at least 128 bytes); its registers are never
  // used.
  const char* const dummy = static_cast<const char*>(a.q);
  auto load_tile = [&](Tile& t, int i) {
    const bool live = i < n_tiles;  // uniform over the wave
    const int ic = live ? i : 0;
    const int j = ic / NT, k = ic % NT;
    const char* kb = live ? lane_ptr(kaddr, j) : dummy;
    const char* vb = live ? lane_ptr(vaddr, j) : dummy;
    const int nt = min(kBS, len - (s + j * n_split) * kBS);
    const int t0 = (k * SLICES + slice) * kTile;
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
      const uint32_t off = live ? lane_off + min(t0 + u, nt - 1) * tok_bytes : 0u;
      t.k[u] = gload16(kb, off);
      t.v[u] = gload16(vb, off);
    }
  };

  auto compute_tile = [&](const Tile& t, int i) {
    const int j = i / NT, k = i % NT;
    const int nt = ((ok_mask >> j) & 1) ? min(kBS, len - (s + j * n_split) * kBS) : 0;
    const int t0 = (k * SLICES + slice) * kTile;
    float p[G][kTile];
#pragma unroll
    for (int jq = 0; jq < G; ++jq) {
      float sc[kTile];
#pragma unroll
      for (int u = 0; u < kTile; ++u) {
        const float d = group_sum<LPT>(dot8<BF16>(qv[jq], t.k[u], 0.f));
        sc[u] = (t0 + u < nt) ? d * scale_log2 : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int u = 1; u < kTile; ++u) mx = fmaxf(mx, sc[u]);
      // Running max.  While nothing is visible it stays -inf; the exponents
      // are then taken against 0 instead, so every weight (and alpha, with l
      // and acc still 0) is exp2(-inf) = 0 with no test per token.
      const float m_new = fmaxf(m[jq], mx);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[jq] - m_ref);
      m[jq] = m_new;
      l[jq] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[jq][e] *= alpha;
#pragma unroll
      for (int u = 0; u < kTile; ++u) {
        p[jq][u] = __builtin_amdgcn_exp2f(sc[u] - m_ref);
        l[jq] += p[jq][u];
      }
    }
    // one widening of each V vector serves every query head of the group
#pragma unroll
    for (int u = 0; u < kTile; ++u) {
      float vf[8];
      widen8<BF16>(t.v[u], vf);
#pragma unroll
      for (int jq = 0; jq < G; ++jq) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[jq][e] = fmaf(p[jq][u], vf[e], acc[jq][e]);
      }
    }
  };

  // NB tiles in flight: tile i + NB - 1 is requested before tile i is
  // consumed (the buffer index is static after unrolling by NB); eight
  // query heads per kv head keep at most two, their state leaves no room
  // for three.
  //
  // No load sits behind a branch.  The compiler places its wait for a
  // loaded register from the loads it knows were issued after it, taking the
  // fewest over every path into the wait; a branch around the loads of the
  // last tiles would make every wait assume the later tiles were never
  // requested and drain the loads in flight down to one tile.  So the
  // prologue and every pass request a tile (the ones past the end read the
  // dummy word above) and only the arithmetic is conditional.
  constexpr int NB = G >= 8 && kBuf > 2 ? 2 : kBuf;
  Tile buf[NB];
#pragma unroll
  for (int r = 0; r < kBuf - 1; ++r) load_tile(buf[r], r);
  for (int i0 = 0; i0 < n_tiles; i0 += NB) {
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int i = i0 + r;
      load_tile(buf[(r + NB - 1) % NB], i + NB - 1);
      if (i < n_tiles) compute_tile(buf[r], i);
    }
  }

  // Stage each wave's state in LDS (lane c of group lg holds columns
  // c*8..c*8+7 of its kv head's query heads), then the waves of each head
  // group merge its slices together: slice sl's wave takes columns [sl W,
  // (sl + 1) W) of every query head of the group, W = D / SLICES, EPL
  // consecutive columns per lane, and merges the slices in slice order, so
  // the result does not depend on which wave finished last.
#pragma unroll
  for (int jq = 0; jq < G; ++jq) {
    const int hq = lg * G + jq;
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[wave][hq][c * 8 + e] = acc[jq][e];
    if (c == 0) {
      s_m[wave][hq] = m[jq];
      s_l[wave][hq] = l[jq];
    }
  }
  __syncthreads();

  constexpr int W = D / SLICES;        // columns per wave
  constexpr int EPL = 8 * G / SLICES;  // columns per lane
  constexpr int LR = W / EPL;          // lanes per query head
  static_assert(EPL >= 1 && W % EPL == 0 && LR * HPL * G == kWave, "merge layout");
  const int r = lane / LR;                        // query head inside the head group
  const int col = slice * W + (lane % LR) * EPL;  // first column of the lane
  float M = -INFINITY;
#pragma unroll
  for (int sl = 0; sl < SLICES; ++sl) M = fmaxf(M, s_m[sl * HGW + hgw][r]);
  float L = 0.f, A[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[e] = 0.f;
#pragma unroll
  for (int sl = 0; sl < SLICES; ++sl) {
    const int wv = sl * HGW + hgw;
    const float mw = s_m[wv][r];
    const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    L = fmaf(s_l[wv][r], f, L);
#pragma unroll
    for (int e = 0; e < EPL; ++e) A[e] = fmaf(s_acc[wv][r][col + e], f, A[e]);
  }
  const size_t hs = (static_cast<size_t>(b) * a.n_q + (hset * HG + hgw * HPL) * G + r) * n_split + s;
  float* dst = a.partials + hs * D + col;
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(A[e], A[e + 1], A[e + 2], A[e + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) dst[e] = A[e];
  }
  if (slice == 0 && lane % LR == 0) {
    float* part_ml = a.partials + a.ml_offset;
    part_ml[hs * 2] = M;
    part_ml[hs * 2 + 1] = L;
  }
}

template <int D, int G, bool BF16, int HGW>
hipError_t launch_row(const DecodeArgs& a, hipStream_t s) {
  constexpr int HG = (kWave / (D / 8)) * HGW;
  // the slices of a head group must tile a block exactly
  constexpr bool kFits = kRowWaves % HGW == 0 && kBS % ((kRowWaves / HGW) * kTile) == 0;
  if constexpr (!kFits) {
    return hipErrorInvalidValue;
  } else {
    const int total = a.B * (a.lv.n_kv / HG) * a.n_split;
    const int grid = round_up(total, kXcds);
    hipLaunchKernelGGL((paged_decode_row_kernel<D, G, BF16, HGW>), dim3(grid), dim3(kRowThreads), 0,
                       s, a);
    return hipGetLastError();
  }
}

template <int D, bool BF16, int HGW>
hipError_t row_by_group(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_row<D, 1, BF16, HGW>(a, s);
    case 2: return launch_row<D, 2, BF16, HGW>(a, s);
    case 4: return launch_row<D, 4, BF16, HGW>(a, s);
    case 8: return launch_row<D, 8, BF16, HGW>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, bool BF16>
hipError_t row_by_hgw(const DecodeArgs& a, int group, int hgw, hipStream_t s) {
  switch (hgw) {
    case 1: return row_by_group<D, BF16, 1>(a, group, s);
    case 2:
      if constexpr (kRowWaves % 2 == 0) return row_by_group<D, BF16, 2>(a, group, s);
      return hipErrorInvalidValue;
    case 4:
      if constexpr (kRowWaves % 4 == 0) return row_by_group<D, BF16, 4>(a, group, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Head groups (of 64/(head_dim/8) kv heads: one 1 KiB wave load per token)
// per row-kernel workgroup, or 0 when the shape does not fit the row kernel.
int row_kernel_kpl(int32_t n_kv, int32_t head_dim, int32_t group, int32_t block_size) {
  if (block_size != 32 || (head_dim != 64 && head_dim != 128 && head_dim != 256)) return 0;
  if (group != 1 && group != 2 && group != 4 && group != 8) return 0;
  const int hpl = kWave / (head_dim / 8);
  if (n_kv % hpl) return 0;
  const int n_groups = n_kv / hpl;
  for (int hgw : {4, 2, 1})  // as many head groups per workgroup as allowed
    if (hgw <= PAGEDKV_ROW_MAX_HEAD_GROUPS && hgw <= kRowWaves && kRowWaves % hgw == 0 &&
        n_groups % hgw == 0 && kBS % ((kRowWaves / hgw) * kTile) == 0)
      return hgw;
  return 0;
}

int row_kernel_heads_per_workgroup(int32_t head_dim, int hgw) {
  return (kWave / (head_dim / 8)) * hgw;
}

hipError_t launch_paged_decode_row(const DecodeArgs& a, bool bf16, int32_t head_dim, int32_t group,
                                   int hgw, hipStream_t s) {
  if (bf16) {
    switch (head_dim) {
      case 64: return row_by_hgw<64, true>(a, group, hgw, s);
      case 128: return row_by_hgw<128, true>(a, group, hgw, s);
      case 256: return row_by_hgw<256, true>(a, group, hgw, s);
    }
  } else {
    switch (head_dim) {
      case 64: return row_by_hgw<64, false>(a, group, hgw, s);
      case 128: return row_by_hgw<128, false>(a, group, hgw, s);
      case 256: return row_by_hgw<256, false>(a, group, hgw, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
