// write_block: token-granular scatter of new K/V into the slab of their row;
// whole-row moves (copy_on_write_block, block export and import); the zero
// fill that backs append_slab; and the duplicate-write check of the debug
// mode.
//
// mlxcel issue #235 ("perf(core): chunked slab storage for the paged pool to
// eliminate growth reallocation entirely"), section "Proposed solution:
// chunked slabs": growth appends a fresh zeros slab (touch point: no copy),
// and write_block's update targets the row's slab instead of one pool tensor
// (touch point 1).  Packed pools quantise here, once per fresh token
// (mlx-swift-lm PR #142, "Add packed paged KV formats with bounded workspace
// admission", section "Summary" and the "After" flowchart: "quantize fresh
// K/V once"): K is rotated by H diag(sigma) / sqrt(D) with a fast
// Walsh-Hadamard butterfly network, then each group of 32 or 64 values is
// mapped to unsigned codes with an fp32 (scale, offset) pair.
#include "device_common.h"
#include "index_math.h"
#include "internal.h"
#include "pack_vector.h"

namespace pagedkv {

namespace {

constexpr int kThreads = 256;
constexpr int kPackedKv = 8;  // kv heads of a packed pool (pd_pool_create refuses others)

// Growth (one launch per append): workgroup row y takes slab y of the launch
// -- pair y / 2, K when y is even, V when odd -- records its base pointer in
// the device table (workgroup column 0) and zero-fills it with the other
// columns' help, 16 bytes per store.
__global__ __launch_bounds__(kThreads) void append_slabs_kernel(AppendArgs a) {
  const int y = blockIdx.y;
  const int pair = y >> 1, kv = y & 1;
  void* mem = kv ? a.v_mem[pair] : a.k_mem[pair];
  if (blockIdx.x == 0 && threadIdx.x == 0) a.tables[a.entry[pair] + kv * a.max_slabs] = mem;
  const size_t n16 = static_cast<size_t>(kv ? a.v_bytes : a.k_bytes) / 16;
  uint4* p = static_cast<uint4*>(mem);
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
}

// True when (row, slot) lies inside the pool; otherwise flags the error word
// (from the calling lane only) so the token can be skipped.
__device__ __forceinline__ bool valid_target(const LayerView& lv, int32_t row, int32_t slot,
                                             bool report) {
  if (row < 0 || row >= lv.capacity_rows) {
    if (report) set_error(lv.err, PD_DEVERR_WRITE_ROW);
    return false;
  }
  if (slot < 0 || slot >= lv.block_size) {
    if (report) set_error(lv.err, PD_DEVERR_WRITE_SLOT);
    return false;
  }
  return true;
}

// Token index inside its slab (row_in_slab * block_size + slot) and the slab.
__device__ __forceinline__ size_t token_in_slab(const LayerView& lv, int32_t row, int32_t slot,
                                                int* slab) {
  *slab = row / lv.slab_blocks;
  return static_cast<size_t>(row - *slab * lv.slab_blocks) * lv.block_size + slot;
}

// 16-bit pools: one workgroup per token copies its n_kv records of K and V
// (contiguous in the source and in the slab) as 16-byte vectors.  Every lane
// resolves the target itself, so no barrier stands between the row lookup
// and the stores; measured fastest when a token fills the workgroup's lanes
// (2 KiB or more of K).
__global__ __launch_bounds__(kThreads) void write_block_native_kernel(WriteArgs a) {
  const size_t tok_bytes = static_cast<size_t>(a.lv.n_kv) * a.lv.k_rec;  // == V bytes
  const int n16 = static_cast<int>(tok_bytes / 16);
  for (int i = blockIdx.x; i < a.n; i += gridDim.x) {
    const int32_t row = a.rows[i], slot = a.slots[i];
    if (!valid_target(a.lv, row, slot, threadIdx.x == 0)) continue;
    int slab;
    const size_t tok = token_in_slab(a.lv, row, slot, &slab);
    const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_src) + i * tok_bytes);
    const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_src) + i * tok_bytes);
    uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.lv.k_tab[slab])) +
                                         tok * tok_bytes);
    uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(const_cast<void*>(a.lv.v_tab[slab])) +
                                         tok * tok_bytes);
    for (int j = threadIdx.x; j < n16; j += kThreads) {
      store_global(kd + j, ks[j]);
      store_global(vd + j, vs[j]);
    }
  }
}

// The same copy when a token is exactly UPL units per lane (unit f < n16 a
// piece of K, the rest of V; 8 kv heads at head_dim 128 are one unit per
// lane): every lane's source loads go out first -- they do not depend on the
// target -- and the token's row, slot and slab base are read behind them, so
// the lookup chain overlaps the loads instead of preceding them.
template <int UPL>
__global__ __launch_bounds__(kThreads) void write_block_native_exact_kernel(WriteArgs a) {
  const size_t tok_bytes = static_cast<size_t>(a.lv.n_kv) * a.lv.k_rec;  // == V bytes
  const int n16 = static_cast<int>(tok_bytes / 16);                      // 2 n16 == UPL * kThreads
  for (int i = blockIdx.x; i < a.n; i += gridDim.x) {
    const char* ks = static_cast<const char*>(a.k_src) + i * tok_bytes;
    const char* vs = static_cast<const char*>(a.v_src) + i * tok_bytes;
    uint4 v[UPL];
#pragma unroll
    for (int r = 0; r < UPL; ++r) {
      const int f = threadIdx.x + r * kThreads;
      v[r] = *reinterpret_cast<const uint4*>(f < n16 ? ks + static_cast<size_t>(f) * 16
                                                     : vs + static_cast<size_t>(f - n16) * 16);
    }
    const int32_t row = a.rows[i], slot = a.slots[i];
    // an empty asm with a memory clobber (no instruction) keeps the loads
    // above from being moved under the target check below
    asm volatile("" ::: "memory");
    if (!valid_target(a.lv, row, slot, threadIdx.x == 0)) continue;
    int slab;
    const size_t tok = token_in_slab(a.lv, row, slot, &slab);
    char* kd = static_cast<char*>(const_cast<void*>(a.lv.k_tab[slab])) + tok * tok_bytes;
    char* vd = static_cast<char*>(const_cast<void*>(a.lv.v_tab[slab])) + tok * tok_bytes;
#pragma unroll
    for (int r = 0; r < UPL; ++r) {
      const int f = threadIdx.x + r * kThreads;
      store_global(f < n16 ? kd + static_cast<size_t>(f) * 16 : vd + static_cast<size_t>(f - n16) * 16, v[r]);
    }
  }
}

// 16-bit pools whose tokens are small (fewer than kWbMultiBelow 16-byte units
// of K per token): a workgroup copies a chunk of consecutive tokens, each
// token's n_kv records of K and of V (contiguous in the source and in the
// slab) as 16-byte vectors.  Unit f of the chunk is 16-byte piece f % (2 n16)
// of token f / (2 n16) (K pieces, then V pieces); every thread issues
// kWbLoads source loads first, and the first lanes resolve the chunk's (row,
// slot) targets into LDS while those loads are in flight.  Several tokens per
// workgroup keep every lane busy when a token's records are small (1 KiB of K
// at head_dim 64 with 8 kv heads).
#ifndef PAGEDKV_WB_LOADS
#define PAGEDKV_WB_LOADS 4
#endif
// Tokens with at least this many 16-byte units of K (2 KiB) take one
// workgroup each; smaller ones are packed several to a workgroup.
constexpr int kWbMultiBelow = 128;
constexpr int kWbLoads = PAGEDKV_WB_LOADS;
static_assert(2 * kWbMultiBelow <= kThreads * kWbLoads, "a token of the multi-token kernel fits one batch");
constexpr int kWbMaxTokens = kThreads * kWbLoads / 16 > 0 ? kThreads * kWbLoads / 16 : 1;

__global__ __launch_bounds__(kThreads) void write_block_native_multi_kernel(WriteArgs a, int tpw, uint32_t m_upt) {
  __shared__ char* s_kd[kWbMaxTokens];  // slab address of each token of the chunk, null = skip
  __shared__ char* s_vd[kWbMaxTokens];
  const size_t tok_bytes = static_cast<size_t>(a.lv.n_kv) * a.lv.k_rec;  // == V bytes
  const int n16 = static_cast<int>(tok_bytes / 16);
  const int upt = 2 * n16;  // units per token
  const char* ksrc = static_cast<const char*>(a.k_src);
  const char* vsrc = static_cast<const char*>(a.v_src);
  uint4 v[kWbLoads];
  // unit f of the chunk starting at token i0: source loads (they do not
  // depend on the targets) and stores to the resolved targets
  auto load = [&](int i0, int f0, int total) {
#pragma unroll
    for (int j = 0; j < kWbLoads; ++j) {
      const int f = f0 + j * kThreads;
      if (f < total) {
        const int t = static_cast<int>(div_by(f, m_upt));
        const int r = f - t * upt;
        const bool is_v = r >= n16;
        const size_t off = static_cast<size_t>(i0 + t) * tok_bytes + static_cast<size_t>(is_v ? r - n16 : r) * 16;
        v[j] = *reinterpret_cast<const uint4*>((is_v ? vsrc : ksrc) + off);
      }
    }
  };
  auto store = [&](int f0, int total) {
#pragma unroll
    for (int j = 0; j < kWbLoads; ++j) {
      const int f = f0 + j * kThreads;
      if (f < total) {
        const int t = static_cast<int>(div_by(f, m_upt));
        const int r = f - t * upt;
        const bool is_v = r >= n16;
        char* d = is_v ? s_vd[t] : s_kd[t];
        if (d) store_global(d + static_cast<size_t>(is_v ? r - n16 : r) * 16, v[j]);
      }
    }
  };
  for (int i0 = blockIdx.x * tpw; i0 < a.n; i0 += gridDim.x * tpw) {
    const int nt = min(tpw, a.n - i0);
    const int total = nt * upt;
    __syncthreads();  // the previous chunk's targets are no longer read
    load(i0, threadIdx.x, total);
    if (threadIdx.x < nt) {
      const int i = i0 + threadIdx.x;
      const int32_t row = a.rows[i], slot = a.slots[i];
      char* kd = nullptr;
      char* vd = nullptr;
      if (valid_target(a.lv, row, slot, true)) {
        int slab;
        const size_t tok = token_in_slab(a.lv, row, slot, &slab);
        kd = static_cast<char*>(const_cast<void*>(a.lv.k_tab[slab])) + tok * tok_bytes;
        vd = static_cast<char*>(const_cast<void*>(a.lv.v_tab[slab])) + tok * tok_bytes;
      }
      s_kd[threadIdx.x] = kd;
      s_vd[threadIdx.x] = vd;
    }
    __syncthreads();
    store(threadIdx.x, total);  // one batch covers the chunk: tpw * upt <= kThreads * kWbLoads
  }
}

// Whole block rows, every layer, K and V: copy_on_write_block (mlxcel #235,
// "Proposed solution", touch point 2: the source slice comes from the source
// row's slab), and the serde block-content extraction and restore path
// (touch point 6: per-block reads and writes localise to the row's slab
// through the same mapping).  A work unit is 4 KiB of one block row of one
// layer's K or V for one block; a workgroup moves it as one 16-byte vector
// per lane.  The rows of a block are contiguous in their slab, so both sides
// are plain streams.
constexpr int kMoveChunk = kThreads * 16;

__device__ __forceinline__ char* pool_row(const RowMoveArgs& a, int layer, int kv, int32_t row) {
  const void* const* tab = a.tables + (static_cast<size_t>(layer) * 2 + kv) * a.max_slabs;
  const int slab = row / a.slab_blocks;
  return static_cast<char*>(const_cast<void*>(tab[slab])) + (row - slab * a.slab_blocks) * a.row_bytes[kv];
}

__device__ __forceinline__ size_t buf_offset(const RowMoveArgs& a, int i, int layer, int kv) {
  return (static_cast<size_t>(i) * a.n_layers + layer) * (a.row_bytes[0] + a.row_bytes[1]) +
         (kv ? a.row_bytes[0] : 0);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void row_move_kernel(RowMoveArgs a) {
  const int64_t max_row = a.row_bytes[0] > a.row_bytes[1] ? a.row_bytes[0] : a.row_bytes[1];
  const int chunks = static_cast<int>((max_row + kMoveChunk - 1) / kMoveChunk);
  const long long units = static_cast<long long>(a.n) * a.n_layers * 2 * chunks;
  for (long long u = blockIdx.x; u < units; u += gridDim.x) {
    const int c = static_cast<int>(u % chunks);
    long long r = u / chunks;
    const int kv = static_cast<int>(r % 2);
    r /= 2;
    const int layer = static_cast<int>(r % a.n_layers);
    const int i = static_cast<int>(r / a.n_layers);
    const bool report = threadIdx.x == 0 && c == 0 && kv == 0 && layer == 0;  // once per block
    const int64_t bytes = a.row_bytes[kv];
    const int64_t off = static_cast<int64_t>(c) * kMoveChunk + threadIdx.x * 16;
    const bool lane_in = off < bytes;
    if constexpr (MODE == kMoveCopy) {
      const int32_t src = a.src_rows[i], dst = a.dst_rows[i];
      const bool src_ok = src >= 0 && src < a.capacity_rows;
      const bool dst_ok = dst >= 0 && dst < a.capacity_rows;
      if (!src_ok || !dst_ok) {
        if (report) set_error(a.err, src_ok ? PD_DEVERR_WRITE_ROW : PD_DEVERR_TABLE_ROW);
        continue;
      }
      if (lane_in)
        store_global(pool_row(a, layer, kv, dst) + off, load_global<uint4>(pool_row(a, layer, kv, src) + off));
    } else if constexpr (MODE == kMoveExport) {
      const int32_t src = a.src_rows[i];
      const bool ok = src >= 0 && src < a.capacity_rows;
      if (!ok && report) set_error(a.err, PD_DEVERR_TABLE_ROW);
      if (lane_in)
        *reinterpret_cast<uint4*>(a.dst_buf + buf_offset(a, i, layer, kv) + off) =
            ok ? load_global<uint4>(pool_row(a, layer, kv, src) + off) : make_uint4(0, 0, 0, 0);
    } else {
      const int32_t dst = a.dst_rows[i];
      if (dst < 0 || dst >= a.capacity_rows) {
        if (report) set_error(a.err, PD_DEVERR_WRITE_ROW);
        continue;
      }
      if (lane_in)
        store_global(pool_row(a, layer, kv, dst) + off,
                     *reinterpret_cast<const uint4*>(a.src_buf + buf_offset(a, i, layer, kv) + off));
    }
  }
}

// ---- packed pools -------------------------------------------------------------
// A lane holds 8 consecutive values of a vector (one token-head of K or V),
// D/8 lanes hold the vector, and a wave works on 64/(D/8) vectors at once, all
// K or all V: the wave tasks are the K vectors in wave-sized runs, then the V
// vectors likewise.

// One wave task: the VPW = 64/(D/8) vectors v0 .. v0 + VPW - 1 of K (task t <
// tasks, rotated) or of V (t - tasks).  VPW divides the 8 kv heads and v0 is
// a multiple of VPW, so the task's vectors are heads of one token: its row,
// slot and slab are the same in every lane and are resolved once per wave.
struct PackIn {
  uint4 u;       // the lane's 16 bytes of the source vector (values 8c .. 8c+7)
  int32_t row, slot;
  int v0;        // first vector of the task (K or V numbering)
  bool is_v;
};

template <int D>
__device__ __forceinline__ PackIn pack_load(const WriteArgs& a, int t, int tasks, int lane) {
  constexpr int VPW = kWave / (D / 8);
  PackIn in;
  in.is_v = t >= tasks;
  in.v0 = (in.is_v ? t - tasks : t) * VPW;
  const uint16_t* src = static_cast<const uint16_t*>(in.is_v ? a.v_src : a.k_src);
  in.u = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(in.v0) * D + 8 * lane);
  const int i = in.v0 / kPackedKv;  // the token
  in.row = __builtin_amdgcn_readfirstlane(a.rows[i]);
  in.slot = __builtin_amdgcn_readfirstlane(a.slots[i]);
  return in;
}

// The record of the lane's vector.  A token whose (row, slot) is outside the
// pool gets ok = false and the record address of row 0, slot 0 (its slab
// base is still read, so no load depends on the check).
template <int D>
__device__ __forceinline__ char* pack_record(const WriteArgs& a, const PackIn& in, int lane, bool& ok) {
  constexpr int LPT = D / 8;
  ok = in.row >= 0 && in.row < a.lv.capacity_rows && in.slot >= 0 && in.slot < a.lv.block_size;
  const int32_t row = ok ? in.row : 0, slot = ok ? in.slot : 0;
  // row / slab_blocks as one high multiply when the host found it exact
  const int slab =
      a.m_slab ? static_cast<int>(div_by(static_cast<uint32_t>(row), a.m_slab)) : row / a.lv.slab_blocks;
  const size_t tok = static_cast<size_t>(row - slab * a.lv.slab_blocks) * a.lv.block_size + slot;
  const int rec_bytes = in.is_v ? a.lv.v_rec : a.lv.k_rec;
  const int head = in.v0 % kPackedKv + lane / LPT;
  const void* const* tab = in.is_v ? a.lv.v_tab : a.lv.k_tab;
  return static_cast<char*>(const_cast<void*>(tab[slab])) + tok * kPackedKv * rec_bytes + head * rec_bytes;
}

template <int D, int GS>
__device__ __forceinline__ Codes8 pack_codes(const WriteArgs& a, const PackIn& in, int c, const float (&sg)[8],
                                             const uint32_t (&odd_sign)[4]) {
  float x[8];  // a token that is not written is still quantised, and not stored
  if (in.is_v) {
    widen8<true>(in.u, x);
    return quantise8<D, GS>(x, c, a.v_bits);
  }
  widen_rotate8<D>(in.u, odd_sign, sg, c, a.inv_sqrt_d, x);  // every lane takes part
  return quantise8<D, GS>(x, c, a.k_bits);
}

// A wave takes two consecutive tasks per pass (the task count, K tasks then
// as many V tasks, is even), and every load of both (the sources, rows and
// slots, then the slab bases) goes out before the first task's arithmetic:
// one task's loads alone leave too few bytes in flight per CU to cover the
// memory latency.  The stores of both come last.  No load sits behind a
// branch, so the compiler's waits for the loaded registers count the loads
// issued after them exactly.
template <int D, int GS>
__global__ __launch_bounds__(kThreads) void write_block_packed_kernel(WriteArgs a) {
  constexpr int LPT = D / 8;        // lanes per vector
  constexpr int VPW = kWave / LPT;  // vectors per wave
  const int lane = threadIdx.x % kWave;
  const int c = lane % LPT;         // values 8c .. 8c+7 of the vector
  const int n_vec = a.n * kPackedKv;  // K vectors; as many V vectors
  const int tasks = (n_vec + VPW - 1) / VPW;
  const int total = 2 * tasks;  // even: every pass below holds tasks t and t + 1
  const int waves = gridDim.x * (kThreads / kWave);
  float sg[8];  // the signs of values 8c .. 8c+7 (the same for every vector)
  {
    const float4* sp4 = reinterpret_cast<const float4*>(a.signs + 8 * c);
    const float4 s0 = sp4[0], s1 = sp4[1];
    sg[0] = s0.x, sg[1] = s0.y, sg[2] = s0.z, sg[3] = s0.w;
    sg[4] = s1.x, sg[5] = s1.y, sg[6] = s1.z, sg[7] = s1.w;
  }
  uint32_t odd_sign[4];  // sign bits of the odd values' signs
#pragma unroll
  for (int i = 0; i < 4; ++i) odd_sign[i] = __float_as_uint(sg[2 * i + 1]) & 0x80000000u;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave);
  static_assert(kPackedKv % VPW == 0, "a wave task covers heads of one token");
  for (int t = 2 * wave; t < total; t += 2 * waves) {
    const PackIn ia = pack_load<D>(a, t, tasks, lane);
    const PackIn ib = pack_load<D>(a, t + 1, tasks, lane);
    bool oka, okb;
    char* const ra = pack_record<D>(a, ia, lane, oka);
    char* const rb = pack_record<D>(a, ib, lane, okb);
    const Codes8 qa = pack_codes<D, GS>(a, ia, c, sg, odd_sign);
    const Codes8 qb = pack_codes<D, GS>(a, ib, c, sg, odd_sign);
    if (oka) store_codes8<D, GS>(qa, c, ia.is_v ? a.v_bits : a.k_bits, ra);
    if (okb) store_codes8<D, GS>(qb, c, ib.is_v ? a.v_bits : a.k_bits, rb);
    // a token outside the pool is reported once, by the wave holding its first K vectors
    if (!oka && lane == 0 && !ia.is_v && ia.v0 % kPackedKv == 0) valid_target(a.lv, ia.row, ia.slot, true);
    if (!okb && lane == 0 && !ib.is_v && ib.v0 % kPackedKv == 0) valid_target(a.lv, ib.row, ib.slot, true);
  }
}

// ---- duplicate-write check (debug) ----------------------------------------------
// A token whose (row, slot) is outside the pool is left to the write, which
// reports it.  Marking uses a vector atomic OR per token; the clear stores
// zero to each touched word (every bit set in it belongs to this call, since
// the bitmap is all zero between calls).

template <bool MARK>
__global__ __launch_bounds__(kThreads) void dup_check_kernel(DupArgs a) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < a.n; i += gridDim.x * kThreads) {
    const int32_t row = a.rows[i], slot = a.slots[i];
    if (row < 0 || row >= a.capacity_rows || slot < 0 || slot >= a.block_size) continue;
    const uint64_t bit = static_cast<uint64_t>(row) * a.block_size + slot;
    uint32_t* word = a.bits + (bit >> 5);
    if constexpr (MARK) {
      const uint32_t m = 1u << (bit & 31);
      if (atomicOr(word, m) & m) set_error(a.err, PD_DEVERR_DUPLICATE);
    } else {
      *word = 0u;
    }
  }
}

}  // namespace

hipError_t launch_append_slabs(const AppendArgs& a, hipStream_t s) {
  if (a.n_pairs <= 0) return hipSuccess;
  if (a.n_pairs > kAppendMaxPairs) return hipErrorInvalidValue;
  // columns per slab: about 4 stores per thread per column, at most 64
  const size_t n16 = static_cast<size_t>(a.k_bytes > a.v_bytes ? a.k_bytes : a.v_bytes) / 16;
  size_t cols = (n16 + 4 * kThreads - 1) / (4 * kThreads);
  if (cols < 1) cols = 1;
  if (cols > 64) cols = 64;
  hipLaunchKernelGGL(append_slabs_kernel, dim3(static_cast<unsigned>(cols), 2 * a.n_pairs), dim3(kThreads), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_dup_check(const DupArgs& a, bool mark, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  long long grid = (a.n + kThreads - 1) / kThreads;
  if (grid > 4096) grid = 4096;
  if (mark)
    hipLaunchKernelGGL(dup_check_kernel<true>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(dup_check_kernel<false>, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row_move(const RowMoveArgs& a, int mode, hipStream_t s) {
  const int64_t max_row = a.row_bytes[0] > a.row_bytes[1] ? a.row_bytes[0] : a.row_bytes[1];
  const long long units = static_cast<long long>(a.n) * a.n_layers * 2 *
                          ((max_row + kMoveChunk - 1) / kMoveChunk);
  const int grid = static_cast<int>(units < 4096 ? units : 4096);
  if (grid == 0) return hipSuccess;
  switch (mode) {
    case kMoveCopy: hipLaunchKernelGGL(row_move_kernel<kMoveCopy>, dim3(grid), dim3(kThreads), 0, s, a); break;
    case kMoveExport: hipLaunchKernelGGL(row_move_kernel<kMoveExport>, dim3(grid), dim3(kThreads), 0, s, a); break;
    case kMoveImport: hipLaunchKernelGGL(row_move_kernel<kMoveImport>, dim3(grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_write_block(const WriteArgs& a, int32_t format, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (format == PD_FMT_FP16 || format == PD_FMT_BF16) {
    const long long upt = 2LL * a.lv.n_kv * a.lv.k_rec / 16;  // 16-byte units per token
    if (upt / 2 >= kWbMultiBelow) {
      // the exact kernel takes one token per workgroup (a workgroup that loops
      // would wait for its previous token's stores before reusing registers)
      const int grid_exact = a.n < (1 << 22) ? a.n : (1 << 22);
      const int grid = a.n < 65536 ? a.n : 65536;
      if (upt == kThreads)
        hipLaunchKernelGGL(write_block_native_exact_kernel<1>, dim3(grid_exact), dim3(kThreads), 0, s, a);
      else if (upt == 2 * kThreads)
        hipLaunchKernelGGL(write_block_native_exact_kernel<2>, dim3(grid_exact), dim3(kThreads), 0, s, a);
      else
        hipLaunchKernelGGL(write_block_native_kernel, dim3(grid), dim3(kThreads), 0, s, a);
      return hipGetLastError();
    }
    int tpw = static_cast<int>(kThreads * kWbLoads / upt);
    tpw = tpw < 1 ? 1 : (tpw > kWbMaxTokens ? kWbMaxTokens : tpw);
    // the reciprocal division is exact while every unit index f < tpw * upt
    // stays below 2^32 / upt
    if (upt < 2 || static_cast<uint64_t>(tpw) * upt * upt >= (uint64_t{1} << 32)) return hipErrorInvalidValue;
    const long long chunks = (a.n + tpw - 1) / tpw;
    const int grid = static_cast<int>(chunks < 65536 ? chunks : 65536);
    hipLaunchKernelGGL(write_block_native_multi_kernel, dim3(grid), dim3(kThreads), 0, s, a, tpw,
                       reciprocal_u32(static_cast<uint32_t>(upt)));
    return hipGetLastError();
  }
  if (a.lv.n_kv != kPackedKv) return hipErrorInvalidValue;  // packed pools hold 8 kv heads
  // one wave per two tasks (a task is one wave-wide pass over 64 lanes' values)
  const long long waves = ((2LL * a.n * a.lv.n_kv * (a.head_dim / 8) + kWave - 1) / kWave + 1) / 2;
  long long grid = (waves + kThreads / kWave - 1) / (kThreads / kWave);
  if (grid > 16384) grid = 16384;  // a few wave tasks per wave: its set-up is shared
  const int key = a.head_dim * 100 + a.qgroup;
  switch (key) {
    case 6432:
      hipLaunchKernelGGL((write_block_packed_kernel<64, 32>), dim3(grid), dim3(kThreads), 0, s, a);
      break;
    case 12832:
      hipLaunchKernelGGL((write_block_packed_kernel<128, 32>), dim3(grid), dim3(kThreads), 0, s, a);
      break;
    case 25632:
      hipLaunchKernelGGL((write_block_packed_kernel<256, 32>), dim3(grid), dim3(kThreads), 0, s, a);
      break;
    case 12864:
      hipLaunchKernelGGL((write_block_packed_kernel<128, 64>), dim3(grid), dim3(kThreads), 0, s, a);
      break;
    case 25664:
      hipLaunchKernelGGL((write_block_packed_kernel<256, 64>), dim3(grid), dim3(kThreads), 0, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pagedkv
