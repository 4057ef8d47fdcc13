// gather_visible: copy each sequence's visible K/V out of the slabs into
// contiguous, transposed tensors [B, n_kv, t_out, record].
//
// mlxcel issue #235 ("perf(core): chunked slab storage for the paged pool to
// eliminate growth reallocation entirely"), section "Proposed solution:
// chunked slabs", touch point 3: one read cannot span slabs, so the block
// table's row list is split into maximal same-slab runs in logical order and
// each run is read from its own slab; the runs' results are laid out in order
// and then reshaped to tokens, sliced to the visible length and transposed to
// head-major.  Here the reshape, slice and transpose are folded into the
// store addresses, so every byte is read once and written once.
//
// Decomposition: one workgroup per (sequence, chunk of kChunk logical
// blocks; one block measured fastest: more, shorter workgroups keep the
// memory system busier than fewer, longer ones).  The copy does not walk the
// runs: lane i of the first wave resolves block i of the chunk itself -- its
// row, the row's slab and that slab's base pointer (the blocks of one
// same-slab run resolve to the same base, a table entry that stays in L2) --
// so every block of every run is copied at once.  The run list is
// split_runs_kernel's output (pd_split_runs).  The workgroup then copies the chunk's blocks in
// logical order as 16-byte vectors: each block's source is one contiguous
// row [block_size, n_kv, record]; the destination is n_kv contiguous pieces
// of block_size records.  A block's K row and V row form one range of
// 16-byte units; every thread issues kUnroll loads of it before it stores, so
// a CU keeps enough reads in flight to stream at the HBM rate, and both sides
// are non-temporal, since each byte is touched once.  A unit's (slot, head,
// piece) comes from reciprocal multiplies rather than divisions.  The first
// chunk's workgroup also counts the sequence's runs over the whole row list
// for n_runs_out.
#include "device_common.h"
#include "index_math.h"
#include "internal.h"

namespace pagedkv {

namespace {

#ifndef PAGEDKV_GATHER_CHUNK
#define PAGEDKV_GATHER_CHUNK 1
#endif
#ifndef PAGEDKV_GATHER_UNROLL
#define PAGEDKV_GATHER_UNROLL 32
#endif

#ifndef PAGEDKV_GATHER_THREADS
#define PAGEDKV_GATHER_THREADS 256
#endif
// Small gathers (under kGatherSmallWgs workgroups, a few per CU) run 512
// threads with 16 loads each: more resident waves with the same 128 KiB in
// flight per workgroup.  Measured on the 8 x 4096-token layer (1024
// workgroups): 47.6 us against 50.8-51.9 us with 256 x 32; on the 32 x
// 16384-token layer (16384 workgroups) 256 x 32 is the faster (746 us against
// 779 us).
constexpr int kGatherSmallWgs = 4096;

constexpr int kThreads = PAGEDKV_GATHER_THREADS;
constexpr int kChunk = PAGEDKV_GATHER_CHUNK;    // logical blocks per workgroup
constexpr int kUnroll = PAGEDKV_GATHER_UNROLL;  // 16-byte loads in flight per thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ int slab_of(int32_t row, const LayerView& lv) {
  return (row < 0 || row >= lv.capacity_rows) ? -1 : row / lv.slab_blocks;
}

struct GatherDiv {
  uint32_t m_kunits, m_vunits, m_nkv;  // reciprocals of the units per K / V record and of n_kv
};

template <int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void gather_kernel(GatherArgs a, GatherDiv dv) {
  __shared__ const char* s_ksrc[kChunk];  // source row of each block, null = zeros
  __shared__ const char* s_vsrc[kChunk];
  __shared__ int s_runs[THREADS / kWave];

  const LayerView& lv = a.lv;
  const int bs = lv.block_size;
  const int chunks = (((a.t_out + bs - 1) / bs) + kChunk - 1) / kChunk;
  const int w = xcd_work_id(blockIdx.x, gridDim.x);
  if (w >= a.B * chunks) return;
  const int b = w / chunks;
  const int ch = w % chunks;

  int len = a.lens[b];
  const int cap_len = min(a.t_out, a.max_blocks * bs);
  if (len < 0 || len > cap_len) {
    if (threadIdx.x == 0 && ch == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + bs - 1) / bs;
  const int32_t* trow = a.table + static_cast<size_t>(b) * a.max_blocks;
  const int n_kv = lv.n_kv;
  const size_t k_row_bytes = static_cast<size_t>(bs) * n_kv * lv.k_rec;
  const size_t v_row_bytes = static_cast<size_t>(bs) * n_kv * lv.v_rec;

  const int blk0 = ch * kChunk;
  if (threadIdx.x < kChunk) {
    const int blk = blk0 + threadIdx.x;
    const char* ks = nullptr;
    const char* vs = nullptr;
    if (blk < nb) {
      const int row = trow[blk];
      const int slab = slab_of(row, lv);
      if (slab < 0) {
        set_error(lv.err, PD_DEVERR_TABLE_ROW);
      } else {
        const size_t r = static_cast<size_t>(row - slab * lv.slab_blocks);
        ks = static_cast<const char*>(lv.k_tab[slab]) + r * k_row_bytes;
        vs = static_cast<const char*>(lv.v_tab[slab]) + r * v_row_bytes;
      }
    }
    s_ksrc[threadIdx.x] = ks;
    s_vsrc[threadIdx.x] = vs;
  }

  // Whole-sequence run count (first chunk only).
  if (ch == 0 && a.n_runs_out) {
    int cnt = 0;
    for (int i = threadIdx.x; i < nb; i += THREADS) {
      const int sl = slab_of(trow[i], lv);
      cnt += (i == 0) || (sl != slab_of(trow[i - 1], lv));
    }
    for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, kWave);
    if (threadIdx.x % kWave == 0) s_runs[threadIdx.x / kWave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      int total = 0;
      for (int i = 0; i < THREADS / kWave; ++i) total += s_runs[i];
      a.n_runs_out[b] = total;
    }
  }
  __syncthreads();

  char* kout = static_cast<char*>(a.k_out);
  char* vout = static_cast<char*>(a.v_out);
  const int ku = lv.k_rec / 16, vu = lv.v_rec / 16;  // 16-byte units per record
  const int KU = bs * n_kv * ku;                       // units of a K block row
  const int TU = KU + bs * n_kv * vu;                  // then those of the V row
  for (int i = 0; i < kChunk; ++i) {
    const int blk = blk0 + i;
    if (blk * bs >= a.t_out) break;
    const char* ksrc = s_ksrc[i];
    const char* vsrc = s_vsrc[i];
    // tokens of this block that exist in the output / are visible
    const int t_end = min(bs, a.t_out - blk * bs);
    const int t_vis = ksrc ? max(0, min(bs, len - blk * bs)) : 0;
    // unit u < KU is (slot, head, 16-byte piece) of the K row, the rest of
    // the V row; K and V loads are in flight together
    for (int u0 = threadIdx.x; u0 < TU; u0 += THREADS * UNROLL) {
      u32x4 v[UNROLL];
      int slot_of[UNROLL];
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int u = u0 + j * THREADS;
        const bool is_v = u >= KU;
        const int uu = is_v ? u - KU : u;
        const uint32_t rr = div_by(uu, is_v ? dv.m_vunits : dv.m_kunits);  // record in the row
        const int slot = static_cast<int>(div_by(rr, dv.m_nkv));
        slot_of[j] = slot;
        v[j] = (u32x4){0u, 0u, 0u, 0u};
        if (u < TU && slot < t_vis)
          v[j] = __builtin_nontemporal_load((const gu32x4*)(is_v ? vsrc : ksrc) + uu);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; ++j) {
        const int u = u0 + j * THREADS;
        const bool is_v = u >= KU;
        const int uu = is_v ? u - KU : u;
        const int units = is_v ? vu : ku;
        const int rr = static_cast<int>(div_by(uu, is_v ? dv.m_vunits : dv.m_kunits));
        const int piece = uu - rr * units;
        const int slot = slot_of[j];
        const int head = rr - slot * n_kv;
        if (u < TU && slot < t_end) {
          const int rec = is_v ? lv.v_rec : lv.k_rec;
          const size_t o = ((static_cast<size_t>(b) * n_kv + head) * a.t_out + blk * bs + slot) * rec +
                           piece * 16;
          __builtin_nontemporal_store(v[j], (gu32x4*)((is_v ? vout : kout) + o));
        }
      }
    }
  }
}



// The run split itself (mlxcel #235, "Proposed solution", touch point 3):
// one wave per sequence walks its visible blocks 64 at a time.  Lane i takes
// block c0 + i and its slab (row / slab_blocks; -1 for a row outside the
// pool, which also sets the error word); a block starts a run when it is
// the first or its slab differs from the previous block's.  A start lane
// writes its run's (slab, first block) at the run's index (the starts before
// it, counted with a ballot) and closes the previous run's count; the chunk
// carries the run count, the last start and the last slab to the next.
constexpr int kRunWaves = 4;

__global__ __launch_bounds__(kRunWaves * kWave) void split_runs_kernel(RunArgs a) {
  const int lane = threadIdx.x % kWave;
  const int b = blockIdx.x * kRunWaves + threadIdx.x / kWave;
  if (b >= a.B) return;
  const LayerView& lv = a.lv;
  const int bs = lv.block_size;
  int len = a.lens[b];
  const int cap_len = a.max_blocks * bs;
  if (len < 0 || len > cap_len) {
    if (lane == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + bs - 1) / bs;
  const int32_t* trow = a.table + static_cast<size_t>(b) * a.max_blocks;
  int32_t* runs = a.runs + static_cast<size_t>(b) * a.max_blocks * 3;
  int n_runs = 0, last_first = -1, last_slab = 0;
  for (int c0 = 0; c0 < nb; c0 += kWave) {
    const int blk = c0 + lane;
    const bool valid = blk < nb;
    int slab = -2;
    if (valid) {
      slab = slab_of(trow[blk], lv);
      if (slab < 0) set_error(lv.err, PD_DEVERR_TABLE_ROW);
    }
    int prev = __shfl_up(slab, 1, kWave);
    if (lane == 0) prev = last_slab;
    const bool start = valid && (blk == 0 || slab != prev);
    const uint64_t mask = __ballot(start);
    const uint64_t below = mask & ((uint64_t{1} << lane) - 1);
    if (start) {
      const int k = n_runs + __popcll(below);
      runs[3 * k] = slab;
      runs[3 * k + 1] = blk;
      // the previous run ends here: its first block is the highest start below this lane
      const int prev_first = below ? c0 + 63 - __clzll(below) : last_first;
      if (k > 0) runs[3 * (k - 1) + 2] = blk - prev_first;
    }
    n_runs += __popcll(mask);
    if (mask) last_first = c0 + 63 - __clzll(mask);
    last_slab = __shfl(slab, kWave - 1, kWave);
  }
  if (lane == 0) {
    if (n_runs > 0) runs[3 * (n_runs - 1) + 2] = nb - last_first;
    if (a.n_runs) a.n_runs[b] = n_runs;
  }
}

}  // namespace

hipError_t launch_split_runs(const RunArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  const int grid = (a.B + kRunWaves - 1) / kRunWaves;
  hipLaunchKernelGGL(split_runs_kernel, dim3(grid), dim3(kRunWaves * kWave), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int bs = a.lv.block_size;
  const int chunks = (((a.t_out + bs - 1) / bs) + kChunk - 1) / kChunk;
  const long long total = static_cast<long long>(a.B) * chunks;
  if (total == 0) return hipSuccess;
  if (total > (1LL << 30)) return hipErrorInvalidValue;
  const int grid = round_up(static_cast<int>(total), kXcds);
  const uint32_t ku = a.lv.k_rec / 16, vu = a.lv.v_rec / 16, n_kv = a.lv.n_kv;
  // the reciprocal divisions are exact while n < 2^32 / d for every index n
  const uint64_t recs = static_cast<uint64_t>(bs) * n_kv;
  const uint64_t max_units = recs * (ku > vu ? ku : vu);
  const uint64_t max_div = ku > vu ? (ku > n_kv ? ku : n_kv) : (vu > n_kv ? vu : n_kv);
  if (ku == 0 || vu == 0 || max_units * max_div >= (uint64_t{1} << 32)) return hipErrorInvalidValue;
  const GatherDiv dv{reciprocal_u32(ku), reciprocal_u32(vu), reciprocal_u32(n_kv)};
  if (total < kGatherSmallWgs)
    hipLaunchKernelGGL((gather_kernel<512, 16>), dim3(grid), dim3(512), 0, s, a, dv);
  else
    hipLaunchKernelGGL((gather_kernel<kThreads, kUnroll>), dim3(grid), dim3(kThreads), 0, s, a, dv);
  return hipGetLastError();
}

}  // namespace pagedkv
