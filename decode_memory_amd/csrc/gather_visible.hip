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
// blocks).  Lane i of the first wave resolves block i of the chunk: its row,
// the row's slab and that slab's base pointer (blocks of one same-slab run
// resolve to the same base).  The workgroup then copies the chunk's blocks in
// logical order as 16-byte vectors: each block's source is one contiguous
// row [block_size, n_kv, record]; the destination is n_kv contiguous pieces
// of block_size records.  Every thread issues kUnroll loads before it
// stores, so a CU keeps enough reads in flight to stream at the HBM rate;
// both sides are non-temporal, since each byte is touched once.  The first
// chunk's workgroup also counts the sequence's runs over the whole row list
// for n_runs_out.
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 2;   // logical blocks per workgroup
constexpr int kUnroll = 16; // 16-byte loads in flight per thread

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

__device__ __forceinline__ int slab_of(int32_t row, const LayerView& lv) {
  return (row < 0 || row >= lv.capacity_rows) ? -1 : row / lv.slab_blocks;
}

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
  __shared__ const char* s_ksrc[kChunk];  // source row of each block, null = zeros
  __shared__ const char* s_vsrc[kChunk];
  __shared__ int s_runs[kThreads / kWave];

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
    for (int i = threadIdx.x; i < nb; i += kThreads) {
      const int sl = slab_of(trow[i], lv);
      cnt += (i == 0) || (sl != slab_of(trow[i - 1], lv));
    }
    for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, kWave);
    if (threadIdx.x % kWave == 0) s_runs[threadIdx.x / kWave] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      int total = 0;
      for (int i = 0; i < kThreads / kWave; ++i) total += s_runs[i];
      a.n_runs_out[b] = total;
    }
  }
  __syncthreads();

  char* kout = static_cast<char*>(a.k_out);
  char* vout = static_cast<char*>(a.v_out);
  for (int i = 0; i < kChunk; ++i) {
    const int blk = blk0 + i;
    if (blk * bs >= a.t_out) break;
    // K then V: unit u of the row covers (slot, head, 16-byte piece)
    for (int pass = 0; pass < 2; ++pass) {
      const int rec = pass ? lv.v_rec : lv.k_rec;
      const int units = rec / 16;
      const char* src = pass ? s_vsrc[i] : s_ksrc[i];
      char* dst = pass ? vout : kout;
      const int total_units = bs * n_kv * units;
      // tokens of this block that exist in the output / are visible
      const int t_end = min(bs, a.t_out - blk * bs);
      const int t_vis = src ? max(0, min(bs, len - blk * bs)) : 0;
      for (int u0 = threadIdx.x; u0 < total_units; u0 += kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int u = u0 + j * kThreads;
          const int slot = u / (units * n_kv);
          v[j] = (u32x4){0u, 0u, 0u, 0u};
          if (u < total_units && slot < t_vis)
            v[j] = __builtin_nontemporal_load((const gu32x4*)src + u);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int u = u0 + j * kThreads;
          const int piece = u % units;
          const int head = (u / units) % n_kv;
          const int slot = u / (units * n_kv);
          if (u < total_units && slot < t_end) {
            const size_t o = ((static_cast<size_t>(b) * n_kv + head) * a.t_out + blk * bs + slot) * rec +
                             piece * 16;
            __builtin_nontemporal_store(v[j], (gu32x4*)(dst + o));
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const GatherArgs& a, hipStream_t s) {
  const int bs = a.lv.block_size;
  const int chunks = (((a.t_out + bs - 1) / bs) + kChunk - 1) / kChunk;
  const long long total = static_cast<long long>(a.B) * chunks;
  if (total == 0) return hipSuccess;
  if (total > (1LL << 30)) return hipErrorInvalidValue;
  const int grid = round_up(static_cast<int>(total), kXcds);
  hipLaunchKernelGGL(gather_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pagedkv
