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
// blocks).  The workgroup splits its chunk into same-slab runs (a run that
// crosses a chunk edge is continued by the neighbouring workgroup), resolves
// each run's slab base pointer once, and copies the chunk's blocks in
// logical order as 16-byte vectors: each block's source is one contiguous
// row [block_size, n_kv, record]; the destination is n_kv contiguous pieces
// of block_size records.  The first chunk's workgroup also counts the
// sequence's runs over the whole row list for n_runs_out.
#include "device_common.h"
#include "internal.h"

namespace pagedkv {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4;  // logical blocks per workgroup

__device__ __forceinline__ int slab_of(int32_t row, const LayerView& lv) {
  return (row < 0 || row >= lv.capacity_rows) ? -1 : row / lv.slab_blocks;
}

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
  __shared__ const char* s_kbase[kChunk];
  __shared__ const char* s_vbase[kChunk];
  __shared__ int s_row[kChunk];
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

  // Run split of this chunk: a run starts at the chunk's first block or where
  // the slab changes; its first block loads the slab base, later blocks of
  // the run reuse it.
  const int blk0 = ch * kChunk;
  if (threadIdx.x == 0) {
    const char* kcur = nullptr;
    const char* vcur = nullptr;
    int prev_slab = -2;
    for (int i = 0; i < kChunk; ++i) {
      const int blk = blk0 + i;
      int row = -1, slab = -1;
      if (blk < nb) {
        row = trow[blk];
        slab = slab_of(row, lv);
        if (slab < 0) set_error(lv.err, PD_DEVERR_TABLE_ROW);
      }
      if (slab >= 0 && slab != prev_slab) {
        kcur = static_cast<const char*>(lv.k_tab[slab]);
        vcur = static_cast<const char*>(lv.v_tab[slab]);
      }
      prev_slab = slab;
      s_row[i] = slab >= 0 ? row - slab * lv.slab_blocks : -1;  // row in slab, -1 = zeros
      s_kbase[i] = kcur;
      s_vbase[i] = vcur;
    }
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

  const int n_kv = lv.n_kv;
  const int k_units = lv.k_rec / 16, v_units = lv.v_rec / 16;  // 16-byte units per record
  const size_t k_row_bytes = static_cast<size_t>(bs) * n_kv * lv.k_rec;
  const size_t v_row_bytes = static_cast<size_t>(bs) * n_kv * lv.v_rec;
  char* kout = static_cast<char*>(a.k_out);
  char* vout = static_cast<char*>(a.v_out);

  for (int i = 0; i < kChunk; ++i) {
    const int blk = blk0 + i;
    if (blk * bs >= a.t_out) break;
    const int ris = s_row[i];
    // K then V: unit u of the row covers (slot, head, 16-byte piece)
    for (int pass = 0; pass < 2; ++pass) {
      const int units = pass ? v_units : k_units;
      const int rec = pass ? lv.v_rec : lv.k_rec;
      const char* src = (ris >= 0) ? (pass ? s_vbase[i] : s_kbase[i]) +
                                         ris * (pass ? v_row_bytes : k_row_bytes)
                                   : nullptr;
      char* dst = pass ? vout : kout;
      const int total_units = bs * n_kv * units;
      for (int u = threadIdx.x; u < total_units; u += kThreads) {
        const int piece = u % units;
        const int head = (u / units) % n_kv;
        const int slot = u / (units * n_kv);
        const int t = blk * bs + slot;
        if (t >= a.t_out) continue;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (src && t < len) v = reinterpret_cast<const uint4*>(src)[u];
        const size_t o = ((static_cast<size_t>(b) * n_kv + head) * a.t_out + t) * rec + piece * 16;
        *reinterpret_cast<uint4*>(dst + o) = v;
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
