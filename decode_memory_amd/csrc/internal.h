// Internal declarations shared by the host side of the library (pool.hip) and
// the kernel translation units.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pagedkv.h"

namespace pagedkv {

// Everything a kernel needs to reach one layer's slabs.
struct LayerView {
  const void* const* k_tab;  // device: slab index -> K slab base
  const void* const* v_tab;  // device: slab index -> V slab base
  int32_t slab_blocks;       // rows per slab
  int32_t block_size;        // tokens per row
  int32_t n_kv;              // kv heads
  int32_t k_rec;             // bytes per K token-head record
  int32_t v_rec;             // bytes per V token-head record
  int64_t capacity_rows;     // rows that exist (n_slabs * slab_blocks)
  int32_t* err;              // device sticky error word
};

struct WriteArgs {
  LayerView lv;
  int32_t n;
  const int32_t* rows;
  const int32_t* slots;
  const void* k_src;
  const void* v_src;
  // packed formats
  int32_t head_dim;
  int32_t k_bits, v_bits;
  int32_t qgroup;      // values per (scale, offset) pair: 32 or 64
  const float* signs;  // device [head_dim] of +-1 (packed only)
  float inv_sqrt_d;
  uint32_t m_slab;     // reciprocal_u32(slab_blocks) when every row / slab_blocks is exact with it, else 0
};

// Whole block rows moved between two pool rows (copy_on_write_block), from
// pool rows to a contiguous buffer (export_blocks) or back (import_blocks).
// Buffer layout: [n][n_layers][K row bytes, V row bytes].
enum RowMoveMode { kMoveCopy = 0, kMoveExport = 1, kMoveImport = 2 };
struct RowMoveArgs {
  const void* const* tables;  // device: [n_layers][2][max_slabs] slab bases
  int32_t max_slabs;
  int32_t n_layers;
  int32_t slab_blocks;
  int64_t capacity_rows;
  int64_t row_bytes[2];       // bytes of one block row of K, of V
  int32_t n;
  const int32_t* src_rows;    // copy, export
  const int32_t* dst_rows;    // copy, import
  const char* src_buf;        // import
  char* dst_buf;              // export
  int32_t* err;
};

struct GatherArgs {
  LayerView lv;
  int32_t B;
  const int32_t* table;
  int32_t max_blocks;
  const int32_t* lens;
  int32_t t_out;
  void* k_out;
  void* v_out;
  int32_t* n_runs_out;
};

// The run split of a block table (split_runs).
struct RunArgs {
  LayerView lv;
  int32_t B;
  const int32_t* table;
  int32_t max_blocks;
  const int32_t* lens;
  int32_t* runs;    // [B][max_blocks][3]: (slab, first logical block, blocks)
  int32_t* n_runs;  // [B]
};

struct DecodeArgs {
  LayerView lv;
  int32_t B;
  int32_t n_q;
  const void* q;
  const int32_t* table;
  int32_t max_blocks;
  const int32_t* lens;
  float scale_log2;      // scale * log2(e): scores live in the exp2 domain
  void* out;
  // Split partials: running-weighted V [B * n_q][n_split][D] at partials,
  // then (max, sum) [B * n_q][n_split][2] at partials + ml_offset.
  float* partials;
  size_t ml_offset;      // floats
  int32_t n_split;       // split s of a sequence takes logical blocks s, s + n_split, ...
  int32_t blocks_per_split;  // most blocks any split takes (<= 64)
  // fused append (row kernel, packed kernel): [B, n_kv, D] 16-bit values of
  // the new token len_b - 1 of each sequence (bf16 for packed pools), or null
  const void* k_new;
  const void* v_new;
  // packed formats
  int32_t k_bits, v_bits;
  int32_t qgroup;  // values per (scale, offset) pair: 32 or 64
  const float* signs;
  float inv_sqrt_d;
};

// An append of new slabs, as one launch per up to kAppendMaxPairs (slab,
// layer) pairs: the launch records each pair's K and V slab base pointers in
// the device tables and zero-fills both slabs.  Passed by value, so the host
// arrays can be reused as soon as the launch is queued.
constexpr int kAppendMaxPairs = 96;
struct AppendArgs {
  void** tables;               // device [n_layers][2][max_slabs]
  int32_t max_slabs;
  int32_t n_pairs;             // pairs in this launch
  int64_t k_bytes, v_bytes;    // bytes of one K slab, one V slab
  int32_t entry[kAppendMaxPairs];  // table index of the pair's K pointer (V: + max_slabs)
  void* k_mem[kAppendMaxPairs];
  void* v_mem[kAppendMaxPairs];
};

// Duplicate-write check of write_block (pd_pool_set_debug): bit row *
// block_size + slot of `bits` per token of the call.
struct DupArgs {
  const int32_t* rows;
  const int32_t* slots;
  int32_t n;
  int64_t capacity_rows;
  int32_t block_size;
  uint32_t* bits;
  int32_t* err;
};

// Launchers (return the hipError_t of the launch; hipErrorInvalidValue when
// no kernel exists for the shape).
// mark == true: set each token's bit and flag PD_DEVERR_DUPLICATE where it
// was set already; mark == false: clear the words the tokens touched.
hipError_t launch_dup_check(const DupArgs& a, bool mark, hipStream_t s);

hipError_t launch_append_slabs(const AppendArgs& a, hipStream_t s);
hipError_t launch_write_block(const WriteArgs& a, int32_t format, hipStream_t s);
hipError_t launch_row_move(const RowMoveArgs& a, int mode, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);
hipError_t launch_split_runs(const RunArgs& a, hipStream_t s);
hipError_t launch_paged_decode_column(const DecodeArgs& a, bool bf16, int32_t head_dim,
                                      int32_t group, hipStream_t s);
hipError_t launch_paged_decode_row(const DecodeArgs& a, bool bf16, int32_t head_dim, int32_t group,
                                   int hgw, hipStream_t s);
hipError_t launch_decode_combine(const DecodeArgs& a, bool bf16, int32_t head_dim, hipStream_t s);
hipError_t launch_paged_decode_packed_mfma(const DecodeArgs& a, int32_t head_dim, int32_t group,
                                           hipStream_t s);
bool packed_mfma_supported(int32_t n_kv, int32_t head_dim, int32_t group, int32_t block_size,
                           int32_t qgroup);
int packed_mfma_target_workgroups(int32_t head_dim);
// Row kernel: head groups per workgroup (0 = shape not supported) and kv
// heads per workgroup.
int row_kernel_kpl(int32_t n_kv, int32_t head_dim, int32_t group, int32_t block_size);
int row_kernel_heads_per_workgroup(int32_t head_dim, int hgw);

// Split policy shared by the workspace query and the launch.
constexpr int kMaxBlocksPerSplit = 64;
constexpr int kMaxSplits = 1024;
inline int64_t max_decode_len(int32_t block_size) {
  return static_cast<int64_t>(kMaxBlocksPerSplit) * kMaxSplits * block_size;
}
struct SplitPlan {
  int32_t n_split;
  int32_t blocks_per_split;
};
// units: independent (sequence, head group) columns of work in the batch.
SplitPlan plan_splits(long long units, int32_t max_len, int32_t block_size, int target_workgroups,
                      int max_blocks_per_split);
size_t decode_ml_offset(int32_t B, int32_t n_q, int32_t head_dim, const SplitPlan& plan);  // floats
size_t decode_workspace_bytes(int32_t B, int32_t n_q, int32_t head_dim, const SplitPlan& plan);

}  // namespace pagedkv
