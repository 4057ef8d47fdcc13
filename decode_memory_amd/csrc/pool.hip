// Host side of libpagedkv: the chunked-slab pool object, its device
// slab-pointer tables, argument validation and kernel dispatch.
//
// mlxcel issue #235 ("perf(core): chunked slab storage for the paged pool to
// eliminate growth reallocation entirely"), section "Proposed solution:
// chunked slabs": per-layer vectors of fixed-size slabs replace the single
// pool tensor; growth appends zeroed slabs (one per layer, since physical
// row ids are shared by all layers) and is counted by a slab-append counter;
// pool byte accounting sums over slabs; one slab_for_row helper is the only
// place that maps a row to (slab, row_in_slab).
#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "index_math.h"
#include "internal.h"

using namespace pagedkv;

// Workgroups a decode launch aims for (column kernel: 3 of 4 waves resident
// per CU; row kernel: one workgroup of 8 waves per CU) and the row kernel's
// largest split.
#ifndef PAGEDKV_DECODE_TARGET_WG
#define PAGEDKV_DECODE_TARGET_WG 768
#endif
#ifndef PAGEDKV_ROW_TARGET_WG
#define PAGEDKV_ROW_TARGET_WG 256
#endif
#ifndef PAGEDKV_ROW_MAX_BLOCKS_PER_SPLIT
#define PAGEDKV_ROW_MAX_BLOCKS_PER_SPLIT 32
#endif

struct pd_pool {
  pd_pool_desc desc{};
  int device = 0;
  int32_t k_rec = 0, v_rec = 0;
  int32_t k_bits = 16, v_bits = 16;
  int32_t qgroup = 0;  // packed: values per (scale, offset) pair
  size_t k_slab_bytes = 0, v_slab_bytes = 0;
  int64_t n_slabs = 0;
  int64_t append_events = 0;
  // tables: layer l uses [l * 2 * max_slabs, +max_slabs) for K and the next
  // max_slabs entries for V.  The pinned host mirror is only ever appended
  // to, so an asynchronous copy out of it never races a later update.
  void** h_tables = nullptr;
  void** d_tables = nullptr;
  int32_t* d_err = nullptr;
  float* d_signs = nullptr;  // packed: [head_dim] of +-1
  uint64_t signs_hash = 0;   // packed: pd_signs_hash of the signs
  float inv_sqrt_d = 1.f;
  uint32_t debug = 0;          // PD_DEBUG_* bits
  uint32_t* d_dup = nullptr;   // duplicate-write bitmap, one bit per slot of max capacity
};

// Device scratch of pd_paged_decode_noalloc, for callers that cannot
// allocate: the split partials of one call live here instead of in a
// caller-provided workspace.  Each device the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: the host reaches the memory only
// through the address hipGetSymbolAddress returns for the current device,
// kept per device in g_scratch.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_last_error;

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  bool resolved = false;  // hipGetSymbolAddress has run on this device
  hipError_t status = hipSuccess;
  void* ptr = nullptr;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

// Once per device, with that device current (pd_pool_create): the device
// address of this device's copy of `scratch`.
void resolve_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[device];
  if (slot.resolved) return;
  void* ptr = nullptr;
  slot.status = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  slot.ptr = slot.status == hipSuccess ? ptr : nullptr;
  slot.resolved = true;
}

pd_status fail(pd_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pd_status fail(pd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pd_status hip_fail(hipError_t e, const char* what) {
  return fail(PD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_native(int32_t f) { return f == PD_FMT_FP16 || f == PD_FMT_BF16; }
bool is_packed(int32_t f) { return f == PD_FMT_K8V8 || f == PD_FMT_K8V4 || f == PD_FMT_K4V4; }

void format_bits(int32_t f, int32_t* kb, int32_t* vb) {
  switch (f) {
    case PD_FMT_K8V8: *kb = 8; *vb = 8; break;
    case PD_FMT_K8V4: *kb = 8; *vb = 4; break;
    case PD_FMT_K4V4: *kb = 4; *vb = 4; break;
    default: *kb = 16; *vb = 16; break;
  }
}

int32_t record_bytes_for(int32_t bits, int32_t d, int32_t qgroup) {
  if (bits == 16) return 2 * d;
  return d * bits / 8 + (d / qgroup) * 8;  // codes + (scale, offset) per group
}

// The packed group size a pool or query asks for (0 means 32); 0 if it is
// not one the kernels take for this head_dim.
int32_t packed_group_or_zero(int32_t group_size, int32_t head_dim) {
  const int32_t g = group_size == 0 ? 32 : group_size;
  if (g == 32) return 32;
  if (g == 64 && head_dim >= 128) return 64;
  return 0;
}

LayerView layer_view(const pd_pool* p, int32_t layer) {
  LayerView lv;
  const int ms = p->desc.max_slabs;
  lv.k_tab = const_cast<const void* const*>(p->d_tables + static_cast<size_t>(layer) * 2 * ms);
  lv.v_tab = lv.k_tab + ms;
  lv.slab_blocks = p->desc.slab_blocks;
  lv.block_size = p->desc.block_size;
  lv.n_kv = p->desc.n_kv_heads;
  lv.k_rec = p->k_rec;
  lv.v_rec = p->v_rec;
  lv.capacity_rows = p->n_slabs * p->desc.slab_blocks;
  lv.err = p->d_err;
  return lv;
}

pd_status check_pool(const pd_pool* p) {
  if (!p) return fail(PD_ERR_ARG, "pool is NULL");
  return PD_OK;
}

pd_status check_layer(const pd_pool* p, int32_t layer) {
  if (layer < 0 || layer >= p->desc.n_layers)
    return fail(PD_ERR_RANGE, "layer %d outside [0, %d)", layer, p->desc.n_layers);
  return PD_OK;
}

// Record `n` new slabs per layer (slab-major pointer arrays) after checks.
pd_status append_slabs(pd_pool* p, int32_t n, void* const* k_mem, void* const* v_mem,
                       hipStream_t stream) {
  const int L = p->desc.n_layers;
  if (n < 0) return fail(PD_ERR_ARG, "negative slab count");
  if (n == 0) return PD_OK;
  if (!k_mem || !v_mem) return fail(PD_ERR_ARG, "slab pointer arrays are NULL");
  if (p->n_slabs + n > p->desc.max_slabs)
    return fail(PD_ERR_CAPACITY, "pool holds %lld slabs, max_slabs is %d",
                static_cast<long long>(p->n_slabs), p->desc.max_slabs);
  for (int64_t i = 0; i < static_cast<int64_t>(n) * L; ++i) {
    if (!k_mem[i] || !v_mem[i]) return fail(PD_ERR_ARG, "slab pointer %lld is NULL", (long long)i);
    if ((reinterpret_cast<uintptr_t>(k_mem[i]) | reinterpret_cast<uintptr_t>(v_mem[i])) & 255)
      return fail(PD_ERR_ARG, "slab pointer %lld is not 256-byte aligned", (long long)i);
  }
  hipError_t e = hipSetDevice(p->device);
  if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
  // One launch per kAppendMaxPairs (slab, layer) pairs records the new base
  // pointers in the device tables and zero-fills the new slabs (one launch
  // for a single slab in up to 96 layers).  Nothing is recorded on the host
  // until every launch is queued.
  const int ms = p->desc.max_slabs;
  const int64_t pairs = static_cast<int64_t>(n) * L;
  AppendArgs a{};
  a.tables = p->d_tables;
  a.max_slabs = ms;
  a.k_bytes = static_cast<int64_t>(p->k_slab_bytes);
  a.v_bytes = static_cast<int64_t>(p->v_slab_bytes);
  for (int64_t i0 = 0; i0 < pairs; i0 += kAppendMaxPairs) {
    a.n_pairs = static_cast<int32_t>(pairs - i0 < kAppendMaxPairs ? pairs - i0 : kAppendMaxPairs);
    for (int j = 0; j < a.n_pairs; ++j) {
      const int64_t i = i0 + j;  // slab-major, as k_mem / v_mem
      const int64_t slab = p->n_slabs + i / L;
      const int64_t l = i % L;
      a.entry[j] = static_cast<int32_t>(l * 2 * ms + slab);
      a.k_mem[j] = k_mem[i];
      a.v_mem[j] = v_mem[i];
    }
    if ((e = launch_append_slabs(a, stream)) != hipSuccess) return hip_fail(e, "append_slabs launch");
  }
  for (int s = 0; s < n; ++s) {
    const int64_t slab = p->n_slabs + s;
    for (int l = 0; l < L; ++l) {
      p->h_tables[static_cast<size_t>(l) * 2 * ms + slab] = k_mem[static_cast<size_t>(s) * L + l];
      p->h_tables[static_cast<size_t>(l) * 2 * ms + ms + slab] = v_mem[static_cast<size_t>(s) * L + l];
    }
  }
  p->n_slabs += n;
  p->append_events += n;
  return PD_OK;
}

}  // namespace

namespace pagedkv {

SplitPlan plan_splits(long long units, int32_t max_len, int32_t block_size, int target_workgroups,
                      int max_blocks_per_split) {
  // Enough splits of the token axis that about target_workgroups workgroups
  // are launched; a split holds 1..max_blocks_per_split blocks (at most 64:
  // the kernels keep one block address per lane of a wave) and there are at
  // most kMaxSplits splits (the combine stages one weight per split in LDS).
  // Split s takes logical blocks s, s + n_split, ... so the blocks read at
  // any moment by the whole launch lie close together.
  SplitPlan p{1, 1};
  const int max_nb = max_len > 0 ? (max_len + block_size - 1) / block_size : 1;
  long long want = units > 0 ? (target_workgroups + units - 1) / units : 1;
  if (want < 1) want = 1;
  if (want > max_nb) want = max_nb;
  int bps = static_cast<int>((max_nb + want - 1) / want);
  const int cap = max_blocks_per_split < kMaxBlocksPerSplit ? max_blocks_per_split : kMaxBlocksPerSplit;
  if (bps > cap) bps = cap;
  if ((max_nb + bps - 1) / bps > kMaxSplits) bps = (max_nb + kMaxSplits - 1) / kMaxSplits;
  p.n_split = (max_nb + bps - 1) / bps;
  p.blocks_per_split = (max_nb + p.n_split - 1) / p.n_split;
  return p;
}

size_t decode_ml_offset(int32_t B, int32_t n_q, int32_t head_dim, const SplitPlan& plan) {
  const size_t acc = static_cast<size_t>(B) * n_q * plan.n_split * head_dim;
  return (acc + 63) / 64 * 64;  // 256-byte aligned
}

size_t decode_workspace_bytes(int32_t B, int32_t n_q, int32_t head_dim, const SplitPlan& plan) {
  const size_t ml = static_cast<size_t>(B) * n_q * plan.n_split * 2;
  return (decode_ml_offset(B, n_q, head_dim, plan) + ml) * sizeof(float);
}

}  // namespace pagedkv

namespace {

// Which decode kernel runs for a call, and how the token axis is split.
struct DecodePlan {
  int kind = 0;  // 0: column kernel, 1: row kernel, 2: packed (matrix-core) kernel
  int kpl = 0;   // row kernel: kv heads per lane group
  SplitPlan split{1, 1};
};

// The kernel and split of the token axis for a call; it depends only on the
// storage shape and (B, group, max_len), so a dense call and a paged call of
// the same shape run the same arithmetic in the same order.
bool make_decode_plan_for(int32_t format, int32_t n_kv, int32_t D, int32_t bs, int32_t B,
                          int32_t group, int32_t max_len, int32_t qgroup, DecodePlan* out) {
  const bool d_ok = D == 64 || D == 128 || D == 256;
  const bool g_ok = group == 1 || group == 2 || group == 4 || group == 8;
  if (!d_ok || !g_ok) return false;
  DecodePlan plan;
  long long units = static_cast<long long>(B) * n_kv;
  int target = PAGEDKV_DECODE_TARGET_WG, max_bps = kMaxBlocksPerSplit;
  if (is_native(format)) {
    if (bs != 16 && bs != 32 && bs != 64) return false;
    plan.kpl = row_kernel_kpl(n_kv, D, group, bs);
    if (plan.kpl > 0) {
      plan.kind = 1;
      units = static_cast<long long>(B) * (n_kv / row_kernel_heads_per_workgroup(D, plan.kpl));
      target = PAGEDKV_ROW_TARGET_WG;
      max_bps = PAGEDKV_ROW_MAX_BLOCKS_PER_SPLIT;
    }
  } else {
    if (!packed_mfma_supported(n_kv, D, group, bs, qgroup)) return false;
    plan.kind = 2;
    units = B;  // a packed workgroup covers every kv head of its sequence
    target = packed_mfma_target_workgroups(D);
  }
  plan.split = plan_splits(units, max_len, bs, target, max_bps);
  *out = plan;
  return true;
}

// Launch sizes stay in 32-bit arithmetic (grids, work ids, partial rows).
pd_status check_decode_size(int32_t B, int32_t n_q_heads, const DecodePlan& plan) {
  const long long rows = static_cast<long long>(B) * n_q_heads * plan.split.n_split;
  if (rows > (1LL << 30))
    return fail(PD_ERR_ARG, "B * n_q_heads * splits = %lld beyond 2^30 (B %d, n_q_heads %d, %d splits)", rows,
                B, n_q_heads, plan.split.n_split);
  return PD_OK;
}

bool make_decode_plan(const pd_pool* p, int32_t B, int32_t group, int32_t max_len, DecodePlan* out) {
  return make_decode_plan_for(p->desc.format, p->desc.n_kv_heads, p->desc.head_dim, p->desc.block_size,
                              B, group, max_len, p->qgroup, out);
}

}  // namespace

extern "C" {

int32_t pd_version(void) { return PD_VERSION; }

const char* pd_last_error(void) { return g_last_error.c_str(); }

pd_status pd_record_bytes(int32_t format, int32_t head_dim, int32_t group_size, int32_t* k_bytes,
                          int32_t* v_bytes) {
  if (!is_native(format) && !is_packed(format)) return fail(PD_ERR_ARG, "unknown format %d", format);
  if (head_dim <= 0) return fail(PD_ERR_ARG, "head_dim must be positive");
  const int32_t g = group_size == 0 ? 32 : group_size;
  if (is_packed(format) && (g <= 0 || head_dim % g != 0))
    return fail(PD_ERR_ARG, "group_size %d does not divide head_dim %d", group_size, head_dim);
  int32_t kb, vb;
  format_bits(format, &kb, &vb);
  if (k_bytes) *k_bytes = record_bytes_for(kb, head_dim, g);
  if (v_bytes) *v_bytes = record_bytes_for(vb, head_dim, g);
  return PD_OK;
}

pd_status pd_pool_create(const pd_pool_desc* d, pd_pool** out) {
  if (!d || !out) return fail(PD_ERR_ARG, "desc and out must not be NULL");
  *out = nullptr;
  if (d->n_layers < 1 || d->n_kv_heads < 1 || d->slab_blocks < 1 || d->max_slabs < 1 ||
      d->block_size < 1)
    return fail(PD_ERR_ARG, "n_layers, n_kv_heads, slab_blocks, max_slabs, block_size must be >= 1");
  if (!is_native(d->format) && !is_packed(d->format))
    return fail(PD_ERR_ARG, "unknown format %d", d->format);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
    return fail(PD_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128, 256)", d->head_dim);
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64)
    return fail(PD_ERR_UNSUPPORTED, "block_size %d (supported: 16, 32, 64)", d->block_size);
  if (is_packed(d->format) && d->block_size != 32)
    return fail(PD_ERR_UNSUPPORTED, "packed formats use block_size 32");
  // the packed decode kernel gives one wave to each of 8 kv heads: a pool it
  // could not decode is refused here, before anything is written to it
  if (is_packed(d->format) && d->n_kv_heads != 8)
    return fail(PD_ERR_UNSUPPORTED, "packed formats need n_kv_heads 8 (got %d)", d->n_kv_heads);
  if (is_native(d->format) && d->group_size != 0)
    return fail(PD_ERR_ARG, "group_size %d: 16-bit formats have no groups (pass 0)", d->group_size);
  if (is_packed(d->format) && packed_group_or_zero(d->group_size, d->head_dim) == 0)
    return fail(PD_ERR_UNSUPPORTED, "group_size %d with head_dim %d (supported: 32; 64 with head_dim 128, 256)",
                d->group_size, d->head_dim);
  if (is_packed(d->format)) {
    if (!d->hadamard_signs) return fail(PD_ERR_ARG, "packed formats need hadamard_signs");
    for (int i = 0; i < d->head_dim; ++i)
      if (d->hadamard_signs[i] != 1 && d->hadamard_signs[i] != -1)
        return fail(PD_ERR_ARG, "hadamard_signs[%d] is %d, not +-1", i, d->hadamard_signs[i]);
  }
  const size_t table_entries = static_cast<size_t>(d->n_layers) * 2 * d->max_slabs;
  if (table_entries > (size_t{1} << 28)) return fail(PD_ERR_ARG, "slab tables too large");

  pd_pool* p = new pd_pool;
  p->desc = *d;
  p->desc.hadamard_signs = nullptr;
  format_bits(d->format, &p->k_bits, &p->v_bits);
  p->qgroup = is_packed(d->format) ? packed_group_or_zero(d->group_size, d->head_dim) : 0;
  p->desc.group_size = p->qgroup;
  p->k_rec = record_bytes_for(p->k_bits, d->head_dim, p->qgroup);
  p->v_rec = record_bytes_for(p->v_bits, d->head_dim, p->qgroup);
  const size_t per = static_cast<size_t>(d->slab_blocks) * d->block_size * d->n_kv_heads;
  p->k_slab_bytes = per * p->k_rec;
  p->v_slab_bytes = per * p->v_rec;
  p->inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d->head_dim)));

  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) resolve_scratch(p->device);  // a failure is reported by the no-alloc call
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&p->h_tables),
                                         table_entries * sizeof(void*), hipHostMallocDefault);
  if (e == hipSuccess) {
    std::memset(p->h_tables, 0, table_entries * sizeof(void*));
    e = hipMalloc(reinterpret_cast<void**>(&p->d_tables), table_entries * sizeof(void*));
  }
  if (e == hipSuccess) e = hipMemset(p->d_tables, 0, table_entries * sizeof(void*));
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&p->d_err), 256);
  if (e == hipSuccess) e = hipMemset(p->d_err, 0, 256);
  if (e == hipSuccess && is_packed(d->format)) {
    pd_signs_hash(d->hadamard_signs, d->head_dim, &p->signs_hash);
    std::vector<float> s(d->head_dim);
    for (int i = 0; i < d->head_dim; ++i) s[i] = static_cast<float>(d->hadamard_signs[i]);
    e = hipMalloc(reinterpret_cast<void**>(&p->d_signs), sizeof(float) * d->head_dim);
    if (e == hipSuccess)
      e = hipMemcpy(p->d_signs, s.data(), sizeof(float) * d->head_dim, hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    pd_pool_destroy(p);
    return hip_fail(e, "pool_create");
  }
  *out = p;
  return PD_OK;
}

pd_status pd_pool_destroy(pd_pool* p) {
  if (!p) return PD_OK;
  int cur = 0;
  hipGetDevice(&cur);
  hipSetDevice(p->device);
  hipDeviceSynchronize();  // kernels may still read the tables
  if (p->d_tables) hipFree(p->d_tables);
  if (p->d_err) hipFree(p->d_err);
  if (p->d_signs) hipFree(p->d_signs);
  if (p->d_dup) hipFree(p->d_dup);
  if (p->h_tables) hipHostFree(p->h_tables);
  hipSetDevice(cur);
  delete p;
  return PD_OK;
}

pd_status pd_slab_bytes(const pd_pool* p, size_t* k_bytes, size_t* v_bytes) {
  if (pd_status st = check_pool(p)) return st;
  if (k_bytes) *k_bytes = p->k_slab_bytes;
  if (v_bytes) *v_bytes = p->v_slab_bytes;
  return PD_OK;
}

pd_status pd_append_slab(pd_pool* p, void* const* k_mem, void* const* v_mem, hipStream_t stream,
                         int32_t* new_index) {
  if (pd_status st = check_pool(p)) return st;
  const int64_t idx = p->n_slabs;
  if (pd_status st = append_slabs(p, 1, k_mem, v_mem, stream)) return st;
  if (new_index) *new_index = static_cast<int32_t>(idx);
  return PD_OK;
}

pd_status pd_slabs_needed(const pd_pool* p, int64_t rows_needed, int32_t* n_slabs) {
  if (pd_status st = check_pool(p)) return st;
  if (rows_needed < 0 || !n_slabs) return fail(PD_ERR_ARG, "rows_needed < 0 or n_slabs NULL");
  const int64_t S = p->desc.slab_blocks;
  const int64_t want = (rows_needed + S - 1) / S;
  *n_slabs = static_cast<int32_t>(want > p->n_slabs ? want - p->n_slabs : 0);
  return PD_OK;
}

pd_status pd_reserve_rows(pd_pool* p, int64_t rows_needed, void* const* k_mem, void* const* v_mem,
                          int32_t n_slabs, hipStream_t stream, int32_t* n_appended) {
  if (pd_status st = check_pool(p)) return st;
  int32_t need = 0;
  if (pd_status st = pd_slabs_needed(p, rows_needed, &need)) return st;
  if (n_slabs != need)
    return fail(PD_ERR_ARG, "reserve_rows(%lld) needs %d slabs, %d given",
                static_cast<long long>(rows_needed), need, n_slabs);
  if (pd_status st = append_slabs(p, need, k_mem, v_mem, stream)) return st;
  if (n_appended) *n_appended = need;
  return PD_OK;
}

pd_status pd_slab_for_row(const pd_pool* p, int32_t layer, int64_t row, void** k_base,
                          void** v_base, int32_t* row_in_slab) {
  if (pd_status st = check_pool(p)) return st;
  if (pd_status st = check_layer(p, layer)) return st;
  const int64_t S = p->desc.slab_blocks;
  if (row < 0 || row >= p->n_slabs * S)
    return fail(PD_ERR_RANGE, "row %lld outside [0, %lld)", static_cast<long long>(row),
                static_cast<long long>(p->n_slabs * S));
  const int64_t slab = row / S;
  const size_t ms = p->desc.max_slabs;
  if (k_base) *k_base = p->h_tables[layer * 2 * ms + slab];
  if (v_base) *v_base = p->h_tables[layer * 2 * ms + ms + slab];
  if (row_in_slab) *row_in_slab = static_cast<int32_t>(row % S);
  return PD_OK;
}

pd_status pd_write_block(pd_pool* p, int32_t layer, int32_t n, const int32_t* rows,
                         const int32_t* slots, const void* k_src, const void* v_src,
                         hipStream_t stream) {
  if (pd_status st = check_pool(p)) return st;
  if (pd_status st = check_layer(p, layer)) return st;
  if (n < 0) return fail(PD_ERR_ARG, "n < 0");
  if (n == 0) return PD_OK;
  if (!rows || !slots || !k_src || !v_src) return fail(PD_ERR_ARG, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(k_src) | reinterpret_cast<uintptr_t>(v_src)) & 15)
    return fail(PD_ERR_ARG, "k_src and v_src must be 16-byte aligned");
  WriteArgs a{};
  a.lv = layer_view(p, layer);
  a.n = n;
  a.rows = rows;
  a.slots = slots;
  a.k_src = k_src;
  a.v_src = v_src;
  a.head_dim = p->desc.head_dim;
  a.k_bits = p->k_bits;
  a.v_bits = p->v_bits;
  a.qgroup = p->qgroup;
  a.signs = p->d_signs;
  a.inv_sqrt_d = p->inv_sqrt_d;
  // the high multiply is exact for every row below capacity while
  // capacity_rows < 2^32 / slab_blocks
  const uint64_t S = static_cast<uint64_t>(p->desc.slab_blocks);
  a.m_slab = static_cast<uint64_t>(a.lv.capacity_rows) * S < (uint64_t{1} << 32) ? reciprocal_u32(static_cast<uint32_t>(S)) : 0u;
  if (S == 1) a.m_slab = 0;  // 0 means divide (by one)
  const bool dup = (p->debug & PD_DEBUG_DUPLICATE_WRITES) != 0;
  DupArgs d{rows, slots, n, a.lv.capacity_rows, p->desc.block_size, p->d_dup, p->d_err};
  if (dup) {
    if (hipError_t e = launch_dup_check(d, true, stream)) return hip_fail(e, "duplicate-write check launch");
  }
  hipError_t e = launch_write_block(a, p->desc.format, stream);
  if (e == hipErrorInvalidValue) e = hipErrorNotSupported;
  // the bitmap is cleared even when the write could not launch, so it is all
  // zero again for the next call
  if (dup) {
    if (hipError_t ec = launch_dup_check(d, false, stream)) return hip_fail(ec, "duplicate-write clear launch");
  }
  if (e == hipErrorNotSupported) return fail(PD_ERR_UNSUPPORTED, "no write_block kernel for this shape");
  if (e != hipSuccess) return hip_fail(e, "write_block launch");
  return PD_OK;
}

pd_status pd_pool_set_debug(pd_pool* p, uint32_t flags) {
  if (pd_status st = check_pool(p)) return st;
  if (flags & ~PD_DEBUG_DUPLICATE_WRITES) return fail(PD_ERR_ARG, "unknown debug flag bits 0x%x", flags);
  if ((flags & PD_DEBUG_DUPLICATE_WRITES) && !p->d_dup) {
    const uint64_t bits = static_cast<uint64_t>(p->desc.max_slabs) * p->desc.slab_blocks * p->desc.block_size;
    const size_t bytes = static_cast<size_t>((bits + 31) / 32) * 4;
    int cur = 0;
    hipGetDevice(&cur);
    hipSetDevice(p->device);
    void* mem = nullptr;
    hipError_t e = hipMalloc(&mem, bytes);
    if (e == hipSuccess) e = hipMemset(mem, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    hipSetDevice(cur);
    if (e != hipSuccess) {
      if (mem) hipFree(mem);
      return hip_fail(e, "duplicate-write bitmap");
    }
    p->d_dup = static_cast<uint32_t*>(mem);
  }
  p->debug = flags;
  return PD_OK;
}

}  // extern "C"

namespace {

RowMoveArgs row_move_args(const pd_pool* p, int32_t n) {
  RowMoveArgs a{};
  a.tables = const_cast<const void* const*>(p->d_tables);
  a.max_slabs = p->desc.max_slabs;
  a.n_layers = p->desc.n_layers;
  a.slab_blocks = p->desc.slab_blocks;
  a.capacity_rows = p->n_slabs * p->desc.slab_blocks;
  const int64_t tok = static_cast<int64_t>(p->desc.block_size) * p->desc.n_kv_heads;
  a.row_bytes[0] = tok * p->k_rec;
  a.row_bytes[1] = tok * p->v_rec;
  a.n = n;
  a.err = p->d_err;
  return a;
}

size_t block_bytes(const pd_pool* p) {
  return static_cast<size_t>(p->desc.n_layers) * p->desc.block_size * p->desc.n_kv_heads *
         static_cast<size_t>(p->k_rec + p->v_rec);
}

void identity_of(const pd_pool* p, pd_storage_identity* id) {
  std::memset(id, 0, sizeof *id);
  id->magic = PD_IDENTITY_MAGIC;
  id->layout = PD_IDENTITY_LAYOUT;
  id->format = p->desc.format;
  id->n_layers = p->desc.n_layers;
  id->block_size = p->desc.block_size;
  id->n_kv_heads = p->desc.n_kv_heads;
  id->head_dim = p->desc.head_dim;
  id->k_record_bytes = p->k_rec;
  id->v_record_bytes = p->v_rec;
  id->group_size = p->qgroup;
  id->signs_hash = p->signs_hash;
}

}  // namespace

extern "C" {

pd_status pd_copy_on_write_block(pd_pool* p, int32_t n, const int32_t* src_rows,
                                 const int32_t* dst_rows, hipStream_t stream) {
  if (pd_status st = check_pool(p)) return st;
  if (n < 0) return fail(PD_ERR_ARG, "n < 0");
  if (n == 0) return PD_OK;
  if (!src_rows || !dst_rows) return fail(PD_ERR_ARG, "NULL device pointer");
  RowMoveArgs a = row_move_args(p, n);
  a.src_rows = src_rows;
  a.dst_rows = dst_rows;
  hipError_t e = launch_row_move(a, kMoveCopy, stream);
  if (e != hipSuccess) return hip_fail(e, "copy_on_write_block launch");
  return PD_OK;
}

pd_status pd_signs_hash(const int8_t* signs, int32_t n, uint64_t* hash) {
  if (!hash || n < 0 || (n > 0 && !signs)) return fail(PD_ERR_ARG, "signs NULL, n < 0 or hash NULL");
  uint64_t h = 0xcbf29ce484222325ull;  // FNV-1a 64 offset basis
  for (int32_t i = 0; i < n; ++i) {
    h ^= static_cast<uint8_t>(signs[i]);
    h *= 0x100000001b3ull;             // FNV-1a 64 prime
  }
  *hash = h;
  return PD_OK;
}

pd_status pd_storage_identity_of(const pd_pool* p, pd_storage_identity* id) {
  if (pd_status st = check_pool(p)) return st;
  if (!id) return fail(PD_ERR_ARG, "id is NULL");
  identity_of(p, id);
  return PD_OK;
}

pd_status pd_identity_check(const pd_pool* p, const pd_storage_identity* id) {
  if (pd_status st = check_pool(p)) return st;
  if (!id) return fail(PD_ERR_ARG, "id is NULL");
  pd_storage_identity mine;
  identity_of(p, &mine);
#define PD_FIELD(f)                                                                            \
  if (id->f != mine.f)                                                                         \
    return fail(PD_ERR_IDENTITY, "storage identity differs in " #f ": blocks have %lld, pool has %lld", \
                static_cast<long long>(id->f), static_cast<long long>(mine.f));
  PD_FIELD(magic)
  PD_FIELD(layout)
  PD_FIELD(format)
  PD_FIELD(n_layers)
  PD_FIELD(block_size)
  PD_FIELD(n_kv_heads)
  PD_FIELD(head_dim)
  PD_FIELD(k_record_bytes)
  PD_FIELD(v_record_bytes)
  PD_FIELD(group_size)
  PD_FIELD(signs_hash)
#undef PD_FIELD
  return PD_OK;
}

pd_status pd_block_bytes(const pd_pool* p, size_t* bytes) {
  if (pd_status st = check_pool(p)) return st;
  if (!bytes) return fail(PD_ERR_ARG, "bytes is NULL");
  *bytes = block_bytes(p);
  return PD_OK;
}

pd_status pd_export_blocks(pd_pool* p, int32_t n, const int32_t* rows, void* dst, size_t dst_bytes,
                           hipStream_t stream) {
  if (pd_status st = check_pool(p)) return st;
  if (n < 0) return fail(PD_ERR_ARG, "n < 0");
  if (n == 0) return PD_OK;
  if (!rows || !dst) return fail(PD_ERR_ARG, "NULL device pointer");
  if (reinterpret_cast<uintptr_t>(dst) & 15) return fail(PD_ERR_ARG, "dst must be 16-byte aligned");
  if (dst_bytes < static_cast<size_t>(n) * block_bytes(p))
    return fail(PD_ERR_CAPACITY, "dst holds %zu bytes, %zu needed", dst_bytes,
                static_cast<size_t>(n) * block_bytes(p));
  RowMoveArgs a = row_move_args(p, n);
  a.src_rows = rows;
  a.dst_buf = static_cast<char*>(dst);
  hipError_t e = launch_row_move(a, kMoveExport, stream);
  if (e != hipSuccess) return hip_fail(e, "export_blocks launch");
  return PD_OK;
}

pd_status pd_import_blocks(pd_pool* p, const pd_storage_identity* id, int32_t n, const int32_t* rows,
                           const void* src, size_t src_bytes, hipStream_t stream) {
  if (pd_status st = pd_identity_check(p, id)) return st;
  if (n < 0) return fail(PD_ERR_ARG, "n < 0");
  if (n == 0) return PD_OK;
  if (!rows || !src) return fail(PD_ERR_ARG, "NULL device pointer");
  if (reinterpret_cast<uintptr_t>(src) & 15) return fail(PD_ERR_ARG, "src must be 16-byte aligned");
  if (src_bytes < static_cast<size_t>(n) * block_bytes(p))
    return fail(PD_ERR_CAPACITY, "src holds %zu bytes, %zu needed", src_bytes,
                static_cast<size_t>(n) * block_bytes(p));
  RowMoveArgs a = row_move_args(p, n);
  a.dst_rows = rows;
  a.src_buf = static_cast<const char*>(src);
  hipError_t e = launch_row_move(a, kMoveImport, stream);
  if (e != hipSuccess) return hip_fail(e, "import_blocks launch");
  return PD_OK;
}

pd_status pd_gather_visible(pd_pool* p, int32_t layer, int32_t B, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* lens, int32_t t_out, void* k_out,
                            void* v_out, int32_t* n_runs_out, hipStream_t stream) {
  if (pd_status st = check_pool(p)) return st;
  if (pd_status st = check_layer(p, layer)) return st;
  if (B < 0 || max_blocks < 1 || t_out < 0) return fail(PD_ERR_ARG, "B < 0, max_blocks < 1 or t_out < 0");
  if (B == 0 || t_out == 0) return PD_OK;
  if (!block_table || !lens || !k_out || !v_out) return fail(PD_ERR_ARG, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(PD_ERR_ARG, "outputs must be 16-byte aligned");
  GatherArgs a{};
  a.lv = layer_view(p, layer);
  a.B = B;
  a.table = block_table;
  a.max_blocks = max_blocks;
  a.lens = lens;
  a.t_out = t_out;
  a.k_out = k_out;
  a.v_out = v_out;
  a.n_runs_out = n_runs_out;
  hipError_t e = launch_gather(a, stream);
  if (e != hipSuccess) return hip_fail(e, "gather_visible launch");
  return PD_OK;
}

pd_status pd_split_runs(pd_pool* p, int32_t B, const int32_t* block_table, int32_t max_blocks,
                        const int32_t* lens, int32_t* runs_out, int32_t* n_runs_out, hipStream_t stream) {
  if (pd_status st = check_pool(p)) return st;
  if (B < 0 || max_blocks < 1) return fail(PD_ERR_ARG, "B < 0 or max_blocks < 1");
  if (B == 0) return PD_OK;
  if (!block_table || !lens || !runs_out || !n_runs_out) return fail(PD_ERR_ARG, "NULL device pointer");
  if (static_cast<int64_t>(max_blocks) * p->desc.block_size > INT32_MAX)
    return fail(PD_ERR_ARG, "max_blocks * block_size beyond 2^31");
  RunArgs a{};
  a.lv = layer_view(p, 0);
  a.B = B;
  a.table = block_table;
  a.max_blocks = max_blocks;
  a.lens = lens;
  a.runs = runs_out;
  a.n_runs = n_runs_out;
  hipError_t e = launch_split_runs(a, stream);
  if (e != hipSuccess) return hip_fail(e, "split_runs launch");
  return PD_OK;
}

pd_status pd_decode_workspace_bytes(const pd_pool* p, int32_t B, int32_t n_q_heads,
                                    int32_t max_len, size_t* bytes) {
  if (pd_status st = check_pool(p)) return st;
  if (!bytes || B < 0 || max_len < 0 || n_q_heads < 1)
    return fail(PD_ERR_ARG, "bytes NULL, B < 0, max_len < 0 or n_q_heads < 1");
  const int32_t n_kv = p->desc.n_kv_heads;
  if (n_q_heads % n_kv) return fail(PD_ERR_ARG, "n_q_heads %d not a multiple of n_kv_heads %d",
                                    n_q_heads, n_kv);
  if (static_cast<int64_t>(max_len) > max_decode_len(p->desc.block_size))
    return fail(PD_ERR_UNSUPPORTED, "max_len %d beyond %lld", max_len,
                static_cast<long long>(max_decode_len(p->desc.block_size)));
  DecodePlan plan;
  if (!make_decode_plan(p, B, n_q_heads / n_kv, max_len, &plan))
    return fail(PD_ERR_UNSUPPORTED, "no decode kernel for format %d, head_dim %d, group %d",
                p->desc.format, p->desc.head_dim, n_q_heads / n_kv);
  if (pd_status st = check_decode_size(B, n_q_heads, plan)) return st;
  *bytes = decode_workspace_bytes(B, n_q_heads, p->desc.head_dim, plan.split);
  return PD_OK;
}

// Stages of paged_decode run by decode_call.
static const int kStageSplit = 1, kStageCombine = 2;

static pd_status decode_call(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads, const void* q,
                      const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
                      int32_t max_len, float scale, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, int stages,
                      const void* k_new = nullptr, const void* v_new = nullptr,
                      bool use_scratch = false) {
  if (pd_status st = check_pool(p)) return st;
  if (pd_status st = check_layer(p, layer)) return st;
  if (B < 0 || max_blocks < 1 || max_len < 0) return fail(PD_ERR_ARG, "B < 0, max_blocks < 1 or max_len < 0");
  if (B == 0) return PD_OK;
  const int32_t n_kv = p->desc.n_kv_heads;
  if (n_q_heads < 1 || n_q_heads % n_kv)
    return fail(PD_ERR_ARG, "n_q_heads %d not a positive multiple of n_kv_heads %d", n_q_heads, n_kv);
  const int32_t group = n_q_heads / n_kv;
  if (use_scratch) {
    if (workspace) return fail(PD_ERR_ARG, "the no-alloc call takes no workspace");
    const ScratchSlot* slot = p->device >= 0 && p->device < kMaxDevices ? &g_scratch[p->device] : nullptr;
    if (!slot || !slot->resolved) return fail(PD_ERR_HIP, "no scratch address for device %d", p->device);
    if (slot->status != hipSuccess) return hip_fail(slot->status, "hipGetSymbolAddress(scratch)");
    workspace = slot->ptr;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!q || !block_table || !lens || !out || !workspace) return fail(PD_ERR_ARG, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PD_ERR_ARG, "q and out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PD_ERR_ARG, "workspace not 256-byte aligned");
  if (!(scale == scale) || std::isinf(scale)) return fail(PD_ERR_ARG, "scale is not finite");
  // the split plan must not depend on data only the device knows
  const int64_t cap_len = static_cast<int64_t>(max_blocks) * p->desc.block_size;
  const int32_t plan_len = static_cast<int32_t>(max_len < cap_len ? max_len : cap_len);
  if (static_cast<int64_t>(plan_len) > max_decode_len(p->desc.block_size))
    return fail(PD_ERR_UNSUPPORTED, "max_len %d beyond %lld", plan_len,
                static_cast<long long>(max_decode_len(p->desc.block_size)));
  DecodePlan plan;
  if (!make_decode_plan(p, B, group, plan_len, &plan))
    return fail(PD_ERR_UNSUPPORTED, "no decode kernel for format %d, head_dim %d, group %d",
                p->desc.format, p->desc.head_dim, group);
  if (pd_status st = check_decode_size(B, n_q_heads, plan)) return st;
  const size_t need = decode_workspace_bytes(B, n_q_heads, p->desc.head_dim, plan.split);
  if (use_scratch && need > workspace_bytes)
    return fail(PD_ERR_CAPACITY,
                "this call needs %zu bytes of partials; the no-alloc scratch holds %zu "
                "(use pd_paged_decode with a workspace)", need, workspace_bytes);
  if (workspace_bytes < need)
    return fail(PD_ERR_CAPACITY, "workspace %zu bytes, %zu needed", workspace_bytes, need);
  if (k_new || v_new) {
    if (!k_new || !v_new) return fail(PD_ERR_ARG, "k_new and v_new go together");
    if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
      return fail(PD_ERR_ARG, "k_new and v_new must be 16-byte aligned");
    if (plan.kind != 1 && plan.kind != 2)
      return fail(PD_ERR_UNSUPPORTED,
                  "the fused append runs in the 16-bit row kernel and the packed kernel only (format %d, "
                  "head_dim %d, group %d): use pd_write_block, then pd_paged_decode",
                  p->desc.format, p->desc.head_dim, group);
  }
  DecodeArgs a{};
  a.lv = layer_view(p, layer);
  a.B = B;
  a.n_q = n_q_heads;
  a.q = q;
  a.table = block_table;
  a.max_blocks = max_blocks;
  a.lens = lens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.partials = static_cast<float*>(workspace);
  a.ml_offset = decode_ml_offset(B, n_q_heads, p->desc.head_dim, plan.split);
  a.n_split = plan.split.n_split;
  a.blocks_per_split = plan.split.blocks_per_split;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_bits = p->k_bits;
  a.v_bits = p->v_bits;
  a.qgroup = p->qgroup;
  a.signs = p->d_signs;
  a.inv_sqrt_d = p->inv_sqrt_d;
  const bool bf16 = p->desc.format == PD_FMT_BF16;
  const int32_t D = p->desc.head_dim;
  hipError_t e = hipSuccess;
  if (stages & kStageSplit) {
    switch (plan.kind) {
      case 1: e = launch_paged_decode_row(a, bf16, D, group, plan.kpl, stream); break;
      case 2: e = launch_paged_decode_packed_mfma(a, D, group, stream); break;
      default: e = launch_paged_decode_column(a, bf16, D, group, stream); break;
    }
  }
  // packed pools produce bf16 outputs
  if (e == hipSuccess && (stages & kStageCombine))
    e = launch_decode_combine(a, bf16 || plan.kind >= 2, D, stream);
  if (e == hipErrorInvalidValue) return fail(PD_ERR_UNSUPPORTED, "no decode kernel for this shape");
  if (e != hipSuccess) return hip_fail(e, "paged_decode launch");
  return PD_OK;
}

pd_status pd_paged_decode(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads, const void* q,
                          const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
                          int32_t max_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return decode_call(p, layer, B, n_q_heads, q, block_table, max_blocks, lens, max_len, scale, out,
                     workspace, workspace_bytes, stream, kStageSplit | kStageCombine);
}

pd_status pd_paged_decode_noalloc(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads,
                                  const void* q, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* lens, int32_t max_len, float scale, void* out,
                                  hipStream_t stream) {
  return decode_call(p, layer, B, n_q_heads, q, block_table, max_blocks, lens, max_len, scale, out,
                     nullptr, 0, stream, kStageSplit | kStageCombine, nullptr, nullptr, true);
}

pd_status pd_paged_decode_append(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads,
                                 const void* q, const void* k_new, const void* v_new,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
                                 int32_t max_len, float scale, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (!k_new || !v_new) return fail(PD_ERR_ARG, "NULL k_new or v_new");
  return decode_call(p, layer, B, n_q_heads, q, block_table, max_blocks, lens, max_len, scale, out,
                     workspace, workspace_bytes, stream, kStageSplit | kStageCombine, k_new, v_new);
}

pd_status pd_paged_decode_split(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads,
                                const void* q, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* lens, int32_t max_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_call(p, layer, B, n_q_heads, q, block_table, max_blocks, lens, max_len, scale, out,
                     workspace, workspace_bytes, stream, kStageSplit);
}

pd_status pd_paged_decode_combine(pd_pool* p, int32_t layer, int32_t B, int32_t n_q_heads,
                                  const void* q, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* lens, int32_t max_len, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_call(p, layer, B, n_q_heads, q, block_table, max_blocks, lens, max_len, scale, out,
                     workspace, workspace_bytes, stream, kStageCombine);
}

namespace {

constexpr int32_t kDenseBlock = 32;  // dense sequences are read as 32-token block rows

pd_status dense_plan(const pd_dense_desc* d, int32_t B, int32_t n_q_heads, int32_t max_len,
                     DecodePlan* plan) {
  if (!d) return fail(PD_ERR_ARG, "desc is NULL");
  if (!is_native(d->format)) return fail(PD_ERR_UNSUPPORTED, "dense decode takes fp16 or bf16");
  if (d->n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % d->n_kv_heads)
    return fail(PD_ERR_ARG, "n_q_heads %d not a positive multiple of n_kv_heads %d", n_q_heads,
                d->n_kv_heads);
  if (B < 0 || max_len < 0) return fail(PD_ERR_ARG, "B < 0 or max_len < 0");
  if (static_cast<int64_t>(max_len) > max_decode_len(kDenseBlock))
    return fail(PD_ERR_UNSUPPORTED, "max_len %d beyond %lld", max_len,
                static_cast<long long>(max_decode_len(kDenseBlock)));
  const int32_t group = n_q_heads / d->n_kv_heads;
  if (!make_decode_plan_for(d->format, d->n_kv_heads, d->head_dim, kDenseBlock, B, group, max_len, 0, plan) ||
      plan->kind != 1)
    return fail(PD_ERR_UNSUPPORTED,
                "dense decode needs the row kernel's shapes (n_kv_heads * head_dim * 2 a multiple of "
                "1024 bytes, head_dim 64/128/256, group 1/2/4/8); got n_kv %d, head_dim %d, group %d",
                d->n_kv_heads, d->head_dim, group);
  if (pd_status st = check_decode_size(B, n_q_heads, *plan)) return st;
  // the kernels form row b * blocks + j (blocks = ceil(max_len / 32)) in 32 bits
  const int64_t blocks = max_len > 0 ? (max_len + kDenseBlock - 1) / kDenseBlock : 1;
  if (static_cast<int64_t>(B) * blocks > INT32_MAX)
    return fail(PD_ERR_ARG, "B %d x %lld blocks beyond 2^31 rows", B, static_cast<long long>(blocks));
  return PD_OK;
}

}  // namespace

pd_status pd_dense_workspace_bytes(const pd_dense_desc* d, int32_t B, int32_t n_q_heads,
                                   int32_t max_len, size_t* bytes) {
  if (!bytes) return fail(PD_ERR_ARG, "bytes is NULL");
  DecodePlan plan;
  if (pd_status st = dense_plan(d, B, n_q_heads, max_len, &plan)) return st;
  *bytes = decode_workspace_bytes(B, n_q_heads, d->head_dim, plan.split);
  return PD_OK;
}

pd_status pd_dense_decode(const pd_dense_desc* d, int32_t B, int32_t n_q_heads, const void* q,
                          const void* const* k_seqs, const void* const* v_seqs, const int32_t* lens,
                          int32_t max_len, float scale, void* out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  DecodePlan plan;
  if (pd_status st = dense_plan(d, B, n_q_heads, max_len, &plan)) return st;
  if (B == 0) return PD_OK;
  if (!q || !k_seqs || !v_seqs || !lens || !out || !workspace) return fail(PD_ERR_ARG, "NULL device pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(PD_ERR_ARG, "q and out must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PD_ERR_ARG, "workspace not 256-byte aligned");
  if (!(scale == scale) || std::isinf(scale)) return fail(PD_ERR_ARG, "scale is not finite");
  const size_t need = decode_workspace_bytes(B, n_q_heads, d->head_dim, plan.split);
  if (workspace_bytes < need)
    return fail(PD_ERR_CAPACITY, "workspace %zu bytes, %zu needed", workspace_bytes, need);
  const int32_t max_blocks = max_len > 0 ? (max_len + kDenseBlock - 1) / kDenseBlock : 1;
  DecodeArgs a{};
  // sequence b is "slab" b whose rows are its consecutive 32-token blocks;
  // with no block table, block j of sequence b is row b * max_blocks + j
  a.lv.k_tab = k_seqs;
  a.lv.v_tab = v_seqs;
  a.lv.slab_blocks = max_blocks;
  a.lv.block_size = kDenseBlock;
  a.lv.n_kv = d->n_kv_heads;
  a.lv.k_rec = a.lv.v_rec = 2 * d->head_dim;
  a.lv.capacity_rows = static_cast<int64_t>(B) * max_blocks;
  a.lv.err = nullptr;
  a.B = B;
  a.n_q = n_q_heads;
  a.q = q;
  a.table = nullptr;
  a.max_blocks = max_blocks;
  a.lens = lens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = out;
  a.partials = static_cast<float*>(workspace);
  a.ml_offset = decode_ml_offset(B, n_q_heads, d->head_dim, plan.split);
  a.n_split = plan.split.n_split;
  a.blocks_per_split = plan.split.blocks_per_split;
  const bool bf16 = d->format == PD_FMT_BF16;
  const int32_t group = n_q_heads / d->n_kv_heads;
  hipError_t e = launch_paged_decode_row(a, bf16, d->head_dim, group, plan.kpl, stream);
  if (e == hipSuccess) e = launch_decode_combine(a, bf16, d->head_dim, stream);
  if (e != hipSuccess) return hip_fail(e, "dense_decode launch");
  return PD_OK;
}

pd_status pd_pool_stats(const pd_pool* p, pd_stats* s) {
  if (pd_status st = check_pool(p)) return st;
  if (!s) return fail(PD_ERR_ARG, "stats is NULL");
  s->n_slabs = p->n_slabs;
  s->slab_append_events = p->append_events;
  s->capacity_rows = p->n_slabs * p->desc.slab_blocks;
  s->bytes_reserved = static_cast<int64_t>(p->desc.n_layers) * p->n_slabs *
                      static_cast<int64_t>(p->k_slab_bytes + p->v_slab_bytes);
  s->bytes_copied_on_growth = 0;
  s->k_slab_bytes = static_cast<int64_t>(p->k_slab_bytes);
  s->v_slab_bytes = static_cast<int64_t>(p->v_slab_bytes);
  s->k_record_bytes = p->k_rec;
  s->v_record_bytes = p->v_rec;
  return PD_OK;
}

pd_status pd_pool_check_error(pd_pool* p, hipStream_t stream, int32_t* device_error) {
  if (pd_status st = check_pool(p)) return st;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, p->d_err, sizeof v, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e == hipSuccess && v) e = hipMemsetAsync(p->d_err, 0, sizeof v, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "check_error");
  if (device_error) *device_error = v;
  if (v) return fail(PD_ERR_DEVICE, "device error bits 0x%x", v);
  return PD_OK;
}

}  // extern "C"
