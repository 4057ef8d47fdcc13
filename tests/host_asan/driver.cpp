// Host-side bookkeeping of the pool under AddressSanitizer and
// UndefinedBehaviorSanitizer: pool.hip built with the host compiler against
// the stand-in runtime of stub/hip, with every kernel launch replaced by a
// host function that does the launch's table writes and zero fills on host
// memory.  Checks growth (slab append, reserve over several launches), the
// roll-back of a failed append, the host table mirror against the device
// tables, argument errors, storage identities and leaks (LeakSanitizer at
// exit).  Prints "host bookkeeping ok" and returns 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "internal.h"
#include "pagedkv.h"

using namespace pagedkv;

// ---- stand-in runtime ---------------------------------------------------------
static int g_fail_host_malloc = 0;   // fail the next hipHostMalloc
static int g_launch_fail_at = -1;    // fail the append launch with this index
static int g_append_launches = 0;
static int g_other_launches = 0;
static int g_dup_launches = 0;       // duplicate-write check launches (mark, clear)
static void** g_tables = nullptr;    // the device tables the last append wrote

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stand-in error"; }
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMalloc(void** p, size_t n) { *p = std::aligned_alloc(256, (n + 255) / 256 * 256); return *p ? hipSuccess : hipErrorOutOfMemory; }
hipError_t hipFree(void* p) { std::free(p); return hipSuccess; }
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) {
  if (g_fail_host_malloc) { g_fail_host_malloc = 0; *p = nullptr; return hipErrorOutOfMemory; }
  *p = std::malloc(n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* p) { std::free(p); return hipSuccess; }
hipError_t hipMemset(void* d, int v, size_t n) { std::memset(d, v, n); return hipSuccess; }
hipError_t hipMemsetAsync(void* d, int v, size_t n, hipStream_t) { std::memset(d, v, n); return hipSuccess; }
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) { std::memcpy(d, s, n); return hipSuccess; }
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) { std::memcpy(d, s, n); return hipSuccess; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) { *p = const_cast<void*>(sym); return hipSuccess; }

// ---- launches -------------------------------------------------------------------
namespace pagedkv {
hipError_t launch_append_slabs(const AppendArgs& a, hipStream_t) {
  const int idx = g_append_launches++;
  if (idx == g_launch_fail_at) return hipErrorLaunchFailure;
  if (a.n_pairs < 1 || a.n_pairs > kAppendMaxPairs) return hipErrorInvalidValue;
  g_tables = a.tables;
  for (int j = 0; j < a.n_pairs; ++j) {
    a.tables[a.entry[j]] = a.k_mem[j];
    a.tables[a.entry[j] + a.max_slabs] = a.v_mem[j];
    std::memset(a.k_mem[j], 0, static_cast<size_t>(a.k_bytes));
    std::memset(a.v_mem[j], 0, static_cast<size_t>(a.v_bytes));
  }
  return hipSuccess;
}
hipError_t launch_write_block(const WriteArgs&, int32_t, hipStream_t) { ++g_other_launches; return hipSuccess; }
// the duplicate-write check on host memory: rows and slots are host arrays here
hipError_t launch_dup_check(const DupArgs& a, bool mark, hipStream_t) {
  ++g_dup_launches;
  for (int i = 0; i < a.n; ++i) {
    const int32_t row = a.rows[i], slot = a.slots[i];
    if (row < 0 || row >= a.capacity_rows || slot < 0 || slot >= a.block_size) continue;
    const uint64_t bit = static_cast<uint64_t>(row) * a.block_size + slot;
    if (mark) {
      const uint32_t m = 1u << (bit & 31);
      if (a.bits[bit >> 5] & m) *a.err |= PD_DEVERR_DUPLICATE;
      a.bits[bit >> 5] |= m;
    } else {
      a.bits[bit >> 5] = 0u;
    }
  }
  return hipSuccess;
}
hipError_t launch_row_move(const RowMoveArgs&, int, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_gather(const GatherArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_split_runs(const RunArgs&, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_paged_decode_column(const DecodeArgs&, bool, int32_t, int32_t, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_paged_decode_row(const DecodeArgs&, bool, int32_t, int32_t, int, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_decode_combine(const DecodeArgs&, bool, int32_t, hipStream_t) { ++g_other_launches; return hipSuccess; }
hipError_t launch_paged_decode_packed_mfma(const DecodeArgs&, int32_t, int32_t, hipStream_t) { ++g_other_launches; return hipSuccess; }
bool packed_mfma_supported(int32_t n_kv, int32_t head_dim, int32_t group, int32_t bs, int32_t qgroup) {
  return n_kv == 8 && bs == 32 && (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4) && (qgroup == 32 || (qgroup == 64 && head_dim >= 128));
}
int packed_mfma_target_workgroups(int32_t head_dim) { return head_dim <= 64 ? 512 : 256; }
int row_kernel_kpl(int32_t n_kv, int32_t head_dim, int32_t, int32_t bs) {
  return (bs == 32 && (n_kv * head_dim * 2) % 1024 == 0) ? 1 : 0;
}
int row_kernel_heads_per_workgroup(int32_t head_dim, int hgw) { return (64 / (head_dim / 8)) * hgw; }
}  // namespace pagedkv

// ---- checks ---------------------------------------------------------------------
static int g_failures = 0;
#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #c, pd_last_error()); \
      ++g_failures;                                                         \
    }                                                                       \
  } while (0)

struct Mem {
  std::vector<void*> blocks;
  void* get(size_t n, unsigned char fill) {
    void* p = std::aligned_alloc(256, (n + 255) / 256 * 256);
    std::memset(p, fill, n);
    blocks.push_back(p);
    return p;
  }
  ~Mem() { for (void* p : blocks) std::free(p); }
};

static pd_pool_desc desc(int L, int S, int max_slabs, int fmt = PD_FMT_BF16) {
  pd_pool_desc d{};
  d.n_layers = L; d.block_size = 32; d.n_kv_heads = 8; d.head_dim = 128;
  d.slab_blocks = S; d.max_slabs = max_slabs; d.format = fmt;
  return d;
}

static bool all_zero(const void* p, size_t n) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) if (c[i]) return false;
  return true;
}

// the device tables written by the appends equal the host mirror for every slab
static void check_tables(pd_pool* p, int L, int S, int ms) {
  pd_stats st{};
  CHECK(pd_pool_stats(p, &st) == PD_OK);
  for (int l = 0; l < L; ++l)
    for (int64_t s = 0; s < st.n_slabs; ++s) {
      void *kb = nullptr, *vb = nullptr;
      int32_t r = -1;
      CHECK(pd_slab_for_row(p, l, s * S + (S - 1), &kb, &vb, &r) == PD_OK);
      CHECK(r == S - 1);
      CHECK(g_tables && g_tables[static_cast<size_t>(l) * 2 * ms + s] == kb);
      CHECK(g_tables && g_tables[static_cast<size_t>(l) * 2 * ms + ms + s] == vb);
    }
}

int main() {
  Mem mem;
  // growth: one slab, then three in one reserve over 40 layers (two launches)
  {
    const int L = 40, S = 4, ms = 8;
    pd_pool_desc d = desc(L, S, ms);
    pd_pool* p = nullptr;
    CHECK(pd_pool_create(&d, &p) == PD_OK && p);
    size_t kb = 0, vb = 0;
    CHECK(pd_slab_bytes(p, &kb, &vb) == PD_OK && kb == 4u * 32 * 8 * 256 && vb == kb);
    std::vector<void*> k(L), v(L);
    for (int l = 0; l < L; ++l) { k[l] = mem.get(kb, 0xAB); v[l] = mem.get(vb, 0xCD); }
    int32_t idx = -1;
    const int before = g_append_launches;
    CHECK(pd_append_slab(p, k.data(), v.data(), nullptr, &idx) == PD_OK && idx == 0);
    CHECK(g_append_launches - before == 1);  // 40 pairs: one launch
    for (int l = 0; l < L; ++l) CHECK(all_zero(k[l], kb) && all_zero(v[l], vb));
    int32_t need = 0;
    CHECK(pd_slabs_needed(p, 4 * S, &need) == PD_OK && need == 3);
    std::vector<void*> k3(3 * L), v3(3 * L);
    for (int i = 0; i < 3 * L; ++i) { k3[i] = mem.get(kb, 0x11); v3[i] = mem.get(vb, 0x22); }
    int32_t got = 0;
    const int b2 = g_append_launches;
    CHECK(pd_reserve_rows(p, 4 * S, k3.data(), v3.data(), 3, nullptr, &got) == PD_OK && got == 3);
    CHECK(g_append_launches - b2 == 2);      // 120 pairs: two launches of at most 96
    pd_stats st{};
    CHECK(pd_pool_stats(p, &st) == PD_OK);
    CHECK(st.n_slabs == 4 && st.slab_append_events == 4 && st.capacity_rows == 16);
    CHECK(st.bytes_reserved == static_cast<int64_t>(L) * 4 * static_cast<int64_t>(kb + vb));
    CHECK(st.bytes_copied_on_growth == 0);
    check_tables(p, L, S, ms);

    // a launch that fails part-way through an append records nothing
    std::vector<void*> k2(3 * L), v2(3 * L);
    for (int i = 0; i < 3 * L; ++i) { k2[i] = mem.get(kb, 0x33); v2[i] = mem.get(vb, 0x44); }
    g_launch_fail_at = g_append_launches + 1;  // the second of two launches (120 pairs)
    CHECK(pd_reserve_rows(p, 7 * S, k2.data(), v2.data(), 3, nullptr, &got) == PD_ERR_HIP);
    CHECK(g_launch_fail_at == g_append_launches - 1);
    g_launch_fail_at = -1;
    pd_stats st2{};
    CHECK(pd_pool_stats(p, &st2) == PD_OK && st2.n_slabs == 4 && st2.slab_append_events == 4);
    void *kx = nullptr, *vx = nullptr;
    int32_t rx = 0;
    CHECK(pd_slab_for_row(p, 0, 4 * S, &kx, &vx, &rx) == PD_ERR_RANGE);
    // argument errors change nothing either: NULL, misaligned, too many slabs
    std::vector<void*> kbad(k2.begin(), k2.begin() + L), vbad(v2.begin(), v2.begin() + L);
    kbad[7] = nullptr;
    CHECK(pd_append_slab(p, kbad.data(), vbad.data(), nullptr, &idx) == PD_ERR_ARG);
    kbad[7] = static_cast<char*>(k2[7]) + 16;
    CHECK(pd_append_slab(p, kbad.data(), vbad.data(), nullptr, &idx) == PD_ERR_ARG);
    CHECK(pd_reserve_rows(p, 7 * S, k2.data(), v2.data(), 2, nullptr, &got) == PD_ERR_ARG);          // needs 3
    CHECK(pd_reserve_rows(p, 100 * S, k2.data(), v2.data(), 96, nullptr, &got) == PD_ERR_CAPACITY);
    CHECK(pd_pool_stats(p, &st2) == PD_OK && st2.n_slabs == 4);
    // the same memory appends cleanly afterwards, at the same slab indices
    CHECK(pd_reserve_rows(p, 7 * S, k2.data(), v2.data(), 3, nullptr, &got) == PD_OK && got == 3);
    CHECK(pd_pool_stats(p, &st2) == PD_OK && st2.n_slabs == 7 && st2.slab_append_events == 7);
    for (int i = 0; i < 3 * L; ++i) CHECK(all_zero(k2[i], kb) && all_zero(v2[i], vb));
    check_tables(p, L, S, ms);
    std::vector<void*> k1(2 * L), v1(2 * L);
    for (int i = 0; i < 2 * L; ++i) { k1[i] = mem.get(kb, 0); v1[i] = mem.get(vb, 0); }
    CHECK(pd_reserve_rows(p, 9 * S, k1.data(), v1.data(), 2, nullptr, &got) == PD_ERR_CAPACITY);  // max_slabs 8
    CHECK(pd_slab_for_row(p, L, 0, &kx, &vx, &rx) == PD_ERR_RANGE);                     // no such layer

    // calls that fail validation launch nothing
    const int o = g_other_launches;
    int32_t* dev_i32 = static_cast<int32_t*>(mem.get(4096, 0));
    void* dev = mem.get(1 << 20, 0);
    CHECK(pd_write_block(p, 0, -1, dev_i32, dev_i32, dev, dev, nullptr) == PD_ERR_ARG);
    CHECK(pd_write_block(p, 0, 2, dev_i32, dev_i32, static_cast<char*>(dev) + 2, dev, nullptr) == PD_ERR_ARG);
    CHECK(pd_gather_visible(p, 0, 1, dev_i32, 0, dev_i32, 8, dev, dev, nullptr, nullptr) == PD_ERR_ARG);
    size_t ws = 0;
    CHECK(pd_decode_workspace_bytes(p, 2, 16, 100, &ws) == PD_OK && ws > 0);
    CHECK(pd_paged_decode(p, 0, 2, 12, dev, dev_i32, 4, dev_i32, 100, 0.1f, dev, dev, ws, nullptr) == PD_ERR_ARG);
    CHECK(pd_paged_decode(p, 0, 2, 16, dev, dev_i32, 4, dev_i32, 100, 0.1f, dev, dev, ws - 4, nullptr) ==
          PD_ERR_CAPACITY);
    CHECK(pd_paged_decode_noalloc(p, 0, 2, 16, dev, dev_i32, 1 << 20, dev_i32, 1 << 24, 0.1f, dev, nullptr) ==
          PD_ERR_UNSUPPORTED);
    CHECK(pd_paged_decode_noalloc(p, 0, 256, 32, dev, dev_i32, 512, dev_i32, 16384, 0.1f, dev, nullptr) ==
          PD_ERR_CAPACITY && std::strstr(pd_last_error(), "scratch"));
    CHECK(g_other_launches == o);
    CHECK(pd_paged_decode(p, 0, 2, 16, dev, dev_i32, 4, dev_i32, 100, 0.1f, dev, dev, ws, nullptr) == PD_OK);
    CHECK(pd_paged_decode_noalloc(p, 0, 2, 16, dev, dev_i32, 4, dev_i32, 100, 0.1f, dev, nullptr) == PD_OK);
    CHECK(g_other_launches == o + 4);  // split + combine, twice
    CHECK(pd_pool_destroy(p) == PD_OK);
  }
  // storage identities of a packed pool; a mismatch names its field
  {
    int8_t signs[128];
    for (int i = 0; i < 128; ++i) signs[i] = (i * 7 % 3) ? 1 : -1;
    pd_pool_desc d = desc(2, 4, 3, PD_FMT_K4V4);
    d.hadamard_signs = signs;
    d.group_size = 64;
    pd_pool* p = nullptr;
    CHECK(pd_pool_create(&d, &p) == PD_OK);
    pd_storage_identity id{};
    CHECK(pd_storage_identity_of(p, &id) == PD_OK && id.group_size == 64 && id.k_record_bytes == 64 + 16);
    CHECK(pd_identity_check(p, &id) == PD_OK);
    pd_storage_identity other = id;
    other.signs_hash ^= 1;
    CHECK(pd_identity_check(p, &other) == PD_ERR_IDENTITY && std::strstr(pd_last_error(), "signs_hash"));
    CHECK(pd_import_blocks(p, &other, 1, nullptr, nullptr, 0, nullptr) == PD_ERR_IDENTITY);
    d.n_kv_heads = 4;  // the packed decode kernel takes 8 kv heads
    pd_pool* q = nullptr;
    CHECK(pd_pool_create(&d, &q) == PD_ERR_UNSUPPORTED && q == nullptr);
    CHECK(pd_pool_destroy(p) == PD_OK);
  }
  // the duplicate-write check: off by default; on, a call with two tokens on
  // one (row, slot) flags the error word, the bitmap is all zero after each
  // call (no false report on the next), and destroy frees it
  {
    pd_pool_desc d = desc(1, 4, 3);
    pd_pool* p = nullptr;
    CHECK(pd_pool_create(&d, &p) == PD_OK);
    size_t kb = 0, vb = 0;
    CHECK(pd_slab_bytes(p, &kb, &vb) == PD_OK);
    void* k[1] = {mem.get(kb, 0)};
    void* v[1] = {mem.get(vb, 0)};
    int32_t idx = -1;
    CHECK(pd_append_slab(p, k, v, nullptr, &idx) == PD_OK && idx == 0);  // rows 0 .. 3
    int32_t rows[3] = {0, 1, 0}, slots[3] = {5, 5, 5}, good_slots[3] = {5, 5, 6};
    static char src[3 * 4096] __attribute__((aligned(16)));
    const int l0 = g_dup_launches;
    CHECK(pd_pool_set_debug(p, 0x80u) == PD_ERR_ARG);
    CHECK(pd_write_block(p, 0, 3, rows, slots, src, src, nullptr) == PD_OK);
    CHECK(g_dup_launches == l0);                 // off: no check
    CHECK(pd_pool_set_debug(p, PD_DEBUG_DUPLICATE_WRITES) == PD_OK);
    CHECK(pd_write_block(p, 0, 3, rows, slots, src, src, nullptr) == PD_OK);
    CHECK(g_dup_launches == l0 + 2);             // mark before the write, clear after
    int32_t err = 0;
    CHECK(pd_pool_check_error(p, nullptr, &err) == PD_ERR_DEVICE && (err & PD_DEVERR_DUPLICATE));
    CHECK(pd_write_block(p, 0, 3, rows, good_slots, src, src, nullptr) == PD_OK);
    CHECK(pd_pool_check_error(p, nullptr, &err) == PD_OK && err == 0);
    CHECK(pd_pool_set_debug(p, 0) == PD_OK);
    CHECK(pd_write_block(p, 0, 3, rows, slots, src, src, nullptr) == PD_OK);
    CHECK(g_dup_launches == l0 + 4);
    CHECK(pd_pool_destroy(p) == PD_OK);
  }
  // a failed host allocation inside create leaves nothing behind
  {
    pd_pool_desc d = desc(2, 4, 3);
    pd_pool* p = reinterpret_cast<pd_pool*>(0x1);
    g_fail_host_malloc = 1;
    CHECK(pd_pool_create(&d, &p) == PD_ERR_HIP && p == nullptr);
  }
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("host bookkeeping ok\n");
  return 0;
}
