// paged_decode for packed pools (K8/V8, K8/V4, K4/V4) on the gfx950 matrix
// cores.
//
// Operation (mlx-swift-lm PR #142, "Add packed paged KV formats with bounded
// workspace admission", section "Summary" and the "After" flowchart): direct
// attention over the packed pages.  Keys were rotated by a fixed signed
// Hadamard basis before they were quantised, so the query gets the same
// rotation (q'.k' = q.k); values are stored unrotated.  A token-head record is
// its codes (8-bit bytes, or 4-bit nibbles with value 2i in the low nibble of
// byte i) followed by one (fp32 scale, fp32 offset) per group of GS = 32 or
// 64 values; a value is code * scale + offset.  Per group g of a key,
//   q'.k = scale_g * sum_{i in g} q'_i c_i + offset_g * sum_{i in g} q'_i,
// and per group of a value
//   sum_t p_t v_t = sum_t (p_t scale_t) c_t + sum_t p_t offset_t.
// The code sums are matrix products with small integer operands, which the
// MFMA units take exactly in f16; q' and p * scale go in as f16 and the
// products accumulate in fp32.
//
// Range and precision of the f16 operands.  q' goes in as two f16 parts (hi =
// f16(y), lo = f16(y - hi): about 22 bits of y), in two rows of the A operand
// that the single-token query leaves free, so the scores carry close to fp32
// precision at no extra product.  Before the split, each query head is scaled
// by a power of two 2^kq (kq <= 0) that keeps its largest |q'| below 2^14;
// the scores are scaled back exactly.  p * scale goes in as f16 times a
// power of two 2^vk per value group and wave: vk starts at 10 and is lowered
// (the accumulator of the group rescaled by the exact ratio) whenever a step
// holds a group scale with p * scale * 2^vk possibly above 2^15 (p <= 1), so
// no operand overflows f16 for any finite record.
//
// Decomposition.  A workgroup owns (sequence, split of the token axis) and
// all 8 kv heads, one wave per kv head; split s takes logical blocks s, s +
// n_split, ...  Whole token rows of a block (every head, K and V) are staged
// in LDS with 16-byte coalesced loads, the next stage's loads in flight in
// registers while the current one is computed.  A wave works through its
// head's tokens in steps of up to 32 (two 16-token sub-tiles whose score
// products are issued together, then one online-softmax update):
//   scores: one 16x16x32 product per 32-value k-block (the k-blocks of one
//     group chain their products), A = q' (query head j in row 4j, other
//     rows zero), B = the 16 tokens' codes of the k-block;
//     the score of (query head j, token n) lands in lane n + 16 j, so the
//     online softmax runs on every lane and its reductions over tokens are
//     16-lane DPP row operations;
//   values: p * scale * 2^vk goes through a small per-wave LDS area into
//     the A operand of 4x4x4 products (16 independent blocks per
//     instruction: 4 query heads x 4 tokens times 4 tokens x 4 dimensions),
//     so a lane accumulates value dimensions of every query head in the four
//     registers of each accumulator; the B operand is one code byte column
//     of 4 tokens, which LDS transpose loads (ds_read_b64_tr_b8) deliver 8
//     tokens at a time (4-bit codes: one byte feeds the two dimensions of
//     its nibbles); the offsets add sum_t p_t offset_t per group.
// Codes become f16 exactly.  Key codes: a byte placed under the exponent
// bits 0x64 is 1024 + byte; the products take these biased codes as they are
// and the first accumulator of each group's chain starts at -1024 * sum(q').
// Value codes: a byte zero-extended to 16 bits is the f16 subnormal byte *
// 2^-24 (the matrix cores take subnormal f16 operands), so no bias is added
// or taken off, and 2^24 is applied once at the end; the value sums run over
// the whole split, where a bias would cancel at a cost in accuracy.  A 4-bit
// key's high nibble is taken in place, as 16 * code, and scaled back by an
// exact power of two in q'.  A 4-bit value byte enters whole (lo + 16 hi)
// for its high nibble and masked (lo) for its low one; the low nibble's sum
// is taken off the high one's at the end.
// Partials go to the same workspace layout as the 16-bit kernels and the same
// combine kernel merges them.
#include "device_common.h"
#include "internal.h"
#include "pack_vector.h"

namespace pagedkv {

namespace {

#ifndef PAGEDKV_PMFMA_STAGE_KIB
#define PAGEDKV_PMFMA_STAGE_KIB 48
#endif
#ifndef PAGEDKV_PMFMA_TARGET_WG_SMALL
#define PAGEDKV_PMFMA_TARGET_WG_SMALL 512
#endif
#ifndef PAGEDKV_PMFMA_TARGET_WG
#define PAGEDKV_PMFMA_TARGET_WG 256
#endif
// Tokens per online-softmax step: 16-token sub-tiles of one stage whose score
// products are issued together and whose softmax update is one step (capped
// by the tokens of a stage).
#ifndef PAGEDKV_PMFMA_STEP_TOKENS
#define PAGEDKV_PMFMA_STEP_TOKENS 32
#endif
// The value products of one transpose load are scheduled together (a
// scheduling barrier after each load's products) from this many loads per
// 16 tokens up.
#ifndef PAGEDKV_PMFMA_TR_BARRIER_NRD
#define PAGEDKV_PMFMA_TR_BARRIER_NRD 4
#endif

constexpr int kPWaves = 8;  // one wave per kv head; packed pools have 8
constexpr int kPThreads = kPWaves * kWave;
constexpr int kPBS = 32;    // tokens per block
constexpr int kPLdsSlabs = kPThreads;  // slab pointers staged in LDS
constexpr int kSub = 16;    // tokens per MFMA sub-tile

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

template <int D, int KB, int VB, int GS>
struct PShape {
  static constexpr int NKB = D / 32;   // 32-value k-blocks of the score products
  static constexpr int NMG = D / GS;   // (scale, offset) groups of a record
  static constexpr int KPG = GS / 32;  // k-blocks per group
  static constexpr int KCODE = D * KB / 8, VCODE = D * VB / 8;
  static constexpr int KREC = KCODE + NMG * 8, VREC = VCODE + NMG * 8;
  static constexpr int KROW = 8 * KREC, VROW = 8 * VREC;  // one token, every head
  // LDS pitch of a staged token row: 16 bytes of padding spread the rows of
  // consecutive tokens over the banks
  static constexpr int PK = KROW + 16, PV = VROW + 16;
  // tokens per stage (inside one block): 32 while a stage is at most
  // PAGEDKV_PMFMA_STAGE_KIB
  static constexpr int T = (KROW + VROW) * kPBS <= PAGEDKV_PMFMA_STAGE_KIB * 1024 ? 32 : 16;
  static constexpr int KU = T * KROW / 16, VU = T * VROW / 16;  // 16-byte units
  static constexpr int UPT = (KU + VU + kPThreads - 1) / kPThreads;
  static constexpr int STAGE = T * (PK + PV);
  // 16-token sub-tiles per softmax step, and the step's tokens
  static constexpr int NSUB = (PAGEDKV_PMFMA_STEP_TOKENS < T ? PAGEDKV_PMFMA_STEP_TOKENS : T) / 16;
  static constexpr int STEP = NSUB * 16;
  static_assert(KREC % 16 == 0 && VREC % 16 == 0, "records are whole 16-byte units");
};

// Waves per SIMD the launch asks for: two workgroups per CU where the
// registers allow it.
template <int D>
constexpr int kPMinWaves = D <= 64 ? 4 : 2;

__device__ __forceinline__ const char* lane_ptr(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), j);
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Two bytes of w (selected by SEL) as the f16 pair (1024 + byte): each byte
// is placed under the exponent bits 0x64.
__device__ __forceinline__ uint32_t bytes_biased(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_perm(0x64646464u, w, sel);
}
constexpr uint32_t kSelB01 = 0x04010400u;  // bytes 0, 1 -> (lo, hi) halves
constexpr uint32_t kSelB23 = 0x04030402u;  // bytes 2, 3

// Two bytes of w (selected by SEL) zero-extended to 16 bits: the f16
// subnormals byte * 2^-24
__device__ __forceinline__ uint32_t bytes_subnormal(uint32_t w, uint32_t sel) {
  return __builtin_amdgcn_perm(0u, w, sel);
}

// B operand of a score product: 8 codes of one token and group as biased
// f16, in the element order the A operand (q') uses.  8-bit codes: 1024 +
// value e of the k-block; 4-bit codes: 1024 + values 0, 2, 4, 6 (low
// nibbles), then 1024 + 16 * values 1, 3, 5, 7 (high nibbles in place).
// The code bytes of one token and k-block (8 bytes, or 4 for 4-bit codes)
template <int KB>
__device__ __forceinline__ uint2 key_load(const unsigned char* p) {
  if constexpr (KB == 8) return *reinterpret_cast<const uint2*>(p);
  else return make_uint2(*reinterpret_cast<const uint32_t*>(p), 0u);
}
template <int KB>
__device__ __forceinline__ h8 key_unpack(uint2 w) {
  uint32_t r[4];
  if constexpr (KB == 8) {
    r[0] = bytes_biased(w.x, kSelB01);
    r[1] = bytes_biased(w.x, kSelB23);
    r[2] = bytes_biased(w.y, kSelB01);
    r[3] = bytes_biased(w.y, kSelB23);
  } else {
    const uint32_t lo = w.x & 0x0f0f0f0fu, hi = w.x & 0xf0f0f0f0u;
    r[0] = bytes_biased(lo, kSelB01);
    r[1] = bytes_biased(lo, kSelB23);
    r[2] = bytes_biased(hi, kSelB01);
    r[3] = bytes_biased(hi, kSelB23);
  }
  return __builtin_bit_cast(h8, r);
}
template <int KB>
__device__ __forceinline__ h8 key_codes(const unsigned char* p) {
  return key_unpack<KB>(key_load<KB>(p));
}

template <int KB>
__device__ __forceinline__ int key_value_index(int e) {  // value of element e in its k-block
  if constexpr (KB == 8) return e;
  else return e < 4 ? 2 * e : 2 * (e - 4) + 1;
}
// q' factor of value v of a group (4-bit high nibbles enter as 16 * code)
template <int KB>
__device__ __forceinline__ float key_q_factor(int v) {
  return (KB == 4 && (v & 1)) ? 0.0625f : 1.f;
}

// The value code bytes are read with LDS transpose loads (ds_read_b64_tr_b8):
// within each 16-lane group, lane i receives byte column i % 8 of the 8 rows
// named by lanes 2m + (i % 16) / 8, m = 0..7.  With lanes naming tokens as
// below, one load gives lane l byte column tr_col(l) (of 32) of 8 consecutive
// tokens, and lanes l and l + 8 of a group hold the two halves of 16 tokens
// (their sums are added at the end).  A value takes D * VB / 256 such loads
// per 16 tokens (32 code bytes each) and D / 32 accumulators per lane.
__device__ __forceinline__ int tr_col(int lane) { return 8 * (lane / 16) + lane % 8; }
__device__ __forceinline__ int tr_token(int lane) { return (lane % 16) / 2 + 8 * (lane % 2); }
// Value dimension that accumulator i of lane l holds: 8-bit codes, byte
// tr_col(l) of load i, dimension 32 i + tr_col(l); 4-bit codes, nibble i % 2
// of byte tr_col(l) of load i / 2, dimension 64 (i / 2) + 2 tr_col(l) + i % 2.
template <int VB>
__device__ __forceinline__ int vdim(int i, int lane) {
  return VB == 8 ? 32 * i + tr_col(lane) : 64 * (i / 2) + 2 * tr_col(lane) + i % 2;
}
// Scale that brings accumulator i of lane l, times 2^24 (the subnormal
// codes), back to sum_t p_t s_t c_t: the prescale 2^vk of p * scale, and 16
// more for a 4-bit high nibble taken in place (exact powers of two).
template <int VB>
__device__ __forceinline__ float vacc_scale(int i, int vk) {
  const bool high = VB == 4 && (i % 2) == 1;
  return __builtin_bit_cast(float, static_cast<uint32_t>(127 - vk - (high ? 4 : 0)) << 23);
}
constexpr float kSubnormalUnit = 16777216.f;  // 2^24: a subnormal code's unit back to 1

typedef int v2i __attribute__((ext_vector_type(2)));
// 8 bytes per lane from LDS, transposed across each 16-lane group as above
__device__ __forceinline__ uint2 lds_read_tr8(const unsigned char* p) {
  const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
  return make_uint2(static_cast<uint32_t>(r.x), static_cast<uint32_t>(r.y));
}

// 2^k as an fp32 (k in [-126, 128]; 128 gives inf)
__device__ __forceinline__ float exp2i(int k) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(127 + k) << 23);
}
// floor(log2(x)) of a normal positive fp32
__device__ __forceinline__ int exponent_of(float x) {
  return static_cast<int>((__builtin_bit_cast(uint32_t, x) >> 23) & 0xffu) - 127;
}
// f16 high and low parts of y: hi = f16(y), lo = f16(y - hi) (y - hi is exact)
__device__ __forceinline__ void split_f16(float y, _Float16& hi, _Float16& lo) {
  hi = static_cast<_Float16>(y);
  lo = static_cast<_Float16>(y - static_cast<float>(hi));
}
// Exponent kq <= 0 of the power-of-two prescale of a query head whose largest
// |q' * qs| is mq: 0 while mq < 2^14, else the one that brings it below 2^14.
__device__ __forceinline__ int query_prescale(float mq) {
  return mq < 16384.f ? 0 : 13 - exponent_of(mq);
}
constexpr int kVk0 = 10;  // first value prescale exponent: p * scale * 1024

__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

template <int D, int KB, int VB, int G, int GS>
__global__ __launch_bounds__(kPThreads, kPMinWaves<D>) void paged_decode_packed_mfma_kernel(DecodeArgs a) {
  using S = PShape<D, KB, VB, GS>;
  constexpr int NKB = S::NKB, NMG = S::NMG, KPG = S::KPG, T = S::T, PK = S::PK, PV = S::PV;
  constexpr int NSUB = S::NSUB, STEP = S::STEP;
  constexpr int KREC = S::KREC, VREC = S::VREC, KROW = S::KROW, VROW = S::VROW;
  constexpr int NACC = D / 32;      // value accumulators per lane
  constexpr int NRD = D * VB / 256;  // transpose loads per 16 tokens of a value
  // floats per wave: the q' transform, then p^T as f16 [group][4][STEP]
  constexpr int AUX = (G * D > NMG * 2 * STEP) ? G * D : NMG * 2 * STEP;
  static_assert(G <= 4, "query heads of a kv head take rows 0, 4, 8, 12");

  __shared__ __attribute__((aligned(16))) unsigned char s_stage[S::STAGE];
  __shared__ __attribute__((aligned(16))) float s_aux[kPWaves][AUX];  // q' transform, then p^T
  __shared__ float s_qs[kPWaves][G * NMG];  // sum of q' per (query head, group)
  __shared__ float s_kb[kPWaves][G * NMG];  // 1024 * sum of the f16 A operand, likewise
  __shared__ int s_qk[kPWaves][4];          // query prescale exponent per query head
  __shared__ uint64_t s_kt[kPLdsSlabs];    // slab base pointers of the layer
  __shared__ uint64_t s_vt[kPLdsSlabs];

  const int lane = threadIdx.x % kWave;
  const int h = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // kv head of this wave
  const int n = lane % kSub;   // token (scores), dimension (values), row (A operands)
  const int J = lane / kSub;   // query head of the score layout; k-block of the operands

  const LayerView& lv = a.lv;
  const int n_split = a.n_split;
  const int w = xcd_work_id(blockIdx.x, gridDim.x);
  if (w >= a.B * n_split) return;
  const int s = w % n_split;
  const int b = w / n_split;
  const int32_t* trow = a.table + static_cast<size_t>(b) * a.max_blocks;

  // Independent loads first: the length, the rows of this split's blocks (one
  // per lane), this wave's query heads and the signs.  A query head vector
  // is held 8 values per lane by QLPT = D/8 lanes (lane c: values 8c ..
  // 8c+7), QVPP vectors per pass of the wave; pass p, lane l holds query head
  // p QVPP + l / QLPT of the wave's G.
  int len = a.lens[b];
  int row = -1;
  {
    const int blk = s + lane * n_split;
    if (lane < a.blocks_per_split && blk < a.max_blocks) row = trow[blk];
  }
  constexpr int QLPT = D / 8, QVPP = kWave / QLPT, QPASS = (G + QVPP - 1) / QVPP;
  const int qc = lane % QLPT;
  uint4 qraw[QPASS];
  float4 sg0, sg1;  // the signs of values 8 qc .. 8 qc + 7
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(b) * a.n_q + h * G) * D;
#pragma unroll
    for (int p = 0; p < QPASS; ++p) {
      const int j = p * QVPP + lane / QLPT;
      qraw[p] = j < G ? *reinterpret_cast<const uint4*>(q + j * D + 8 * qc) : make_uint4(0, 0, 0, 0);
    }
    const float4* sp4 = reinterpret_cast<const float4*>(a.signs + 8 * qc);
    sg0 = sp4[0];
    sg1 = sp4[1];
  }
  const int cap_len = min(a.max_blocks, n_split * a.blocks_per_split) * kPBS;
  const bool len_ok = len >= 0 && len <= cap_len;
  if (!len_ok) {
    if (threadIdx.x == 0 && s == 0) set_error(lv.err, PD_DEVERR_LENGTH);
    len = len < 0 ? 0 : cap_len;
  }
  const int nb = (len + kPBS - 1) / kPBS;
  if (s >= nb) return;  // inactive split (uniform over the workgroup)
  const int nblk = (nb - s + n_split - 1) / n_split;
  // The layer's slab pointer tables go to LDS while the row reads are in
  // flight, so a block's address costs one dependent global read (its row),
  // not two; slabs past kPLdsSlabs are looked up in global memory.
  {
    const int n_slabs = static_cast<int>(lv.capacity_rows / lv.slab_blocks);
    const int t = threadIdx.x;
    uint64_t kt = 0, vt = 0;
    if (t < n_slabs) {
      kt = reinterpret_cast<uint64_t>(lv.k_tab[t]);
      vt = reinterpret_cast<uint64_t>(lv.v_tab[t]);
    }
    s_kt[t] = kt;
    s_vt[t] = vt;
  }
  __syncthreads();
  const bool row_ok = row >= 0 && row < lv.capacity_rows;
  const uint64_t ok_mask = __ballot(row_ok);
  if (h == 0 && lane < nblk && !row_ok) set_error(lv.err, PD_DEVERR_TABLE_ROW);
  uint64_t kaddr = 0, vaddr = 0;
  if (lv.capacity_rows > 0) {
    const int r = row_ok ? row : 0;  // rows outside the pool read row 0 and are masked
    const int slab = r / lv.slab_blocks;
    const size_t in_slab = static_cast<size_t>(r - slab * lv.slab_blocks);
    const uint64_t kbase = slab < kPLdsSlabs ? s_kt[slab] : reinterpret_cast<uint64_t>(lv.k_tab[slab]);
    const uint64_t vbase = slab < kPLdsSlabs ? s_vt[slab] : reinterpret_cast<uint64_t>(lv.v_tab[slab]);
    kaddr = kbase + in_slab * kPBS * KROW;
    vaddr = vbase + in_slab * kPBS * VROW;
  }
  constexpr int SPB = kPBS / T;  // stages per block
  const int n_stages = lv.capacity_rows > 0 ? nblk * SPB : 0;

  // Fused append (pd_paged_decode_append): token len - 1 of the sequence is
  // new.  The workgroup whose split owns its block -- the only one that reads
  // those bytes -- packs it before the first stage is requested: wave h takes
  // kv head h, its first D/8 lanes the K vector (rotated) and the next D/8
  // the V vector, and stores both records into the token's slot; the stores
  // are waited for and a barrier orders them before the stage loads.  A
  // rejected length or row appends nothing.
  if (a.k_new && len_ok && len > 0) {
    const int p = len - 1;
    const int jb = p / kPBS;
    if (jb % n_split == s) {  // uniform over the workgroup
      constexpr int LPT = D / 8;
      const int jj = jb / n_split;  // this split's jj-th block
      const bool row_live = (ok_mask >> jj) & 1;
      const int c = lane % LPT, part = lane / LPT;  // part 0: K, 1: V, others idle
      char* kb = const_cast<char*>(lane_ptr(kaddr, jj));
      char* vb = const_cast<char*>(lane_ptr(vaddr, jj));
      float x[8];
      {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (part < 2)
          u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(part ? a.v_new : a.k_new) +
                                              (static_cast<size_t>(b) * kPWaves + h) * D + 8 * c);
        widen8<true>(u, x);
      }
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = x[e];
      fwht_rotate8<D>(y, a.signs, c, a.inv_sqrt_d);  // every lane takes part
      if (part == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = y[e];
      }
      char* rec = nullptr;
      if (row_live && part < 2) {
        const int slot = p % kPBS;
        rec = part == 0 ? kb + static_cast<size_t>(slot) * KROW + h * KREC
                        : vb + static_cast<size_t>(slot) * VROW + h * VREC;
      }
      quantise_store8<D, GS>(x, c, part == 0 ? KB : VB, rec);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have reached L2
      __syncthreads();
    }
  }

  // Stage loads: unit u < KU is 16 bytes of the K rows, the rest of the V rows.
  u32x4 rg[S::UPT];
  auto fetch = [&](int i) {
    const int jb = i / SPB, t0 = (i % SPB) * T;
    const char* kb = lane_ptr(kaddr, jb) + static_cast<size_t>(t0) * KROW;
    const char* vb = lane_ptr(vaddr, jb) + static_cast<size_t>(t0) * VROW;
#pragma unroll
    for (int r = 0; r < S::UPT; ++r) {
      const int u = threadIdx.x + r * kPThreads;
      if (u < S::KU) rg[r] = __builtin_nontemporal_load((const gu32x4*)(kb + static_cast<size_t>(u) * 16));
      else if (u < S::KU + S::VU)
        rg[r] = __builtin_nontemporal_load((const gu32x4*)(vb + static_cast<size_t>(u - S::KU) * 16));
    }
  };
  if (n_stages > 0) fetch(0);

  // ---- query: widen, signs, fp32 Walsh-Hadamard butterflies (in registers),
  // then into this wave's LDS area as [G][D] -----------------------------
  float* sq = s_aux[h];
  const float qs = a.inv_sqrt_d * a.scale_log2;  // scores live in the exp2 domain
  // and per (query head, group): the sum of q' (offset term) and 1024 times
  // the sum of the A operand's f16 values, both parts (the bias the biased
  // key codes add), each over the lane's 8 values and then its group's GS/8
  // lanes; all of it at the query head's prescale 2^kq
#pragma unroll
  for (int p = 0; p < QPASS; ++p) {
    const int j = p * QVPP + lane / QLPT;
    float x[8];
    widen8<true>(qraw[p], x);
    const float sgq[8] = {sg0.x, sg0.y, sg0.z, sg0.w, sg1.x, sg1.y, sg1.z, sg1.w};
    signed_fwht8<D>(x, qc, sgq);  // exact sign flips, then the butterflies; every lane takes part
    float mq = 0.f;  // largest |q' * qs| of the query head, over its QLPT lanes
#pragma unroll
    for (int e = 0; e < 8; ++e) mq = fmaxf(mq, fabsf(x[e] * qs));
#pragma unroll
    for (int m = 1; m < QLPT; m <<= 1) mq = fmaxf(mq, __shfl_xor(mq, m, kWave));
    const int kq = query_prescale(mq);
    const float qsf = qs * exp2i(kq);  // exact: a power of two
    float qsum_l = 0.f, ab_l = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qsum_l += x[e];
      _Float16 hi, lo;
      split_f16(x[e] * qsf * key_q_factor<KB>(e), hi, lo);
      ab_l += static_cast<float>(hi) + static_cast<float>(lo);
    }
#pragma unroll
    for (int m = 1; m < GS / 8; m <<= 1) {
      qsum_l += __shfl_xor(qsum_l, m, kWave);
      ab_l += __shfl_xor(ab_l, m, kWave);
    }
    if (j < G) {
      float4* dst = reinterpret_cast<float4*>(sq + j * D + 8 * qc);
      dst[0] = make_float4(x[0], x[1], x[2], x[3]);
      dst[1] = make_float4(x[4], x[5], x[6], x[7]);
      if (qc % (GS / 8) == 0) {
        s_qs[h][j * NMG + qc / (GS / 8)] = qsum_l * qsf;
        s_kb[h][j * NMG + qc / (GS / 8)] = ab_l * 1024.f;
      }
      if (qc == 0) s_qk[h][j] = kq;
    }
  }
  __syncthreads();  // q', its group sums in LDS
  // A operands of the score products, k-block J: row m = n holds the high
  // f16 part of query head m / 4 when m % 4 == 0 and its low part when m % 4
  // == 1 (rows of absent query heads and the rest are zero), so output
  // registers 0 and 1 of a score lane hold the two parts' products
  h8 aq[NKB];
  {
    const int part = n % 4;
    const bool live = part < 2 && n / 4 < G;
    const int jq = live ? n / 4 : 0;
    const float qsf = qs * exp2i(s_qk[h][jq]);
#pragma unroll
    for (int g = 0; g < NKB; ++g) {
      // the lane's 8 values of the k-block are contiguous (4-bit codes take them permuted)
      const float4* src = reinterpret_cast<const float4*>(sq + jq * D + g * 32 + J * 8);
      const float4 lo4 = src[0], hi4 = src[1];
      const float vals[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = key_value_index<KB>(e);
        _Float16 hi, lo;
        split_f16(vals[v] * qsf * key_q_factor<KB>(v), hi, lo);
        aq[g][e] = live ? (part == 0 ? hi : lo) : static_cast<_Float16>(0.f);
      }
    }
  }
  // each lane takes the group sums of query head J of the score layout; the
  // stage loop's first barrier orders these LDS reads before p^T reuses the area
  float qsum[NMG], kbias[NMG];
#pragma unroll
  for (int g = 0; g < NMG; ++g) {
    qsum[g] = J < G ? s_qs[h][J * NMG + g] : 0.f;
    kbias[g] = J < G ? s_kb[h][J * NMG + g] : 0.f;
  }
  const float qinv = J < G ? exp2i(-s_qk[h][J]) : 1.f;  // undoes the query prescale (exact)
  // first accumulator of each group's score products: the bias the biased
  // key codes add, taken off inside the product (score register 0; register
  // 1 collects the low part of q')
  f4 cinit[NMG];
#pragma unroll
  for (int g = 0; g < NMG; ++g) cinit[g] = f4{-kbias[g], 0.f, 0.f, 0.f};

  f4 acc[NACC];  // lane l: dimension vdim(i, l), register r: query head r
#pragma unroll
  for (int i = 0; i < NACC; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  // value prescale exponents per group, and the factors 2^vk (wave-uniform)
  int vk[NMG];
  float pf[NMG];
#pragma unroll
  for (int g = 0; g < NMG; ++g) {
    vk[g] = kVk0;
    pf[g] = exp2i(kVk0);
  }
  // The f16 operands of a step are p * scale * 2^vk (p <= 1).  A step whose
  // value scales (read unmasked: cheaper, and a stale invisible scale costs
  // at most a needless look) may exceed 2^15 / 2^vk takes the slow path:
  // each group whose largest visible scale s has s * 2^vk above 2^15 gets
  // the exponent that brings s below 2^15, and its accumulator columns are
  // rescaled by the exact ratio.  Then no operand can reach f16's range.
  int vk_top = kVk0;  // max over groups of vk: the lowest threshold is 2^(15 - vk_top)
  auto fit_value_prescale = [&](const bool (&tv)[NSUB], const float2 (&vm)[NSUB][NMG]) {
    // scales are >= 0, so their bit patterns order as unsigned integers
    // (a NaN or -0 only sends the step to the slow path)
    uint32_t big = 0u;
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int g = 0; g < NMG; ++g) big = max(big, __builtin_bit_cast(uint32_t, vm[u][g].x));
    if (!__ballot(big > __builtin_bit_cast(uint32_t, exp2i(15 - vk_top)))) return;  // uniform; rare
    vk_top = -1000;
#pragma unroll
    for (int g = 0; g < NMG; ++g) {
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) mx = fmaxf(mx, tv[u] ? vm[u][g].x : 0.f);
      mx = row_max16(mx);
      mx = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), 48))));
      if (mx > exp2i(15 - vk[g])) {
        const int knew = __builtin_amdgcn_readfirstlane(14 - exponent_of(mx));
        const float ratio = exp2i(knew - vk[g]);
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
          const float f = vdim<VB>(i, lane) / GS == g ? ratio : 1.f;
          acc[i] *= f;
        }
        vk[g] = knew;
        pf[g] = exp2i(knew);
      }
      vk_top = max(vk_top, vk[g]);
    }
    vk_top = __builtin_amdgcn_readfirstlane(vk_top);
  };

  float m_run = -INFINITY, l_run = 0.f, bias[NMG];
#pragma unroll
  for (int g = 0; g < NMG; ++g) bias[g] = 0.f;
  // p * scale * 1024 as f16: [group][query head][token of the step]
  _Float16* sp = reinterpret_cast<_Float16*>(s_aux[h]);

  for (int i = 0; i < n_stages; ++i) {
    if constexpr (kPMinWaves<D> >= 4) {
      // Two workgroups share a CU here, and the older one's waves win issue
      // ties, so it finished its stages well before the younger one.  A
      // workgroup's priority falls as it advances (3 at the start, 0 in the
      // last quarter), so one that is behind gets the ties instead (K8V8 at
      // head_dim 64: 58.1-58.6 -> 55.9 us).
      const int pr = 3 - (4 * i) / n_stages;
      if (pr == 3) __builtin_amdgcn_s_setprio(3);
      else if (pr == 2) __builtin_amdgcn_s_setprio(2);
      else if (pr == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();  // every wave is done with the previous stage
#pragma unroll
    for (int r = 0; r < S::UPT; ++r) {
      const int u = threadIdx.x + r * kPThreads;
      if (u < S::KU) {
        const int t = u / (KROW / 16), c = u % (KROW / 16);
        *reinterpret_cast<u32x4*>(s_stage + t * PK + c * 16) = rg[r];
      } else if (u < S::KU + S::VU) {
        const int v = u - S::KU;
        const int t = v / (VROW / 16), c = v % (VROW / 16);
        *reinterpret_cast<u32x4*>(s_stage + T * PK + t * PV + c * 16) = rg[r];
      }
    }
    if (i + 1 < n_stages) fetch(i + 1);
    __syncthreads();  // stage i is in LDS

    const int jb = i / SPB, t0 = (i % SPB) * T;
    const int nt = ((ok_mask >> jb) & 1) ? min(kPBS, len - (s + jb * n_split) * kPBS) : 0;
#pragma unroll
    for (int st = 0; st < T / STEP; ++st) {
      const int lt0 = st * STEP;  // first token of the step in the stage
      if (t0 + lt0 >= nt) break;  // uniform: the rest of the stage is past the length

      float alpha;
      if constexpr (NSUB == 1) {
        // scores: lane (n, J) = (token n, query head J)
        const unsigned char* krow = s_stage + (lt0 + n) * PK + h * KREC;
        float sv = 0.f;
#pragma unroll
        for (int mg = 0; mg < NMG; ++mg) {
          // the k-blocks of one group accumulate in one product chain
          f4 c = cinit[mg];
#pragma unroll
          for (int kk = 0; kk < KPG; ++kk) {
            const int g = mg * KPG + kk;
            const h8 bk = key_codes<KB>(krow + g * (32 * KB / 8) + J * KB);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[g], bk, c, 0, 0, 0);
          }
          const float2 km = *reinterpret_cast<const float2*>(krow + S::KCODE + 8 * mg);
          sv = fmaf(c[0] + c[1], km.x, fmaf(km.y, qsum[mg], sv));
        }
        const bool tv = J < G && t0 + lt0 + n < nt;
        // sv carries the query prescale: qinv takes it off (in the max, and
        // in the exponent's fma)
        const float sc = tv ? sv : -INFINITY;
        const float m_new = fmaxf(m_run, row_max16(sc) * qinv);  // -inf while nothing is visible
        alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float p = (sc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(fmaf(sc, qinv, -m_new));
        m_run = m_new;
        l_run = fmaf(l_run, alpha, p);
        // value metadata of token n; invisible tokens add nothing even if it is garbage
        const unsigned char* vrow = s_stage + T * PK + (lt0 + n) * PV + h * VREC;
        float2 vm[1][NMG];
#pragma unroll
        for (int g = 0; g < NMG; ++g) vm[0][g] = *reinterpret_cast<const float2*>(vrow + S::VCODE + 8 * g);
        const bool ta[1] = {tv};
        fit_value_prescale(ta, vm);
#pragma unroll
        for (int g = 0; g < NMG; ++g) {
          bias[g] = fmaf(bias[g], alpha, tv ? p * vm[0][g].y : 0.f);
          sp[(g * 4 + J) * STEP + n] = static_cast<_Float16>(tv ? (p * pf[g]) * vm[0][g].x : 0.f);
        }
      } else {
        // scores of each sub-tile: lane (n, J) = (token n, query head J);
        // sub-tiles past the length are computed and masked.  Every LDS read
        // of the step goes out first (key codes and metadata, then the value
        // metadata), then the sub-tiles' product chains, which are
        // independent, so that one chain's latency hides behind the others.
        uint2 kr[NSUB][NKB];
        float2 km[NSUB][NMG], vm[NSUB][NMG];
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          const unsigned char* krow = s_stage + (lt0 + u * kSub + n) * PK + h * KREC;
#pragma unroll
          for (int g = 0; g < NKB; ++g) kr[u][g] = key_load<KB>(krow + g * (32 * KB / 8) + J * KB);
#pragma unroll
          for (int mg = 0; mg < NMG; ++mg) km[u][mg] = *reinterpret_cast<const float2*>(krow + S::KCODE + 8 * mg);
        }
        // value metadata of the step's tokens; invisible tokens add nothing
        // even if it is garbage
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          const unsigned char* vrow = s_stage + T * PK + (lt0 + u * kSub + n) * PV + h * VREC;
#pragma unroll
          for (int g = 0; g < NMG; ++g) vm[u][g] = *reinterpret_cast<const float2*>(vrow + S::VCODE + 8 * g);
        }
        f4 c[NSUB][NMG];
#pragma unroll
        for (int u = 0; u < NSUB; ++u)
#pragma unroll
          for (int mg = 0; mg < NMG; ++mg) c[u][mg] = cinit[mg];
#pragma unroll
        for (int kk = 0; kk < KPG; ++kk)
#pragma unroll
          for (int u = 0; u < NSUB; ++u)
#pragma unroll
            for (int mg = 0; mg < NMG; ++mg) {
              const int g = mg * KPG + kk;
              c[u][mg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aq[g], key_unpack<KB>(kr[u][g]), c[u][mg], 0, 0, 0);
            }
        float sc[NSUB];
        bool tv[NSUB];
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          float sv = 0.f;
#pragma unroll
          for (int mg = 0; mg < NMG; ++mg) sv = fmaf(c[u][mg][0] + c[u][mg][1], km[u][mg].x, fmaf(km[u][mg].y, qsum[mg], sv));
          tv[u] = J < G && t0 + lt0 + u * kSub + n < nt;
          sc[u] = tv[u] ? sv : -INFINITY;  // carries the query prescale, taken off by qinv below
        }
        float mx = sc[0];
#pragma unroll
        for (int u = 1; u < NSUB; ++u) mx = fmaxf(mx, sc[u]);
        const float m_new = fmaxf(m_run, row_max16(mx) * qinv);  // -inf while nothing is visible
        alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float p[NSUB];
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          // NaN when both are -inf: not used
          const float e = __builtin_amdgcn_exp2f(fmaf(sc[u], qinv, -m_new));
          p[u] = (sc[u] == -INFINITY) ? 0.f : e;
        }
        m_run = m_new;
        l_run = fmaf(l_run, alpha, p[0]);
#pragma unroll
        for (int u = 1; u < NSUB; ++u) l_run += p[u];
        fit_value_prescale(tv, vm);
#pragma unroll
        for (int g = 0; g < NMG; ++g) {
          float bg = fmaf(bias[g], alpha, tv[0] ? p[0] * vm[0][g].y : 0.f);
#pragma unroll
          for (int u = 0; u < NSUB; ++u) {
            if (u > 0) bg += tv[u] ? p[u] * vm[u][g].y : 0.f;
            sp[(g * 4 + J) * STEP + u * kSub + n] =
                static_cast<_Float16>(tv[u] ? (p[u] * pf[g]) * vm[u][g].x : 0.f);
          }
          bias[g] = bg;
        }
      }
      if (__ballot(alpha != 1.f)) {
        // alpha of query head r is uniform over score row r
#pragma unroll
        for (int r = 0; r < G; ++r) {
          const float ar = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), kSub * r));
#pragma unroll
          for (int i = 0; i < NACC; ++i) acc[i][r] *= ar;
        }
      }
      __builtin_amdgcn_wave_barrier();
      // values: block lane / 4 of a 4x4x4 product; A row lane % 4 is query
      // head lane % 4 (rows of absent query heads hold zeros); the B/C column
      // of lane l is dimension vdim(i, l)
      const int qa = lane % 4;
      {
        // one transpose load per 16 tokens and 32 code bytes gives lane l byte
        // column tr_col(l) of the 8 tokens t8 .. t8 + 7; each dword of it (4
        // tokens) feeds the products of its dimensions
        const int col = tr_col(lane);
        const int t8 = 8 * ((lane % 16) / 8);
        const unsigned char* vcol = s_stage + T * PK + (lt0 + tr_token(lane)) * PV + h * VREC + 8 * (lane / 16);
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
#pragma unroll
          for (int rd = 0; rd < NRD; ++rd) {
            const uint2 w = lds_read_tr8(vcol + u * kSub * PV + 32 * rd);
#pragma unroll
            for (int dw = 0; dw < 2; ++dw) {
              const uint32_t x = dw ? w.y : w.x;
              const int tq0 = u * kSub + t8 + 4 * dw;  // the dword's first token in the step
              const uint32_t p01 = bytes_subnormal(x, kSelB01), p23 = bytes_subnormal(x, kSelB23);
              if constexpr (VB == 8) {
                const h4 ap = *reinterpret_cast<const h4*>(sp + ((32 * rd + col) / GS * 4 + qa) * STEP + tq0);
                const uint32_t u2[2] = {p01, p23};
                acc[rd] = __builtin_amdgcn_mfma_f32_4x4x4f16(ap, __builtin_bit_cast(h4, u2), acc[rd], 0, 0, 0);
              } else {
                // low nibbles masked (code), high nibbles with the low one
                // beside them (lo + 16 hi; the low sum comes off at the end)
                const h4 ap = *reinterpret_cast<const h4*>(sp + ((64 * rd + 2 * col) / GS * 4 + qa) * STEP + tq0);
                const uint32_t ul[2] = {p01 & 0x000f000fu, p23 & 0x000f000fu};
                const uint32_t uh[2] = {p01, p23};
                acc[2 * rd] = __builtin_amdgcn_mfma_f32_4x4x4f16(ap, __builtin_bit_cast(h4, ul), acc[2 * rd], 0, 0, 0);
                acc[2 * rd + 1] =
                    __builtin_amdgcn_mfma_f32_4x4x4f16(ap, __builtin_bit_cast(h4, uh), acc[2 * rd + 1], 0, 0, 0);
              }
            }
            // keep each load next to its products (bounds the registers the
            // scheduler would otherwise spend hoisting loads)
            if constexpr (NRD >= PAGEDKV_PMFMA_TR_BARRIER_NRD) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // partials: (max, sum) and the group offsets' sums are uniform over score
  // row r; lane l holds dimension vdim(i, l) of query head r in register r
  // (lanes l and l + 8 of a 16-lane group hold the two token halves of the
  // same dimensions, added here; the lower lane writes)
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < G; ++r) acc[i][r] += __shfl_down(acc[i][r], 8, 16);
  if constexpr (VB == 4) {  // a high nibble's sum holds its low nibble's
#pragma unroll
    for (int i = 1; i < NACC; i += 2) acc[i] -= acc[i - 1];
  }
  const bool writer = lane % 16 < 8;
  const float l_tot = group_sum<kSub>(l_run);
  float btot[NMG];
#pragma unroll
  for (int g = 0; g < NMG; ++g) btot[g] = group_sum<kSub>(bias[g]);
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const size_t hs = (static_cast<size_t>(b) * a.n_q + h * G + r) * n_split + s;
    float* part_acc = a.partials + hs * D;
    float bq[NMG];  // the group offsets' sums of query head r
#pragma unroll
    for (int g = 0; g < NMG; ++g)
      bq[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, btot[g]), kSub * r));
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      const int d = vdim<VB>(i, lane);
      float bsel = 0.f;
      int ksel = kVk0;
#pragma unroll
      for (int g = 0; g < NMG; ++g) {
        bsel = d / GS == g ? bq[g] : bsel;
        ksel = d / GS == g ? vk[g] : ksel;
      }
      if (writer) part_acc[d] = fmaf(acc[i][r] * kSubnormalUnit, vacc_scale<VB>(i, ksel), bsel);
    }
    if (lane == kSub * r) {
      a.partials[a.ml_offset + hs * 2] = m_run;
      a.partials[a.ml_offset + hs * 2 + 1] = l_tot;
    }
  }
}

template <int D, int KB, int VB, int G, int GS>
hipError_t launch_mfma(const DecodeArgs& a, hipStream_t s) {
  const int grid = round_up(a.B * a.n_split, kXcds);
  hipLaunchKernelGGL((paged_decode_packed_mfma_kernel<D, KB, VB, G, GS>), dim3(grid), dim3(kPThreads), 0, s, a);
  return hipGetLastError();
}

template <int D, int KB, int VB, int GS>
hipError_t mfma_by_group(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_mfma<D, KB, VB, 1, GS>(a, s);
    case 2: return launch_mfma<D, KB, VB, 2, GS>(a, s);
    case 4: return launch_mfma<D, KB, VB, 4, GS>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KB, int VB>
hipError_t mfma_by_dim(const DecodeArgs& a, int head_dim, int group, hipStream_t s) {
  switch (head_dim * 100 + a.qgroup) {
    case 6432: return mfma_by_group<64, KB, VB, 32>(a, group, s);
    case 12832: return mfma_by_group<128, KB, VB, 32>(a, group, s);
    case 25632: return mfma_by_group<256, KB, VB, 32>(a, group, s);
    case 12864: return mfma_by_group<128, KB, VB, 64>(a, group, s);
    case 25664: return mfma_by_group<256, KB, VB, 64>(a, group, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool packed_mfma_supported(int32_t n_kv, int32_t head_dim, int32_t group, int32_t block_size,
                           int32_t qgroup) {
  return n_kv == kPWaves && block_size == kPBS && (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
         (group == 1 || group == 2 || group == 4) && (qgroup == 32 || (qgroup == 64 && head_dim >= 128));
}

// Workgroups a launch aims for: two per CU where a workgroup's registers allow it.
int packed_mfma_target_workgroups(int32_t head_dim) {
  return head_dim <= 64 ? PAGEDKV_PMFMA_TARGET_WG_SMALL : PAGEDKV_PMFMA_TARGET_WG;
}

hipError_t launch_paged_decode_packed_mfma(const DecodeArgs& a, int32_t head_dim, int32_t group,
                                           hipStream_t s) {
  if (a.k_bits == 8 && a.v_bits == 8) return mfma_by_dim<8, 8>(a, head_dim, group, s);
  if (a.k_bits == 8 && a.v_bits == 4) return mfma_by_dim<8, 4>(a, head_dim, group, s);
  if (a.k_bits == 4 && a.v_bits == 4) return mfma_by_dim<4, 4>(a, head_dim, group, s);
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
