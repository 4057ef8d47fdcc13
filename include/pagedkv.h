/*
 * pagedkv -- single-token paged decode attention over a chunked-slab KV pool,
 * for AMD Instinct MI355X (gfx950).
 *
 * The pool follows mlxcel issue #235 ("perf(core): chunked slab storage for
 * the paged pool to eliminate growth reallocation entirely", section
 * "Proposed solution: chunked slabs"): every layer keeps a growing list of
 * fixed-size K slabs and V slabs, each slab shaped
 *     [slab_blocks, block_size, n_kv_heads, record]
 * where a record is one token-head vector.  Physical row r lives in slab
 * r / slab_blocks at row r % slab_blocks.  Growth appends a zeroed slab and
 * never copies.  Kernels reach a row through a per-layer device table of slab
 * base pointers, so no single pool buffer exists and nothing is gathered
 * before attention.
 *
 * Records:
 *   PD_FMT_FP16, PD_FMT_BF16 : head_dim 16-bit values (2 * head_dim bytes).
 *   PD_FMT_K8V8, PD_FMT_K8V4, PD_FMT_K4V4 (mlx-swift-lm PR #142, "Add packed
 *   paged KV formats with bounded workspace admission", section "Summary"):
 *   unsigned codes of the given bit width (8-bit: one byte per value; 4-bit:
 *   value 2i in the low nibble of byte i), then one (fp32 scale, fp32 offset)
 *   pair per group of 32 or 64 values (pd_pool_desc.group_size), little
 *   endian; a value is code*scale+offset.
 *   K is rotated by the fixed signed Hadamard basis H*diag(sigma)/sqrt(D)
 *   before it is quantised; V is not rotated.  Packed pools take bf16 keys,
 *   values and queries and produce bf16 outputs.
 *
 * Conventions for every call:
 *   - Device memory is allocated by the caller (slabs, inputs, outputs,
 *     workspace).  The library owns only its slab-pointer tables and a
 *     4-byte device error word per pool.
 *   - Pointers documented as "device" must be device-accessible memory of the
 *     pool's device; "host" pointers are read before the call returns.
 *   - All device work is enqueued on the caller's stream and is ordered by it;
 *     no call below synchronises the host except pd_pool_check_error, and
 *     none allocates device memory except pd_pool_create.
 *   - Argument errors return a negative pd_status and enqueue nothing;
 *     pd_last_error() then describes the problem (thread-local string).
 *   - Data-dependent errors found by a kernel (a block-table row or a
 *     write_block row/slot outside the pool, a sequence length the call
 *     cannot hold) set a sticky bit in the pool's device error word; the
 *     offending block or token is skipped (a bad length is clamped) and no
 *     memory outside the pool, the inputs and the outputs is touched.  Read
 *     and clear the word with pd_pool_check_error.
 *   - One pool is used from one host thread at a time.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PD_VERSION 1

typedef enum pd_status {
  PD_OK = 0,
  PD_ERR_ARG = -1,          /* invalid argument (null, negative, inconsistent) */
  PD_ERR_RANGE = -2,        /* layer / row / size outside the pool             */
  PD_ERR_CAPACITY = -3,     /* slab-pointer table full or workspace too small  */
  PD_ERR_UNSUPPORTED = -4,  /* shape or format without a kernel                */
  PD_ERR_HIP = -5,          /* a HIP runtime call failed                       */
  PD_ERR_DEVICE = -6,       /* a kernel reported a data-dependent error        */
  PD_ERR_IDENTITY = -7      /* block bytes of another storage identity         */
} pd_status;

typedef enum pd_format {
  PD_FMT_FP16 = 0,
  PD_FMT_BF16 = 1,
  PD_FMT_K8V8 = 2,
  PD_FMT_K8V4 = 3,
  PD_FMT_K4V4 = 4
} pd_format;

/* Device error word bits (pd_pool_check_error). */
#define PD_DEVERR_WRITE_ROW   0x1  /* write_block: row outside [0, capacity_rows) */
#define PD_DEVERR_WRITE_SLOT  0x2  /* write_block: slot outside [0, block_size)   */
#define PD_DEVERR_TABLE_ROW   0x4  /* a block-table row outside the pool          */
#define PD_DEVERR_LENGTH      0x8  /* lens[b] < 0, or beyond max_blocks*block_size,
                                      t_out (gather) or max_len (decode)        */
#define PD_DEVERR_DUPLICATE   0x10 /* write_block, duplicate-write check on: two
                                      tokens of one call target one (row, slot) */

/* Debug checks (pd_pool_set_debug). */
#define PD_DEBUG_DUPLICATE_WRITES 0x1u

typedef struct pd_pool_desc {
  int32_t n_layers;      /* >= 1                                                */
  int32_t block_size;    /* tokens per block (row): 16, 32 or 64                */
  int32_t n_kv_heads;    /* >= 1; packed formats: 8                             */
  int32_t head_dim;      /* 64, 128 or 256                                      */
  int32_t slab_blocks;   /* POOL_SLAB_BLOCKS: rows per slab, >= 1               */
  int32_t max_slabs;     /* capacity of the slab-pointer tables, >= 1           */
  int32_t format;        /* pd_format                                           */
  const int8_t* hadamard_signs; /* host, [head_dim] of +1/-1; packed formats
                                   only (copied at create), else NULL           */
  int32_t group_size;    /* packed formats: values per (fp32 scale, offset)
                            pair, 32 or 64 (64 needs head_dim 128 or 256, so
                            that a record is whole 16-byte units); 0 means 32.
                            16-bit formats: 0                                  */
} pd_pool_desc;

typedef struct pd_stats {
  int64_t n_slabs;                /* slabs per layer (same for K and V)         */
  int64_t slab_append_events;     /* appends since create (one per new slab)    */
  int64_t capacity_rows;          /* n_slabs * slab_blocks                      */
  int64_t bytes_reserved;         /* n_layers * n_slabs * (K + V slab bytes)    */
  int64_t bytes_copied_on_growth; /* always 0: growth never copies              */
  int64_t k_slab_bytes;           /* bytes of one K slab of one layer           */
  int64_t v_slab_bytes;           /* bytes of one V slab of one layer           */
  int32_t k_record_bytes;         /* bytes of one K token-head record           */
  int32_t v_record_bytes;         /* bytes of one V token-head record           */
} pd_stats;

/*
 * Storage identity: everything the bytes of a block depend on.  Blocks
 * exported from one pool can be imported into another only when their
 * identities are equal (mlx-swift-lm PR #142, section "Summary": resident
 * reuse and complete checkpoints preserve packed bytes and reject
 * incompatible storage identities before allocation; the "After" flowchart:
 * exact packed checkpoint with format identity).  48 bytes, little endian,
 * no padding; the slab geometry (slab_blocks, max_slabs) is not part of it:
 * a block is a row, wherever its slab is.
 */
#define PD_IDENTITY_MAGIC 0x564B4450u /* bytes "PDKV" */
#define PD_IDENTITY_LAYOUT 1u          /* record layout described at the top */
typedef struct pd_storage_identity {
  uint32_t magic;           /* PD_IDENTITY_MAGIC                                */
  uint32_t layout;          /* PD_IDENTITY_LAYOUT                               */
  int32_t format;           /* pd_format                                        */
  int32_t n_layers;
  int32_t block_size;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t k_record_bytes;
  int32_t v_record_bytes;
  int32_t group_size;       /* values per (scale, offset) pair: 32 or 64 packed,
                               0 for 16-bit formats                            */
  uint64_t signs_hash;      /* packed: pd_signs_hash of the Hadamard signs; 0   */
} pd_storage_identity;

typedef struct pd_pool pd_pool;

/* Library version (PD_VERSION). */
int32_t pd_version(void);

/* Description of the last error on this thread ("" if none). */
const char* pd_last_error(void);

/* Bytes of one K and one V token-head record for a format, head_dim and
 * group size (packed: codes + 8 bytes per group; group_size 0 means 32;
 * 16-bit formats ignore it).  mlx-swift-lm PR #142, section "Summary": with
 * 4-bit codes and groups of 64 a value costs five bits. */
pd_status pd_record_bytes(int32_t format, int32_t head_dim, int32_t group_size, int32_t* k_bytes,
                          int32_t* v_bytes);

/*
 * Create an empty pool (no slabs) on the current HIP device.
 * mlxcel #235, "Proposed solution": per-layer slab vectors replace the single
 * pool tensor.  Allocates the device slab-pointer tables
 * (n_layers * 2 * max_slabs pointers) and the device error word.
 * out: host, receives the handle.  Errors: PD_ERR_ARG, PD_ERR_UNSUPPORTED,
 * PD_ERR_HIP.  Packed pools are refused (PD_ERR_UNSUPPORTED) unless the
 * packed decode kernel can read them: block_size 32, n_kv_heads 8, head_dim
 * 64/128/256, group_size 32 (or 64 with head_dim 128, 256).  Their decode
 * calls take 8, 16 or 32 query heads (1, 2 or 4 per kv head).
 */
pd_status pd_pool_create(const pd_pool_desc* desc, pd_pool** out);

/* Release the library's tables.  Slab memory stays the caller's.  Waits for
 * the device to finish work that may still read the tables. */
pd_status pd_pool_destroy(pd_pool* pool);

/* Bytes of one K slab and one V slab of one layer
 * (slab_blocks * block_size * n_kv_heads * record bytes); host outputs. */
pd_status pd_slab_bytes(const pd_pool* pool, size_t* k_bytes, size_t* v_bytes);

/*
 * Append one slab to every layer.  mlxcel #235, "Proposed solution": growth
 * appends a fresh zeros slab -- no copy, no free, no transient old+new pair.
 * k_mem, v_mem: host arrays of n_layers device pointers, each to
 * pd_slab_bytes() bytes (256-byte aligned) that the caller keeps alive until
 * pd_pool_destroy.  The library zero-fills them on `stream`, records the
 * pointers in its tables and increments slab_append_events.  All-or-nothing:
 * on any error nothing is recorded.  new_index (host, optional) receives the
 * new slab's index.  Errors: PD_ERR_ARG, PD_ERR_CAPACITY (table full),
 * PD_ERR_HIP.
 */
pd_status pd_append_slab(pd_pool* pool, void* const* k_mem, void* const* v_mem,
                         hipStream_t stream, int32_t* new_index);

/* Number of slabs that pd_reserve_rows must append so that rows
 * [0, rows_needed) exist (0 if they already do); host output. */
pd_status pd_slabs_needed(const pd_pool* pool, int64_t rows_needed, int32_t* n_slabs);

/*
 * presize_for_span (mlxcel #235, "Proposed solution"): append as many slabs
 * as a span needs in one step.  n_slabs must equal pd_slabs_needed(); k_mem
 * and v_mem hold n_slabs * n_layers device pointers, slab-major
 * (entry s * n_layers + layer).  All-or-nothing.  n_appended: host, optional.
 */
pd_status pd_reserve_rows(pd_pool* pool, int64_t rows_needed, void* const* k_mem,
                          void* const* v_mem, int32_t n_slabs, hipStream_t stream,
                          int32_t* n_appended);

/*
 * slab_for_row (mlxcel #235, "Proposed solution", touch point 7): the K and V
 * slab base pointers (device addresses, host outputs) of the slab holding
 * `row` in `layer`, and the row's index inside that slab.
 * Errors: PD_ERR_RANGE if layer or row is outside the pool.
 */
pd_status pd_slab_for_row(const pd_pool* pool, int32_t layer, int64_t row, void** k_base,
                          void** v_base, int32_t* row_in_slab);

/*
 * write_block (mlxcel #235, "Proposed solution", touch point 1): scatter new
 * tokens into the slab of their row.  Token i goes to (rows[i], slots[i]) of
 * `layer`, K and V.
 *   rows, slots: device int32 [n].
 *   k_src, v_src: device [n, n_kv_heads, head_dim], fp16/bf16 as the pool
 *     format (packed formats: bf16; K is rotated and both are quantised here,
 *     once, as mlx-swift-lm PR #142's "quantize fresh K/V once").
 * A row outside [0, capacity_rows) or a slot outside [0, block_size) sets a
 * device error bit and that token is skipped.  Two tokens with the same
 * (row, slot) in one call give an unspecified winner.  n == 0 is a no-op.
 * Errors: PD_ERR_ARG (null or misaligned pointers, n < 0), PD_ERR_RANGE
 * (layer), PD_ERR_HIP.
 */
pd_status pd_write_block(pd_pool* pool, int32_t layer, int32_t n, const int32_t* rows,
                         const int32_t* slots, const void* k_src, const void* v_src,
                         hipStream_t stream);

/*
 * pool_set_debug: turn debug checks on or off for the calls that follow.
 * PD_DEBUG_DUPLICATE_WRITES checks the scatter of pd_write_block (mlxcel
 * #235, "Proposed solution", touch point 1: new K/V rows land in the row's
 * slab): two tokens of one call that target the same (row, slot) leave which
 * one is stored unspecified, so with the check on such a call sets
 * PD_DEVERR_DUPLICATE in the device error word (the call still writes).  The
 * check marks one bit per token in a device bitmap of one bit per slot of
 * the pool's largest capacity (max_slabs * slab_blocks * block_size bits,
 * allocated here the first time the check is turned on, freed by
 * pd_pool_destroy), and clears its bits again after the write: two more
 * launches per pd_write_block on `stream`.  Turning the check on allocates
 * and synchronises the device, so it is for set-up, not for graph capture;
 * calls that run at once on several streams of one pool share the bitmap.
 *   flags: a combination of PD_DEBUG_* bits; 0 turns every check off.
 * Errors: PD_ERR_ARG (unknown flag bits), PD_ERR_HIP (allocation).
 */
pd_status pd_pool_set_debug(pd_pool* pool, uint32_t flags);

/*
 * copy_on_write_block (mlxcel #235, "Proposed solution", touch point 2):
 * copy whole block rows inside the pool.  For each i, row dst_rows[i] of
 * every layer, K and V, receives the bytes of row src_rows[i]: the source
 * slice comes from the source row's slab and lands in the destination row's
 * slab, through the same row mapping as every other call.  This is the
 * block-level step of copy-on-write: a block shared by several sequences
 * (a common prefix) is duplicated into a row the caller has taken from its
 * free list before one sequence writes into it.  Packed pools copy records
 * byte for byte (no requantisation).
 *   n: number of pairs (>= 0); src_rows, dst_rows: device int32 [n].
 *   Destination rows must be distinct and must not appear among the source
 *   rows of the same call; otherwise the result is unspecified.
 * A pair with a source row outside [0, capacity_rows) sets
 * PD_DEVERR_TABLE_ROW, one with a destination row outside it sets
 * PD_DEVERR_WRITE_ROW, and that pair is skipped.  n == 0 is a no-op.
 */
pd_status pd_copy_on_write_block(pd_pool* pool, int32_t n, const int32_t* src_rows,
                                 const int32_t* dst_rows, hipStream_t stream);

/*
 * gather_visible (mlxcel #235, "Proposed solution", touch point 3): copy each
 * sequence's visible K and V out of the pool into contiguous, transposed
 * tensors: the same bytes the page's take-per-run, concatenate, reshape,
 * slice and transpose produce.  The kernel reads every block from the slab
 * its row names (the blocks of one same-slab run share that slab's base), so
 * all runs are copied at once; pd_split_runs returns the runs themselves.
 *   block_table: device int32 [B, max_blocks]; entry (b, i) is the physical
 *     row of logical block i of sequence b; entries past the sequence's block
 *     count are ignored.
 *   lens: device int32 [B], visible tokens per sequence, 0 <= lens[b] <= t_out
 *     and <= max_blocks * block_size.
 *   k_out, v_out: device [B, n_kv_heads, t_out, record] (record = head_dim
 *     16-bit values, or the packed record bytes).  Positions >= lens[b] are
 *     written as zero bytes.
 *   n_runs_out: device int32 [B], optional (NULL): number of same-slab runs
 *     of each sequence.
 */
pd_status pd_gather_visible(pd_pool* pool, int32_t layer, int32_t B, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* lens, int32_t t_out, void* k_out,
                            void* v_out, int32_t* n_runs_out, hipStream_t stream);

/*
 * split_runs (mlxcel #235, "Proposed solution", touch point 3): the maximal
 * same-slab runs of each sequence's visible blocks, in logical order.
 *   block_table, lens: as pd_gather_visible (max_blocks * block_size < 2^31).
 *   runs_out: device int32 [B, max_blocks, 3]; run k of sequence b is
 *     (slab, first logical block, number of blocks) at runs_out[b][k]; the
 *     entries past the sequence's run count are left as they were.
 *   n_runs_out: device int32 [B], the run count of each sequence (0 for an
 *     empty sequence).
 * A row outside [0, capacity_rows) counts as slab -1 (consecutive such rows
 * form one run) and sets PD_DEVERR_TABLE_ROW; a length outside [0,
 * max_blocks * block_size] is clamped and sets PD_DEVERR_LENGTH.  Layer
 * independent: rows name the same slab in every layer.
 */
pd_status pd_split_runs(pd_pool* pool, int32_t B, const int32_t* block_table, int32_t max_blocks,
                        const int32_t* lens, int32_t* runs_out, int32_t* n_runs_out, hipStream_t stream);

/*
 * Workspace bytes that pd_paged_decode needs for B sequences, n_q_heads query
 * heads and a longest sequence of at most max_len tokens (host output).
 * B * n_q_heads * splits above 2^30 (the split kernels' partial rows, in 32
 * bits) is PD_ERR_ARG, here and from pd_paged_decode.
 */
pd_status pd_decode_workspace_bytes(const pd_pool* pool, int32_t B, int32_t n_q_heads,
                                    int32_t max_len, size_t* bytes);

/*
 * paged_decode: attention of one query token per sequence over its visible
 * tokens, read in place from the slabs.  mlxcel #2171 ("refactor: one KV
 * storage abstraction with dense and paged backends", section "Proposed
 * Solution"): attend(q, k, v, scale, mask) with one query token and no mask;
 * query head h reads kv head h / (n_q_heads / n_kv_heads).
 *   q: device [B, n_q_heads, head_dim], the pool's 16-bit dtype (bf16 for
 *     packed pools; the kernel applies the Hadamard rotation itself).
 *   block_table, lens: as pd_gather_visible; tokens >= lens[b] are not read.
 *   max_len: host, >= max(lens); sizes the split of the token axis without a
 *     host-device synchronisation.  At most 65,536 blocks (1024 splits of 64
 *     blocks: 2,097,152 tokens at block_size 32); beyond that
 *     PD_ERR_UNSUPPORTED.
 *   scale: multiplies q.k (typically 1/sqrt(head_dim)).
 *   out: device [B, n_q_heads, head_dim], same dtype as q, rounded to nearest
 *     even once at the end.  A sequence with lens[b] == 0 gets zeros.
 *   workspace: device, >= pd_decode_workspace_bytes(), 256-byte aligned; it
 *     receives one partial (running max, sum, weighted V) per split of the
 *     token axis and needs no initialisation.  Calls sharing a workspace must
 *     be ordered (same stream).
 * Two kernels run: the split kernel, then a combine kernel that merges the
 * splits of each (sequence, kv head) in split order.
 * The result is bit-identical from run to run and independent of which
 * physical rows and slabs hold the data.
 * Packed pools: the matrix cores take f16 operands.  The rotated query goes
 * in as high and low f16 parts after a power-of-two scaling that keeps it in
 * f16 range (any finite query); p * scale goes in as f16 at a power-of-two
 * prescale per value group that the kernel lowers whenever a group's scale
 * demands it (any finite record).  Admitted inputs: finite values whose
 * rotated keys, group ranges (max - min), scores and outputs stay finite in
 * fp32 and in bf16 (every bf16 input with |x| <= 2^100 and a finite
 * output).  Error against exact arithmetic over the same records: at most
 * 2^-11 of sum_t p_t |v_t - offset_t| / sum_t p_t per output (f16 value
 * operands) plus what a score error of about 2^-18 of scale * sum_i |q'_i
 * k_i| moves, before the final rounding to bf16.
 */
pd_status pd_paged_decode(pd_pool* pool, int32_t layer, int32_t B, int32_t n_q_heads,
                          const void* q, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* lens, int32_t max_len, float scale, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * pd_paged_decode with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials go to a scratch
 * array inside the library, 16 MiB per device (a file-scope device array
 * that every device the library runs on holds until the process ends; its
 * address is looked up once per device, in the first pd_pool_create on that
 * device).  The call allocates nothing: no hipMalloc, hipFree or allocating
 * library routine.  Arguments, kernels, split plan and output are those of
 * pd_paged_decode with the same inputs, bit for bit.  A call whose partials
 * (pd_decode_workspace_bytes for its B, n_q_heads and max_len) exceed the
 * scratch is PD_ERR_CAPACITY and enqueues nothing.  Nothing in the scratch
 * needs to start at zero: every partial the combine reads is written by the
 * same call.  All calls on one device share that device's scratch, which
 * keeps the last call's contents: calls that overlap on one device (other
 * streams, other threads, other pools) race and give undefined outputs;
 * order them on one stream.
 */
pd_status pd_paged_decode_noalloc(pd_pool* pool, int32_t layer, int32_t B, int32_t n_q_heads,
                                  const void* q, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* lens, int32_t max_len, float scale, void* out,
                                  hipStream_t stream);

/*
 * Append then attend, in one launch of the split kernel: mlxcel #2171
 * ("refactor: one KV storage abstraction with dense and paged backends",
 * section "Proposed Solution"): attend(q, k, v, scale, mask) takes the new
 * token's K and V with its query; mlxcel #235, "Proposed solution", touch
 * point 1: the write lands in the slab of its row.  Token lens[b] - 1 of each
 * sequence is the new one: k_new[b], v_new[b] (device [B, n_kv_heads,
 * head_dim], the pool's 16-bit dtype, bf16 for packed pools, 16-byte
 * aligned) are written to row
 * block_table[b][(lens[b] - 1) / block_size], slot (lens[b] - 1) %
 * block_size, of `layer`, and the attention reads them there.  Pool bytes
 * and outputs are bit for bit those of pd_write_block of the same tokens
 * followed by pd_paged_decode.  Sequences with lens[b] == 0 append nothing;
 * a length or row the kernel rejects (device error word, as pd_paged_decode)
 * appends nothing for that sequence.  Other arguments as pd_paged_decode.
 * In a packed pool the new token is rotated (keys) and quantised in the
 * launch to the records pd_write_block stores (mlx-swift-lm PR #142, "Add
 * packed paged KV formats with bounded workspace admission", section
 * "Summary": fresh K/V are quantised once, attention reads the packed pages).
 * Only where the 16-bit row kernel runs (n_kv_heads * head_dim * 2 a multiple
 * of 1024 bytes, block_size 32, head_dim 64/128/256, group 1/2/4/8) or the
 * packed kernel runs (n_kv_heads 8, block_size 32, head_dim 64/128/256, group
 * 1/2/4; group_size 64 needs head_dim >= 128); else PD_ERR_UNSUPPORTED (use
 * pd_write_block, then pd_paged_decode).
 */
pd_status pd_paged_decode_append(pd_pool* pool, int32_t layer, int32_t B, int32_t n_q_heads,
                                 const void* q, const void* k_new, const void* v_new,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* lens,
                                 int32_t max_len, float scale, void* out, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * Dense decode: the same attention as pd_paged_decode over per-sequence
 * contiguous K/V, with no pool.  mlxcel #2171 ("refactor: one KV storage
 * abstraction with dense and paged backends", section "Proposed Solution":
 * dense and paged backends behind one attend(q, k, v, scale, mask); section
 * "Acceptance Criteria": dense and paged results identical under a
 * deterministic mode).
 *   desc: host; format PD_FMT_FP16 or PD_FMT_BF16, n_kv_heads, head_dim.
 *   k_seqs, v_seqs: device arrays [B] of device pointers; sequence b's K (V)
 *     is [lens[b], n_kv_heads, head_dim] contiguous and 16-byte aligned: the
 *     pool's block-row layout without the pool.
 *   q, lens, max_len, scale, out, workspace: as pd_paged_decode; the
 *     workspace size comes from pd_dense_workspace_bytes.
 * The kernels and the split of the token axis are those of a 16-bit pool of
 * block_size 32 with the same (B, n_q_heads, max_len), so the output is bit
 * for bit that of pd_paged_decode over the same tokens, wherever the pool
 * keeps them.  Shapes: those of the row kernel (n_kv_heads * head_dim * 2 a
 * multiple of 1024 bytes; head_dim 64, 128, 256; group 1, 2, 4, 8), else
 * PD_ERR_UNSUPPORTED.  There is no device error word: a length beyond
 * max_len is clamped to it.  B * ceil(max_len / 32) above 2^31 - 1, or B *
 * n_q_heads * splits above 2^30, is PD_ERR_ARG (here and from
 * pd_dense_workspace_bytes): the kernels index rows and partials in 32 bits.
 */
typedef struct pd_dense_desc {
  int32_t format;      /* PD_FMT_FP16 or PD_FMT_BF16 */
  int32_t n_kv_heads;
  int32_t head_dim;
} pd_dense_desc;

pd_status pd_dense_workspace_bytes(const pd_dense_desc* desc, int32_t B, int32_t n_q_heads,
                                   int32_t max_len, size_t* bytes);
pd_status pd_dense_decode(const pd_dense_desc* desc, int32_t B, int32_t n_q_heads, const void* q,
                          const void* const* k_seqs, const void* const* v_seqs,
                          const int32_t* lens, int32_t max_len, float scale, void* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two stages of pd_paged_decode as separate calls, same arguments and
 * checks: _split writes the per-split partials into the workspace, _combine
 * merges them into `out`.  pd_paged_decode == _split then _combine on one
 * stream.  For callers that place other work between the stages and for
 * per-stage timing.
 */
pd_status pd_paged_decode_split(pd_pool* pool, int32_t layer, int32_t B, int32_t n_q_heads,
                                const void* q, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* lens, int32_t max_len, float scale, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);
pd_status pd_paged_decode_combine(pd_pool* pool, int32_t layer, int32_t B, int32_t n_q_heads,
                                  const void* q, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* lens, int32_t max_len, float scale, void* out,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block serialisation (mlxcel #235, "Proposed solution", touch point 6: serde
 * block-content extraction and the restore path read and write each block in
 * the row's slab through the same row mapping).
 *
 * pd_signs_hash: FNV-1a, 64 bit (offset basis 0xcbf29ce484222325, prime
 * 0x100000001b3) over the n sign bytes as stored (+1 -> 0x01, -1 -> 0xFF).
 * Host only; needs no device.
 */
pd_status pd_signs_hash(const int8_t* signs, int32_t n, uint64_t* hash);

/* The pool's storage identity (host output). */
pd_status pd_storage_identity_of(const pd_pool* pool, pd_storage_identity* id);

/*
 * PD_OK when blocks of identity `id` (host) can be imported into `pool`;
 * otherwise PD_ERR_IDENTITY, and pd_last_error() names the first field that
 * differs.  Host only: call it before allocating anything for a restore.
 */
pd_status pd_identity_check(const pd_pool* pool, const pd_storage_identity* id);

/* Bytes of one exported block: n_layers * block_size * n_kv_heads *
 * (k_record_bytes + v_record_bytes) (host output). */
pd_status pd_block_bytes(const pd_pool* pool, size_t* bytes);

/*
 * export_blocks: the bytes of block rows rows[0..n), every layer, into a
 * contiguous buffer laid out [n][n_layers][K row, V row], where a K (V) row
 * is the block's [block_size, n_kv_heads, record] bytes exactly as stored.
 *   rows: device int32 [n]; dst: device, >= n * pd_block_bytes() bytes,
 *   16-byte aligned.
 * A row outside [0, capacity_rows) sets PD_DEVERR_TABLE_ROW and its slot of
 * dst is zero-filled.  n == 0 is a no-op.
 */
pd_status pd_export_blocks(pd_pool* pool, int32_t n, const int32_t* rows, void* dst,
                           size_t dst_bytes, hipStream_t stream);

/*
 * import_blocks: the restore path.  `id` (host) is the identity the bytes
 * were exported under; it is checked first, and a mismatch returns
 * PD_ERR_IDENTITY and enqueues nothing.  Then block i of src (layout as
 * pd_export_blocks) is written into row rows[i] of every layer, K and V.
 *   rows: device int32 [n], distinct; src: device, >= n * pd_block_bytes()
 *   bytes, 16-byte aligned.
 * A row outside [0, capacity_rows) sets PD_DEVERR_WRITE_ROW and that block is
 * skipped.  n == 0 is a no-op (after the identity check).
 */
pd_status pd_import_blocks(pd_pool* pool, const pd_storage_identity* id, int32_t n,
                           const int32_t* rows, const void* src, size_t src_bytes,
                           hipStream_t stream);

/* Pool counters (host output).  mlxcel #235: slab-append counter and
 * bytes_reserved summed over slabs. */
pd_status pd_pool_stats(const pd_pool* pool, pd_stats* stats);

/*
 * Synchronise `stream`, then read and clear the pool's sticky device error
 * word.  device_error (host, optional) receives the PD_DEVERR_* bits.
 * Returns PD_ERR_DEVICE if any bit was set, else PD_OK.
 */
pd_status pd_pool_check_error(pd_pool* pool, hipStream_t stream, int32_t* device_error);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
