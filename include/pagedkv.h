/*
 * pagedkv.h - C ABI of the paged KV-cache decode library for AMD MI355X (gfx950).
 *
 * The library implements the decode hot path of PagedAttention:
 *   - pa_decode:   single-query attention over a KV cache stored in fixed-size
 *                  physical blocks reached through per-sequence block tables;
 *   - kv_append:   write each new token's K/V into its slot;
 *   - copy_blocks: whole-block copies for copy-on-write of shared blocks;
 *   - a host-side block allocator (FIFO free list, reference counts, block
 *     tables, fork, copy-on-write decisions, free).
 *
 * Pages cited below:
 *   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
 *   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
 *   [KVM] "深入解析 vLLM 的 KV Cache 管理器：从内存碎片到 PagedAttention 的完整技术剖析"
 *         (zingnex.cn)
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Return value: PA_OK (0) or a negative pa_status. pa_last_error() gives a
 *    message for the calling thread's last failure. Nothing throws across the ABI.
 *  - Device pointers are caller-owned, contiguous, row-major, and live on the
 *    current HIP device. The library never allocates or frees device memory on
 *    these paths; pa_decode's scratch space is a caller-provided workspace.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued asynchronously; device-side results are visible after the
 *    caller synchronises the stream. Calls that share buffers must be ordered
 *    on one stream (copy_blocks of a step before that step's kv_append, both
 *    before the pa_decode that reads them).
 *  - Shapes, dtypes and pointers are validated on the host from the
 *    descriptors (PA_ERR_INVALID / PA_ERR_UNSUPPORTED, nothing enqueued).
 *    Contents (block ids, slots, context lengths) are range-checked inside the
 *    kernels so that no input can make a kernel read or write outside its
 *    buffers: out-of-range entries are skipped (kv_append, copy_blocks) or give
 *    NaN output rows (pa_decode). With the environment variable PA_DEBUG=1 the
 *    contents are also checked on the host before launch (this synchronises)
 *    and a bad entry returns PA_ERR_INVALID.
 *  - Cache layout (per layer): k_cache and v_cache are separate arrays
 *      [num_blocks][num_kv_heads][block_size][head_dim]
 *    so that one (block, head) chunk of block_size * head_dim elements is
 *    contiguous ([VM] "PagedAttention的注意力计算流程": the K/V data inside a block
 *    is stored contiguously) and starts on a 256-byte boundary whenever the
 *    cache base is 256-byte aligned ([PA] §4.2 访存优化技术, address alignment).
 *  - Slot of a token: physical_block * block_size + offset_in_block
 *    ([PA] §3.2 块表与地址转换: logical block -> table -> physical id -> base + offset).
 *  - One dtype covers q, k, v, both caches and out; attention accumulates in fp32.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,      /* bad argument, shape, id or state                   */
  PA_ERR_UNSUPPORTED = -2,  /* dtype / head_dim / block_size / group outside the compiled set */
  PA_ERR_NO_BLOCKS = -3,    /* the free pool cannot cover the call; state unchanged */
  PA_ERR_HIP = -4           /* a HIP runtime call failed                            */
} pa_status;

/* Element types. PA_FP8_E4M3 and PA_INT8 are cache-only types, one byte per
 * element with one float32 scale per (block, head, token) row kept in a
 * separate array; the row's values are code * scale ([PA] §7 演进方向与优化空间:
 * FP8 / INT8 compressed blocks):
 *   PA_FP8_E4M3 - OCP FP8 E4M3 codes (bias 7, 3 mantissa bits, largest value
 *                 448, no infinities, 0x7F / 0xFF = NaN); scale = max|x| / 448;
 *   PA_INT8     - signed int8 codes in [-127, 127]; scale = max|x| / 127.
 * The "_fp8" calls below (kv_append_fp8, copy_blocks_fp8) serve both. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3, PA_INT8 = 4 } pa_dtype;

/* Message for the calling thread's last failed call ("" if none). */
const char* pa_last_error(void);

/* Geometry of one layer's K and V caches. */
typedef struct {
  int32_t num_blocks;    /* physical blocks in the pool                        */
  int32_t num_kv_heads;  /* KV heads                                           */
  int32_t block_size;    /* tokens per block: 8, 16 or 32                      */
  int32_t head_dim;      /* 64 or 128                                          */
  int32_t dtype;         /* pa_dtype                                           */
} pa_cache_desc;

/* Everything pa_decode needs besides the tensors themselves. */
typedef struct {
  pa_cache_desc cache;
  int32_t num_seqs;            /* S                                                    */
  int32_t num_q_heads;         /* Hq, a multiple of num_kv_heads; Hq/Hkv in {1,2,4,8}  */
  int32_t max_blocks_per_seq;  /* row stride of block_tables (compact tables: an upper
                                  bound on every row's length)                         */
  int32_t max_context_len;     /* host-known bound on every context_lens[s]; 0 = table
                                  capacity (max_blocks_per_seq * block_size). Sizes the
                                  launch and the workspace.                            */
  int32_t partition_size;      /* tokens per split-context partition, a multiple of
                                  block_size, at most 64 * block_size;
                                  0 = min(1024, 64 * block_size)                      */
  int32_t num_work;            /* items in `work` (ignored when work is NULL)           */
  void* workspace;             /* device scratch of pa_decode_workspace_bytes(desc)
                                  bytes; may be NULL when that size is 0               */
  size_t workspace_bytes;
  void* prof_events[2];        /* optional hipEvent_t pair (both or none) that take the
                                  partition kernel's start and end time on `stream`
                                  (launched with hipExtLaunchKernel, so no marker packet
                                  of their own sits between the kernels)              */
  const int32_t* work;         /* optional device launch schedule: int32 [num_work][8]
                                  items (sequence s, first token t0, token count n,
                                  slot, member offset, member count, row start, row
                                  length), made by pa_decode_schedule (which leaves
                                  the last two 0; they matter with compact_tables). An item attends over tokens
                                  [t0, t0 + n) of s (t0 a multiple of block_size,
                                  1 <= n <= 64 * block_size) and leaves its partial
                                  result in slot `slot` of s (and of each member).
                                  Each sequence's ranges - its own items and the
                                  shared items it is a member of - must tile
                                  [0, context_lens[s]) exactly, with slots
                                  0 .. num_slots[s] - 1; an empty or out-of-range
                                  context has one item (s, 0, 0, 0, ...). Items run in
                                  list order. NULL = the dense launch: partition p of
                                  every sequence is tokens [p * P, (p + 1) * P). A list
                                  that breaks the tiling leaves outputs undefined
                                  (PA_DEBUG=1 checks it on the host).                  */
  const int32_t* members;      /* device int32 [num_members]: for an item with member
                                  count c > 0, members[offset .. offset + c) are other
                                  sequences whose block tables hold the same physical
                                  blocks over the item's range; the item computes their
                                  partial results too, reading the blocks once.
                                  c < pa_decode_share_width() and Hq == Hkv are
                                  required; NULL = no sharing.                          */
  int32_t num_members;
  const int32_t* num_slots;    /* device int32 [S], required with `work`: partial results
                                  (ranges) of each sequence                            */
  int32_t max_slots;           /* host-known largest num_slots entry (0 = unknown); no
                                  merge pass runs when it is 1                          */
  int32_t q_dtype;             /* FP8 / INT8 caches only: dtype of q and out (PA_F16 or PA_BF16);
                                  otherwise q and out have the cache dtype             */
  const float* k_scale;        /* FP8 / INT8 caches only: float32 [num_blocks][Hkv][block_size]
                                  row scales of k_cache and v_cache (device)           */
  const float* v_scale;
  int32_t compact_tables;      /* non-zero: block_tables is int32 [table_entries], the
                                  tables of the sequences back to back, and every
                                  schedule item gives its sequence's row as entries
                                  [row start, row start + row length) (at least
                                  ceil(context_lens[s] / block_size) entries; every
                                  item of one sequence names the same row; members
                                  of a shared item read the leader's row). Needs
                                  `work`. A row outside the array poisons the item's
                                  outputs with NaN. 0: padded rows (the default).  */
  int32_t table_entries;       /* entries of a compact block_tables array              */
} pa_decode_desc;

/*
 * pa_decode - single-query paged attention for S sequences.
 *
 * Defines ([VM] "PagedAttention的注意力计算流程"; [KVM] Part 2 "PagedAttention 的核心思想"):
 * for sequence s and query head h, with KV head kv = h / (Hq / Hkv) and
 * context length n = context_lens[s], token t < n lives in physical block
 * block_tables[s][t / B] at offset t % B;
 *     score_t = scale * q[s][h] . K_t ,
 *     w = softmax(score)                       (maximum subtracted),
 *     out[s][h] = sum_t w_t * V_t .
 * The softmax is assembled from local pieces as in the five-step blockwise
 * scheme of [PA] §5.1 (local maxima, global maximum, shifted exponentials,
 * global sum, normalisation): inside each context partition of partition_size
 * tokens, batches of rows are folded into a running (maximum, sum, weighted
 * sum of V); across partitions a merge pass applies steps 2-5 to the
 * partitions' states (run only for sequences longer than one partition).
 *
 *   q             [S][Hq][d]                   device, dtype
 *   k_cache/v_cache                            device, layout above
 *   block_tables  int32 [S][max_blocks_per_seq] device; entries past
 *                 ceil(n / B) are ignored (pad with -1); the whole row must
 *                 be readable
 *   context_lens  int32 [S]                    device; 0 gives an all-zero row;
 *                 n < 0 or n > max_context_len (or the table capacity) gives NaN
 *   scale         softmax scale (1/sqrt(d) in the usual case)
 *   out           [S][Hq][d]                   device, dtype; fully overwritten
 *
 * Deterministic: the summation order depends only on logical token
 * positions, so the result is bit-identical for any placement of the blocks.
 */
int pa_decode(const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, float scale,
              void* out, const pa_decode_desc* desc, void* stream);

/*
 * pa_decode_noalloc - pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that must not call
 * hipMalloc, harnesses that forbid it). Arguments, results and errors are
 * those of pa_decode, except that desc->workspace and desc->workspace_bytes
 * are ignored: the partial results of a split launch go to a scratch array
 * the library holds on each GPU it runs on (pa_decode_noalloc_scratch_bytes(),
 * 16 MiB, kept until the process ends). A launch whose workspace
 * (pa_decode_workspace_bytes) exceeds it is refused with PA_ERR_INVALID.
 * Nothing is allocated on any call; the first call on a device looks up that
 * device's scratch address. All calls on one GPU share its scratch, which
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls that overlap on one GPU - on two streams, or from two threads
 * without ordering - race and give undefined results.
 */
int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      void* out, const pa_decode_desc* desc, void* stream);

/* Bytes of the scratch pa_decode_noalloc uses (the largest workspace it takes). */
size_t pa_decode_noalloc_scratch_bytes(void);

/* Bytes of workspace pa_decode needs for `desc` (fp32 partial max and sum,
 * and the partial output in the output dtype, per sequence, query head and
 * slot: one slot per partition, plus one with a schedule). `scheduled`
 * non-zero sizes it for a launch with a schedule (desc->work non-NULL), zero
 * for the dense launch; desc->work itself is not read. 0 for a dense launch
 * whose contexts fit one partition.
 * Returns 0 and sets pa_last_error for an invalid desc. */
size_t pa_decode_workspace_bytes(const pa_decode_desc* desc, int32_t scheduled);

/* Most sequences one shared schedule item serves (the item's own + members). */
int32_t pa_decode_share_width(void);

/*
 * pa_decode_schedule - a launch schedule for pa_decode from host context
 * lengths and block tables (int32 [num_seqs][max_blocks_per_seq], host memory;
 * may be NULL when share_width is 1).
 *
 * Each sequence's context is tiled into ranges of at most partition_size
 * tokens (0 = the pa_decode default). With share_width > 1 (at most
 * pa_decode_share_width()), up to share_width sequences whose tables start
 * with the same physical blocks - a prompt shared by forked beams or parallel
 * samples ([VM] "写时复制与块共享机制") - form a group: the run of whole blocks
 * they all hold is tiled once, as items whose members are the other sequences,
 * so those blocks are read once for the group ([PA] §5.2 logical regrouping:
 * queries that hit the same physical block are handled together); each
 * sequence's own tokens follow. Order, longest first: shared items, the other
 * ranges by decreasing length, then one (s, 0, 0, 0, ...) item per sequence
 * whose length is <= 0 or above max_context_len (when that is > 0). Launching
 * only real ranges, longest first, leaves no idle workgroups and the shortest
 * tail ([PA] §3.2 batches requests with the same access pattern). Without
 * sharing the ranges are exactly the dense launch's partitions.
 *
 * Writes int32 [n][8] items to out_work, the member list to out_members
 * (*out_num_members entries), each sequence's range count to out_num_slots
 * (int32 [num_seqs]) and the largest to *out_max_slots - all host memory.
 * Returns n, or -1 (and pa_last_error) for bad arguments or capacities below
 * what is needed.
 */
int32_t pa_decode_schedule(const int32_t* context_lens, const int32_t* block_tables, int32_t num_seqs,
                           int32_t max_blocks_per_seq, int32_t block_size, int32_t partition_size,
                           int32_t max_context_len, int32_t share_width, int32_t* out_work,
                           int32_t capacity, int32_t* out_members, int32_t member_capacity,
                           int32_t* out_num_members, int32_t* out_num_slots, int32_t* out_max_slots);

/* 1 if pa_decode has a kernel for this (dtype, head_dim, block_size, Hq/Hkv). */
int pa_decode_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group);

/* 1 if pa_decode has a kernel for q/out of q_dtype over a cache of cache_dtype
 * (the same dtype, or PA_FP8_E4M3 / PA_INT8 codes under PA_F16 / PA_BF16 queries). */
int pa_decode_supported_kv(int32_t q_dtype, int32_t cache_dtype, int32_t head_dim, int32_t block_size,
                           int32_t group);

/*
 * kv_append - write new tokens' K and V rows into their slots
 * ([PA] §3.3 按需分配策略, step 4: write the new token's K/V vectors).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim]   device, dtype
 *   slot_mapping  int64 [num_tokens]                     device-accessible (device or pinned
 *                                                        host memory); -1 = skip the token
 *   k_cache/v_cache                                      device, layout above
 * For every token i with slot >= 0, every head's row goes to block
 * slot / B, offset slot % B. Bitwise copy. Slots must be distinct within one
 * call; slots >= num_blocks * B are skipped (PA_DEBUG=1: PA_ERR_INVALID).
 */
int kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
              void* k_cache, void* v_cache, const pa_cache_desc* desc, void* stream);

/*
 * kv_append_staged - kv_append and pa_stage_copy in one launch: copies
 * stage_bytes from stage_src to the device buffer stage_dst (as pa_stage_copy)
 * and writes the new tokens' K/V rows (as kv_append). slot_mapping may point
 * into stage_src's pinned host memory (the kernel reads it there), so a decode
 * step's upload and append cost one kernel launch. The staged bytes must not
 * overlap the caches, k, v or slot_mapping; stage_bytes may be 0.
 */
int kv_append_staged(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                     void* k_cache, void* v_cache, const pa_cache_desc* desc, void* stage_dst,
                     const void* stage_src, size_t stage_bytes, void* stream);

/*
 * kv_append_fp8 - write new tokens' K and V rows into an FP8 or INT8 cache,
 * quantised ([PA] §7: historical blocks stored as FP8 / INT8; [VM]
 * "PagedAttention的工程实践与局限": quantised KV values in the blocks).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim]   device, src_dtype (f32/f16/bf16)
 *   slot_mapping  int64 [num_tokens], device-accessible; -1 = skip
 *   k_cache/v_cache  one-byte codes [num_blocks][Hkv][B][d]  device (desc->dtype
 *                 PA_FP8_E4M3 or PA_INT8)
 *   k_scale/v_scale  float32 [num_blocks][Hkv][B]          device
 * Each (token, head) row x is stored as one float32 scale and d codes. FP8:
 * scale = max|x| / 448 (correctly rounded; 0 for an all-zero row) and codes
 * E4M3(clamp(x / scale, -448, 448)) rounded to nearest, ties to even. INT8:
 * scale = max|x| / 127 and codes x / scale rounded to nearest, ties to even,
 * in [-127, 127]. All codes are 0 when the scale is 0; the stored values are
 * code * scale. head_dim 64 or 128; inputs must be finite.
 * k, v and both code caches must be 16-byte aligned, slot_mapping 8-byte and
 * the scale arrays 4-byte aligned (PA_ERR_INVALID otherwise).
 * As kv_append_staged, stage_bytes (may be 0) are copied from stage_src
 * (pinned host or device) to stage_dst in the same launch.
 */
int kv_append_fp8(const void* k, const void* v, int32_t src_dtype, const int64_t* slot_mapping,
                  int32_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                  const pa_cache_desc* desc, void* stage_dst, const void* stage_src, size_t stage_bytes,
                  void* stream);

/*
 * copy_blocks_fp8 - copy_blocks for an FP8 or INT8 cache: whole blocks of codes and
 * of their row scales (same pair rules as copy_blocks). Hkv * B must be a
 * multiple of 4 and the scale arrays 16-byte aligned.
 */
int copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int64_t* src_dst_pairs,
                    int32_t num_pairs, const pa_cache_desc* desc, void* stream);

/*
 * copy_blocks - whole-block copies for copy-on-write
 * ([VM] "写时复制与块共享机制"; [PA] §4.1: allocate a new block, copy the original
 * data, remap, drop the old block's count).
 *
 *   src_dst_pairs int64 [num_pairs][2]   device-accessible (device or pinned host memory);
 *                                        (src, dst) physical block ids
 * For each pair, K[dst] <- K[src] and V[dst] <- V[src]: every head and every
 * slot of the block, bitwise. Destinations must be distinct and must not also
 * be sources within one call (pairs are then independent and run in
 * parallel); out-of-range ids are skipped (PA_DEBUG=1: PA_ERR_INVALID).
 */
int copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int32_t num_pairs,
                const pa_cache_desc* desc, void* stream);

/* Direction of swap_blocks. */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

/*
 * swap_blocks - whole-block moves between the device cache and a swap space
 * ([VM] "显存管理与调度策略设计": under sustained memory pressure the blocks of a
 * waiting request go to CPU memory, and come back to the GPU when the request
 * is scheduled again).
 *
 *   k_cache/v_cache, desc     the device cache (layout above)
 *   k_scale/v_scale           float32 [num_blocks][Hkv][B] for an FP8 / INT8 cache, else NULL
 *   swap_k/swap_v             [swap_num_blocks][Hkv][B][d], the cache's element type (uint8
 *                             codes for FP8 / INT8): pinned host memory (hipHostMalloc'd; the
 *                             kernel reads or writes it over the bus) or device memory
 *   swap_k_scale/swap_v_scale float32 [swap_num_blocks][Hkv][B] for FP8 / INT8, else NULL
 *   src_dst_pairs int64 [num_pairs][2], device-accessible:
 *     PA_SWAP_OUT  (device block, swap block): swap[dst] <- cache[src]
 *     PA_SWAP_IN   (swap block, device block): cache[dst] <- swap[src]
 * Every head and slot of K and V (and of the FP8 / INT8 scales), bitwise, in one
 * launch per array pair on `stream`. Destinations must be distinct within one
 * call; out-of-range ids are skipped (PA_DEBUG=1: PA_ERR_INVALID). The pairs
 * are what pa_alloc_swap_out / pa_alloc_swap_in return. Host memory written
 * by PA_SWAP_OUT is complete once the stream has been synchronised.
 */
int swap_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const pa_cache_desc* desc,
                void* swap_k, void* swap_v, float* swap_k_scale, float* swap_v_scale, int32_t swap_num_blocks,
                const int64_t* src_dst_pairs, int32_t num_pairs, int32_t direction, void* stream);

/*
 * pa_stage_copy - copy `bytes` from src to the device buffer dst with a kernel
 * on `stream`. src may be pinned host memory (hipHostMalloc'd; the kernel
 * reads it over the bus), so a decode step's slots, copy pairs, block tables
 * and context lengths - written by pa_alloc_step into one pinned buffer
 * ([PA] §3.2: the flattened block table) - reach the device in stream order
 * without a hand-off to a copy engine. Both pointers and `bytes` must be
 * multiples of 16; the buffers must not overlap. src must stay unchanged
 * until the copy has run (the caller's event or stream synchronisation).
 */
int pa_stage_copy(void* dst, const void* src, size_t bytes, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator. Host memory only; no HIP call. Not thread-safe: one
 * handle per thread, or external locking.
 *
 * Rules: the free pool is a FIFO queue - allocation pops its head, a freed
 * block returns to its tail (a doubly-linked list, so a prefix-cache hit can
 * also take a block from its middle) ([VM] "Python 演示"; [KVM] Part 4 BlockPool). A block
 * has a reference count; a sequence's block table lists its physical blocks
 * in logical order ([PA] §3.2). Calls that need blocks are all-or-nothing:
 * if the pool cannot cover them they return PA_ERR_NO_BLOCKS and change
 * nothing ([KVM] Part 4 allocate_slots; [VM] "Python 演示" raises on an empty pool).
 * ---------------------------------------------------------------------- */
typedef struct pa_allocator pa_allocator;

/* New allocator over blocks 0..num_blocks-1. initial_free_order (nullable)
 * gives the initial queue order and must be a permutation of 0..num_blocks-1;
 * NULL means 0, 1, ..., num_blocks-1. The handle is owned by the caller. */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_free_order,
                    pa_allocator** out);
void pa_alloc_destroy(pa_allocator* a);

/* New sequence holding num_tokens tokens: ceil(num_tokens / B) blocks from
 * the head of the queue, each with count 1. */
int pa_alloc_add_seq(pa_allocator* a, int64_t seq_id, int32_t num_tokens);

/* Child shares every block of the parent: same table, each count + 1, same
 * context length ([VM] "写时复制与块共享机制"). */
int pa_alloc_fork(pa_allocator* a, int64_t parent_id, int64_t child_id);

/*
 * One new token for each of the n listed (distinct) sequences, in the given
 * order ([PA] §3.3 on-demand growth; [VM] "写时复制与块共享机制" copy-on-write):
 *   pos = context length; if pos % B == 0 a new block is taken from the queue
 *   head and appended to the table; otherwise, if the last block's count is
 *   above 1, a new block is taken, (last, new) is recorded as a copy, the old
 *   count drops by one and the table entry is remapped; a count of 1 writes in
 *   place. out_slots[i] = table[pos / B] * B + pos % B; context length + 1.
 * out_cow_pairs receives *out_num_cow (src, dst) pairs (int64, row-major
 * [cow_capacity][2]); at most n pairs are produced, and PA_ERR_INVALID is
 * returned (nothing changed) if cow_capacity is smaller than the number needed.
 */
int pa_alloc_append_slots(pa_allocator* a, const int64_t* seq_ids, int32_t n, int64_t* out_slots,
                          int64_t* out_cow_pairs, int32_t cow_capacity, int32_t* out_num_cow);

/* Longest block table among the n listed sequences, counted as after
 * pa_alloc_append_slots for them when `append` is non-zero (nothing changes).
 * -1 (and pa_last_error) for an unknown or repeated sequence. Sizes the
 * `max_blocks` of pa_alloc_step. */
int32_t pa_alloc_table_width(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append);

/*
 * One decode step's host work in one call, for a runtime that stages it to the
 * device in a single copy: when `append` is non-zero, exactly
 * pa_alloc_append_slots for the n listed sequences (out_slots, out_cow_pairs,
 * out_num_cow as there); then, as pa_alloc_block_tables, their tables padded
 * with -1 to max_blocks columns (out_tables, row-major [n][max_blocks] int32)
 * and context lengths (out_context_lens, int32 [n]); *out_max_context gets the
 * largest context length. Output pointers other than out_slots (with append)
 * may be NULL. All-or-nothing: PA_ERR_NO_BLOCKS, or PA_ERR_INVALID for a table
 * longer than max_blocks after the append or too small a cow_capacity, leave
 * the state unchanged.
 */
int pa_alloc_step(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, int32_t max_blocks,
                  int64_t* out_slots, int64_t* out_cow_pairs, int32_t cow_capacity, int32_t* out_num_cow,
                  int32_t* out_tables, int32_t* out_context_lens, int32_t* out_max_context);

/* Release a finished sequence: every block of its table loses one count, in
 * ascending logical order; a block reaching 0 goes to the tail of the queue
 * ([VM] "写时复制与块共享机制"). */
int pa_alloc_free_seq(pa_allocator* a, int64_t seq_id);

/* Slots of positions [start, start + count) of a sequence, into out_slots. */
int pa_alloc_seq_slots(const pa_allocator* a, int64_t seq_id, int32_t start, int32_t count,
                       int64_t* out_slots);

/* Block tables of the n listed sequences, row-major [n][max_blocks] int32 padded
 * with -1, and their context lengths. PA_ERR_INVALID if a table is longer than
 * max_blocks. Either output may be NULL. */
int pa_alloc_block_tables(const pa_allocator* a, const int64_t* seq_ids, int32_t n,
                          int32_t max_blocks, int32_t* out_tables, int32_t* out_context_lens);

/* State queries (for schedulers and for bit-exact checks). */
int32_t pa_alloc_num_free(const pa_allocator* a);
int32_t pa_alloc_num_blocks(const pa_allocator* a);
int32_t pa_alloc_ref_count(const pa_allocator* a, int32_t block);      /* -1 if out of range */
int32_t pa_alloc_context_len(const pa_allocator* a, int64_t seq_id);   /* -1 if unknown */
int32_t pa_alloc_num_table_blocks(const pa_allocator* a, int64_t seq_id); /* -1 if unknown */
/* Copies min(cap, num_free) queue entries, head first; returns num_free. */
int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap);

/*
 * Swap space ([VM] "显存管理与调度策略设计": a waiting request's blocks can be
 * evicted to CPU memory and restored when it is scheduled again). A second
 * FIFO pool of swap_num_blocks host-side block ids, with the same queue rules.
 * A swapped-out sequence keeps its context length; its table then lists swap
 * blocks, and append, step, fork, seq_slots and block_tables reject it
 * (PA_ERR_INVALID) until it is swapped in.
 *
 * pa_alloc_set_swap_space: (re)create the swap pool over ids
 *   0..num_blocks-1, queue order initial_free_order (nullable, a permutation)
 *   as for pa_alloc_create. PA_ERR_INVALID while a sequence is swapped out.
 * pa_alloc_swap_out: for each table entry j in logical order, take a swap
 *   block from the swap queue head, record (device block, swap block) in
 *   out_pairs[j] (int64 [capacity][2]), and drop the device block's count by
 *   one (a block reaching 0 goes to the tail of the device queue; one that
 *   other sequences share stays with them). The caller moves the data with
 *   swap_blocks(PA_SWAP_OUT) before it lets a later call reuse the freed
 *   blocks. Each swapped sequence gets its own copy of every block it shared.
 * pa_alloc_swap_in: for each swap block in logical order, take a device
 *   block from the device queue head (count 1), record (swap block, device
 *   block), and return the swap block to the swap queue tail; then
 *   swap_blocks(PA_SWAP_IN).
 * Both are all-or-nothing: PA_ERR_NO_BLOCKS when the target pool has fewer
 * free blocks than the table has entries, PA_ERR_INVALID when capacity is
 * smaller or the sequence is not in the required state; *out_num (nullable)
 * receives the pair count. pa_alloc_free_seq of a swapped-out sequence returns
 * its swap blocks to the swap queue tail.
 */
int pa_alloc_set_swap_space(pa_allocator* a, int32_t num_blocks, const int32_t* initial_free_order);
int pa_alloc_swap_out(pa_allocator* a, int64_t seq_id, int64_t* out_pairs, int32_t capacity, int32_t* out_num);
int pa_alloc_swap_in(pa_allocator* a, int64_t seq_id, int64_t* out_pairs, int32_t capacity, int32_t* out_num);
int32_t pa_alloc_num_free_swap(const pa_allocator* a);
/* Copies min(cap, free swap blocks) swap-queue entries, head first; returns the free count. */
int32_t pa_alloc_swap_free_list(const pa_allocator* a, int32_t* out, int32_t cap);
int32_t pa_alloc_is_swapped(const pa_allocator* a, int64_t seq_id);  /* 1, 0, or -1 if unknown */
/* A sequence's table as it stands (device block ids, or swap block ids while
 * swapped out): copies min(cap, length) entries; returns the length, -1 if unknown. */
int32_t pa_alloc_seq_table(const pa_allocator* a, int64_t seq_id, int32_t* out, int32_t cap);

/*
 * Automatic prefix caching ([KVM] Part 3 "APC 的工作机制", "哈希链的设计"; Part 4
 * FreeKVCacheBlockQueue, BlockPool, allocate_slots). Optional; off by default.
 *
 * A full block of a prompt is indexed by a chained 64-bit hash of the
 * previous block's hash, an extra key (an adapter id, or any other value
 * that must not be shared across) and its tokens; the index entry also keeps
 * that parent hash, extra key and the tokens, and a lookup compares them, so
 * blocks are shared only when the tokens of every block up to and including
 * them match. Only full prompt blocks are indexed.
 *
 * pa_alloc_enable_prefix_caching: turn it on (PA_ERR_INVALID once any sequence
 *   exists). Blocks of finished sequences then return to the free queue still
 *   indexed; a block taken from the queue head drops its index entry first.
 * pa_alloc_add_seq_cached: a new sequence for the prompt tokens[0..n) (int32
 *   token ids, host memory): the longest run of leading full blocks found in
 *   the index is reused - a free one leaves the queue from wherever it sits
 *   (O(1)), one in use gains a count - the rest come from the queue head, and
 *   the prompt's full blocks past the run are indexed. *out_cached_tokens
 *   (nullable) = reused blocks * B: the caller writes K/V only for positions
 *   from there on. All-or-nothing (PA_ERR_NO_BLOCKS changes nothing).
 * pa_alloc_prefix_hits: the same lookup without allocating; copies
 *   min(cap, hits) block ids to out_blocks (nullable); returns the number of
 *   leading blocks found, or -1 for bad arguments. 0 when caching is off.
 * pa_alloc_num_cached_blocks: index entries; pa_alloc_block_is_cached: 1 if
 *   the block holds one, 0 if not, -1 for an id out of range.
 */
int pa_alloc_enable_prefix_caching(pa_allocator* a);
int pa_alloc_add_seq_cached(pa_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t num_tokens,
                            int64_t extra_key, int32_t* out_cached_tokens);
int32_t pa_alloc_prefix_hits(const pa_allocator* a, const int32_t* tokens, int32_t num_tokens, int64_t extra_key,
                             int32_t* out_blocks, int32_t cap);
int32_t pa_alloc_num_cached_blocks(const pa_allocator* a);
int32_t pa_alloc_block_is_cached(const pa_allocator* a, int32_t block);

/*
 * pa_alloc_admit - admit n prompts in order in one call, for a batched
 * prefill whose K/V rows lie back to back: prompt i (sequence seq_ids[i],
 * lengths[i] tokens) is pa_alloc_add_seq_cached with its token ids taken
 * from `tokens` (all prompts' ids concatenated, host int32) and extra key
 * extra_keys[i] (nullable: 0), or pa_alloc_add_seq when `tokens` is NULL.
 * out_slots (int64 [sum(lengths)], host) receives every position's slot, -1
 * inside a cached prefix and for prompts not admitted, so it can be handed to
 * kv_append unchanged; out_cached[i] (nullable) the cached-prefix length.
 * Prompts are admitted one by one: at the first that does not fit the call
 * stops and returns its status (PA_ERR_NO_BLOCKS, or PA_ERR_INVALID for a
 * repeated id), and *out_admitted (nullable) says how many went in; those
 * stay admitted.
 */
int pa_alloc_admit(pa_allocator* a, const int64_t* seq_ids, int32_t n, const int32_t* tokens,
                   const int32_t* lengths, const int64_t* extra_keys, int64_t* out_slots, int32_t* out_cached,
                   int32_t* out_admitted);

/* Watermark ([VM] "显存管理与调度策略设计": keep a reserve of free blocks, e.g. 5%).
 * can_allocate(n) is 1 when taking n blocks leaves at least fraction * num_blocks
 * free, else 0. The watermark is advisory: allocation calls do not consult it. */
int pa_alloc_set_watermark(pa_allocator* a, double fraction);
int pa_alloc_can_allocate(const pa_allocator* a, int32_t num_blocks);

/* ------------------------------------------------------------------------
 * One decode step in one call ([PA] §3.3 on-demand allocation then the new
 * token's K/V write; [VM] "写时复制与块共享机制" copy before write): the host
 * allocator's step, the launch schedule, and the copy / append / attention
 * launches on one stream, with the step's small inputs staged in one buffer.
 * ---------------------------------------------------------------------- */

/* Byte offsets (256-aligned) of the regions of the step buffer, in this
 * order: slots int64 [n] | copy pairs int64 [n][2] | context lengths int32
 * [n] | ranges per sequence int32 [n] | members int32 [n] | schedule int32
 * [work_capacity][8] | block tables int32 [n][width]. The allocator writes
 * padded tables at `tables`; the step then packs them back to back right
 * after the schedule items it made (16-byte aligned), and uploads only the
 * buffer's prefix up to the end of the packed tables. */
typedef struct {
  size_t slots, pairs, tables, context_lens, work, members, num_slots;
  size_t total;              /* bytes of the whole buffer (a multiple of 256)       */
  int32_t num_seqs;          /* n                                                   */
  int32_t width;             /* table columns: >= the longest table after the step  */
  int32_t work_capacity;     /* schedule items the buffer holds (enough for any step) */
  int32_t partition_size;    /* the effective partition size in tokens              */
} pa_step_layout_t;

/* Layout for n sequences, tables of `width` columns, blocks of block_size
 * tokens and partition_size (0 = the default). */
int pa_step_layout(int32_t num_seqs, int32_t width, int32_t block_size, int32_t partition_size,
                   pa_step_layout_t* out);

typedef struct {
  pa_cache_desc cache;       /* the device caches                                   */
  int32_t num_q_heads;       /* Hq                                                  */
  int32_t q_dtype;           /* dtype of q, out and the new K/V rows (the cache dtype,
                                or PA_F16 / PA_BF16 over an FP8 / INT8 cache)        */
  int32_t share_width;       /* 1 .. pa_decode_share_width(); 1 = no shared items    */
  int32_t schedule;          /* non-zero: longest-first launch schedule; 0: dense     */
  float scale;               /* softmax scale                                       */
  float* k_scale;            /* FP8 / INT8 caches: row scales (device), else NULL   */
  float* v_scale;
  void* workspace;           /* device scratch (16-byte aligned): at least
                                pa_decode_workspace_bytes of a desc with
                                max_context_len 0 (the table capacity of layout.width
                                columns), scheduled = `schedule`                      */
  size_t workspace_bytes;
  void* prof_events[2];      /* optional hipEvent_t pair around the partition kernel */
  pa_step_layout_t layout;   /* from pa_step_layout                                 */
  void* host_stage;          /* pinned host buffer of layout.total bytes; this call
                                writes it, the launches read it: the caller must not
                                rewrite it before they have run                       */
  void* dev_stage;           /* device buffer of layout.total bytes                   */
  uint64_t* done_flag;       /* optional word of pinned host memory: as this step's
                                staging launch (kv_append_staged / kv_append_fp8 / the
                                upload alone) starts, one of its threads stores
                                done_value there with a system-scope store. Kernels on
                                one stream run one after another, so from then on
                                every launch enqueued on `stream` before this call has
                                completed - earlier steps' host_stage buffers may be
                                rewritten - and a host that polls the word learns it
                                without an event or a marker packet on the stream. A
                                call that fails before that launch leaves it unset.
                                8-byte aligned; NULL = none                         */
  uint64_t done_value;
} pa_step_desc;

/* What the host half of a decode step leaves for its launches. */
typedef struct {
  int32_t num_cow;           /* copy-on-write pairs written at layout.pairs          */
  int32_t num_work;          /* schedule items at layout.work (0 without `schedule`) */
  int32_t num_members;       /* member entries at layout.members                     */
  int32_t max_slots;         /* largest ranges-per-sequence count                    */
  int32_t max_context;       /* longest context after the step (at least 1)          */
  int32_t table_entries;     /* packed table entries (with `schedule`)               */
  size_t tables_at;          /* byte offset of the tables the decode reads           */
  size_t upload_bytes;       /* prefix of host_stage that goes to the device         */
} pa_step_plan_t;

/*
 * pa_decode_step_plan - the host half of pa_decode_step, nothing launched:
 * the allocator step for the n listed sequences (exactly pa_alloc_step, one
 * token each with `append`), the launch schedule and the packed tables, all
 * written into d->host_stage at the offsets of d->layout ([PA] §3.3 on-demand
 * allocation; [PA] §3.2 the table a kernel walks). Only d->cache, layout,
 * share_width, schedule and host_stage (16-byte aligned) are read.
 * Refusals (PA_ERR_INVALID for bad arguments or a table longer than
 * layout.width, PA_ERR_NO_BLOCKS) leave the allocator unchanged.
 */
int pa_decode_step_plan(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append,
                        const pa_step_desc* d, pa_step_plan_t* plan);

/*
 * pa_decode_step - one decode step for the n listed (distinct) sequences:
 * pa_decode_step_plan, then the launches. With `append`, exactly
 * pa_alloc_append_slots for them; the copy-on-write
 * copies run (copy_blocks / copy_blocks_fp8, pairs read from host_stage),
 * then the new rows k_new / v_new [n][Hkv][d] (device, q_dtype) are written
 * (kv_append_staged / kv_append_fp8), in the same launch as the upload of the
 * staged tables, lengths and schedule to dev_stage. Without `append`, only the
 * upload. Then pa_decode of q [n][Hq][d] into out over every listed sequence.
 * With `schedule`, the tables travel packed (compact_tables of pa_decode), so
 * the upload carries about 4 bytes per block in use rather than the padded
 * n * width; without it, padded.
 * *out_max_context (nullable) gets the longest context.
 *
 * Refusals that leave the allocator unchanged: PA_ERR_NO_BLOCKS; PA_ERR_INVALID
 * for bad arguments (NULL or misaligned pointers - every pointer 16-byte
 * aligned, done_flag 8-byte aligned -, a q_dtype that does not go with the
 * cache dtype, a non-finite scale), a table longer than layout.width, or a
 * workspace that is too small;
 * PA_ERR_UNSUPPORTED for a shape no kernel covers. Every check the launches
 * make is done before the allocator step, so a launch error (PA_ERR_HIP) is
 * the only failure that leaves the allocator advanced.
 */
int pa_decode_step(pa_allocator* a, const int64_t* seq_ids, int32_t n, int32_t append, const void* k_new,
                   const void* v_new, const void* q, void* out, void* k_cache, void* v_cache,
                   const pa_step_desc* desc, void* stream, int32_t* out_max_context);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
