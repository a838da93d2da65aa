// Paged single-query decode attention for gfx950 (CDNA4): partition pass +
// merge pass, and the pa_decode C ABI entry point.
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//   [KVM] "深入解析 vLLM 的 KV Cache 管理器：从内存碎片到 PagedAttention 的完整技术剖析"
//
// What is computed ([VM] "PagedAttention的注意力计算流程"; [KVM] Part 2): for each
// sequence and query head, walk the sequence's physical blocks through its
// block table, take q.K for every token, softmax over them, and sum the V rows
// weighted by the softmax. The softmax is assembled from local pieces as in the
// five steps of [PA] §5.1: local maxima, the global maximum, exponentials
// shifted by it, the global sum, and the division. Inside a context partition
// (1024 tokens, at most 64 blocks, by default) each wave folds batches of rows into a running
// (maximum, sum, weighted sum) - the local maximum of a batch, rescaling to the
// new maximum, then the batch's shifted exponentials - and the waves' states
// are merged the same way at the end. For sequences longer than one partition
// the merge kernel applies steps 2-5 across the partitions' (max, sum, output).
//
// Mapping onto CDNA4 (not a translation of the pages' shared-memory / 32-lane
// warp design):
//   * one workgroup of NW wave64s per (KV head, sequence, partition); it serves
//     the G query heads that share the KV head, so each K/V byte is read once;
//   * a token row of one head (head_dim * elem bytes, 256 B for fp16 d=128 or
//     fp32 d=64) is read by LPR lanes with one 16-byte load each; one wave
//     load instruction covers 64 * 16 B = 1 KiB, i.e. RPC consecutive rows of
//     one (block, head) chunk, which is contiguous in the cache layout - fully
//     coalesced whatever the physical block order;
//   * K and V of a batch of U chunks are loaded together (2U KiB in flight per
//     wave) and never staged: registers only, LDS holds just the final
//     cross-wave combine;
//   * the partition's physical block ids are loaded once per wave into one
//     VGPR (lane j holds logical block j) and moved to SGPRs with v_readlane,
//     so every K/V address is scalar base + lane offset ("hoisted" block-table
//     lookup, [PA] §3.2); the ids come from a padded table row or, with a
//     schedule, from a packed array of rows whose start each item carries;
//   * FP8 / INT8 caches: a lane loads 8 codes, or 16 (one 16-byte load, 8
//     lanes per row) when the workgroup serves one query vector at head_dim
//     128; codes are widened exactly to the query's 16-bit type for dot2 (FP8
//     by the hardware convert, INT8 by a byte permute into the mantissa of an
//     f16 and one subtract) and to fp32 for the V sums; row scales multiply
//     the score (K) and the softmax weight (V);
//   * q.k: fp16 / bf16 dot2 instructions with fp32 accumulation, then a
//     row reduction over the LPR lanes with DPP (quad_perm, row_half_mirror,
//     row_mirror) - no LDS traffic; the batch maximum across rows uses
//     cross-row lane swaps;
//   * each lane accumulates 2^(s - m) * V for its 16-byte column slice in
//     fp32 registers; rows and waves are combined once at the end in a fixed
//     order, so the result depends only on logical positions (bitwise
//     identical for any block placement);
//   * rows past the context are never fetched (the last block is read only up
//     to the chunk holding the last token);
//   * the pass stays bound by HBM: per (token, KV head) it reads 2*d*elem
//     bytes and does 4*G*d flops, i.e. 2G/elem flop/byte (0.5 - 4), far below
//     the ~20 flop/byte where the vector ALUs would stop being fed by 8 TB/s;
//   * with four query heads per KV head (16-bit cache, head_dim 128) the
//     scores of a 16-row tile are one small dense product, K (16 x 128) times
//     q^T (128 x 4), and go to the matrix cores (16 x 16 x 32 MFMA, the four
//     heads repeated over its 16 columns). That is not for flops: it removes
//     the dot2 + DPP row sums that made this the one form whose vector ALUs
//     were busy enough to slow the stream. K is loaded as whole rows like V
//     and regrouped for the MFMA operand through a per-wave LDS tile; the
//     weighted V sums stay on the vector ALUs.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "internal.h"
#include "pagedkv.h"
#include "status.h"

namespace pagedkv {
namespace {

constexpr int kWave = 64;
// Compile-time tuning knobs (the defaults are the measured best on MI355X).
#ifndef PA_NUM_WAVES
#define PA_NUM_WAVES 4        // waves per partition workgroup
#endif
#ifndef PA_UNROLL
#define PA_UNROLL 12          // chunks per batch (each chunk: 1 KiB of K and 1 KiB of V per wave)
#endif
#ifndef PA_UNROLL_FP8
#define PA_UNROLL_FP8 8       // chunks per batch for FP8 caches (each chunk: 512 B of K and of V per wave)
#endif
#ifndef PA_FP8_WIDE_NQ
#define PA_FP8_WIDE_NQ 1      // FP8, head_dim 128: lanes hold 16 codes when a workgroup serves at most this many query vectors
#endif
#ifndef PA_UNROLL_FP8_WIDE
#define PA_UNROLL_FP8_WIDE 4  // chunks per batch for FP8 caches in the wide form (1 KiB of K and of V per wave)
#endif
#ifndef PA_FP8_WIDE_MIN_WGS
#define PA_FP8_WIDE_MIN_WGS 5 // workgroups per CU the wide FP8 form must fit (1: no constraint)
#endif
#ifndef PA_UNROLL_GQA
#define PA_UNROLL_GQA 8       // chunks per batch when one workgroup serves 4 or more query heads of a KV head
                              // outside the matrix-core form (more would take g = 8 past 256 registers)
#endif
#ifndef PA_UNROLL_SHARED
#define PA_UNROLL_SHARED 4    // chunks per batch in shared-prefix items (four query sets per chunk)
#endif
#ifndef PA_MFMA_TILES
#define PA_MFMA_TILES 2       // 16-row tiles per batch in that form (each tile: 4 KiB of K and of V per wave)
#endif
constexpr int kNumWaves = PA_NUM_WAVES;
constexpr int kUnroll = PA_UNROLL;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  void* ws_o;           // [S][Hq][slot_stride][D] normalised partial outputs, in the output dtype
  float2* ws_ml;        // [S][Hq][slot_stride] (max in log2 units, sum)
  float scale_log2;     // softmax scale * log2(e): scores are kept in log2 units
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t partition_size;
  int32_t max_partitions;
  int32_t slot_stride;  // partial-result slots per (sequence, query head) in the workspace
  const int32_t* work;  // optional launch schedule: kItemInts ints per item (see pa_decode_desc)
  int32_t num_work;
  const int32_t* members;   // sequences sharing a scheduled item's token range
  int32_t num_members;
  const int32_t* num_slots; // with a schedule: partial results per sequence
  const float* k_scale;     // FP8 caches: one scale per (block, head, token) row
  const float* v_scale;
  int32_t compact_tables;   // non-zero: block_tables holds the rows back to back; a
                            // scheduled item's ints 6 and 7 give its sequence's row
  int32_t table_entries;    // entries of the compact array
};

// ---------------------------------------------------------------------------
// element formats
// ---------------------------------------------------------------------------
template <int DT> struct Fmt;
template <> struct Fmt<PA_F32> { static constexpr int kBytes = 4; };
template <> struct Fmt<PA_F16> { static constexpr int kBytes = 2; };
template <> struct Fmt<PA_BF16> { static constexpr int kBytes = 2; };
template <> struct Fmt<PA_FP8_E4M3> { static constexpr int kBytes = 1; };
template <> struct Fmt<PA_INT8> { static constexpr int kBytes = 1; };
// one-byte codes with a float32 scale per row
template <int KT> constexpr bool kQuantized = KT == PA_FP8_E4M3 || KT == PA_INT8;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16 bytes of q (one lane's column slice of one head) dotted with 16 bytes of K.
template <int DT> __device__ __forceinline__ float dot16(const uint4& q, const uint4& k);
template <> __device__ __forceinline__ float dot16<PA_F16>(const uint4& q, const uint4& k) {
  float acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.x), __builtin_bit_cast(half2_t, k.x), 0.0f, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.y), __builtin_bit_cast(half2_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.z), __builtin_bit_cast(half2_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q.w), __builtin_bit_cast(half2_t, k.w), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float dot16<PA_BF16>(const uint4& q, const uint4& k) {
  float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.x), __builtin_bit_cast(bf162_t, k.x), 0.0f, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.y), __builtin_bit_cast(bf162_t, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.z), __builtin_bit_cast(bf162_t, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, q.w), __builtin_bit_cast(bf162_t, k.w), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float dot16<PA_F32>(const uint4& q, const uint4& k) {
  float acc = __builtin_bit_cast(float, q.x) * __builtin_bit_cast(float, k.x);
  acc = fmaf(__builtin_bit_cast(float, q.y), __builtin_bit_cast(float, k.y), acc);
  acc = fmaf(__builtin_bit_cast(float, q.z), __builtin_bit_cast(float, k.z), acc);
  acc = fmaf(__builtin_bit_cast(float, q.w), __builtin_bit_cast(float, k.w), acc);
  return acc;
}

// The 16 bytes of V as fp32 values.
template <int DT> struct Unpack;
template <> struct Unpack<PA_F16> {
  __device__ __forceinline__ static void run(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h = __builtin_bit_cast(half2_t, w[i]);
      f[2 * i] = static_cast<float>(h.x);
      f[2 * i + 1] = static_cast<float>(h.y);
    }
  }
};
template <> struct Unpack<PA_BF16> {
  __device__ __forceinline__ static void run(const uint4& v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};
template <> struct Unpack<PA_F32> {
  __device__ __forceinline__ static void run(const uint4& v, float (&f)[4]) {
    f[0] = __builtin_bit_cast(float, v.x);
    f[1] = __builtin_bit_cast(float, v.y);
    f[2] = __builtin_bit_cast(float, v.z);
    f[3] = __builtin_bit_cast(float, v.w);
  }
};

// One 16 x 16 x 32 matrix-core product with fp32 accumulation, C += A B, for
// 16-bit operands. Lane l passes 8 consecutive k-elements of row l % 16 of A
// and of column l % 16 of B (k-block l / 16 of the 32); it gets back
// C[4 (l / 16) + r][l % 16] in element r.
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int DT> struct Mfma;
template <> struct Mfma<PA_F16> {
  typedef _Float16 x8 __attribute__((ext_vector_type(8)));
  __device__ __forceinline__ static f32x4 run(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<PA_BF16> {
  typedef __bf16 x8 __attribute__((ext_vector_type(8)));
  __device__ __forceinline__ static f32x4 run(const uint4& a, const uint4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a), __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
};

template <int DT> __device__ __forceinline__ void store_out(void* base, int64_t idx, float x);
template <> __device__ __forceinline__ void store_out<PA_F32>(void* base, int64_t idx, float x) {
  static_cast<float*>(base)[idx] = x;
}
template <> __device__ __forceinline__ void store_out<PA_F16>(void* base, int64_t idx, float x) {
  static_cast<_Float16*>(base)[idx] = static_cast<_Float16>(x);
}
template <> __device__ __forceinline__ void store_out<PA_BF16>(void* base, int64_t idx, float x) {
  static_cast<uint16_t*>(base)[idx] = to_bf16_bits(x);
}

// store_out with a non-temporal store, for the partial rows only the merge
// reads: amid the partition kernel's read stream these stores cost the
// long-context decode 1.3-2% less than cached ones.
template <int DT> __device__ __forceinline__ void store_out_nt(void* base, int64_t idx, float x);
template <> __device__ __forceinline__ void store_out_nt<PA_F32>(void* base, int64_t idx, float x) {
  __builtin_nontemporal_store(x, static_cast<float*>(base) + idx);
}
template <> __device__ __forceinline__ void store_out_nt<PA_F16>(void* base, int64_t idx, float x) {
  __builtin_nontemporal_store(static_cast<_Float16>(x), static_cast<_Float16*>(base) + idx);
}
template <> __device__ __forceinline__ void store_out_nt<PA_BF16>(void* base, int64_t idx, float x) {
  __builtin_nontemporal_store(to_bf16_bits(x), static_cast<uint16_t*>(base) + idx);
}

// An element stored by store_out<DT>, as fp32 (exact).
template <int DT> __device__ __forceinline__ float load_out(const void* base, int64_t idx);
template <> __device__ __forceinline__ float load_out<PA_F32>(const void* base, int64_t idx) {
  return static_cast<const float*>(base)[idx];
}
template <> __device__ __forceinline__ float load_out<PA_F16>(const void* base, int64_t idx) {
  return static_cast<float>(static_cast<const _Float16*>(base)[idx]);
}
template <> __device__ __forceinline__ float load_out<PA_BF16>(const void* base, int64_t idx) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16);
}

// A 32-bit word of a stored partial output: kCols output elements.
template <int DT> struct Word;
template <> struct Word<PA_F32> {
  static constexpr int kCols = 1;
  __device__ __forceinline__ static void unpack(uint32_t w, float (&r)[1]) { r[0] = __builtin_bit_cast(float, w); }
};
template <> struct Word<PA_F16> {
  static constexpr int kCols = 2;
  __device__ __forceinline__ static void unpack(uint32_t w, float (&r)[2]) {
    const half2_t h = __builtin_bit_cast(half2_t, w);
    r[0] = static_cast<float>(h.x);
    r[1] = static_cast<float>(h.y);
  }
};
template <> struct Word<PA_BF16> {
  static constexpr int kCols = 2;
  __device__ __forceinline__ static void unpack(uint32_t w, float (&r)[2]) {
    r[0] = bf16_lo(w);
    r[1] = bf16_hi(w);
  }
};

// ---------------------------------------------------------------------------
// wave64 reductions
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16
constexpr int kRowRor4 = 0x124;        // lane i <- lane (i + 4) mod 16 within 16
constexpr int kRowRor8 = 0x128;        // lane i <- lane (i + 8) mod 16 within 16
// quad_perm [j,j,j,j]: every lane of a quad reads its quad's lane j
template <int J> __device__ __forceinline__ float quad_bcast(float x) { return dpp<J * 0x55>(x); }

// Sum over aligned groups of N lanes; every lane of the group gets the sum.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kQuadSwap1>(x);
  x += dpp<kQuadSwap2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N == 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ int readlane_i(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// ---------------------------------------------------------------------------
// merging partitions: steps 2-5 of [PA] §5.1 across a sequence's partitions
// ---------------------------------------------------------------------------
// Block-wide reduction over NT threads (fixed order). Starts with a barrier, so
// lds_red may be reused right after a previous reduction.
template <int NT, bool kMax> __device__ __forceinline__ float block_reduce(float x, float* lds_red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float y = __shfl_xor(x, off);
    x = kMax ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds_red[wave] = x;
  __syncthreads();
  float r = lds_red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) r = kMax ? fmaxf(r, lds_red[w]) : r + lds_red[w];
  return r;
}


// Merge the P partitions of query head hq of sequence s with the NT threads of
// one workgroup. Partition p left (m_p, l_p, o_p) with o_p already divided by
// l_p; with m = max_p m_p (step 2) and w_p = l_p * 2^(m_p - m) (steps 3-4),
// out = sum_p w_p o_p / sum_p w_p (step 5). Column col of o is summed by
// R = NT / D threads over interleaved partitions, then those R sums are added
// in a fixed order. The first BATCH partial outputs are loaded together with
// the (m_p, l_p) pairs, since neither depends on the other. LDS: lds_red
// [NT / 64], lds_w [WCAP] (weights of the first WCAP partitions; later ones are
// recomputed), part_o [NT].
template <int DT, int D, int NT, int WCAP, int BATCH>
__device__ __forceinline__ void merge_head(const DecodeArgs& a, int s, int hq, int P, float* lds_red, float* lds_w,
                                           float* part_o) {
  constexpr int R = NT / D;
  const int tid = threadIdx.x;
  const int64_t row = (static_cast<int64_t>(s) * a.num_q_heads + hq) * a.slot_stride;
  const float2* ml = a.ws_ml + row;
  const int col = tid % D;
  const int r = tid / D;
  const int64_t o_col = row * D + col;               // element index of slot 0's column in ws_o

  float ov[BATCH];
#pragma unroll
  for (int i = 0; i < BATCH; ++i) {
    const int p = r + i * R;
    ov[i] = p < P ? load_out<DT>(a.ws_o, o_col + static_cast<int64_t>(p) * D) : 0.0f;
  }
  float m = -INFINITY;
  for (int p = tid; p < P; p += NT) m = fmaxf(m, ml[p].x);
  m = block_reduce<NT, true>(m, lds_red);                           // step 2
  float L = 0.0f;
  for (int p = tid; p < P; p += NT) {
    const float w = ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - m);   // step 3
    if (p < WCAP) lds_w[p] = w;
    L += w;
  }
  L = block_reduce<NT, false>(L, lds_red);                          // step 4 (its barriers publish lds_w)
  auto weight = [&](int p) {
    return p < WCAP ? lds_w[p] : ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - m);
  };

  float o = 0.0f;
#pragma unroll
  for (int i = 0; i < BATCH; ++i) {
    const int p = r + i * R;
    if (p < P) o = fmaf(weight(p), ov[i], o);
  }
  for (int p0 = r + BATCH * R; p0 < P; p0 += BATCH * R) {
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int p = p0 + i * R;
      ov[i] = p < P ? load_out<DT>(a.ws_o, o_col + static_cast<int64_t>(p) * D) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int p = p0 + i * R;
      if (p < P) o = fmaf(weight(p), ov[i], o);
    }
  }
  part_o[r * D + col] = o;
  __syncthreads();
  if (r == 0) {
    float sum = part_o[col];
#pragma unroll
    for (int i = 1; i < R; ++i) sum += part_o[i * D + col];
    store_out<DT>(a.out, (static_cast<int64_t>(s) * a.num_q_heads + hq) * D + col, sum / L);   // step 5
  }
}

constexpr int kMergeThreads = 512;
constexpr int kMergeWeights = 2048;

// Stand-alone merge pass: one workgroup per (query head, sequence).
template <int DT, int D>
__global__ __launch_bounds__(kMergeThreads) void pa_decode_merge_kernel(DecodeArgs a) {
  __shared__ float lds_red[kMergeThreads / kWave];
  __shared__ float lds_w[kMergeWeights];
  __shared__ float part_o[kMergeThreads];
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int ctx = a.context_lens[s];
  if (ctx <= 0 || ctx > a.max_context_len) return;   // written by the partition kernel
  const int P = a.num_slots != nullptr ? min(a.num_slots[s], a.slot_stride)
                                       : (ctx + a.partition_size - 1) / a.partition_size;
  if (P <= 1) return;
  merge_head<DT, D, kMergeThreads, kMergeWeights, 16>(a, s, hq, P, lds_red, lds_w, part_o);
}

// Merge passes for up to 64 partials per sequence. Every load a (sequence,
// query head) needs - its count of partials, then all of its (m, l) pairs
// and partial outputs at once - goes out before any is used, so a head
// costs two memory round trips: lane p holds partial p's (m_p, l_p), the
// wave's maximum and sum of weights come from butterfly reductions (the
// same order whatever the data), and each lane folds its columns' partial
// outputs in partial order, the weights taken from their lanes.
constexpr int kMergeHeadsPerWg = 4;        // one wave per (sequence, query head)
constexpr int kMergeWaveParts = 16;        // partials one wave folds in one go
constexpr int kMergeLanesMaxParts = 64;    // the lane-parallel merges take up to this many

template <int DT, int D> struct MergeRow {
  using W = Word<DT>;
  static constexpr int kWords = D / W::kCols;                       // 32-bit words per partial row
  static constexpr int kWPL = (kWords + kWave - 1) / kWave;         // words per lane
};

// Partials [p0, p0 + 16) of one head: lane `lane` folds its words.
template <int DT, int D>
__device__ __forceinline__ void fold_parts(const DecodeArgs& a, int64_t row, int P, int p0, int lane, float w_lane,
                                           float (&acc)[MergeRow<DT, D>::kWPL][Word<DT>::kCols]) {
  using R = MergeRow<DT, D>;
  const uint32_t* po = static_cast<const uint32_t*>(a.ws_o);
  uint32_t v[kMergeWaveParts][R::kWPL];
#pragma unroll
  for (int i = 0; i < kMergeWaveParts; ++i)
#pragma unroll
    for (int k = 0; k < R::kWPL; ++k) {
      const int wd = lane + k * kWave;
      v[i][k] = (p0 + i < P && wd < R::kWords) ? po[(row + p0 + i) * R::kWords + wd] : 0u;
    }
#pragma unroll
  for (int i = 0; i < kMergeWaveParts; ++i) {
    if (p0 + i >= P) break;
    const float w = __builtin_bit_cast(float, readlane_i(__builtin_bit_cast(int, w_lane), p0 + i));
#pragma unroll
    for (int k = 0; k < R::kWPL; ++k) {
      float x[Word<DT>::kCols];
      Word<DT>::unpack(v[i][k], x);
#pragma unroll
      for (int c = 0; c < Word<DT>::kCols; ++c) acc[k][c] = fmaf(w, x[c], acc[k][c]);
    }
  }
}

// Step 2-4 of [PA] §5.1 over a head's partials: lane p < P holds w_p =
// l_p 2^(m_p - m); returns the sum of the weights (every lane).
__device__ __forceinline__ float merge_weights(const DecodeArgs& a, int64_t row, int P, int lane, float* w_lane) {
  const float2 ml = lane < P ? a.ws_ml[row + lane] : make_float2(-INFINITY, 0.0f);
  float m = ml.x;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));        // step 2
  const float w = lane < P ? ml.y * __builtin_amdgcn_exp2f(ml.x - m) : 0.0f;        // step 3
  float L = w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);                   // step 4
  *w_lane = w;
  return L;
}

__device__ __forceinline__ int merge_parts_of(const DecodeArgs& a, int s) {
  if (a.num_slots != nullptr) return min(a.num_slots[s], a.slot_stride);
  const int ctx = a.context_lens[s];
  if (ctx <= 0 || ctx > a.max_context_len) return 0;   // written by the partition kernel
  return (ctx + a.partition_size - 1) / a.partition_size;
}

// Up to 16 partials: one wave per (query head, sequence), four heads per workgroup.
template <int DT, int D>
__global__ __launch_bounds__(kMergeHeadsPerWg * kWave) void pa_decode_merge_small_kernel(DecodeArgs a) {
  using R = MergeRow<DT, D>;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int hq = blockIdx.x * kMergeHeadsPerWg + wave;
  const int s = blockIdx.y;
  if (hq >= a.num_q_heads) return;
  if (a.num_slots != nullptr) {
    const int ctx = a.context_lens[s];
    if (ctx <= 0 || ctx > a.max_context_len) return;
  }
  const int P = merge_parts_of(a, s);
  if (P <= 1) return;
  const int64_t row = (static_cast<int64_t>(s) * a.num_q_heads + hq) * a.slot_stride;
  float w_lane;
  const float L = merge_weights(a, row, P, lane, &w_lane);
  float acc[R::kWPL][Word<DT>::kCols] = {};
  fold_parts<DT, D>(a, row, P, 0, lane, w_lane, acc);
  const int64_t o = (static_cast<int64_t>(s) * a.num_q_heads + hq) * D;
#pragma unroll
  for (int k = 0; k < R::kWPL; ++k) {
    const int wd = lane + k * kWave;
    if (wd < R::kWords)
#pragma unroll
      for (int c = 0; c < Word<DT>::kCols; ++c)
        store_out<DT>(a.out, o + wd * Word<DT>::kCols + c, acc[k][c] / L);                        // step 5
  }
}

// 17 to 64 partials: four waves per (query head, sequence); wave w folds
// partials [16 w, 16 w + 16), and the four sums are added in wave order.
template <int DT, int D>
__global__ __launch_bounds__(4 * kWave) void pa_decode_merge_mid_kernel(DecodeArgs a) {
  using R = MergeRow<DT, D>;
  constexpr int C = Word<DT>::kCols;
  __shared__ float part[4][R::kWPL][C][kWave];
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & (kWave - 1);
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  if (a.num_slots != nullptr) {
    const int ctx = a.context_lens[s];
    if (ctx <= 0 || ctx > a.max_context_len) return;
  }
  const int P = merge_parts_of(a, s);
  if (P <= 1) return;
  const int64_t row = (static_cast<int64_t>(s) * a.num_q_heads + hq) * a.slot_stride;
  float w_lane;
  const float L = merge_weights(a, row, min(P, kMergeLanesMaxParts), lane, &w_lane);
  float acc[R::kWPL][C] = {};
  fold_parts<DT, D>(a, row, min(P, kMergeLanesMaxParts), wave * kMergeWaveParts, lane, w_lane, acc);
#pragma unroll
  for (int k = 0; k < R::kWPL; ++k)
#pragma unroll
    for (int c = 0; c < C; ++c) part[wave][k][c][lane] = acc[k][c];
  __syncthreads();
  if (wave != 0) return;
  const int64_t o = (static_cast<int64_t>(s) * a.num_q_heads + hq) * D;
#pragma unroll
  for (int k = 0; k < R::kWPL; ++k) {
    const int wd = lane + k * kWave;
    if (wd < R::kWords)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float sum = ((part[0][k][c][lane] + part[1][k][c][lane]) + part[2][k][c][lane]) + part[3][k][c][lane];
        store_out<DT>(a.out, o + wd * C + c, sum / L);                                           // step 5
      }
  }
}

// ---------------------------------------------------------------------------
// partition kernel
// ---------------------------------------------------------------------------
// A lane's share of one cached K or V row: kElems elements in one vector load
// of kBytes bytes - 16 bytes of a 16/32-bit cache; 8 FP8 codes, or 16 in the
// wide form (W), where a row of 128 codes spans 8 lanes and one wave load
// covers 8 rows (1 KiB) instead of 4 (512 B).
template <int KT, bool W = false> struct Lane;
template <bool W> struct Lane<PA_F32, W> { using vec = uint4; static constexpr int kElems = 4, kBytes = 16; };
template <bool W> struct Lane<PA_F16, W> { using vec = uint4; static constexpr int kElems = 8, kBytes = 16; };
template <bool W> struct Lane<PA_BF16, W> { using vec = uint4; static constexpr int kElems = 8, kBytes = 16; };
template <> struct Lane<PA_FP8_E4M3, false> { using vec = uint2; static constexpr int kElems = 8, kBytes = 8; };
template <> struct Lane<PA_FP8_E4M3, true> { using vec = uint4; static constexpr int kElems = 16, kBytes = 16; };
template <> struct Lane<PA_INT8, false> { using vec = uint2; static constexpr int kElems = 8, kBytes = 8; };
template <> struct Lane<PA_INT8, true> { using vec = uint4; static constexpr int kElems = 16, kBytes = 16; };

template <int KT, int D, int BS, bool W = false>
struct Geometry {
  static constexpr int kElem = Fmt<KT>::kBytes;           // bytes per cached element
  static constexpr int kRowBytes = D * kElem;              // one token row of one head
  static constexpr int kEPL = Lane<KT, W>::kElems;         // elements per lane
  static constexpr int kLPR = D / kEPL;                    // lanes per row
  static constexpr int kRPC = kWave / kLPR;                // rows per wave load ("chunk")
  static constexpr int kChunkBytes = kWave * Lane<KT, W>::kBytes;
  static constexpr int kCPB = BS / kRPC;                   // chunks per (block, head)
  static constexpr int kBlockHeadBytes = BS * kRowBytes;
  static_assert(D % kEPL == 0 && kLPR >= 8 && kLPR <= 32, "row must span 8..32 lanes");
  static_assert(BS % kRPC == 0, "block must hold whole wave loads");
};

template <int KT, bool W> __device__ __forceinline__ typename Lane<KT, W>::vec load_lane(const char* p) {
  using V = typename Lane<KT, W>::vec;
  // non-temporal: K/V are streamed past the caches (each byte is read once per launch)
  if constexpr (Lane<KT, W>::kBytes == 16) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
  } else {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(V, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
  }
}

// FP8 row scales: ordinary cached loads, so that the waves reading one run of
// scales share the fetch.
__device__ __forceinline__ float load_scale(const float* p) { return *p; }

// The query slice a lane holds: the packed query elements of its columns - 16
// bytes, or 32 (16 fp16 / bf16 values) against the wide FP8 form; FP8 codes
// are widened to the query's type.
template <int QT, int KT, bool W> struct QSlice { uint4 v[W ? 2 : 1]; };

template <int QT, int KT, bool W> __device__ __forceinline__ QSlice<QT, KT, W> load_q(const char* p) {
  QSlice<QT, KT, W> r;
#pragma unroll
  for (int i = 0; i < (W ? 2 : 1); ++i) r.v[i] = reinterpret_cast<const uint4*>(p)[i];
  return r;
}

// Two FP8 E4M3 codes (the low or high 16 bits of w) widened to the query's
// 16-bit type; exact, since every E4M3 value is an fp16 and a bf16 value.
template <int QT> __device__ __forceinline__ uint32_t fp8x2_widen(uint32_t w, bool high);
template <> __device__ __forceinline__ uint32_t fp8x2_widen<PA_F16>(uint32_t w, bool high) {
  return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}
template <> __device__ __forceinline__ uint32_t fp8x2_widen<PA_BF16>(uint32_t w, bool high) {
  return __builtin_bit_cast(uint32_t, high ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

// Two int8 codes (bytes 0-1, or 2-3 when `high`, of w) widened to the
// query's 16-bit type; exact, since |code| <= 127. fp16: the biased byte
// b + 128 goes under the exponent of 1024, whose unit in the last place is 1,
// and 1152 comes off again; bf16: through fp32, whose low half is then zero.
template <int QT> __device__ __forceinline__ uint32_t int8x2_widen(uint32_t w, bool high);
template <> __device__ __forceinline__ uint32_t int8x2_widen<PA_F16>(uint32_t w, bool high) {
  const uint32_t biased = __builtin_amdgcn_perm(w ^ 0x80808080u, 0x64646464u, high ? 0x00070006u : 0x00050004u);
  const half2_t v = __builtin_bit_cast(half2_t, biased) - half2_t{1152.0f16, 1152.0f16};
  return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t int8x2_widen<PA_BF16>(uint32_t w, bool high) {
  const int sh = high ? 16 : 0;
  const float lo = static_cast<float>(static_cast<int8_t>((w >> sh) & 0xffu));
  const float hi = static_cast<float>(static_cast<int8_t>((w >> (sh + 8)) & 0xffu));
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

// 4 * NW int8 codes (NW 32-bit words) as fp32 values (exact).
template <int NW>
__device__ __forceinline__ void int8_words_to_f32(const uint32_t (&w)[NW], float (&f)[4 * NW]) {
#pragma unroll
  for (int i = 0; i < NW; ++i)
#pragma unroll
    for (int b = 0; b < 4; ++b) f[4 * i + b] = static_cast<float>(static_cast<int8_t>((w[i] >> (8 * b)) & 0xffu));
}

// 4 * NW FP8 E4M3 codes (NW 32-bit words) as fp32 values (exact).
template <int NW>
__device__ __forceinline__ void fp8_words_to_f32(const uint32_t (&w)[NW], float (&f)[4 * NW]) {
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    f[4 * i] = lo[0];
    f[4 * i + 1] = lo[1];
    f[4 * i + 2] = hi[0];
    f[4 * i + 3] = hi[1];
  }
}

// Two codes of a quantised cache widened to the query's 16-bit type.
template <int QT, int KT> __device__ __forceinline__ uint32_t codes_widen(uint32_t w, bool high) {
  if constexpr (KT == PA_FP8_E4M3) return fp8x2_widen<QT>(w, high);
  else return int8x2_widen<QT>(w, high);
}

// A lane's part of q . K for one row. FP8 / INT8 codes are widened to the
// query's type two at a time and go through the same dot2 instructions as
// 16-bit K.
template <int QT, int KT, bool W>
__device__ __forceinline__ float dot_lane(const QSlice<QT, KT, W>& q, const typename Lane<KT, W>::vec& k) {
  if constexpr (kQuantized<KT>) {
    const uint4 k0 = {codes_widen<QT, KT>(k.x, false), codes_widen<QT, KT>(k.x, true),
                      codes_widen<QT, KT>(k.y, false), codes_widen<QT, KT>(k.y, true)};
    if constexpr (W) {
      const uint4 k1 = {codes_widen<QT, KT>(k.z, false), codes_widen<QT, KT>(k.z, true),
                        codes_widen<QT, KT>(k.w, false), codes_widen<QT, KT>(k.w, true)};
      return dot16<QT>(q.v[0], k0) + dot16<QT>(q.v[1], k1);
    } else {
      return dot16<QT>(q.v[0], k0);
    }
  } else {
    return dot16<KT>(q.v[0], k);
  }
}

// A lane's V elements as fp32.
template <int KT, bool W> __device__ __forceinline__ void unpack_lane(const typename Lane<KT, W>::vec& v,
                                                                    float (&f)[Lane<KT, W>::kElems]) {
  if constexpr (KT == PA_FP8_E4M3) {
    if constexpr (W) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      fp8_words_to_f32<4>(w, f);
    } else {
      const uint32_t w[2] = {v.x, v.y};
      fp8_words_to_f32<2>(w, f);
    }
  } else if constexpr (KT == PA_INT8) {
    if constexpr (W) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      int8_words_to_f32<4>(w, f);
    } else {
      const uint32_t w[2] = {v.x, v.y};
      int8_words_to_f32<2>(w, f);
    }
  } else {
    Unpack<KT>::run(v, f);
  }
}

// Max over the rows of a wave of a value that is uniform inside each row group
// of N lanes; the result is wave-uniform.
template <int N> __device__ __forceinline__ float rows_max(float x) {
  if constexpr (N <= 8) x = fmaxf(x, __shfl_xor(x, 8));
  if constexpr (N <= 16) x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// One workgroup = NW waves on one (KV head, partition) of one sequence - and,
// in a shared item of the launch schedule, of up to QM - 1 more sequences
// whose block tables hold the same physical blocks for the whole partition
// ([PA] §5.2: queries that hit the same physical blocks are handled together,
// so those blocks are read once). The workgroup serves NQ = G * QM query
// vectors: query set m (m = 0 the item's own sequence, m > 0 its members)
// times the G query heads of the KV head.
//
// Each wave takes every NW-th chunk (RPC consecutive token rows of one block)
// and keeps its own running softmax state per query vector: the running
// maximum m (in log2 units, wave-uniform), the lane's share of sum 2^(s - m)
// and of sum 2^(s - m) * V for its column slice. A batch of U chunks is loaded
// (K and V together), its local maximum found (step 1 of [PA] §5.1 at batch
// granularity), the running state rescaled to the new maximum (step 2), and
// the batch's exponentials and weighted V rows added (steps 3-4). The waves'
// states are combined at the end in a fixed order; step 5 (the division) is
// done here for a single-partition sequence, else by the merge kernel.
// Workgroups per CU the compiler must fit (register budget): the wide FP8
// form is held to PA_FP8_WIDE_MIN_WGS, the others are left to the compiler.
template <int KT, int D, int G, int QM> constexpr int partition_min_wgs() {
  return (kQuantized<KT> && D == 128 && G * QM <= PA_FP8_WIDE_NQ) ? PA_FP8_WIDE_MIN_WGS : 1;
}

template <int QT, int KT, int D, int BS, int G, int QM>
__global__ __launch_bounds__(kNumWaves * kWave, (partition_min_wgs<KT, D, G, QM>())) void pa_decode_partition_kernel(
    DecodeArgs a) {
  constexpr bool kFp8 = kQuantized<KT>;   // one-byte codes with a scale per row (FP8 or INT8)
  constexpr bool kWide = kFp8 && D == 128 && G * QM <= PA_FP8_WIDE_NQ;
  // four query heads over a 16-bit cache at head_dim 128: scores on the matrix cores
  constexpr bool kMfma = G == 4 && QM == 1 && D == 128 && QT == KT && (KT == PA_F16 || KT == PA_BF16);
  using Geo = Geometry<KT, D, BS, kWide>;
  using KVec = typename Lane<KT, kWide>::vec;
  constexpr int LPR = Geo::kLPR, RPC = Geo::kRPC, EPL = Geo::kEPL, CPB = Geo::kCPB;
  constexpr int QB = Fmt<QT>::kBytes;        // bytes per query element
  constexpr int NQ = G * QM;
  constexpr int NW = kNumWaves, U = kFp8 ? (kWide ? PA_UNROLL_FP8_WIDE : PA_UNROLL_FP8)
                                          : (QM > 1 ? PA_UNROLL_SHARED : (G >= 4 ? PA_UNROLL_GQA : kUnroll));

  __shared__ float lds_o[NW][NQ][D];
  __shared__ float lds_m[NW][NQ];
  __shared__ float lds_l[NW][NQ];
  __shared__ uint4 lds_k[kMfma ? NW : 1][kMfma ? 16 * 17 : 1];   // matrix-core form: per-wave K tile

  // What this workgroup covers: tokens [t0, t0 + n_tok) of sequence s (and of
  // its members), whose partial result goes to slot `slot`.
  const bool scheduled = a.work != nullptr;
  int h, s, t0, slot, item_tok = 0;
  int64_t row_base;                                // first table entry of sequence s
  int row_cols;                                    // entries in that row
  int mbase = 0, mcount = 0;   // members of a shared item (QM > 1 only)
  if (scheduled) {
    // workgroup x serves KV head x % Hkv of work item x / Hkv
    int x = static_cast<int>(blockIdx.x);
    if constexpr (kFp8) {
      // The row scales of heads 2k and 2k + 1 of a block share one 128-byte
      // line. Workgroups are handed to the 8 XCDs (each with its own L2) in
      // turn, so ids 8 apart land on the same XCD at about the same time:
      // within every 16 ids, id k and id k + 8 take heads 2k and 2k + 1, so
      // the line is fetched once. Only the order inside groups of 16 changes.
      if (x < static_cast<int>(gridDim.x) / 16 * 16) {
        const int r = x & 15;
        x = (x & ~15) | ((r & 7) << 1) | (r >> 3);
      }
    }
    const int item = x / a.num_kv_heads;
    h = x - item * a.num_kv_heads;
    const int32_t* w = a.work + kItemInts * static_cast<int64_t>(item);
    s = w[0];
    t0 = w[1];
    item_tok = w[2];
    slot = w[3];
    if (s < 0 || s >= a.num_seqs || t0 < 0 || t0 % BS != 0 || slot < 0 || slot >= a.slot_stride) return;
    if (a.compact_tables) {
      // a row outside the array reads nothing, and its blocks then poison the output
      const bool row_ok = w[6] >= 0 && w[7] >= 0 && w[6] <= a.table_entries - w[7];
      row_base = row_ok ? w[6] : 0;
      row_cols = row_ok ? w[7] : 0;
    } else {
      row_base = static_cast<int64_t>(s) * a.max_blocks_per_seq;
      row_cols = a.max_blocks_per_seq;
    }
    if constexpr (QM > 1) {
      mbase = w[4];
      mcount = min(max(w[5], 0), QM - 1);
      if (mcount > 0 && (mbase < 0 || mbase + mcount > a.num_members)) mcount = 0;
    }
  } else {
    h = blockIdx.x;                                // KV head
    s = blockIdx.y;                                // sequence
    slot = blockIdx.z;
    t0 = slot * a.partition_size;
    row_base = static_cast<int64_t>(s) * a.max_blocks_per_seq;
    row_cols = a.max_blocks_per_seq;
  }
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = a.num_q_heads;

  // sequence of each query set (m <= mcount)
  int seq[QM];
  seq[0] = s;
#pragma unroll
  for (int m = 1; m < QM; ++m) {
    const int sm = m <= mcount ? a.members[mbase + m - 1] : -1;
    seq[m] = (sm >= 0 && sm < a.num_seqs) ? sm : -1;
  }

  // The context lengths, the range's block ids and q do not depend on each
  // other: all are loaded before any is used, so a workgroup waits for one
  // memory latency before it starts streaming K/V.
  const int part = a.partition_size;
  const int tb = t0 / BS;                          // first logical block of the range
  int raw_blk = 0;
  if (tb + lane < row_cols)                        // inside the table row (at most 64 blocks used)
    raw_blk = a.block_tables[row_base + tb + lane];
  // q slices of query vector m*G+g: sequence seq[m], head h*G+g, columns (lane % LPR) * EPL ...
  QSlice<QT, KT, kWide> qv[NQ];
#pragma unroll
  for (int m = 0; m < QM; ++m) {
    const int sm = seq[m] < 0 ? s : seq[m];        // an absent member reads the leader's q, result unused
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(sm) * Hq + h * G) * D + (lane % LPR) * EPL) * QB;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[m * G + g] = load_q<QT, KT, kWide>(qb + static_cast<int64_t>(g) * D * QB);
  }
  // Matrix-core form: q is the B operand of the score product. Lane l holds
  // query head h * G + l % 4, columns 32 i + 8 (l / 16) .. + 7 for d-block i;
  // the 16 columns of B are the four heads, each repeated four times.
  uint4 qmf[kMfma ? 4 : 1];
  if constexpr (kMfma) {
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(s) * Hq + h * G + (lane & 3)) * D + 8 * (lane >> 4)) * QB;
#pragma unroll
    for (int i = 0; i < 4; ++i) qmf[i] = *reinterpret_cast<const uint4*>(qb + 64 * i);
  }
  int ctx_m[QM], nslot_m[QM];
#pragma unroll
  for (int m = 0; m < QM; ++m) {
    ctx_m[m] = seq[m] < 0 ? -1 : a.context_lens[seq[m]];
    nslot_m[m] = (scheduled && seq[m] >= 0) ? a.num_slots[seq[m]] : 0;
  }
  const int ctx = ctx_m[0];
  const bool bad_ctx = ctx < 0 || ctx > a.max_context_len;

  if (ctx == 0 || bad_ctx) {
    // empty context -> zeros; invalid length -> NaN rows (written once, by the
    // workgroup of slot 0)
    if (slot != 0) return;
    const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int i = tid; i < G * D; i += NW * kWave)
      store_out<QT>(a.out, (static_cast<int64_t>(s) * Hq + h * G) * D + i, fill);
    return;
  }
  // a scheduled range must lie inside the context; one that does not is computed
  // over its clamped extent and gives NaN
  bool range_bad = false;
  int n_tok;
  if (scheduled) {
    range_bad = item_tok < 1 || item_tok > kWave * BS || t0 + item_tok > ctx;
    n_tok = min(max(item_tok, 1), kWave * BS);
  } else {
    if (t0 >= ctx) return;                         // past the sequence's end
    n_tok = min(ctx - t0, part);
  }
  const int n_blk = (n_tok + BS - 1) / BS;
  const int n_chunks = (n_tok + RPC - 1) / RPC;   // rows past the context are never fetched

  // Block ids of the partition: lane j holds logical block tb + j; entries
  // past the context are ignored, out-of-pool ids poison the output.
  const bool blk_bad = lane < n_blk && (tb + lane >= row_cols || raw_blk < 0 || raw_blk >= a.num_blocks);
  const int my_blk = (lane < n_blk && !blk_bad) ? raw_blk : 0;   // keep every address inside the pool
  const bool any_bad = __ballot(blk_bad) != 0;

  const char* kbase = static_cast<const char*>(a.k_cache) + static_cast<int64_t>(h) * Geo::kBlockHeadBytes +
                      lane * Lane<KT, kWide>::kBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + static_cast<int64_t>(h) * Geo::kBlockHeadBytes +
                      lane * Lane<KT, kWide>::kBytes;
  const int64_t block_stride = static_cast<int64_t>(a.num_kv_heads) * Geo::kBlockHeadBytes;
  const int row_in_chunk = lane / LPR;
  const int row_back = row_in_chunk * Geo::kRowBytes;   // from this lane's row to the chunk's first
  // FP8: the row scales of (block phys, head h) start at scale + (phys * Hkv + h) * BS
  const float* kscale_h = kFp8 ? a.k_scale + static_cast<int64_t>(h) * BS + row_in_chunk : nullptr;
  const float* vscale_h = kFp8 ? a.v_scale + static_cast<int64_t>(h) * BS + row_in_chunk : nullptr;
  const int64_t scale_stride = static_cast<int64_t>(a.num_kv_heads) * BS;

  float m_run[NQ], l_run[NQ], acc[NQ][EPL];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.0f;
  }

  // query vector j belongs to a query set that exists in this item (uniform)
  auto present = [&](int j) { return QM == 1 || j / G <= mcount; };

  // Loads of one batch; chunk indices past the end are clamped to the last
  // chunk (a repeat of an address already in flight) and ignored later.
  // FP8 caches also load each row's K and V scales. Every K load goes out
  // before the first V load: loads complete in order, so the scores and the
  // batch maximum can start while V is still arriving.
  // The i-th chunk this wave takes. 16/32-bit caches: whole blocks, chunk
  // i % CPB of block (i / CPB) * NW + wave, so each wave reads every block it
  // touches end to end (0.5-0.8% faster on the 13B and 7B shapes); FP8 / INT8
  // (two chunks per block): every NW-th chunk.
  auto chunk_of = [&](int i) {
    if constexpr (kFp8) return wave + i * NW;
    else return ((i / CPB) * NW + wave) * CPB + (i % CPB);
  };
  auto load_batch = [&](int i0, KVec (&kb)[U], KVec (&vb)[U], float (&ks)[U], float (&vs)[U]) {
    int64_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(chunk_of(i0 + u), n_chunks - 1);
      const int phys = readlane_i(my_blk, c / CPB);
      // a lane whose row lies past the range's last token reads its columns of
      // the chunk's first row instead (a token of the range): the chunk fetches
      // only its valid rows' lines (FP8 13B traffic -1.0%, fp16 -0.3%; the
      // matrix-core form, whose long ranges have few such rows, goes without)
      const int valid_rows = n_tok - c * RPC;                      // uniform
      off[u] = phys * block_stride + (c % CPB) * Geo::kChunkBytes - (row_in_chunk >= valid_rows ? row_back : 0);
      kb[u] = load_lane<KT, kWide>(kbase + off[u]);
      if constexpr (kFp8) {
        const int64_t so = phys * scale_stride + (c % CPB) * RPC;
        ks[u] = load_scale(kscale_h + so);
        vs[u] = load_scale(vscale_h + so);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) vb[u] = load_lane<KT, kWide>(vbase + off[u]);
  };

  auto process_batch = [&](int i0, const KVec (&kb)[U], const KVec (&vb)[U], const float (&ks)[U],
                           const float (&vs)[U]) {
    float sc[U][NQ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = chunk_of(i0 + u);
      const int row = c * RPC + row_in_chunk;                 // token index in the range
      const bool valid = c < n_chunks && row < n_tok;
      const float kscale = kFp8 ? ks[u] * a.scale_log2 : a.scale_log2;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        if (!present(j)) continue;
        const float x = group_sum<LPR>(dot_lane<QT, KT, kWide>(qv[j], kb[u])) * kscale;
        sc[u][j] = valid ? x : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      if (!present(j)) continue;
      float bm = sc[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) bm = fmaxf(bm, sc[u][j]);
      bm = rows_max<LPR>(bm);
      const float m_new = fmaxf(m_run[j], bm);   // finite: chunk chunk_of(i0) holds a valid row
      const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_new);
      m_run[j] = m_new;
      l_run[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = chunk_of(i0 + u);
      if (c < n_chunks) {
        const int row = c * RPC + row_in_chunk;
        float f[EPL];
        unpack_lane<KT, kWide>(vb[u], f);
        float vscale = kFp8 ? vs[u] : 1.0f;
        if (c * RPC + RPC > n_tok) {
          // rows past the context (stale data, possibly NaN) must not reach acc
#pragma unroll
          for (int e = 0; e < EPL; ++e) f[e] = row < n_tok ? f[e] : 0.0f;
          vscale = row < n_tok ? vscale : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
          if (!present(j)) continue;
          const float e = __builtin_amdgcn_exp2f(sc[u][j] - m_run[j]);   // 0 for masked rows
          l_run[j] += e;
          const float ev = kFp8 ? e * vscale : e;                          // FP8: code * scale
#pragma unroll
          for (int k = 0; k < EPL; ++k) acc[j][k] = fmaf(ev, f[k], acc[j][k]);
        }
      }
    }
  };

  if constexpr (kMfma) {
    // Tiles of 16 rows: 4 chunks of V (rows 4i .. 4i + 3 in chunk i, loaded as
    // in the other forms) and the same 16 rows of K loaded for the A operand of
    // the score product. A-row m of a tile is token row (m / 4) + 4 (m % 4), so
    // that the product S = K q^T lands with lane l holding, in element r, the
    // score of query head l % 4 for row (l / 16) + 4 r - the row this lane
    // holds of V chunk r. The four heads' weights of that row then sit in the
    // lane's quad (lane 4 (l / 4) + j, head j) and reach it by a quad
    // broadcast. Each lane keeps the running maximum and sum of head l % 4;
    // the weighted V sums of all four heads stay per lane as in the other forms.
    constexpr int T = PA_MFMA_TILES, TSTEP = NW * T;
    static_assert(RPC == 4 && LPR == 16, "16-bit rows of 128 elements");
    const int n_tiles = (n_tok + 15) / 16;
    const int krow = ((lane & 15) >> 2) + 4 * (lane & 3);   // token row of A-row lane % 16
    uint4* stage = lds_k[wave];                              // this wave's K tile, rows padded to 17 x 16 B
    float m_lane = -INFINITY, l_lane = 0.0f;                 // query head h * G + lane % 4

    for (int tile = wave; tile < n_tiles; tile += TSTEP) {
      uint4 kb[T][4], vb[T][4];
#pragma unroll
      for (int u = 0; u < T; ++u) {
        // tiles past the range repeat the last one (addresses already in flight);
        // K and V: chunks 4t .. 4t + 3, clamped to the last chunk of the range
        const int t = min(tile + u * NW, n_tiles - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = min(4 * t + i, n_chunks - 1);
          const int64_t off = readlane_i(my_blk, c / CPB) * block_stride + (c % CPB) * Geo::kChunkBytes;
          kb[u][i] = load_lane<KT, false>(kbase + off);
          vb[u][i] = load_lane<KT, false>(vbase + off);
        }
      }
      // scores in log2 units; rows past the range (or tiles past it) are -inf
      float sc[T][4];
#pragma unroll
      for (int u = 0; u < T; ++u) {
        // K arrives as whole rows (lane l: row 4 i + l / 16, 16-byte column
        // segment l % 16); the A operand of d-block i wants row krow, segment
        // 4 i + l / 16. The wave regroups it through its own LDS tile: LDS
        // operations of one wave complete in order, so no barrier is needed, and
        // the padded row stride keeps the 16 rows of a read on distinct banks.
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(4 * i + (lane >> 4)) * 17 + (lane & 15)] = kb[u][i];
        __builtin_amdgcn_wave_barrier();
        f32x4 c4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) c4 = Mfma<KT>::run(stage[krow * 17 + 4 * i + (lane >> 4)], qmf[i], c4);
        __builtin_amdgcn_wave_barrier();
        const int t = tile + u * NW;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * t + (lane >> 4) + 4 * r;
          sc[u][r] = (t < n_tiles && row < n_tok) ? c4[r] * a.scale_log2 : -INFINITY;
        }
      }
      // batch maximum of head lane % 4: this lane's rows, then the 16 lanes
      // that hold the same head
      float bm = sc[0][0];
#pragma unroll
      for (int u = 0; u < T; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) bm = fmaxf(bm, sc[u][r]);
      bm = fmaxf(bm, dpp<kRowRor4>(bm));
      bm = fmaxf(bm, dpp<kRowRor8>(bm));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float m_new = fmaxf(m_lane, bm);                  // finite: row 0 of the first tile is in range
      const float alpha = __builtin_amdgcn_exp2f(m_lane - m_new);
      m_lane = m_new;
      l_lane *= alpha;
      const float al[4] = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha), quad_bcast<3>(alpha)};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] *= al[j];
#pragma unroll
      for (int u = 0; u < T; ++u) {
        const int t = tile + u * NW;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(sc[u][r] - m_new);    // 0 for masked rows
          l_lane += p[r];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * t + i;
          if (t < n_tiles && c < n_chunks) {
            const int row = c * RPC + row_in_chunk;
            float f[EPL];
            unpack_lane<KT, false>(vb[u][i], f);
            if (c * RPC + RPC > n_tok) {
              // rows past the range (stale data, possibly NaN) must not reach acc
#pragma unroll
              for (int e = 0; e < EPL; ++e) f[e] = row < n_tok ? f[e] : 0.0f;
            }
            const float w[4] = {quad_bcast<0>(p[i]), quad_bcast<1>(p[i]), quad_bcast<2>(p[i]), quad_bcast<3>(p[i])};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(w[j], f[e], acc[j][e]);
          }
        }
      }
    }
    // the per-head state in the form the combine below takes: lanes of one
    // 16-lane row with the same lane % 4 hold equal sums over that row's rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m_run[j] = j == 0 ? quad_bcast<0>(m_lane) : j == 1 ? quad_bcast<1>(m_lane) : j == 2 ? quad_bcast<2>(m_lane)
                                                                                            : quad_bcast<3>(m_lane);
      l_run[j] = j == 0 ? quad_bcast<0>(l_lane) : j == 1 ? quad_bcast<1>(l_lane) : j == 2 ? quad_bcast<2>(l_lane)
                                                                                            : quad_bcast<3>(l_lane);
    }
  } else {
    for (int i0 = 0; chunk_of(i0) < n_chunks; i0 += U) {
      KVec kb[U], vb[U];
      float ks[U], vs[U];
      load_batch(i0, kb, vb, ks, vs);
      process_batch(i0, kb, vb, ks, vs);
    }
  }

  // ---- combine the rows of each wave, then the waves (fixed order) -----------
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      l_run[j] += __shfl_xor(l_run[j], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] += __shfl_xor(acc[j][e], off);
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) lds_o[wave][j][lane * EPL + e] = acc[j][e];
      if (lane == 0) {
        lds_m[wave][j] = m_run[j];
        lds_l[wave][j] = l_run[j];
      }
    }
  }
  __syncthreads();

  for (int i = tid; i < NQ * D; i += NW * kWave) {
    const int j = i / D;
    const int col = i - j * D;
    const int m = j / G;
    const int g = j - m * G;
    const int sm = seq[m];
    if (sm < 0) continue;                           // no such member
    // a member's context must hold the whole range
    const int cm = ctx_m[m];
    const bool member_ok = cm >= t0 + n_tok && cm <= a.max_context_len;
    const int parts_m = scheduled ? nslot_m[m] : (cm + part - 1) / part;
    float M = lds_m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, lds_m[w][j]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = __builtin_amdgcn_exp2f(lds_m[w][j] - M);   // 0 for a wave without rows
      o = fmaf(lds_o[w][j][col], sw, o);
      l = fmaf(lds_l[w][j], sw, l);
    }
    float r = o / l;
    const bool poison = any_bad || range_bad || !member_ok || parts_m < 1 || slot >= parts_m;
    if (poison) r = __builtin_nanf("");
    const int hq = h * G + g;
    if (m > 0 && !(cm > 0 && cm <= a.max_context_len)) continue;   // its own slot-0 item writes it
    if (parts_m <= 1) {
      store_out<QT>(a.out, (static_cast<int64_t>(sm) * Hq + hq) * D + col, r);
    } else {
      const int64_t row = (static_cast<int64_t>(sm) * Hq + hq) * a.slot_stride + slot;
      store_out_nt<QT>(a.ws_o, row * D + col, r);
      if (col == 0) a.ws_ml[row] = make_float2(poison ? __builtin_nanf("") : M, poison ? __builtin_nanf("") : l);
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
using KernelFn = void (*)(DecodeArgs);

template <int QT, int KT, int D, int BS>
KernelFn pick_group(int g, int qm) {
  if (qm == kShareWidth) return g == 1 ? pa_decode_partition_kernel<QT, KT, D, BS, 1, kShareWidth> : nullptr;
  if (qm != 1) return nullptr;
  switch (g) {
    case 1: return pa_decode_partition_kernel<QT, KT, D, BS, 1, 1>;
    case 2: return pa_decode_partition_kernel<QT, KT, D, BS, 2, 1>;
    case 4: return pa_decode_partition_kernel<QT, KT, D, BS, 4, 1>;
    case 8: return pa_decode_partition_kernel<QT, KT, D, BS, 8, 1>;
  }
  return nullptr;
}
template <int QT, int KT, int D>
KernelFn pick_block(int bs, int g, int qm) {
  switch (bs) {
    case 8: return pick_group<QT, KT, D, 8>(g, qm);
    case 16: return pick_group<QT, KT, D, 16>(g, qm);
    case 32: return pick_group<QT, KT, D, 32>(g, qm);
  }
  return nullptr;
}
template <int QT, int KT>
KernelFn pick_dim(int d, int bs, int g, int qm) {
  // fp32 rows of 128 elements are 512 B (32 lanes/row): 2 rows per wave load,
  // so block_size 8 still holds whole wave loads.
  switch (d) {
    case 64: return pick_block<QT, KT, 64>(bs, g, qm);
    case 128: return pick_block<QT, KT, 128>(bs, g, qm);
  }
  return nullptr;
}
// qt: query / output type; kt: cache type (the same, or FP8 codes under
// fp16 / bf16 queries).
KernelFn pick_partition_kernel(int qt, int kt, int d, int bs, int g, int qm) {
  if (kt == PA_FP8_E4M3) {
    switch (qt) {
      case PA_F16: return pick_dim<PA_F16, PA_FP8_E4M3>(d, bs, g, qm);
      case PA_BF16: return pick_dim<PA_BF16, PA_FP8_E4M3>(d, bs, g, qm);
    }
    return nullptr;
  }
  if (kt == PA_INT8) {
    switch (qt) {
      case PA_F16: return pick_dim<PA_F16, PA_INT8>(d, bs, g, qm);
      case PA_BF16: return pick_dim<PA_BF16, PA_INT8>(d, bs, g, qm);
    }
    return nullptr;
  }
  if (qt != kt) return nullptr;
  switch (kt) {
    case PA_F32: return pick_dim<PA_F32, PA_F32>(d, bs, g, qm);
    case PA_F16: return pick_dim<PA_F16, PA_F16>(d, bs, g, qm);
    case PA_BF16: return pick_dim<PA_BF16, PA_BF16>(d, bs, g, qm);
  }
  return nullptr;
}
KernelFn pick_mid_merge_kernel(int dt, int d) {
#define PA_MERGE_CASE(DT_)                                             \
  case DT_:                                                            \
    return d == 64 ? pa_decode_merge_mid_kernel<DT_, 64>               \
                   : (d == 128 ? pa_decode_merge_mid_kernel<DT_, 128> : nullptr);
  switch (dt) {
    PA_MERGE_CASE(PA_F32)
    PA_MERGE_CASE(PA_F16)
    PA_MERGE_CASE(PA_BF16)
  }
#undef PA_MERGE_CASE
  return nullptr;
}
KernelFn pick_small_merge_kernel(int dt, int d) {
#define PA_MERGE_CASE(DT_)                                             \
  case DT_:                                                            \
    return d == 64 ? pa_decode_merge_small_kernel<DT_, 64>             \
                   : (d == 128 ? pa_decode_merge_small_kernel<DT_, 128> : nullptr);
  switch (dt) {
    PA_MERGE_CASE(PA_F32)
    PA_MERGE_CASE(PA_F16)
    PA_MERGE_CASE(PA_BF16)
  }
#undef PA_MERGE_CASE
  return nullptr;
}
KernelFn pick_merge_kernel(int dt, int d) {
#define PA_MERGE_CASE(DT_)                                       \
  case DT_:                                                      \
    return d == 64 ? pa_decode_merge_kernel<DT_, 64>             \
                   : (d == 128 ? pa_decode_merge_kernel<DT_, 128> : nullptr);
  switch (dt) {
    PA_MERGE_CASE(PA_F32)
    PA_MERGE_CASE(PA_F16)
    PA_MERGE_CASE(PA_BF16)
  }
#undef PA_MERGE_CASE
  return nullptr;
}

bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Validates the descriptor; fills the derived partition size / count.
int check_desc(const pa_decode_desc* d, int* part, int* max_ctx, int* max_parts) {
  if (d == nullptr) return fail(PA_ERR_INVALID, "pa_decode: NULL desc");
  const pa_cache_desc& c = d->cache;
  if (c.dtype != PA_F32 && c.dtype != PA_F16 && c.dtype != PA_BF16 && c.dtype != PA_FP8_E4M3 && c.dtype != PA_INT8)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: dtype %d", c.dtype);
  if ((c.dtype == PA_FP8_E4M3 || c.dtype == PA_INT8) && d->q_dtype != PA_F16 && d->q_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: FP8 / INT8 caches take f16 or bf16 queries (q_dtype %d)", d->q_dtype);
  if (c.head_dim != 64 && c.head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d", c.head_dim);
  if (c.block_size != 8 && c.block_size != 16 && c.block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d", c.block_size);
  if (c.num_kv_heads <= 0 || c.num_blocks < 1 || d->num_seqs < 0 || d->max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID, "pa_decode: kv_heads=%d blocks=%d seqs=%d max_blocks=%d", c.num_kv_heads,
                c.num_blocks, d->num_seqs, d->max_blocks_per_seq);
  if (d->num_q_heads <= 0 || d->num_q_heads % c.num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "pa_decode: num_q_heads %d not a multiple of num_kv_heads %d", d->num_q_heads,
                c.num_kv_heads);
  const int g = d->num_q_heads / c.num_kv_heads;
  if (!group_ok(g)) return fail(PA_ERR_UNSUPPORTED, "pa_decode: query heads per KV head = %d", g);
  if (d->num_seqs > 65535 || c.num_kv_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: more than 65535 sequences or KV heads");
  // a partition's block ids live in one VGPR: at most 64 blocks
  const int max_part = kWave * c.block_size;
  const int p = d->partition_size == 0 ? (kDefaultPartition < max_part ? kDefaultPartition : max_part)
                                       : d->partition_size;
  if (p <= 0 || p > max_part || p % c.block_size != 0)
    return fail(PA_ERR_INVALID, "pa_decode: partition_size %d (multiple of block_size, <= %d)", p, max_part);
  const int64_t cap = static_cast<int64_t>(d->max_blocks_per_seq) * c.block_size;
  int64_t mc = d->max_context_len == 0 ? cap : d->max_context_len;
  if (mc < 0 || mc > cap || mc > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_decode: max_context_len %d outside [0, %lld]", d->max_context_len, (long long)cap);
  const int64_t np = mc == 0 ? 1 : (mc + p - 1) / p;
  if (np > 65535) return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld partitions", (long long)np);
  *part = p;
  *max_ctx = static_cast<int>(mc);
  *max_parts = static_cast<int>(np);
  return PA_OK;
}

// Partial-result slots per (sequence, query head). Dense launch: one per
// partition. Scheduled launch: a sequence split into shared and own ranges
// has at most one range more than partitions.
int slot_stride_for(bool scheduled, int max_parts) { return scheduled ? max_parts + 1 : max_parts; }

// Workspace layout: (m, l) float2 [S][Hq][slots] | o float [S][Hq][slots][d].
// None is needed by a dense launch whose contexts fit one partition.
size_t workspace_for(const pa_decode_desc* d, bool scheduled, int max_parts) {
  const int slots = slot_stride_for(scheduled, max_parts);
  if (!scheduled && slots <= 1) return 0;
  const size_t rows = static_cast<size_t>(d->num_seqs) * d->num_q_heads * slots;
  // partial outputs in the output dtype (q's for an FP8 cache), max and sum in fp32
  const int out_dtype = (d->cache.dtype == PA_FP8_E4M3 || d->cache.dtype == PA_INT8) ? d->q_dtype : d->cache.dtype;
  const size_t out_bytes = out_dtype == PA_F32 ? sizeof(float) : sizeof(uint16_t);
  return rows * (static_cast<size_t>(d->cache.head_dim) * out_bytes + sizeof(float2));
}

// PA_DEBUG: check table entries, lengths and the schedule on the host (synchronises).
// Compact tables are first expanded to padded rows through the items' row
// fields; a sequence that leads no item (only a member of shared ones) has no
// known row, and its block checks are skipped.
int debug_check(const int32_t* block_tables, const int32_t* context_lens, const pa_decode_desc* d, int max_ctx,
                int slot_stride, hipStream_t stream) {
  const int S = d->num_seqs;
  const int MB = d->max_blocks_per_seq;
  const bool compact = d->compact_tables != 0;
  std::vector<int32_t> ctx(S), tab(static_cast<size_t>(S) * MB, -1);
  std::vector<int32_t> flat(compact ? d->table_entries : 0);
  std::vector<int32_t> w(d->work != nullptr ? static_cast<size_t>(kItemInts) * d->num_work : 0);
  std::vector<int32_t> mem(d->work != nullptr && d->members && d->num_members > 0 ? d->num_members : 0);
  std::vector<int32_t> nslots(d->work != nullptr ? S : 0);
  std::vector<int32_t>& tsrc = compact ? flat : tab;
  auto copy_in = [&](void* dst, const void* src, size_t bytes) {
    return bytes == 0 || hipMemcpyAsync(dst, src, bytes, hipMemcpyDefault, stream) == hipSuccess;
  };
  if (!copy_in(ctx.data(), context_lens, S * sizeof(int32_t)) ||
      !copy_in(tsrc.data(), block_tables, tsrc.size() * sizeof(int32_t)) ||
      !copy_in(w.data(), d->work, w.size() * sizeof(int32_t)) ||
      !copy_in(nslots.data(), d->num_slots, nslots.size() * sizeof(int32_t)) ||
      !copy_in(mem.data(), d->members, mem.size() * sizeof(int32_t)) || hipStreamSynchronize(stream) != hipSuccess)
    return fail(PA_ERR_HIP, "pa_decode: debug copy failed");
  const int B = d->cache.block_size;
  std::vector<char> known(S, compact ? 0 : 1);
  if (compact) {
    for (int i = 0; i < d->num_work; ++i) {
      const int32_t* it = &w[static_cast<size_t>(kItemInts) * i];
      const int32_t s = it[0], rb = it[6], rc = it[7];
      if (s < 0 || s >= S) return fail(PA_ERR_INVALID, "pa_decode: schedule item %d: sequence %d", i, s);
      if (rb < 0 || rc < 0 || rc > MB || rb > d->table_entries - rc || rc < (ctx[s] + B - 1) / B)
        return fail(PA_ERR_INVALID, "pa_decode: schedule item %d: table row (%d, %d) of %d entries", i, rb, rc,
                    d->table_entries);
      int32_t* row = &tab[static_cast<size_t>(s) * MB];
      if (known[s]) {
        for (int j = 0; j < rc; ++j)
          if (row[j] != flat[rb + j]) return fail(PA_ERR_INVALID, "pa_decode: items of sequence %d name different rows", s);
        continue;
      }
      std::copy(flat.begin() + rb, flat.begin() + rb + rc, row);
      known[s] = 1;
    }
  }
  for (int s = 0; s < S; ++s) {
    if (ctx[s] < 0 || ctx[s] > max_ctx) return fail(PA_ERR_INVALID, "pa_decode: context_lens[%d] = %d", s, ctx[s]);
    if (!known[s]) continue;
    const int nb = (ctx[s] + B - 1) / B;
    for (int j = 0; j < nb; ++j) {
      const int32_t b = tab[static_cast<size_t>(s) * MB + j];
      if (b < 0 || b >= d->cache.num_blocks)
        return fail(PA_ERR_INVALID, "pa_decode: block_tables[%d][%d] = %d outside the pool", s, j, b);
    }
  }
  if (d->work == nullptr) return PA_OK;
  // The schedule: each sequence's ranges (its own items and the shared items
  // it is a member of) must tile [0, ctx) exactly, one per slot 0..n-1 with
  // n = num_slots; a member must hold the item's blocks over the range.
  struct Range { int32_t t0, n, slot; };
  std::vector<std::vector<Range>> ranges(S);
  for (int i = 0; i < d->num_work; ++i) {
    const int32_t* it = &w[static_cast<size_t>(kItemInts) * i];
    const int32_t s = it[0], t0 = it[1], n = it[2], slot = it[3], mb = it[4], mc = it[5];
    if (s < 0 || s >= S) return fail(PA_ERR_INVALID, "pa_decode: schedule item %d: sequence %d", i, s);
    ranges[s].push_back({t0, n, slot});
    if (mc == 0) continue;
    if (mem.empty() || mc < 0 || mc >= kShareWidth || mb < 0 || mb + mc > static_cast<int64_t>(mem.size()))
      return fail(PA_ERR_INVALID, "pa_decode: schedule item %d has bad members (%d, %d)", i, mb, mc);
    for (int k = 0; k < mc; ++k) {
      const int32_t m = mem[mb + k];
      if (m < 0 || m >= S || m == s) return fail(PA_ERR_INVALID, "pa_decode: schedule item %d: member %d", i, m);
      if (t0 < 0 || n < 1 || t0 % B || t0 + n > ctx[m] || t0 + n > ctx[s])
        return fail(PA_ERR_INVALID, "pa_decode: member %d of item %d covers the range differently", m, i);
      for (int j = t0 / B; known[m] && j < (t0 + n + B - 1) / B; ++j)
        if (tab[static_cast<size_t>(m) * MB + j] != tab[static_cast<size_t>(s) * MB + j])
          return fail(PA_ERR_INVALID, "pa_decode: member %d of item %d does not share its blocks", m, i);
      ranges[m].push_back({t0, n, slot});
    }
  }
  for (int s = 0; s < S; ++s) {
    auto& r = ranges[s];
    std::sort(r.begin(), r.end(), [](const Range& x, const Range& y) { return x.t0 < y.t0; });
    if (ctx[s] == 0) {
      if (r.size() != 1 || r[0].slot != 0 || nslots[s] != 1)
        return fail(PA_ERR_INVALID, "pa_decode: schedule: sequence %d (empty) needs one slot-0 item", s);
      continue;
    }
    if (nslots[s] < 1 || nslots[s] > slot_stride || static_cast<int>(r.size()) != nslots[s])
      return fail(PA_ERR_INVALID, "pa_decode: schedule: sequence %d has %zu ranges, num_slots %d", s, r.size(), nslots[s]);
    std::vector<char> used(nslots[s], 0);
    int32_t t = 0;
    for (const Range& x : r) {
      if (x.t0 != t || x.n < 1 || x.n > kWave * B || x.t0 % B || x.slot < 0 || x.slot >= nslots[s] || used[x.slot]++)
        return fail(PA_ERR_INVALID, "pa_decode: schedule: sequence %d range [%d, +%d) slot %d breaks the tiling", s,
                    x.t0, x.n, x.slot);
      t += x.n;
    }
    if (t != ctx[s]) return fail(PA_ERR_INVALID, "pa_decode: schedule covers %d of %d tokens of sequence %d", t, ctx[s], s);
  }
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

// ---------------------------------------------------------------------------
// library-held scratch for pa_decode_noalloc
// ---------------------------------------------------------------------------
// Partial results of a split launch live in this device array when the caller
// cannot allocate a workspace. Every GPU the library runs on holds its own
// copy (zero at load) until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up once
// per device with hipGetSymbolAddress, and only that address is used.
namespace pagedkv {
namespace {
constexpr size_t kScratchBytes = size_t{16} << 20;   // 16 MiB
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on first use).
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "pa_decode_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(PA_ERR_HIP, "pa_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}
}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, float scale, void* out, const pa_decode_desc* desc,
                      void* stream) {
  clear_error();
  int part, max_ctx, max_parts;
  int rc = check_desc(desc, &part, &max_ctx, &max_parts);
  if (rc != PA_OK) return rc;
  const size_t need = workspace_for(desc, desc->work != nullptr, max_parts);
  if (need > kScratchBytes)
    return fail(PA_ERR_INVALID, "pa_decode_noalloc: this launch needs %zu bytes of scratch, the library holds %zu "
                "(use pa_decode with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    rc = scratch_for_current_device(&ws);
    if (rc != PA_OK) return rc;
  }
  pa_decode_desc d = *desc;
  d.workspace = ws;
  d.workspace_bytes = need > 0 ? kScratchBytes : 0;
  return pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale, out, &d, stream);
}

size_t pa_decode_workspace_bytes(const pa_decode_desc* desc, int32_t scheduled) {
  clear_error();
  int part, max_ctx, max_parts;
  if (check_desc(desc, &part, &max_ctx, &max_parts) != PA_OK) return 0;
  return workspace_for(desc, scheduled != 0, max_parts);
}

int pa_decode_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
  return pa_decode_supported_kv(dtype, dtype, head_dim, block_size, group);
}

int pa_decode_supported_kv(int32_t q_dtype, int32_t cache_dtype, int32_t head_dim, int32_t block_size,
                           int32_t group) {
  if (!group_ok(group)) return 0;
  return pick_partition_kernel(q_dtype, cache_dtype, head_dim, block_size, group, 1) != nullptr ? 1 : 0;
}

int pa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              const int32_t* context_lens, float scale, void* out, const pa_decode_desc* desc, void* stream_) {
  clear_error();
  int part, max_ctx, max_parts;
  int rc = check_desc(desc, &part, &max_ctx, &max_parts);
  if (rc != PA_OK) return rc;
  const int S = desc->num_seqs;
  if (S == 0) return PA_OK;
  const auto aligned = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; };
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PA_ERR_INVALID, "pa_decode: NULL tensor pointer");
  if (!aligned(q) || !aligned(k_cache) || !aligned(v_cache) || !aligned(out) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return fail(PA_ERR_INVALID, "pa_decode: q/caches/out must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_decode: scale is not finite");
  const bool scheduled = desc->work != nullptr;
  const size_t need = workspace_for(desc, scheduled, max_parts);
  if (need > 0 && (desc->workspace == nullptr || desc->workspace_bytes < need || !aligned(desc->workspace)))
    return fail(PA_ERR_INVALID, "pa_decode: workspace of %zu bytes needed (%zu given)", need, desc->workspace_bytes);
  const int slot_stride = slot_stride_for(scheduled, max_parts);
  if (desc->work != nullptr) {
    if (desc->num_work <= 0 || (reinterpret_cast<uintptr_t>(desc->work) & 7u) ||
        static_cast<int64_t>(desc->num_work) * desc->cache.num_kv_heads > INT32_MAX)
      return fail(PA_ERR_INVALID, "pa_decode: schedule of %d items (8-byte aligned, non-empty)", desc->num_work);
    if (desc->num_slots == nullptr || (reinterpret_cast<uintptr_t>(desc->num_slots) & 3u))
      return fail(PA_ERR_INVALID, "pa_decode: a schedule needs num_slots (4-byte aligned)");
    if (desc->max_slots < 0 || desc->max_slots > slot_stride)
      return fail(PA_ERR_INVALID, "pa_decode: max_slots %d outside [0, %d]", desc->max_slots, slot_stride);
  }
  if (desc->compact_tables && (desc->work == nullptr || desc->table_entries < 0))
    return fail(PA_ERR_INVALID, "pa_decode: compact block tables need a schedule and table_entries >= 0");
  const int g = desc->num_q_heads / desc->cache.num_kv_heads;
  const bool shared = desc->work != nullptr && desc->members != nullptr && desc->num_members > 0;
  if (shared && (reinterpret_cast<uintptr_t>(desc->members) & 3u))
    return fail(PA_ERR_INVALID, "pa_decode: members must be 4-byte aligned");
  const bool fp8 = desc->cache.dtype == PA_FP8_E4M3 || desc->cache.dtype == PA_INT8;   // codes + row scales
  const int qt = fp8 ? desc->q_dtype : desc->cache.dtype;   // q / out dtype
  if (fp8 && (!desc->k_scale || !desc->v_scale || (reinterpret_cast<uintptr_t>(desc->k_scale) & 3u) ||
              (reinterpret_cast<uintptr_t>(desc->v_scale) & 3u)))
    return fail(PA_ERR_INVALID, "pa_decode: FP8 / INT8 caches need 4-byte aligned k_scale / v_scale");
  KernelFn kpart = pick_partition_kernel(qt, desc->cache.dtype, desc->cache.head_dim, desc->cache.block_size, g,
                                         shared ? kShareWidth : 1);
  if (shared && !kpart)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: shared schedule items need one query head per KV head (got %d)", g);
  KernelFn kmerge = pick_merge_kernel(qt, desc->cache.head_dim);
  if (!kpart || !kmerge) return fail(PA_ERR_UNSUPPORTED, "pa_decode: no kernel for this configuration");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (debug_enabled()) {
    rc = debug_check(block_tables, context_lens, desc, max_ctx, slot_stride, stream);
    if (rc != PA_OK) return rc;
  }

  DecodeArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.ws_ml = static_cast<float2*>(desc->workspace);
  const size_t rows = static_cast<size_t>(S) * desc->num_q_heads * slot_stride;
  a.ws_o = need > 0 ? static_cast<void*>(static_cast<float2*>(desc->workspace) + rows) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = S;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->cache.num_kv_heads;
  a.num_blocks = desc->cache.num_blocks;
  a.max_blocks_per_seq = desc->max_blocks_per_seq;
  a.max_context_len = max_ctx;
  a.partition_size = part;
  a.max_partitions = max_parts;
  a.work = desc->work;
  a.num_work = desc->num_work;
  a.members = shared ? desc->members : nullptr;
  a.num_members = shared ? desc->num_members : 0;
  a.slot_stride = slot_stride;
  a.num_slots = desc->work != nullptr ? desc->num_slots : nullptr;
  a.k_scale = fp8 ? desc->k_scale : nullptr;
  a.v_scale = fp8 ? desc->v_scale : nullptr;
  a.compact_tables = desc->compact_tables ? 1 : 0;
  a.table_entries = desc->compact_tables ? desc->table_entries : 0;

  hipEvent_t ev0 = static_cast<hipEvent_t>(desc->prof_events[0]);
  hipEvent_t ev1 = static_cast<hipEvent_t>(desc->prof_events[1]);
  if ((ev0 == nullptr) != (ev1 == nullptr)) return fail(PA_ERR_INVALID, "pa_decode: give both prof_events or none");
  dim3 grid(desc->cache.num_kv_heads, S, max_parts);
  if (desc->work != nullptr) grid = dim3(static_cast<uint32_t>(desc->num_work) * desc->cache.num_kv_heads, 1, 1);
  if (ev0 != nullptr) {
    // the events take the kernel's own start and end time: no marker packets
    // of their own between the kernels, which would stall the stream
    hipExtLaunchKernelGGL(kpart, grid, dim3(kNumWaves * kWave), 0, stream, ev0, ev1, 0, a);
  } else {
    hipLaunchKernelGGL(kpart, grid, dim3(kNumWaves * kWave), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: partition launch: %s", hipGetErrorString(e));
  // a merge is needed when some sequence has more than one partial result
  const int most_parts = desc->work != nullptr ? (desc->max_slots == 0 ? slot_stride : desc->max_slots) : max_parts;
  const bool merge = most_parts > 1;
  if (merge && most_parts <= kMergeWaveParts) {
    KernelFn ksmall = pick_small_merge_kernel(qt, desc->cache.head_dim);
    hipLaunchKernelGGL(ksmall, dim3((desc->num_q_heads + kMergeHeadsPerWg - 1) / kMergeHeadsPerWg, S),
                       dim3(kMergeHeadsPerWg * kWave), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: merge launch: %s", hipGetErrorString(e));
  } else if (merge && most_parts <= kMergeLanesMaxParts) {
    KernelFn kmid = pick_mid_merge_kernel(qt, desc->cache.head_dim);
    hipLaunchKernelGGL(kmid, dim3(desc->num_q_heads, S), dim3(4 * kWave), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: merge launch: %s", hipGetErrorString(e));
  } else if (merge) {
    hipLaunchKernelGGL(kmerge, dim3(desc->num_q_heads, S), dim3(kMergeThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: merge launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // extern "C"
