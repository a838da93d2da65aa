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
// block table, take q.K for every token, softmax, then walk the blocks again
// for sum(w * V). The softmax follows the five steps of [PA] §5.1: local
// maxima, global maximum, exponentials shifted by it, global sum, and the
// division. Steps 1-4 run inside one context partition (up to 512 tokens) in
// the partition kernel; for sequences longer than one partition, the merge
// kernel runs steps 2-5 again across the partitions' (max, sum, output).
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
//   * the partition's physical block ids are loaded once per wave into one
//     VGPR (lane j holds logical block j) and moved to SGPRs with v_readlane,
//     so every K/V address is scalar base + lane offset ("hoisted" block-table
//     lookup, [PA] §3.2);
//   * q.k: fp16 / bf16 dot2 instructions with fp32 accumulation, then a
//     row reduction over the LPR lanes with DPP (quad_perm, row_half_mirror,
//     row_mirror) - no LDS traffic;
//   * scores go to LDS; the partition maximum is reduced with DPP + readlane,
//     then across waves through LDS;
//   * V pass: each lane accumulates exp2(s - m) * V for its 16-byte column
//     slice in fp32 registers; rows and waves are combined once at the end in a
//     fixed order, so the result depends only on logical positions (bitwise
//     identical for any block placement);
//   * no MFMA: per (token, KV head) the pass reads 2*d*elem bytes and does
//     4*G*d flops, i.e. 2G/elem flop/byte (0.5 - 4), far below the ~20 flop/byte
//     where the vector ALUs would stop being fed by 8 TB/s of HBM.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <vector>

#include "pagedkv.h"
#include "status.h"

namespace pagedkv {
namespace {

constexpr int kWave = 64;
constexpr int kMaxPartition = 512;   // tokens per partition (LDS score buffer)
constexpr int kNumWaves = 4;         // waves per partition workgroup
constexpr int kUnroll = 8;           // 1 KiB wave loads in flight per wave

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_o;          // [S][Hq][max_partitions][D] normalised partial outputs
  float2* ws_ml;        // [S][Hq][max_partitions] (max in log2 units, sum)
  float scale_log2;     // softmax scale * log2(e): scores are kept in log2 units
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t partition_size;
  int32_t max_partitions;
};

// ---------------------------------------------------------------------------
// element formats
// ---------------------------------------------------------------------------
template <int DT> struct Fmt;
template <> struct Fmt<PA_F32> { static constexpr int kBytes = 4; };
template <> struct Fmt<PA_F16> { static constexpr int kBytes = 2; };
template <> struct Fmt<PA_BF16> { static constexpr int kBytes = 2; };

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

// Max over the whole wave of a value that is uniform inside each group of N lanes.
template <int N> __device__ __forceinline__ float wave_max_grouped(float x) {
  float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
#pragma unroll
  for (int r = N; r < kWave; r += N)
    m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), r)));
  return m;
}

__device__ __forceinline__ int readlane_i(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// ---------------------------------------------------------------------------
// partition kernel
// ---------------------------------------------------------------------------
template <int DT, int D, int BS, int G>
struct Geometry {
  static constexpr int kElem = Fmt<DT>::kBytes;
  static constexpr int kRowBytes = D * kElem;           // one token row of one head
  static constexpr int kLPR = kRowBytes / 16;            // lanes per row
  static constexpr int kRPC = kWave / kLPR;              // rows per wave load
  static constexpr int kEPL = 16 / kElem;                // elements per lane
  static constexpr int kCPB = BS / kRPC;                 // wave loads per (block, head)
  static constexpr int kBlockHeadBytes = BS * kRowBytes;
  static_assert(kRowBytes % 16 == 0 && kLPR >= 8 && kLPR <= 32, "row must be 128..512 bytes");
  static_assert(BS % kRPC == 0, "block must hold whole wave loads");
  static_assert(kMaxPartition / BS <= kWave, "partition block ids must fit one VGPR");
};

template <int DT, int D, int BS, int G>
__global__ __launch_bounds__(kNumWaves * kWave) void pa_decode_partition_kernel(DecodeArgs a) {
  using Geo = Geometry<DT, D, BS, G>;
  constexpr int LPR = Geo::kLPR, RPC = Geo::kRPC, EPL = Geo::kEPL, CPB = Geo::kCPB;
  constexpr int NW = kNumWaves, U = kUnroll;

  // LDS: scores [G][kMaxPartition]; reused after the V pass for the cross-wave
  // combine: partial outputs [NW][G][D] and sums [NW][G].
  constexpr int kScoreFloats = G * kMaxPartition;
  constexpr int kCombineFloats = NW * G * D + NW * G;
  __shared__ float lds[kScoreFloats > kCombineFloats ? kScoreFloats : kCombineFloats];
  __shared__ float lds_max[NW][G];

  const int h = blockIdx.x;                       // KV head
  const int s = blockIdx.y;                       // sequence
  const int p = a.max_partitions - 1 - static_cast<int>(blockIdx.z);   // longest work first
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Hq = a.num_q_heads;

  const int ctx = a.context_lens[s];
  const bool bad_ctx = ctx < 0 || ctx > a.max_context_len;
  const int part = a.partition_size;
  const int num_parts = bad_ctx ? 1 : (ctx + part - 1) / part;

  if (ctx == 0 || bad_ctx) {
    // empty context -> zeros; invalid length -> NaN rows (written once, by p == 0)
    if (p != 0) return;
    const float fill = bad_ctx ? __builtin_nanf("") : 0.0f;
    for (int i = tid; i < G * D; i += NW * kWave)
      store_out<DT>(a.out, (static_cast<int64_t>(s) * Hq + h * G) * D + i, fill);
    return;
  }
  if (p >= num_parts) return;

  const int t0 = p * part;
  const int n_tok = min(ctx - t0, part);
  const int n_blk = (n_tok + BS - 1) / BS;
  const int n_chunks = n_blk * CPB;

  // Block ids of the partition: lane j holds logical block t0/BS + j.
  const int32_t* table = a.block_tables + static_cast<int64_t>(s) * a.max_blocks_per_seq + t0 / BS;
  int my_blk = 0;
  bool blk_bad = false;
  if (lane < n_blk) {
    my_blk = table[lane];
    blk_bad = my_blk < 0 || my_blk >= a.num_blocks;
    if (blk_bad) my_blk = 0;   // keep every address inside the pool
  }
  const bool any_bad = __ballot(blk_bad) != 0;

  // q slices: head h*G+g, columns (lane % LPR) * EPL ...
  uint4 qv[G];
  {
    const char* qb = static_cast<const char*>(a.q) +
                     ((static_cast<int64_t>(s) * Hq + h * G) * D) * Geo::kElem + (lane % LPR) * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g] = *reinterpret_cast<const uint4*>(qb + static_cast<int64_t>(g) * Geo::kRowBytes);
  }

  const char* kbase = static_cast<const char*>(a.k_cache) + static_cast<int64_t>(h) * Geo::kBlockHeadBytes + lane * 16;
  const char* vbase = static_cast<const char*>(a.v_cache) + static_cast<int64_t>(h) * Geo::kBlockHeadBytes + lane * 16;
  const int64_t block_stride = static_cast<int64_t>(a.num_kv_heads) * Geo::kBlockHeadBytes;
  const int row_in_chunk = lane / LPR;
  const bool row_leader = (lane % LPR) == 0;

  // ---- pass 1: scores (steps 1-2 of [PA] §5.1 inside the partition) ----------
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = -INFINITY;

  for (int c0 = wave; c0 < n_chunks; c0 += NW * U) {
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * NW, n_chunks - 1);   // past the end: reload a valid chunk, ignored below
      const int phys = readlane_i(my_blk, c / CPB);
      kv[u] = *reinterpret_cast<const uint4*>(kbase + phys * block_stride + (c % CPB) * 1024);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * NW;
      if (c < n_chunks) {
        const int row = (c / CPB) * BS + (c % CPB) * RPC + row_in_chunk;   // token index in the partition
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float sc = group_sum<LPR>(dot16<DT>(qv[g], kv[u])) * a.scale_log2;
          sc = row < n_tok ? sc : -INFINITY;
          if (row_leader) lds[g * kMaxPartition + row] = sc;
          mx[g] = fmaxf(mx[g], sc);
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float m = wave_max_grouped<LPR>(mx[g]);
    if (lane == 0) lds_max[wave][g] = m;
  }
  __syncthreads();
  float m_part[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = lds_max[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, lds_max[w][g]);
    m_part[g] = m;
  }

  // ---- pass 2: exp2(s - m), their sum and sum(e * V) (steps 3-4) --------------
  float acc[G][EPL];
  float lsum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[g][j] = 0.0f;
  }
  for (int c0 = wave; c0 < n_chunks; c0 += NW * U) {
    uint4 vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + u * NW, n_chunks - 1);
      const int phys = readlane_i(my_blk, c / CPB);
      vv[u] = *reinterpret_cast<const uint4*>(vbase + phys * block_stride + (c % CPB) * 1024);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * NW;
      if (c < n_chunks) {
        const int row0 = (c / CPB) * BS + (c % CPB) * RPC;
        const int row = row0 + row_in_chunk;
        float f[EPL];
        Unpack<DT>::run(vv[u], f);
        if (row0 + RPC > n_tok) {
          // rows past the context hold stale data (possibly NaN): zero them
          // rather than rely on a zero weight
#pragma unroll
          for (int j = 0; j < EPL; ++j) f[j] = row < n_tok ? f[j] : 0.0f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float e = __builtin_amdgcn_exp2f(lds[g * kMaxPartition + row] - m_part[g]);
          lsum[g] += e;
#pragma unroll
          for (int j = 0; j < EPL; ++j) acc[g][j] = fmaf(e, f[j], acc[g][j]);
        }
      }
    }
  }

  // ---- combine rows of the wave, then waves (fixed order) ---------------------
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      lsum[g] += __shfl_xor(lsum[g], off);
#pragma unroll
      for (int j = 0; j < EPL; ++j) acc[g][j] += __shfl_xor(acc[g][j], off);
    }
  }
  __syncthreads();   // every wave is done reading scores: reuse the LDS
  float* lds_o = lds;                       // [NW][G][D]
  float* lds_l = lds + NW * G * D;          // [NW][G]
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < EPL; ++j) lds_o[(wave * G + g) * D + lane * EPL + j] = acc[g][j];
      if (lane == 0) lds_l[wave * G + g] = lsum[g];
    }
  }
  __syncthreads();

  const bool single = num_parts == 1;
  for (int i = tid; i < G * D; i += NW * kWave) {
    const int g = i / D;
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      o += lds_o[w * G * D + i];
      l += lds_l[w * G + g];
    }
    float r = o / l;
    if (any_bad) r = __builtin_nanf("");
    const int hq = h * G + g;
    if (single) {
      store_out<DT>(a.out, (static_cast<int64_t>(s) * Hq + hq) * D + (i - g * D), r);
    } else {
      const int64_t row = (static_cast<int64_t>(s) * Hq + hq) * a.max_partitions + p;
      a.ws_o[row * D + (i - g * D)] = r;
      if (i - g * D == 0) a.ws_ml[row] = make_float2(any_bad ? __builtin_nanf("") : m_part[g], any_bad ? __builtin_nanf("") : l);
    }
  }
}

// ---------------------------------------------------------------------------
// merge kernel: steps 2-5 of [PA] §5.1 across partitions
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(kWave) void pa_decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = threadIdx.x;
  const int ctx = a.context_lens[s];
  if (ctx <= 0 || ctx > a.max_context_len) return;   // written by the partition kernel
  const int P = (ctx + a.partition_size - 1) / a.partition_size;
  if (P <= 1) return;
  const int64_t row = (static_cast<int64_t>(s) * a.num_q_heads + hq) * a.max_partitions;
  const float2* ml = a.ws_ml + row;

  // global maximum (step 2)
  float m = -INFINITY;
  for (int p = 0; p < P; ++p) m = fmaxf(m, ml[p].x);
  // global sum (step 4): L = sum_p l_p * 2^(m_p - m)
  float L = 0.0f;
  for (int p = 0; p < P; ++p) L += ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - m);
  const float inv_L = 1.0f / L;
  for (int col = lane; col < D; col += kWave) {
    float o = 0.0f;
    for (int p = 0; p < P; ++p) {
      const float w = ml[p].y * __builtin_amdgcn_exp2f(ml[p].x - m);
      o = fmaf(w, a.ws_o[(row + p) * D + col], o);
    }
    store_out<DT>(a.out, (static_cast<int64_t>(s) * a.num_q_heads + hq) * D + col, o * inv_L);
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
using KernelFn = void (*)(DecodeArgs);

template <int DT, int D, int BS>
KernelFn pick_group(int g) {
  switch (g) {
    case 1: return pa_decode_partition_kernel<DT, D, BS, 1>;
    case 2: return pa_decode_partition_kernel<DT, D, BS, 2>;
    case 4: return pa_decode_partition_kernel<DT, D, BS, 4>;
    case 8: return pa_decode_partition_kernel<DT, D, BS, 8>;
  }
  return nullptr;
}
template <int DT, int D>
KernelFn pick_block(int bs, int g) {
  switch (bs) {
    case 8: return pick_group<DT, D, 8>(g);
    case 16: return pick_group<DT, D, 16>(g);
    case 32: return pick_group<DT, D, 32>(g);
  }
  return nullptr;
}
template <int DT>
KernelFn pick_dim(int d, int bs, int g) {
  // fp32 rows of 128 elements are 512 B (32 lanes/row): 2 rows per wave load,
  // so block_size 8 still holds whole wave loads.
  switch (d) {
    case 64: return pick_block<DT, 64>(bs, g);
    case 128: return pick_block<DT, 128>(bs, g);
  }
  return nullptr;
}
KernelFn pick_partition_kernel(int dt, int d, int bs, int g) {
  switch (dt) {
    case PA_F32: return pick_dim<PA_F32>(d, bs, g);
    case PA_F16: return pick_dim<PA_F16>(d, bs, g);
    case PA_BF16: return pick_dim<PA_BF16>(d, bs, g);
  }
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
  if (c.dtype != PA_F32 && c.dtype != PA_F16 && c.dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: dtype %d", c.dtype);
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
  const int p = d->partition_size == 0 ? kMaxPartition : d->partition_size;
  if (p <= 0 || p > kMaxPartition || p % c.block_size != 0)
    return fail(PA_ERR_INVALID, "pa_decode: partition_size %d (multiple of block_size, <= %d)", p, kMaxPartition);
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

size_t workspace_for(const pa_decode_desc* d, int max_parts) {
  if (max_parts <= 1) return 0;
  const size_t rows = static_cast<size_t>(d->num_seqs) * d->num_q_heads * max_parts;
  return rows * (static_cast<size_t>(d->cache.head_dim) * sizeof(float) + sizeof(float2));
}

// PA_DEBUG: check table entries and lengths on the host (synchronises).
int debug_check(const int32_t* block_tables, const int32_t* context_lens, const pa_decode_desc* d, int max_ctx,
                hipStream_t stream) {
  const int S = d->num_seqs;
  std::vector<int32_t> ctx(S), tab(static_cast<size_t>(S) * d->max_blocks_per_seq);
  if (hipMemcpyAsync(ctx.data(), context_lens, S * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      (!tab.empty() && hipMemcpyAsync(tab.data(), block_tables, tab.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                                      stream) != hipSuccess) ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(PA_ERR_HIP, "pa_decode: debug copy failed");
  const int B = d->cache.block_size;
  for (int s = 0; s < S; ++s) {
    if (ctx[s] < 0 || ctx[s] > max_ctx) return fail(PA_ERR_INVALID, "pa_decode: context_lens[%d] = %d", s, ctx[s]);
    const int nb = (ctx[s] + B - 1) / B;
    for (int j = 0; j < nb; ++j) {
      const int32_t b = tab[static_cast<size_t>(s) * d->max_blocks_per_seq + j];
      if (b < 0 || b >= d->cache.num_blocks)
        return fail(PA_ERR_INVALID, "pa_decode: block_tables[%d][%d] = %d outside the pool", s, j, b);
    }
  }
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

extern "C" {

size_t pa_decode_workspace_bytes(const pa_decode_desc* desc) {
  clear_error();
  int part, max_ctx, max_parts;
  if (check_desc(desc, &part, &max_ctx, &max_parts) != PA_OK) return 0;
  return workspace_for(desc, max_parts);
}

int pa_decode_supported(int32_t dtype, int32_t head_dim, int32_t block_size, int32_t group) {
  if (!group_ok(group)) return 0;
  return pick_partition_kernel(dtype, head_dim, block_size, group) != nullptr ? 1 : 0;
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
  const size_t need = workspace_for(desc, max_parts);
  if (need > 0 && (desc->workspace == nullptr || desc->workspace_bytes < need || !aligned(desc->workspace)))
    return fail(PA_ERR_INVALID, "pa_decode: workspace of %zu bytes needed (%zu given)", need, desc->workspace_bytes);
  const int g = desc->num_q_heads / desc->cache.num_kv_heads;
  KernelFn kpart = pick_partition_kernel(desc->cache.dtype, desc->cache.head_dim, desc->cache.block_size, g);
  KernelFn kmerge = pick_merge_kernel(desc->cache.dtype, desc->cache.head_dim);
  if (!kpart || !kmerge) return fail(PA_ERR_UNSUPPORTED, "pa_decode: no kernel for this configuration");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (debug_enabled()) {
    rc = debug_check(block_tables, context_lens, desc, max_ctx, stream);
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
  a.ws_o = need > 0 ? reinterpret_cast<float*>(static_cast<float2*>(desc->workspace) +
                                               static_cast<size_t>(S) * desc->num_q_heads * max_parts)
                    : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = S;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->cache.num_kv_heads;
  a.num_blocks = desc->cache.num_blocks;
  a.max_blocks_per_seq = desc->max_blocks_per_seq;
  a.max_context_len = max_ctx;
  a.partition_size = part;
  a.max_partitions = max_parts;

  hipEvent_t ev0 = static_cast<hipEvent_t>(desc->prof_events[0]);
  hipEvent_t ev1 = static_cast<hipEvent_t>(desc->prof_events[1]);
  if (ev0 && hipEventRecord(ev0, stream) != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: hipEventRecord");
  dim3 grid(desc->cache.num_kv_heads, S, max_parts);
  hipLaunchKernelGGL(kpart, grid, dim3(kNumWaves * kWave), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: partition launch: %s", hipGetErrorString(e));
  if (ev1 && hipEventRecord(ev1, stream) != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: hipEventRecord");
  if (max_parts > 1) {
    hipLaunchKernelGGL(kmerge, dim3(desc->num_q_heads, S), dim3(kWave), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_decode: merge launch: %s", hipGetErrorString(e));
  }
  return PA_OK;
}

}  // extern "C"
