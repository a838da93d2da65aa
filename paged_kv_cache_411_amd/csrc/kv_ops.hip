// kv_append and copy_blocks for gfx950, and their C ABI entry points.
//
// Pages cited:
//   [VM]  "vLLM用虚拟内存分页思想管理KV Cache" (aiqz.cc)
//   [PA]  "PagedAttention：大模型KV Cache分页管理优化实践" (intelliparadigm.com)
//
// Both are byte moves: 16-byte vector loads and stores of raw bits, so the
// result is bit-exact for every dtype (NaN payloads and signed zeros kept).
//   kv_append   - [PA] §3.3 按需分配策略 step 4: a new token's K and V vectors go
//                 to its slot (block slot / B, offset slot % B) for every head.
//   copy_blocks - [VM] "写时复制与块共享机制" and [PA] §4.1: before a shared block
//                 is modified, its whole content (every head, every slot, K and
//                 V) is copied to the writer's new block.
//   swap_blocks - [VM] "显存管理与调度策略设计": the blocks of a request that
//                 is evicted move whole to CPU memory, and back to (other)
//                 device blocks when the request is scheduled again.
// Ids and slots are range-checked on the device (out-of-range entries are
// skipped), so no input content can make these kernels touch memory outside
// the caches.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <unordered_set>
#include <vector>

#include "internal.h"
#include "pagedkv.h"
#include "status.h"

namespace pagedkv {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kCopyThreads = 256;
constexpr int kCopyVecsPerThread = 4;   // 16 KiB per workgroup

constexpr int kAppendBatch = 4;         // 16-byte vectors of K and of V each thread has in flight

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The new rows are read once and the cache rows are not read again until a
// later decode: both directions stream past the caches.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ void stream_store(uint4* p, uint4 x) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x), reinterpret_cast<u32x4*>(p));
}

// Progress word for the host (a decode step's done_flag): this kernel has
// started, so every launch enqueued before it on the stream has completed.
// One thread stores the value into pinned host memory with a system-scope
// (vector) store; the host polls the word.
__device__ __forceinline__ void mark_progress(uint64_t* flag, uint64_t value) {
  if (flag != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
    __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// All heads' rows of K and V of token i (row_vecs 16-byte vectors per head
// row), by one workgroup: each thread loads up to kAppendBatch vectors of K
// and of V before it stores any, so the workgroup's whole token is in flight
// at once (640 vectors each for 40 heads of 256 B). kEarlyRows issues the
// first batch of row loads before the slot is known, beside the slot's own
// load (which may cross the bus from pinned host memory): a decode step's
// tokens all have slots, so the rows are wanted anyway; without it a token
// whose slot is -1 (a cached prompt row) reads nothing.
template <bool kEarlyRows>
__device__ __forceinline__ void append_token(const uint4* __restrict__ k, const uint4* __restrict__ v,
                                             const int64_t* __restrict__ slot_mapping, uint4* __restrict__ k_cache,
                                             uint4* __restrict__ v_cache, int num_kv_heads, int block_size,
                                             int row_vecs, int64_t num_slots, int64_t i) {
  const int64_t slot = slot_mapping[i];
  if (!kEarlyRows && (slot < 0 || slot >= num_slots)) return;
  const int per_token = num_kv_heads * row_vecs;
  for (int base = 0; base < per_token; base += kAppendThreads * kAppendBatch) {
    uint4 kk[kAppendBatch], vv[kAppendBatch];
#pragma unroll
    for (int j = 0; j < kAppendBatch; ++j) {
      const int idx = base + j * kAppendThreads + static_cast<int>(threadIdx.x);
      if (idx < per_token) {
        const int64_t src = i * per_token + idx;
        kk[j] = stream_load(k + src);
        vv[j] = stream_load(v + src);
      }
    }
    if (kEarlyRows && (slot < 0 || slot >= num_slots)) return;
    const int64_t blk = slot / block_size;
    const int64_t off = slot - blk * block_size;
#pragma unroll
    for (int j = 0; j < kAppendBatch; ++j) {
      const int idx = base + j * kAppendThreads + static_cast<int>(threadIdx.x);
      if (idx < per_token) {
        const int h = idx / row_vecs;
        const int c = idx - h * row_vecs;
        const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * row_vecs + c;
        stream_store(k_cache + dst, kk[j]);
        stream_store(v_cache + dst, vv[j]);
      }
    }
  }
}

// One workgroup per token.
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int num_kv_heads, int block_size, int row_vecs,
    int64_t num_slots) {
  append_token<false>(k, v, slot_mapping, k_cache, v_cache, num_kv_heads, block_size, row_vecs, num_slots,
                      blockIdx.x);
}

// kv_append and a staging copy in one launch: the first stage_wgs workgroups
// copy stage_n 16-byte vectors (grid-stride among themselves), the rest append
// one token each. The two parts touch disjoint memory.
__global__ __launch_bounds__(kAppendThreads) void kv_append_staged_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int num_kv_heads, int block_size, int row_vecs,
    int64_t num_slots, uint4* __restrict__ stage_dst, const uint4* __restrict__ stage_src, int64_t stage_n,
    int stage_wgs, uint64_t* done_flag, uint64_t done_value) {
  mark_progress(done_flag, done_value);
  if (static_cast<int>(blockIdx.x) < stage_wgs) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAppendThreads + threadIdx.x; i < stage_n;
         i += static_cast<int64_t>(stage_wgs) * kAppendThreads)
      stage_dst[i] = stage_src[i];
    return;
  }
  append_token<true>(k, v, slot_mapping, k_cache, v_cache, num_kv_heads, block_size, row_vecs, num_slots,
                     static_cast<int64_t>(blockIdx.x) - stage_wgs);
}

// grid (slices of a block, pairs, 2 = K/V): each workgroup copies one 16 KiB
// slice of one block from a source pool to a destination pool - the same
// pool for copy-on-write, the device cache and the host swap space for swaps.
// Source and destination blocks of one call never overlap (distinct
// destinations, and no destination that is a source of the same pool), and a
// thread loads its whole share before it stores any of it.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const uint4* src_k, const uint4* src_v, uint4* dst_k, uint4* dst_v, const int64_t* __restrict__ pairs,
    int64_t block_vecs, int64_t src_blocks, int64_t dst_blocks) {
  const int64_t src = pairs[2 * static_cast<int64_t>(blockIdx.y)];
  const int64_t dst = pairs[2 * static_cast<int64_t>(blockIdx.y) + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* from = (blockIdx.z == 0 ? src_k : src_v) + src * block_vecs;
  uint4* to = (blockIdx.z == 0 ? dst_k : dst_v) + dst * block_vecs;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kCopyThreads * kCopyVecsPerThread + threadIdx.x;
  uint4 r[kCopyVecsPerThread];
#pragma unroll
  for (int j = 0; j < kCopyVecsPerThread; ++j) {
    const int64_t e = base + j * kCopyThreads;
    if (e < block_vecs) r[j] = from[e];
  }
#pragma unroll
  for (int j = 0; j < kCopyVecsPerThread; ++j) {
    const int64_t e = base + j * kCopyThreads;
    if (e < block_vecs) to[e] = r[j];
  }
}

// ---------------------------------------------------------------------------
// FP8 (E4M3) quantising append
// ---------------------------------------------------------------------------
// E4M3 code of y, |y| <= 448 and finite: round to nearest, ties to even.
// Subnormals (|y| < 2^-6) are multiples of 2^-9: the code is the rounded
// multiple itself (8 lands exactly on the smallest normal, code 0x08).
// Normals keep the top 3 of fp32's 23 mantissa bits, rounded; a carry out of
// the mantissa moves to the next exponent.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  int k = static_cast<int>((u >> 23) & 0xFFu) - 127;
  const uint32_t m23 = u & 0x7FFFFFu;
  uint32_t m3 = m23 >> 20;
  const uint32_t rem = m23 & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
  if (m3 == 8u) {
    m3 = 0;
    ++k;
  }
  return sign | (static_cast<uint32_t>(k + 7) << 3) | m3;
}

constexpr int kQuantHeadsPerWg = 4;   // one wave per (token, head): K in lanes 0-31, V in lanes 32-63

// EPL consecutive source elements as fp32 (8 or 16 bytes of a 16-bit source,
// 8 or 16 of fp32: one load).
template <int SRC, int EPL> __device__ __forceinline__ void load_elems(const void* base, int64_t i, float (&x)[EPL]);
template <> __device__ __forceinline__ void load_elems<PA_F32, 4>(const void* base, int64_t i, float (&x)[4]) {
  const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
  x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
template <> __device__ __forceinline__ void load_elems<PA_F32, 2>(const void* base, int64_t i, float (&x)[2]) {
  const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + i);
  x[0] = v.x; x[1] = v.y;
}
template <int SRC, int EPL> __device__ __forceinline__ void load_elems(const void* base, int64_t i, float (&x)[EPL]) {
  static_assert(SRC == PA_F16 || SRC == PA_BF16, "16-bit source");
  uint32_t w[EPL / 2];
  if constexpr (EPL == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
    w[0] = v.x; w[1] = v.y;
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + i);
  }
#pragma unroll
  for (int j = 0; j < EPL / 2; ++j) {
    if constexpr (SRC == PA_F16) {
      x[2 * j] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] & 0xffffu)));
      x[2 * j + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w[j] >> 16)));
    } else {
      x[2 * j] = __builtin_bit_cast(float, w[j] << 16);
      x[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
    }
  }
}

// Quantise one (token, head) row of K (lanes 0-31) and the same row of V
// (lanes 32-63) with one wave: scale = max |x| / 448 (fp32, correctly
// rounded), codes = E4M3(clamp(x / scale)) (0 when the scale is 0); INT8:
// scale = max |x| / 127, codes = x / scale rounded to nearest, ties to even.
// Each lane takes D / 32 consecutive elements and returns their codes packed
// in one word, so they leave as one 2- or 4-byte store (store_kv_row) and a
// half-wave writes its 64- or 128-byte code row in one instruction.
struct QuantRow {
  uint32_t packed;
  float scale;
};

template <int SRC, int D, int FMT>
__device__ __forceinline__ QuantRow quantize_kv_row(const void* k, const void* v, int64_t src_off, int lane) {
  constexpr int EPL = D / 32;
  static_assert(EPL == 2 || EPL == 4, "head_dim 64 or 128");
  const bool is_v = lane >= 32;
  const int l = lane & 31;
  float x[EPL];
  load_elems<SRC, EPL>(is_v ? v : k, src_off + l * EPL, x);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));   // within each half
  constexpr float kTop = FMT == PA_FP8_E4M3 ? 448.0f : 127.0f;
  const float scale = amax / kTop;
  uint32_t packed = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    uint32_t c = 0;
    if (scale > 0.0f) {
      const float y = fminf(fmaxf(x[e] / scale, -kTop), kTop);
      if constexpr (FMT == PA_FP8_E4M3) c = encode_e4m3(y);
      else c = static_cast<uint32_t>(static_cast<int32_t>(__builtin_rintf(y))) & 0xffu;
    }
    packed |= c << (8 * e);
  }
  return {packed, scale};
}

// Stores what quantize_kv_row returned as row `row` ([N][Hkv][B] order) of
// the codes and scales; lanes 0 and 32 write the scales.
template <int D>
__device__ __forceinline__ void store_kv_row(QuantRow r, uint8_t* k_codes, uint8_t* v_codes, float* k_scales,
                                             float* v_scales, int64_t row, int lane) {
  constexpr int EPL = D / 32;
  const bool is_v = lane >= 32;
  const int l = lane & 31;
  uint8_t* dst = (is_v ? v_codes : k_codes) + row * D + l * EPL;
  if constexpr (EPL == 4) {
    *reinterpret_cast<uint32_t*>(dst) = r.packed;
  } else {
    *reinterpret_cast<uint16_t*>(dst) = static_cast<uint16_t>(r.packed);
  }
  if (l == 0) (is_v ? v_scales : k_scales)[row] = r.scale;
}

// Workgroups [0, stage_wgs) copy the staging bytes (as kv_append_staged); the
// rest quantise: workgroup stage_wgs + t * ceil(Hkv / 4) + j serves heads
// 4j .. 4j + 3 of token t, one wave each.
template <int SRC, int D, int FMT>
__global__ __launch_bounds__(kAppendThreads) void kv_append_fp8_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache, float* __restrict__ k_scale,
    float* __restrict__ v_scale, int num_kv_heads, int block_size, int64_t num_slots, uint4* __restrict__ stage_dst,
    const uint4* __restrict__ stage_src, int64_t stage_n, int stage_wgs, uint64_t* done_flag, uint64_t done_value) {
  mark_progress(done_flag, done_value);
  if (static_cast<int>(blockIdx.x) < stage_wgs) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kAppendThreads + threadIdx.x; i < stage_n;
         i += static_cast<int64_t>(stage_wgs) * kAppendThreads)
      stage_dst[i] = stage_src[i];
    return;
  }
  const int groups = (num_kv_heads + kQuantHeadsPerWg - 1) / kQuantHeadsPerWg;
  const int64_t w = static_cast<int64_t>(blockIdx.x) - stage_wgs;
  const int64_t t = w / groups;
  const int h = static_cast<int>(w - t * groups) * kQuantHeadsPerWg + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (h >= num_kv_heads) return;
  // the slot's load (over the bus from pinned host memory in a decode step)
  // and the row's loads and quantisation overlap
  const int64_t slot = slot_mapping[t];
  const QuantRow r = quantize_kv_row<SRC, D, FMT>(k, v, (t * num_kv_heads + h) * D, lane);
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  store_kv_row<D>(r, k_cache, v_cache, k_scale, v_scale, (blk * num_kv_heads + h) * block_size + off, lane);
}

// Plain 16-byte copy, grid-stride; src may be pinned host memory (read over
// the bus by the kernel itself).
__global__ __launch_bounds__(kCopyThreads) void stage_copy_kernel(uint4* __restrict__ dst,
                                                                 const uint4* __restrict__ src, int64_t n,
                                                                 uint64_t* done_flag, uint64_t done_value) {
  mark_progress(done_flag, done_value);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kCopyThreads)
    dst[i] = src[i];
}

bool quantized(int dtype) { return dtype == PA_FP8_E4M3 || dtype == PA_INT8; }
int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : (quantized(dtype) ? 1 : 2); }

int check_cache(const pa_cache_desc* c, const char* who) {
  if (c == nullptr) return fail(PA_ERR_INVALID, "%s: NULL desc", who);
  if (c->dtype != PA_F32 && c->dtype != PA_F16 && c->dtype != PA_BF16 && !quantized(c->dtype))
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", who, c->dtype);
  const int eb = elem_bytes(c->dtype);
  if (c->num_blocks < 0 || c->num_kv_heads <= 0 || c->block_size <= 0 || c->head_dim <= 0)
    return fail(PA_ERR_INVALID, "%s: blocks=%d kv_heads=%d block_size=%d head_dim=%d", who, c->num_blocks,
                c->num_kv_heads, c->block_size, c->head_dim);
  if ((static_cast<int64_t>(c->head_dim) * eb) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim * element bytes must be a multiple of 16", who);
  return PA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pagedkv

using namespace pagedkv;

namespace {

// Validation shared by kv_append and kv_append_staged (and the PA_DEBUG slot
// check); fills the row geometry.
int check_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                 void* v_cache, const pa_cache_desc* desc, hipStream_t stream, const char* who, int* row_vecs,
                 int64_t* num_slots) {
  int rc = check_cache(desc, who);
  if (rc != PA_OK) return rc;
  if (quantized(desc->dtype))
    return fail(PA_ERR_INVALID, "%s: FP8 / INT8 caches take kv_append_fp8 (codes and scales)", who);
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "%s: num_tokens %d", who, num_tokens);
  const int eb = elem_bytes(desc->dtype);
  *row_vecs = desc->head_dim * eb / 16;
  *num_slots = static_cast<int64_t>(desc->num_blocks) * desc->block_size;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(PA_ERR_INVALID, "%s: NULL pointer", who);
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return fail(PA_ERR_INVALID, "%s: k/v/caches must be 16-byte aligned", who);
  if (debug_enabled()) {
    std::vector<int64_t> s(num_tokens);
    if (hipMemcpyAsync(s.data(), slot_mapping, num_tokens * sizeof(int64_t), hipMemcpyDefault, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return fail(PA_ERR_HIP, "%s: debug copy failed", who);
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (s[i] < 0) continue;
      if (s[i] >= *num_slots)
        return fail(PA_ERR_INVALID, "%s: slot_mapping[%d] = %lld outside the pool", who, i, (long long)s[i]);
      if (!seen.insert(s[i]).second) return fail(PA_ERR_INVALID, "%s: slot %lld appears twice", who, (long long)s[i]);
    }
  }
  return PA_OK;
}

// Whole-block copies from the block arrays (src_k, src_v) to (dst_k, dst_v),
// block_vecs 16-byte vectors per block; pairs are checked under PA_DEBUG by
// the caller.
int launch_block_copy(const void* src_k, const void* src_v, void* dst_k, void* dst_v, const int64_t* pairs,
                      int32_t num_pairs, int64_t block_vecs, int64_t src_blocks, int64_t dst_blocks,
                      hipStream_t stream, const char* who) {
  const int64_t per_wg = static_cast<int64_t>(kCopyThreads) * kCopyVecsPerThread;
  const int64_t slices = (block_vecs + per_wg - 1) / per_wg;
  if (slices > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "%s: block too large", who);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(slices), num_pairs, 2), dim3(kCopyThreads), 0,
                     stream, static_cast<const uint4*>(src_k), static_cast<const uint4*>(src_v),
                     static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), pairs, block_vecs, src_blocks,
                     dst_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch: %s", who, hipGetErrorString(e));
  return PA_OK;
}

// PA_DEBUG check of copy pairs (device or pinned host memory): sources in the
// source pool, destinations in the destination pool and distinct, and - when
// both sides are the same pool - no destination that is also a source.
int check_pairs(const int64_t* src_dst_pairs, int32_t num_pairs, int64_t src_blocks, int64_t dst_blocks,
                bool same_pool, hipStream_t stream, const char* who) {
  std::vector<int64_t> pr(2 * static_cast<size_t>(num_pairs));
  if (hipMemcpyAsync(pr.data(), src_dst_pairs, pr.size() * sizeof(int64_t), hipMemcpyDefault, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: debug copy failed", who);
  std::unordered_set<int64_t> dsts, srcs;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int64_t s = pr[2 * i], d = pr[2 * i + 1];
    if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%lld, %lld) outside the pool", who, i, (long long)s, (long long)d);
    if (!dsts.insert(d).second) return fail(PA_ERR_INVALID, "%s: destination %lld repeated", who, (long long)d);
    srcs.insert(s);
  }
  if (same_pool)
    for (int64_t d : dsts)
      if (srcs.count(d))
        return fail(PA_ERR_INVALID, "%s: block %lld is both source and destination", who, (long long)d);
  return PA_OK;
}

}  // namespace

extern "C" {

int kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
              void* v_cache, const pa_cache_desc* desc, void* stream_) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int row_vecs;
  int64_t num_slots;
  int rc = check_append(k, v, slot_mapping, num_tokens, k_cache, v_cache, desc, stream, "kv_append", &row_vecs,
                        &num_slots);
  if (rc != PA_OK || num_tokens == 0) return rc;
  hipLaunchKernelGGL(kv_append_kernel, dim3(num_tokens), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), desc->num_kv_heads,
                     desc->block_size, row_vecs, num_slots);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_append: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int kv_append_staged(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                     void* v_cache, const pa_cache_desc* desc, void* stage_dst, const void* stage_src,
                     size_t stage_bytes, void* stream_) {
  return pagedkv::append_staged(k, v, slot_mapping, num_tokens, k_cache, v_cache, desc, stage_dst, stage_src,
                                stage_bytes, stream_, nullptr, 0);
}

}  // extern "C"

int pagedkv::append_staged(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                           void* k_cache, void* v_cache, const pa_cache_desc* desc, void* stage_dst,
                           const void* stage_src, size_t stage_bytes, void* stream_, uint64_t* done_flag,
                           uint64_t done_value) {
  clear_error();
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  int row_vecs;
  int64_t num_slots;
  int rc = check_append(k, v, slot_mapping, num_tokens, k_cache, v_cache, desc, stream, "kv_append_staged",
                        &row_vecs, &num_slots);
  if (rc != PA_OK) return rc;
  if (stage_bytes > 0 && (!stage_dst || !stage_src || !aligned16(stage_dst) || !aligned16(stage_src) ||
                          stage_bytes % 16 != 0))
    return fail(PA_ERR_INVALID, "kv_append_staged: staging pointers and size must be multiples of 16 bytes");
  const int64_t stage_n = static_cast<int64_t>(stage_bytes / 16);
  const int64_t want = (stage_n + kAppendThreads - 1) / kAppendThreads;
  const int stage_wgs = static_cast<int>(want < 256 ? want : 256);
  const int64_t grid = static_cast<int64_t>(stage_wgs) + num_tokens;
  if (grid == 0) return PA_OK;
  hipLaunchKernelGGL(kv_append_staged_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k), static_cast<const uint4*>(v), slot_mapping,
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), desc->num_kv_heads,
                     desc->block_size, row_vecs, num_slots, static_cast<uint4*>(stage_dst),
                     static_cast<const uint4*>(stage_src), stage_n, stage_wgs, done_flag, done_value);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_append_staged: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" {

int copy_blocks(void* k_cache, void* v_cache, const int64_t* src_dst_pairs, int32_t num_pairs,
                const pa_cache_desc* desc, void* stream_) {
  clear_error();
  int rc = check_cache(desc, "copy_blocks");
  if (rc != PA_OK) return rc;
  if (quantized(desc->dtype))
    return fail(PA_ERR_INVALID, "copy_blocks: FP8 / INT8 caches take copy_blocks_fp8 (codes and scales)");
  if (num_pairs < 0 || num_pairs > 65535) return fail(PA_ERR_INVALID, "copy_blocks: num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !src_dst_pairs) return fail(PA_ERR_INVALID, "copy_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || (reinterpret_cast<uintptr_t>(src_dst_pairs) & 7u))
    return fail(PA_ERR_INVALID, "copy_blocks: caches must be 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (debug_enabled()) {
    const int rc = check_pairs(src_dst_pairs, num_pairs, desc->num_blocks, desc->num_blocks, true, stream,
                               "copy_blocks");
    if (rc != PA_OK) return rc;
  }
  const int eb = elem_bytes(desc->dtype);
  const int64_t block_vecs = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * desc->head_dim * eb / 16;
  return launch_block_copy(k_cache, v_cache, k_cache, v_cache, src_dst_pairs, num_pairs, block_vecs, desc->num_blocks,
                           desc->num_blocks, stream, "copy_blocks");
}

}  // extern "C"

extern "C" int kv_append_fp8(const void* k, const void* v, int32_t src_dtype, const int64_t* slot_mapping,
                             int32_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                             const pa_cache_desc* desc, void* stage_dst, const void* stage_src, size_t stage_bytes,
                             void* stream_) {
  return pagedkv::append_fp8(k, v, src_dtype, slot_mapping, num_tokens, k_cache, v_cache, k_scale, v_scale, desc,
                             stage_dst, stage_src, stage_bytes, stream_, nullptr, 0);
}

int pagedkv::append_fp8(const void* k, const void* v, int32_t src_dtype, const int64_t* slot_mapping,
                        int32_t num_tokens, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                        const pa_cache_desc* desc, void* stage_dst, const void* stage_src, size_t stage_bytes,
                        void* stream_, uint64_t* done_flag, uint64_t done_value) {
  clear_error();
  int rc = check_cache(desc, "kv_append_fp8");
  if (rc != PA_OK) return rc;
  if (!quantized(desc->dtype))
    return fail(PA_ERR_INVALID, "kv_append_fp8: the cache dtype must be PA_FP8_E4M3 or PA_INT8");
  if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "kv_append_fp8: source dtype %d", src_dtype);
  if (desc->head_dim != 64 && desc->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "kv_append_fp8: head_dim %d (64 or 128)", desc->head_dim);
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "kv_append_fp8: num_tokens %d", num_tokens);
  if (stage_bytes > 0 && (!stage_dst || !stage_src || !aligned16(stage_dst) || !aligned16(stage_src) ||
                          stage_bytes % 16 != 0))
    return fail(PA_ERR_INVALID, "kv_append_fp8: staging pointers and size must be multiples of 16 bytes");
  if (num_tokens > 0 && (!k || !v || !slot_mapping || !k_cache || !v_cache || !k_scale || !v_scale))
    return fail(PA_ERR_INVALID, "kv_append_fp8: NULL pointer");
  if (num_tokens > 0 && ((reinterpret_cast<uintptr_t>(slot_mapping) & 7u) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
                         (reinterpret_cast<uintptr_t>(v_scale) & 3u)))
    return fail(PA_ERR_INVALID, "kv_append_fp8: misaligned slot_mapping or scales");
  if (num_tokens > 0 && (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)))
    return fail(PA_ERR_INVALID, "kv_append_fp8: k/v/caches must be 16-byte aligned");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const int64_t num_slots = static_cast<int64_t>(desc->num_blocks) * desc->block_size;
  if (debug_enabled() && num_tokens > 0) {
    std::vector<int64_t> sl(num_tokens);
    if (hipMemcpyAsync(sl.data(), slot_mapping, num_tokens * sizeof(int64_t), hipMemcpyDefault, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return fail(PA_ERR_HIP, "kv_append_fp8: debug copy failed");
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (sl[i] < 0) continue;
      if (sl[i] >= num_slots)
        return fail(PA_ERR_INVALID, "kv_append_fp8: slot_mapping[%d] = %lld outside the pool", i, (long long)sl[i]);
      if (!seen.insert(sl[i]).second) return fail(PA_ERR_INVALID, "kv_append_fp8: slot %lld appears twice", (long long)sl[i]);
    }
  }
  const int64_t stage_n = static_cast<int64_t>(stage_bytes / 16);
  const int64_t want = (stage_n + kAppendThreads - 1) / kAppendThreads;
  const int stage_wgs = static_cast<int>(want < 256 ? want : 256);
  const int groups = (desc->num_kv_heads + kQuantHeadsPerWg - 1) / kQuantHeadsPerWg;
  const int64_t grid = static_cast<int64_t>(stage_wgs) + static_cast<int64_t>(num_tokens) * groups;
  if (grid == 0) return PA_OK;
  if (grid > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "kv_append_fp8: too many tokens");
  using Fn = void (*)(const void*, const void*, const int64_t*, uint8_t*, uint8_t*, float*, float*, int, int, int64_t,
                      uint4*, const uint4*, int64_t, int, uint64_t*, uint64_t);
  Fn fn = nullptr;
  const bool d64 = desc->head_dim == 64;
#define PA_APPEND_CASE(FMT_)                                                                                    \
  switch (src_dtype) {                                                                                          \
    case PA_F32: fn = d64 ? kv_append_fp8_kernel<PA_F32, 64, FMT_> : kv_append_fp8_kernel<PA_F32, 128, FMT_>; break; \
    case PA_F16: fn = d64 ? kv_append_fp8_kernel<PA_F16, 64, FMT_> : kv_append_fp8_kernel<PA_F16, 128, FMT_>; break; \
    case PA_BF16:                                                                                               \
      fn = d64 ? kv_append_fp8_kernel<PA_BF16, 64, FMT_> : kv_append_fp8_kernel<PA_BF16, 128, FMT_>;           \
      break;                                                                                                    \
  }
  if (desc->dtype == PA_FP8_E4M3) {
    PA_APPEND_CASE(PA_FP8_E4M3)
  } else {
    PA_APPEND_CASE(PA_INT8)
  }
#undef PA_APPEND_CASE
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(kAppendThreads), 0, stream, k, v, slot_mapping,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), k_scale, v_scale,
                     desc->num_kv_heads, desc->block_size, num_slots, static_cast<uint4*>(stage_dst),
                     static_cast<const uint4*>(stage_src), stage_n, stage_wgs, done_flag, done_value);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "kv_append_fp8: launch: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" {

int copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int64_t* src_dst_pairs,
                    int32_t num_pairs, const pa_cache_desc* desc, void* stream_) {
  clear_error();
  int rc = check_cache(desc, "copy_blocks_fp8");
  if (rc != PA_OK) return rc;
  if (!quantized(desc->dtype))
    return fail(PA_ERR_INVALID, "copy_blocks_fp8: the cache dtype must be PA_FP8_E4M3 or PA_INT8");
  if (num_pairs < 0 || num_pairs > 65535) return fail(PA_ERR_INVALID, "copy_blocks_fp8: num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_scale || !v_scale || !src_dst_pairs)
    return fail(PA_ERR_INVALID, "copy_blocks_fp8: NULL pointer");
  const int64_t scale_bytes = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * 4;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_scale) || !aligned16(v_scale) ||
      (reinterpret_cast<uintptr_t>(src_dst_pairs) & 7u) || scale_bytes % 16 != 0)
    return fail(PA_ERR_INVALID, "copy_blocks_fp8: caches and scales must be 16-byte aligned (Hkv * B a multiple of 4)");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (debug_enabled()) {
    rc = check_pairs(src_dst_pairs, num_pairs, desc->num_blocks, desc->num_blocks, true, stream, "copy_blocks_fp8");
    if (rc != PA_OK) return rc;
  }
  const int64_t code_vecs = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * desc->head_dim / 16;
  rc = launch_block_copy(k_cache, v_cache, k_cache, v_cache, src_dst_pairs, num_pairs, code_vecs, desc->num_blocks,
                         desc->num_blocks, stream, "copy_blocks_fp8");
  if (rc != PA_OK) return rc;
  return launch_block_copy(k_scale, v_scale, k_scale, v_scale, src_dst_pairs, num_pairs, scale_bytes / 16,
                           desc->num_blocks, desc->num_blocks, stream, "copy_blocks_fp8");
}

int swap_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const pa_cache_desc* desc,
                void* swap_k, void* swap_v, float* swap_k_scale, float* swap_v_scale, int32_t swap_num_blocks,
                const int64_t* src_dst_pairs, int32_t num_pairs, int32_t direction, void* stream_) {
  clear_error();
  int rc = check_cache(desc, "swap_blocks");
  if (rc != PA_OK) return rc;
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID, "swap_blocks: direction %d (PA_SWAP_OUT or PA_SWAP_IN)", direction);
  if (swap_num_blocks < 0) return fail(PA_ERR_INVALID, "swap_blocks: swap_num_blocks %d", swap_num_blocks);
  if (num_pairs < 0 || num_pairs > 65535) return fail(PA_ERR_INVALID, "swap_blocks: num_pairs %d", num_pairs);
  if (num_pairs == 0) return PA_OK;
  const bool fp8 = quantized(desc->dtype);   // codes with a scale per row
  if (!k_cache || !v_cache || !swap_k || !swap_v || !src_dst_pairs) return fail(PA_ERR_INVALID, "swap_blocks: NULL pointer");
  if (fp8 && (!k_scale || !v_scale || !swap_k_scale || !swap_v_scale))
    return fail(PA_ERR_INVALID, "swap_blocks: an FP8 / INT8 cache needs its scales on both sides");
  if (!fp8 && (k_scale || v_scale || swap_k_scale || swap_v_scale))
    return fail(PA_ERR_INVALID, "swap_blocks: scales are only for FP8 / INT8 caches");
  const int64_t scale_bytes = static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * 4;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(swap_k) || !aligned16(swap_v) ||
      (reinterpret_cast<uintptr_t>(src_dst_pairs) & 7u))
    return fail(PA_ERR_INVALID, "swap_blocks: pools must be 16-byte aligned");
  if (fp8 && (!aligned16(k_scale) || !aligned16(v_scale) || !aligned16(swap_k_scale) || !aligned16(swap_v_scale) ||
              scale_bytes % 16 != 0))
    return fail(PA_ERR_INVALID, "swap_blocks: scales must be 16-byte aligned (Hkv * B a multiple of 4)");
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  const bool out = direction == PA_SWAP_OUT;
  const int64_t src_blocks = out ? desc->num_blocks : swap_num_blocks;
  const int64_t dst_blocks = out ? swap_num_blocks : desc->num_blocks;
  if (debug_enabled()) {
    rc = check_pairs(src_dst_pairs, num_pairs, src_blocks, dst_blocks, false, stream, "swap_blocks");
    if (rc != PA_OK) return rc;
  }
  const int64_t block_vecs =
      static_cast<int64_t>(desc->num_kv_heads) * desc->block_size * desc->head_dim * elem_bytes(desc->dtype) / 16;
  rc = out ? launch_block_copy(k_cache, v_cache, swap_k, swap_v, src_dst_pairs, num_pairs, block_vecs, src_blocks,
                               dst_blocks, stream, "swap_blocks")
           : launch_block_copy(swap_k, swap_v, k_cache, v_cache, src_dst_pairs, num_pairs, block_vecs, src_blocks,
                               dst_blocks, stream, "swap_blocks");
  if (rc != PA_OK || !fp8) return rc;
  return out ? launch_block_copy(k_scale, v_scale, swap_k_scale, swap_v_scale, src_dst_pairs, num_pairs,
                                 scale_bytes / 16, src_blocks, dst_blocks, stream, "swap_blocks")
             : launch_block_copy(swap_k_scale, swap_v_scale, k_scale, v_scale, src_dst_pairs, num_pairs,
                                 scale_bytes / 16, src_blocks, dst_blocks, stream, "swap_blocks");
}

int pa_stage_copy(void* dst, const void* src, size_t bytes, void* stream_) {
  return pagedkv::stage_copy(dst, src, bytes, stream_, nullptr, 0);
}

}  // extern "C"

int pagedkv::stage_copy(void* dst, const void* src, size_t bytes, void* stream_, uint64_t* done_flag,
                        uint64_t done_value) {
  clear_error();
  if (bytes == 0) return PA_OK;
  if (!dst || !src) return fail(PA_ERR_INVALID, "pa_stage_copy: NULL pointer");
  if (!aligned16(dst) || !aligned16(src) || bytes % 16 != 0)
    return fail(PA_ERR_INVALID, "pa_stage_copy: pointers and size must be multiples of 16 bytes");
  const int64_t n = static_cast<int64_t>(bytes / 16);
  const int64_t want = (n + kCopyThreads - 1) / kCopyThreads;
  const int grid = static_cast<int>(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(stage_copy_kernel, dim3(grid), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream_),
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n, done_flag, done_value);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "pa_stage_copy: launch: %s", hipGetErrorString(e));
  return PA_OK;
}
