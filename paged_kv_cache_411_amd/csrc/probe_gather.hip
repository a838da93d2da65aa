// A gather probe with known bytes, for calibrating HBM byte counters and for
// the streaming ceiling of the paged-decode access pattern. Measurement only:
// built into its own library (libpagedkv_probe.so), not part of the decode
// path, and called only by the benchmark.
//
// The access pattern is the decode's ([VM] "PagedAttention的注意力计算流程":
// the K/V of a block are contiguous, the blocks are scattered): chunks of
// 4 KiB (one (block, head) of K or V at 16 tokens x 128 fp16 values) read in
// the order given by an index array, by workgroups of 4 wave64s, each lane
// loading 16 bytes per wave load with the decode's non-temporal loads, 8 wave
// loads in flight per wave. A workgroup reads `chunks_per_item` consecutive
// entries of the order (an "item", like a partition of one head). Every
// loaded word is folded into one value per wave so that no load is dead.
//
// Bytes: exactly num_chunks * 4096 read from `buf`, 4 bytes of the order per
// chunk, and 4 bytes per wave written to `sink`.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kChunkBytes = 4096;
constexpr int kWaves = 4;
constexpr int kBatch = 8;   // wave loads (1 KiB each) in flight per wave

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kWaves * 64) void probe_gather_kernel(const char* __restrict__ buf,
                                                                   int64_t buf_chunks,
                                                                   const int32_t* __restrict__ order,
                                                                   int32_t num_chunks, int32_t chunks_per_item,
                                                                   uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * chunks_per_item;
  const int64_t end = min(first + chunks_per_item, static_cast<int64_t>(num_chunks));
  const int64_t loads = (end - first) * (kChunkBytes / 1024);     // 1 KiB wave loads in the item
  uint32_t acc = 0;
  for (int64_t l0 = wave; l0 < loads; l0 += kWaves * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t l = min(l0 + static_cast<int64_t>(b) * kWaves, loads - 1);   // repeats stay in flight
      int64_t c = order[first + l / 4];
      c = c < 0 ? 0 : (c >= buf_chunks ? buf_chunks - 1 : c);
      const char* p = buf + c * kChunkBytes + (l % 4) * 1024 + lane * 16;
      v[b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
      if (l0 + static_cast<int64_t>(b) * kWaves < loads) acc ^= v[b].x ^ v[b].y ^ v[b].z ^ v[b].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  if (lane == 0) sink[blockIdx.x * kWaves + wave] = acc;
}

}  // namespace

extern "C" {

// Reads the num_chunks 4 KiB chunks of `buf` (buf_chunks of them) named by
// `order` (int32, device; entries are clamped into the buffer), in items of
// chunks_per_item chunks per workgroup; `sink` (device) receives 4 words per
// workgroup. Returns 0, or -1 for bad arguments, -4 for a launch error.
int pa_probe_gather(const void* buf, int64_t buf_chunks, const int32_t* order, int32_t num_chunks,
                    int32_t chunks_per_item, uint32_t* sink, void* stream) {
  if (buf == nullptr || order == nullptr || sink == nullptr || buf_chunks < 1 || num_chunks < 0 ||
      chunks_per_item < 1 || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return -1;
  if (num_chunks == 0) return 0;
  const int64_t grid = (static_cast<int64_t>(num_chunks) + chunks_per_item - 1) / chunks_per_item;
  hipLaunchKernelGGL(probe_gather_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kWaves * 64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(buf), buf_chunks, order, num_chunks,
                     chunks_per_item, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Words `sink` must hold for a launch: 4 per workgroup.
int64_t pa_probe_gather_sink_words(int32_t num_chunks, int32_t chunks_per_item) {
  if (num_chunks < 0 || chunks_per_item < 1) return -1;
  return (static_cast<int64_t>(num_chunks) + chunks_per_item - 1) / chunks_per_item * kWaves;
}

}  // extern "C"
