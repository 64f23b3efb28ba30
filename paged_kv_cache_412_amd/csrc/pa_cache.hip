// pa_cache.hip -- cache-side kernels for gfx950: slot mapping, the cache
// write (reshape_and_cache) and the copy-on-write block copy.
//
// P1 = Ultralytics glossary page "PagedAttention".
//   * Slot of a token: block table entry pos / bs, offset pos % bs (P1
//     "Sayfalama Nasıl Çalışır", code sketch write loop).
//   * Cache write: the new token's K and V rows go to that slot; an fp8 cache
//     (e4m3 or e5m2) quantises them with the pool's scale (P1 "İlgili
//     Teknikler").
//   * Block copy: a block that other sequences still use is copied before a
//     sequence writes into it (P1 "Diziler Arasında Blokları Paylaşma").
// All three are pure data movement; every byte is moved with 16-byte vector
// loads and stores.

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ slot mapping

// Slot of sequence b's token at positions[b]: -1 for a negative position, a
// position past the table, a negative block id or a slot past int32.
__device__ __forceinline__ int slot_of(const int32_t* __restrict__ tables,
                                       const int32_t* __restrict__ positions, int b, int max_blocks,
                                       int bs) {
  const int pos = positions[b];
  int slot = -1;
  if (pos >= 0 && pos / bs < max_blocks) {
    const int blk = tables[static_cast<size_t>(b) * max_blocks + pos / bs];
    const int64_t s = static_cast<int64_t>(blk) * bs + pos % bs;
    if (blk >= 0 && s <= INT32_MAX) slot = static_cast<int>(s);
  }
  return slot;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(const int32_t* __restrict__ tables,
                                                           const int32_t* __restrict__ positions,
                                                           int32_t B, int32_t max_blocks,
                                                           int32_t bs, int32_t* __restrict__ slots) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  slots[b] = slot_of(tables, positions, b, max_blocks, bs);
}

// The slot of cache-write row t (grid (T, 2)): given, or computed from the
// table and position (and then stored once, by the K work-group).
__device__ __forceinline__ int row_slot(const SlotSource& src, int t, int bs) {
  if (src.slots) return src.slots[t];
  const int slot = slot_of(src.tables, src.positions, t, src.max_blocks, bs);
  if (src.slots_out && blockIdx.y == 0 && threadIdx.x == 0) src.slots_out[t] = slot;
  return slot;
}

// ------------------------------------------------------------------ cache write

// Same dtype on both sides: a bit copy of each token's [Hkv][D] row, K and V.
// grid (T, 2): y selects K or V; 16-byte chunks strided over the work-group.
__global__ __launch_bounds__(256) void cache_copy_kernel(const u32x4* __restrict__ k_new,
                                                         const u32x4* __restrict__ v_new,
                                                         u32x4* __restrict__ k_cache,
                                                         u32x4* __restrict__ v_cache,
                                                         const SlotSource slots, int32_t bs,
                                                         int32_t row_chunks, int64_t num_slots) {
  const int t = blockIdx.x;
  const int slot = row_slot(slots, t, bs);
  if (slot < 0 || slot >= num_slots) return;
  const u32x4* src = (blockIdx.y == 0 ? k_new : v_new) + static_cast<size_t>(t) * row_chunks;
  u32x4* dst = (blockIdx.y == 0 ? k_cache : v_cache) + static_cast<size_t>(slot) * row_chunks;
  for (int i = threadIdx.x; i < row_chunks; i += blockDim.x) dst[i] = src[i];
}

// Quantise 8 source elements to 8 codes of format FMT (e4m3 or e5m2):
// code = fp8(fl32(x * inv_scale)).
template <int SRC, int FMT>
__device__ __forceinline__ u32x2 quantize8(const void* src8, float inv) {
  float x[8];
  if constexpr (SRC == PA_F32) {
    const u32x4* p = static_cast<const u32x4*>(src8);
    const u32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = u2f(a[i]);
      x[4 + i] = u2f(b[i]);
    }
  } else {
    const u32x4 a = *static_cast<const u32x4*>(src8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SRC == PA_BF16) {
        x[2 * i] = u2f(a[i] << 16);
        x[2 * i + 1] = u2f(a[i] & 0xffff0000u);
      } else {
        // bind the vector element to a scalar first: __builtin_bit_cast applied
        // to an ext-vector element expression reads element 0 whatever the index
        const uint32_t word = a[i];
        const f16x2 h = __builtin_bit_cast(f16x2, word);
        x[2 * i] = static_cast<float>(h[0]);
        x[2 * i + 1] = static_cast<float>(h[1]);
      }
    }
  }
  u32x2 out;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // one correctly rounded fp32 multiply, then the 8-bit rounding
      word |= f32_to_fp8<FMT>(x[4 * w + i] * inv) << (8 * i);
    }
    out[w] = word;
  }
  return out;
}

// grid (T, 2); each thread quantises groups of 8 elements of one row.
template <int SRC, int FMT>
__global__ __launch_bounds__(256) void cache_quant_kernel(const char* __restrict__ k_new,
                                                          const char* __restrict__ v_new,
                                                          u32x2* __restrict__ k_cache,
                                                          u32x2* __restrict__ v_cache,
                                                          const SlotSource slots, int32_t bs,
                                                          int32_t row_elems, int64_t num_slots,
                                                          float k_inv, float v_inv,
                                                          const float* __restrict__ k_scales,
                                                          const float* __restrict__ v_scales,
                                                          int32_t D) {
  constexpr int SB = Elem<SRC>::bytes;
  const int t = blockIdx.x;
  const int slot = row_slot(slots, t, bs);
  if (slot < 0 || slot >= num_slots) return;
  const bool is_k = blockIdx.y == 0;
  const char* src = (is_k ? k_new : v_new) + static_cast<size_t>(t) * row_elems * SB;
  u32x2* dst = (is_k ? k_cache : v_cache) + static_cast<size_t>(slot) * (row_elems / 8);
  const float inv = is_k ? k_inv : v_inv;
  const float* heads = is_k ? k_scales : v_scales;
  for (int i = threadIdx.x; i < row_elems / 8; i += blockDim.x) {
    // per-head scales: fl32(1 / scale) of the head these 8 elements belong
    // to (a correctly rounded division, as the pool-wide inverse on the host)
    const float hinv = heads ? 1.0f / heads[(8 * i) / D] : inv;
    dst[i] = quantize8<SRC, FMT>(src + static_cast<size_t>(i) * 8 * SB, hinv);
  }
}

// ------------------------------------------------------------------ block copy

// Flat grid of P * 2 * slices work-groups: (pair, K or V, slice), where a
// slice is kSliceChunks 16-byte chunks of one block.  Source and destination
// pools may be one pool (copy-on-write) or two (swap between device memory
// and pinned host memory, which the loads and stores reach over the host
// link).  Each thread loads all of its chunks before it stores any, so a
// work-group keeps a whole slice in flight: host-link round trips are long.
constexpr int kSliceChunks = kCopySliceChunks;
constexpr int kCopyThreads = 256;
constexpr int kChunksPerThread = kSliceChunks / kCopyThreads;
static_assert(kSliceChunks % kCopyThreads == 0, "slice shape");

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const u32x4* __restrict__ src_k, const u32x4* __restrict__ src_v, u32x4* __restrict__ dst_k,
    u32x4* __restrict__ dst_v, const int32_t* __restrict__ mapping, int32_t src_blocks,
    int32_t dst_blocks, int64_t block_chunks, int32_t slices) {
  const int slice = blockIdx.x % slices;
  const int kv = (blockIdx.x / slices) & 1;
  const int pair = blockIdx.x / (2 * slices);
  const int src = mapping[2 * pair];
  const int dst = mapping[2 * pair + 1];
  if (static_cast<unsigned>(src) >= static_cast<unsigned>(src_blocks) ||
      static_cast<unsigned>(dst) >= static_cast<unsigned>(dst_blocks))
    return;
  const u32x4* s = (kv == 0 ? src_k : src_v) + static_cast<size_t>(src) * block_chunks;
  u32x4* d = (kv == 0 ? dst_k : dst_v) + static_cast<size_t>(dst) * block_chunks;
  const int64_t beg = static_cast<int64_t>(slice) * kSliceChunks + threadIdx.x;
  u32x4 v[kChunksPerThread];
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    const int64_t i = beg + static_cast<int64_t>(k) * kCopyThreads;
    if (i < block_chunks) v[k] = s[i];
  }
#pragma unroll
  for (int k = 0; k < kChunksPerThread; ++k) {
    const int64_t i = beg + static_cast<int64_t>(k) * kCopyThreads;
    if (i < block_chunks) d[i] = v[k];
  }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* positions, int32_t B,
                               int32_t max_blocks, int32_t block_size, int32_t* slots,
                               hipStream_t stream) {
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, block_tables,
                     positions, B, max_blocks, block_size, slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const SlotSource& slots, int32_t T, int32_t Hkv,
                                    int32_t D, int32_t block_size, int32_t num_blocks,
                                    pa_dtype src_dtype, pa_dtype kv_dtype, float k_inv_scale,
                                    float v_inv_scale, const float* k_scales,
                                    const float* v_scales, hipStream_t stream) {
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const int32_t row_elems = Hkv * D;
  dim3 grid(T, 2);
  if (src_dtype == kv_dtype) {
    int ebytes = kv_dtype == PA_F32 ? 4 : (is_fp8(kv_dtype) ? 1 : 2);
    const int32_t row_chunks = row_elems * ebytes / 16;
    hipLaunchKernelGGL(cache_copy_kernel, grid, dim3(256), 0, stream,
                       static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slots, block_size,
                       row_chunks, num_slots);
  } else {
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, static_cast<const char*>(k_new),
                         static_cast<const char*>(v_new), static_cast<u32x2*>(k_cache),
                         static_cast<u32x2*>(v_cache), slots, block_size, row_elems, num_slots, k_inv_scale,
                         v_inv_scale, k_scales, v_scales, D);
    };
    const bool e5 = kv_dtype == PA_FP8_E5M2;
    if (src_dtype == PA_F32)
      e5 ? go(cache_quant_kernel<PA_F32, PA_FP8_E5M2>) : go(cache_quant_kernel<PA_F32, PA_FP8_E4M3>);
    else if (src_dtype == PA_F16)
      e5 ? go(cache_quant_kernel<PA_F16, PA_FP8_E5M2>) : go(cache_quant_kernel<PA_F16, PA_FP8_E4M3>);
    else
      e5 ? go(cache_quant_kernel<PA_BF16, PA_FP8_E5M2>) : go(cache_quant_kernel<PA_BF16, PA_FP8_E4M3>);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int32_t* mapping, int32_t P, int32_t src_blocks,
                              int32_t dst_blocks, size_t block_bytes, hipStream_t stream) {
  const int64_t block_chunks = static_cast<int64_t>(block_bytes / 16);
  const int32_t slices = static_cast<int32_t>((block_chunks + kSliceChunks - 1) / kSliceChunks);
  dim3 grid(static_cast<unsigned>(static_cast<int64_t>(P) * 2 * slices));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v),
                     static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v), mapping, src_blocks,
                     dst_blocks, block_chunks, slices);
  return hipGetLastError();
}

}  // namespace pa
