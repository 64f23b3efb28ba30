// pa_internal.h -- launch interfaces shared by the host layer (pa_api.hip)
// and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Everything a decode-partition or reduce launch needs, resolved on the host.
struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_m;    // [B][Hq][P] running max (log2 units)
  float* ws_l;    // [B][Hq][P] running sum
  float* ws_acc;  // [B][Hq][P][D] unnormalised V-weighted sums (v_scale applied)
  int32_t B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq;
  int32_t partition_size;  // tokens
  int32_t num_partitions;  // P: partitions of the longest possible sequence
  float qk_scale_log2;     // scale * k_scale * log2(e)
  float v_scale;
  int32_t out_dtype;
};

// The default split-K partition size aims for at least kTargetWaves waves (a
// few rounds of the 256 compute units of a gfx950 part) and at least
// kMinPartitions partitions of the longest sequence the table can hold.
constexpr int64_t kTargetWaves = 4096;
constexpr int64_t kMinPartitions = 4;

// Grid limit on the partition axis (grid y).
constexpr int32_t kMaxPartitions = 65535;

// Block copy: 16-byte chunks handled by one work-group (16 KiB).
constexpr int kCopySliceChunks = 1024;

hipError_t launch_decode_partition(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                                   hipStream_t stream, bool* supported);
// The two partition kernels: matrix cores for query groups of 4 or 8 over
// 16-bit or e4m3 caches, vector ALUs for everything else.
bool decode_mfma_serves(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t group);
hipError_t launch_decode_mfma(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                              hipStream_t stream, bool* supported);
hipError_t launch_decode_valu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                              hipStream_t stream, bool* supported);
hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* block_tables, const int32_t* positions, int32_t B,
                               int32_t max_blocks, int32_t block_size, int32_t* slots,
                               hipStream_t stream);
hipError_t launch_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const int32_t* slots, int32_t T, int32_t Hkv,
                                    int32_t D, int32_t block_size, int32_t num_blocks,
                                    pa_dtype src_dtype, pa_dtype kv_dtype, float k_inv_scale,
                                    float v_inv_scale, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* mapping, int32_t P,
                              int32_t num_blocks, size_t block_bytes, hipStream_t stream);

}  // namespace pa
