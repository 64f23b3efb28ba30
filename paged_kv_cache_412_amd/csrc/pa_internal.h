// pa_internal.h -- launch interfaces shared by the host layer (pa_api.hip)
// and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Everything a decode-partition launch needs, resolved on the host.
//
// Two schedules split the work of a decode step among work-groups of
// heads_per_wg waves (one KV head each):
//  * fixed partitions (partition_size > 0 in the call): work-group
//    (head group, sequence, partition) covers partition_size tokens of one
//    sequence; partials rows are ws_row(hq, partition).
//  * balanced (partition_size == 0): from the prefix sums prefix[b] of the
//    sequences' block counts, work-group (head group, w) of `groups` per head
//    group takes blocks [w*F/groups, (w+1)*F/groups) of the concatenation of
//    all sequences (F = prefix[B]).  It writes the output of every sequence
//    it covers whole and partials only for the (at most two) sequences it
//    covers in part; rows are balanced_row(...).
// Split sequences are combined either by the last of their segments to
// finish, in the same launch (fused; arrival counters, pa_decode_common.h),
// or by the reduce kernel launched after it.
// Balanced schedule: up to this many sequences, the attention kernel's
// work-groups compute the block-count prefix sums themselves (in LDS) instead
// of a plan kernel launched before them.
constexpr int kInlinePlanMaxB = 1024;

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;  // partial rows x D: unnormalised V-weighted sums (v_scale applied)
  float* ws_m;    // partial rows: running max (log2 units)
  float* ws_l;    // partial rows: running sum
  int32_t* prefix;  // balanced: [B+1] block-count prefix sums (plan kernel, B > kInlinePlanMaxB)
  int32_t* counters;  // [Hkv][B] arrivals of a split sequence's segments; zero between calls
  // block_size, num_blocks and max_blocks_per_seq count the blocks the
  // kernels walk: 2^sub_shift of them make one block of the table (a block
  // is contiguous, so its halves are blocks of half the size); table rows
  // hold max_blocks_per_seq >> sub_shift entries
  int32_t B, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq;
  int32_t sub_shift;
  int32_t partition_size;  // fixed: tokens per partition
  int32_t num_partitions;  // fixed: partitions of the longest possible sequence
  int32_t balanced;        // 1 = balanced schedule
  int32_t heads_per_wg;    // waves (KV heads) per work-group
  int32_t head_groups;     // ceil(Hkv / heads_per_wg)
  int32_t groups;          // balanced: work-groups per head group
  int32_t inline_plan;     // balanced, B <= kInlinePlanMaxB: each work-group computes the plan
  int32_t fused;           // 1: the partition kernels combine split sequences (no reduce launch)
  float qk_scale_log2;     // scale * k_scale * log2(e) (scale * log2(e) with per-head scales)
  float v_scale;
  const float* k_scales;   // per-head scales [Hkv] (device) or nullptr
  const float* v_scales;
  int32_t out_dtype;
};

// Row of the split-K partials of query head hq (= b*Hq + h) and partition
// `part` (fixed schedule).  Partition-major: the work-groups that run
// together (one partition of many sequences) write one contiguous region.
__host__ __device__ inline size_t ws_row(const DecodeParams& p, size_t hq, int part) {
  return static_cast<size_t>(part) * (static_cast<size_t>(p.B) * p.Hq) + hq;
}

// Row of the balanced schedule's partials: work-group w of head group hg,
// slot `which` (0: the first sequence of its range, 1: the last), wave
// (KV head within the group) and query q of the KV head's group of G.
__host__ __device__ inline size_t balanced_row(const DecodeParams& p, int hg, int w, int which,
                                               int wave, int q) {
  const int G = p.Hq / p.Hkv;
  return ((static_cast<size_t>(hg) * p.groups + w) * 2 + which) *
             (static_cast<size_t>(p.heads_per_wg) * G) +
         static_cast<size_t>(wave) * G + q;
}

// Work-groups per head group that take part: at most one per block, so that
// every one of them owns at least one block (w*F/n < (w+1)*F/n for n <= F).
__host__ __device__ inline int balanced_groups(const DecodeParams& p, int64_t F) {
  return static_cast<int>(F < p.groups ? F : p.groups);
}

// First block (in the concatenation of all sequences' blocks) of balanced
// work-group w out of n, for F blocks in all.
__host__ __device__ inline int64_t balanced_start(int64_t F, int w, int n) {
  return static_cast<int64_t>(w) * F / n;
}

// The balanced work-group whose range holds block x: the largest w with
// balanced_start(F, w, n) <= x.
__host__ __device__ inline int balanced_owner(int64_t F, int64_t x, int n) {
  return static_cast<int>(((x + 1) * n - 1) / F);
}

// Balanced schedule: at most this many waves in one launch bounds the
// workspace (16 waves on each of 256 compute units).
constexpr int64_t kBalancedMaxWaves = 4096;

// Grid limit on the partition axis (grid y).
constexpr int32_t kMaxPartitions = 65535;

// Everything a prefill launch needs, resolved on the host.  Work-group
// (sequence b, KV head, query tile) covers up to kPrefillRows rows of (new
// token, query head of the KV head's group) pairs: floor(128 / G)
// consecutive new tokens of sequence b with all G query heads each.
struct PrefillParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* q_starts;  // [B+1]
  int32_t B, T, max_q_len, Hq, Hkv, D, block_size, num_blocks, max_blocks_per_seq;
  int32_t q_tiles;          // query tiles per (sequence, KV head): ceil(max_q_len / floor(128/G))
  int32_t total_groups;     // B * Hkv * q_tiles (the 1-D grid)
  float qk_scale_log2;      // scale * k_scale * log2(e) (scale * log2(e) with per-head scales)
  float v_scale;
  const float* k_scales;    // per-head scales [Hkv] (device) or nullptr
  const float* v_scales;
  int32_t out_dtype;
};

constexpr int kPrefillRows = 128;  // (token, head) rows per work-group: 4 waves x 32
constexpr int kPrefillKeys = 64;   // keys per LDS tile of the prefill kernel

bool prefill_serves(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t D, int32_t block_size,
                    int32_t group);
hipError_t launch_prefill(const PrefillParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                          hipStream_t stream, bool* supported);
hipError_t launch_prefill_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                       const int32_t* q_starts, int32_t B, int32_t T,
                                       int32_t max_blocks, int32_t block_size, int32_t* slots,
                                       hipStream_t stream);

// Block copy: 16-byte chunks handled by one work-group (16 KiB).
constexpr int kCopySliceChunks = 1024;

hipError_t launch_decode_partition(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                                   hipStream_t stream, bool* supported);
// Waves per work-group of the partition kernel that serves these arguments.
int32_t decode_heads_per_wg(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t Hq, int32_t Hkv);
int32_t decode_mfma_heads();  // most KV heads per work-group of each kernel
int32_t decode_valu_heads();
// Work-groups of `threads` threads running kernel `fn` that one compute unit
// of the current device holds at once, from the runtime's occupancy
// calculator, cached per (device, kernel); 0 when the runtime cannot say.
int32_t groups_per_cu(const void* fn, int threads);
// Compute units of the current device (cached); 256 (gfx950) if unknown.
int32_t compute_units();
// Work-groups of that kernel one compute unit holds at once (0 if unknown).
int32_t decode_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype);
int32_t decode_mfma_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype);
int32_t decode_valu_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype);
hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream);
// The two partition kernels: matrix cores for query groups of 3 to 16 over
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
// Where the cache write takes each row's slot: from `slots`, or (slots null)
// computed from the row's block table and position as the slot mapping does,
// and then also stored to slots_out when that is not null.
struct SlotSource {
  const int32_t* slots;
  const int32_t* tables;     // [T][max_blocks]
  const int32_t* positions;  // [T]
  int32_t max_blocks;
  int32_t* slots_out;
};
// The cache write; an 8-bit cache takes one inverse scale per pool, or (when
// k_scales is not null) one scale per KV head from device arrays.
hipError_t launch_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache,
                                    void* v_cache, const SlotSource& slots, int32_t T, int32_t Hkv,
                                    int32_t D, int32_t block_size, int32_t num_blocks,
                                    pa_dtype src_dtype, pa_dtype kv_dtype, float k_inv_scale,
                                    float v_inv_scale, const float* k_scales,
                                    const float* v_scales, hipStream_t stream);
// Whole-block copies from the source pools to the destination pools (the
// same pools for copy-on-write, a device and a pinned host pool for swap).
hipError_t launch_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              const int32_t* mapping, int32_t P, int32_t src_blocks,
                              int32_t dst_blocks, size_t block_bytes, hipStream_t stream);

}  // namespace pa
