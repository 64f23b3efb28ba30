// pa_decode_common.h -- pieces shared by the two decode-partition kernels
// (the VALU kernel for small query groups and the MFMA kernel for grouped
// query attention): the work-group -> (KV head, partition, sequence) mapping,
// the per-wave block-id prefetch, and the cross-wave merge that finishes a
// partition.
//
// Both kernels compute, for one KV head g of one sequence b and one split-K
// partition of the sequence's blocks, the online-softmax state of the G query
// heads that share g (grouped-query attention, P1 = Ultralytics glossary page
// "PagedAttention", section "İlgili Teknikler"): the running maximum m of the
// scores (log2 units), the running sum l of 2^(s - m) and the unnormalised
// V-weighted sum acc.  A partition covering the whole sequence writes
// out = v_scale * acc / l directly; otherwise (m, l, v_scale * acc) go to the
// workspace for the reduce kernel.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Running-max start value: finite, so that exp2(m_old - m_new) is 0 or 1
// (never NaN) while a wave has seen no valid token; real scores are far above.
constexpr float kMaxInit = -1.0e30f;

// Grid: x = KV head (fastest), y = partition, z = sequence.  Work-groups are
// dispatched in x order, so the work-groups running at one moment read the
// rows of every KV head of the same blocks: each token row of a block is one
// contiguous Hkv*D run of the pool, and reading it in one sweep keeps DRAM
// pages open instead of touching D-element slices of many rows.
struct PartitionSpan {
  int L;        // sequence length, clamped to the table's capacity
  int jbeg;     // first logical block of the partition
  int jend;     // one past its last logical block
  bool single;  // one partition covers the sequence: write `out` directly
  bool skip;    // partition lies past the end of the sequence
};

template <int BS>
__device__ __forceinline__ PartitionSpan partition_span(const DecodeParams& p, int b, int part) {
  PartitionSpan s;
  const int max_tokens = p.max_blocks_per_seq * BS;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
  const int PB = p.partition_size / BS;
  const int nblk = (L + BS - 1) / BS;
  s.L = L;
  s.jbeg = part * PB;
  s.jend = min(s.jbeg + PB, nblk);
  s.single = L <= p.partition_size;
  s.skip = part > 0 && s.jbeg >= nblk;
  return s;
}

// Number of the partition's blocks that wave `wave` of NW handles (blocks
// jbeg + wave, jbeg + wave + NW, ...).
template <int NW>
__device__ __forceinline__ int wave_block_count(const PartitionSpan& s, int wave) {
  const int n = s.jend - s.jbeg;
  return n > wave ? (n - wave + NW - 1) / NW : 0;
}

// Block ids of up to 64 consecutive iterations of one wave, one per lane
// (lane i: iteration base + i), fetched with one vector load; each iteration
// then takes its id with v_readlane, so no scalar load sits on the path
// between two blocks.  Lanes past `cnt` hold -1.
template <int NW>
__device__ __forceinline__ int prefetch_block_ids(const int32_t* table, const PartitionSpan& s,
                                                  int wave, int base, int cnt, int lane) {
  return lane < cnt ? table[s.jbeg + wave + (base + lane) * NW] : -1;
}

__device__ __forceinline__ int block_id_at(int ids, int i) {
  return __builtin_amdgcn_readlane(ids, i);
}

// Cross-wave merge of the per-wave states held in LDS, then the partition's
// output: out (single partition) or the workspace partials.  One thread per
// (query head of the group, element).
template <int G, int D, int NW>
__device__ __forceinline__ void merge_waves_and_store(const DecodeParams& p,
                                                      const float (&sm_m)[NW][G],
                                                      const float (&sm_l)[NW][G],
                                                      const float (&sm_acc)[NW][G][D], int b,
                                                      int g, int part, bool single) {
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float M = kMaxInit;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
    float Ls = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(sm_m[w][h] - M);
      Ls = __builtin_fmaf(sm_l[w][h], a, Ls);
      A = __builtin_fmaf(sm_acc[w][h][d], a, A);
    }
    const size_t hq = static_cast<size_t>(b) * p.Hq + g * G + h;
    if (single) {
      const float o = Ls > 0.f ? (A / Ls) * p.v_scale : 0.f;
      store_out(p.out, hq * D + d, o, p.out_dtype);
    } else {
      const size_t pi = hq * p.num_partitions + part;
      p.ws_acc[pi * D + d] = A * p.v_scale;
      if (d == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = Ls;
      }
    }
  }
}

}  // namespace pa
