// pa_decode_common.h -- pieces shared by the two decode-partition kernels
// (the VALU kernel for small query groups and the MFMA kernel for grouped
// query attention): the work-group -> (KV heads, partition, sequence)
// mapping, the per-wave block-id prefetch, the load pipeline, and the store
// of a finished partition.
//
// Both kernels compute, for one KV head g of one sequence b and one split-K
// partition of the sequence's blocks, the online-softmax state of the G query
// heads that share g (grouped-query attention, P1 = Ultralytics glossary page
// "PagedAttention", section "İlgili Teknikler"): the running maximum m of the
// scores (log2 units), the running sum l of 2^(s - m) and the unnormalised
// V-weighted sum acc.  A partition covering the whole sequence writes
// out = v_scale * acc / l directly; otherwise (m, l, v_scale * acc) go to the
// workspace for the reduce kernel.
//
// Work decomposition.  One wave64 per (KV head, partition, sequence); a
// work-group holds the waves of up to NW consecutive KV heads of the same
// partition (NW = 4 for the VALU kernel, 8 for the MFMA kernel).  All waves of a work-group walk the same blocks in the same
// order, and a token row of a block stores every KV head contiguously, so
// together they read each block as one contiguous sweep (DRAM pages stay
// open) rather than D-element slices scattered over many rows.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Running-max start value: finite, so that exp2(m_old - m_new) is 0 or 1
// (never NaN) while a wave has seen no valid token; real scores are far above.
constexpr float kMaxInit = -1.0e30f;

// Waves per work-group for Hkv KV heads: the smallest power of two covering
// them, at most max_nw.
inline int heads_per_group(int hkv, int max_nw) {
  int nw = 1;
  while (nw < hkv && nw < max_nw) nw <<= 1;
  return nw;
}

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

// Grid: x = group of NW KV heads (fastest), y = sequence, z = partition;
// block = NW wave64s, wave w serving KV head x*NW + w.  With the partition
// slowest, every sequence's first partitions (always full) are dispatched
// before the later, shorter or empty ones, which then fill the tail.
struct WaveTask {
  int g, part, b;
  bool idle;  // KV head beyond Hkv (last group) or partition past the end
  PartitionSpan span;
};

template <int BS>
__device__ __forceinline__ WaveTask wave_task(const DecodeParams& p) {
  WaveTask t;
  const int nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  t.g = blockIdx.x * nw + wave;
  t.b = blockIdx.y;
  t.part = blockIdx.z;
  t.span = partition_span<BS>(p, t.b, t.part);
  t.idle = t.g >= p.Hkv || t.span.skip;
  return t;
}

// Walk blocks jbeg..jend-1 of a partition with ST register sets in rotation:
// the loads of the next ST-1 blocks are in flight while a block is consumed.
// Block ids come 64 at a time, one per lane, from a single vector load, and
// each iteration takes its id with v_readlane, so no scalar load sits between
// two blocks.
//
// `load(blk, buf)` issues the loads of block id blk into buf, through a
// buffer resource that is empty when blk < 0: ids outside the pool and the
// look-ahead past the partition's end load nothing but still issue the same
// instructions.  Every path through the loop therefore has the same loads in
// flight, and the compiler's wait counts stay exact (a load issued on one path
// only would force it to wait for all loads, the look-ahead included).
// `consume(j, ok, buf)` folds logical block j into the running state; ok is
// false for an id outside the pool, whose block then counts no valid token.
template <int ST, typename Buf, typename Load, typename Consume>
__device__ __forceinline__ void walk_blocks(const int32_t* table, const PartitionSpan& s,
                                            int num_blocks, int lane, Load&& load,
                                            Consume&& consume) {
  for (int base = s.jbeg; base < s.jend; base += 64) {
    const int cnt = min(64, s.jend - base);
    int ids = lane < cnt ? table[base + lane] : -1;
    if (static_cast<unsigned>(ids) >= static_cast<unsigned>(num_blocks)) ids = -1;
    Buf buf[ST];
#pragma unroll
    for (int u = 0; u < ST - 1; ++u) load(__builtin_amdgcn_readlane(ids, u), buf[u]);
    for (int i = 0; i < cnt; i += ST) {
#pragma unroll
      for (int u = 0; u < ST; ++u) {
        const int ii = i + u;
        if (ii >= cnt) break;
        const int nx = ii + ST - 1;
        load(nx < 64 ? __builtin_amdgcn_readlane(ids, nx) : -1, buf[(u + ST - 1) % ST]);
        consume(base + ii, __builtin_amdgcn_readlane(ids, ii) >= 0, buf[u]);
      }
    }
  }
}

// Store N consecutive output elements (out_dtype F32, F16 or BF16) starting at
// element i; i is a multiple of N, N*elem a multiple of 4 bytes.
template <int N>
__device__ __forceinline__ void store_out_n(void* base, size_t i, const float* v, int out_dtype) {
  if (out_dtype == PA_F32) {
    float* o = static_cast<float*>(base) + i;
#pragma unroll
    for (int k = 0; k < N; ++k) o[k] = v[k];
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
      uint32_t lo, hi;
      if (out_dtype == PA_F16) {
        lo = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * k]));
        hi = __builtin_bit_cast(uint16_t, static_cast<_Float16>(v[2 * k + 1]));
      } else {
        lo = f32_to_bf16_rne(v[2 * k]);
        hi = f32_to_bf16_rne(v[2 * k + 1]);
      }
      w[k] = lo | (hi << 16);
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(base) + i);
#pragma unroll
    for (int k = 0; k < N / 2; ++k) o[k] = w[k];
  }
}

// Finish N elements [d0, d0+N) of query head h (of the group of KV head g)
// for one partition: out (single partition) or the workspace partials.
// m, l: the head's final running max and sum; acc: its unnormalised sums.
template <int N>
__device__ __forceinline__ void store_partition(const DecodeParams& p, int b, int g, int G, int h,
                                                int part, bool single, int d0, float m, float l,
                                                const float* acc) {
  const size_t hq = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G + h;
  float v[N];
  if (single) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = l > 0.f ? (acc[k] / l) * p.v_scale : 0.f;
    store_out_n<N>(p.out, hq * p.D + d0, v, p.out_dtype);
  } else {
    const size_t pi = hq * p.num_partitions + part;
    float* o = p.ws_acc + pi * p.D + d0;
#pragma unroll
    for (int k = 0; k < N; ++k) o[k] = acc[k] * p.v_scale;
    if (d0 == 0) {
      p.ws_m[pi] = m;
      p.ws_l[pi] = l;
    }
  }
}

}  // namespace pa
