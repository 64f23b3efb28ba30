// pa_decode_common.h -- pieces shared by the two decode-partition kernels
// (the VALU kernel for small query groups and the MFMA kernel for grouped
// query attention): the work schedule, the per-wave block walk with its load
// pipeline, and the store of a finished segment.
//
// Both kernels compute, for one KV head g of one sequence b and one segment
// of the sequence's blocks, the online-softmax state of the G query heads
// that share g (grouped-query attention, P1 = Ultralytics glossary page
// "PagedAttention", section "İlgili Teknikler"): the running maximum m of the
// scores (log2 units), the running sum l of 2^(s - m) and the unnormalised
// V-weighted sum acc.  A segment covering the whole sequence writes
// out = v_scale * acc / l directly; otherwise (m, l, v_scale * acc) go to a
// partials row for the reduce kernel.
//
// Work decomposition.  A work-group holds one wave64 per KV head of a group
// of up to NW consecutive KV heads (NW = 4 for the VALU kernel, 8 for the
// MFMA kernel).  All waves of a work-group walk the same blocks in the same
// order, and a token row of a block stores every KV head contiguously, so
// together they read each block as one contiguous sweep (DRAM pages stay
// open) rather than D-element slices scattered over many rows.  Which blocks
// a work-group walks is the schedule's business (pa_internal.h): one
// partition of one sequence, or an equal share of all sequences' blocks.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Running-max start value: finite, so that exp2(m_old - m_new) is 0 or 1
// (never NaN) while a wave has seen no valid token; real scores are far above.
constexpr float kMaxInit = -1.0e30f;


// One segment of one sequence: blocks [jbeg, jend) of sequence b, which
// holds L tokens.
struct PartitionSpan {
  int L;        // sequence length, clamped to the table's capacity
  int jbeg;     // first logical block of the segment
  int jend;     // one past its last logical block
};

__device__ __forceinline__ int clamped_len(const DecodeParams& p, int b) {
  const int max_tokens = p.max_blocks_per_seq * p.block_size;
  const int L = p.seq_lens[b];
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

// Where a finished segment goes: complete -> out rows out_row + h (h < G);
// otherwise -> partials rows part_row + h.
struct SegmentDest {
  bool complete;
  size_t out_row;   // b*Hq + g*G
  size_t part_row;  // partials row of query 0
};

// The balanced schedule's prefix sums, prefix[b] = blocks of sequences
// before b and prefix[B] = all blocks.  With p.inline_plan every work-group
// computes them into LDS (its threads take contiguous runs of sequences, a
// wave scan and one pass over the wave totals; two barriers), and
// work-group (0, 0) also stores them where the reduce kernel reads them;
// otherwise the plan kernel has written them to p.prefix.  Every thread of
// the work-group calls this, before any of them leaves.
struct PlanLds {
  int32_t prefix[kInlinePlanMaxB + 1];
  int32_t wave_sum[16];
};

__device__ __forceinline__ const int32_t* schedule_prefix(const DecodeParams& p, PlanLds& lds) {
  if (!p.inline_plan) return p.prefix;
  const int T = blockDim.x, t = threadIdx.x, lane = t & 63;
  auto nblk = [&](int b) { return (clamped_len(p, b) + p.block_size - 1) / p.block_size; };
  const int run = (p.B + T - 1) / T;
  const int b0 = min(p.B, t * run), b1 = min(p.B, b0 + run);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += nblk(b);
  int x = local;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds.wave_sum[t >> 6] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < (t >> 6); ++w) base += lds.wave_sum[w];
  int acc = base + x - local;
  for (int b = b0; b < b1; ++b) {
    lds.prefix[b] = acc;
    acc += nblk(b);
  }
  if (t == T - 1) lds.prefix[p.B] = base + x;
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = t; i <= p.B; i += T) p.prefix[i] = lds.prefix[i];
  return lds.prefix;
}

// Calls fn(b, span, dest) for every segment this wave works on, for KV head
// g = head_group * NW + wave.  Fixed schedule: work-group (hg, b, part) has
// one segment, partition `part` of sequence b.  Balanced schedule:
// work-group (hg, w) walks the sequences that overlap blocks
// [w*F/groups, (w+1)*F/groups) of the concatenated block list.
template <typename Fn>
__device__ __forceinline__ void for_each_segment(const DecodeParams& p, const int32_t* prefix, int hg,
                                                 int wave, int G, Fn&& fn) {
  const int g = hg * p.heads_per_wg + wave;
  if (!p.balanced) {
    const int b = blockIdx.y;
    const int part = blockIdx.z;
    PartitionSpan s;
    s.L = clamped_len(p, b);
    const int PB = p.partition_size / p.block_size;
    const int nblk = (s.L + p.block_size - 1) / p.block_size;
    s.jbeg = part * PB;
    s.jend = min(s.jbeg + PB, nblk);
    if (part > 0 && s.jbeg >= nblk) return;  // partition past the end of this sequence
    SegmentDest d;
    d.complete = s.L <= p.partition_size;
    d.out_row = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G;
    d.part_row = ws_row(p, d.out_row, part);
    fn(b, s, d);
    return;
  }
  const int w = blockIdx.y;
  const int64_t F = prefix[p.B];
  const int n = balanced_groups(p, F);
  if (w >= n) return;  // fewer blocks than work-groups: the rest idle
  const int64_t x0 = balanced_start(F, w, n);
  const int64_t x1 = balanced_start(F, w + 1, n);
  // the sequence holding block x0: the largest b with prefix[b] <= x0
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= x0) lo = mid;
    else hi = mid;
  }
  int which = 0;
  for (int b = lo; b < p.B; ++b) {
    const int64_t pb = prefix[b];
    if (pb >= x1) break;
    const int64_t pn = prefix[b + 1];
    if (pn <= x0 || pn == pb) continue;  // before the range, or no blocks
    PartitionSpan s;
    s.L = clamped_len(p, b);
    s.jbeg = static_cast<int>((x0 > pb ? x0 : pb) - pb);
    s.jend = static_cast<int>((x1 < pn ? x1 : pn) - pb);
    SegmentDest d;
    d.complete = s.jbeg == 0 && pn <= x1;
    d.out_row = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G;
    d.part_row = balanced_row(p, hg, w, which, wave, 0);
    fn(b, s, d);
    which = 1;
  }
}

// Walk blocks jbeg..jend-1 of a partition in units of UB consecutive blocks,
// with ST register sets in rotation: the loads of the next ST-1 units are in
// flight while a unit is consumed.  Block ids come 64 at a time, one per lane,
// from a single vector load, and each unit takes its ids with v_readlane, so
// no scalar load sits between two units.
//
// `load(ids, buf)` issues the loads of the unit's UB block ids into buf,
// through buffer resources that are empty for ids < 0: ids outside the pool
// and the look-ahead past the partition's end load nothing but still issue
// the same instructions.  Every path through the loop therefore has the same
// loads in flight, and the compiler's wait counts stay exact (a load issued on
// one path only would force it to wait for all loads, the look-ahead
// included).  `consume(j0, ok, buf)` folds logical blocks j0..j0+UB-1 into the
// running state; bit u of ok is clear for a block that counts no valid token
// (an id outside the pool, or past the partition's end).
// Logical block j is sub-block j % 2^sub of table entry j / 2^sub; its id
// is entry * 2^sub + j % 2^sub (blocks of the pool seen as 2^sub smaller ones).
template <int ST, int UB, typename Buf, typename Load, typename Consume>
__device__ __forceinline__ void walk_blocks(const int32_t* table, const PartitionSpan& s,
                                            int num_blocks, int sub, int lane, Load&& load,
                                            Consume&& consume) {
  for (int base = s.jbeg; base < s.jend; base += 64) {
    const int cnt = min(64, s.jend - base);
    int ids = -1;
    if (lane < cnt) {
      const int j = base + lane;
      const int e = table[j >> sub];
      // entries outside the pool (num_blocks >> sub table blocks) count none
      ids = static_cast<unsigned>(e) < static_cast<unsigned>(num_blocks >> sub)
                ? (e << sub) | (j & ((1 << sub) - 1))
                : -1;
    }
    const int units = (cnt + UB - 1) / UB;
    // ids of unit k (k uniform; 64 is a multiple of UB, so a unit never
    // straddles two 64-block chunks)
    auto unit_ids = [&](int k, int (&out)[UB]) {
#pragma unroll
      for (int u = 0; u < UB; ++u) out[u] = k < 64 / UB ? __builtin_amdgcn_readlane(ids, k * UB + u) : -1;
    };
    Buf buf[ST];
#pragma unroll
    for (int u = 0; u < ST - 1; ++u) {
      int id[UB];
      unit_ids(u, id);
      load(id, buf[u]);
    }
    for (int i = 0; i < units; i += ST) {
#pragma unroll
      for (int u = 0; u < ST; ++u) {
        const int ii = i + u;
        if (ii >= units) break;
        int nid[UB], cid[UB];
        unit_ids(ii + ST - 1, nid);
        load(nid, buf[(u + ST - 1) % ST]);
        unit_ids(ii, cid);
        unsigned ok = 0;
#pragma unroll
        for (int b = 0; b < UB; ++b) ok |= (cid[b] >= 0 ? 1u : 0u) << b;
        consume(base + ii * UB, ok, buf[u]);
      }
    }
  }
}

// Vector stores.  Every lane's run of N outputs goes out in 16-byte (or, for
// 8-byte runs, 8-byte) stores: element-wise stores would cost the address unit
// one pass per lane and per element, and the address unit is the bottleneck
// of these kernels while the K/V loads stream.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// N fp32 values to a 16-byte aligned destination (N a multiple of 4).
template <int N>
__device__ __forceinline__ void store_f32_n(float* dst, const float* v) {
  static_assert(N % 4 == 0, "16-byte stores");
#pragma unroll
  for (int k = 0; k < N; k += 4)
    *reinterpret_cast<f32x4_t*>(dst + k) = f32x4_t{v[k], v[k + 1], v[k + 2], v[k + 3]};
}

// N consecutive output elements (out_dtype F32, F16 or BF16) starting at
// element i; the destination is aligned to the run's size (or 16 bytes).
template <int N>
__device__ __forceinline__ void store_out_n(void* base, size_t i, const float* v, int out_dtype) {
  if (out_dtype == PA_F32) {
    store_f32_n<N>(static_cast<float*>(base) + i, v);
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
    uint16_t* o = static_cast<uint16_t*>(base) + i;
    if constexpr (N / 2 >= 4) {
#pragma unroll
      for (int k = 0; k < N / 2; k += 4)
        *reinterpret_cast<u32x4_t*>(o + 2 * k) = u32x4_t{w[k], w[k + 1], w[k + 2], w[k + 3]};
    } else {
      static_assert(N / 2 == 2, "8-byte run");
      *reinterpret_cast<u32x2_t*>(o) = u32x2_t{w[0], w[1]};
    }
  }
}

// Finish N elements [d0, d0+N) of query h of a segment: out (the segment
// covers its sequence) or its partials row.  m, l: the query's final running
// max and sum; acc: its unnormalised sums; vs: the V scale of its KV head.
template <int N>
__device__ __forceinline__ void store_segment(const DecodeParams& p, const SegmentDest& dst, int h,
                                              int d0, float m, float l, const float* acc, float vs) {
  float v[N];
  if (dst.complete) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = l > 0.f ? (acc[k] / l) * vs : 0.f;
    store_out_n<N>(p.out, (dst.out_row + h) * p.D + d0, v, p.out_dtype);
  } else {
    const size_t r = dst.part_row + h;
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = acc[k] * vs;
    store_f32_n<N>(p.ws_acc + r * p.D + d0, v);
    if (d0 == 0) {
      p.ws_m[r] = m;
      p.ws_l[r] = l;
    }
  }
}

}  // namespace pa
