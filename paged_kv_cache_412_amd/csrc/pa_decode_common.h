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
// partials row, and the last segment of the sequence to finish combines the
// rows (finish_splits below).
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

// s_waitcnt immediate that waits for every outstanding vector memory
// access, stores included (vmcnt = 0; expcnt and lgkmcnt left at their
// maxima, so they do not wait): gfx9 encoding, vmcnt in bits 3:0 and 15:14.
constexpr unsigned kWaitVmcnt0 = 0x0F70;

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
// wave scan and one pass over the wave totals; two barriers), and when a
// reduce kernel follows, work-group (0, 0) also stores them where it reads
// them; otherwise the plan kernel has written them to p.prefix.  Every
// thread of the work-group calls this, before any of them leaves.
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
  if (!p.fused && blockIdx.x == 0 && blockIdx.y == 0)
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

// The block-table side of a walk over blocks jbeg..jend-1 of a segment, in
// units of UB consecutive blocks.  Logical block j is sub-block j % 2^sub of
// table entry j / 2^sub; its id is entry * 2^sub + j % 2^sub (blocks of the
// pool seen as 2^sub smaller ones).  Entries are fetched by small vector
// loads through the same in-order memory queue as the K/V loads and reach
// the scalar unit by v_readlane, so no scalar load sits between two units.
template <int UB>
struct TableCursor {
  int jbeg, jend, sub, lane, submask;
  unsigned pool_entries;
  uint32_t tbytes;
  __amdgpu_buffer_rsrc_t trs;

  // The span and the table row are the same in every lane, but they come
  // from loads through a generic pointer (the schedule's prefix sums), which
  // the compiler cannot prove uniform: without the v_readfirstlane the block
  // ids would be per-lane values and every buffer load a loop over distinct
  // resources.
  __device__ __forceinline__ TableCursor(const int32_t* table, const PartitionSpan& s,
                                         int num_blocks, int sub_, int lane_)
      : jbeg(__builtin_amdgcn_readfirstlane(s.jbeg)),
        jend(__builtin_amdgcn_readfirstlane(s.jend)),
        sub(sub_),
        lane(lane_),
        submask((1 << sub_) - 1),
        pool_entries(static_cast<unsigned>(num_blocks >> sub_)) {
    // the table entries the segment names; a fetch at or past them reads nothing
    tbytes = jend > jbeg ? static_cast<uint32_t>(((jend - 1) >> sub) + 1) * 4u : 0u;
    trs = block_rsrc(uniform_ptr(table), tbytes);
  }
  __device__ __forceinline__ int units() const { return jend > jbeg ? (jend - jbeg + UB - 1) / UB : 0; }
  // the table entries of logical blocks jbeg + first + l in lanes l < n
  // (entry (jbeg + first) / 2^sub + l: consecutive entries, as many as the
  // blocks span); the other lanes point past the resource
  __device__ __forceinline__ int fetch(int first, int n) const {
    const int e0 = (jbeg + first) >> sub;
    const int off = lane < n ? (e0 + lane) * 4 : static_cast<int>(tbytes);
    return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(trs, off, 0, 0));
  }
  // ids of unit k from entries e fetched from logical block jbeg + first (k,
  // first uniform); returns the unit's ok bits: bit u is clear for a block
  // that counts no valid token (an id outside the pool, or past the end)
  __device__ __forceinline__ unsigned ids_of(int k, int e, int first, int (&id)[UB]) const {
    const int e0 = (jbeg + first) >> sub;
    unsigned ok = 0;
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int j = jbeg + k * UB + u;
      const int x = __builtin_amdgcn_readlane(e, (j >> sub) - e0);
      const bool valid = j < jend && static_cast<unsigned>(x) < pool_entries;
      id[u] = valid ? (x << sub) | (j & submask) : -1;
      ok |= (valid ? 1u : 0u) << u;
    }
    return ok;
  }
};

// Walk a segment with ST register sets in rotation: the loads of the next
// ST-1 units are in flight while a unit is consumed.  A unit's table entries
// are fetched ST units before its loads are issued (one small load per unit,
// lanes 0..UB-1), so the stream never stops to read the table; only the
// entries of the segment's first ST-1 units are waited for at once.
//
// `load(ids, buf)` issues the loads of the unit's UB block ids into buf,
// through buffer resources that are empty for ids < 0: ids outside the pool
// and the look-ahead past the segment's end load nothing but still issue
// the same instructions, as does the table fetch past the segment's end.
// Every path through the loop therefore has the same loads in flight, and the
// compiler's wait counts stay exact (a load issued on one path only would
// force it to wait for all loads, the look-ahead included).
// `consume(j0, ok, buf)` folds logical blocks j0..j0+UB-1 into the running
// state, with the unit's ok bits.
//
// SYNC > 0 (a power of two): every SYNC units the waves of the work-group meet
// at a barrier.  The waves walk the same blocks (one KV head each), and
// without it the oldest waves win the memory-issue arbitration and run ahead:
// the blocks in flight then spread over more of the pool, and the last waves
// finish alone.  Every wave of the work-group must walk the same segments
// (waves that have exited are not waited for).
template <int ST, int UB, int SYNC, typename Buf, typename Load, typename Consume>
__device__ __forceinline__ void walk_blocks(const int32_t* table, const PartitionSpan& s,
                                            int num_blocks, int sub, int lane, Load&& load,
                                            Consume&& consume) {
  const TableCursor<UB> tc(table, s, num_blocks, sub, lane);
  const int units = tc.units();
  if (units == 0) return;
  Buf buf[ST];
  unsigned ok[ST];
  int tv[ST];  // at unit ii, slot ii % ST: the entries of unit ii + ST - 1
  {
    const int e = tc.fetch(0, (ST - 1) * UB);
#pragma unroll
    for (int u = 0; u < ST - 1; ++u) {
      int id[UB];
      ok[u] = tc.ids_of(u, e, 0, id);
      load(id, buf[u]);
    }
#pragma unroll
    for (int u = 0; u < ST; ++u) tv[u] = tc.fetch((u + ST - 1) * UB, UB);
  }
  static_assert(SYNC == 0 || ((SYNC & (SYNC - 1)) == 0 && SYNC % ST == 0), "barrier interval");
  for (int i = 0; i < units; i += ST) {
    if constexpr (SYNC > 0) {
      if ((i & (SYNC - 1)) == 0) __builtin_amdgcn_s_barrier();
    }
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      const int ii = i + u;
      if (ii >= units) break;
      const int nu = (u + ST - 1) % ST;
      int id[UB];
      ok[nu] = tc.ids_of(ii + ST - 1, tv[u], (ii + ST - 1) * UB, id);
      tv[u] = tc.fetch((ii + 2 * ST - 1) * UB, UB);
      load(id, buf[nu]);
      consume(tc.jbeg + ii * UB, ok[u], buf[u]);
    }
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of the wave are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14;
// the other counters at their no-wait values).
constexpr unsigned wait_vmcnt(int n) {
  return 0x0F70u | static_cast<unsigned>(n & 15) | (static_cast<unsigned>((n >> 4) & 3) << 14);
}

// Walk a segment with the work-group's waves loading each unit together into
// NS LDS stages: NS-1 units are in flight while one is consumed.
// `issue(ids, stage)` starts this wave's DW loads of the unit into stage
// `stage`; `read(stage, buf)` copies this wave's operands of the unit into
// registers; `consume(j0, ok, buf)` folds them in.
//
// Per unit, each wave waits for its own loads of it and then meets the others
// at a barrier: after it the unit is whole in LDS, and every wave is done
// with the unit before, whose stage the next loads then overwrite.  The unit
// is read out before those loads are issued: the compiler cannot tell the
// stages apart and would otherwise wait for the new loads before the reads.
// The wait is explicit, so the vector-memory operations of every unit must
// be the same: each unit (the first NS-1 in the prologue included) issues one
// table fetch and then its DW loads, also past the segment's end (empty
// loads), so that the unit's loads are followed by exactly (NS-2)(DW+1)
// operations when they are waited for.  The table entries a unit's loads use
// are fetched two units earlier (a fetch is then followed by 2DW+1
// operations when it is read, and the compiler's own wait for it leaves the
// stage loads in flight).  The walk ends with all its loads complete.  Every
// wave of the work-group must walk the same segments and issue its share.
template <int UB, int NS, int DW, typename Buf, typename Issue, typename Read, typename Consume>
__device__ __forceinline__ void walk_blocks_coop(const int32_t* table, const PartitionSpan& s,
                                                 int num_blocks, int sub, int lane, Issue&& issue,
                                                 Read&& read, Consume&& consume) {
  static_assert(NS >= 2 && NS * UB <= 32 && NS * UB <= 64, "stages");
  const TableCursor<UB> tc(table, s, num_blocks, sub, lane);
  const int units = tc.units();
  if (units == 0) return;
  __syncthreads();  // every wave is past its reads of the stages (a previous segment)
  const int e = tc.fetch(0, NS * UB);  // units 0 .. NS-1, waited for at once
  int tv[2];                           // entries for the unit issued at iteration ii, slot ii % 2 ...
  int tfirst[2];                       // ... fetched from logical block jbeg + tfirst
  unsigned okq = 0;                    // ok bits of the NS-1 units in flight, oldest lowest
  if constexpr (NS == 2) {
    tv[0] = e;
    tfirst[0] = 0;
  }
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) {  // the issues of iterations u - NS + 1
    const int f = tc.fetch((u + 2) * UB, UB);
    if (u == NS - 3) {
      tv[0] = f;
      tfirst[0] = (u + 2) * UB;
    }
    if (u == NS - 2) {
      tv[1] = f;
      tfirst[1] = (u + 2) * UB;
    }
    int id[UB];
    okq |= tc.ids_of(u, e, 0, id) << (u * UB);
    asm volatile("" ::: "memory");  // the fetch goes out before the unit's loads
    issue(id, u);
  }
  for (int i = 0; i < units; i += 2) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int ii = i + s2;
      if (ii >= units) break;
      __builtin_amdgcn_s_waitcnt(wait_vmcnt((NS - 2) * (DW + 1)));  // this wave's loads of unit ii
      // A bare barrier: __syncthreads() would add a release fence, which
      // waits for every load into LDS this wave has in flight, the later
      // stages' included.  The empty asm keeps the compiler from moving the
      // reads of the stage above it.
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      Buf buf;
      read(ii % NS, buf);
      int id[UB];
      const unsigned okn = tc.ids_of(ii + NS - 1, tv[s2], tfirst[s2], id);
      tv[s2] = tc.fetch((ii + NS + 1) * UB, UB);
      tfirst[s2] = (ii + NS + 1) * UB;
      asm volatile("" ::: "memory");  // the fetch goes out before the unit's loads
      issue(id, (ii + NS - 1) % NS);
      const unsigned ok = okq & ((1u << UB) - 1u);
      okq = (okq >> UB) | (okn << (UB * (NS - 2)));  // units ii+1 .. ii+NS-1 remain
      consume(tc.jbeg + ii * UB, ok, buf);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // no load into a stage outlives the walk
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

// Partial rows of split sequences cross work-groups, which may run on
// different XCDs, each with its own L2.  They are written and read with
// device-scope 16-byte buffer accesses (cache policy sc1), which go to the
// device-coherent level instead of a non-coherent L2 copy, so no cache-wide
// write-back or invalidate is needed to pass them between XCDs.  The host
// keeps each partial region under 2 GiB, so 32-bit byte offsets reach it.
constexpr int kCoherent = 16;  // sc1: device scope

// (The workspace pointers are kernel arguments, but the combine after the
// walk reads them back from the kernel-argument segment through a copy that
// the compiler cannot prove uniform.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(uniform_ptr(base)), 0, 0x7fffffff,
                                           0x00020000);
}
// N partial sums of row r from element d0 (16-byte stores), and the row's m
// and l from the lane that holds element 0; cache policy CP.
template <int CP, int N>
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rm,
                                              __amdgpu_buffer_rsrc_t rl, uint32_t r, int D, int d0,
                                              const float* v, float m, float l) {
#pragma unroll
  for (int k = 0; k < N; k += 4) {
    const f32x4_t x = {v[k], v[k + 1], v[k + 2], v[k + 3]};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), ra, (r * D + d0 + k) * 4u, 0, CP);
  }
  if (d0 == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m), rm, r * 4u, 0, CP);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), rl, r * 4u, 0, CP);
  }
}
__device__ __forceinline__ f32x4_t load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4u, 0, kCoherent));
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t elem) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, kCoherent));
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
    const uint32_t r = static_cast<uint32_t>(dst.part_row + h);
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = acc[k] * vs;
    const __amdgpu_buffer_rsrc_t ra = partial_rsrc(p.ws_acc);
    const __amdgpu_buffer_rsrc_t rm = partial_rsrc(p.ws_m);
    const __amdgpu_buffer_rsrc_t rl = partial_rsrc(p.ws_l);
    if (p.fused) {
      // straight to the device-coherent level, where the wave that combines
      // the sequence in this launch reads them
      store_partial<kCoherent, N>(ra, rm, rl, r, p.D, d0, v, m, l);
    } else {
      // through the L2 as usual: the reduce kernel reads them after this launch
      store_partial<0, N>(ra, rm, rl, r, p.D, d0, v, m, l);
    }
  }
}

// ------------------------------------------------------------------ split sequences
//
// A sequence that several segments cover (partitions of it under the fixed
// schedule; the work-groups whose block ranges overlap it under the balanced
// one) leaves one partial row group per segment: for each of the G query
// heads of a KV head, the segment's running max m_i (log2 units), running sum
// l_i and unnormalised weighted sum acc_i (v_scale applied).  Softmax over
// the whole sequence follows from rescaling every segment to the common
// maximum, the identity the FlashAttention-style tiling uses inside a segment
// (P1 = Ultralytics glossary page "PagedAttention", section "İlgili
// Teknikler"):
//   M = max_i m_i,  out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
//
// No separate launch combines them.  Each wave that wrote a partial row
// group waits until its stores are complete and then counts its arrival on
// the (KV head, sequence) counter in the workspace; the wave whose arrival
// completes the count reads the others' rows, combines them and resets the
// counter to zero.  The rows are written and read with device-scope accesses
// (store_partial with sc1, load_coherent*), so what one XCD wrote is what another
// reads without any cache-wide write-back or invalidate; the reads are
// issued only after the arrival that completed the count has returned.  No
// wave ever waits for another, and every call leaves every counter zero for
// the next.

// Maximum over the 64 lanes of a wave; every lane receives it.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}

// Where the n partial row groups of one (sequence, KV head) are: row group i
// starts at row split_row(i) (query 0; query q is the row after it by q).
struct SplitRows {
  int n;              // row groups (segments that cover the sequence)
  int hg, w0, wave;   // balanced: head group, first work-group, wave
  int first_second;   // balanced: the first work-group used its second slot
  size_t row0, step;  // fixed: row of partition 0, rows between partitions
};

__device__ __forceinline__ size_t split_row(const DecodeParams& p, const SplitRows& s, int i) {
  if (p.balanced) return balanced_row(p, s.hg, s.w0 + i, (i == 0 && s.first_second) ? 1 : 0, s.wave, 0);
  return s.row0 + static_cast<size_t>(i) * s.step;
}

// Combine the partial row groups of one (sequence, KV head) for queries
// q0 .. q0 + QB - 1 (those below G) into their output rows.  Pass 1: lane i
// holds the (m, l) of row group i, so the common maximum and the rescaled
// sum are wave reductions.  Pass 2: a query's D partial sums are D/4 lanes
// of 16-byte loads, so one load instruction covers 64 / (D/4) row groups
// (the lane's `sub`); LOADS 16-byte loads per lane go out at once per batch
// of row groups (the first batch together with pass 1's loads), each lane
// takes its row group's weight from the lane that holds it, and the
// sub-groups' sums are added at the end.  The order of every sum
// is fixed by the row groups' order, not by timing.  LOADS trades the
// batches' round trips against registers: the combine runs after the block
// walk, and a kernel whose walk needs few registers keeps it small so that
// the combine does not set its register count.
template <int D, int QB, int LOADS>
__device__ __forceinline__ void combine_queries(const DecodeParams& p, const SplitRows& sr, int G,
                                                int q0, size_t out_row, int lane) {
  constexpr int QL = D / 4;                             // lanes per query row
  constexpr int RPL = 64 / QL;                          // row groups per load instruction
  constexpr int NB = LOADS / QB > 0 ? LOADS / QB : 1;   // load instructions per query and batch
  constexpr int RB = RPL * NB;                          // row groups per batch
  const int n = sr.n;
  const int sub = lane / QL;
  const int col = 4 * (lane % QL);
  // every load is issued unconditionally, at a clamped row group and query
  // (then discarded), so that a batch's loads go out back to back
  int qc[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) qc[q] = min(q0 + q, G - 1);
  auto valid = [&](int q) { return q0 + q < G; };

  const __amdgpu_buffer_rsrc_t racc = partial_rsrc(p.ws_acc);
  const __amdgpu_buffer_rsrc_t rm = partial_rsrc(p.ws_m);
  const __amdgpu_buffer_rsrc_t rl = partial_rsrc(p.ws_l);
  f32x4_t buf[NB][QB];
  auto load_batch = [&](int r0, int c1) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int r = min(r0 + j * RPL + sub, c1 - 1);  // past the end: repeat the last row group
      const uint32_t row = static_cast<uint32_t>(split_row(p, sr, r));
#pragma unroll
      for (int q = 0; q < QB; ++q) buf[j][q] = load_coherent4(racc, (row + qc[q]) * D + col);
    }
  };
  // (m, l) of row group i = lane, and the first batch of partial sums
  float m0[QB], l0[QB], M[QB];
  {
    const uint32_t r = static_cast<uint32_t>(split_row(p, sr, min(lane, n - 1)));
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      m0[q] = load_coherent1(rm, r + qc[q]);
      l0[q] = load_coherent1(rl, r + qc[q]);
    }
  }
  load_batch(0, min(n, 64));
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    if (lane >= n) {
      m0[q] = kMaxInit;
      l0[q] = 0.f;
    }
    M[q] = m0[q];
  }
  for (int i0 = 64; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t r = static_cast<uint32_t>(split_row(p, sr, min(i, n - 1)));
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const float mi = load_coherent1(rm, r + qc[q]);
      if (i < n) M[q] = fmaxf(M[q], mi);
    }
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) M[q] = wave_max(M[q]);

  f32x4_t A[QB];
  float Ls[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    A[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Ls[q] = 0.f;
  }
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int c1 = min(n, c0 + 64);
    float w[QB];  // weight of row group c0 + lane
    if (c0 == 0) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        w[q] = lane < n ? fast_exp2(m0[q] - M[q]) : 0.f;
        Ls[q] += l0[q] * w[q];
      }
    } else {
      const int i = c0 + lane;
      const uint32_t r = static_cast<uint32_t>(split_row(p, sr, min(i, n - 1)));
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const float mi = load_coherent1(rm, r + qc[q]);
        const float li = load_coherent1(rl, r + qc[q]);
        w[q] = i < n ? fast_exp2(mi - M[q]) : 0.f;
        Ls[q] += i < n ? li * w[q] : 0.f;
      }
    }
    for (int r0 = c0; r0 < c1; r0 += RB) {
      if (r0 > 0) load_batch(r0, c1);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int r = r0 + j * RPL + sub;
        const int src = min(r, c1 - 1) - c0;
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const float wr = __shfl(w[q], src, 64);
          if (r < c1) A[q] += wr * buf[j][q];  // a repeated row group adds nothing, NaN included
        }
      }
    }
  }
#pragma unroll
  for (int off = QL; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
#pragma unroll
      for (int k = 0; k < 4; ++k) A[q][k] += __shfl_xor(A[q][k], off, 64);
    }
  }
#pragma unroll
  for (int q = 0; q < QB; ++q) Ls[q] = group_sum<64>(Ls[q]);
  if (sub == 0) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (valid(q)) {
        float v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = Ls[q] > 0.f ? A[q][k] / Ls[q] : 0.f;
        store_out_n<4>(p.out, (out_row + q0 + q) * D + col, v, p.out_dtype);
      }
    }
  }
}

// All G queries of one (sequence, KV head), QB at a time.
template <int D, int QB, int LOADS>
__device__ __forceinline__ void combine_split(const DecodeParams& p, const SplitRows& sr, int G,
                                              size_t out_row, int lane) {
  for (int q0 = 0; q0 < G; q0 += QB) combine_queries<D, QB, LOADS>(p, sr, G, q0, out_row, lane);
}

// Where the partial row groups of split sequence b (KV head g of head
// group hg, wave `wave`) are.
__device__ __forceinline__ SplitRows split_rows(const DecodeParams& p, const int32_t* prefix, int b,
                                                int hg, int wave, int G) {
  SplitRows sr{};
  if (p.balanced) {
    const int64_t pb = prefix[b], pn = prefix[b + 1], F = prefix[p.B];
    const int ng = balanced_groups(p, F);
    sr.w0 = balanced_owner(F, pb, ng);
    sr.n = balanced_owner(F, pn - 1, ng) - sr.w0 + 1;
    sr.first_second = balanced_start(F, sr.w0, ng) != pb ? 1 : 0;
    sr.hg = hg;
    sr.wave = wave;
  } else {
    const int L = clamped_len(p, b);
    sr.n = (L + p.partition_size - 1) / p.partition_size;
    const int g = hg * p.heads_per_wg + wave;
    sr.row0 = ws_row(p, static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G, 0);
    sr.step = static_cast<size_t>(p.B) * p.Hq;
  }
  return sr;
}

// Balanced schedule: a sequence without tokens has no blocks, so no segment
// covers it; work-group w writes the zero outputs of the empty sequences
// b = w, w + groups, ... (queries of KV head g).
template <int D>
__device__ __forceinline__ void zero_empty_sequences(const DecodeParams& p, const int32_t* prefix,
                                                     int g, int G, int lane) {
  for (int b = blockIdx.y; b < p.B; b += p.groups) {
    if (prefix[b + 1] != prefix[b]) continue;
    const size_t e0 = (static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G) * D;
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = lane; i < G * D / 4; i += 64) store_out_n<4>(p.out, e0 + 4 * static_cast<size_t>(i), z, p.out_dtype);
  }
}

// The largest b < B with prefix[b] <= x: for 0 <= x < prefix[B], the
// (non-empty) sequence that holds block x.
__device__ __forceinline__ int sequence_of_block(const int32_t* prefix, int B, int64_t x) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= x) lo = mid;
    else hi = mid;
  }
  return lo;
}

// What a wave does after its block walk: under the balanced schedule, zero
// the empty sequences it is assigned; then, once its partial rows are
// stored, count an arrival on the counter of each sequence it left partial
// rows for, and combine the sequence's row groups if its arrival completed
// the count (the counter then goes back to zero).  Those sequences follow from the schedule alone: under the balanced
// schedule the ones holding the work-group's first and last blocks, unless
// it covers them whole; under the fixed schedule its sequence, if longer
// than one partition.  Nothing about them is kept through the walk, whose
// registers are nearly all taken: the kernel's argument is read again from
// the argument segment here, and the prefix sums from where they live.
template <int D, int QB, int LOADS>
__device__ __forceinline__ void finish_splits(PlanLds& lds, int lane) {
  typedef const __attribute__((address_space(4))) DecodeParams KernArg;
  KernArg* pk = (KernArg*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pk));
  DecodeParams p;
  __builtin_memcpy(&p, (const void*)pk, sizeof(p));
  if (!p.fused) return;  // the reduce kernel combines split sequences and zeroes empty ones
  const int hg = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = hg * p.heads_per_wg + wave;
  const int G = p.Hq / p.Hkv;
  int split[2] = {-1, -1};
  const int32_t* prefix = p.inline_plan ? lds.prefix : p.prefix;
  if (p.balanced) {
    zero_empty_sequences<D>(p, prefix, g, G, lane);
    const int64_t F = prefix[p.B];
    const int n = balanced_groups(p, F);
    const int w = blockIdx.y;
    if (w >= n) return;
    const int64_t x0 = balanced_start(F, w, n), x1 = balanced_start(F, w + 1, n);
    const int ba = sequence_of_block(prefix, p.B, x0);
    const int bz = sequence_of_block(prefix, p.B, x1 - 1);
    if (!(prefix[ba] == x0 && prefix[ba + 1] <= x1)) split[0] = ba;
    if (bz != ba && prefix[bz + 1] > x1) split[1] = bz;
  } else {
    const int b = blockIdx.y;
    const int L = clamped_len(p, b);
    const int nblk = (L + p.block_size - 1) / p.block_size;
    if (L > p.partition_size && static_cast<int64_t>(blockIdx.z) * (p.partition_size / p.block_size) < nblk)
      split[0] = b;
  }
  if (split[0] < 0 && split[1] < 0) return;
  // this wave's partial rows (device-scope stores) complete before its arrival counts
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int b = __builtin_amdgcn_readfirstlane(split[k]);
    if (b < 0) continue;
    const SplitRows sr = split_rows(p, prefix, b, hg, wave, G);
    int32_t* cnt = p.counters + static_cast<size_t>(g) * p.B + b;
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readlane(old, 0);
    if (old != sr.n - 1) continue;  // another segment of the sequence is still running
    // every other segment's rows were complete before its arrival counted;
    // they are read (device-scope loads) only after this arrival returned
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    combine_split<D, QB, LOADS>(p, sr, G, static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G, lane);
  }
}

}  // namespace pa
