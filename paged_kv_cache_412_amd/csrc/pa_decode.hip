// pa_decode.hip -- the plan and reduce kernels of paged decode attention,
// and the choice between the two partition kernels.
//
// A sequence longer than one partition leaves, per query head and partition
// p, the partition's running max m_p (log2 units), running sum l_p and
// unnormalised V-weighted sum acc_p in the workspace.  Softmax over the whole
// sequence follows from rescaling every partition to the common maximum:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,
// the same identity the FlashAttention-style tiling uses inside a partition
// (P1 = Ultralytics glossary page "PagedAttention", section "İlgili
// Teknikler").  Either the partition kernels combine the partials themselves
// (the last piece of a sequence to finish does it, pa_decode_common.h) or
// the reduce kernel below does, in a launch of its own; the host picks per
// call (DecodeParams::fused).

#include <hip/hip_runtime.h>

#include "pa_decode_common.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// ------------------------------------------------------------------ plan

// Balanced schedule, step 0: prefix[b] = sum over b' < b of the number of
// blocks of sequence b' (ceil(L / block_size), L clamped to the table), and
// prefix[B] = F, the blocks of all sequences.  One work-group of 1024
// threads; thread t handles a contiguous run of sequences.
constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(const DecodeParams p) {
  __shared__ int32_t sums[kPlanThreads];
  const int t = threadIdx.x;
  const int run = (p.B + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(p.B, t * run);
  const int b1 = min(p.B, b0 + run);
  auto nblk = [&](int b) { return (clamped_len(p, b) + p.block_size - 1) / p.block_size; };
  int32_t local = 0;
  for (int b = b0; b < b1; ++b) local += nblk(b);
  sums[t] = local;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {  // inclusive scan
    const int32_t v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int32_t acc = sums[t] - local;
  for (int b = b0; b < b1; ++b) {
    p.prefix[b] = acc;
    acc += nblk(b);
  }
  if (t == kPlanThreads - 1) p.prefix[p.B] = sums[t];
}

// ------------------------------------------------------------------ reduce

// Waves of the reduce kernel per work-group (one head each, or all four on
// one head's rows; see below).
constexpr int kReduceWaves = 4;

// Value of v in lane i (i wave-uniform).
__device__ __forceinline__ float lane_value(float v, int i) {
  return u2f(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(f2u(v)), i)));
}

// Combines the partials of one (query head, sequence): output elements
// l + 64e (e < E = D / 64) belong to lane l.  The partials are rows
// row(0..n-1): for the fixed schedule the sequence's partitions, for the
// balanced schedule the work-groups whose ranges overlap it.
//
// WPH waves serve one head.  WPH = 1: wave k of work-group x serves query
// head 4x + k and all its rows.  WPH = 4 (sequences split into many rows):
// the work-group serves head x, and wave k takes rows [k n/4, (k+1) n/4).
// Every wave holds the running max and sum of row i in lane i (for each
// chunk of 64 rows), so the common maximum and the rescaled sum are wave
// reductions; the weights 2^(m_i - M) stay in the lane of their row and
// reach the others with v_readlane.  Each wave's weighted sum is one in-order
// chain of fused multiply-adds over its rows, whose loads go out 16 rows at a
// time (a short batch repeats its last row's loads and skips their FMAs, so
// any batch is one round trip); with WPH = 4 the four sums are added in wave
// order through LDS.
template <bool BALANCED, int E, int WPH>
__global__ __launch_bounds__(64 * kReduceWaves) void decode_reduce_kernel(const DecodeParams p) {
  static_assert(WPH == 1 || WPH == kReduceWaves, "one wave or the whole work-group per head");
  __shared__ float part[WPH == 1 ? 1 : kReduceWaves - 1][E * 64];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int hq = WPH == 1 ? blockIdx.x * kReduceWaves + wid : blockIdx.x;
  const int b = blockIdx.y;
  if (hq >= p.Hq) return;  // wave-uniform; only with WPH = 1 (grid x = Hq otherwise)
  const size_t orow = static_cast<size_t>(b) * p.Hq + hq;
  const bool writer = WPH == 1 || wid == 0;

  int n;                  // partial rows of this (sequence, head)
  size_t row0 = 0;        // fixed: row of partition 0; rows step by B*Hq
  int w0 = 0, hg = 0, wave = 0, q = 0;
  bool first_is_second_slot = false;
  if constexpr (BALANCED) {
    const int64_t pb = p.prefix[b], pn = p.prefix[b + 1];
    if (pn == pb) {  // no tokens: zeros (no work-group touched this sequence)
      if (writer) {
#pragma unroll
        for (int e = 0; e < E; ++e) store_out(p.out, orow * p.D + lane + 64 * e, 0.f, p.out_dtype);
      }
      return;
    }
    const int64_t F = p.prefix[p.B];
    const int ng = balanced_groups(p, F);  // F >= 1 here
    w0 = balanced_owner(F, pb, ng);
    const int w1 = balanced_owner(F, pn - 1, ng);
    if (w0 == w1) return;  // one work-group covered the sequence and wrote out
    n = w1 - w0 + 1;
    const int G = p.Hq / p.Hkv;
    const int g = hq / G;
    q = hq % G;
    hg = g / p.heads_per_wg;
    wave = g % p.heads_per_wg;
    // the first work-group used slot 1 if its range began in an earlier sequence
    first_is_second_slot = balanced_start(F, w0, ng) != pb;
  } else {
    const int L = clamped_len(p, b);
    if (L <= p.partition_size) return;  // finished by the partition kernel
    n = (L + p.partition_size - 1) / p.partition_size;
    row0 = ws_row(p, orow, 0);
  }
  // every early return above is uniform over the work-group when WPH > 1
  auto row = [&](int i) -> size_t {
    if constexpr (BALANCED)
      return balanced_row(p, hg, w0 + i, (i == 0 && first_is_second_slot) ? 1 : 0, wave, q);
    else
      return row0 + static_cast<size_t>(i) * (static_cast<size_t>(p.B) * p.Hq);
  };
  const int r0 = WPH == 1 ? 0 : wid * n / WPH;        // this wave's rows
  const int r1 = WPH == 1 ? n : (wid + 1) * n / WPH;

  // rows 0..63 stay in their lanes; later chunks are read again below
  float m0 = kMaxInit, l0 = 0.f;
  if (lane < n) {
    const size_t r = row(lane);
    m0 = p.ws_m[r];
    l0 = p.ws_l[r];
  }
  float M = m0;
  for (int i = lane + 64; i < n; i += 64) M = fmaxf(M, p.ws_m[row(i)]);
  M = wave_max(M);

  float A[E];
#pragma unroll
  for (int e = 0; e < E; ++e) A[e] = 0.f;
  float Ls = 0.f;  // this lane's rows' share of sum_i l_i 2^(m_i - M)
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int cn = min(64, n - c0);
    float wl = 0.f;  // weight of row c0 + lane
    if (c0 == 0) {
      if (lane < cn) wl = fast_exp2(m0 - M);
      Ls += l0 * wl;
    } else if (lane < cn) {
      const size_t r = row(c0 + lane);
      wl = fast_exp2(p.ws_m[r] - M);
      Ls += p.ws_l[r] * wl;
    }
    const int i_end = min(r1, c0 + cn) - c0;  // this wave's rows within the chunk
    constexpr int U = 16;
    for (int i = max(r0, c0) - c0; i < i_end; i += U) {
      const int cnt = min(U, i_end - i);
      float a[U][E];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const float* src = p.ws_acc + row(c0 + i + min(k, cnt - 1)) * p.D + lane;
#pragma unroll
        for (int e = 0; e < E; ++e) a[k][e] = src[64 * e];
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        if (k < cnt) {
          const float w = lane_value(wl, i + k);
#pragma unroll
          for (int e = 0; e < E; ++e) A[e] = __builtin_fmaf(a[k][e], w, A[e]);
        }
      }
    }
  }
  Ls = group_sum<64>(Ls);
  if constexpr (WPH > 1) {
    if (wid > 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) part[wid - 1][lane + 64 * e] = A[e];
    }
    __syncthreads();
    if (wid > 0) return;
#pragma unroll
    for (int w = 0; w < WPH - 1; ++w) {
#pragma unroll
      for (int e = 0; e < E; ++e) A[e] += part[w][lane + 64 * e];
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    store_out(p.out, orow * p.D + lane + 64 * e, Ls > 0.f ? A[e] / Ls : 0.f, p.out_dtype);
}

// ------------------------------------------------------------------ host side

int32_t decode_heads_per_wg(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t Hq, int32_t Hkv) {
  const int32_t max_nw =
      decode_mfma_serves(q_dtype, kv_dtype, Hq / Hkv) ? decode_mfma_heads() : decode_valu_heads();
  int32_t nw = 1;
  while (nw < Hkv && nw < max_nw) nw <<= 1;
  return nw;
}

int32_t decode_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype) {
  if (decode_mfma_serves(q_dtype, kv_dtype, p.Hq / p.Hkv))
    return decode_mfma_groups_per_cu(p, q_dtype, kv_dtype);
  return decode_valu_groups_per_cu(p, q_dtype, kv_dtype);
}

hipError_t launch_decode_plan(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_partition(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                                   hipStream_t stream, bool* supported) {
  if (decode_mfma_serves(q_dtype, kv_dtype, p.Hq / p.Hkv))
    return launch_decode_mfma(p, q_dtype, kv_dtype, stream, supported);
  return launch_decode_valu(p, q_dtype, kv_dtype, stream, supported);
}

template <bool BALANCED, int E>
static void launch_reduce_as(const DecodeParams& p, bool split, hipStream_t stream) {
  const dim3 block(64 * kReduceWaves);
  if (split)
    hipLaunchKernelGGL((decode_reduce_kernel<BALANCED, E, kReduceWaves>), dim3(p.Hq, p.B), block,
                       0, stream, p);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<BALANCED, E, 1>),
                       dim3((p.Hq + kReduceWaves - 1) / kReduceWaves, p.B), block, 0, stream, p);
}

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
  if (p.D != 64 && p.D != 128) return hipErrorInvalidValue;
  // Expected partial rows per sequence: balanced, about groups / B + 1 (a
  // sequence's share of the work-groups plus the one it starts in); fixed,
  // the partitions of the longest possible sequence.  Past 16 rows the
  // work-group's four waves split one head's rows.
  const int64_t rows = p.balanced ? static_cast<int64_t>(p.groups) / (p.B > 0 ? p.B : 1) + 1
                                  : p.num_partitions;
  const bool split = rows > 16;
  if (p.balanced) {
    if (p.D == 64) launch_reduce_as<true, 1>(p, split, stream);
    else launch_reduce_as<true, 2>(p, split, stream);
  } else {
    if (p.D == 64) launch_reduce_as<false, 1>(p, split, stream);
    else launch_reduce_as<false, 2>(p, split, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
