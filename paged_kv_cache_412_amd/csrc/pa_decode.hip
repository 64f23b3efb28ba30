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
// Teknikler").

#include <hip/hip_runtime.h>

#include "pa_decode_common.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Partitions whose weights one pass of the reduce stages in LDS.
constexpr int kReduceChunk = 256;

// Block-wide reduction (max or sum) of one value per thread; blockDim.x is a
// multiple of 64 and at most 256.  Every thread receives the result.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* lds4) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(v, off, 64);
    v = MAX ? fmaxf(v, o) : v + o;
  }
  const int nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = v;
  __syncthreads();
  v = lds4[0];
  for (int w = 1; w < nw; ++w) v = MAX ? fmaxf(v, lds4[w]) : v + lds4[w];
  return v;
}

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

// One work-group of D threads per (query head, sequence); thread d owns
// output element d.  The partials of the sequence are rows row(0..n-1): for
// the fixed schedule its partitions, for the balanced schedule the
// work-groups whose ranges overlap it.  The weights 2^(m_i - M) are computed
// once per row and shared through LDS, so the per-element loop is one fused
// multiply-add and one coalesced load per row.
template <bool BALANCED>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeParams p) {
  __shared__ float w_lds[kReduceChunk];
  __shared__ float red[4];
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const size_t orow = static_cast<size_t>(b) * p.Hq + hq;

  int n;                  // partial rows of this (sequence, head)
  size_t row0 = 0;        // fixed: row of partition 0; rows step by B*Hq
  int w0 = 0, hg = 0, wave = 0, q = 0;
  int64_t F = 0;
  bool first_is_second_slot = false;
  if constexpr (BALANCED) {
    const int64_t pb = p.prefix[b], pn = p.prefix[b + 1];
    if (pn == pb) {  // no tokens: zeros (no work-group touched this sequence)
      for (int d = tid; d < p.D; d += nt) store_out(p.out, orow * p.D + d, 0.f, p.out_dtype);
      return;
    }
    F = p.prefix[p.B];
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
  auto row = [&](int i) -> size_t {
    if constexpr (BALANCED)
      return balanced_row(p, hg, w0 + i, (i == 0 && first_is_second_slot) ? 1 : 0, wave, q);
    else
      return row0 + static_cast<size_t>(i) * (static_cast<size_t>(p.B) * p.Hq);
  };

  float M = kMaxInit;
  for (int i = tid; i < n; i += nt) M = fmaxf(M, p.ws_m[row(i)]);
  M = block_reduce<true>(M, red);
  float Ls = 0.f;
  for (int i = tid; i < n; i += nt) {
    const size_t r = row(i);
    Ls += p.ws_l[r] * fast_exp2(p.ws_m[r] - M);
  }
  Ls = block_reduce<false>(Ls, red);

  float A = 0.f;
  for (int c0 = 0; c0 < n; c0 += kReduceChunk) {
    const int cn = min(kReduceChunk, n - c0);
    __syncthreads();
    for (int i = tid; i < cn; i += nt) w_lds[i] = fast_exp2(p.ws_m[row(c0 + i)] - M);
    __syncthreads();
    if (tid < p.D) {
      // the loads of 16 rows go out together, then the same in-order chain
      // of fused multiply-adds
      constexpr int U = 16;
      int i = 0;
      for (; i + U <= cn; i += U) {
        float a[U];
#pragma unroll
        for (int k = 0; k < U; ++k) a[k] = p.ws_acc[row(c0 + i + k) * p.D + tid];
#pragma unroll
        for (int k = 0; k < U; ++k) A = __builtin_fmaf(a[k], w_lds[i + k], A);
      }
      for (; i + 4 <= cn; i += 4) {
        float a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = p.ws_acc[row(c0 + i + k) * p.D + tid];
#pragma unroll
        for (int k = 0; k < 4; ++k) A = __builtin_fmaf(a[k], w_lds[i + k], A);
      }
      for (; i < cn; ++i) A = __builtin_fmaf(p.ws_acc[row(c0 + i) * p.D + tid], w_lds[i], A);
    }
  }
  if (tid < p.D) store_out(p.out, orow * p.D + tid, Ls > 0.f ? A / Ls : 0.f, p.out_dtype);
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

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.Hq, p.B);
  const int threads = (p.D + 63) / 64 * 64;
  if (p.balanced)
    hipLaunchKernelGGL(decode_reduce_kernel<true>, grid, dim3(threads), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<false>, grid, dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
