// pa_decode.hip -- split-K reduce kernel for paged decode attention, and the
// choice between the two partition kernels.
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

// One work-group of D threads per (query head, sequence); thread d owns
// output element d.  The partition weights 2^(m_p - M) are computed once per
// partition and shared through LDS, so the per-element loop is one fused
// multiply-add and one coalesced load per partition.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const DecodeParams p) {
  __shared__ float w_lds[kReduceChunk];
  __shared__ float red[4];
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int max_tokens = p.max_blocks_per_seq * p.block_size;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
  if (L <= p.partition_size) return;  // finished by the partition kernel
  const int n = (L + p.partition_size - 1) / p.partition_size;
  const size_t base = (static_cast<size_t>(b) * p.Hq + hq) * p.num_partitions;
  const int tid = threadIdx.x;
  const int nt = blockDim.x;

  float M = kMaxInit;
  for (int i = tid; i < n; i += nt) M = fmaxf(M, p.ws_m[base + i]);
  M = block_reduce<true>(M, red);
  float Ls = 0.f;
  for (int i = tid; i < n; i += nt) Ls += p.ws_l[base + i] * fast_exp2(p.ws_m[base + i] - M);
  Ls = block_reduce<false>(Ls, red);

  float A = 0.f;
  const float* acc = p.ws_acc + base * p.D + tid;
  for (int c0 = 0; c0 < n; c0 += kReduceChunk) {
    const int cn = min(kReduceChunk, n - c0);
    __syncthreads();
    for (int i = tid; i < cn; i += nt) w_lds[i] = fast_exp2(p.ws_m[base + c0 + i] - M);
    __syncthreads();
    if (tid < p.D) {
      int i = 0;
      for (; i + 4 <= cn; i += 4) {
        const float a0 = acc[static_cast<size_t>(c0 + i) * p.D];
        const float a1 = acc[static_cast<size_t>(c0 + i + 1) * p.D];
        const float a2 = acc[static_cast<size_t>(c0 + i + 2) * p.D];
        const float a3 = acc[static_cast<size_t>(c0 + i + 3) * p.D];
        A = __builtin_fmaf(a0, w_lds[i], A);
        A = __builtin_fmaf(a1, w_lds[i + 1], A);
        A = __builtin_fmaf(a2, w_lds[i + 2], A);
        A = __builtin_fmaf(a3, w_lds[i + 3], A);
      }
      for (; i < cn; ++i) A = __builtin_fmaf(acc[static_cast<size_t>(c0 + i) * p.D], w_lds[i], A);
    }
  }
  if (tid < p.D)
    store_out(p.out, (static_cast<size_t>(b) * p.Hq + hq) * p.D + tid, Ls > 0.f ? A / Ls : 0.f,
              p.out_dtype);
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
  hipLaunchKernelGGL(decode_reduce_kernel, grid, dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
