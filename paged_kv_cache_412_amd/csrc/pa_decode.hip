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

// One work-group per (query head, sequence).
__global__ __launch_bounds__(128) void decode_reduce_kernel(const DecodeParams p) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int max_tokens = p.max_blocks_per_seq * p.block_size;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
  if (L <= p.partition_size) return;  // finished by the partition kernel
  const int n = (L + p.partition_size - 1) / p.partition_size;
  const size_t base = (static_cast<size_t>(b) * p.Hq + hq) * p.num_partitions;
  float M = kMaxInit;
  for (int i = 0; i < n; ++i) M = fmaxf(M, p.ws_m[base + i]);
  float Ls = 0.f;
  for (int i = 0; i < n; ++i)
    Ls = __builtin_fmaf(p.ws_l[base + i], fast_exp2(p.ws_m[base + i] - M), Ls);
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  for (int d = threadIdx.x; d < p.D; d += blockDim.x) {
    float A = 0.f;
    for (int i = 0; i < n; ++i)
      A = __builtin_fmaf(p.ws_acc[(base + i) * p.D + d], fast_exp2(p.ws_m[base + i] - M), A);
    store_out(p.out, (static_cast<size_t>(b) * p.Hq + hq) * p.D + d, Ls > 0.f ? A * inv : 0.f,
              p.out_dtype);
  }
}

hipError_t launch_decode_partition(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                                   hipStream_t stream, bool* supported) {
  if (decode_mfma_serves(q_dtype, kv_dtype, p.Hq / p.Hkv))
    return launch_decode_mfma(p, q_dtype, kv_dtype, stream, supported);
  return launch_decode_valu(p, q_dtype, kv_dtype, stream, supported);
}

hipError_t launch_decode_reduce(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.Hq, p.B);
  hipLaunchKernelGGL(decode_reduce_kernel, grid, dim3(128), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
