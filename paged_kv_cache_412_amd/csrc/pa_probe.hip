// pa_probe.hip -- a measurement kernel, not a step of the path: it reads
// whole pieces of a pool in a given order, with the non-temporal 16-byte
// buffer loads the attention kernels use, and folds every loaded word into
// one word per work-group so that no load is dead.  Timed over pieces of a
// block's size in random order, it gives the practical HBM read rate of a
// block gather on this part: the ceiling the attention kernels are measured
// against, beside the vendor peak.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadChunks = 8;  // 16-byte loads per thread and iteration, all issued before folding
constexpr int kReadSpan = kReadThreads * kReadChunks;  // 16-byte chunks per work-group iteration (32 KiB)
constexpr uint32_t kReadMaxPiece = kReadSpan * 16;
constexpr uint32_t kReadMinPiece = 64 * 16;  // one wave load (64 lanes x 16 bytes)
constexpr int kReadGroupsPerCU = 8;

// Each iteration of a work-group reads 32 KiB: the next floor(32 KiB /
// piece) pieces of its share of ids.  Load k of wave v covers chunks
// 64v + 256k .. +63 of that span, which lie in one piece (pieces are whole
// multiples of a wave load), so its buffer resource is wave-uniform.  A
// piece id outside the pool, and the span's tail past its last whole piece,
// read nothing (zero-length buffer resources).
__global__ __launch_bounds__(kReadThreads) void read_blocks_kernel(const char* pool, int32_t num_pieces,
                                                                   uint32_t piece_bytes, const int32_t* ids,
                                                                   int32_t n, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar ids, one resource per wave load
  const int cpp = static_cast<int>(piece_bytes / 16);  // chunks per piece
  const int ppi = kReadSpan / cpp;                     // pieces per iteration
  uint32_t acc = 0;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * ppi; base < n;
       base += static_cast<int64_t>(gridDim.x) * ppi) {
    uint32_t w[kReadChunks][4];
#pragma unroll
    for (int k = 0; k < kReadChunks; ++k) {
      const int c0 = 64 * wave + kReadThreads * k;  // first chunk of this wave load
      const int ps = c0 / cpp;                       // piece within the iteration
      const int64_t idx = base + ps;
      const int id = ps < ppi && idx < n ? ids[idx] : -1;
      const bool ok = id >= 0 && id < num_pieces;
      const __amdgpu_buffer_rsrc_t r =
          block_rsrc(pool + static_cast<int64_t>(ok ? id : 0) * piece_bytes, ok ? piece_bytes : 0u);
      buffer_load<4>(r, (c0 % cpp + lane) * 16, 0, w[k]);
    }
#pragma unroll
    for (int k = 0; k < kReadChunks; ++k) acc ^= w[k][0] ^ w[k][1] ^ w[k][2] ^ w[k][3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t wave_acc[kReadThreads / 64];
  if (lane == 0) wave_acc[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int k = 0; k < kReadThreads / 64; ++k) s ^= wave_acc[k];
    sink[blockIdx.x] = s;
  }
}

}  // namespace
}  // namespace pa

extern "C" {

pa_status pa_read_blocks(const void* pool, int32_t num_pieces, size_t piece_bytes, const int32_t* ids,
                         int32_t n, uint32_t* sink, int32_t sink_len, void* stream) {
  if (n < 0 || num_pieces < 1 || sink_len < 1 || piece_bytes < pa::kReadMinPiece ||
      piece_bytes % pa::kReadMinPiece != 0 || piece_bytes > pa::kReadMaxPiece)
    return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!pool || !ids || !sink) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(pool) % 16 != 0) return PA_ERR_SHAPE;
  const int32_t grid = std::min(sink_len, pa::compute_units() * pa::kReadGroupsPerCU);
  hipLaunchKernelGGL(pa::read_blocks_kernel, dim3(grid), dim3(pa::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(pool), num_pieces,
                     static_cast<uint32_t>(piece_bytes), ids, n, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // extern "C"
