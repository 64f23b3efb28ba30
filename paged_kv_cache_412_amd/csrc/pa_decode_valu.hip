// pa_decode_valu.hip -- decode-partition kernel on the vector ALUs, used when
// few query heads share a KV head (G = Hq/Hkv of 1 or 2) and for fp32 caches.
//
// What is computed (P1 = Ultralytics glossary page "PagedAttention"):
//   * the kernel follows each sequence's block table and gathers K and V
//     block by block, so the cache need not be contiguous (P1 "Sayfalama
//     Nasıl Çalışır");
//   * attention is exact softmax attention computed in tiles, FlashAttention
//     style: scores live only in registers, never in device memory (P1
//     "İlgili Teknikler");
//   * grouped-query attention: the G query heads that share a KV head are
//     served by one work-group, so each K/V block is read once for all of
//     them (P1 "İlgili Teknikler").
//
// Work decomposition.  One wave64 per (KV head g, partition, sequence),
// grouped into work-groups of consecutive KV heads (see pa_decode_common.h).
// Inside a wave, a K/V row of D elements is split into 16-byte chunks: LPT =
// D*elem/16 lanes cover one token row, so one wave load instruction covers
// TPL = 64/LPT token rows as whole contiguous row segments, and each lane owns
// the same chunk of NL = bs/TPL rows of the block.  q.k partial sums are
// reduced across the LPT lanes of a row with DPP (bitwise identical in every
// lane), so every lane holds the scores of its own rows.  Each lane keeps an
// online-softmax state (m, l, acc[G][chunk]) over its own rows; no cross-lane
// exchange happens inside the block loop.  The loads of a wave's next block
// are issued before the current block is consumed.  At the end the per-lane
// states are merged across the TPL row groups with shuffles.  Scores are kept in
// log2 units (scale * k_scale * log2 e folded in) so the exponentials are
// single v_exp_f32 instructions.

#include <hip/hip_runtime.h>

#include "pa_decode_common.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// ------------------------------------------------------------------ q . k ops

template <int KV, int Q>
struct Ops;

template <>
struct Ops<PA_F32, PA_F32> {
  static constexpr int CE = 4;  // elements per 16-byte chunk
  struct QReg {
    float f[4];
  };
  __device__ static QReg load_q(const char* row, int e0) {
    QReg r;
    Chunk c = *reinterpret_cast<const Chunk*>(row + e0 * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.f[i] = u2f(c.w[i]);
    return r;
  }
  __device__ static float dot(const QReg& q, const Chunk& k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = __builtin_fmaf(q.f[i], u2f(k.w[i]), s);
    return s;
  }
  __device__ static void to_f32(const Chunk& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = u2f(v.w[i]);
  }
};

template <>
struct Ops<PA_F16, PA_F16> {
  static constexpr int CE = 8;
  struct QReg {
    uint32_t w[4];
  };
  __device__ static QReg load_q(const char* row, int e0) {
    Chunk c = *reinterpret_cast<const Chunk*>(row + e0 * 2);
    QReg r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = c.w[i];
    return r;
  }
  // v_dot2_f32_f16: two exact fp16 products added into an fp32 accumulator
  __device__ static float dot(const QReg& q, const Chunk& k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qw = q.w[i], kw = k.w[i];
      s = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qw), __builtin_bit_cast(f16x2, kw), s,
                                 false);
    }
    return s;
  }
  __device__ static void to_f32(const Chunk& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = v.w[i];
      const f16x2 h = __builtin_bit_cast(f16x2, w);
      o[2 * i] = static_cast<float>(h[0]);
      o[2 * i + 1] = static_cast<float>(h[1]);
    }
  }
};

template <>
struct Ops<PA_BF16, PA_BF16> {
  static constexpr int CE = 8;
  struct QReg {
    uint32_t w[4];
  };
  __device__ static QReg load_q(const char* row, int e0) {
    Chunk c = *reinterpret_cast<const Chunk*>(row + e0 * 2);
    QReg r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = c.w[i];
    return r;
  }
  // v_dot2_f32_bf16: two exact bf16 products added into an fp32 accumulator
  __device__ static float dot(const QReg& q, const Chunk& k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t qw = q.w[i], kw = k.w[i];
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qw),
                                          __builtin_bit_cast(bf16x2, kw), s, false);
    }
    return s;
  }
  __device__ static void to_f32(const Chunk& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = u2f(v.w[i] << 16);
      o[2 * i + 1] = u2f(v.w[i] & 0xffff0000u);
    }
  }
};

// 8-bit cache (e4m3 or e5m2) with 16-bit queries: codes decoded to fp32,
// fp32 FMAs.
template <int Q, int FMT>
struct OpsFP8 {
  static constexpr int CE = 16;
  struct QReg {
    float f[16];
  };
  __device__ static QReg load_q(const char* row, int e0) {
    QReg r;
#pragma unroll
    for (int i = 0; i < 16; ++i) r.f[i] = load_elem<Q>(row, e0 + i);
    return r;
  }
  __device__ static void to_f32(const Chunk& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fp8x4_to_f32<FMT>(v.w[i], o + 4 * i);
  }
  __device__ static float dot(const QReg& q, const Chunk& k) {
    float kf[16];
    to_f32(k, kf);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = __builtin_fmaf(q.f[i], kf[i], s);
    return s;
  }
};
template <>
struct Ops<PA_FP8_E4M3, PA_BF16> : OpsFP8<PA_BF16, PA_FP8_E4M3> {};
template <>
struct Ops<PA_FP8_E4M3, PA_F16> : OpsFP8<PA_F16, PA_FP8_E4M3> {};
template <>
struct Ops<PA_FP8_E5M2, PA_BF16> : OpsFP8<PA_BF16, PA_FP8_E5M2> {};
template <>
struct Ops<PA_FP8_E5M2, PA_F16> : OpsFP8<PA_F16, PA_FP8_E5M2> {};

// ------------------------------------------------------------------ kernel

// KV heads (waves) per work-group
constexpr int kValuHeads = 4;

template <int KV, int Q, int D, int BS, int G, int ST>
__global__ __launch_bounds__(kValuHeads * 64) void decode_valu_kernel(const DecodeParams p) {
  using O = Ops<KV, Q>;
  constexpr int CE = O::CE;
  constexpr int KVB = Elem<KV>::bytes;
  constexpr int QB = Elem<Q>::bytes;
  constexpr int LPT = D / CE;    // lanes per token row
  constexpr int TPL = 64 / LPT;  // token rows per wave load
  // A wave load of TPL rows spans UB blocks: 1, or 2 for 8-bit D = 64 rows
  // (16 per load) in 8-token blocks.  Then each load goes out once per
  // block, the other block's lanes out of range (they read zeros), and the
  // results are merged.
  constexpr int UB = TPL > BS ? TPL / BS : 1;
  constexpr int NL = UB > 1 ? 1 : BS / TPL;  // rows per lane per unit of UB blocks
  static_assert(D % CE == 0 && 64 % LPT == 0 && (UB > 1 ? TPL == UB * BS : BS % TPL == 0),
                "unsupported tile shape");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = blockIdx.x;
  const int g = hg * p.heads_per_wg + wave;
  __shared__ PlanLds plan_lds;
  const int32_t* prefix = schedule_prefix(p, plan_lds);  // every thread, before any leaves
  if (g >= p.Hkv) return;  // last head group of a head count that is not a multiple
  const int c = lane % LPT;   // chunk of the row this lane owns
  const int tg = lane / LPT;  // row within a wave load

  const uint32_t row_stride = static_cast<uint32_t>(p.Hkv) * D * KVB;  // bytes between token rows
  const uint32_t blk_bytes = row_stride * BS;
  // this lane's chunk of row tg of a block (row tg % BS of block tg / BS
  // when a load spans blocks), relative to that block's start
  const int lane_off = static_cast<int>(g * D * KVB + c * 16 + (UB > 1 ? tg % BS : tg) * row_stride);
  const char* kpool = static_cast<const char*>(p.k_cache);
  const char* vpool = static_cast<const char*>(p.v_cache);
  // score scale in log2 units and V scale of this wave's KV head
  const float qk = p.k_scales ? p.qk_scale_log2 * p.k_scales[g] : p.qk_scale_log2;
  const float vs = p.v_scales ? p.v_scales[g] : p.v_scale;

  struct Buf {
    Chunk k[NL], v[NL];
  };

  // Loads of the unit's blocks (nothing is read for an id < 0).
  auto load = [&](const int (&id)[UB], Buf& r) {
    if constexpr (UB > 1) {
#pragma unroll
      for (int w = 0; w < 4; ++w) r.k[0].w[w] = r.v[0].w[w] = 0u;
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int blk = id[u];
        const size_t off = static_cast<size_t>(blk < 0 ? 0 : blk) * blk_bytes;
        const uint32_t n = blk < 0 ? 0u : blk_bytes;
        const __amdgpu_buffer_rsrc_t kr = block_rsrc(kpool + off, n);
        const __amdgpu_buffer_rsrc_t vr = block_rsrc(vpool + off, n);
        const int o = tg / BS == u ? lane_off : 0x7fffff00;
        Chunk a, b;
        buffer_load<4>(kr, o, 0, a.w);
        buffer_load<4>(vr, o, 0, b.w);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          r.k[0].w[w] |= a.w[w];
          r.v[0].w[w] |= b.w[w];
        }
      }
      return;
    }
    const int blk = id[0];
    const size_t off = static_cast<size_t>(blk < 0 ? 0 : blk) * blk_bytes;
    const uint32_t n = blk < 0 ? 0u : blk_bytes;
    const __amdgpu_buffer_rsrc_t kr = block_rsrc(kpool + off, n);
    const __amdgpu_buffer_rsrc_t vr = block_rsrc(vpool + off, n);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load<4>(kr, lane_off, i * TPL * row_stride, r.k[i].w);
#pragma unroll
    for (int i = 0; i < NL; ++i) buffer_load<4>(vr, lane_off, i * TPL * row_stride, r.v[i].w);
  };

  for_each_segment(p, prefix, hg, wave, G, [&](int b, const PartitionSpan& span, const SegmentDest& dst) {
    typename O::QReg qr[G];
    {
      const char* qrow =
          static_cast<const char*>(p.q) + (static_cast<size_t>(b) * p.Hq + g * G) * D * QB;
#pragma unroll
      for (int h = 0; h < G; ++h) qr[h] = O::load_q(qrow + h * D * QB, c * CE);
    }

    float m[G], l[G], acc[G][CE];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kMaxInit;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < CE; ++e) acc[h][e] = 0.f;
    }

    auto consume = [&](int j, unsigned ok, Buf& r) {
      // valid rows of this block (only the last block of a sequence is
      // partial; a block id outside the pool counts none).  A unit of two
      // blocks: this lane's row tg is row tg % BS of block j + tg / BS.
      int valid;
      if constexpr (UB > 1) {
        const int u = tg / BS;
        valid = ((ok >> u) & 1u) && (j + u) * BS + tg % BS < span.L ? TPL : 0;
      } else {
        valid = ok ? min(BS, span.L - j * BS) : 0;
      }
      float s[NL][G];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int h = 0; h < G; ++h) s[i][h] = group_sum<LPT>(O::dot(qr[h], r.k[i])) * qk;
      }
      if (valid < BS) {
        // rows past the end are excluded outright: their K and V may hold
        // anything (NaN included), so they get weight 0 and a zeroed V row.
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          if (i * TPL + tg >= valid) {
#pragma unroll
            for (int h = 0; h < G; ++h) s[i][h] = -__builtin_inff();
#pragma unroll
            for (int w = 0; w < 4; ++w) r.v[i].w[w] = 0u;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = m[h];
#pragma unroll
        for (int i = 0; i < NL; ++i) mx = fmaxf(mx, s[i][h]);
        const float alpha = fast_exp2(m[h] - mx);
        m[h] = mx;
        float lh = l[h] * alpha;
#pragma unroll
        for (int e = 0; e < CE; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const float pw = fast_exp2(s[i][h] - mx);
          lh += pw;
          float vf[CE];  // V row i in fp32, converted where it is used
          O::to_f32(r.v[i], vf);
#pragma unroll
          for (int e = 0; e < CE; ++e) acc[h][e] = __builtin_fmaf(pw, vf[e], acc[h][e]);
        }
        l[h] = lh;
      }
    };

    const int32_t* table =
        p.block_tables + static_cast<size_t>(b) * (p.max_blocks_per_seq >> p.sub_shift);
    walk_blocks<ST, UB, 0, Buf>(table, span, p.num_blocks, p.sub_shift, lane, load, consume);

    // merge the per-lane states of the TPL row groups that own the same
    // chunk; the butterfly leaves the merged state in every lane
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = __shfl_xor(m[h], off, 64);
        const float lo = __shfl_xor(l[h], off, 64);
        const float M = fmaxf(m[h], mo);
        const float a = fast_exp2(m[h] - M);
        const float ao = fast_exp2(mo - M);
        l[h] = l[h] * a + lo * ao;
#pragma unroll
        for (int e = 0; e < CE; ++e)
          acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], off, 64) * ao;
        m[h] = M;
      }
    }

    if (tg == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) store_segment<CE>(p, dst, h, c * CE, m[h], l[h], acc[h], vs);
    }
  });
  finish_splits<D, (G < 4 ? G : 4), 4>(plan_lds, lane);
}

// ------------------------------------------------------------------ dispatch

namespace {

// register sets in the load pipeline (blocks in flight per wave, plus one);
// fp32 caches take one, their rows already fill the register file
template <int KV>
constexpr int kStages = KV == PA_F32 ? 1 : 2;

template <int KV_, int Q_, int D_, int BS_, int G_>
struct Tag {
  static constexpr int KV = KV_, Q = Q_, D = D_, BS = BS_, G = G_;
  static const void* kernel() {
    return reinterpret_cast<const void*>(&decode_valu_kernel<KV, Q, D, BS, G, kStages<KV>>);
  }
  static hipError_t launch(const DecodeParams& p, hipStream_t s) {
    const dim3 grid = p.balanced ? dim3(p.head_groups, p.groups, 1)
                                 : dim3(p.head_groups, p.B, p.num_partitions);
    hipLaunchKernelGGL((decode_valu_kernel<KV, Q, D, BS, G, kStages<KV>>), grid,
                       dim3(p.heads_per_wg * 64), 0, s, p);
    return hipGetLastError();
  }
};

// Calls f(Tag<...>{}) for the instance serving p; false if none is built.
template <int KV, int Q, int D, int BS, typename F>
bool by_group(const DecodeParams& p, F&& f) {
  switch (p.Hq / p.Hkv) {
    case 1: f(Tag<KV, Q, D, BS, 1>{}); return true;
    case 2: f(Tag<KV, Q, D, BS, 2>{}); return true;
    case 4:
      if constexpr (KV == PA_F32) {
        f(Tag<KV, Q, D, BS, 4>{});
        return true;
      }
      return false;
    case 8:
      if constexpr (KV == PA_F32) {
        f(Tag<KV, Q, D, BS, 8>{});
        return true;
      }
      return false;
    default: return false;
  }
}

template <int KV, int Q, int D, typename F>
bool by_block(const DecodeParams& p, F&& f) {
  switch (p.block_size) {
    case 8: return by_group<KV, Q, D, 8>(p, f);
    case 16: return by_group<KV, Q, D, 16>(p, f);
    case 32: return by_group<KV, Q, D, 32>(p, f);
    default: return false;
  }
}

template <int KV, int Q, typename F>
bool by_dim(const DecodeParams& p, F&& f) {
  switch (p.D) {
    case 64: return by_block<KV, Q, 64>(p, f);
    case 128: return by_block<KV, Q, 128>(p, f);
    default: return false;
  }
}

template <typename F>
bool dispatch(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype, F&& f) {
  if (kv_dtype == PA_F32 && q_dtype == PA_F32) return by_dim<PA_F32, PA_F32>(p, f);
  if (kv_dtype == PA_F16 && q_dtype == PA_F16) return by_dim<PA_F16, PA_F16>(p, f);
  if (kv_dtype == PA_BF16 && q_dtype == PA_BF16) return by_dim<PA_BF16, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16) return by_dim<PA_FP8_E4M3, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_F16) return by_dim<PA_FP8_E4M3, PA_F16>(p, f);
  if (kv_dtype == PA_FP8_E5M2 && q_dtype == PA_BF16) return by_dim<PA_FP8_E5M2, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E5M2 && q_dtype == PA_F16) return by_dim<PA_FP8_E5M2, PA_F16>(p, f);
  return false;
}

}  // namespace

int32_t decode_valu_heads() { return kValuHeads; }

hipError_t launch_decode_valu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                              hipStream_t stream, bool* supported) {
  hipError_t e = hipSuccess;
  *supported = dispatch(p, q_dtype, kv_dtype, [&](auto t) { e = decltype(t)::launch(p, stream); });
  return e;
}

int32_t decode_valu_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype) {
  const void* fn = nullptr;
  if (!dispatch(p, q_dtype, kv_dtype, [&](auto t) { fn = decltype(t)::kernel(); })) return 0;
  return groups_per_cu(fn, p.heads_per_wg * 64);
}

}  // namespace pa
