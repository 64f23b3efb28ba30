// pa_decode_mfma.hip -- decode-partition kernel on the matrix cores, used for
// grouped-query attention with G = Hq/Hkv from 3 to 16 and 16-bit or e4m3
// caches.
//
// With grouped-query attention (P1 = Ultralytics glossary page
// "PagedAttention", section "İlgili Teknikler") the G query heads that share
// a KV head read the same K/V block, so per 16-token tile the scores are a
// dense G x 16 x D contraction and the weighted sum a G x D x 16 one: at G = 8
// and 16-bit caches that is 8 flop per byte of K/V, more than the vector ALUs
// sustain at full HBM bandwidth.  Both contractions run here as 16x16 MFMAs
// with the query group padded to 16 rows; the softmax between them runs on
// the MFMA result layout.  The paging itself is as in the VALU kernel: each
// wave follows the block table, one block at a time, and the scores never
// leave registers (P1 "Sayfalama Nasıl Çalışır"; "İlgili Teknikler",
// FlashAttention-style tiling).
//
// Lane layout of a 16x16 MFMA on gfx950 (lane l, lo = l % 16, grp = l / 16):
//   A (16 x K): row lo, a run of K/4 values picked by (grp, element);
//   B (K x 16): column lo, the same (grp, element) -> k pairing as A;
//   D (16 x 16, four fp32 per lane): D[4*grp + r][lo] in element r.
// Only the pairing of A and B slots matters for a contraction, so each side
// may assign head-dim positions (or tokens) to (grp, element) slots freely as
// long as both use the same assignment.
//
// Scores:  S^T[t][q] = sum_d K[t][d] Q[q][d], one v_mfma_f32_16x16x32 per 32
//   head-dim values: A = 16 token rows of K (lane: token lo), B = Q^T (lane:
//   query lo; zero for lo >= G).  Lane l then holds the scores of query lo
//   for tokens 4*grp + r, r = 0..3.
// Weighted sum: O[q][d] += sum_t P[q][t] V[t][d], one v_mfma_f32_16x16x16 per
//   16 output columns: A = P straight from the score layout (lane: query lo,
//   tokens 4*grp + e), B = V with lane l holding tokens 4*grp + e of column
//   lo, where MFMA number mm maps column lo to head-dim d = (D/16)*lo + mm.
//   Each lane therefore loads one contiguous D/16-element run of four token
//   rows, and the 16 lanes of a group cover each row whole (coalesced).
// The running maximum is kept exact per query: when a block raises it, the
// accumulators of the affected queries are rescaled (rare after the first
// blocks).  8-bit codes (e4m3 or e5m2) are widened to the operand type (bf16
// or f16, both hold every value of either format exactly) in registers
// before the MFMAs.

#include <hip/hip_runtime.h>

#include "pa_decode_common.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

// KV heads (waves) per work-group
constexpr int kMfmaHeads = 8;

// COOP (8-bit caches, D = 128, blocks of 16 or 32 tokens, every KV head of
// the work-group present): the
// work-group loads each unit together, every token row's slice of the group's
// eight heads (1 KiB, contiguous) by one 64-lane load straight into LDS, and
// each wave then reads its head's K and V from there.  The pool is then read
// in whole 1 KiB pieces instead of one head's 128 bytes per row, which the
// memory system serves faster.
template <int KV, int Q, int D, int BS, int ST, bool COOP>
__global__ __launch_bounds__(kMfmaHeads * 64) void decode_mfma_kernel(const DecodeParams p) {
  using M = Mfma<Q>;
  constexpr bool FP8 = is_fp8(KV);
  constexpr int KVB = FP8 ? 1 : 2;
  constexpr int SS = D / 32;                    // score MFMAs per tile (32 head-dim values each)
  constexpr int EPL = D / 16;                   // V elements per lane per row = PV MFMAs per tile
  // 8-token blocks: a 16-token tile spans two blocks, so each lane reads
  // through its own address (its K row's block, its V rows' block) instead
  // of one buffer resource per block
  constexpr bool SPLIT = BS < 16;
  constexpr int TPB = SPLIT ? 1 : BS / 16;      // 16-token tiles per block (or per 16/BS blocks)
  // tokens per pipeline unit: 32 (two 16-token tiles), or one tile per LDS
  // stage when cooperative loads walk 16-token blocks (four stages fit)
  constexpr int UT = (COOP && BS == 16) ? 16 : 32;
  constexpr int UB = UT / BS;                   // blocks per pipeline unit
  constexpr int TT = UT / 16;                   // 16-token tiles per unit
  constexpr int KW = D / 8;                     // dwords of 16-bit K per lane per tile
  constexpr int KR = FP8 ? D / 16 : D / 8;      // dwords of stored K per lane per tile
  constexpr int VW = EPL / 2;                   // dwords of 16-bit V per lane per row
  constexpr int VR = FP8 ? EPL / 4 : EPL / 2;   // dwords of stored V per lane per row
  constexpr int KLD = KR >= 4 ? 4 : KR;         // dwords per K load instruction
  const int G = p.Hq / p.Hkv;  // 3..16: the query group padded to the MFMA's 16 rows
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BS == 8 || BS == 16 || BS == 32, "block size");
  static_assert(!COOP || (FP8 && D == 128 && BS >= 16), "cooperative loads: 8-bit caches, D = 128");
  // cooperative stages: the unit's token rows of K, then of V, each row the
  // group's 1 KiB slice padded by 16 bytes (rows 16 bytes apart in the banks);
  // wave w loads rows kRpw*w .. kRpw*w + kRpw - 1 of both
  constexpr int kRows = UT;
  constexpr int kRpw = kRows / kMfmaHeads;
  constexpr int kPitch = kMfmaHeads * D * KVB + 16;
  constexpr int kStageBytes = 2 * kRows * kPitch;
  constexpr int kLdsStages = kRows == 16 ? 4 : 2;  // 133 KiB of LDS either way
  __shared__ __attribute__((aligned(16))) unsigned char coop_lds[COOP ? kLdsStages * kStageBytes : 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = blockIdx.x;
  const int g = hg * p.heads_per_wg + wave;
  __shared__ PlanLds plan_lds;
  const int32_t* prefix = schedule_prefix(p, plan_lds);  // every thread, before any leaves
  if (g >= p.Hkv) return;  // last head group of a head count that is not a multiple
  const int lo = lane & 15;
  const int grp = lane >> 4;

  // Head-dim chunk (8 values) that lane group grp feeds into score MFMA s.
  // 16-bit caches: chunk 4s+grp, so each K load instruction reads 64
  // contiguous bytes of every one of the tile's 16 rows.  e4m3: chunk
  // SS*grp+s, so a lane's K bytes for the tile are one contiguous run.
  auto chunk_of = [&](int s) { return FP8 ? SS * grp + s : 4 * s + grp; };

  const uint32_t row_stride = static_cast<uint32_t>(p.Hkv) * D * KVB;
  const uint32_t blk_bytes = row_stride * BS;
  const int head_off = g * D * KVB;
  // K: token row lo of each tile; e4m3 lanes start at their contiguous run,
  // 16-bit lanes at chunk grp (chunk 4s+grp is 64*s bytes further)
  const int k_off = head_off + lo * row_stride + (FP8 ? grp * (D / 4) : grp * 16);
  // V: token rows 4*grp + e of each tile, elements [EPL*lo, EPL*lo + EPL)
  const int v_off = head_off + 4 * grp * row_stride + EPL * lo * KVB;
  const char* kpool = static_cast<const char*>(p.k_cache);
  const char* vpool = static_cast<const char*>(p.v_cache);
  // 8-token blocks: K row lo of a tile is row lo % 8 of the tile's block
  // lo / 8; V rows 4*grp + e are rows 4*(grp % 2) + e of block grp / 2
  const int k_off8 = head_off + (lo & 7) * row_stride + (FP8 ? grp * (D / 4) : grp * 16);
  const int v_off8 = head_off + 4 * (grp & 1) * row_stride + EPL * lo * KVB;
  // score scale in log2 units and V scale of this wave's KV head
  const float qk = p.k_scales ? p.qk_scale_log2 * p.k_scales[g] : p.qk_scale_log2;
  const float vs = p.v_scales ? p.v_scales[g] : p.v_scale;

  struct Raw {
    uint32_t k[TT][KR];
    uint32_t v[TT][4][VR];
  };

  // Loads of the unit's blocks (nothing is read for an id < 0; with 8-token
  // blocks block 0 is read instead, and consume() excludes those rows).
  auto load = [&](const int (&id)[UB], Raw& r) {
    if constexpr (SPLIT) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int kb = lo < 8 ? id[2 * tt] : id[2 * tt + 1];
        const int vb = grp < 2 ? id[2 * tt] : id[2 * tt + 1];
        const char* kp = kpool + static_cast<size_t>(kb < 0 ? 0 : kb) * blk_bytes + k_off8;
        const char* vp = vpool + static_cast<size_t>(vb < 0 ? 0 : vb) * blk_bytes + v_off8;
        if constexpr (FP8) {
          global_load<KLD, 0>(kp, &r.k[tt][0]);
          if constexpr (KR > KLD) global_load<KLD, 16>(kp, &r.k[tt][KLD]);
        } else {
          global_load<4, 0>(kp, &r.k[tt][0]);
          global_load<4, 64>(kp, &r.k[tt][4]);
          if constexpr (SS > 2) {
            global_load<4, 128>(kp, &r.k[tt][8]);
            global_load<4, 192>(kp, &r.k[tt][12]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) global_load<VR, 0>(vp + e * row_stride, r.v[tt][e]);
      }
      return;
    }
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int blk = id[ub];
      const size_t off = static_cast<size_t>(blk < 0 ? 0 : blk) * blk_bytes;
      const uint32_t n = blk < 0 ? 0u : blk_bytes;
      const __amdgpu_buffer_rsrc_t kr = block_rsrc(kpool + off, n);
#pragma unroll
      for (int tb = 0; tb < TPB; ++tb) {
        const int tt = ub * TPB + tb;
        const int ts = tb * 16 * row_stride;
        if constexpr (FP8) {
          buffer_load<KLD, 0>(kr, k_off, ts, &r.k[tt][0]);
          if constexpr (KR > KLD) buffer_load<KLD, 16>(kr, k_off, ts, &r.k[tt][KLD]);
        } else {
          buffer_load<4, 0>(kr, k_off, ts, &r.k[tt][0]);
          buffer_load<4, 64>(kr, k_off, ts, &r.k[tt][4]);
          if constexpr (SS > 2) {
            buffer_load<4, 128>(kr, k_off, ts, &r.k[tt][8]);
            buffer_load<4, 192>(kr, k_off, ts, &r.k[tt][12]);
          }
        }
      }
    }
#pragma unroll
    for (int ub = 0; ub < UB; ++ub) {
      const int blk = id[ub];
      const size_t off = static_cast<size_t>(blk < 0 ? 0 : blk) * blk_bytes;
      const uint32_t n = blk < 0 ? 0u : blk_bytes;
      const __amdgpu_buffer_rsrc_t vr = block_rsrc(vpool + off, n);
#pragma unroll
      for (int tb = 0; tb < TPB; ++tb) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          buffer_load<VR>(vr, v_off, (tb * 16 + e) * row_stride, r.v[ub * TPB + tb][e]);
      }
    }
  };

  for_each_segment(p, prefix, hg, wave, G, [&](int b, const PartitionSpan& span, const SegmentDest& dst) {
    // Q^T operand: query lo of the group, zero rows beyond G.
    uint32_t qw[KW];
    if (lo < G) {
      const char* qrow =
          static_cast<const char*>(p.q) + ((static_cast<size_t>(b) * p.Hq + g * G + lo) * D) * 2;
#pragma unroll
      for (int s = 0; s < SS; ++s) {
        const Chunk c = *reinterpret_cast<const Chunk*>(qrow + chunk_of(s) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) qw[4 * s + i] = c.w[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < KW; ++i) qw[i] = 0u;
    }

    f32x4 O[EPL];
#pragma unroll
    for (int mm = 0; mm < EPL; ++mm) O[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kMaxInit;  // running max of query lo (log2 units), same in all four groups
    float l_part = 0.f;      // this lane's share of the running sum of query lo

    auto consume = [&](int j0, unsigned ok, Raw& r) {
      // valid rows of each 16-token tile (a mask, bit r for row r); a block
      // that is not ok counts none
      uint32_t vmask[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if constexpr (SPLIT) {
          uint32_t mk = 0;
#pragma unroll
          for (int h = 0; h < 16 / BS; ++h) {
            const int ub = tt * (16 / BS) + h;
            const int n = (ok >> ub) & 1u ? min(BS, max(0, span.L - (j0 + ub) * BS)) : 0;
            mk |= ((1u << n) - 1u) << (h * BS);
          }
          vmask[tt] = mk;
        } else {
          const int ub = tt / TPB;
          const int first = (j0 + ub) * BS + (tt % TPB) * 16;
          const int n = (ok >> ub) & 1u ? min(16, max(0, span.L - first)) : 0;
          vmask[tt] = (1u << n) - 1u;
        }
      }
      float sc[TT][4];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        uint32_t kw[KW];
        if constexpr (FP8) {
#pragma unroll
          for (int i = 0; i < KR; ++i) widen_fp8<Q, KV>(r.k[tt][i], kw[2 * i], kw[2 * i + 1]);
        } else {
#pragma unroll
          for (int i = 0; i < KW; ++i) kw[i] = r.k[tt][i];
        }
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SS; ++s) S = M::qk(&kw[4 * s], &qw[4 * s], S);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // rows past the end may hold anything (NaN included): excluded outright
          sc[tt][i] = (vmask[tt] >> (4 * grp + i)) & 1u ? S[i] * qk : -__builtin_inff();
        }
      }
      float bm = sc[0][0];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) bm = fmaxf(bm, sc[tt][i]);
      }
      bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float mn = fmaxf(m_run, bm);
      if (__ballot(mn > m_run)) {
        const float alpha = fast_exp2(m_run - mn);
        l_part *= alpha;
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
        for (int mm = 0; mm < EPL; ++mm) {
#pragma unroll
          for (int i = 0; i < 4; ++i) O[mm][i] *= a[i];
        }
        m_run = mn;
      }
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = fast_exp2(sc[tt][i] - m_run);
        const uint32_t pa0 = M::pack2(pw[0], pw[1]);
        const uint32_t pa1 = M::pack2(pw[2], pw[3]);
        // the running sum takes the weights as the weighted sum uses them,
        // rounded to the operand type: the output is then an exact weighted
        // mean of V rows (the fp32 weights would scale it by up to a
        // half-ulp of that type)
        l_part += M::pair_sum(pa0) + M::pair_sum(pa1);
        if (vmask[tt] != 0xffffu) {
          // zero the V rows past the end so that 0 * NaN cannot reach the sum
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!((vmask[tt] >> (4 * grp + e)) & 1u)) {
#pragma unroll
              for (int i = 0; i < VR; ++i) r.v[tt][e][i] = 0u;
            }
          }
        }
        uint32_t vw[4][VW];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < VR; ++i) widen_fp8<Q, KV>(r.v[tt][e][i], vw[e][2 * i], vw[e][2 * i + 1]);
          } else {
#pragma unroll
            for (int i = 0; i < VW; ++i) vw[e][i] = r.v[tt][e][i];
          }
        }
#pragma unroll
        for (int mm = 0; mm < EPL; ++mm) {
          const uint32_t b0 = pick_halves(vw[0][mm >> 1], vw[1][mm >> 1], mm & 1);
          const uint32_t b1 = pick_halves(vw[2][mm >> 1], vw[3][mm >> 1], mm & 1);
          O[mm] = M::pv(pa0, pa1, b0, b1, O[mm]);
        }
      }
    };

    const int32_t* table =
        p.block_tables + static_cast<size_t>(b) * (p.max_blocks_per_seq >> p.sub_shift);
    if constexpr (COOP) {
      // wave w loads its unit rows (one block: a unit is one block here) of K
      // and of V, each row the slice of the group's heads, into the stage;
      // the whole unit is there after the walk's barrier
      static_assert(!COOP || UB == 1, "a cooperative unit is one block");
      const int grp_off = hg * kMfmaHeads * D * KVB;
      auto issue = [&](const int (&id)[UB], int stage) {
        unsigned char* st = coop_lds + stage * kStageBytes;
        const int blk = id[0];
        const size_t off = static_cast<size_t>(blk < 0 ? 0 : blk) * blk_bytes;
        const uint32_t n = blk < 0 ? 0u : blk_bytes;
        const __amdgpu_buffer_rsrc_t kr = block_rsrc(kpool + off, n);
        const __amdgpu_buffer_rsrc_t vr = block_rsrc(vpool + off, n);
#pragma unroll
        for (int q = 0; q < kRpw; ++q) {
          const int r = kRpw * wave + q;
          const int vo = r * static_cast<int>(row_stride) + grp_off + lane * 16;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              kr, (__attribute__((address_space(3))) void*)(st + r * kPitch), 16, vo, 0, 0, kLoadNT);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              vr, (__attribute__((address_space(3))) void*)(st + (kRows + r) * kPitch), 16, vo, 0, 0,
              kLoadNT);
        }
      };
      // this wave's head from the stage, in the register layout of the
      // direct loads: K bytes [32*grp, +32) of row lo of each tile, V bytes
      // [8*lo, +8) of rows 4*grp + e.  The reads are one asm block per tile
      // that waits for them itself: as plain loads the compiler would first
      // wait for every load into LDS in flight (it cannot tell the stages
      // apart), which would leave no stage loading during the arithmetic.
      static_assert(!COOP || EPL == 8, "8-byte V runs");
      const uint32_t lds0 = static_cast<uint32_t>(
          reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)coop_lds));
      auto read = [&](int stage, Raw& r) {
        const uint32_t st = lds0 + static_cast<uint32_t>(stage * kStageBytes);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const uint32_t ka = st + (16 * tt + lo) * kPitch + wave * D + grp * (D / 4);
          const uint32_t va = st + (kRows + 16 * tt + 4 * grp) * kPitch + wave * D + EPL * lo;
          u32x4 k0, k1;
          u32x2 v0, v1, v2, v3;
          asm volatile(
              "ds_read_b128 %0, %6\n"
              "ds_read_b128 %1, %6 offset:16\n"
              "ds_read_b64 %2, %7\n"
              "ds_read_b64 %3, %7 offset:%8\n"
              "ds_read_b64 %4, %7 offset:%9\n"
              "ds_read_b64 %5, %7 offset:%10\n"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(k0), "=&v"(k1), "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
              : "v"(ka), "v"(va), "n"(kPitch), "n"(2 * kPitch), "n"(3 * kPitch)
              : "memory");
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            r.k[tt][i] = k0[i];
            r.k[tt][4 + i] = k1[i];
          }
          r.v[tt][0][0] = v0[0];
          r.v[tt][0][1] = v0[1];
          r.v[tt][1][0] = v1[0];
          r.v[tt][1][1] = v1[1];
          r.v[tt][2][0] = v2[0];
          r.v[tt][2][1] = v2[1];
          r.v[tt][3][0] = v3[0];
          r.v[tt][3][1] = v3[1];
        }
      };
      walk_blocks_coop<UB, kLdsStages, 2 * kRpw, Raw>(table, span, p.num_blocks, p.sub_shift, lane, issue,
                                                   read, consume);
    } else {
      // waves meet every 8 units (8-bit caches) or 4 (16-bit), the intervals
      // that measured fastest for each
      walk_blocks<ST, UB, (FP8 ? 8 : 4), Raw>(table, span, p.num_blocks, p.sub_shift, lane, load,
                                                consume);
    }

    // l of query lo summed over the four lane groups; every lane then fetches
    // m and l of the queries whose accumulators it holds (4*grp + i)
    float lt = l_part + __shfl_xor(l_part, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = 4 * grp + i;
      const float lq = __shfl(lt, q, 64);
      const float mq = __shfl(m_run, q, 64);
      if (q < G) {
        float o[EPL];
#pragma unroll
        for (int mm = 0; mm < EPL; ++mm) o[mm] = O[mm][i];
        store_segment<EPL>(p, dst, q, EPL * lo, mq, lq, o, vs);
      }
    }
  });
  finish_splits<D, 4, (D == 128 ? 16 : 8)>(plan_lds, lane);  // 4 queries per combine pass
}

// ------------------------------------------------------------------ dispatch

namespace {

// register sets in the load pipeline (units in flight per wave, plus one)
constexpr int kStages = 2;

// Cooperative loads need every wave of a work-group to load its share, so
// every KV head of the group present: the head count a multiple of eight.
bool use_coop(const DecodeParams& p, int kv, int d) {
  return is_fp8(kv) && d == 128 && p.heads_per_wg == kMfmaHeads && p.Hkv % kMfmaHeads == 0;
}

template <int KV_, int Q_, int D_, int BS_>
struct Tag {
  static constexpr int KV = KV_, Q = Q_, D = D_, BS = BS_;
  // instances that have the mode (a unit of 8-token blocks spans four blocks,
  // which the per-wave row assignment does not cover)
  static constexpr bool kCoop = is_fp8(KV) && D == 128 && BS >= 16;
  template <bool C>
  static const void* fn() {
    return reinterpret_cast<const void*>(&decode_mfma_kernel<KV, Q, D, BS, kStages, C>);
  }
  static const void* kernel(const DecodeParams& p) {
    if constexpr (kCoop) {
      if (use_coop(p, KV, D)) return fn<true>();
    }
    return fn<false>();
  }
  static hipError_t launch(const DecodeParams& p, hipStream_t s) {
    const dim3 grid = p.balanced ? dim3(p.head_groups, p.groups, 1)
                                 : dim3(p.head_groups, p.B, p.num_partitions);
    hipLaunchKernelGGL(reinterpret_cast<void (*)(DecodeParams)>(const_cast<void*>(kernel(p))), grid,
                       dim3(p.heads_per_wg * 64), 0, s, p);
    return hipGetLastError();
  }
};

template <int KV, int Q, int D, typename F>
bool by_block(const DecodeParams& p, F&& f) {
  switch (p.block_size) {
    case 8: f(Tag<KV, Q, D, 8>{}); return true;
    case 16: f(Tag<KV, Q, D, 16>{}); return true;
    case 32: f(Tag<KV, Q, D, 32>{}); return true;
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
  if (kv_dtype == PA_F16 && q_dtype == PA_F16) return by_dim<PA_F16, PA_F16>(p, f);
  if (kv_dtype == PA_BF16 && q_dtype == PA_BF16) return by_dim<PA_BF16, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_BF16) return by_dim<PA_FP8_E4M3, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E4M3 && q_dtype == PA_F16) return by_dim<PA_FP8_E4M3, PA_F16>(p, f);
  if (kv_dtype == PA_FP8_E5M2 && q_dtype == PA_BF16) return by_dim<PA_FP8_E5M2, PA_BF16>(p, f);
  if (kv_dtype == PA_FP8_E5M2 && q_dtype == PA_F16) return by_dim<PA_FP8_E5M2, PA_F16>(p, f);
  return false;
}

}  // namespace

int32_t decode_mfma_heads() { return kMfmaHeads; }

bool decode_mfma_serves(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t group) {
  if (group < 3 || group > 16) return false;
  return (kv_dtype == PA_F16 && q_dtype == PA_F16) || (kv_dtype == PA_BF16 && q_dtype == PA_BF16) ||
         (is_fp8(kv_dtype) && (q_dtype == PA_BF16 || q_dtype == PA_F16));
}

hipError_t launch_decode_mfma(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                              hipStream_t stream, bool* supported) {
  hipError_t e = hipSuccess;
  *supported = dispatch(p, q_dtype, kv_dtype, [&](auto t) { e = decltype(t)::launch(p, stream); });
  return e;
}

int32_t decode_mfma_groups_per_cu(const DecodeParams& p, pa_dtype q_dtype, pa_dtype kv_dtype) {
  const void* fn = nullptr;
  if (!dispatch(p, q_dtype, kv_dtype, [&](auto t) { fn = decltype(t)::kernel(p); })) return 0;
  return groups_per_cu(fn, p.heads_per_wg * 64);
}

}  // namespace pa
