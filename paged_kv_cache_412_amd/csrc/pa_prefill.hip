// pa_prefill.hip -- paged prefill attention on the matrix cores (gfx950):
// several new tokens per sequence, each attending causally to its
// sequence's cached context and to the new tokens up to itself, with every
// key and value read through the block table from the same paged pools the
// decode step reads.
//
// P1 = Ultralytics glossary page "PagedAttention".  The cache holds earlier
// tokens' K/V so later tokens can use them ("Çözdüğü Bellek Sorunu"); the
// attention kernel gathers them block by block through the table ("Sayfalama
// Nasıl Çalışır"); current engines run FlashAttention-style kernels over the
// paged blocks, so the score matrix never reaches device memory ("İlgili
// Teknikler"); grouped-query attention shares a KV head among G query heads
// (same section).
//
// Work split.  A work-group of four waves owns up to 128 rows of (new token,
// query head) pairs of one KV head: floor(128 / G) consecutive new tokens of
// one sequence with all G heads of the group (G from 1 to 16), so every K/V
// tile it loads serves all of them.  Wave w owns rows [32w, 32w + 32) as
// two 16-column MFMA tiles.  The keys run in tiles of 64 (four 16-token
// blocks or two 32-token ones): the work-group copies each tile's K and V
// rows from the pool into LDS (double buffered, the next tile's loads in
// flight during the current tile's matrix work), and every wave reads its
// MFMA operands from there.
//
// Contractions (lane l, lo = l % 16, grp = l / 16; layouts in pa_mfma.h):
//   S^T = K Q^T, one 16x16x32 MFMA per 32 head-dim values: A = 16 key rows
//     (lane: key lo, head-dim run grp*D/4 + [0, D/4)), B = Q^T (lane: query
//     row lo, the same run).  Lane l ends up with the scores of query row lo
//     for keys 4*grp + r of each 16-key half.
//   O^T += V^T P^T, one 16x16x32 MFMA per 16 head-dim rows: B = P^T straight
//     from the score registers (slots e < 4: keys 4*grp + e of the first
//     half, e >= 4: the same of the second half); A = V^T, MFMA number mm
//     covering head dims 16*mm + [0, 16).  Lane l needs head dim 16*mm + lo
//     of its eight keys: two transposing LDS reads (ds_read_b64_tr_b16) give
//     it directly.  In such a read each lane of a 16-lane group addresses
//     four consecutive 16-bit values, and lane d receives value d % 4 of the
//     runs addressed by lanes d/4 + 4k, k = 0..3; so lane lo addresses key
//     row 4*grp + lo/4 (+16 for the second half), head dims 16*mm + 4*(lo%4)
//     .. + 3, and receives head dim 16*mm + lo of keys 4*grp .. 4*grp + 3.
//     Lane l then holds output columns 16*mm + 4*grp + r of query row lo.
// Softmax runs in log2 units on the score layout, with no cross-lane
// traffic in the common case (each lane checks its own scores against the
// shared running max).  The weights enter the
// weighted sum rounded to the 16-bit operand type, and the running sum adds
// up exactly those rounded weights (one more MFMA per tile, against a row of
// ones), so the output is a weighted mean of V rows (a dominant key returns
// its value row).  Each query's running
// maximum may lag the true maximum by at most 8 (a factor 256): the
// accumulators are rescaled only when a tile raises some maximum further
// than that, which after the first tiles is rare.  The result does not
// depend on the lag (sum 2^(s-m) v / sum 2^(s-m) is the same for any m),
// and weights stay below 2^8, far inside the 16-bit operand range.

#include <hip/hip_runtime.h>

#include "pa_decode_common.h"
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr int kWaves = 4;                  // waves per work-group
constexpr int kNT = kPrefillRows / (kWaves * 16);  // 16-column query tiles per wave
constexpr int kKeys = kPrefillKeys;        // keys per LDS tile
constexpr int kMinGroupsPerCU = kNT > 2 ? 1 : 2;
constexpr float kSlack = 8.f;              // allowed lag of the running max (log2 units)

// Maximum of two scores without the quieting copies fmaxf costs in IEEE
// mode (v_maximum3_f32 on gfx950).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// XCD-aware order: the hardware deals consecutive work-groups round-robin to
// the 8 XCDs, each with its own L2.  Map hardware index i to a logical index
// so that each XCD receives one contiguous run of logical work-groups: the
// query tiles of one (sequence, KV head), which read the same K/V, then run
// close together on one XCD and share its L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_logical(int i, int n) {
  constexpr int X = 8;
  const int q = n / X, r = n % X;
  const int x = i % X, k = i / X;
  return x * q + min(x, r) + k;
}

// Inverse of xcd_logical: contiguous index c -> the round-robin index whose
// logical image is c.  Applied to the (sequence, KV head) index, it deals
// those pairs to the XCDs in turn, so every XCD's run mixes all sequences:
// runs of whole sequences left the XCDs with unequal work when context
// lengths differ (the kernel then waits for the slowest XCD).
__device__ __forceinline__ int xcd_round_robin(int c, int n) {
  constexpr int X = 8;
  const int q = n / X, r = n % X;
  int x, k;
  if (c < r * (q + 1)) {
    x = c / (q + 1);
    k = c % (q + 1);
  } else {
    x = r + (c - r * (q + 1)) / q;
    k = (c - r * (q + 1)) % q;
  }
  return k * X + x;
}

// MHA: the instance for one query head per KV head (G = 1) with 16-bit K/V;
// it differs in how the transposing V reads are issued (read_v_all) and in
// how the weighted sum's products are ordered against the weights.
template <int KV, int Q, int D, int BS, bool MHA>
__global__ __launch_bounds__(kWaves * 64, kMinGroupsPerCU) void prefill_kernel(const PrefillParams p) {
  using M = Mfma<Q>;
  constexpr int KVB = Elem<KV>::bytes;
  constexpr int NT = kNT;                  // 16-column query tiles per wave
  constexpr int RW = 16 * NT;              // rows per wave
  constexpr int KS = kKeys / 16;           // 16-key score tiles per key tile
  constexpr int KP = kKeys / 32;           // 32-key weighted-sum steps per key tile
  constexpr int EPL = D / 16;              // head-dim values per lane and key row (PV)
  constexpr int KK = D / 32;               // score MFMAs per 16-key tile
  const int G = p.Hq / p.Hkv;              // 1..16 query heads per KV head
  const int TOK = kPrefillRows / G;        // new tokens per work-group
  constexpr int CH = D / 8;                // 16-byte chunks per LDS row (16-bit values)
  constexpr int ROWB = D * 2;              // LDS bytes per key row
  constexpr int TILE = kKeys * ROWB;
  constexpr int CPR = D * KVB / 16;        // 16-byte global chunks per key row
  constexpr int WR = kKeys / kWaves;        // rows of a tile each wave stages
  constexpr int WROWS = 64 / CPR;          // rows one wave load covers
  constexpr int PASSES = WR / WROWS;       // staging loads per thread, K and V each
  static_assert(kPrefillRows == kWaves * RW, "rows per work-group");
  static_assert(WR % WROWS == 0 && kKeys % 32 == 0, "tile shape");
  static_assert(EPL % 2 == 0 && (CH == 8 || CH == 16), "head dim");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][TILE];  // [buffer][K, V]

  // LDS placement of 16-byte chunk c of key row r: XOR-swizzled so that the
  // reads of one chunk column of 16 rows (K operands: 16 distinct chunks)
  // and the transposing reads of two adjacent chunks of 8 consecutive rows
  // (V operands, two 16-lane groups at once: the rows' swizzles differ above
  // bit 0, so the pairs land on distinct chunks) touch distinct banks; the
  // staging fills write whole rows.  With 256-byte rows a row spans every
  // bank, so rows r and r + 4 must not share a chunk pair: the first
  // swizzle, 2(r mod 4) + (r div 4) mod 2, gave them the same one, and a
  // third of the LDS's active cycles were bank conflicts.
  auto swz = [](int r) {
    if constexpr (CH == 16) return ((r & 7) << 1) | ((r >> 3) & 1);
    return ((r & 3) << 1) | ((r >> 2) & 1);
  };
  auto lds_off = [&](int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); };

  const int lid = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lo = lid & 15, grp = lid >> 4;

  // ---- which (sequence, KV head, query tile); heavy (late) tiles first
  const int logical = xcd_logical(blockIdx.x, p.total_groups);
  const int qt = p.q_tiles - 1 - logical % p.q_tiles;
  const int nbh = p.total_groups / p.q_tiles;
  const int bh = xcd_round_robin(logical / p.q_tiles, nbh);
  const int kvh = bh % p.Hkv;
  const int b = bh / p.Hkv;

  const int qs = p.q_starts[b];
  const int L = min(max(p.seq_lens[b], 0), p.max_blocks_per_seq * BS);
  int n = min(p.q_starts[b + 1] - qs, p.max_q_len);
  n = min(n, L);
  n = (qs < 0 || qs > p.T) ? 0 : min(n, p.T - qs);  // rows stay inside q and out
  const int t0 = qt * TOK;
  if (t0 >= n) return;  // whole work-group, before any barrier
  const int ntok = min(TOK, n - t0);
  const int ctx = L - n;                   // cached tokens before the new ones
  const int n_keys = ctx + t0 + ntok;      // keys the tile's last token sees
  const int tiles = (n_keys + kKeys - 1) / kKeys;

  // Scores are scaled by c = scale * k_scale * log2(e) inside one fused
  // multiply-add before the exponential.  A negative c is taken as |c| with
  // the queries negated (exact for 16-bit values), so the running max can be
  // taken over unscaled scores; c = 0 is taken as the smallest normal float
  // (every weight still rounds to 1) so that masked scores stay -inf.
  const float c_in = p.k_scales ? p.qk_scale_log2 * p.k_scales[kvh] : p.qk_scale_log2;
  const float vs = p.v_scales ? p.v_scales[kvh] : p.v_scale;
  const uint32_t qflip = c_in < 0.f ? 0x80008000u : 0u;
  const float c = fmaxf(fabsf(c_in), 1.17549435e-38f);

  // ---- this lane's NT query rows (row -> token row / G, head row % G)
  int pos[NT];
  bool valid[NT];
  size_t orow[NT];
  u32x4 qv[NT][KK];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = wave * RW + nt * 16 + lo;
    const int tok = row / G;
    valid[nt] = tok < ntok;
    const int tk = min(tok, ntok - 1);  // rows past the tile repeat its last token
    pos[nt] = ctx + t0 + tk;
    orow[nt] = (static_cast<size_t>(qs + t0 + tk) * p.Hq + static_cast<size_t>(kvh) * G + row % G) * D;
    const uint8_t* qp = static_cast<const uint8_t*>(p.q) + (orow[nt] + grp * (D / 4)) * 2;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qv[nt][kk] = *reinterpret_cast<const u32x4*>(qp + 16 * kk) ^ qflip;
  }
  const int wtok0 = wave * RW / G;
  const bool wave_active = wtok0 < ntok;
  const int pmin = ctx + t0 + wtok0;
  const int pmax = ctx + t0 + min((wave * RW + RW - 1) / G, ntok - 1);

  // ---- staging: wave wv stages the tile's rows [wv*WR, wv*WR + WR), WROWS
  // rows per load (lane -> row within the load, 16-byte chunk).  The rows
  // of one load lie in one block, and with blocks of WR rows or more all of
  // a wave's rows do, so the wave builds its buffer resources over that
  // block once per tile.  Absent blocks get a resource of 0 bytes and rows
  // past the last key an offset past the end, and both read as zeros.  Every
  // path thus issues the same loads, and the compiler's wait counts stay
  // exact (loads retire in order).
  //
  // 16-bit K/V go from the pool straight into LDS (buffer loads with the LDS
  // bit): one such load fills 1 KiB from a wave-uniform base, lane i at byte
  // 16 i, which is WROWS whole rows, so the lane at physical chunk pc of row
  // r fetches the logical chunk pc ^ swizzle(r) that belongs there.  The
  // next tile's fills run during the current tile's matrix work, into the
  // buffer no wave reads in this iteration; each wave waits for its own
  // fills before the barrier that ends the iteration.  8-bit K/V are loaded
  // into registers and widened to the 16-bit operand type on their way to LDS.
  constexpr int TB = kKeys / BS > 0 ? kKeys / BS : 1;  // blocks per key tile
  // blocks one wave load spans: 1, or 2 for 8-bit D = 64 rows (16 per load)
  // in 8-token blocks, loaded once per block with the other block's lanes
  // out of range (zeros) and the two results merged
  constexpr int LB = WROWS > BS ? WROWS / BS : 1;
  static_assert(LB == 1 ? BS % WROWS == 0 : (KVB == 1 && WROWS == LB * BS), "a wave load's rows");
  constexpr bool ONE_BLOCK = BS >= WR;                  // all of a wave's rows in one block
  static_assert(KVB != 2 || WROWS * ROWB == 1024, "one LDS fill per wave and pass");
  const int64_t row_stride = static_cast<int64_t>(p.Hkv) * D * KVB;
  const uint32_t blk_bytes = static_cast<uint32_t>(row_stride * BS);
  const int32_t* table = p.block_tables + static_cast<size_t>(b) * p.max_blocks_per_seq;
  const int nblk = (n_keys + BS - 1) / BS;  // table entries this work-group reads
  const __amdgpu_buffer_rsrc_t trs = block_rsrc(table, static_cast<uint32_t>(nblk) * 4u);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int srow = lid / CPR, schunk = lid % CPR;  // row within a wave load, 16-byte chunk
  u32x4 kst[KVB == 2 ? 1 : PASSES], vst[KVB == 2 ? 1 : PASSES];  // 8-bit codes in flight
  // ids of the blocks of a tile, lane t < TB holding its t-th block
  auto load_ids = [&](int j) {
    return static_cast<int>(
        __builtin_amdgcn_raw_buffer_load_b32(trs, (j * TB + (lid % TB)) * 4, 0, 0));
  };
  // each lane's byte offset inside a block for its row of every load (the
  // same in every tile: kKeys is a multiple of the block size), its head's
  // column and its 16-byte chunk included (for 16-bit K/V the logical chunk
  // the swizzle puts at the lane's LDS position)
  static_assert(kKeys % BS == 0, "tiles start on block boundaries");
  int lane_off[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int r = wv * WR + ps * WROWS + srow;
    int c = schunk;
    if constexpr (KVB == 2) c ^= swz(r);
    lane_off[ps] = static_cast<int>((r % BS) * row_stride) + kvh * D * KVB + (c << 4);
  }
  const int lane_row = wv * WR + srow;  // this lane's row of the tile in its first load

  // issue tile j's loads (into LDS buffer buf for 16-bit K/V).  Wave wv
  // stages rows [wv*WR, wv*WR + WR) of the tile, WROWS per load.
  auto fetch = [&](int j, int ids, int buf) {
    __amdgpu_buffer_rsrc_t kr, vr;
    auto block_of = [&](int row0) {  // resources over the block holding tile row row0
      const int blk = __builtin_amdgcn_readlane(ids, (row0 / BS) % TB);
      const bool ok = blk >= 0 && blk < p.num_blocks;
      const char* kb = static_cast<const char*>(p.k_cache) + static_cast<int64_t>(ok ? blk : 0) * blk_bytes;
      const char* vb = static_cast<const char*>(p.v_cache) + static_cast<int64_t>(ok ? blk : 0) * blk_bytes;
      kr = block_rsrc(kb, ok ? blk_bytes : 0u);
      vr = block_rsrc(vb, ok ? blk_bytes : 0u);
    };
    if constexpr (ONE_BLOCK) block_of(wv * WR);
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int row0 = wv * WR + ps * WROWS;          // first row of this wave load
      if constexpr (!ONE_BLOCK && LB == 1) block_of(row0);
      // rows past the last key read zeros (an offset past the end)
      const int voff = lane_row + ps * WROWS < n_keys - j * kKeys ? lane_off[ps] : 0x7fffff00;
      if constexpr (LB > 1) {
        u32x4 ka = {0u, 0u, 0u, 0u}, va = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < LB; ++h) {
          block_of(row0 + h * BS);
          const int o = srow / BS == h ? voff : 0x7fffff00;
          ka |= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, o, 0, 0));
          va |= __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, o, 0, 0));
        }
        kst[ps] = ka;
        vst[ps] = va;
      } else if constexpr (KVB == 2) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            kr, (__attribute__((address_space(3))) void*)(lds[buf][0] + row0 * ROWB), 16, voff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (__attribute__((address_space(3))) void*)(lds[buf][1] + row0 * ROWB), 16, voff, 0, 0, 0);
      } else {
        kst[ps] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, voff, 0, 0));
        vst[ps] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, voff, 0, 0));
      }
    }
  };
  // complete the fetched tile in LDS buffer buf (before the barrier)
  auto stage = [&](int buf) {
    if constexpr (KVB == 2) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's LDS fills have landed
    } else {
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int r = wv * WR + ps * WROWS + srow;
        uint8_t* kd = lds[buf][0];
        uint8_t* vd = lds[buf][1];
        // 16 8-bit codes -> 16 operand values (exact), two chunks
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          widen_fp8<Q, KV>(kst[ps][i], w[2 * i], w[2 * i + 1]);
          widen_fp8<Q, KV>(vst[ps][i], w[8 + 2 * i], w[8 + 2 * i + 1]);
        }
        *reinterpret_cast<u32x4*>(kd + lds_off(r, 2 * schunk)) = u32x4{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(kd + lds_off(r, 2 * schunk + 1)) = u32x4{w[4], w[5], w[6], w[7]};
        *reinterpret_cast<u32x4*>(vd + lds_off(r, 2 * schunk)) = u32x4{w[8], w[9], w[10], w[11]};
        *reinterpret_cast<u32x4*>(vd + lds_off(r, 2 * schunk + 1)) = u32x4{w[12], w[13], w[14], w[15]};
      }
    }
  };

  const float ninf = -__builtin_huge_valf();
  float m[NT];   // running max of query row lo (log2 units)
  f32x4 l[NT];   // running sum of query row lo (four equal copies)
  f32x4 o[NT][EPL];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = kMaxInit;
    l[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mm = 0; mm < EPL; ++mm) o[nt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // A operand of all ones: ones x P^T sums the rounded weights of each query
  // over 32 keys on the matrix cores (every row of the result)
  const u32x4 ones = {M::kOnePair, M::kOnePair, M::kOnePair, M::kOnePair};
  // byte addresses of the lanes l ^ 16 and l ^ 32 (the other groups' lanes of
  // the same query column) for ds_bpermute
  const int xor16 = (lid ^ 16) << 2, xor32 = (lid ^ 32) << 2;

  // value rows of 32-key step kp: keys 32*kp + 4*grp + e (e < 4) and
  // 32*kp + 16 + 4*grp + e - 4, this lane's D/16 head-dim values of each
  // LDS operand addresses split into a per-lane part and a constant: K row
  // 16*ks + lo and V row 16*h + 4*grp + e (h, e < 4 fixed per read) take
  // the swizzle of rows lo and 4*grp + e, so their offsets are koff[kk] +
  // 16*ks*ROWB and voff4[e] + 16*h*ROWB.
  int koff[KK], vtr[EPL];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = lds_off(lo, grp * KK + kk);
  // transposing reads of V: within each 16-lane group, lane lo addresses
  // row 4*grp + lo/4, head dims 16*mm + 4*(lo%4) .. + 3, and then receives
  // head dim 16*mm + lo of rows 4*grp .. 4*grp + 3
#pragma unroll
  for (int mm = 0; mm < EPL; ++mm)
    vtr[mm] = lds_off(4 * grp + (lo >> 2), 2 * mm + ((lo >> 1) & 1)) + ((lo & 1) << 3);
  // The transposing reads of the value rows.  Through the builtin the
  // compiler cannot tell which LDS buffer they read, and with 16-bit K/V
  // (filled straight into LDS) it first waits for the next tile's fills.
  // Without grouping every work-group reads K/V of its own, the fills come
  // from memory, and that wait costs more than the reads' latency: the MHA
  // instance issues the whole tile's reads as one asm block that waits for
  // them itself.  With grouping the fills are mostly L2 hits, and the builtin
  // reads of each 32-key step, issued a step ahead of its products, keep
  // their latency hidden.
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  static_assert(!MHA || (KVB == 2 && (EPL == 8 || EPL == 4)), "MHA instance: 16-bit K/V");
  // MHA: both 32-key steps' value operands in one block, issued right after
  // the score products (the wait at its end then overlaps their execution
  // instead of stalling between the two steps' products)
  auto read_v_all = [&](const uint8_t* Vt, u32x4 (&va)[KP][EPL]) {
    static_assert(KP == 2, "two 32-key steps per tile");
    const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const uint8_t*)Vt));
    // y[4*mm + q]: head dims 16*mm.. of key rows 16*q + 4*grp .. + 3
    u32x2 y[4 * EPL];
    if constexpr (EPL == 8) {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %32\n ds_read_b64_tr_b16 %1, %32 offset:%40\n"
          "ds_read_b64_tr_b16 %2, %32 offset:%41\n ds_read_b64_tr_b16 %3, %32 offset:%42\n"
          "ds_read_b64_tr_b16 %4, %33\n ds_read_b64_tr_b16 %5, %33 offset:%40\n"
          "ds_read_b64_tr_b16 %6, %33 offset:%41\n ds_read_b64_tr_b16 %7, %33 offset:%42\n"
          "ds_read_b64_tr_b16 %8, %34\n ds_read_b64_tr_b16 %9, %34 offset:%40\n"
          "ds_read_b64_tr_b16 %10, %34 offset:%41\n ds_read_b64_tr_b16 %11, %34 offset:%42\n"
          "ds_read_b64_tr_b16 %12, %35\n ds_read_b64_tr_b16 %13, %35 offset:%40\n"
          "ds_read_b64_tr_b16 %14, %35 offset:%41\n ds_read_b64_tr_b16 %15, %35 offset:%42\n"
          "ds_read_b64_tr_b16 %16, %36\n ds_read_b64_tr_b16 %17, %36 offset:%40\n"
          "ds_read_b64_tr_b16 %18, %36 offset:%41\n ds_read_b64_tr_b16 %19, %36 offset:%42\n"
          "ds_read_b64_tr_b16 %20, %37\n ds_read_b64_tr_b16 %21, %37 offset:%40\n"
          "ds_read_b64_tr_b16 %22, %37 offset:%41\n ds_read_b64_tr_b16 %23, %37 offset:%42\n"
          "ds_read_b64_tr_b16 %24, %38\n ds_read_b64_tr_b16 %25, %38 offset:%40\n"
          "ds_read_b64_tr_b16 %26, %38 offset:%41\n ds_read_b64_tr_b16 %27, %38 offset:%42\n"
          "ds_read_b64_tr_b16 %28, %39\n ds_read_b64_tr_b16 %29, %39 offset:%40\n"
          "ds_read_b64_tr_b16 %30, %39 offset:%41\n ds_read_b64_tr_b16 %31, %39 offset:%42\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]),
            "=&v"(y[6]), "=&v"(y[7]), "=&v"(y[8]), "=&v"(y[9]), "=&v"(y[10]), "=&v"(y[11]),
            "=&v"(y[12]), "=&v"(y[13]), "=&v"(y[14]), "=&v"(y[15]), "=&v"(y[16]), "=&v"(y[17]),
            "=&v"(y[18]), "=&v"(y[19]), "=&v"(y[20]), "=&v"(y[21]), "=&v"(y[22]), "=&v"(y[23]),
            "=&v"(y[24]), "=&v"(y[25]), "=&v"(y[26]), "=&v"(y[27]), "=&v"(y[28]), "=&v"(y[29]),
            "=&v"(y[30]), "=&v"(y[31])
          : "v"(base + vtr[0]), "v"(base + vtr[1]), "v"(base + vtr[2]), "v"(base + vtr[3]),
            "v"(base + vtr[4]), "v"(base + vtr[5]), "v"(base + vtr[6]), "v"(base + vtr[7]),
            "n"(16 * ROWB), "n"(32 * ROWB), "n"(48 * ROWB)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %16 offset:%20\n"
          "ds_read_b64_tr_b16 %2, %16 offset:%21\n ds_read_b64_tr_b16 %3, %16 offset:%22\n"
          "ds_read_b64_tr_b16 %4, %17\n ds_read_b64_tr_b16 %5, %17 offset:%20\n"
          "ds_read_b64_tr_b16 %6, %17 offset:%21\n ds_read_b64_tr_b16 %7, %17 offset:%22\n"
          "ds_read_b64_tr_b16 %8, %18\n ds_read_b64_tr_b16 %9, %18 offset:%20\n"
          "ds_read_b64_tr_b16 %10, %18 offset:%21\n ds_read_b64_tr_b16 %11, %18 offset:%22\n"
          "ds_read_b64_tr_b16 %12, %19\n ds_read_b64_tr_b16 %13, %19 offset:%20\n"
          "ds_read_b64_tr_b16 %14, %19 offset:%21\n ds_read_b64_tr_b16 %15, %19 offset:%22\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]),
            "=&v"(y[6]), "=&v"(y[7]), "=&v"(y[8]), "=&v"(y[9]), "=&v"(y[10]), "=&v"(y[11]),
            "=&v"(y[12]), "=&v"(y[13]), "=&v"(y[14]), "=&v"(y[15])
          : "v"(base + vtr[0]), "v"(base + vtr[1]), "v"(base + vtr[2]), "v"(base + vtr[3]),
            "n"(16 * ROWB), "n"(32 * ROWB), "n"(48 * ROWB)
          : "memory");
    }
#pragma unroll
    for (int mm = 0; mm < EPL; ++mm) {
      va[0][mm] = u32x4{y[4 * mm][0], y[4 * mm][1], y[4 * mm + 1][0], y[4 * mm + 1][1]};
      va[1][mm] = u32x4{y[4 * mm + 2][0], y[4 * mm + 2][1], y[4 * mm + 3][0], y[4 * mm + 3][1]};
    }
  };
  // other instances: one 32-key step's value operands through the builtin
  auto read_v = [&](const uint8_t* Vt, int kp, u32x4 (&va)[EPL]) {
#pragma unroll
    for (int mm = 0; mm < EPL; ++mm) {
      const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + vtr[mm] + 32 * kp * ROWB));
      const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vt + vtr[mm] + (32 * kp + 16) * ROWB));
      const u32x2 y0 = __builtin_bit_cast(u32x2, x0), y1 = __builtin_bit_cast(u32x2, x1);
      va[mm] = u32x4{y0[0], y0[1], y1[0], y1[1]};
    }
  };

  int ids_next = load_ids(1);  // tile 1's blocks (consumed one iteration later)
  fetch(0, load_ids(0), 0);
  stage(0);
  __syncthreads();

  for (int j = 0; j < tiles; ++j) {
    const int k0 = j * kKeys;
    // tile j+2's block ids, then tile j+1's rows: the same loads on every
    // iteration (past the last tile they read zeros into a buffer no one reads)
    const int ids = ids_next;
    ids_next = load_ids(j + 2);
    fetch(j + 1, ids, (j + 1) & 1);
    if (wave_active && k0 <= pmax) {
      const uint8_t* Kt = lds[j & 1][0];
      const uint8_t* Vt = lds[j & 1][1];
      // scores
      f32x4 s[KS][NT];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[ks][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(Kt + koff[kk] + 16 * ks * ROWB);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) s[ks][nt] = M::mma32(a, qv[nt][kk], s[ks][nt]);
        }
      }
      // the first value rows, read now so that their LDS latency hides
      // behind the softmax
      u32x4 vop[KP][EPL];
      if constexpr (MHA) read_v_all(Vt, vop);
      else read_v(Vt, 0, vop[0]);
      // mask keys after each query's position (only near the diagonal)
      if (k0 + kKeys - 1 > pmin) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (k0 + 16 * ks + 4 * grp + r > pos[nt]) s[ks][nt][r] = ninf;
      }
      // This lane's max over its own scores of each query (unscaled; IEEE
      // maximum, v_maximum3_f32: the scores hold no signalling NaNs).  Only
      // when some lane exceeds the running max by more than the allowed lag
      // does the wave reduce across its lanes and rescale: the common path
      // needs no cross-lane traffic, and every weight stays below 2^kSlack.
      float lmx[NT];
      bool up = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float x = s[0][nt][0];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int r = (ks == 0 ? 1 : 0); r < 4; ++r) x = vmax(x, s[ks][nt][r]);
        lmx[nt] = x;
        up = up || x * c > m[nt] + kSlack;
      }
      if (__ballot(up)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // the query's max over all four lane groups, in log2 units (c > 0)
          float x = lmx[nt];
          x = vmax(x, u2f(__builtin_amdgcn_ds_bpermute(xor16, f2u(x))));
          x = vmax(x, u2f(__builtin_amdgcn_ds_bpermute(xor32, f2u(x))));
          const float mn = fmaxf(m[nt], x * c);
          const float alpha = fast_exp2(m[nt] - mn);
          m[nt] = mn;
          l[nt] *= alpha;  // all four copies
#pragma unroll
          for (int mm = 0; mm < EPL; ++mm) o[nt][mm] *= alpha;
        }
      }
      // weighted sum, 32 keys at a time.  Weights of 32-key step kp, packed
      // as the B operand: slots e < 4 are keys 4*grp + e of the first 16-key
      // tile, e >= 4 the same of the second
      u32x4 pb[KP][NT];
      auto weights = [&](int kp) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          float w[2][4];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              w[h][r] = fast_exp2(__builtin_fmaf(s[2 * kp + h][nt][r], c, -m[nt]));
          pb[kp][nt] = u32x4{M::pack2(w[0][0], w[0][1]), M::pack2(w[0][2], w[0][3]),
                             M::pack2(w[1][0], w[1][1]), M::pack2(w[1][2], w[1][3])};
        }
      };
      // the running sum takes the weights as rounded for the matrix cores, so
      // the result is an exact weighted mean of V rows under those weights
      auto products = [&](int kp) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) l[nt] = M::mma32(ones, pb[kp][nt], l[nt]);
#pragma unroll
        for (int mm = 0; mm < EPL; ++mm) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt][mm] = M::mma32(vop[kp][mm], pb[kp][nt], o[nt][mm]);
        }
      };
      if constexpr (MHA) {
        // The second step's weights are computed while the first step's
        // products run: one product, then two vector ops, in turn, so that
        // the matrix cores and the vector ALUs work at the same time within
        // the wave (left to itself the compiler computes every weight first).
        constexpr int MPK = NT * (EPL + 1);  // products per step
        weights(0);
        __builtin_amdgcn_sched_barrier(0);
        products(0);
        weights(1);
#pragma unroll
        for (int i = 0; i < MPK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one matrix product
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // two vector ops
        }
        __builtin_amdgcn_sched_barrier(0);
        products(1);
      } else {
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
          weights(kp);
          // the next step's value operands go out before this step's products
          if (kp + 1 < KP) read_v(Vt, kp + 1, vop[kp + 1]);
          products(kp);
        }
      }
    }
    stage((j + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l[nt][0];
    if (!valid[nt]) continue;
    // lt > 0: the running max never exceeds the largest score seen, whose
    // weight 2^(s - m) is therefore about 1 or more
    const float inv = vs / lt;
#pragma unroll
    for (int mm = 0; mm < EPL; ++mm) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = o[nt][mm][r] * inv;
      store_out_n<4>(p.out, orow[nt] + 16 * mm + 4 * grp, v, p.out_dtype);
    }
  }
}

// ---------------------------------------------------------------- dispatch

template <int KV_, int Q_, int D_, int BS_>
struct Tag {
  static hipError_t launch(const PrefillParams& p, hipStream_t s) {
    if constexpr (Elem<KV_>::bytes == 2) {
      if (p.Hq == p.Hkv) {
        hipLaunchKernelGGL((prefill_kernel<KV_, Q_, D_, BS_, true>), dim3(p.total_groups),
                           dim3(kWaves * 64), 0, s, p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((prefill_kernel<KV_, Q_, D_, BS_, false>), dim3(p.total_groups), dim3(kWaves * 64), 0,
                       s, p);
    return hipGetLastError();
  }
};

template <int KV, int Q, int D, typename F>
bool by_block(int32_t bs, int32_t G, F&& f) {
  if (G < 1 || G > 16) return false;
  switch (bs) {
    case 8: f(Tag<KV, Q, D, 8>{}); return true;
    case 16: f(Tag<KV, Q, D, 16>{}); return true;
    case 32: f(Tag<KV, Q, D, 32>{}); return true;
    case 64: f(Tag<KV, Q, D, 64>{}); return true;
    default: return false;
  }
}

template <int KV, int Q, typename F>
bool by_dim(int32_t D, int32_t bs, int32_t G, F&& f) {
  switch (D) {
    case 64: return by_block<KV, Q, 64>(bs, G, f);
    case 128: return by_block<KV, Q, 128>(bs, G, f);
    default: return false;
  }
}

template <typename F>
bool dispatch(pa_dtype q, pa_dtype kv, int32_t D, int32_t bs, int32_t G, F&& f) {
  if (kv == PA_F16 && q == PA_F16) return by_dim<PA_F16, PA_F16>(D, bs, G, f);
  if (kv == PA_BF16 && q == PA_BF16) return by_dim<PA_BF16, PA_BF16>(D, bs, G, f);
  if (kv == PA_FP8_E4M3 && q == PA_BF16) return by_dim<PA_FP8_E4M3, PA_BF16>(D, bs, G, f);
  if (kv == PA_FP8_E4M3 && q == PA_F16) return by_dim<PA_FP8_E4M3, PA_F16>(D, bs, G, f);
  if (kv == PA_FP8_E5M2 && q == PA_BF16) return by_dim<PA_FP8_E5M2, PA_BF16>(D, bs, G, f);
  if (kv == PA_FP8_E5M2 && q == PA_F16) return by_dim<PA_FP8_E5M2, PA_F16>(D, bs, G, f);
  return false;
}

// ---------------------------------------------------------------- slot mapping

// Slot of every new row: row r of sequence b (q_starts[b] <= r < q_starts[b+1])
// is new token i = r - q_starts[b] at position seq_lens[b] - n_b + i.
__global__ __launch_bounds__(256) void prefill_slot_mapping_kernel(
    const int32_t* __restrict__ tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ q_starts, int32_t B, int32_t T, int32_t max_blocks, int32_t bs,
    int32_t* __restrict__ slots) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= T) return;
  // last b with q_starts[b] <= r (binary search over the B + 1 starts)
  int lo_b = 0, hi_b = B;  // invariant: answer in [lo_b, hi_b)
  while (hi_b - lo_b > 1) {
    const int mid = (lo_b + hi_b) >> 1;
    if (q_starts[mid] <= r) lo_b = mid; else hi_b = mid;
  }
  const int b = lo_b;
  int slot = -1;
  const int s0 = q_starts[b], s1 = q_starts[b + 1];
  if (s0 <= r && r < s1) {
    const int64_t pos = static_cast<int64_t>(seq_lens[b]) - (s1 - s0) + (r - s0);
    if (pos >= 0 && pos / bs < max_blocks) {
      const int blk = tables[static_cast<size_t>(b) * max_blocks + pos / bs];
      const int64_t s = static_cast<int64_t>(blk) * bs + pos % bs;
      if (blk >= 0 && s <= INT32_MAX) slot = static_cast<int>(s);
    }
  }
  slots[r] = slot;
}

}  // namespace

bool prefill_serves(pa_dtype q_dtype, pa_dtype kv_dtype, int32_t D, int32_t block_size,
                    int32_t group) {
  return dispatch(q_dtype, kv_dtype, D, block_size, group, [](auto) {});
}

hipError_t launch_prefill(const PrefillParams& p, pa_dtype q_dtype, pa_dtype kv_dtype,
                          hipStream_t stream, bool* supported) {
  hipError_t e = hipSuccess;
  *supported = dispatch(q_dtype, kv_dtype, p.D, p.block_size, p.Hq / p.Hkv,
                        [&](auto t) { e = decltype(t)::launch(p, stream); });
  return e;
}

hipError_t launch_prefill_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                       const int32_t* q_starts, int32_t B, int32_t T,
                                       int32_t max_blocks, int32_t block_size, int32_t* slots,
                                       hipStream_t stream) {
  const int threads = 256;
  hipLaunchKernelGGL(prefill_slot_mapping_kernel, dim3((T + threads - 1) / threads), dim3(threads),
                     0, stream, block_tables, seq_lens, q_starts, B, T, max_blocks, block_size,
                     slots);
  return hipGetLastError();
}

}  // namespace pa
