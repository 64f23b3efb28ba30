/*
 * pa.h -- C ABI of libpa, the paged KV-cache attention path for AMD Instinct
 * MI355X (gfx950): decode, prefill and the cache-side kernels.
 *
 * Sources (web pages on PagedAttention, cited by title and section):
 *   P1  Ultralytics glossary page "PagedAttention" (Turkish): introduction;
 *       "Sayfalama Nasıl Çalışır" (how paging works, with a PyTorch code
 *       sketch of a block pool, a free list and a block table);
 *       "Diziler Arasında Blokları Paylaşma" (sharing blocks between
 *       sequences); "İlgili Teknikler" (related techniques: FlashAttention,
 *       grouped-query attention, FP8 cache quantisation).
 *   P3  gyaansetu.com page on KV memory and PagedAttention (Persian),
 *       article A "how PagedAttention solves it" (on-demand pages, shared
 *       prefix with copy-on-write) and article B "the solution" (page table).
 *
 * Data layout (all device memory, row-major, owned by the caller):
 *   K pool, V pool   [num_blocks][block_size][Hkv][D] of the KV dtype.  A
 *                    physical block holds block_size consecutive tokens of
 *                    one sequence for every KV head (P1 "Sayfalama Nasıl
 *                    Çalışır": fixed-size blocks, 16 tokens by default).
 *   block_tables     int32 [B][max_blocks_per_seq]: entry j of row b is the
 *                    physical block holding tokens [j*bs, (j+1)*bs) of
 *                    sequence b (P1 introduction: one block table per
 *                    request, like an OS page table; P3 article B).  Only the
 *                    first ceil(seq_lens[b] / bs) entries are read.
 *   seq_lens         int32 [B]: tokens in each sequence's context.
 *   flat slot        block * block_size + offset, the index of one token row
 *                    of one block (P1 code sketch, write loop).
 *
 * Conventions:
 *   - Every call is a host function that validates its arguments, then
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the default
 *     stream) and returns without synchronising.  Validation reads only the
 *     arguments, except pa_swap_blocks, which also asks the HIP runtime
 *     which kind of memory each pool is.  The library never
 *     allocates, frees or synchronises device memory; it keeps no state
 *     except per-device caches (the compute-unit count, each kernel's
 *     occupancy, and pa_decode_no_alloc's scratch address).
 *   - The decode step's calls (pa_copy_blocks, pa_append_kv or the slot
 *     mapping and cache write, pa_decode_partition, pa_decode_reduce) and
 *     the prefill step's can be captured into a HIP graph on `stream` and
 *     replayed: none records a memset or waits on the host, and the kernels
 *     reset the workspace's arrival counters themselves.  Replays give the
 *     eager call's results bit for bit.
 *   - Host-side validation failures return a pa_status other than PA_OK,
 *     enqueue nothing and print nothing.  PA_ERR_LAUNCH reports a failed
 *     kernel launch (hipGetLastError).  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Device-side index checks: block ids outside [0, num_blocks), slots
 *     outside [0, num_blocks*block_size) and block-copy pairs outside the
 *     pool are skipped (nothing read or written for them); seq_lens are
 *     clamped to [0, max_blocks_per_seq*block_size].  Results for a sequence
 *     whose table holds such ids are then meaningless, but no access leaves
 *     the caller's buffers.
 *   - Calls on one stream are ordered; the library is thread-safe.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 3

/* Element types.  The 8-bit cache formats (P1 "İlgili Teknikler": an 8-bit
 * KV cache, about half the memory of 16-bit) store a code c meaning
 * value(c) * scale with one fp32 scale per pool:
 *   PA_FP8_E4M3  OCP e4m3 "fn": 1 sign, 4 exponent (bias 7), 3 mantissa
 *                bits, S.1111.111 = NaN, max +-448, no infinities;
 *   PA_FP8_E5M2  OCP e5m2: 1 sign, 5 exponent (bias 15), 2 mantissa bits,
 *                IEEE-style infinities and NaNs, max +-57344. */
typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3,
  PA_FP8_E5M2 = 4
} pa_dtype;

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                         */
  PA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent              */
  PA_ERR_UNSUPPORTED = 3, /* dtype / head dim / block size / group not built     */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required          */
  PA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch            */
  PA_ERR_OUT_OF_BLOCKS = 6 /* block manager: no free or evictable block left;     */
                           /* the operation changed nothing                      */
} pa_status;

/* Arguments of one decode step over a batch (one layer). */
typedef struct pa_decode_args {
  void* out;                   /* [B][Hq][D] out_dtype, written                       */
  const void* q;               /* [B][Hq][D] q_dtype                                  */
  const void* k_cache;         /* [num_blocks][block_size][Hkv][D] kv_dtype           */
  const void* v_cache;         /* same shape and dtype as k_cache                     */
  const int32_t* block_tables; /* [B][max_blocks_per_seq]                             */
  const int32_t* seq_lens;     /* [B]                                                 */
  int32_t B, Hq, Hkv, D;
  int32_t block_size, num_blocks, max_blocks_per_seq;
  float scale;                 /* softmax scale, e.g. 1/sqrt(D)                       */
  float k_scale, v_scale;      /* fp8 dequantisation scales; must be 1 otherwise      */
  pa_dtype q_dtype, kv_dtype, out_dtype;
  int32_t partition_size;      /* > 0: fixed split-K partitions of this many tokens,  */
                               /* a multiple of block_size; 0: balanced schedule      */
  void* workspace;             /* device scratch (layout below), 16-byte aligned      */
  size_t workspace_bytes;      /* >= pa_decode_workspace_size(args)                   */
  const float* k_scales;       /* NULL, or per-KV-head scales [Hkv] (device memory)   */
  const float* v_scales;       /* for an 8-bit cache: replace k_scale / v_scale, head */
                               /* g's codes meaning value * k_scales[g]; both or      */
                               /* neither; positive and finite (not checked)          */
  int32_t combine;             /* who combines split sequences (PA_COMBINE_*)         */
} pa_decode_args;

/* Who combines the pieces of a sequence that several work-groups share
 * (pa_decode_args.combine; Schedules below). */
enum {
  PA_COMBINE_AUTO = 0,      /* the library picks: IN_LAUNCH under the balanced   */
                            /* schedule when its work-groups per KV-head group   */
                            /* do not outnumber the sequences, else REDUCE       */
  PA_COMBINE_IN_LAUNCH = 1, /* the partition launch itself: no reduce kernel     */
  PA_COMBINE_REDUCE = 2     /* a reduce kernel after the partition launch        */
};

/* Supported decode combinations (others return PA_ERR_UNSUPPORTED):
 *   D in {64, 128}; block_size in {8, 16, 32, 64};
 *   (q, kv) in {(F32,F32), (F16,F16), (BF16,BF16), and BF16 or F16 over
 *   FP8_E4M3 or FP8_E5M2}; out_dtype = q_dtype or PA_F32;
 *   G = Hq/Hkv from 1 to 16, except fp32 caches: G in {1, 2, 4, 8}.
 *   64-token blocks are read as two 32-token halves: the balanced schedule
 *   then splits work at half-block granularity (block ids times 2 must fit
 *   int32, as must B * max_blocks_per_seq * 2). */

/* Schedules.
 *   partition_size > 0 (fixed): one work-group per (KV heads, sequence,
 *     partition of partition_size tokens).  P = ceil(max_blocks_per_seq *
 *     block_size / partition_size) may not exceed 65535.
 *   partition_size == 0 (balanced, the default): the sequences' block counts
 *     are summed on the device (by every work-group itself up to 1024
 *     sequences, else by a plan kernel first), then one round of
 *     work-groups splits the concatenation of all sequences' blocks into
 *     equal ranges, so the work per work-group does not depend on the
 *     length mix.
 *   Either way a sequence longer than one piece leaves fp32 partials (m, l
 *   and the unnormalised V-weighted sum of each piece) in the workspace, to
 *   be combined as M = max_p m_p,
 *   out = sum_p e^(m_p-M) acc_p / sum_p e^(m_p-M) l_p:
 *   - PA_COMBINE_IN_LAUNCH: the work-group that finishes the sequence's last
 *     piece combines them in the same launch.  It counts the pieces'
 *     arrivals on an int32 counter per (KV head, sequence) in the workspace;
 *     no work-group ever waits for another.  The pieces' rows then pass
 *     through device-coherent memory, and the combine runs at the end of the
 *     launch, so this pays when few sequences are split (no reduce launch).
 *   - PA_COMBINE_REDUCE: pa_decode_reduce's kernel combines them (and writes
 *     zeros for empty sequences) in a launch of its own, which pays when
 *     many sequences are split into many pieces.
 *   pa_decode_partition runs the first launch, pa_decode_reduce the reduce
 *   kernel when there is one (it enqueues nothing otherwise); pa_decode runs
 *   both.
 *
 * Workspace layout (device memory, 16-byte aligned):
 *   1. counters: int32 [Hkv][B], padded to a multiple of 256 bytes
 *      (pa_decode_workspace_zero_bytes), used by PA_COMBINE_IN_LAUNCH.
 *      They must be zero when a call starts, and every call that returns
 *      PA_OK leaves them zero once its kernels have run.  So zero the workspace once after allocating it;
 *      before reusing it for arguments with another B or Hkv (whose
 *      counters would cover other bytes), zero the new counter bytes again.
 *   2. balanced only: int32 block prefix sums [B+1], padded to a multiple of
 *      256 bytes;
 *   3. fp32 partial rows: acc [rows][D], then m [rows], then l [rows], with
 *      rows = B*Hq*P (fixed; partition-major) or HG * W * 2 * NW * G
 *      (balanced).  NW = KV heads per work-group (the smallest power of two
 *      >= min(Hkv, 8) when the matrix-core kernel serves the call: G from 3
 *      to 16 with a 16-bit query over a 16-bit or 8-bit cache; else the
 *      smallest power of two >= min(Hkv, 4)), HG = ceil(Hkv / NW),
 *      W = max(1, floor(4096 / (HG*NW))).
 *   The fixed schedule with P == 1 splits nothing and needs no workspace.
 *   The acc rows (rows * D * 4 bytes) must stay under 2 GiB (PA_ERR_SHAPE
 *   otherwise; the balanced schedule's stay under 70 MB).
 * Workspace sizes depend only on these host-side sizes, never on device
 * contents.  Apart from the counters, contents need not be initialised.
 * Two calls in flight at once (other streams) need separate workspaces.
 *
 * Bytes of workspace pa_decode needs for these arguments; 0 for invalid
 * arguments (and for a fixed schedule with P == 1). */
size_t pa_decode_workspace_size(const pa_decode_args* a);

/* Bytes at the start of the workspace (the arrival counters) that must hold
 * zeros when a call with these arguments starts; every call leaves them
 * zero.  0 for invalid arguments and when no workspace is needed.  Host
 * only. */
size_t pa_decode_workspace_zero_bytes(const pa_decode_args* a);

/* Tokens per fixed split-K partition pa_decode will use for these arguments
 * (partition_size); 0 for the balanced schedule and for invalid arguments.
 * Host only. */
int32_t pa_decode_partition_size(const pa_decode_args* a);

/* Validate decode arguments without touching the GPU. */
pa_status pa_decode_check(const pa_decode_args* a);

/* Paged decode attention (P1 "Sayfalama Nasıl Çalışır": the attention kernel
 * follows the block table to gather keys and values block by block; P1
 * "İlgili Teknikler": FlashAttention-style tiling, the score matrix never
 * reaches device memory; grouped-query attention).  For every sequence b and
 * query head h, with g = h / (Hq/Hkv) and L = seq_lens[b]:
 *   s_t   = scale * k_scale * sum_d q[b,h,d] * K[t,g,d]      for t < L
 *   out   = v_scale * sum_t exp(s_t - max s) V[t,g,:] / sum_t exp(s_t - max s)
 * (k_scales[g] and v_scales[g] in place of k_scale and v_scale when given)
 * where K[t,g,:] is row (t mod bs, g) of block block_tables[b][t / bs].
 * L = 0 gives zeros.  fp32 accumulation; out rounded to nearest even.
 * Equivalent to pa_decode_partition followed by pa_decode_reduce. */
pa_status pa_decode(const pa_decode_args* a, void* stream);

/* Split-K step 1 (with the plan kernel first under the balanced schedule
 * past 1024 sequences): each work-group computes, for each piece of a
 * sequence it covers, the piece's running max m, sum l and unnormalised
 * V-weighted sum with an online softmax.  Sequences covered by one
 * work-group are finished here (out written); split ones too under
 * PA_COMBINE_IN_LAUNCH, else they leave fp32 partials in the workspace. */
pa_status pa_decode_partition(const pa_decode_args* a, void* stream);

/* Split-K step 2 under PA_COMBINE_REDUCE: for sequences split between
 * work-groups, combine the partials (Schedules above); under the balanced
 * schedule it also writes zeros for sequences with seq_lens 0.  Enqueues
 * nothing under PA_COMBINE_IN_LAUNCH or for a fixed schedule with P == 1. */
pa_status pa_decode_reduce(const pa_decode_args* a, void* stream);

/* pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments and the result are those of pa_decode; workspace and
 * workspace_bytes are ignored.  Instead the library uses a fixed array of
 * 32 MiB per GPU, in its own code object, held until the process ends: its
 * first 256 KiB hold the arrival counters (so B * Hkv may not exceed 65536),
 * the rest the prefix sums and partial rows that pa_decode_workspace_size
 * would count for this launch.  Arguments that need more return
 * PA_ERR_WORKSPACE, with nothing enqueued.  The call allocates and frees
 * nothing; the first call on a GPU also enqueues one small kernel that
 * clears the counters.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (two streams, or two threads) race and give
 * wrong results; calls ordered on one stream are safe.  PA_ERR_LAUNCH if the
 * HIP runtime cannot give the array's address. */
pa_status pa_decode_no_alloc(const pa_decode_args* a, void* stream);

/* Slot of each sequence's new token (P1 "Sayfalama Nasıl Çalışır", code
 * sketch: position pos goes to block table[pos / bs] at offset pos % bs):
 *   slots[b] = block_tables[b][positions[b] / block_size] * block_size
 *              + positions[b] % block_size
 * and -1 when positions[b] < 0, when positions[b] / block_size >=
 * max_blocks_per_seq or when that table entry is negative.
 * block_tables int32 [B][max_blocks_per_seq], positions and slots int32 [B],
 * device memory. */
pa_status pa_slot_mapping(const int32_t* block_tables, const int32_t* positions, int32_t B,
                          int32_t max_blocks_per_seq, int32_t block_size, int32_t* slots,
                          void* stream);

/* Cache write (P1 "Sayfalama Nasıl Çalışır", code sketch write loop): for
 * every i < T with 0 <= slot_mapping[i] < num_blocks*block_size,
 *   k_cache[slot / bs][slot % bs][:][:] = enc(k_new[i][:][:]), same for V.
 * k_new, v_new: [T][Hkv][D] of src_dtype.  enc is the identity (a bit copy)
 * when src_dtype == kv_dtype.  For an 8-bit kv_dtype and src_dtype in
 * {F32, F16, BF16}: enc(x) = fp8(fl32(x * fl32(1/k_scale))) (v_scale for V),
 * rounded to nearest even and saturating to the format's largest finite
 * value (+-448 for e4m3, +-57344 for e5m2; +-inf too), NaN -> 0x7F with the
 * NaN's sign.  Other combinations return PA_ERR_UNSUPPORTED. */
pa_status pa_reshape_and_cache(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                               int32_t block_size, int32_t num_blocks, pa_dtype src_dtype,
                               pa_dtype kv_dtype, float k_scale, float v_scale, void* stream);

/* Cache write into an 8-bit cache with one scale per KV head (P1 "İlgili
 * Teknikler": 8-bit caches; a finer scale than one per pool).  As
 * pa_reshape_and_cache with src_dtype in {F32, F16, BF16} and kv_dtype
 * 8-bit, except that head g of every row uses k_scales[g] (v_scales[g] for
 * V): enc(x) = fp8(fl32(x * fl32(1/k_scales[g]))).  k_scales, v_scales:
 * device arrays [Hkv] of positive finite fp32 (not checked).  Other dtype
 * combinations return PA_ERR_UNSUPPORTED. */
pa_status pa_reshape_and_cache_scales(const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, const int32_t* slot_mapping, int32_t T,
                                      int32_t Hkv, int32_t D, int32_t block_size,
                                      int32_t num_blocks, pa_dtype src_dtype, pa_dtype kv_dtype,
                                      const float* k_scales, const float* v_scales, void* stream);

/* The slot mapping and the cache write of one new token per sequence in one
 * launch (P1 "Sayfalama Nasıl Çalışır": the token's slot from its block
 * table, then its K/V rows written there).  Equivalent to
 *   pa_slot_mapping(block_tables, positions, B, max_blocks_per_seq,
 *                   block_size, slots)
 * followed by pa_reshape_and_cache (k_scales null) or
 * pa_reshape_and_cache_scales (k_scales and v_scales device arrays [Hkv]) of
 * the B rows k_new, v_new [B][Hkv][D] at those slots.  slots (int32 [B],
 * device) receives the slots and may be NULL.  Rows whose slot is -1 or
 * outside the pool are not written.  Argument checks are those of the two
 * calls; k_scale and v_scale are ignored when k_scales is given. */
pa_status pa_append_kv(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int32_t* block_tables, const int32_t* positions, int32_t B,
                       int32_t max_blocks_per_seq, int32_t* slots, int32_t Hkv, int32_t D,
                       int32_t block_size, int32_t num_blocks, pa_dtype src_dtype,
                       pa_dtype kv_dtype, float k_scale, float v_scale, const float* k_scales,
                       const float* v_scales, void* stream);

/* Copy-on-write block copy (P1 "Diziler Arasında Blokları Paylaşma": a
 * sequence about to write into a block that other sequences still use gets a
 * copy first; P3 article A, shared prefix support).  For each of the P rows
 * (src, dst) of block_mapping (int32 [P][2], device memory), copies the whole
 * block -- every slot, every head, K and V -- from src to dst.
 * Precondition: dst blocks are distinct and no dst is also a src in the same
 * call (otherwise the result depends on scheduling).  P == 0 enqueues
 * nothing. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping, int32_t P,
                         int32_t num_blocks, int32_t block_size, int32_t Hkv, int32_t D,
                         pa_dtype kv_dtype, void* stream);

/* Page-granular swap between two pools (P3 article A: single pages move
 * between GPU memory and CPU memory instead of whole sequences).  For each of
 * the P rows (src, dst) of block_mapping (int32 [P][2], device memory),
 * copies the whole block src of the source pools (src_k, src_v; src_num_blocks
 * blocks) over block dst of the destination pools (dst_k, dst_v;
 * dst_num_blocks blocks), every slot and head, K and V.  Both sides have the
 * block shape [block_size][Hkv][D] of kv_dtype.  Each pool is device memory
 * or pinned host memory (hipHostMalloc, e.g. a pinned torch tensor), which
 * the kernel reads or writes over the host link: eviction is device -> host,
 * restore host -> device.  A pointer the GPU cannot reach (pageable host
 * memory) returns PA_ERR_UNSUPPORTED; this check asks the HIP runtime about
 * each pool pointer.  A destination pool overlapping a source pool, other
 * than being the same pool, returns PA_ERR_SHAPE.  Pairs with an id outside
 * its pool are skipped.  Precondition: dst ids distinct, and within one pool
 * no dst is also a src.  P == 0 enqueues nothing. */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                         const int32_t* block_mapping, int32_t P, int32_t src_num_blocks,
                         int32_t dst_num_blocks, int32_t block_size, int32_t Hkv, int32_t D,
                         pa_dtype kv_dtype, void* stream);

/* Arguments of one prefill call over a batch (one layer): several new
 * tokens per sequence, attended causally over the paged context. */
typedef struct pa_prefill_args {
  void* out;                   /* [T][Hq][D] out_dtype; rows of new tokens written    */
  const void* q;               /* [T][Hq][D] q_dtype: the new tokens of all           */
                               /* sequences, packed in sequence order                 */
  const void* k_cache;         /* [num_blocks][block_size][Hkv][D] kv_dtype           */
  const void* v_cache;         /* same shape and dtype as k_cache                     */
  const int32_t* block_tables; /* [B][max_blocks_per_seq]                             */
  const int32_t* seq_lens;     /* [B]: tokens in context, the new ones included       */
  const int32_t* q_starts;     /* [B+1]: sequence b owns q rows                       */
                               /* q_starts[b] .. q_starts[b+1]-1                      */
  int32_t B, T;                /* sequences; rows of q and out                        */
  int32_t max_q_len;           /* >= every q_starts[b+1] - q_starts[b] (host bound    */
                               /* that sizes the grid)                                */
  int32_t Hq, Hkv, D;
  int32_t block_size, num_blocks, max_blocks_per_seq;
  float scale;                 /* softmax scale, e.g. 1/sqrt(D)                       */
  float k_scale, v_scale;      /* fp8 dequantisation scales; must be 1 otherwise      */
  pa_dtype q_dtype, kv_dtype, out_dtype;
  const float* k_scales;       /* NULL, or per-KV-head scales [Hkv] (device memory),  */
  const float* v_scales;       /* as in pa_decode_args                                */
} pa_prefill_args;

/* Supported prefill combinations (others return PA_ERR_UNSUPPORTED):
 *   D in {64, 128}; block_size in {8, 16, 32, 64}; G = Hq/Hkv from 1 to 16;
 *   (q, kv) in {(F16,F16), (BF16,BF16), and BF16 or F16 over FP8_E4M3 or
 *   FP8_E5M2};
 *   out_dtype = q_dtype or PA_F32.  No workspace. */

/* Validate prefill arguments without touching the GPU. */
pa_status pa_prefill_check(const pa_prefill_args* a);

/* Paged prefill attention (P1 "Çözdüğü Bellek Sorunu": the cache keeps
 * earlier tokens' K/V for later tokens; P1 "Sayfalama Nasıl Çalışır": keys
 * and values are gathered block by block through the table; P1 "İlgili
 * Teknikler": FlashAttention-style kernels over paged blocks, grouped-query
 * attention).  The new tokens' K and V must already be in the pools
 * (pa_prefill_slot_mapping, then pa_reshape_and_cache over the T rows).
 * Sequence b has n_b = q_starts[b+1] - q_starts[b] new tokens, the last n_b
 * of its L = seq_lens[b] tokens; the earlier L - n_b are cached context (an
 * earlier chunk, or shared prefix blocks).  New token i sits at position
 * p = L - n_b + i, and for q row r = q_starts[b] + i and query head h, with
 * g = h / (Hq/Hkv):
 *   s_t = scale * k_scale * sum_d q[r,h,d] * K[t,g,d]          for t <= p
 *   out[r,h,:] = v_scale * sum_{t<=p} exp(s_t - max s) V[t,g,:] / sum_{t<=p} exp(s_t - max s)
 * K[t,g,:] as in pa_decode.  fp32 accumulation; the weights enter the
 * weighted sum rounded to the 16-bit operand type (e4m3 caches compute in
 * q_dtype).  Device-side: n_b is clamped to [0, min(max_q_len, L,
 * T - q_starts[b])] (rows past it are not written); rows no sequence owns
 * are not written; L is clamped as in pa_decode; block ids outside the pool
 * are read as zeros. */
pa_status pa_prefill(const pa_prefill_args* a, void* stream);

/* Slots of the new tokens of a prefill batch (P1 "Sayfalama Nasıl
 * Çalışır", code sketch): q row r of sequence b (q_starts[b] <= r <
 * q_starts[b+1]) is new token i = r - q_starts[b] at position
 * p = seq_lens[b] - n_b + i, and
 *   slots[r] = block_tables[b][p / block_size] * block_size + p % block_size,
 * or -1 when p < 0, when p / block_size >= max_blocks_per_seq, when that
 * table entry is negative, or when no sequence owns row r.  q_starts must be
 * nondecreasing; T > 0 with B == 0 returns PA_ERR_SHAPE.  All arrays in
 * device memory: block_tables int32
 * [B][max_blocks_per_seq], seq_lens [B], q_starts [B+1], slots [T]. */
pa_status pa_prefill_slot_mapping(const int32_t* block_tables, const int32_t* seq_lens,
                                  const int32_t* q_starts, int32_t B, int32_t T,
                                  int32_t max_blocks_per_seq, int32_t block_size, int32_t* slots,
                                  void* stream);

/* ------------------------------------------------------------------ */
/* Host block manager with prefix caching (host memory only; no GPU calls). */
/*                                                                      */
/* Which physical block each sequence's table points at (P1 "Sayfalama   */
/* Nasıl Çalışır": free list, block table, a new block only when the last */
/* one is full), shared blocks with reference counts and copy-on-write    */
/* (P1 "Diziler Arasında Blokları Paylaşma"), hashing every block so that */
/* requests starting with the same tokens share cached blocks (same       */
/* section: prompt caching), and a finished sequence's blocks returned at */
/* once (P1 "İlgili Teknikler": continuous batching).                     */
/*                                                                      */
/* Rules.  Free blocks leave from the front of a FIFO list (initially     */
/* free_order, or 0..num_blocks-1) and return to its back.  A full        */
/* block's key is the 64-bit FNV-1a hash of every token from the start    */
/* of its sequence through the block (token ids as 4-byte little-endian   */
/* integers); a hit also matches the block's stored tokens and its        */
/* parent's key.  Admitting a prompt reuses cached blocks for its leading */
/* full blocks, stopping at the first miss; new full blocks register     */
/* their key unless it is taken.  A new block is the front of the free    */
/* list or, when that is empty, the cached block with no users released   */
/* longest ago (it loses its key).  Freeing a sequence releases its       */
/* blocks last block first: keyed blocks stay cached, others go to the   */
/* free list.  Not thread-safe: one manager per thread, or a lock around  */
/* it.                                                                   */
typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens; prefix_caching 0
 * turns keys off (no sharing across requests).  free_order: NULL, or a
 * permutation of 0..num_blocks-1 (host memory).  NULL on invalid arguments
 * or allocation failure. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_caching,
                               const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* m);

/* Admit a sequence with n prompt tokens (host array): *seq receives its id
 * (ids count up from 0 and are never reused), *cached_tokens how many of
 * its leading tokens sit in reused cached blocks (their K/V need no
 * recomputation).  PA_ERR_OUT_OF_BLOCKS if the new blocks do not fit. */
pa_status pa_bm_add(pa_block_manager* m, const int32_t* tokens, int32_t n, int32_t* seq,
                    int32_t* cached_tokens);

/* Append one token: *slot receives its flat slot (block * block_size +
 * offset); when the last block was shared, a private copy replaces it in
 * this sequence's table and (*copy_src, *copy_dst) name the block copy to
 * run before the cache write (pa_copy_blocks), else both are -1. */
pa_status pa_bm_append(pa_block_manager* m, int32_t seq, int32_t token, int32_t* slot,
                       int32_t* copy_src, int32_t* copy_dst);

/* A new sequence sharing every block of seq (parallel sampling, beams). */
pa_status pa_bm_fork(pa_block_manager* m, int32_t seq, int32_t* new_seq);

/* Release a finished sequence's blocks at once. */
pa_status pa_bm_free(pa_block_manager* m, int32_t seq);

/* The block table of seq: returns its length and copies up to capacity
 * entries to out (may be NULL); -1 for an unknown sequence. */
int32_t pa_bm_table(const pa_block_manager* m, int32_t seq, int32_t* out, int32_t capacity);

/* Tokens of seq (-1 if unknown); free plus evictable blocks; keyed blocks. */
int32_t pa_bm_length(const pa_block_manager* m, int32_t seq);
int32_t pa_bm_free_blocks(const pa_block_manager* m);
int32_t pa_bm_cached_blocks(const pa_block_manager* m);

/* Measurement utility, not a step of the path (the pages define no such
 * operation): reads pieces ids[0..n) of `pool` (num_pieces pieces of
 * piece_bytes each, a multiple of 1024 up to 32768, pool 16-byte aligned,
 * device memory) in that order, with the non-temporal 16-byte buffer loads
 * of the attention kernels, and folds every loaded word into sink (uint32
 * [sink_len], device), one word per work-group, so that no load is dead.
 * Ids outside [0, num_pieces) read nothing.  Timed over pieces of a block's
 * size in random order it gives the practical HBM read rate of a block
 * gather: the ceiling the attention kernels are measured against beside the
 * vendor peak.  Launches min(sink_len, 8 * compute units) work-groups. */
pa_status pa_read_blocks(const void* pool, int32_t num_pieces, size_t piece_bytes,
                         const int32_t* ids, int32_t n, uint32_t* sink, int32_t sink_len,
                         void* stream);

/* Static description of a status code. */
const char* pa_status_str(pa_status s);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
