// Kernel 2 (bf16): causal grouped-query flash attention for prefill on gfx950
// matrix cores.
//
// Computes, for every request and query head h, softmax(q~ k~^T / sqrt(D)) v
// with the lower-triangular (causal) mask, query head h reading KV head
// floor(h / G) (zero-to-sglang code walkthrough, section 3.3; the concept
// chapter's section 2.6 names FlashAttention as the I/O-aware way to compute
// the same result).  Keys and values are read from the per-request cache that
// kernel 1 has just written.
//
// Design (one workgroup = 8 wavefronts = 512 threads, one workgroup per CU):
//  * Work item = (KV-head chunk, request, query tile).  A chunk is HC query
//    heads of one KV group; the tile is 8/HC blocks of 32 consecutive tokens,
//    so every workgroup owns 8 "query blocks" of 32 (head, token) rows and each
//    K/V tile it stages in LDS feeds all of them (GQA sharing).
//  * Each wavefront owns one query block.  Scores are formed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A
//    operand, Q^T stays in registers as the B operand for the whole loop.  In
//    the 32x32 accumulator layout a lane then holds one query (lane % 32) and
//    16 of the 32 keys of a block, so the row max needs one exchange with lane
//    ^ 32.  The row sum is formed on the matrix cores as well: a 16x16x32
//    product of a 0/1 selection matrix with each P^T operand hands every lane
//    its own query's sum over both lane halves.
//  * O^T = V^T P^T with the same instruction: P^T goes straight from the
//    score accumulators into the B operand (after rounding to bf16).  V stays
//    row-major in LDS, as the cache holds it; the V^T operand comes from it
//    through gfx950's transposing LDS read (ds_read_b64_tr_b16), two per
//    operand, whose lanes receive exactly the keys the P^T operand holds.
//    The O^T accumulator is again one query per lane, so the online-softmax
//    rescale is a per-lane multiply.
//  * Softmax in the log2 domain: q~ is multiplied by log2(e)/sqrt(D) before
//    its bf16 rounding, so a score is already the exponent of 2 that softmax
//    takes.  Softmax is unchanged by a common shift of a row's scores, and
//    with normalised Q and K the scores cannot leave a small range: RMSNorm
//    leaves a head vector of norm at most max|w| sqrt(D) and the rotation
//    keeps norms, so |s| <= max|w_q| max|w_k| sqrt(D) log2(e) (Cauchy-
//    Schwarz).  When that bound is at most BOUND_LOG2 and the request has no
//    cached history (every key it reads is written by this call), p = 2^s is
//    taken with no shift at all: no row max, no rescale, no subtraction, and
//    p, its row sum and P.V stay far inside fp32 and bf16 range.  Otherwise
//    (larger weights, or a request whose history the caller wrote) the fp32
//    online softmax subtracts a running max that is raised lazily (only when
//    a tile max exceeds it by more than 2^8), so the O rescale is rare.  The
//    two are separate kernels over the same grid (prefill_mfma_kernel<..,
//    true> and <.., false>); each work item runs in one of them.  K/V tiles
//    run only up to the causal diagonal of the workgroup's last token; tiles
//    entirely above a wavefront's rows are skipped by that wavefront; only
//    tiles that cross the diagonal are masked.
//  * K/V tiles go from global memory straight into LDS (buffer loads with
//    the LDS flag, no registers, no LDS stores): 16 bytes per lane, the
//    lanes spread over the rows so that the tile lands with its padded row
//    strides.  Keys at or past the request's length read as zeros (the
//    buffer range ends at the last key), so whatever the cache holds there
//    never reaches the accumulators.
//  * Three LDS slots, each K and V slot an array of its own: step kt forms
//    tile kt+1's scores while it turns tile kt's scores into probabilities
//    and multiplies them by tile kt's V; tile kt+2 streams into the third
//    slot meanwhile.  Separate arrays let the compiler see that the loads
//    into one slot do not touch the slots being read, so it waits for them
//    only at the step's end.  One barrier per step.  The tile loop is
//    unrolled by six so that every slot, hence every LDS address, is a
//    compile-time constant.  Steps whose next tile masks nothing for any row
//    of the workgroup run first, in groups of six, as straight blocks.
//  * Grid: work items ordered by (KV-head chunk, request, query tile from the
//    last), and block ids remapped so that consecutive items land on the same
//    XCD (the hardware deals workgroups round-robin over the 8 XCDs).  The
//    CUs of an XCD then work on the tiles of one request and KV head at a
//    time, whose K/V stays in that XCD's L2 (ordering by tile across requests
//    instead made a chunked prefill onto long caches fetch its history from
//    HBM about 25 times); within a request the heaviest tiles go first.  For
//    a batch of equal-length requests with no history the order is (KV-head
//    chunk, query tile from the last, request): heaviest first over the whole
//    batch, which shortens the tail.  Where lengths differ that order would
//    put the empty items of the short requests (each still a workgroup
//    launch) among the first, so the request order is kept.

#include "decode_body.h"
#include "device_common.h"
#include "launch.h"
#include "../../include/qkra_phase_stamps.h"

namespace qkra {
namespace {

// Launch shape: QB = 1 query block (32 rows) per wavefront and 8 wavefronts
// per workgroup, so a workgroup owns 8 query blocks; BN keys per K/V tile.
// Two wavefronts share each SIMD, so their matrix and vector work interleave.
// The LDS slots, the DMA lane map and the Q and output staging below are laid
// out for exactly this shape (their static_asserts say so).
constexpr int QB = 1;
constexpr int BN = 64;
constexpr int NWAVES = 8 / QB;
constexpr int NTHREADS = 64 * NWAVES;
constexpr float TAU = 8.0f;   // lazy-rescale threshold (log2 units)
// Largest score bound (log2 units) taken without a shift: p then lies in
// [2^-48, 2^48], a row sum of up to 2^31 keys below 2^79.
constexpr float BOUND_LOG2 = 48.0f;

// Max of a value held by lanes l and l ^ 32 (gfx950 v_permlane32_swap).
__device__ __forceinline__ float half_wave_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

constexpr int NSLOT = 3;  // LDS tile slots

// Launch flags: the host launched only the kernel its weight bound selects;
// work items in query-tile order across the requests.
constexpr int kFlagSinglePath = 1;
constexpr int kFlagTileMajor = 2;

// ds_read_b64_tr_b16 from a generic pointer into LDS (the address-space cast
// keeps which LDS array it reads, so loads into other arrays need not be
// waited for).
__device__ __forceinline__ dbody::s16x4 read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) dbody::s16x4*)(const_cast<bf16*>(p)));
}

// ---- phase stamps (the profiling build, -DQKRA_PHASE_STAMPS, only) ----------
// Every prefill workgroup's wavefronts record the 100 MHz constant clock
// (s_memrealtime) at fixed points of their life and where they ran, so the
// time of a work item splits into its prologue (item decode, first loads,
// Q normalise and rotate), its tile loop and its epilogue.  The record's
// address stays in vector registers, so the stamps take no scalar register
// across the tile loop.  In the normal build every stamp compiles to nothing.
#ifdef QKRA_PHASE_STAMPS
static_assert(QKRA_STAMP_SLOTS == 8 && QKRA_STAMP_WAVES == NWAVES, "the stamp record layout");
__device__ unsigned long long g_phase_stamps[static_cast<size_t>(QKRA_STAMP_WGS) * QKRA_STAMP_WAVES * QKRA_STAMP_SLOTS];
#endif
struct PhaseStamps {
#ifdef QKRA_PHASE_STAMPS
  unsigned long long addr;
  __device__ __forceinline__ PhaseStamps() {
    addr = reinterpret_cast<unsigned long long>(
        g_phase_stamps +
        (static_cast<size_t>(blockIdx.x % QKRA_STAMP_WGS) * QKRA_STAMP_WAVES + (threadIdx.x >> 6)) * QKRA_STAMP_SLOTS);
    asm volatile("" : "+v"(addr));
  }
  __device__ __forceinline__ void mark(int slot, unsigned long long v) const {
    if ((threadIdx.x & 63) == 0 && blockIdx.x < QKRA_STAMP_WGS) reinterpret_cast<unsigned long long*>(addr)[slot] = v;
  }
  __device__ __forceinline__ void now(int slot) const { mark(slot, __builtin_amdgcn_s_memrealtime()); }
  __device__ __forceinline__ unsigned long long hw_where() const {
    return (__builtin_amdgcn_s_getreg((15 << 11) | 4) & 0xffffull) |
           ((__builtin_amdgcn_s_getreg((3 << 11) | 20) & 0xfull) << 16);
  }
  // HW_ID (wave, SIMD, CU, shader array, engine), XCC_ID, the item's tiles and its logical index.
  __device__ __forceinline__ void where(int ntiles, int logical) const {
    mark(QKRA_STAMP_WHERE, hw_where() | ((static_cast<unsigned long long>(ntiles) & 0xffffull) << 20) |
                               (static_cast<unsigned long long>(logical) << 36));
  }
  // A workgroup of the fused step's decode role: bit 63 set, no item.
  __device__ __forceinline__ void where_decode_role() const { mark(QKRA_STAMP_WHERE, hw_where() | (1ull << 63)); }
#else
  __device__ __forceinline__ void now(int) const {}
  __device__ __forceinline__ void where(int, int) const {}
  __device__ __forceinline__ void where_decode_role() const {}
#endif
};

// The decode role of the fused step kernel: the first `wgs` workgroups each
// run kFusedDecodeWavesPerWg wavefronts of the decode split (decode_body.h)
// over the plan built for kDecodeWaves wavefronts, with their K/V tiles in
// this kernel's LDS slots; the other workgroups run prefill work items.
constexpr int kFusedDecodeWavesPerWg = 6;
constexpr int kFusedDecodeWgs = kDecodeWaves / kFusedDecodeWavesPerWg;
static_assert(kDecodeWaves % kFusedDecodeWavesPerWg == 0 && kFusedDecodeWgs % 8 == 0,
              "the decode workgroups keep the prefill items' XCD mapping");
struct DecodeRole {
  const bf16* q;
  const bf16* k_cache;
  const bf16* v_cache;
  const int32_t* cache_lens;
  const int32_t* plan;
  float* partials;
  int cache_capacity, chunks_per_kv, num_units, wgs;
};

// Whether p = 2^s may be taken without a shift: a request with no cached
// history (every key it reads is written by this call with k_norm_weight)
// and max|w_q| max|w_k| at most
// `limit` = BOUND_LOG2 / (1.02 D scale_log2).  |s| <= |q~'| |k~| with
// |q~'| <= max|w_q| sqrt(D) scale_log2 and |k~| <= max|w_k| sqrt(D); the
// factor 1.02 covers the bf16 roundings of q~' and k~ and the fp32
// arithmetic before them.  Every wavefront of both prefill kernels reduces
// the same weights the same way (max is exact, one rounded product), so the
// answer is the same everywhere.  An infinite weight fails the test; a NaN
// one is passed over by the max (IEEE maxNum), and then every score of the
// head is NaN on either path.
// The test is split in two so that the kernel that runs can issue its first
// loads between the weight loads and the decision.
struct WeightMax {
  float q, k;  // this lane's largest |w|, then the wavefront's
};
template <int D>
__device__ __forceinline__ WeightMax weight_max_lane(const bf16* __restrict__ q_norm_weight,
                                                     const bf16* __restrict__ k_norm_weight) {
  const int lane = threadIdx.x & 63;
  WeightMax w{0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    w.q = fmaxf(w.q, fabsf(static_cast<float>(q_norm_weight[lane + 64 * i])));
    w.k = fmaxf(w.k, fabsf(static_cast<float>(k_norm_weight[lane + 64 * i])));
  }
  return w;
}
__device__ __forceinline__ bool scores_bounded(WeightMax w, int past, float limit) {
  if (past != 0) return false;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    w.q = fmaxf(w.q, xor_shuffle(w.q, m));
    w.k = fmaxf(w.k, xor_shuffle(w.k, m));
  }
  return __builtin_amdgcn_readfirstlane(w.q * w.k <= limit ? 1 : 0) != 0;
}

// One work item, with the softmax path fixed at compile time (kBounded: no
// shift).  Each path is a kernel of its own: in one kernel, the register
// allocation shared by the two tile loops spilled in the shifted one and
// slowed both.  Without the caller's weight bound a call launches both
// kernels over the same grid, and each workgroup of the one whose path its
// request and the weights do not select returns at once; with it, only the
// selected kernel is launched (flag kFlagSinglePath).
// kPaged: k_cache and v_cache are pools read through `paged` (a K/V tile of
// BN keys always lies in one page: pages hold a multiple of BN slots).
template <int D, int HC, bool kBounded, int kDecGW = 0, bool kPaged = false>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_mfma_kernel(
    const bf16* __restrict__ qkv, const bf16* __restrict__ q_norm_weight, const bf16* __restrict__ k_norm_weight,
    const float* __restrict__ rope_table,
    const bf16* __restrict__ k_cache, const bf16* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ past_lens, bf16* __restrict__ out,
    int num_q_heads, int num_kv_heads,
    int cache_capacity, int num_seqs, int tiles_per_seq, int chunks_per_kv, int num_items,
    float rms_eps, float scale_log2, float bound_limit, DecodeRole dec, PagedTable paged, int flags) {
  const bool single_path = (flags & kFlagSinglePath) != 0;
  constexpr int TBN = 8 / HC;       // token blocks (of 32) per workgroup
  constexpr int TM = 32 * TBN;      // tokens per workgroup
  constexpr int DS = D / 16;        // k-steps over D for the scores
  constexpr int DB = D / 32;        // 32-wide blocks of D in the output
  constexpr int KB = BN / 32;       // 32-key blocks per tile
  constexpr int KSTEPS = BN / 16;   // 16-key steps per tile
  constexpr int KST = D + 8;        // LDS row stride of K (elements): 16 bytes of pad
  constexpr int VRS = D + 32;       // LDS row stride of V, row-major (elements): 64 bytes of pad
  // One LDS array per slot: the compiler then knows that a tile load into
  // one slot does not touch another, and waits for it only where its slot is read.
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * KST], sK1[BN * KST], sK2[BN * KST];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * VRS], sV1[BN * VRS], sV2[BN * VRS];
  auto kslot = [&](auto sc) -> bf16* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return sK0; else if constexpr (s == 1) return sK1; else return sK2;
  };
  auto vslot = [&](auto sc) -> bf16* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return sV0; else if constexpr (s == 1) return sV1; else return sV2;
  };
  // The six slot arrays by a wave-uniform index (K slots first).
  auto region = [&](int i) -> bf16* {
    return i == 0 ? sK0 : i == 1 ? sK1 : i == 2 ? sK2 : i == 3 ? sV0 : i == 4 ? sV1 : sV2;
  };

  // ---- work item (XCD-aware remap; per request, heaviest tiles first) -------
  const PhaseStamps stamps;
  stamps.now(QKRA_STAMP_ENTRY);
  int bid = blockIdx.x;
  int nb = gridDim.x;  // a multiple of 8
  if constexpr (kDecGW > 0) {
    if (bid < dec.wgs) {  // decode role (the fused step): its wavefronts' tiles in the K and V slots
      const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      constexpr int DT = kDecodeStepKeys * (D + 8);  // elements of one decode tile
      static_assert(2 * DT <= BN * KST && 2 * DT <= BN * VRS && kFusedDecodeWavesPerWg == 6 && NWAVES >= 6,
                    "a decode wavefront's K and V tiles fit in one slot array");
      if (wv < kFusedDecodeWavesPerWg) {
        bf16* base = region(wv);
        dbody::decode_wave<D, kDecGW>(base, base + DT, bid * kFusedDecodeWavesPerWg + wv, dec.q, dec.k_cache,
                                      dec.v_cache, dec.cache_lens, dec.plan, dec.partials, num_q_heads, num_kv_heads,
                                      dec.cache_capacity, dec.chunks_per_kv, dec.num_units, scale_log2);
      }
      stamps.now(QKRA_STAMP_END);
      stamps.where_decode_role();
      return;
    }
    bid -= dec.wgs;  // a multiple of 8: the XCD mapping below is unchanged
    nb -= dec.wgs;
  }
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  if (logical >= num_items) return;
  const int per_chunk = tiles_per_seq * num_seqs;
  const int chunk = logical / per_chunk;
  const int rem = logical - chunk * per_chunk;
  const bool tile_major = (flags & kFlagTileMajor) != 0;
  const int seq = tile_major ? rem % num_seqs : rem / tiles_per_seq;
  const int tile = tiles_per_seq - 1 - (tile_major ? rem / num_seqs : rem % tiles_per_seq);
  // Entries cached before the chunk (its token t sits at slot past + t).
  // Lengths are clamped to the cache so out-of-contract inputs cannot address past it.
  const int past = past_lens ? min(max(past_lens[seq], 0), cache_capacity) : 0;
  // Which kernel runs the item.  The workgroup of the other one returns as
  // early as it can: the unshifted kernel as soon as it sees a history, the
  // shifted one once the weights are reduced, before anything else is
  // loaded.  The unshifted kernel tests the weights once its first K/V tile
  // and Q loads are in flight (below).
  // With `single_path` the host launched only this kernel (the caller's
  // weight bound selected it): the running-max kernel then takes every item.
  if constexpr (kBounded) {
    if (past != 0) return;
  } else {
    if (!single_path && past == 0 &&
        scores_bounded(weight_max_lane<D>(q_norm_weight, k_norm_weight), 0, bound_limit))
      return;
  }
  const int cu0 = cu_seqlens[seq];
  const int seqlen = min(cu_seqlens[seq + 1] - cu0, cache_capacity - past);
  const int t0 = tile * TM;
  if (t0 >= seqlen) return;
  WeightMax wmax{0.f, 0.f};
  if constexpr (kBounded) wmax = weight_max_lane<D>(q_norm_weight, k_norm_weight);
  const int group = num_q_heads / num_kv_heads;
  const int g = chunk / chunks_per_kv;
  const int h0 = g * group + (chunk % chunks_per_kv) * HC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: per-wave branches stay scalar
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int qtok[QB], qhead[QB], qfirst[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int bi = QB * wave + qb;
    qfirst[qb] = t0 + 32 * (bi / HC);
    qtok[qb] = qfirst[qb] + l32;
    qhead[qb] = h0 + bi % HC;
  }

  // Q^T fragments (B operand): lane holds query l32, d = 16*ds + 8*hi .. +7.
  // Q comes raw from qkv and is RMS-normalised with w_q and rotated with the
  // row's cos/sin pairs (kernel 1 forms them in fp64) in a row-coalesced
  // layout: QLPR lanes per row, lane j holding d = 8j .. 8j+7 and its
  // rotate-half partners D/2 + 8j .. +7, so every 16-byte load instruction
  // reads whole 128-byte lines (a lane-per-row load touches 32 lines per
  // instruction and made the prologue twice as long).  The row's sum of
  // squares is reduced over its QLPR lanes.  Each wavefront then passes its
  // 32 x D tile through its own LDS region into the fragment layout.  Rows
  // past the request's end are zero.
  constexpr int QLPR = D / 16;       // lanes per row
  constexpr int QRPI = 64 / QLPR;    // rows per load instruction
  constexpr int QNG = 32 / QRPI;     // load groups per 32-row block
  constexpr int EST = D + 8;         // LDS row stride of a staged 32 x D tile (elements)
  // Slots 0 and 1 take the first two K/V tiles while Q is staged: wavefronts 0-1 stage in slot 2 of the K
  // array, 2-3 in slot 2 of the V array, the others in a region of their own.
  static_assert(NWAVES == 8 && 2 * 32 * EST <= BN * KST && 2 * 32 * EST <= BN * VRS, "Q staging layout");
  __shared__ __attribute__((aligned(16))) bf16 sQ[(NWAVES - 4) * 32 * EST];
  const int qj = lane % QLPR;
  const int qr = lane / QLPR;
  bf16x8 qf[QB][DS];
  u32x4 qraw[QB][QNG][2];
  f32x4 qtab[QB][QNG][4];
  bool qvalid[QB][QNG];
  // Issue every Q, table and weight load; nothing waits for them here.
  auto q_issue = [&]() {
    const int qkv_width = (num_q_heads + 2 * num_kv_heads) * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int gi = 0; gi < QNG; ++gi) {
        const int t = qfirst[qb] + QRPI * gi + qr;
        qvalid[qb][gi] = t < seqlen;
        const int tok = cu0 + (qvalid[qb][gi] ? t : 0);
        const bf16* src = qkv + static_cast<size_t>(tok) * qkv_width + qhead[qb] * D + 8 * qj;
        qraw[qb][gi][0] = *reinterpret_cast<const u32x4*>(src);
        qraw[qb][gi][1] = *reinterpret_cast<const u32x4*>(src + D / 2);
        // Table row: four runs of D/4 floats (cos of pair indices 8j..8j+3,
        // cos 8j+4..8j+7, sin 8j..8j+3, sin 8j+4..8j+7), lane j's 4 floats at 4j.
        const float* tab = rope_table + static_cast<size_t>(tok) * D + 4 * qj;
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) qtab[qb][gi][pc] = *reinterpret_cast<const f32x4*>(tab + pc * (D / 4));
      }
  };
  // Normalise, rotate, scale by log2(e)/sqrt(D), stage and read back as
  // fragments.
  auto q_finish = [&]() {
    const u32x4 wlo = *reinterpret_cast<const u32x4*>(q_norm_weight + 8 * qj);
    const u32x4 whi = *reinterpret_cast<const u32x4*>(q_norm_weight + D / 2 + 8 * qj);
    bf16* stage = wave < 2 ? sK2 + wave * 32 * EST : (wave < 4 ? sV2 + (wave - 2) * 32 * EST : sQ + (wave - 4) * 32 * EST);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int gi = 0; gi < QNG; ++gi) {
        float xl[8], xh[8];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wl = qraw[qb][gi][0][e >> 1], wh = qraw[qb][gi][1][e >> 1];
          xl[e] = (e & 1) ? bf16_hi_to_f32(wl) : bf16_lo_to_f32(wl);
          xh[e] = (e & 1) ? bf16_hi_to_f32(wh) : bf16_lo_to_f32(wh);
          ss += xl[e] * xl[e] + xh[e] * xh[e];
        }
#pragma unroll
        for (int m = 1; m < QLPR; m <<= 1) ss += xor_shuffle(ss, m);
        const float inv_rms = rsqrtf(ss * (1.0f / D) + rms_eps) * scale_log2;
        float y1[8], y2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float c = qtab[qb][gi][e >> 2][e & 3], sv = qtab[qb][gi][2 + (e >> 2)][e & 3];
          const float wl = (e & 1) ? bf16_hi_to_f32(wlo[e >> 1]) : bf16_lo_to_f32(wlo[e >> 1]);
          const float wh = (e & 1) ? bf16_hi_to_f32(whi[e >> 1]) : bf16_lo_to_f32(whi[e >> 1]);
          const float a = xl[e] * inv_rms * wl;
          const float b = xh[e] * inv_rms * wh;
          y1[e] = a * c - b * sv;
          y2[e] = b * c + a * sv;
        }
        u32x4 w1 = {pack_bf16x2(y1[0], y1[1]), pack_bf16x2(y1[2], y1[3]), pack_bf16x2(y1[4], y1[5]),
                    pack_bf16x2(y1[6], y1[7])};
        u32x4 w2 = {pack_bf16x2(y2[0], y2[1]), pack_bf16x2(y2[2], y2[3]), pack_bf16x2(y2[4], y2[5]),
                    pack_bf16x2(y2[6], y2[7])};
        if (!qvalid[qb][gi]) w1 = w2 = u32x4{};
        const int r = QRPI * gi + qr;
        *reinterpret_cast<u32x4*>(&stage[r * EST + 8 * qj]) = w1;
        *reinterpret_cast<u32x4*>(&stage[r * EST + D / 2 + 8 * qj]) = w2;
      }
      // A wavefront's LDS accesses complete in order, so its lanes read what
      // the others wrote without a barrier (and the next block's writes come
      // after these reads).
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qf[qb][ds] = *reinterpret_cast<const bf16x8*>(&stage[l32 * EST + 16 * ds + 8 * hi]);
    }
  };

  f32x16 acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  float m_run[QB];
  // Row sums on the matrix cores (see probs below): every element of
  // lsum[qb] holds the sum for the lane's query, over both key halves.
  f32x4 lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    lsum[qb] = f32x4{};
  }

  const int kv_end = past + min(seqlen, t0 + TM);
  const int ntiles = (kv_end + BN - 1) / BN;
  int qlast = qfirst[0];
#pragma unroll
  for (int qb = 1; qb < QB; ++qb) qlast = max(qlast, qfirst[qb]);
  // Tiles holding a key visible to this wavefront's rows (the rest are only loaded).
  const int wtiles = min(kv_end - 1, past + qlast + 31) / BN + 1;
  const size_t head_off = (static_cast<size_t>(seq) * num_kv_heads + g) * cache_capacity * D;
  const bf16* kbase = k_cache + head_off;
  const bf16* vbase = v_cache + head_off;

  // ---- global -> LDS, by DMA --------------------------------------------------
  // Buffer loads that write LDS directly (no registers): each instruction
  // moves 64 16-byte pieces to 1 KB of consecutive LDS, lane i to piece i,
  // and a lane whose offset is past the buffer range writes zeros without
  // touching memory.  The pieces are assigned so that LDS holds K rows at a
  // stride of D+8 elements and V rows (row-major) at D+32; the lanes that
  // land on a row's pad take an offset past the range.  The resource covers
  // the tile's rows below kv_end, so rows at or past kv_end arrive as zeros
  // too (finite, so p = 0 times V stays 0; every such key lies after every
  // stored query row and is removed by the causal mask).  Each wavefront
  // issues instructions wave, wave + 8, ... of a tile; its lane offsets are
  // loop-invariant.  The 16-byte padding spreads a K fragment read over all
  // banks; V's 64 bytes do the same for the transposing reads below.
  constexpr int KRC = KST / 8, VRC = VRS / 8;               // 16-byte pieces per LDS row
  constexpr int KDMA = BN * KRC / 64, VDMA = BN * VRC / 64;  // instructions per tile
  constexpr int KJ = (KDMA + NWAVES - 1) / NWAVES, VJ = (VDMA + NWAVES - 1) / NWAVES;
  static_assert(BN * KRC % 64 == 0 && BN * VRC % 64 == 0, "whole instructions per tile");
  constexpr uint32_t kPastRange = 0x7ffffff0u;
  uint32_t koff[KJ], voff[VJ];
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int p = 64 * (wave + NWAVES * j) + lane, r = p / KRC, c = p % KRC;
    koff[j] = c < D / 8 ? static_cast<uint32_t>(r * D * 2 + c * 16) : kPastRange;
  }
#pragma unroll
  for (int j = 0; j < VJ; ++j) {
    const int p = 64 * (wave + NWAVES * j) + lane, r = p / VRC, c = p % VRC;
    voff[j] = c < D / 8 ? static_cast<uint32_t>(r * D * 2 + c * 16) : kPastRange;
  }
  auto load_tile = [&](int kt, auto slotc) {
    const int k0 = kt * BN;
    const uint32_t bytes = static_cast<uint32_t>(min(kv_end - k0, BN)) * D * 2;
    const bf16* kt_base = kbase + static_cast<size_t>(k0) * D;
    const bf16* vt_base = vbase + static_cast<size_t>(k0) * D;
    if constexpr (kPaged) {  // the tile's rows, from the page that holds them
      const size_t row = paged_row<true>(paged, seq, g, k0, num_kv_heads, D);
      kt_base = k_cache + row;
      vt_base = v_cache + row;
    }
    const auto rk = buffer_rsrc(kt_base, bytes);
    const auto rv = buffer_rsrc(vt_base, bytes);
    static_for<KJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int i = wave + NWAVES * j;
      if (j + 1 < KJ || i < KDMA) buffer_load16_lds(rk, kslot(slotc) + i * 512, koff[j]);
    });
    static_for<VJ>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const int i = wave + NWAVES * j;
      if (j + 1 < VJ || i < VDMA) buffer_load16_lds(rv, vslot(slotc) + i * 512, voff[j]);
    });
  };
  // V^T operands come from row-major V by transposing reads: lane (hi, g16, l16)
  // of a read gives keys R0 .. R0+3 of column C0 + l16, R0 = 16ks + 4hi (then
  // + 8), C0 = 32db + 16g16, i.e. d = 32db + l32 and the keys the P^T operand
  // of lane half hi holds.  With rows 320 (D = 128) or 192 (D = 64) bytes apart
  // the 64 lanes' 8-byte reads cover every bank exactly twice.
  const int vlane = (4 * hi + ((lane & 15) >> 2)) * VRS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // ---- the matrix and softmax pieces ----------------------------------------
  // S^T = K Q^T for the tile in `slot`: lane holds query l32 and, per 32-key
  // block kb, keys 32kb + 8(j/4) + 4hi + j%4 in register j.
  auto scores = [&](auto slotc, f32x16 (&S)[QB][KB]) {
    const bf16* sk = kslot(slotc);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) S[qb][kb] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sk[(kb * 32 + l32) * KST + 16 * ds + 8 * hi]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], S[qb][kb], 0, 0, 0);
      }
    }
  };

  // Causal mask (tiles that cross the diagonal only).
  auto tile_mask = [&](int kt, f32x16 (&S)[QB][KB]) {
    const int k0 = kt * BN;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (k0 + BN - 1 > past + qfirst[qb]) {
        const int lim = past + qtok[qb] - k0 - 4 * hi;  // register j of block kb holds key k0 + 32kb + 8(j/4) + 4hi + j%4
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * kb + 8 * (j >> 2) + (j & 3) > lim) S[qb][kb][j] = kNegInf;
      }
    }
  };

  // The tile's row max (shifted path only).
  auto tile_max = [&](f32x16 (&S)[QB][KB], float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) m = fmaxf(m, S[qb][kb][j]);
      mx[qb] = half_wave_max(m);
    }
  };

  // Lazy rescale: the running max is raised only when a tile max exceeds it
  // by more than 2^TAU; the stale max is used consistently for p and the row
  // sum, so the result is exact.
  auto raise_max = [&](const float (&mx)[QB]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const bool need = mx[qb] > m_run[qb] + TAU;
      if (__any(need)) {
        const float m_new = need ? mx[qb] : m_run[qb];
        const float alpha = need ? fast_exp2(m_run[qb] - m_new) : 1.0f;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
        m_run[qb] = m_new;
      }
    }
  };

  // p = 2^s (bounded path) or 2^(s - m), rounded to bf16 as the B operand of
  // the P.V product; the row sum accumulates the same rounded values, on the
  // matrix cores (a chain of 16 v_dot2 per tile cost more than the four
  // small products below).  16-key step ks uses registers 8*(ks%2) .. +7 of
  // key block ks/2.
  // Taken as the B operand of v_mfma_f32_16x16x32_bf16, P^T operand pf[qb][ks]
  // puts lane l's eight probabilities (all of query l % 32) in column l % 16,
  // k block l / 16.  Column n thus holds query n in k blocks 0 and 2 and query
  // n + 16 in blocks 1 and 3.  With A[m][k] = 1 where bit 2 of m equals bit 0
  // of k's block (0 elsewhere), output row m of column n is the sum of query
  // n's (m / 4 even) or n + 16's (m / 4 odd) sixteen probabilities, and lane l
  // receives rows 4 (l / 16) .. +3 of column l % 16: its own query's sum.
  const bf16 sel1 = static_cast<bf16>(((lane >> 2) & 1) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
  const bf16x8 rsel = {sel1, sel1, sel1, sel1, sel1, sel1, sel1, sel1};
  auto probs = [&](f32x16 (&S)[QB][KB], bf16x8 (&pf)[QB][KSTEPS]) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -m_run[qb];
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int kb = ks >> 1, base = 8 * (ks & 1);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(kBounded ? S[qb][kb][base + 2 * e] : S[qb][kb][base + 2 * e] + nm);
          const float p1 = fast_exp2(kBounded ? S[qb][kb][base + 2 * e + 1] : S[qb][kb][base + 2 * e + 1] + nm);
          w[e] = pack_bf16x2(p0, p1);
        }
        pf[qb][ks] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, pf[qb][ks], lsum[qb], 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T for the tile in `slot`.
  auto pv = [&](auto slotc, const bf16x8 (&pf)[QB][KSTEPS]) {
    const bf16* sv = vslot(slotc) + vlane;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16* vp = sv + 16 * ks * VRS + 32 * db;
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(read_tr16(vp), read_tr16(vp + 8 * VRS),
                                                                             0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ks], acc[qb][db], 0, 0, 0);
      }
  };

  // ---- software pipeline.  Entering step kt, S holds tile kt's masked
  // scores and m_run already covers them.  Step kt forms tile kt+1's scores
  // on the matrix cores while the vector units turn tile kt into
  // probabilities, then issues tile kt's P.V while the vector units mask and
  // reduce tile kt+1.  Tile kt+2 streams into the third LDS slot meanwhile.
  // The next tile's scores are formed even on a wavefront's last tile (from
  // whatever the slot holds, and then dropped): that keeps the score, the
  // probability and the P.V work of a step in one branch-free block, so the
  // matrix and vector instructions can interleave.
  // Step kt (J = kt mod 2*NSLOT) reads slots kt mod NSLOT (P.V) and kt+1 mod
  // NSLOT (scores) and fills slot kt+2 mod NSLOT.
  auto step = [&](auto jc, int kt, f32x16 (&Scur)[QB][KB], f32x16 (&Snext)[QB][KB]) {
    constexpr int J = decltype(jc)::value;
    using SlotPv = std::integral_constant<int, J % NSLOT>;
    using SlotS = std::integral_constant<int, (J + 1) % NSLOT>;
    using SlotLd = std::integral_constant<int, (J + 2) % NSLOT>;
    const bool prefetch = kt + 2 < ntiles;
    if (prefetch) load_tile(kt + 2, SlotLd{});
    if (kt < wtiles) {
      bf16x8 pf[QB][KSTEPS];
      scores(SlotS{}, Snext);
      probs(Scur, pf);
      pv(SlotPv{}, pf);
      if (kt + 1 < wtiles) {
        tile_mask(kt + 1, Snext);
        if constexpr (!kBounded) {
          float mx[QB];
          tile_max(Snext, mx);
          raise_max(mx);
        }
      }
    }
    if (prefetch) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wavefront's tile kt+2 is in LDS
    __syncthreads();
  };

  // A step whose next tile lies at or below the diagonal of the workgroup's
  // first row (tiles below kclean) masks nothing, and its tile kt + 2 exists:
  // it runs as one straight block, with no per-wavefront test and no mask
  // block between its P.V products and the barrier.
  const int kclean = (past + t0 + 1) / BN;
  const int nclean = min(kclean - 1, ntiles - 2);
  auto clean_step = [&](auto jc, int kt, f32x16 (&Scur)[QB][KB], f32x16 (&Snext)[QB][KB]) {
    constexpr int J = decltype(jc)::value;
    using SlotPv = std::integral_constant<int, J % NSLOT>;
    using SlotS = std::integral_constant<int, (J + 1) % NSLOT>;
    using SlotLd = std::integral_constant<int, (J + 2) % NSLOT>;
    load_tile(kt + 2, SlotLd{});
    bf16x8 pf[QB][KSTEPS];
    scores(SlotS{}, Snext);
    probs(Scur, pf);
    pv(SlotPv{}, pf);
    if constexpr (!kBounded) {
      float mx[QB];
      tile_max(Snext, mx);
      raise_max(mx);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Tiles 0 and 1 stream into slots 0 and 1 while Q is loaded, normalised,
  // rotated and staged (in slot 2 and a region of its own).
  load_tile(0, C0{});
  if (ntiles > 1) load_tile(1, C1{});
  q_issue();
  if constexpr (kBounded) {
    if (!scores_bounded(wmax, past, bound_limit)) {
      __builtin_amdgcn_s_waitcnt(0);  // leave with no load outstanding
      if (single_path) {
        // The weights break the caller's bound that launched this kernel
        // alone: no kernel computes these rows, so they are written as NaN
        // (bf16 0x7fc0), whole 16-byte pieces, D/8 lanes per row.
        constexpr int LPR = D / 8, RPI = 64 / LPR;
        const u32x4 nan8 = {0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          for (int r = lane / LPR; r < 32; r += RPI) {
            const int tok = qfirst[qb] + r;
            if (tok < seqlen)
              *reinterpret_cast<u32x4*>(out + (static_cast<size_t>(cu0 + tok) * num_q_heads + qhead[qb]) * D +
                                        8 * (lane % LPR)) = nan8;
          }
      }
      return;
    }
  }
  stamps.now(QKRA_STAMP_ISSUED);
  q_finish();
  stamps.now(QKRA_STAMP_Q_READY);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // tiles 0 and 1 are in LDS
  __syncthreads();
  f32x16 sA[QB][KB], sB[QB][KB];
  scores(C0{}, sA);
  tile_mask(0, sA);
  if constexpr (!kBounded) {
    float mx[QB];
    tile_max(sA, mx);
    raise_max(mx);
  }
  // Unrolled by 2*NSLOT: the score buffers alternate every step and the LDS
  // slots cycle every NSLOT steps.
  static_assert(NSLOT == 3, "the unroll below assumes a ring of three slots");
  stamps.now(QKRA_STAMP_LOOP);
  // Whole groups of six clean steps first, then the general loop from phase 0
  // (a loop that chose between the two step kinds at every step spilled).
  int kt0 = 0;
  const int nclean6 = nclean >= 6 ? nclean - nclean % 6 : 0;
  for (; kt0 < nclean6; kt0 += 6) {
    clean_step(std::integral_constant<int, 0>{}, kt0, sA, sB);
    if (kt0 == 0) stamps.now(QKRA_STAMP_FIRST_STEP);
    clean_step(std::integral_constant<int, 1>{}, kt0 + 1, sB, sA);
    clean_step(std::integral_constant<int, 2>{}, kt0 + 2, sA, sB);
    clean_step(std::integral_constant<int, 3>{}, kt0 + 3, sB, sA);
    clean_step(std::integral_constant<int, 4>{}, kt0 + 4, sA, sB);
    clean_step(std::integral_constant<int, 5>{}, kt0 + 5, sB, sA);
  }
  for (int kt = kt0; kt < ntiles; kt += 6) {
    step(std::integral_constant<int, 0>{}, kt, sA, sB);
    if (kt == 0) stamps.now(QKRA_STAMP_FIRST_STEP);
    if (kt + 1 >= ntiles) break;
    step(std::integral_constant<int, 1>{}, kt + 1, sB, sA);
    if (kt + 2 >= ntiles) break;
    step(std::integral_constant<int, 2>{}, kt + 2, sA, sB);
    if (kt + 3 >= ntiles) break;
    step(std::integral_constant<int, 3>{}, kt + 3, sB, sA);
    if (kt + 4 >= ntiles) break;
    step(std::integral_constant<int, 4>{}, kt + 4, sA, sB);
    if (kt + 5 >= ntiles) break;
    step(std::integral_constant<int, 5>{}, kt + 5, sB, sA);
  }
  stamps.now(QKRA_STAMP_LOOP_END);

  // ---- normalise and store.  A lane holds query l32 and d = 32db + 8(j/4) +
  // 4hi + j%4, so storing from registers would write 16 bytes into each of 32
  // output rows per instruction.  Instead each wavefront writes its 32 x D
  // tile row-major into its own LDS region (the K/V slots are free: the last
  // step ended with a barrier) and stores whole rows from there, 16 lanes
  // per row, 16 bytes each.
  static_assert(NWAVES == 8 && 2 * 32 * EST <= BN * KST && 2 * 32 * EST <= BN * VRS,
                "two output tiles fit in each slot array");
  bf16* stile = region(wave / 2) + (wave % 2) * 32 * EST;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = lsum[qb][0];
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const f32x16& a = acc[qb][db];
        const u32x2 w = {pack_bf16x2(a[4 * jq] * inv, a[4 * jq + 1] * inv),
                         pack_bf16x2(a[4 * jq + 2] * inv, a[4 * jq + 3] * inv)};
        *reinterpret_cast<u32x2*>(&stile[l32 * EST + 32 * db + 8 * jq + 4 * hi]) = w;
      }
    // Lane L then stores bytes 16(L%16) .. +15 of row L/16 + 4p, p = 0 .. 7.
    constexpr int LPR = D / 8;        // lanes per row
    constexpr int RPI = 64 / LPR;     // rows per store instruction
    const int r0 = lane / LPR, c = lane % LPR;
#pragma unroll
    for (int p = 0; p < 32 / RPI; ++p) {
      const int r = r0 + RPI * p;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&stile[r * EST + 8 * c]);
      const int tok = qfirst[qb] + r;
      if (tok < seqlen)
        *reinterpret_cast<u32x4*>(out + (static_cast<size_t>(cu0 + tok) * num_q_heads + qhead[qb]) * D + 8 * c) = v;
    }
  }
  stamps.now(QKRA_STAMP_END);
  stamps.where(ntiles, logical);
}

int launch_flags(const PrefillAttnArgs& a) {
  return (a.single_path ? kFlagSinglePath : 0) | (a.tile_major ? kFlagTileMajor : 0);
}

template <int D, int HC, bool kBounded, bool kPaged>
hipError_t launch_typed(const PrefillAttnArgs& a, hipStream_t stream) {
  constexpr int TM = 32 * (8 / HC);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks_per_kv = group / HC;
  const int tiles = (a.max_seqlen + TM - 1) / TM;
  const long long items = static_cast<long long>(a.num_kv_heads) * chunks_per_kv * a.num_seqs * tiles;
  if (items <= 0) return hipSuccess;
  const long long grid = (items + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float bound_limit = prefill_unshifted_limit(D, a.scale_log2);
  launch_kernel((prefill_mfma_kernel<D, HC, kBounded, 0, kPaged>), dim3(static_cast<unsigned>(grid)), dim3(NTHREADS), 0, stream,
                     static_cast<const bf16*>(a.qkv), static_cast<const bf16*>(a.q_norm_weight),
                     static_cast<const bf16*>(a.k_norm_weight), a.rope_table,
                     static_cast<const bf16*>(a.k_cache),
                     static_cast<const bf16*>(a.v_cache), a.cu_seqlens, a.past_lens, static_cast<bf16*>(a.out),
                     a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_seqs, tiles, chunks_per_kv,
                     static_cast<int>(items), a.rms_eps, a.scale_log2, bound_limit, DecodeRole{}, a.paged,
                     launch_flags(a));
  return hipGetLastError();
}

template <int D, bool kBounded, bool kPaged>
hipError_t launch_grouped(const PrefillAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 8 == 0) return launch_typed<D, 8, kBounded, kPaged>(a, stream);
  if (group % 4 == 0) return launch_typed<D, 4, kBounded, kPaged>(a, stream);
  if (group % 2 == 0) return launch_typed<D, 2, kBounded, kPaged>(a, stream);
  return launch_typed<D, 1, kBounded, kPaged>(a, stream);
}

template <int D, bool kBounded>
hipError_t launch_dim(const PrefillAttnArgs& a, hipStream_t stream) {
  return a.paged.table ? launch_grouped<D, kBounded, true>(a, stream) : launch_grouped<D, kBounded, false>(a, stream);
}

}  // namespace

namespace {

template <int D, int G>
hipError_t launch_fused_typed(const PrefillAttnArgs& a, const DecodeAttnArgs& d, hipStream_t stream) {
  constexpr int HC = G < 8 ? G : 8;
  constexpr int TM = 32 * (8 / HC);
  const int tiles = (a.max_seqlen + TM - 1) / TM;
  const int chunks_per_kv = G / HC;
  const long long items = static_cast<long long>(a.num_kv_heads) * chunks_per_kv * a.num_seqs * tiles;
  const long long grid = kFusedDecodeWgs + (items + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float bound_limit = prefill_unshifted_limit(D, a.scale_log2);
  const DecodeRole dec{static_cast<const bf16*>(d.q), static_cast<const bf16*>(d.k_cache),
                       static_cast<const bf16*>(d.v_cache), d.cache_lens, d.plan, d.partials, d.cache_capacity,
                       1, d.num_units, kFusedDecodeWgs};
  launch_kernel((prefill_mfma_kernel<D, HC, true, G>), dim3(static_cast<unsigned>(grid)), dim3(NTHREADS), 0,
                     stream, static_cast<const bf16*>(a.qkv), static_cast<const bf16*>(a.q_norm_weight),
                     static_cast<const bf16*>(a.k_norm_weight), a.rope_table, static_cast<const bf16*>(a.k_cache),
                     static_cast<const bf16*>(a.v_cache), a.cu_seqlens, a.past_lens, static_cast<bf16*>(a.out),
                     a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_seqs, tiles, chunks_per_kv,
                     static_cast<int>(items), a.rms_eps, a.scale_log2, bound_limit, dec, PagedTable{},
                     launch_flags(a));
  return hipGetLastError();
}

template <int D>
hipError_t launch_fused_dim(const PrefillAttnArgs& a, const DecodeAttnArgs& d, hipStream_t stream) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_fused_typed<D, 1>(a, d, stream);
    case 2: return launch_fused_typed<D, 2>(a, d, stream);
    case 4: return launch_fused_typed<D, 4>(a, d, stream);
    case 8: return launch_fused_typed<D, 8>(a, d, stream);
    case 16: return launch_fused_typed<D, 16>(a, d, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

float prefill_unshifted_limit(int head_dim, float scale_log2) {
  return BOUND_LOG2 / (1.02f * static_cast<float>(head_dim) * scale_log2);
}

bool fused_step_supported(int head_dim, int group) {
  return (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8 || group == 16);
}

hipError_t launch_fused_step(const PrefillAttnArgs& a, const DecodeAttnArgs& d, hipStream_t stream) {
  if (a.head_dim == 128) return launch_fused_dim<128>(a, d, stream);
  if (a.head_dim == 64) return launch_fused_dim<64>(a, d, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, bool unshifted, hipStream_t stream) {
  if (a.head_dim == 128) return unshifted ? launch_dim<128, true>(a, stream) : launch_dim<128, false>(a, stream);
  if (a.head_dim == 64) return unshifted ? launch_dim<64, true>(a, stream) : launch_dim<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra

#ifdef QKRA_PHASE_STAMPS
extern "C" {

QKRA_STAMPS_API size_t qkra_phase_stamps_bytes(void) { return sizeof(qkra::g_phase_stamps); }

QKRA_STAMPS_API int32_t qkra_phase_stamps_read(void* dst, size_t bytes) {
  if (dst == nullptr) return 1;
  const size_t n = bytes < sizeof(qkra::g_phase_stamps) ? bytes : sizeof(qkra::g_phase_stamps);
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(qkra::g_phase_stamps), n, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0 : 6;
}

QKRA_STAMPS_API int32_t qkra_phase_stamps_clear(void* hip_stream) {
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(qkra::g_phase_stamps)) != hipSuccess) return 6;
  return hipMemsetAsync(ptr, 0, sizeof(qkra::g_phase_stamps), static_cast<hipStream_t>(hip_stream)) == hipSuccess
             ? 0 : 6;
}

}  // extern "C"
#endif
