// Kernels 3p/3a/3b for bf16: decode attention on the matrix cores with an
// evenly balanced split of the cached keys (one new token per request).
//
// The new token's query attends over cache slots 0..L_b of its request, the
// L_b cached entries plus its own K/V that kernel 1 has just appended (concept
// chapter "Chapter 3 Forward Pass and Generation", section 4.2; jq-wei
// "transformer basics", "Prefill vs Decode": one more row of the causal
// triangle).  Query head h reads KV head floor(h / G).
//
// Decode reads every cached K/V byte once and does ~G multiply-adds per byte,
// so it is bound by HBM bandwidth; the design keeps every wavefront streaming:
//  * Work: a unit is (request b, KV head g, chunk of GW query heads of g); it
//    covers ceil(n_b / 32) steps of 32 keys, n_b = L_b + 1.  All units' steps
//    are laid end to end and cut into equal contiguous ranges, one per
//    wavefront of a persistent grid, so every wavefront streams the same
//    number of bytes whatever the length mix.  A wavefront whose range crosses
//    unit boundaries carries its load pipeline across them and writes one
//    partial (m, l, o) per unit portion; 3b merges a unit's portions.
//  * The plan (decode_plan.h: the step prefix over units, the range length and
//    each wavefront's first unit) is built on the device from the cache
//    lengths, by one extra block of kernel 1's decode launch.
//  * Per 32-key step a wavefront loads its K and V rows lane-linearly (1 KB of
//    contiguous rows per instruction, non-temporal: read once) into registers,
//    while it computes the previous step from LDS; the rows then go to padded
//    per-wavefront LDS tiles.
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with the GW
//    query heads as the 16 columns (unused columns are zero).  The score
//    accumulators hold, for lane l, query l%16 and keys 4g+r and 16+4g+r
//    (g = l/16, r = 0..3): exactly the k-slots of a 32-key B operand, so P^T
//    needs no lane exchange.  V^T comes from ds_read_b64_tr_b16, whose 16-lane
//    transpose hands lane i four keys of one d column.
//  * Online softmax per query in the log2 domain; the running max is only
//    raised when a score exceeds it by more than 2^8, which keeps the
//    arithmetic exact (every p and the sum use the same stale max) and makes
//    rescaling rare.
//  * 3b merges the portions of a (request, head) in a fixed order with the
//    log-sum-exp rule m = max m_s, l = sum l_s 2^(m_s - m),
//    o = sum o_s 2^(m_s - m) / l.  Deterministic, no atomics.

#include "device_common.h"
#include "launch.h"

#include "decode_body.h"

namespace qkra {
namespace {

// ---- 3a: one wavefront per range of steps; 4 independent wavefronts per workgroup.
// kPaged: the caches are pools read through `paged`.
template <int D, int GW, bool kPaged>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_cache, const bf16* __restrict__ v_cache,
    const int32_t* __restrict__ cache_lens, const int32_t* __restrict__ plan, float* __restrict__ partials,
    int num_q_heads, int num_kv_heads, int cache_capacity, int chunks_per_kv, int num_units, float scale_log2,
    PagedTable paged) {
  constexpr int TILE = kDecodeStepKeys * (D + 8);
  __shared__ __attribute__((aligned(16))) bf16 lds[4][2 * TILE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  dbody::decode_wave<D, GW, kPaged>(lds[wave], lds[wave] + TILE, blockIdx.x * 4 + wave, q, k_cache, v_cache,
                                    cache_lens, plan, partials, num_q_heads, num_kv_heads, cache_capacity,
                                    chunks_per_kv, num_units, scale_log2, paged);
}

// ---- 3b: merge the portions of one (request, head); one wavefront each.
template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ partials,
                                                            const int32_t* __restrict__ plan, bf16* __restrict__ out,
                                                            int num_q_heads, int num_kv_heads, int chunks_per_kv,
                                                            int gw) {
  constexpr int PER_LANE = D / 64;
  constexpr int PREC = D + 4;
  const int bh = blockIdx.x;
  const int b = bh / num_q_heads, h = bh % num_q_heads;
  const int group = num_q_heads / num_kv_heads;
  const int g = h / group, within = h % group;
  const int i = (b * num_kv_heads + g) * chunks_per_kv + within / gw;
  const int hh = within % gw;
  const int per = plan[1];
  const int32_t* S0 = plan + 2;
  const int s_first = S0[i] / per, s_last = (S0[i + 1] - 1) / per;
  const int lane = threadIdx.x;
  auto rec = [&](int s) { return partials + (static_cast<size_t>(i + s) * gw + hh) * PREC; };
  // Portions are read CH at a time, every load of a group issued before any
  // is used (one memory latency per group instead of two per portion).  The
  // merge keeps the portion order: a group's max first, then l and o scaled
  // by 2^(m_s - m) and added in order; a later group first rescales what came
  // before.  With at most CH portions this is exactly the two-pass merge
  // (max over all, then the ordered sums).
  constexpr int CH = 8;
  float m = kNegInf, l = 0.f, acc[PER_LANE];
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) acc[e] = 0.f;
  for (int s0 = s_first; s0 <= s_last; s0 += CH) {
    float ms[CH], ls[CH], os[CH][PER_LANE];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool live = s0 + j <= s_last;
      const float* r = rec(live ? s0 + j : s_first);
      ms[j] = live ? r[0] : kNegInf;
      ls[j] = live ? r[1] : 0.f;
#pragma unroll
      for (int e = 0; e < PER_LANE; ++e) os[j][e] = live ? r[4 + lane + 64 * e] : 0.f;
    }
    float mg = m;
#pragma unroll
    for (int j = 0; j < CH; ++j) mg = fmaxf(mg, ms[j]);
    if (s0 != s_first) {
      const float alpha = fast_exp2(m - mg);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < PER_LANE; ++e) acc[e] *= alpha;
    }
    m = mg;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (s0 + j > s_last) break;
      const float wgt = fast_exp2(ms[j] - m);
      l += ls[j] * wgt;
#pragma unroll
      for (int e = 0; e < PER_LANE; ++e) acc[e] += os[j][e] * wgt;
    }
  }
  const float inv = 1.0f / l;
  bf16* dst = out + static_cast<size_t>(bh) * D;
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) dst[lane + 64 * e] = static_cast<bf16>(acc[e] * inv);
}

template <int D, int GW, bool kPaged>
hipError_t launch_mfma_paged(const DecodeAttnArgs& a, hipStream_t stream) {
  const int chunks_per_kv = (a.num_q_heads / a.num_kv_heads) / GW;
  launch_kernel((decode_mfma_kernel<D, GW, kPaged>), dim3(kDecodeWaves / 4), dim3(256), 0, stream,
                static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k_cache),
                static_cast<const bf16*>(a.v_cache), a.cache_lens, a.plan, a.partials, a.num_q_heads,
                a.num_kv_heads, a.cache_capacity, chunks_per_kv, a.num_units, a.scale_log2, a.paged);
  return hipGetLastError();
}

template <int D, int GW>
hipError_t launch_mfma_typed(const DecodeAttnArgs& a, hipStream_t stream) {
  return a.paged.table ? launch_mfma_paged<D, GW, true>(a, stream) : launch_mfma_paged<D, GW, false>(a, stream);
}

template <int D>
hipError_t launch_mfma_dim(const DecodeAttnArgs& a, hipStream_t stream) {
  switch (a.heads_per_wave) {
    case 16: return launch_mfma_typed<D, 16>(a, stream);
    case 15: return launch_mfma_typed<D, 15>(a, stream);
    case 14: return launch_mfma_typed<D, 14>(a, stream);
    case 13: return launch_mfma_typed<D, 13>(a, stream);
    case 12: return launch_mfma_typed<D, 12>(a, stream);
    case 11: return launch_mfma_typed<D, 11>(a, stream);
    case 10: return launch_mfma_typed<D, 10>(a, stream);
    case 9: return launch_mfma_typed<D, 9>(a, stream);
    case 8: return launch_mfma_typed<D, 8>(a, stream);
    case 7: return launch_mfma_typed<D, 7>(a, stream);
    case 6: return launch_mfma_typed<D, 6>(a, stream);
    case 5: return launch_mfma_typed<D, 5>(a, stream);
    case 4: return launch_mfma_typed<D, 4>(a, stream);
    case 3: return launch_mfma_typed<D, 3>(a, stream);
    case 2: return launch_mfma_typed<D, 2>(a, stream);
    case 1: return launch_mfma_typed<D, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeAttnArgs& a, hipStream_t stream) {
  if (a.num_units <= 0) return hipSuccess;
  if (a.head_dim == 128) return launch_mfma_dim<128>(a, stream);
  if (a.head_dim == 64) return launch_mfma_dim<64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma_combine(const DecodeAttnArgs& a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.num_seqs) * a.num_q_heads;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int chunks_per_kv = (a.num_q_heads / a.num_kv_heads) / a.heads_per_wave;
  if (a.head_dim == 128) {
    launch_kernel(decode_combine_kernel<128>, dim3(static_cast<unsigned>(items)), dim3(64), 0, stream,
                       a.partials, a.plan, static_cast<bf16*>(a.out), a.num_q_heads, a.num_kv_heads, chunks_per_kv,
                       a.heads_per_wave);
  } else if (a.head_dim == 64) {
    launch_kernel(decode_combine_kernel<64>, dim3(static_cast<unsigned>(items)), dim3(64), 0, stream,
                       a.partials, a.plan, static_cast<bf16*>(a.out), a.num_q_heads, a.num_kv_heads, chunks_per_kv,
                       a.heads_per_wave);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qkra
