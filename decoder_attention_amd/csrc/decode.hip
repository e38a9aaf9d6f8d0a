// Kernels 3a/3b for fp32: decode attention, one new token per request, split
// over the cached keys and merged with a log-sum-exp combine.  (bf16 runs on
// the matrix cores with an evenly balanced split; see decode_mfma.hip.)
//
// The new token's query attends over cache slots 0..L_b of its request, the
// L_b cached entries plus its own K/V that kernel 1 has just appended (concept
// chapter "Chapter 3 Forward Pass and Generation", section 4.2; jq-wei
// "transformer basics", "Prefill vs Decode": one more row of the causal
// triangle).  Query head h reads KV head floor(h / G).
//
//  * 3a: one workgroup per (request, KV-head chunk, split of 1024 keys), four
//    wavefronts of 256 keys each; a wavefront serves the GW (<= 2) query heads
//    of its chunk that share the KV head, so every K/V byte is fetched once
//    for all of them.
//  * Eight lanes share one key row: each lane owns D/8 of it and issues
//    16-byte loads, the eight lanes of a key reading 128 contiguous bytes per
//    instruction; 8 keys per wavefront step, with three further steps' loads
//    in flight (a ring of four register buffers) while one is consumed.  K/V
//    are read exactly once, so the loads are non-temporal.
//  * Scores by fp32 FMA, summed over the 8 lanes of a key with DPP permutes.
//    Each lane octet keeps its own online-softmax state (running max, sum,
//    partial output); the running max is only raised when a score exceeds it
//    by more than 2^8, which keeps the arithmetic exact (every p and the sum
//    use the same stale max) and makes rescaling rare.
//  * The octets, then the four wavefronts (through LDS), are merged with the
//    log-sum-exp rule; each workgroup writes (m, l, o[D]) for its split.  3b
//    merges the splits of a (request, head) in a fixed order: m = max m_s,
//    l = sum l_s 2^(m_s - m), o = sum o_s 2^(m_s - m) / l.  Deterministic, no
//    atomics.

#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace {

constexpr int SPLIT = kDecodeKeysPerSplit;
constexpr float TAU = 8.0f;  // lazy-rescale threshold (log2 units)

// Partial dot product of 16 bytes (four fp32) of q and k.
__device__ __forceinline__ float dot16(u32x4 q, u32x4 k, float acc) {
  acc += __uint_as_float(q.x) * __uint_as_float(k.x);
  acc += __uint_as_float(q.y) * __uint_as_float(k.y);
  acc += __uint_as_float(q.z) * __uint_as_float(k.z);
  acc += __uint_as_float(q.w) * __uint_as_float(k.w);
  return acc;
}

// acc[hh][off + e] += p[hh] * v[e] for the four fp32 of 16 bytes of v, all
// heads at once.
template <int GW, int EPL>
__device__ __forceinline__ void axpy16_heads(float (&acc)[GW][EPL], int off, const float (&p)[GW], u32x4 v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float f = __uint_as_float(v[i]);
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) acc[hh][off + i] += p[hh] * f;
  }
}

template <int D, int GW>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const float* __restrict__ q, const float* __restrict__ k_cache, const float* __restrict__ v_cache,
    const int32_t* __restrict__ cache_lens, float* __restrict__ partials, int num_q_heads, int num_kv_heads,
    int cache_capacity, int num_splits, int chunks_per_kv, float scale_log2, PagedTable paged) {
  typedef float T;
  constexpr int ES = sizeof(T);
  constexpr int E16 = 16 / ES;          // elements per 16-byte load
  constexpr int LPK = 8;                // lanes per key row
  constexpr int KPS = 64 / LPK;         // keys per wavefront step
  constexpr int EPL = D / LPK;          // elements per lane per key row
  constexpr int NL = EPL / E16;         // 16-byte loads per lane per key row
  constexpr int KPW = SPLIT / 4;        // keys per wavefront

  __shared__ float s_part[4][GW][D + 2];

  const int item = blockIdx.x;
  const int split = item % num_splits;
  const int rest = item / num_splits;
  const int nchunks = num_kv_heads * chunks_per_kv;
  const int hc = rest % nchunks;
  const int b = rest / nchunks;
  const int nkeys = min(cache_lens[b] + 1, cache_capacity);  // clamp: never read past the cache
  if (split * SPLIT >= nkeys) return;                          // whole workgroup idle (uniform)
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int ks = split * SPLIT + wave * KPW;
  const int ke = min(nkeys, ks + KPW);
  const int group = num_q_heads / num_kv_heads;
  const int g = hc / chunks_per_kv;
  const int h0 = g * group + (hc % chunks_per_kv) * GW;
  const int kl = lane / LPK;  // key slot within a step
  const int c = lane % LPK;   // which 16-byte column of each 128-byte row segment

  // The 8 lanes of a key read 128 contiguous bytes per load instruction.
  auto elem_off = [&](int i) { return (128 * i + 16 * c) / ES; };

  u32x4 qr[GW][NL];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh)
#pragma unroll
    for (int i = 0; i < NL; ++i)
      qr[hh][i] = *reinterpret_cast<const u32x4*>(q + (static_cast<size_t>(b) * num_q_heads + h0 + hh) * D + elem_off(i));

  // Per key slot (lane octet) online-softmax state: each octet runs its own
  // max over the keys it sees; the octets are merged once at the end.
  float acc[GW][EPL];
  float m_run[GW], l_run[GW];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    m_run[hh] = kNegInf;
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
  }

  const size_t head_off = (static_cast<size_t>(b) * num_kv_heads + g) * cache_capacity * D;

  // Four register buffers in a ring: three steps' loads stay in flight while
  // the fourth step is consumed.  Loads are unconditional (rows past the
  // split's end are clamped to its last row, a valid row) so that the only
  // waits are the in-order ones on the buffer about to be consumed; the
  // clamped duplicates are masked out of the softmax by `ok`.
  u32x4 kr0[NL], vr0[NL], kr1[NL], vr1[NL], kr2[NL], vr2[NL], kr3[NL], vr3[NL];
  auto load = [&](u32x4 (&kr)[NL], u32x4 (&vr)[NL], int base) {
    const int key = min(base + kl, ke - 1);
    // A paged cache: the key's row through the block table.
    const size_t row = paged.table ? paged_row(paged, b, g, key, num_kv_heads, D) : head_off + static_cast<size_t>(key) * D;
    const T* kp = k_cache + row;
    const T* vp = v_cache + row;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + elem_off(i)));
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + elem_off(i)));
    }
  };
  // One step: the GW heads run as independent instruction chains (no branch
  // between them), so their dependent dot/reduce/exp sequences interleave.
  auto consume = [&](const u32x4 (&kr)[NL], const u32x4 (&vr)[NL], int base) {
    const bool ok = base + kl < ke;
    float s[GW][2];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) s[hh][0] = s[hh][1] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) s[hh][i & 1] = dot16(qr[hh][i], kr[i], s[hh][i & 1]);
    float x[GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) x[hh] = s[hh][0] + s[hh][1];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) x[hh] += dpp_f32<0xB1>(x[hh]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) x[hh] += dpp_f32<0x4E>(x[hh]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) x[hh] += dpp_f32<0x141>(x[hh]);  // row_half_mirror
    bool need = false;
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      x[hh] *= scale_log2;
      need |= ok && x[hh] > m_run[hh] + TAU;
    }
    if (__any(need)) {  // rare after the first key of each octet
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        // alpha stays 1 where this head's max does not rise (the octet may
        // still hold m = -inf, and 2^(-inf - -inf) would be NaN).
        const bool up = ok && x[hh] > m_run[hh] + TAU;
        const float m_new = up ? x[hh] : m_run[hh];
        const float alpha = up ? fast_exp2(m_run[hh] - m_new) : 1.0f;
        l_run[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
        m_run[hh] = m_new;
      }
    }
    float p[GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      p[hh] = ok ? fast_exp2(x[hh] - m_run[hh]) : 0.f;
      l_run[hh] += p[hh];
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) axpy16_heads<GW, EPL>(acc, i * E16, p, vr[i]);
  };

  if (ks < ke) {
    // Straight-line ring: every load and consume is issued unconditionally
    // (trailing steps read clamped rows and contribute p = 0), which keeps the
    // waits exact: consuming buffer j waits only for buffer j's loads.
    const int nquads = (ke - ks + 4 * KPS - 1) / (4 * KPS);
    // The scheduling barriers keep each refill ahead of the next consume (the
    // scheduler would otherwise sink the loads and shorten the ring).
    __builtin_amdgcn_sched_barrier(0);
    load(kr0, vr0, ks);
    __builtin_amdgcn_sched_barrier(0);
    load(kr1, vr1, ks + KPS);
    __builtin_amdgcn_sched_barrier(0);
    load(kr2, vr2, ks + 2 * KPS);
    for (int it = 0, base = ks; it < nquads; ++it, base += 4 * KPS) {
      load(kr3, vr3, base + 3 * KPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(kr0, vr0, base);
      load(kr0, vr0, base + 4 * KPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(kr1, vr1, base + KPS);
      load(kr1, vr1, base + 5 * KPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(kr2, vr2, base + 2 * KPS);
      load(kr2, vr2, base + 6 * KPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(kr3, vr3, base + 3 * KPS);
    }
  }

  // Merge the 8 octets of the wavefront (lanes with equal c hold the same d).
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    float mw = m_run[hh];
    mw = fmaxf(mw, xor_shuffle(mw, 8));
    mw = fmaxf(mw, xor_shuffle(mw, 16));
    mw = fmaxf(mw, xor_shuffle(mw, 32));
    const float sc = m_run[hh] == kNegInf ? 0.f : fast_exp2(m_run[hh] - mw);
    float l = l_run[hh] * sc;
    l += xor_shuffle(l, 8);
    l += xor_shuffle(l, 16);
    l += xor_shuffle(l, 32);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[hh][e] * sc;
      v += xor_shuffle(v, 8);
      v += xor_shuffle(v, 16);
      v += xor_shuffle(v, 32);
      acc[hh][e] = v;
    }
    if (lane == 0) {
      s_part[wave][hh][0] = ks < ke ? mw : kNegInf;
      s_part[wave][hh][1] = l;
    }
    if (kl == 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < E16; ++e) s_part[wave][hh][2 + elem_off(i) + e] = acc[hh][i * E16 + e];
    }
  }
  __syncthreads();

  // Merge the four wavefronts and write one partial per (request, head, split).
  for (int idx = threadIdx.x; idx < GW * D; idx += blockDim.x) {
    const int hh = idx / D, d = idx % D;
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, s_part[w][hh][0]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = s_part[w][hh][0];
      const float sc = mw == kNegInf ? 0.f : fast_exp2(mw - m);
      o += s_part[w][hh][2 + d] * sc;
      l += s_part[w][hh][1] * sc;
    }
    float* dst = partials + ((static_cast<size_t>(b) * num_q_heads + h0 + hh) * num_splits + split) * (D + 2);
    dst[2 + d] = o;
    if (d == 0) {
      dst[0] = m;
      dst[1] = l;
    }
  }
}

template <int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ partials,
                                                            const int32_t* __restrict__ cache_lens,
                                                            float* __restrict__ out, int num_q_heads, int num_splits) {
  constexpr int PER = D / 64;
  const int bh = blockIdx.x;
  const int b = bh / num_q_heads;
  const int lane = threadIdx.x;
  const int ns = min((cache_lens[b] + 1 + SPLIT - 1) / SPLIT, num_splits);
  const float* src = partials + static_cast<size_t>(bh) * num_splits * (D + 2);
  float m = kNegInf;
  for (int s = 0; s < ns; ++s) m = fmaxf(m, src[static_cast<size_t>(s) * (D + 2)]);
  float l = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float* p = src + static_cast<size_t>(s) * (D + 2);
    const float w = fast_exp2(p[0] - m);
    l += p[1] * w;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += p[2 + lane + 64 * e] * w;
  }
  const float inv = 1.0f / l;
  float* dst = out + static_cast<size_t>(bh) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[lane + 64 * e] = o[e] * inv;
}

template <int D, int GW>
hipError_t launch_split_typed(const DecodeAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks_per_kv = group / GW;
  const long long items = static_cast<long long>(a.num_seqs) * a.num_kv_heads * chunks_per_kv * a.num_splits;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_kernel((decode_split_kernel<D, GW>), dim3(static_cast<unsigned>(items)), dim3(256), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k_cache),
                     static_cast<const float*>(a.v_cache), a.cache_lens, a.partials, a.num_q_heads, a.num_kv_heads,
                     a.cache_capacity, a.num_splits, chunks_per_kv, a.scale_log2, a.paged);
  return hipGetLastError();
}

// Two heads per wavefront at most: four fp32 heads would not fit in registers.
template <int D>
hipError_t launch_split_dim(const DecodeAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 2 == 0) return launch_split_typed<D, 2>(a, stream);
  return launch_split_typed<D, 1>(a, stream);
}

template <int D>
hipError_t launch_combine_typed(const DecodeAttnArgs& a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.num_seqs) * a.num_q_heads;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_kernel((decode_combine_kernel<D>), dim3(static_cast<unsigned>(items)), dim3(64), 0, stream,
                     a.partials, a.cache_lens, static_cast<float*>(a.out), a.num_q_heads, a.num_splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeAttnArgs& a, hipStream_t stream) {
  if (a.dtype != 1) return hipErrorInvalidValue;  // fp32 only
  if (a.head_dim == 128) return launch_split_dim<128>(a, stream);
  if (a.head_dim == 64) return launch_split_dim<64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeAttnArgs& a, hipStream_t stream) {
  if (a.dtype != 1) return hipErrorInvalidValue;
  if (a.head_dim == 128) return launch_combine_typed<128>(a, stream);
  if (a.head_dim == 64) return launch_combine_typed<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra
