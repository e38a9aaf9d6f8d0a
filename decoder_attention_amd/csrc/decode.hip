// Kernels 3a/3b: decode attention, one new token per request, split over the
// cached keys and merged with a log-sum-exp combine.
//
// The new token's query attends over cache slots 0..L_b of its request, the
// L_b cached entries plus its own K/V that kernel 1 has just appended (concept
// chapter "Chapter 3 Forward Pass and Generation", section 4.2; jq-wei
// "transformer basics", "Prefill vs Decode": one more row of the causal
// triangle).  Query head h reads KV head floor(h / G).
//
// Decode reads every cached K/V byte once and does only ~G multiply-adds per
// byte, so it is bound by HBM bandwidth.  The kernel is laid out for that:
//  * 3a: one workgroup per (request, KV head, split of 1024 keys), four
//    wavefronts of 256 keys each; a wavefront serves the GW query heads of its
//    group that share the KV head (GW = 4 for Qwen3's G = 4), so every K/V
//    byte is fetched once for all of them.
//  * Eight lanes share one key row: each lane owns D/8 of it and issues
//    16-byte loads, the eight lanes of a key reading 128 contiguous bytes per
//    instruction; 8 keys per wavefront step, the next step's loads in flight
//    while the current one is consumed.  Few registers per lane, so several
//    wavefronts per SIMD hide HBM latency.
//  * Scores via v_dot2_f32_bf16 (bf16) or fp32 FMA, summed over the 8 lanes
//    of a key with DPP permutes.  Each lane octet keeps its own online-softmax
//    state (running max, sum, partial output), so no cross-octet traffic is
//    needed per step; the running max is only raised when a score exceeds it
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
constexpr int CHUNK = 16;

template <typename T> __device__ __forceinline__ void store_elem(T* p, float v);
template <> __device__ __forceinline__ void store_elem<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_elem<bf16>(bf16* p, float v) { *p = static_cast<bf16>(v); }

// Partial dot product of 16 bytes of q and k.
__device__ __forceinline__ float dot16(u32x4 q, u32x4 k, float acc, bf16*) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), acc, false);
  return acc;
}
__device__ __forceinline__ float dot16(u32x4 q, u32x4 k, float acc, float*) {
  acc += __uint_as_float(q.x) * __uint_as_float(k.x);
  acc += __uint_as_float(q.y) * __uint_as_float(k.y);
  acc += __uint_as_float(q.z) * __uint_as_float(k.z);
  acc += __uint_as_float(q.w) * __uint_as_float(k.w);
  return acc;
}

// acc[0..n) += p * v for the elements of 16 bytes of v.
__device__ __forceinline__ void axpy16(float* acc, float p, u32x4 v, bf16*) {
  const u32x4 w = v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += p * bf16_lo_to_f32(w[i]);
    acc[2 * i + 1] += p * bf16_hi_to_f32(w[i]);
  }
}
__device__ __forceinline__ void axpy16(float* acc, float p, u32x4 v, float*) {
  acc[0] += p * __uint_as_float(v.x);
  acc[1] += p * __uint_as_float(v.y);
  acc[2] += p * __uint_as_float(v.z);
  acc[3] += p * __uint_as_float(v.w);
}

// Sum over the 8 lanes of an aligned lane octet (xor 1, xor 2, then the
// mirrored half-row), all through DPP lane permutes.
__device__ __forceinline__ float octet_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  return x;
}

template <typename T, int D, int GW>
__global__ __launch_bounds__(256, 2) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ cache_lens, float* __restrict__ partials, int num_q_heads, int num_kv_heads,
    int cache_capacity, int num_splits, int chunks_per_kv, float scale_log2) {
  constexpr int ES = sizeof(T);
  constexpr int E16 = 16 / ES;          // elements per 16-byte load
  constexpr int LPK = 8;                // lanes per key row
  constexpr int KPS = 64 / LPK;         // keys per wavefront step
  constexpr int EPL = D / LPK;          // elements per lane per key row
  constexpr int NL = EPL / E16;         // 16-byte loads per lane per key row
  constexpr int KPW = SPLIT / 4;        // keys per wavefront
  constexpr float TAU = 8.0f;           // rescale only when the max grows by more than 2^TAU

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
  const T* kb = k_cache + head_off;
  const T* vb = v_cache + head_off;

  u32x4 k0r[NL], v0r[NL], k1r[NL], v1r[NL];
  auto load = [&](u32x4 (&kr)[NL], u32x4 (&vr)[NL], int base) {
    const int key = base + kl;
    const bool ok = key < ke;
    const T* kp = kb + static_cast<size_t>(ok ? key : 0) * D;
    const T* vp = vb + static_cast<size_t>(ok ? key : 0) * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kr[i] = ok ? *reinterpret_cast<const u32x4*>(kp + elem_off(i)) : u32x4{0, 0, 0, 0};
      vr[i] = ok ? *reinterpret_cast<const u32x4*>(vp + elem_off(i)) : u32x4{0, 0, 0, 0};
    }
  };
  auto consume = [&](const u32x4 (&kr)[NL], const u32x4 (&vr)[NL], int base) {
    const bool ok = base + kl < ke;
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) s = dot16(qr[hh][i], kr[i], s, static_cast<T*>(nullptr));
      s = octet_sum(s);
      const float x = s * scale_log2;
      if (ok && x > m_run[hh] + TAU) {  // rare after the first key of the octet
        const float alpha = fast_exp2(m_run[hh] - x);
        l_run[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
        m_run[hh] = x;
      }
      const float p = ok ? fast_exp2(x - m_run[hh]) : 0.f;
      l_run[hh] += p;
#pragma unroll
      for (int i = 0; i < NL; ++i) axpy16(&acc[hh][i * E16], p, vr[i], static_cast<T*>(nullptr));
    }
  };

  if (ks < ke) {
    load(k0r, v0r, ks);
    for (int base = ks; base < ke; base += 2 * KPS) {
      const bool second = base + KPS < ke;
      if (second) load(k1r, v1r, base + KPS);
      consume(k0r, v0r, base);
      if (base + 2 * KPS < ke) load(k0r, v0r, base + 2 * KPS);
      if (second) consume(k1r, v1r, base + KPS);
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

template <typename T, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ partials,
                                                            const int32_t* __restrict__ cache_lens,
                                                            T* __restrict__ out, int num_q_heads, int num_splits) {
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
  T* dst = out + static_cast<size_t>(bh) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) store_elem<T>(dst + lane + 64 * e, o[e] * inv);
}

template <typename T, int D, int GW>
hipError_t launch_split_typed(const DecodeAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks_per_kv = group / GW;
  const long long items = static_cast<long long>(a.num_seqs) * a.num_kv_heads * chunks_per_kv * a.num_splits;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GW>), dim3(static_cast<unsigned>(items)), dim3(256), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k_cache), static_cast<const T*>(a.v_cache),
                     a.cache_lens, a.partials, a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_splits,
                     chunks_per_kv, a.scale_log2);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_dim(const DecodeAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 4 == 0) return launch_split_typed<T, D, 4>(a, stream);
  if (group % 2 == 0) return launch_split_typed<T, D, 2>(a, stream);
  return launch_split_typed<T, D, 1>(a, stream);
}

template <typename T, int D>
hipError_t launch_combine_typed(const DecodeAttnArgs& a, hipStream_t stream) {
  const long long items = static_cast<long long>(a.num_seqs) * a.num_q_heads;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(static_cast<unsigned>(items)), dim3(64), 0, stream,
                     a.partials, a.cache_lens, static_cast<T*>(a.out), a.num_q_heads, a.num_splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeAttnArgs& a, hipStream_t stream) {
  const bool bf = a.dtype == 0;
  if (a.head_dim == 128) return bf ? launch_split_dim<bf16, 128>(a, stream) : launch_split_dim<float, 128>(a, stream);
  if (a.head_dim == 64) return bf ? launch_split_dim<bf16, 64>(a, stream) : launch_split_dim<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_combine(const DecodeAttnArgs& a, hipStream_t stream) {
  const bool bf = a.dtype == 0;
  if (a.head_dim == 128) return bf ? launch_combine_typed<bf16, 128>(a, stream) : launch_combine_typed<float, 128>(a, stream);
  if (a.head_dim == 64) return bf ? launch_combine_typed<bf16, 64>(a, stream) : launch_combine_typed<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra
