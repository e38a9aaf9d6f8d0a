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
//  * 3a: one wavefront per (request, KV head, split of 512 keys); it serves the
//    GW query heads of its group that share the KV head (GW = 4 for Qwen3's
//    G = 4), so every K/V byte is fetched once for all of them.
//  * Four lanes share one key row: each lane owns a quarter of D and issues
//    16-byte loads; the four lanes of a key read 64 contiguous bytes per
//    instruction.  16 keys per wavefront step, the next step's loads in flight
//    while the current one is consumed.
//  * Scores via v_dot2_f32_bf16 (bf16) or fp32 FMA, reduced over the 4 lanes
//    of a key; per-step max over the 16 keys; fp32 online softmax in the log2
//    domain, rescaling only when the running max grows.
//  * Each wavefront writes (m, l, o[D]) for its split; 3b merges the splits of
//    a (request, head) in a fixed order: m = max m_s, l = sum l_s 2^(m_s - m),
//    o = sum o_s 2^(m_s - m) / l.  Deterministic, no atomics.

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
__device__ __forceinline__ float dot16(uint4 q, uint4 k, float acc, bf16*) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.x), __builtin_bit_cast(bf16x2, k.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.y), __builtin_bit_cast(bf16x2, k.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.z), __builtin_bit_cast(bf16x2, k.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w), __builtin_bit_cast(bf16x2, k.w), acc, false);
  return acc;
}
__device__ __forceinline__ float dot16(uint4 q, uint4 k, float acc, float*) {
  acc += __uint_as_float(q.x) * __uint_as_float(k.x);
  acc += __uint_as_float(q.y) * __uint_as_float(k.y);
  acc += __uint_as_float(q.z) * __uint_as_float(k.z);
  acc += __uint_as_float(q.w) * __uint_as_float(k.w);
  return acc;
}

// acc[0..n) += p * v for the elements of 16 bytes of v.
__device__ __forceinline__ void axpy16(float* acc, float p, uint4 v, bf16*) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += p * bf16_lo_to_f32(w[i]);
    acc[2 * i + 1] += p * bf16_hi_to_f32(w[i]);
  }
}
__device__ __forceinline__ void axpy16(float* acc, float p, uint4 v, float*) {
  acc[0] += p * __uint_as_float(v.x);
  acc[1] += p * __uint_as_float(v.y);
  acc[2] += p * __uint_as_float(v.z);
  acc[3] += p * __uint_as_float(v.w);
}

template <typename T, int D, int GW>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ cache_lens, float* __restrict__ partials, int num_q_heads, int num_kv_heads,
    int cache_capacity, int num_splits, int chunks_per_kv, int wgs_per_seq, float scale_log2) {
  constexpr int ES = sizeof(T);
  constexpr int E16 = 16 / ES;          // elements per 16-byte load
  constexpr int EPL = D / 4;            // elements per lane per key row
  constexpr int NL = EPL / E16;         // 16-byte loads per lane per key row

  const int item = blockIdx.x;
  const int wgs = item % wgs_per_seq;
  const int rest = item / wgs_per_seq;
  const int nchunks = num_kv_heads * chunks_per_kv;
  const int hc = rest % nchunks;
  const int b = rest / nchunks;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int split = wgs * 4 + wave;
  const int nkeys = min(cache_lens[b] + 1, cache_capacity);  // clamp: never read past the cache
  const int ks = split * SPLIT;
  if (ks >= nkeys) return;
  const int ke = min(nkeys, ks + SPLIT);
  const int group = num_q_heads / num_kv_heads;
  const int g = hc / chunks_per_kv;
  const int h0 = g * group + (hc % chunks_per_kv) * GW;
  const int kl = lane >> 2;   // key within the 16-key step
  const int c = lane & 3;     // quarter of the row

  // Element offset of this lane's i-th 16-byte piece of a row: the four lanes
  // of a key cover 64 contiguous bytes per load instruction.
  auto elem_off = [&](int i) { return (64 * i + 16 * c) / ES; };

  uint4 qr[GW][NL];
#pragma unroll
  for (int hh = 0; hh < GW; ++hh)
#pragma unroll
    for (int i = 0; i < NL; ++i)
      qr[hh][i] = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(b) * num_q_heads + h0 + hh) * D + elem_off(i));

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

  // Two register buffers, used alternately, so the next step's loads are in
  // flight while the current step is consumed.
  uint4 k0r[NL], v0r[NL], k1r[NL], v1r[NL];
  auto load = [&](uint4 (&kr)[NL], uint4 (&vr)[NL], int base) {
    const int key = base + kl;
    const bool ok = key < ke;
    const T* kp = kb + static_cast<size_t>(ok ? key : 0) * D;
    const T* vp = vb + static_cast<size_t>(ok ? key : 0) * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kr[i] = ok ? *reinterpret_cast<const uint4*>(kp + elem_off(i)) : make_uint4(0, 0, 0, 0);
      vr[i] = ok ? *reinterpret_cast<const uint4*>(vp + elem_off(i)) : make_uint4(0, 0, 0, 0);
    }
  };
  auto consume = [&](const uint4 (&kr)[NL], const uint4 (&vr)[NL], int base) {
    const bool ok = base + kl < ke;
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) s = dot16(qr[hh][i], kr[i], s, static_cast<T*>(nullptr));
      s += xor_shuffle(s, 1);
      s += xor_shuffle(s, 2);
      const float x = ok ? s * scale_log2 : kNegInf;
      float mx = x;
      mx = fmaxf(mx, xor_shuffle(mx, 4));
      mx = fmaxf(mx, xor_shuffle(mx, 8));
      mx = fmaxf(mx, xor_shuffle(mx, 16));
      mx = fmaxf(mx, xor_shuffle(mx, 32));
      if (mx > m_run[hh]) {  // uniform across the wavefront
        const float alpha = fast_exp2(m_run[hh] - mx);
        l_run[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
        m_run[hh] = mx;
      }
      const float p = fast_exp2(x - m_run[hh]);
      l_run[hh] += p;
#pragma unroll
      for (int i = 0; i < NL; ++i) axpy16(&acc[hh][i * E16], p, vr[i], static_cast<T*>(nullptr));
    }
  };

  load(k0r, v0r, ks);
  for (int base = ks; base < ke; base += 2 * CHUNK) {
    const bool second = base + CHUNK < ke;
    if (second) load(k1r, v1r, base + CHUNK);
    consume(k0r, v0r, base);
    if (base + 2 * CHUNK < ke) load(k0r, v0r, base + 2 * CHUNK);
    if (second) consume(k1r, v1r, base + CHUNK);
  }

  // Sum over the 16 keys of a step (lanes with equal c), then write the split.
#pragma unroll
  for (int hh = 0; hh < GW; ++hh) {
    float l = l_run[hh];
#pragma unroll
    for (int m = 4; m < 64; m <<= 1) l += xor_shuffle(l, m);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[hh][e];
#pragma unroll
      for (int m = 4; m < 64; m <<= 1) v += xor_shuffle(v, m);
      acc[hh][e] = v;
    }
    float* dst = partials + ((static_cast<size_t>(b) * num_q_heads + h0 + hh) * num_splits + split) * (D + 2);
    if (lane == 0) {
      dst[0] = m_run[hh];
      dst[1] = l;
    }
    if (kl == 0) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < E16; ++e) dst[2 + elem_off(i) + e] = acc[hh][i * E16 + e];
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
  const int wgs_per_seq = (a.num_splits + 3) / 4;
  const long long items = static_cast<long long>(a.num_seqs) * a.num_kv_heads * chunks_per_kv * wgs_per_seq;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GW>), dim3(static_cast<unsigned>(items)), dim3(256), 0, stream,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k_cache), static_cast<const T*>(a.v_cache),
                     a.cache_lens, a.partials, a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_splits,
                     chunks_per_kv, wgs_per_seq, a.scale_log2);
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
