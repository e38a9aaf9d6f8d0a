// Kernel 2 (fp32 mode): causal grouped-query attention for prefill with fp32
// inputs, fp32 products and fp32 accumulation throughout (no reduced-precision
// matrix formats, so results stay within 1e-4 of the exact values).
//
// Same definition as the bf16 kernel (zero-to-sglang code walkthrough, section
// 3.3): scores q~ . k~ / sqrt(D), causal mask, softmax, weighted sum of V,
// query head h reading KV head floor(h / G).  This is the precision path, not
// the throughput path: one workgroup per (request, 64-token tile, query head);
// two lanes share a query row (half of D each), K/V tiles of 32 keys are staged
// in LDS and read as broadcasts; online softmax per tile.

#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace {

constexpr int QT = 64;    // query tokens per workgroup
constexpr int KT = 32;    // keys per tile
constexpr int NT = 2 * QT;

template <int D>
__global__ __launch_bounds__(NT) void prefill_fp32_kernel(
    const float* __restrict__ q, const float* __restrict__ k_cache, const float* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ past_lens, float* __restrict__ out,
    int num_q_heads, int num_kv_heads, int cache_capacity, int num_seqs, int tiles_per_seq, float scale_log2,
    PagedTable paged) {
  constexpr int HD = D / 2;
  __shared__ float sK[KT][D + 1];
  __shared__ float sV[KT][D + 1];

  const int item = blockIdx.x;
  const int head = item % num_q_heads;
  const int rest = item / num_q_heads;
  const int tile = tiles_per_seq - 1 - rest / num_seqs;
  const int seq = rest % num_seqs;
  const int cu0 = cu_seqlens[seq];
  // Entries cached before the chunk; the chunk is clamped to the cache so
  // out-of-contract inputs cannot address past it.
  const int past = past_lens ? min(max(past_lens[seq], 0), cache_capacity) : 0;
  const int seqlen = min(cu_seqlens[seq + 1] - cu0, cache_capacity - past);
  const int t0 = tile * QT;
  if (t0 >= seqlen) return;
  const int g = head / (num_q_heads / num_kv_heads);

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int tok = t0 + (tid >> 1);
  const bool valid = tok < seqlen;

  float qr[HD], acc[HD];
  const float* qsrc = q + (static_cast<size_t>(cu0 + (valid ? tok : 0)) * num_q_heads + head) * D + half * HD;
#pragma unroll
  for (int e = 0; e < HD; ++e) {
    qr[e] = valid ? qsrc[e] : 0.f;
    acc[e] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;

  const int kv_end = past + min(seqlen, t0 + QT);
  const size_t head_off = (static_cast<size_t>(seq) * num_kv_heads + g) * cache_capacity * D;
  for (int k0 = 0; k0 < kv_end; k0 += KT) {
    __syncthreads();
    for (int i = tid; i < KT * D; i += NT) {
      const int r = i / D, c = i % D;
      const int key = k0 + r;
      // A paged cache: the key's row through the block table.
      const size_t row = key >= kv_end ? 0
                         : paged.table ? paged_row(paged, seq, g, key, num_kv_heads, D)
                                       : head_off + static_cast<size_t>(key) * D;
      sK[r][c] = key < kv_end ? k_cache[row + c] : 0.f;
      sV[r][c] = key < kv_end ? v_cache[row + c] : 0.f;
    }
    __syncthreads();
    float s[KT];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < HD; ++e) dot += qr[e] * sK[j][half * HD + e];
      dot += xor_shuffle(dot, 1);
      const int key = k0 + j;
      s[j] = (key <= past + tok && key < kv_end) ? dot * scale_log2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      s[j] = exp2f(s[j] - m_use);
      rs += s[j];
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int e = 0; e < HD; ++e) {
      float a = acc[e] * alpha;
#pragma unroll
      for (int j = 0; j < KT; ++j) a += s[j] * sV[j][half * HD + e];
      acc[e] = a;
    }
  }
  if (valid) {
    const float inv = 1.0f / l_run;
    float* dst = out + (static_cast<size_t>(cu0 + tok) * num_q_heads + head) * D + half * HD;
#pragma unroll
    for (int e = 0; e < HD; ++e) dst[e] = acc[e] * inv;
  }
}

template <int D>
hipError_t launch_typed(const PrefillAttnArgs& a, hipStream_t stream) {
  const int tiles = (a.max_seqlen + QT - 1) / QT;
  const long long items = static_cast<long long>(tiles) * a.num_seqs * a.num_q_heads;
  if (items <= 0) return hipSuccess;
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  launch_kernel((prefill_fp32_kernel<D>), dim3(static_cast<unsigned>(items)), dim3(NT), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k_cache),
                     static_cast<const float*>(a.v_cache), a.cu_seqlens, a.past_lens, static_cast<float*>(a.out),
                     a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_seqs, tiles, a.scale_log2, a.paged);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_attn_fp32(const PrefillAttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_typed<128>(a, stream);
  if (a.head_dim == 64) return launch_typed<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra
