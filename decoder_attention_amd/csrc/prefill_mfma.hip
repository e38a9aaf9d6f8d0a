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
// Design (one workgroup = 4 wavefronts = 256 threads):
//  * Work item = (KV-head chunk, request, query tile).  A chunk is HC query
//    heads of one KV group; the tile is 8/HC blocks of 32 consecutive tokens,
//    so every workgroup owns 8 "query blocks" of 32 (head, token) rows and each
//    K/V tile it stages in LDS feeds all of them (GQA sharing).
//  * Each wavefront owns two query blocks.  Scores are formed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A
//    operand, Q^T stays in registers as the B operand for the whole loop.  In
//    the 32x32 accumulator layout a lane then holds one query (lane % 32) and
//    16 of the 32 keys of a block, so the row max needs one exchange with lane
//    ^ 32 and the row sum none until the very end.
//  * O^T = V^T P^T with the same instruction: P^T goes straight from the
//    score accumulators into the B operand (after rounding to bf16), and V is
//    staged in LDS transposed ([d][key]) with the keys of every 16-key step
//    permuted so that each lane's 8 keys are one 16-byte read.  The O^T
//    accumulator is again one query per lane, so the online-softmax rescale
//    is a per-lane multiply.
//  * fp32 online softmax in the log2 domain (scale log2(e)/sqrt(D) folded into
//    one multiply).  K/V tiles run only up to the causal diagonal of the
//    workgroup's last token; tiles entirely above a wavefront's rows are
//    skipped by that wavefront; only tiles that cross the diagonal are masked.
//  * Keys at or past the request's length are zero-filled on load so that
//    whatever the cache holds there never reaches the accumulators.
//  * Double-buffered LDS: the next tile's global loads are issued before the
//    current tile's matrix work and written to the other buffer after it.
//  * Grid: heaviest (latest) query tiles first; block ids are remapped so
//    that consecutive work items land on the same XCD (the hardware deals
//    workgroups round-robin over the 8 XCDs), keeping one KV head's tiles in
//    one L2.

#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace {

constexpr int BN = 64;        // keys per K/V tile
constexpr int NTHREADS = 256;

template <int D, int HC>
__global__ __launch_bounds__(NTHREADS, 1) void prefill_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k_cache, const bf16* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens, bf16* __restrict__ out, int num_q_heads, int num_kv_heads,
    int cache_capacity, int num_seqs, int tiles_per_seq, int chunks_per_kv, int num_items,
    float scale_log2) {
  constexpr int TBN = 8 / HC;       // token blocks (of 32) per workgroup
  constexpr int TM = 32 * TBN;      // tokens per workgroup
  constexpr int DS = D / 16;        // k-steps over D for the scores
  constexpr int DB = D / 32;        // 32-wide blocks of D in the output
  constexpr int KST = D + 8;        // LDS row stride of K (elements)
  constexpr int VST = BN + 8;       // LDS row stride of V^T (elements)
  constexpr int KCHUNKS = BN * D / 8 / NTHREADS;  // 16-byte K loads per thread per tile
  constexpr int VITEMS = 16 * (D / 8);             // (4 keys x 8 d) V items per tile

  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * KST];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][D * VST];

  // ---- work item (XCD-aware remap, heaviest tiles first) -------------------
  const int nb = gridDim.x;  // a multiple of 8
  const int logical = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
  if (logical >= num_items) return;
  const int per_chunk = tiles_per_seq * num_seqs;
  const int chunk = logical / per_chunk;
  const int rem = logical - chunk * per_chunk;
  const int tile = tiles_per_seq - 1 - rem / num_seqs;
  const int seq = rem % num_seqs;
  const int cu0 = cu_seqlens[seq];
  // Lengths are clamped to the cache so out-of-contract inputs cannot address past it.
  const int seqlen = min(cu_seqlens[seq + 1] - cu0, cache_capacity);
  const int t0 = tile * TM;
  if (t0 >= seqlen) return;
  const int group = num_q_heads / num_kv_heads;
  const int g = chunk / chunks_per_kv;
  const int h0 = g * group + (chunk % chunks_per_kv) * HC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int qtok[2], qhead[2], qfirst[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int bi = 2 * wave + qb;
    qfirst[qb] = t0 + 32 * (bi / HC);
    qtok[qb] = qfirst[qb] + l32;
    qhead[qb] = h0 + bi % HC;
  }

  // Q^T fragments (B operand): lane holds query l32, d = 16*ds + 8*hi .. +7.
  bf16x8 qf[2][DS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const bool valid = qtok[qb] < seqlen;
    const bf16* src = q + (static_cast<size_t>(cu0 + (valid ? qtok[qb] : 0)) * num_q_heads + qhead[qb]) * D + 8 * hi;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(src + 16 * ds);
      if (!valid) v = bf16x8{};
      qf[qb][ds] = v;
    }
  }

  f32x16 acc[2][DB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = f32x16{};
  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};

  const int kv_end = min(seqlen, t0 + TM);
  const int ntiles = (kv_end + BN - 1) / BN;
  const size_t head_off = (static_cast<size_t>(seq) * num_kv_heads + g) * cache_capacity * D;
  const bf16* kbase = k_cache + head_off;
  const bf16* vbase = v_cache + head_off;

  uint4 kreg[KCHUNKS];
  uint4 vreg[4];
  const int v_kq = tid & 15;   // which 4-key quad of the tile
  const int v_dq = tid >> 4;   // which 8-wide slice of D
  const bool v_loader = tid < VITEMS;

  auto load_tile = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int c = tid + NTHREADS * i;
      const int r = c / (D / 8);
      const int col = c % (D / 8);
      const int key = k0 + r;
      kreg[i] = key < kv_end ? *reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(key) * D + col * 8)
                             : make_uint4(0, 0, 0, 0);
    }
    if (v_loader) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kq + r;
        vreg[r] = key < kv_end ? *reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(key) * D + v_dq * 8)
                               : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const int c = tid + NTHREADS * i;
      const int r = c / (D / 8);
      const int col = c % (D / 8);
      *reinterpret_cast<uint4*>(&sK[buf][r * KST + col * 8]) = kreg[i];
    }
    if (v_loader) {
      // Keys 4*kq..4*kq+3 of one 8-wide d slice, written transposed.  Within
      // each 16-key step the key quads are stored in the order 0, 2, 1, 3, so
      // that lane half `hi` finds its keys {4hi..4hi+3, 8+4hi..8+4hi+3} as 8
      // contiguous elements.
      const int step = v_kq >> 2;
      const int quad = v_kq & 3;
      const int pos = 16 * step + 4 * ((quad & 1) * 2 + (quad >> 1));
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint2 lo = make_uint2((w0[p] & 0xffffu) | (w1[p] << 16), (w2[p] & 0xffffu) | (w3[p] << 16));
        const uint2 hi2 = make_uint2((w0[p] >> 16) | (w1[p] & 0xffff0000u), (w2[p] >> 16) | (w3[p] & 0xffff0000u));
        *reinterpret_cast<uint2*>(&sV[buf][(v_dq * 8 + 2 * p) * VST + pos]) = lo;
        *reinterpret_cast<uint2*>(&sV[buf][(v_dq * 8 + 2 * p + 1) * VST + pos]) = hi2;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const int k0 = kt * BN;

    // A wavefront whose rows all precede this tile's first key skips it.
    const bool live0 = k0 <= qfirst[0] + 31;
    const bool live1 = k0 <= qfirst[1] + 31;
    if (live0 || live1) {
      // ---- S^T = K Q^T ------------------------------------------------------
      f32x16 s[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&sK[buf][(kb * 32 + l32) * KST + 16 * ds + 8 * hi]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][ds], s[qb][kb], 0, 0, 0);
        }
      }

      // ---- online softmax (lane = query l32) --------------------------------
      bf16x8 pf[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bool diag = k0 + BN - 1 > qfirst[qb];
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float x = s[qb][kb][j] * scale_log2;
            if (diag) {
              const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
              if (key > qtok[qb]) x = kNegInf;
            }
            s[qb][kb][j] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run[qb] - m_use);
        m_run[qb] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float p = fast_exp2(s[qb][kb][j] - m_use);
            s[qb][kb][j] = p;
            rs += p;
          }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
        // P^T as the B operand: 16-key step ks = 2*kb + half uses the
        // accumulator registers 8*half .. 8*half+7 of key block kb.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int kb = ks >> 1, base = 8 * (ks & 1);
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(s[qb][kb][base + 2 * e], s[qb][kb][base + 2 * e + 1]);
          pf[qb][ks] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }

      // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&sV[buf][(db * 32 + l32) * VST + 16 * ks + 8 * hi]);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][ks], acc[qb][db], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds query l32, d = 32*db + 8*(j/4) + 4*hi + j%4
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_run[qb] + xor_shuffle(l_run[qb], 32);
    const float inv = 1.0f / l_tot;
    if (qtok[qb] < seqlen) {
      bf16* dst = out + (static_cast<size_t>(cu0 + qtok[qb]) * num_q_heads + qhead[qb]) * D + 4 * hi;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x16& a = acc[qb][db];
          const uint2 w = make_uint2(pack_bf16x2(a[4 * jq] * inv, a[4 * jq + 1] * inv),
                                     pack_bf16x2(a[4 * jq + 2] * inv, a[4 * jq + 3] * inv));
          *reinterpret_cast<uint2*>(dst + 32 * db + 8 * jq) = w;
        }
    }
  }
}

template <int D, int HC>
hipError_t launch_typed(const PrefillAttnArgs& a, hipStream_t stream) {
  constexpr int TM = 32 * (8 / HC);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int chunks_per_kv = group / HC;
  const int tiles = (a.max_seqlen + TM - 1) / TM;
  const long long items = static_cast<long long>(a.num_kv_heads) * chunks_per_kv * a.num_seqs * tiles;
  if (items <= 0) return hipSuccess;
  const long long grid = (items + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_mfma_kernel<D, HC>), dim3(static_cast<unsigned>(grid)), dim3(NTHREADS), 0, stream,
                     static_cast<const bf16*>(a.q), static_cast<const bf16*>(a.k_cache),
                     static_cast<const bf16*>(a.v_cache), a.cu_seqlens, static_cast<bf16*>(a.out),
                     a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.num_seqs, tiles, chunks_per_kv,
                     static_cast<int>(items), a.scale_log2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const PrefillAttnArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  if (group % 8 == 0) return launch_typed<D, 8>(a, stream);
  if (group % 4 == 0) return launch_typed<D, 4>(a, stream);
  if (group % 2 == 0) return launch_typed<D, 2>(a, stream);
  return launch_typed<D, 1>(a, stream);
}

}  // namespace

hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_dim<128>(a, stream);
  if (a.head_dim == 64) return launch_dim<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra
