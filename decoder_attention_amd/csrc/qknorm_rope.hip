// Kernel 1: fused per-head Q/K RMSNorm + rotate-half RoPE + K/V cache write.
//
// Follows zero-to-sglang "Chapter 3 Forward Pass and Generation (Code
// Walkthrough)", section 3.3: the packed projection is split into Q, K and V
// heads, each Q and K head is RMS-normalised over its last dimension with a
// learned weight, Q and K are rotated at the token's position, V is left as it
// is.  The cache write follows the concept chapter, section 4.1 (prefill keeps
// every prompt token's K and V) and jq-wei "transformer basics", "Prefill vs
// Decode" (a decode step appends one entry).
//
// With a rope table (bf16 prefill), the kernel writes the row's fp32 cos/sin
// pairs there instead of q~ and skips the Q heads: the attention kernel
// normalises and rotates Q itself while loading it.
//
// Layout of the work: one workgroup per token row (one wavefront with a rope
// table, four otherwise).  The D/2 rotation angles
// of the row are formed once in fp64 (position * base^(-2i/D), then sin/cos)
// and kept in LDS, so positions up to tens of thousands keep full fp32
// accuracy in cos/sin.  Each head row is handled by D/16 (bf16) or D/8 (fp32)
// lanes: a lane holds 16 bytes of the first half and the matching 16 bytes of
// the second half, so every rotate-half pair stays inside one lane and the
// rotation needs no cross-lane traffic; only the sum of squares is reduced
// across the row's lanes.  Loads and stores are 16 B per lane, contiguous
// across the lanes of a head (8-byte pieces ran 2-3% slower).  A wavefront's first four passes are loaded before the
// request lookup and the angle computation, so those latencies overlap.  With
// a block table the cache rows are found through it (a paged pool); slots
// still count from the request's first entry.

#include "decode_plan.h"
#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace {

// A lane's 16-byte piece of a half row: 8 bf16 or 4 fp32 elements.
template <typename T> constexpr int kLaneElems = 16 / sizeof(T);

__device__ __forceinline__ void unpack(u32x4 r, float x[8], const bf16*) {
  x[0] = bf16_lo_to_f32(r.x); x[1] = bf16_hi_to_f32(r.x); x[2] = bf16_lo_to_f32(r.y); x[3] = bf16_hi_to_f32(r.y);
  x[4] = bf16_lo_to_f32(r.z); x[5] = bf16_hi_to_f32(r.z); x[6] = bf16_lo_to_f32(r.w); x[7] = bf16_hi_to_f32(r.w);
}
__device__ __forceinline__ void unpack(u32x4 r, float x[4], const float*) {
  x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y); x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
}
__device__ __forceinline__ u32x4 pack(const float y[8], const bf16*) {
  return u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}
__device__ __forceinline__ u32x4 pack(const float y[4], const float*) {
  return u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]), __float_as_uint(y[3])};
}

// One row of a batch: its Q and K heads normalised and rotated (Q only
// without a rope table), its V heads copied, K~ and V into the cache.
template <typename T, int D>
__device__ __forceinline__ void qknorm_rope_row(
    const int row_id, const T* __restrict__ qkv, const T* __restrict__ q_weight, const T* __restrict__ k_weight,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ seq_info,
    const int32_t* __restrict__ slot_offsets, int decode_mode,
    int num_seqs, int num_q_heads, int num_kv_heads, int cache_capacity, float eps,
    double log2_base, T* __restrict__ q_out, float* __restrict__ rope_table, T* __restrict__ k_cache,
    T* __restrict__ v_cache, PagedTable paged, float* s_cos, float* s_sin) {
  using Raw = u32x4;
  constexpr int E = kLaneElems<T>;  // elements per lane and half row
  constexpr const T* kT = nullptr;   // selects the element type's unpack and pack
  constexpr int HALF = D / 2;
  constexpr int LPH = HALF / E;  // lanes per head row
  constexpr int HPW = 64 / LPH;  // head rows per wavefront pass
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int sub = lane % LPH;
  const int hslot = lane / LPH;
  const int i0 = sub * E;
  const int heads = num_q_heads + 2 * num_kv_heads;
  const T* row = qkv + static_cast<size_t>(row_id) * heads * D;
  // With a rope table the attention kernel rotates Q itself: only K and V heads here.
  const int head0 = rope_table ? num_q_heads : 0;

  // The row's first PRE passes are loaded before anything else: they depend
  // only on the row, so their latency overlaps the request lookup, the angle
  // computation and the barrier.  Rows are read once (non-temporal).
  constexpr int PRE = 4;
  Raw pre1[PRE], pre2[PRE];
#pragma unroll
  for (int p = 0; p < PRE; ++p) {
    const int head = head0 + (wave + p * nwaves) * HPW + hslot;
    pre1[p] = Raw{};
    pre2[p] = Raw{};
    if (head < heads) {
      pre1[p] = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(row + head * D + i0));
      pre2[p] = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(row + head * D + HALF + i0));
    }
  }

  int req, slot;
  if (decode_mode) {
    req = row_id;
    slot = seq_info[row_id];
  } else {
    // Request r with cu[r] <= row < cu[r+1]; empty requests are skipped over.
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seq_info[mid] <= row_id) lo = mid; else hi = mid;
    }
    req = lo;
    slot = row_id - seq_info[lo] + (slot_offsets ? slot_offsets[lo] : 0);
  }
  // Rows outside the caller's contract (slot past the cache) write no cache entry.
  const bool slot_ok = slot >= 0 && slot < cache_capacity;

  const double pos = static_cast<double>(positions[row_id]);
  for (int i = threadIdx.x; i < HALF; i += blockDim.x) {
    const double theta = exp2(-static_cast<double>(2 * i) / static_cast<double>(D) * log2_base);
    double sn, cs;
    sincos(pos * theta, &sn, &cs);
    s_cos[i] = static_cast<float>(cs);
    s_sin[i] = static_cast<float>(sn);
    if (rope_table) {
      // fp32, D per row: cos in the first half, sin in the second, each half
      // as two runs of D/4 (pair indices i with i%8 < 4, then i%8 >= 4), i at
      // 4*(i/8) + i%4 within its run.  A reader holding pairs 8j..8j+7 finds
      // each four of them as one 16-byte piece, and D/16 such readers cover
      // a run with one contiguous line.
      const size_t at = static_cast<size_t>(row_id) * D + (D / 4) * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
      rope_table[at] = static_cast<float>(cs);
      rope_table[at + HALF] = static_cast<float>(sn);
    }
  }
  __syncthreads();

  float cs[E], sn[E], wq1[E], wq2[E], wk1[E], wk2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    cs[e] = s_cos[i0 + e];
    sn[e] = s_sin[i0 + e];
  }
  unpack(*reinterpret_cast<const Raw*>(q_weight + i0), wq1, kT);
  unpack(*reinterpret_cast<const Raw*>(q_weight + HALF + i0), wq2, kT);
  unpack(*reinterpret_cast<const Raw*>(k_weight + i0), wk1, kT);
  unpack(*reinterpret_cast<const Raw*>(k_weight + HALF + i0), wk2, kT);

  int pass = 0;
  for (int hb = head0 + wave * HPW; hb < heads; hb += nwaves * HPW, ++pass) {
    const int head = hb + hslot;
    const bool active = head < heads;
    Raw r1 = {}, r2 = {};
    if (pass < PRE) {
#pragma unroll
      for (int p = 0; p < PRE; ++p)
        if (p == pass) {
          r1 = pre1[p];
          r2 = pre2[p];
        }
    } else if (active) {
      r1 = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(row + head * D + i0));
      r2 = __builtin_nontemporal_load(reinterpret_cast<const Raw*>(row + head * D + HALF + i0));
    }
    float x1[E], x2[E];
    unpack(r1, x1, kT);
    unpack(r2, x2, kT);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += x1[e] * x1[e] + x2[e] * x2[e];
#pragma unroll
    for (int m = 1; m < LPH; m <<= 1) ss += xor_shuffle(ss, m);
    if (!active) continue;

    if (head >= num_q_heads + num_kv_heads) {  // V head: bit copy into the cache
      if (!slot_ok) continue;
      const int g = head - num_q_heads - num_kv_heads;
      T* dst = v_cache + cache_row(paged, req, g, slot, num_kv_heads, cache_capacity, D);
      *reinterpret_cast<Raw*>(dst + i0) = r1;
      *reinterpret_cast<Raw*>(dst + HALF + i0) = r2;
      continue;
    }
    const bool is_q = head < num_q_heads;
    if (!is_q && !slot_ok) continue;
    const float inv_rms = rsqrtf(ss * (1.0f / D) + eps);
    float y1[E], y2[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float a = x1[e] * inv_rms * (is_q ? wq1[e] : wk1[e]);
      const float b = x2[e] * inv_rms * (is_q ? wq2[e] : wk2[e]);
      y1[e] = a * cs[e] - b * sn[e];
      y2[e] = b * cs[e] + a * sn[e];
    }
    T* dst = is_q ? q_out + (static_cast<size_t>(row_id) * num_q_heads + head) * D
                  : k_cache + cache_row(paged, req, head - num_q_heads, slot, num_kv_heads, cache_capacity, D);
    *reinterpret_cast<Raw*>(dst + i0) = pack(y1, kT);
    *reinterpret_cast<Raw*>(dst + HALF + i0) = pack(y2, kT);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void qknorm_rope_kv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ q_weight, const T* __restrict__ k_weight,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ seq_info,
    const int32_t* __restrict__ slot_offsets, int decode_mode,
    int num_seqs, int num_q_heads, int num_kv_heads, int cache_capacity, float eps,
    double log2_base, T* __restrict__ q_out, float* __restrict__ rope_table, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int num_rows, int32_t* __restrict__ plan, int plan_units, int plan_nchunks,
    PagedTable paged) {
  __shared__ float s_cos[D / 2];
  __shared__ float s_sin[D / 2];
  const int row_id = blockIdx.x;
  if (row_id == num_rows) {  // bf16 decode: the block past the rows builds the split kernel's plan
    __shared__ int32_t s_scan[256];
    build_decode_plan<256>(seq_info, plan, plan_units, plan_nchunks, cache_capacity, s_scan);
    return;
  }
  qknorm_rope_row<T, D>(row_id, qkv, q_weight, k_weight, positions, seq_info, slot_offsets, decode_mode, num_seqs,
                        num_q_heads, num_kv_heads, cache_capacity, eps, log2_base, q_out, rope_table, k_cache,
                        v_cache, paged, s_cos, s_sin);
}

// Two batches in one launch of single-wavefront blocks (the mixed step: the
// decode rows with q~, a block for the split kernel's plan, then the prefill
// rows with their rope table), so the decode rows run beside the prefill rows
// instead of in a launch of their own.  Both use the same norm weights and
// contiguous caches.
template <typename T, int D>
__global__ __launch_bounds__(64) void qknorm_rope_kv_pair_kernel(
    const T* __restrict__ q_weight, const T* __restrict__ k_weight, int num_q_heads, int num_kv_heads, float eps,
    double log2_base,
    const T* __restrict__ p_qkv, const int32_t* __restrict__ p_positions, const int32_t* __restrict__ p_cu,
    int p_num_seqs, int p_cache_capacity, float* __restrict__ p_rope_table, T* __restrict__ p_k_cache,
    T* __restrict__ p_v_cache, int p_rows,
    const T* __restrict__ d_qkv, const int32_t* __restrict__ d_positions, const int32_t* __restrict__ d_lens,
    int d_cache_capacity, T* __restrict__ d_q_out, T* __restrict__ d_k_cache, T* __restrict__ d_v_cache,
    int d_rows, int32_t* __restrict__ plan, int plan_units, int plan_nchunks) {
  __shared__ float s_cos[D / 2];
  __shared__ float s_sin[D / 2];
  // The decode rows (every head of a row in one wavefront, so each takes longer than a prefill row) and the plan
  // go first, beside the prefill rows that follow.
  const int block = blockIdx.x;
  if (block < d_rows) {
    qknorm_rope_row<T, D>(block, d_qkv, q_weight, k_weight, d_positions, d_lens, nullptr, 1, d_rows, num_q_heads,
                          num_kv_heads, d_cache_capacity, eps, log2_base, d_q_out, nullptr, d_k_cache, d_v_cache,
                          PagedTable{}, s_cos, s_sin);
  } else if (block == d_rows) {
    __shared__ int32_t s_scan[64];
    build_decode_plan<64>(d_lens, plan, plan_units, plan_nchunks, d_cache_capacity, s_scan);
  } else {
    qknorm_rope_row<T, D>(block - d_rows - 1, p_qkv, q_weight, k_weight, p_positions, p_cu, nullptr, 0, p_num_seqs,
                          num_q_heads, num_kv_heads, p_cache_capacity, eps, log2_base, nullptr, p_rope_table,
                          p_k_cache, p_v_cache, PagedTable{}, s_cos, s_sin);
  }
}

template <typename T, int D>
hipError_t launch_pair_typed(const QkNormRopeArgs& p, const QkNormRopeArgs& d, hipStream_t stream) {
  const int blocks = p.num_rows + d.num_rows + 1;
  launch_kernel((qknorm_rope_kv_pair_kernel<T, D>), dim3(blocks), dim3(64), 0, stream,
                static_cast<const T*>(p.q_norm_weight), static_cast<const T*>(p.k_norm_weight), p.num_q_heads,
                p.num_kv_heads, p.rms_eps, p.log2_rope_base,
                static_cast<const T*>(p.qkv), p.positions, p.seq_info, p.num_seqs, p.cache_capacity, p.rope_table,
                static_cast<T*>(p.k_cache), static_cast<T*>(p.v_cache), p.num_rows,
                static_cast<const T*>(d.qkv), d.positions, d.seq_info, d.cache_capacity, static_cast<T*>(d.q_out),
                static_cast<T*>(d.k_cache), static_cast<T*>(d.v_cache), d.num_rows, d.plan, d.plan_units,
                d.plan_nchunks);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const QkNormRopeArgs& a, hipStream_t stream) {
  // bf16 prefill (K and V heads only): one wavefront per token, whose four
  // prefetched passes cover its 2*Hkv rows for Hkv <= 16 at D = 128 and whose fp64 angles
  // then overlap other tokens' work on the CU (four wavefronts waiting on the
  // first one's angles made the kernel a third slower).  Otherwise four.
  const int threads = a.rope_table ? 64 : 256;
  if (a.plan && threads != 256) return hipErrorInvalidValue;  // the plan block is written for 256 threads
  const int blocks = a.num_rows + (a.plan ? 1 : 0);
  launch_kernel((qknorm_rope_kv_kernel<T, D>), dim3(blocks), dim3(threads), 0, stream,
                     static_cast<const T*>(a.qkv), static_cast<const T*>(a.q_norm_weight),
                     static_cast<const T*>(a.k_norm_weight), a.positions, a.seq_info, a.slot_offsets,
                     a.decode_mode,
                     a.num_seqs, a.num_q_heads, a.num_kv_heads, a.cache_capacity, a.rms_eps,
                     a.log2_rope_base, static_cast<T*>(a.q_out), a.rope_table, static_cast<T*>(a.k_cache),
                     static_cast<T*>(a.v_cache), a.num_rows, a.plan, a.plan_units, a.plan_nchunks, a.paged);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, hipStream_t stream) {
  const bool bf = a.dtype == 0;
  if (a.head_dim == 128) return bf ? launch_typed<bf16, 128>(a, stream) : launch_typed<float, 128>(a, stream);
  if (a.head_dim == 64) return bf ? launch_typed<bf16, 64>(a, stream) : launch_typed<float, 64>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_qknorm_rope_pair(const QkNormRopeArgs& prefill, const QkNormRopeArgs& decode, hipStream_t stream) {
  // bf16 only: a prefill batch with its rope table and no history, a decode batch with its plan; contiguous caches,
  // one set of norm weights.
  if (prefill.dtype != 0 || decode.dtype != 0 || !prefill.rope_table || prefill.slot_offsets || prefill.decode_mode ||
      !decode.decode_mode || !decode.plan || decode.rope_table || prefill.paged.table || decode.paged.table ||
      prefill.q_norm_weight != decode.q_norm_weight || prefill.k_norm_weight != decode.k_norm_weight ||
      prefill.head_dim != decode.head_dim || prefill.num_q_heads != decode.num_q_heads ||
      prefill.num_kv_heads != decode.num_kv_heads)
    return hipErrorInvalidValue;
  if (prefill.head_dim == 128) return launch_pair_typed<bf16, 128>(prefill, decode, stream);
  if (prefill.head_dim == 64) return launch_pair_typed<bf16, 64>(prefill, decode, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkra
