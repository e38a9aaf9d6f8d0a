// The decoder-layer steps next to the attention layer, on gfx950 vector units
// (all of them HBM-bound: no contraction here, so no matrix cores).
//
//  * Fused residual add + RMSNorm (zero-to-sglang, "Chapter 3 Forward Pass and
//    Generation (Code Walkthrough)", section 3.2 "Computation inside a decoder
//    layer").  The first call of a forward pass keeps x as the residual and
//    returns RMSNorm(x) * w; later calls add the sublayer output x to the
//    residual stream, keep the sum as the new residual and return its
//    RMSNorm.  One workgroup per row: every thread keeps its 16-byte pieces of
//    the row in registers, so x and the residual are read once and the sum and
//    the output written once.  The sum and the sum of squares are fp32; the
//    new residual is the fp32 sum rounded to the dtype, and the output
//    normalises the fp32 sum.
//  * Last-position gather (same page, section 4.1 "Keep the last position of
//    each request"): row cu[r+1]-1 of the packed hidden states for every
//    request r with tokens.
//  * Greedy argmax (section 4.3 "Find sampling in the engine"): per logits
//    row, the index of the largest value; ties go to the lowest index and a
//    NaN beats every number.  Rows are cut into segments so that a small batch
//    of long rows still fills the chip: pass 1 reduces each segment to a
//    (value, index) record, pass 2 merges a row's records in index order.

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace {

constexpr int kNormThreads = 256;   // one workgroup per row
constexpr int kGatherThreads = 256;
constexpr int kArgmaxThreads = 256;

// 8 elements of a row as fp32, from one 16-byte (bf16) or two 16-byte (fp32) loads.
template <typename T>
struct Piece;

template <>
struct Piece<bf16> {
  u32x4 raw;
  __device__ __forceinline__ void load(const bf16* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  // Rows read once: non-temporal loads (measured 6.4 TB/s for the norm's two
  // reads and two writes, against 5.6 with plain loads; non-temporal stores
  // were slower).
  __device__ __forceinline__ void load_stream(const bf16* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ float at(int i) const {
    const uint32_t w = raw[i >> 1];
    return (i & 1) ? bf16_hi_to_f32(w) : bf16_lo_to_f32(w);
  }
  __device__ __forceinline__ static void store(bf16* p, const float (&v)[8]) {
    const u32x4 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    *reinterpret_cast<u32x4*>(p) = w;
  }
};

template <>
struct Piece<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const f32x4*>(p);
    hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load_stream(const float* p) {
    lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ float at(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
  __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += xor_shuffle(v, m);
  return v;
}

// NCH: 8-element pieces per thread (a row has C/8 pieces, piece c at thread
// c % 256, slot c / 256).  mode 0: first call (residual := x unless they are
// the same buffer); mode 1: residual := x + residual.
template <typename T, int NCH>
__global__ __launch_bounds__(kNormThreads) void fused_add_rmsnorm_kernel(
    const T* __restrict__ x, T* residual, const T* __restrict__ weight, T* out, int hidden, int mode,
    int copy_residual, float eps) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int pieces = hidden >> 3;
  const size_t base = static_cast<size_t>(row) * hidden;
  float v[NCH][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + kNormThreads * i;
    if (c < pieces) {
      Piece<T> px;
      px.load_stream(x + base + 8 * c);
      if (mode == 1) {
        Piece<T> pr;
        pr.load_stream(residual + base + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = px.at(e) + pr.at(e);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = px.at(e);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[i][e], v[i][e], ss);
    }
  }
  // Sum of squares over the row: within each wavefront, then across the four.
  __shared__ float part[kNormThreads / 64];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) tot += part[w];
  const float inv = 1.0f / __builtin_sqrtf(tot / static_cast<float>(hidden) + eps);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + kNormThreads * i;
    if (c < pieces) {
      if (mode == 1 || copy_residual) Piece<T>::store(residual + base + 8 * c, v[i]);
      Piece<T> pw;
      pw.load(weight + 8 * c);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[i][e] * inv * pw.at(e);
      Piece<T>::store(out + base + 8 * c, o);
    }
  }
}

template <typename T>
hipError_t launch_norm_typed(const AddRmsNormArgs& a, hipStream_t s) {
  const int pieces_per_thread = (a.hidden_size / 8 + kNormThreads - 1) / kNormThreads;
  const dim3 grid(static_cast<unsigned>(a.num_tokens)), block(kNormThreads);
  const T* x = static_cast<const T*>(a.x);
  T* r = static_cast<T*>(a.residual);
  const T* w = static_cast<const T*>(a.weight);
  T* o = static_cast<T*>(a.out);
#define QKRA_NORM_CASE(N)                                                                                   \
  if (pieces_per_thread <= N) {                                                                             \
    launch_kernel((fused_add_rmsnorm_kernel<T, N>), grid, block, 0, s, x, r, w, o, a.hidden_size,      \
                       a.has_residual ? 1 : 0, a.copy_residual ? 1 : 0, a.rms_eps);                         \
    return hipGetLastError();                                                                               \
  }
  QKRA_NORM_CASE(1)
  QKRA_NORM_CASE(2)
  QKRA_NORM_CASE(4)
  QKRA_NORM_CASE(8)
  QKRA_NORM_CASE(16)
#undef QKRA_NORM_CASE
  return hipErrorInvalidValue;
}

// ---- last-position gather ---------------------------------------------------
// Grid (pieces / 256, num_seqs): thread copies one 16-byte piece of a row.
__global__ __launch_bounds__(kGatherThreads) void gather_last_kernel(const uint8_t* __restrict__ hidden,
                                                                     const int32_t* __restrict__ cu_seqlens,
                                                                     uint8_t* __restrict__ out, int row_bytes,
                                                                     int num_rows) {
  const int r = blockIdx.y;
  const int piece = blockIdx.x * kGatherThreads + threadIdx.x;
  if (16 * piece >= row_bytes) return;
  const int lo = cu_seqlens[r], hi = cu_seqlens[r + 1];
  if (hi <= lo || hi > num_rows || lo < 0) return;  // no tokens (or out of contract): the row is not written
  const u32x4 v = *reinterpret_cast<const u32x4*>(hidden + static_cast<size_t>(hi - 1) * row_bytes + 16 * piece);
  *reinterpret_cast<u32x4*>(out + static_cast<size_t>(r) * row_bytes + 16 * piece) = v;
}

// ---- greedy argmax ------------------------------------------------------------
struct Best {
  float v;
  int i;
};

// Does candidate a come before b: larger value, NaN above every number, and
// the lower index among equals (and among NaNs).
__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  const bool an = av != av, bn = bv != bv;
  if (an || bn) return an && (!bn || ai < bi);
  return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ Best wave_best(Best b) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = xor_shuffle(b.v, m);
    const int oi = __shfl_xor(b.i, m, 64);
    if (better(ov, oi, b.v, b.i)) b = Best{ov, oi};
  }
  return b;
}

// Best of a workgroup's candidates, returned to every thread.
__device__ __forceinline__ Best block_best(Best b) {
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  b = wave_best(b);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) {
    sv[tid >> 6] = b.v;
    si[tid >> 6] = b.i;
  }
  __syncthreads();
  Best r{sv[0], si[0]};
#pragma unroll
  for (int w = 1; w < kArgmaxThreads / 64; ++w)
    if (better(sv[w], si[w], r.v, r.i)) r = Best{sv[w], si[w]};
  return r;
}

// Pass 1.  Grid (segments, rows): segment s of row b covers indices
// [s*seg_len, min((s+1)*seg_len, vocab)); seg_len is a multiple of 8 so every
// thread reads whole 8-element pieces, in increasing index order.
template <typename T>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_partial_kernel(const T* __restrict__ logits,
                                                                        long long row_stride, int vocab,
                                                                        int seg_len, float* __restrict__ part_v,
                                                                        int* __restrict__ part_i) {
  const int s = blockIdx.x, b = blockIdx.y;
  const int lo = s * seg_len;
  const int hi = min(lo + seg_len, vocab);
  const T* row = logits + static_cast<long long>(b) * row_stride;
  Best best{kNegInf, lo < vocab ? lo : 0};
  bool have_nan = false;
  auto take = [&](const Piece<T>& pc, int p) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float z = pc.at(e);
      if (!have_nan && (z != z || z > best.v)) {
        best = Best{z, p + e};
        have_nan = z != z;
      }
    }
  };
  constexpr int kStride = 8 * kArgmaxThreads;  // elements between a thread's consecutive pieces
  constexpr int kBatch = 4;                    // pieces loaded before any is compared
  int p = lo + 8 * static_cast<int>(threadIdx.x);
  for (; p + (kBatch - 1) * kStride + 8 <= hi; p += kBatch * kStride) {
    Piece<T> pc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) pc[u].load(row + p + u * kStride);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) take(pc[u], p + u * kStride);
  }
  for (; p < hi; p += kStride) {
    if (p + 8 <= hi) {
      Piece<T> pc;
      pc.load(row + p);
      take(pc, p);
    } else {
      for (int e = 0; p + e < hi; ++e) {
        const float z = static_cast<float>(row[p + e]);
        if (!have_nan && (z != z || z > best.v)) {
          best = Best{z, p + e};
          have_nan = z != z;
        }
      }
    }
  }
  // A thread that saw only -inf (or nothing) keeps value -inf at an index of
  // its segment no lower than the segment's first -inf; the lowest index among
  // equal values wins in the reduction below, so an all -inf segment reports lo.
  const Best r = block_best(best);
  if (threadIdx.x == 0) {
    part_v[b * gridDim.x + s] = r.v;
    part_i[b * gridDim.x + s] = r.i;
  }
}

// Pass 2: one wavefront per row merges its segment records.
__global__ __launch_bounds__(64) void argmax_final_kernel(const float* __restrict__ part_v,
                                                          const int* __restrict__ part_i, int segments,
                                                          int32_t* __restrict__ out) {
  const int b = blockIdx.x;
  Best best{kNegInf, 0x7fffffff};
  for (int s = threadIdx.x; s < segments; s += 64) {
    const float v = part_v[b * segments + s];
    const int i = part_i[b * segments + s];
    if (better(v, i, best.v, best.i)) best = Best{v, i};
  }
  best = wave_best(best);
  if (threadIdx.x == 0) out[b] = best.i;
}

}  // namespace

hipError_t launch_fused_add_rmsnorm(const AddRmsNormArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  if (a.dtype == 0) return launch_norm_typed<bf16>(a, stream);
  return launch_norm_typed<float>(a, stream);
}

hipError_t launch_gather_last(const GatherLastArgs& a, hipStream_t stream) {
  if (a.num_seqs <= 0) return hipSuccess;
  const int row_bytes = a.hidden_size * (a.dtype == 0 ? 2 : 4);
  const int pieces = row_bytes / 16;
  const dim3 grid(static_cast<unsigned>((pieces + kGatherThreads - 1) / kGatherThreads),
                  static_cast<unsigned>(a.num_seqs));
  launch_kernel(gather_last_kernel, grid, dim3(kGatherThreads), 0, stream,
                     static_cast<const uint8_t*>(a.hidden), a.cu_seqlens, static_cast<uint8_t*>(a.out), row_bytes,
                     a.num_rows);
  return hipGetLastError();
}

int argmax_segments(int num_rows, int vocab) {
  // Enough workgroups to cover the chip about four times, each segment at
  // least 2048 elements.
  const long long want = (4LL * 256 + num_rows - 1) / num_rows;
  const long long most = (vocab + 2047LL) / 2048;
  return static_cast<int>(std::max(1LL, std::min(want, most)));
}

int argmax_segment_length(int vocab, int segments) {
  const int len = (vocab + segments - 1) / segments;
  return (len + 7) / 8 * 8;
}

hipError_t launch_argmax_partial(const ArgmaxArgs& a, hipStream_t stream) {
  if (a.num_rows <= 0) return hipSuccess;
  const int seg_len = argmax_segment_length(a.vocab, a.segments);
  const dim3 grid(static_cast<unsigned>(a.segments), static_cast<unsigned>(a.num_rows));
  if (a.dtype == 0)
    launch_kernel((argmax_partial_kernel<bf16>), grid, dim3(kArgmaxThreads), 0, stream,
                       static_cast<const bf16*>(a.logits), a.row_stride, a.vocab, seg_len, a.part_v, a.part_i);
  else
    launch_kernel((argmax_partial_kernel<float>), grid, dim3(kArgmaxThreads), 0, stream,
                       static_cast<const float*>(a.logits), a.row_stride, a.vocab, seg_len, a.part_v, a.part_i);
  return hipGetLastError();
}

hipError_t launch_argmax_final(const ArgmaxArgs& a, hipStream_t stream) {
  if (a.num_rows <= 0) return hipSuccess;
  launch_kernel(argmax_final_kernel, dim3(static_cast<unsigned>(a.num_rows)), dim3(64), 0, stream, a.part_v,
                     a.part_i, a.segments, a.out);
  return hipGetLastError();
}

}  // namespace qkra
