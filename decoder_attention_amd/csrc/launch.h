// Host-side launch descriptors for the gfx950 kernels.  Every launcher enqueues
// on the given stream and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qkra {

// Kernel-timing instrumentation: the C ABI sets these events on the calling
// thread around one launcher call, and the launch records them on its own
// dispatch (start and end of the kernel's execution), so timing inserts no
// packet between kernels.  Null events: an untimed launch.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;  // set by launch_kernel when a kernel took the events
};
extern thread_local LaunchEvents g_launch_events;

// Every kernel of the library is launched through here.
template <typename Kernel, typename... Args>
inline void launch_kernel(Kernel kernel, dim3 grid, dim3 block, uint32_t shared_bytes, hipStream_t stream,
                          Args... args) {
  LaunchEvents& ev = g_launch_events;
  hipExtLaunchKernelGGL(kernel, grid, block, shared_bytes, stream, ev.start, ev.stop, 0, args...);
  if (ev.start != nullptr) ev.used = true;
}

enum KernelId : int {
  kKernelQkNormRopePrefill = 0,
  kKernelPrefillMfma = 1,
  kKernelPrefillFp32 = 2,
  kKernelDecodeSplit = 3,
  kKernelDecodeCombine = 4,
  kKernelQkNormRopeDecode = 5,
  kKernelAddRmsNorm = 6,
  kKernelGatherLast = 7,
  kKernelArgmaxPartial = 8,
  kKernelArgmaxFinal = 9,
  kKernelPrefillMfmaShifted = 10,
  kKernelFusedStep = 11,
  kNumKernels = 12,
};

// Paged K/V caches: slot s of request b is row s % P of page table[b][s / P]
// of a pool [num_pages, Hkv, P, D] (P = 1 << page_shift).  A null table means
// the contiguous caches [B, Hkv, S_cap, D].  Page numbers are clamped to the
// pool, so out-of-contract tables cannot address past it.
struct PagedTable {
  const int32_t* table = nullptr;  // int32 [num_seqs, pages_per_seq]
  int pages_per_seq = 0, page_shift = 0, num_pages = 0;
};

// Element offset of the first element of row s of request b, KV head g.
// kUniform: the row is the same for the whole wavefront; the table entry is
// then made wave-uniform, so a buffer resource formed from it stays in scalar
// registers (a resource in vector registers costs a waterfall loop around
// every load that uses it).
template <bool kUniform = false>
__device__ __forceinline__ size_t paged_row(const PagedTable& pt, int b, int g, int s, int num_kv_heads, int head_dim) {
  int page = pt.table[static_cast<size_t>(b) * pt.pages_per_seq + (s >> pt.page_shift)];
  if constexpr (kUniform) page = __builtin_amdgcn_readfirstlane(page);
  page = min(max(page, 0), pt.num_pages - 1);
  return ((static_cast<size_t>(page) * num_kv_heads + g) * (static_cast<size_t>(1) << pt.page_shift) +
          (s & ((1 << pt.page_shift) - 1))) * head_dim;
}
__device__ __forceinline__ size_t cache_row(const PagedTable& pt, int b, int g, int s, int num_kv_heads,
                                            int cache_capacity, int head_dim) {
  if (pt.table != nullptr) return paged_row(pt, b, g, s, num_kv_heads, head_dim);
  return ((static_cast<size_t>(b) * num_kv_heads + g) * cache_capacity + s) * head_dim;
}

// Kernel 1: per token row, RMSNorm + RoPE of the Q and K heads; q~ to
// q_out[row, Hq, D], k~ and v to the cache at (request, slot).
struct QkNormRopeArgs {
  const void* qkv;
  const void* q_norm_weight;
  const void* k_norm_weight;
  const int32_t* positions;
  const int32_t* seq_info;  // prefill: cu_seqlens[num_seqs+1]; decode: cache_lens[num_seqs]
  const int32_t* slot_offsets;  // prefill: per-request first slot (entries already cached), or null for 0
  int decode_mode;          // 0: slot = offset + in-request index; 1: row b, slot = cache_lens[b]
  int num_rows;
  int num_seqs;
  int num_q_heads, num_kv_heads, head_dim, dtype, cache_capacity;
  float rms_eps;
  double log2_rope_base;
  void* q_out;              // q~ [rows, Hq, D], or null when rope_table is set
  float* rope_table;        // prefill, bf16: per row D fp32, cos then sin (order in qknorm_rope.hip); Q heads skipped
  void* k_cache;
  void* v_cache;
  int32_t* plan;            // bf16 decode: one more block builds the split kernel's plan there (or null)
  int plan_units, plan_nchunks;
  PagedTable paged;         // table null: contiguous caches
};
hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, hipStream_t stream);
// A bf16 prefill batch (rope table, no history) and a bf16 decode batch (with its plan) in one launch; both
// contiguous and with the same norm weights (the mixed step).
hipError_t launch_qknorm_rope_pair(const QkNormRopeArgs& prefill, const QkNormRopeArgs& decode, hipStream_t stream);

// Kernel 2: causal GQA attention over the prefill caches.  Request r's new token j
// sits at slot P_r + j and sees slots 0..P_r + j (P_r = past_lens[r], or 0).
struct PrefillAttnArgs {
  const void* q;            // q~ [N, Hq, D] (fp32 path)
  // bf16 path: Q comes raw from qkv and is normalised and rotated on load.
  const void* qkv;          // [N, (Hq + 2Hkv) D]
  const void* q_norm_weight;
  const void* k_norm_weight; // its largest |w| bounds every score (see prefill_mfma.hip)
  const float* rope_table;  // [N][D] fp32: cos then sin, in kernel 1's order
  float rms_eps;
  const void* k_cache;      // [B, Hkv, S, D]
  const void* v_cache;
  const int32_t* cu_seqlens;
  const int32_t* past_lens; // per request: entries cached before this chunk (null: none)
  void* out;                // [N, Hq*D]
  int num_q_heads, num_kv_heads, head_dim, cache_capacity, num_seqs, max_seqlen;
  float scale_log2;         // log2(e) / sqrt(D)
  PagedTable paged;         // table null: contiguous caches (k_cache/v_cache are the pools otherwise)
  bool single_path = false; // bf16: only one of the two prefill attention kernels is launched
  // bf16: work items ordered by query tile across the requests (heaviest first over the whole batch)
  // instead of request by request.  Set where no item can be empty: every request holds max_seqlen
  // tokens and none has history.
  bool tile_major = false;
};
// The largest max|w_q| * max|w_k| for which the unshifted bf16 prefill
// kernel takes a request (and every kernel computes this same value).
float prefill_unshifted_limit(int head_dim, float scale_log2);
// bf16: two kernels over the same grid, both launched by every call.
// unshifted = true launches the one that takes p = 2^s without a shift (a
// workgroup returns at once unless its request has no cached history and the
// norm weights bound the scores); false, the online-softmax one with a
// running max (it returns at once where the other runs).
hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, bool unshifted, hipStream_t stream);
hipError_t launch_prefill_attn_fp32(const PrefillAttnArgs& a, hipStream_t stream);

struct DecodeAttnArgs;
// The fused step (bf16): one launch whose first workgroups run the decode
// split over the plan built for kDecodeWaves wavefronts and whose other
// workgroups run the unshifted prefill's work items; supported for D = 64
// or 128 and G in {1, 2, 4, 8, 16} (fused_step_supported).  The running-max
// prefill kernel and the decode combine still follow it.
bool fused_step_supported(int head_dim, int group);
hipError_t launch_fused_step(const PrefillAttnArgs& a, const DecodeAttnArgs& d, hipStream_t stream);

// Kernels 3a/3b: split-KV decode attention and the log-sum-exp combine.
//
// fp32 (decode.hip): one workgroup per (request, KV-head chunk, split of
// kDecodeKeysPerSplit keys); partials [B, Hq, num_splits, D + 2] = (m, l, o[D]).
constexpr int kDecodeKeysPerSplit = 1024;  // keys per workgroup (4 wavefronts)

inline int decode_num_splits(int max_cache_len) {
  return (max_cache_len + 1 + kDecodeKeysPerSplit - 1) / kDecodeKeysPerSplit;
}

// bf16 (decode_mfma.hip): units (request, KV head, chunk of GW query heads)
// cut into steps of kDecodeStepKeys keys; the steps of all units are split
// evenly over kDecodeWaves persistent wavefronts (at least
// kDecodeMinStepsPerWave each).  One extra block of kernel 1's decode launch
// writes the plan [T, per, S0[0..N], first_unit[0..W)] (int32, decode_plan.h),
// 3a one partial record
// (m, l, pad, pad, o[D]) fp32 per (unit, wavefront) that meet, at slot
// unit + wavefront of [N + W, GW, D + 4].
constexpr int kDecodeStepKeys = 32;
constexpr int kDecodeWaves = 768;  // 192 workgroups of 4: faster than 512, 1024, 1536 or 2048 on both decode workloads
constexpr int kDecodeMinStepsPerWave = 8;

// Query heads per wavefront on the matrix-core path: the whole group if it
// fits in the 16 columns of the MFMA tile, else its largest divisor that does.
inline int decode_heads_per_wave(int group) {
  for (int c = 16; c >= 1; --c)
    if (group % c == 0) return c;
  return 1;
}

inline size_t decode_plan_ints(long long num_units) { return static_cast<size_t>(3 + num_units + kDecodeWaves); }

struct DecodeAttnArgs {
  const void* q;            // q~ [B, Hq, D]
  const void* k_cache;      // [B, Hkv, S, D]
  const void* v_cache;
  const int32_t* cache_lens;
  float* partials;          // fp32 partial records (layout per path, above)
  int32_t* plan;            // bf16 path: the step plan
  void* out;                // [B, Hq*D]
  int num_q_heads, num_kv_heads, head_dim, dtype, cache_capacity, num_seqs;
  int num_splits;           // fp32 path
  int num_units, heads_per_wave;  // bf16 path
  float scale_log2;
  PagedTable paged;         // table null: contiguous caches (k_cache/v_cache are the pools otherwise)
};
hipError_t launch_decode_split(const DecodeAttnArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeAttnArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeAttnArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma_combine(const DecodeAttnArgs& a, hipStream_t stream);

// Steps next to the attention layer (layer_ops.hip).
struct AddRmsNormArgs {
  const void* x;          // [N, C]
  void* residual;         // [N, C]: read when has_residual, written when has_residual or copy_residual
  const void* weight;     // [C]
  void* out;              // [N, C] (may be x itself)
  int num_tokens, hidden_size, dtype;
  int has_residual;       // 1: residual := x + residual; 0: residual := x
  int copy_residual;      // with has_residual 0: write x into residual (0 when they are one buffer)
  float rms_eps;
};
hipError_t launch_fused_add_rmsnorm(const AddRmsNormArgs& a, hipStream_t stream);

struct GatherLastArgs {
  const void* hidden;     // [num_rows, C]
  const int32_t* cu_seqlens;
  void* out;              // [num_seqs, C]
  int num_rows, num_seqs, hidden_size, dtype;
};
hipError_t launch_gather_last(const GatherLastArgs& a, hipStream_t stream);

struct ArgmaxArgs {
  const void* logits;     // row b at logits + b * row_stride elements, vocab entries each
  long long row_stride;
  int num_rows, vocab, dtype;
  int segments;           // per row; pass-1 records [num_rows, segments]
  float* part_v;
  int* part_i;
  int32_t* out;           // [num_rows]
};
int argmax_segments(int num_rows, int vocab);
int argmax_segment_length(int vocab, int segments);
hipError_t launch_argmax_partial(const ArgmaxArgs& a, hipStream_t stream);
hipError_t launch_argmax_final(const ArgmaxArgs& a, hipStream_t stream);

}  // namespace qkra
