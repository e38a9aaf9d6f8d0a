// Host-side launch descriptors for the gfx950 kernels.  Every launcher enqueues
// on the given stream and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qkra {

enum KernelId : int {
  kKernelQkNormRopePrefill = 0,
  kKernelPrefillMfma = 1,
  kKernelPrefillFp32 = 2,
  kKernelDecodeSplit = 3,
  kKernelDecodeCombine = 4,
  kKernelQkNormRopeDecode = 5,
  kNumKernels = 6,
};

// Kernel 1: per token row, RMSNorm + RoPE of the Q and K heads; q~ to
// q_out[row, Hq, D], k~ and v to the cache at (request, slot).
struct QkNormRopeArgs {
  const void* qkv;
  const void* q_norm_weight;
  const void* k_norm_weight;
  const int32_t* positions;
  const int32_t* seq_info;  // prefill: cu_seqlens[num_seqs+1]; decode: cache_lens[num_seqs]
  int decode_mode;          // 0: slot = in-request index; 1: row b, slot = cache_lens[b]
  int num_rows;
  int num_seqs;
  int num_q_heads, num_kv_heads, head_dim, dtype, cache_capacity;
  float rms_eps;
  double log2_rope_base;
  void* q_out;
  void* k_cache;
  void* v_cache;
};
hipError_t launch_qknorm_rope(const QkNormRopeArgs& a, hipStream_t stream);

// Kernel 2: causal GQA attention over the prefill caches.
struct PrefillAttnArgs {
  const void* q;            // q~ [N, Hq, D]
  const void* k_cache;      // [B, Hkv, S, D]
  const void* v_cache;
  const int32_t* cu_seqlens;
  void* out;                // [N, Hq*D]
  int num_q_heads, num_kv_heads, head_dim, cache_capacity, num_seqs, max_seqlen;
  float scale_log2;         // log2(e) / sqrt(D)
};
hipError_t launch_prefill_attn_bf16(const PrefillAttnArgs& a, hipStream_t stream);
hipError_t launch_prefill_attn_fp32(const PrefillAttnArgs& a, hipStream_t stream);

// Kernels 3a/3b: split-KV decode attention and the log-sum-exp combine.
constexpr int kDecodeKeysPerSplit = 1024;  // keys per workgroup (4 wavefronts x 256)

inline int decode_num_splits(int max_cache_len) {
  return (max_cache_len + 1 + kDecodeKeysPerSplit - 1) / kDecodeKeysPerSplit;
}

struct DecodeAttnArgs {
  const void* q;            // q~ [B, Hq, D]
  const void* k_cache;      // [B, Hkv, S, D]
  const void* v_cache;
  const int32_t* cache_lens;
  float* partials;          // [B, Hq, num_splits, D + 2] fp32: (m, l, o[D])
  void* out;                // [B, Hq*D]
  int num_q_heads, num_kv_heads, head_dim, dtype, cache_capacity, num_seqs, num_splits;
  float scale_log2;
};
hipError_t launch_decode_split(const DecodeAttnArgs& a, hipStream_t stream);
hipError_t launch_decode_combine(const DecodeAttnArgs& a, hipStream_t stream);

}  // namespace qkra
