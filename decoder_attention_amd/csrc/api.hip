// C ABI of the attention library: host-side argument checks, workspace
// sizing and the launch sequence of each call.  Nothing here allocates
// device memory or synchronises the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/qknorm_rope_attn.h"
#include "launch.h"

namespace qkra {

thread_local LaunchEvents g_launch_events;

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int32_t dtype) { return dtype == QKRA_BF16 ? 2 : 4; }

int32_t check_config(const qkra_config* cfg) {
  if (cfg == nullptr) return QKRA_ERR_INVALID_ARGUMENT;
  if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (cfg->num_q_heads % cfg->num_kv_heads != 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (!(cfg->qk_weight_bound >= 0.0f) || !std::isfinite(cfg->qk_weight_bound)) return QKRA_ERR_INVALID_ARGUMENT;
  if (!(cfg->rms_eps >= 0.0f) || !std::isfinite(cfg->rms_eps)) return QKRA_ERR_INVALID_ARGUMENT;
  if (!(cfg->rope_base > 0.0) || !std::isfinite(cfg->rope_base)) return QKRA_ERR_INVALID_ARGUMENT;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return QKRA_ERR_UNSUPPORTED;
  if (cfg->dtype != QKRA_BF16 && cfg->dtype != QKRA_FP32) return QKRA_ERR_UNSUPPORTED;
  // Keep every index inside 32-bit signed arithmetic where the kernels use it.
  if (static_cast<long long>(cfg->num_q_heads + 2LL * cfg->num_kv_heads) * cfg->head_dim > (1LL << 24))
    return QKRA_ERR_UNSUPPORTED;
  return QKRA_OK;
}

// bf16: the per-token RoPE table [N][D] (fp32, cos then sin, in the order
// kernel 1 documents), from which the attention kernel rotates Q itself;
// fp32: q~ [N, Hq, D].
size_t prefill_workspace(const qkra_config* cfg, int64_t num_tokens) {
  if (cfg->dtype == QKRA_BF16) return align_up(static_cast<size_t>(num_tokens) * cfg->head_dim * sizeof(float));
  return align_up(static_cast<size_t>(num_tokens) * cfg->num_q_heads * cfg->head_dim * elem_size(cfg->dtype));
}

size_t decode_q_bytes(const qkra_config* cfg, int64_t num_seqs) {
  return align_up(static_cast<size_t>(num_seqs) * cfg->num_q_heads * cfg->head_dim * elem_size(cfg->dtype));
}

// bf16: units of (request, KV head, chunk of GW query heads).
int64_t decode_units(const qkra_config* cfg, int64_t num_seqs) {
  const int group = cfg->num_q_heads / cfg->num_kv_heads;
  return num_seqs * cfg->num_kv_heads * (group / decode_heads_per_wave(group));
}

size_t decode_plan_bytes(const qkra_config* cfg, int64_t num_seqs) {
  return align_up(decode_plan_ints(decode_units(cfg, num_seqs)) * sizeof(int32_t));
}

size_t decode_workspace(const qkra_config* cfg, int64_t num_seqs, int32_t max_cache_len) {
  if (cfg->dtype == QKRA_BF16) {
    const int gw = decode_heads_per_wave(cfg->num_q_heads / cfg->num_kv_heads);
    const size_t records = static_cast<size_t>(decode_units(cfg, num_seqs) + kDecodeWaves) * gw;
    return decode_q_bytes(cfg, num_seqs) + decode_plan_bytes(cfg, num_seqs) +
           align_up(records * (cfg->head_dim + 4) * sizeof(float));
  }
  const size_t splits = static_cast<size_t>(decode_num_splits(max_cache_len));
  return decode_q_bytes(cfg, num_seqs) +
         align_up(static_cast<size_t>(num_seqs) * cfg->num_q_heads * splits * (cfg->head_dim + 2) * sizeof(float));
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Paged caches (qkra_paged_cache).
size_t pool_bytes(const qkra_config* cfg, const PagedTable& pt) {
  return static_cast<size_t>(pt.num_pages) * cfg->num_kv_heads * (static_cast<size_t>(1) << pt.page_shift) *
         cfg->head_dim * elem_size(cfg->dtype);
}
size_t table_bytes(int32_t num_seqs, const PagedTable& pt) {
  return static_cast<size_t>(num_seqs) * pt.pages_per_seq * sizeof(int32_t);
}
// Checks the descriptor; on QKRA_OK, `pt` describes it and `capacity` is the
// slots each request's table row covers.
int32_t paged_view(const qkra_paged_cache* c, int32_t num_seqs, PagedTable* pt, int32_t* capacity) {
  if (c == nullptr || c->reserved != 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (c->num_pages <= 0 || c->pages_per_seq <= 0) return QKRA_ERR_INVALID_ARGUMENT;
  int shift = -1;
  for (int k = 6; k <= 10; ++k)
    if (c->page_size == (1 << k)) shift = k;
  if (shift < 0) return QKRA_ERR_UNSUPPORTED;  // 64, 128, 256, 512 or 1024 slots per page
  const long long cap = static_cast<long long>(c->pages_per_seq) * c->page_size;
  if (cap > 0x7fffffffLL || static_cast<long long>(num_seqs) * c->pages_per_seq > 0x7fffffffLL)
    return QKRA_ERR_UNSUPPORTED;
  if (!c->k_pool || !c->v_pool || (num_seqs > 0 && !c->block_table)) return QKRA_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(c->block_table) & 3u) != 0) return QKRA_ERR_INVALID_ARGUMENT;
  pt->table = c->block_table;
  pt->pages_per_seq = c->pages_per_seq;
  pt->page_shift = shift;
  pt->num_pages = c->num_pages;
  *capacity = static_cast<int32_t>(cap);
  return QKRA_OK;
}

// ---- per-kernel timing (benchmark instrumentation) ------------------------
// Process-wide: a pool of events is created when timing is switched on
// (qknorm_rope_attn_set_kernel_timing), so no call creates an event; a launch
// that finds the pool empty runs untimed.
constexpr int kTimingEvents = 8192;
struct TimingRecord {
  int kernel;
  hipEvent_t start, stop;
};
std::mutex g_timing_mu;
uint32_t g_timing_mask = 0;  // bit k: time kernel id k
std::vector<TimingRecord> g_timing_records;
std::vector<hipEvent_t> g_event_pool;
int g_events_created = 0;

template <typename Launch>
hipError_t timed(int kernel, hipStream_t stream, Launch&& launch) {
  (void)stream;
  hipEvent_t start = nullptr, stop = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_timing_mu);
    if (((g_timing_mask >> kernel) & 1u) == 0 || g_event_pool.size() < 2) return launch();
    start = g_event_pool.back();
    g_event_pool.pop_back();
    stop = g_event_pool.back();
    g_event_pool.pop_back();
  }
  g_launch_events = LaunchEvents{start, stop, false};
  const hipError_t err = launch();
  const bool used = g_launch_events.used;
  g_launch_events = LaunchEvents{};
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (err != hipSuccess || !used) {  // nothing launched (or the launch failed): the events go back
    g_event_pool.push_back(start);
    g_event_pool.push_back(stop);
    return err;
  }
  g_timing_records.push_back(TimingRecord{kernel, start, stop});
  return hipSuccess;
}

int32_t hip_status(hipError_t err) {
  if (err == hipSuccess) return QKRA_OK;
  g_last_hip_error = static_cast<int32_t>(err);
  return QKRA_ERR_HIP;
}

double log2_of(double base) { return std::log2(base); }

constexpr int kMaxNormHidden = 16 * 256 * 8;  // 16 pieces of 8 per thread, 256 threads

float softmax_scale_log2(int head_dim) {
  return static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(head_dim)));
}

// Which bf16 prefill attention kernels a call launches.
enum class SoftmaxPath { kBoth, kUnshifted, kShifted };
SoftmaxPath softmax_path(const qkra_config* cfg, const int32_t* cache_lens) {
  if (cfg->dtype != QKRA_BF16 || cache_lens != nullptr || cfg->qk_weight_bound <= 0.0f) return SoftmaxPath::kBoth;
  return cfg->qk_weight_bound <= prefill_unshifted_limit(cfg->head_dim, softmax_scale_log2(cfg->head_dim))
             ? SoftmaxPath::kUnshifted
             : SoftmaxPath::kShifted;
}

}  // namespace
}  // namespace qkra

using namespace qkra;

extern "C" {

QKRA_API size_t qknorm_rope_attn_workspace_bytes(const qkra_config* cfg, int32_t mode, int32_t n,
                                                 int32_t max_len) {
  if (check_config(cfg) != QKRA_OK || n < 0 || max_len < 0) return 0;
  if (mode == QKRA_MODE_PREFILL) return prefill_workspace(cfg, n);
  if (mode == QKRA_MODE_DECODE) return decode_workspace(cfg, n, max_len);
  return 0;
}

QKRA_API const char* qknorm_rope_attn_status_string(int32_t status) {
  switch (status) {
    case QKRA_OK: return "ok";
    case QKRA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case QKRA_ERR_UNSUPPORTED: return "unsupported head_dim or dtype";
    case QKRA_ERR_CAPACITY: return "cache capacity too small";
    case QKRA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QKRA_ERR_ALIASING: return "output or cache buffers overlap another buffer";
    case QKRA_ERR_HIP: return "HIP runtime error";
    case QKRA_ERR_SCRATCH_LIMIT: return "the call needs more than the fixed scratch of the no-allocation entry point";
    default: return "unknown status";
  }
}

QKRA_API int32_t qknorm_rope_attn_last_hip_error(void) { return g_last_hip_error; }

QKRA_API float qknorm_rope_attn_unshifted_weight_limit(int32_t head_dim) {
  if (head_dim != 64 && head_dim != 128) return 0.0f;
  return prefill_unshifted_limit(head_dim, softmax_scale_log2(head_dim));
}

QKRA_API int32_t qknorm_rope_attn_version(void) { return 400; }

}  // extern "C"

namespace {

// Prefill of packed requests onto caches holding cache_lens[r] entries each
// (cache_lens null: empty caches, max_cache_len 0).
// A bf16 prefill whose attention the fused step runs (qknorm_rope_attn_mixed_step).
struct DeferredPrefill {
  PrefillAttnArgs args{};
  bool set = false;
  QkNormRopeArgs k1{};  // kernel 1 of the prefill, launched with the decode's as one launch
  bool k1_set = false;
};

int32_t prefill_impl(const qkra_config* cfg, const void* qkv, const void* q_norm_weight, const void* k_norm_weight,
                     const int32_t* positions, const int32_t* cu_seqlens, const int32_t* cache_lens,
                     int32_t num_tokens, int32_t num_seqs, int32_t max_seqlen, int32_t max_cache_len,
                     void* k_cache, void* v_cache, int32_t cache_capacity, void* out, void* workspace,
                     size_t workspace_bytes, void* hip_stream, DeferredPrefill* defer = nullptr,
                     const PagedTable* paged = nullptr) {
  const int32_t cs = check_config(cfg);
  if (cs != QKRA_OK) return cs;
  if (num_tokens < 0 || num_seqs < 0 || max_seqlen < 0 || max_cache_len < 0 || cache_capacity < 0)
    return QKRA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return QKRA_OK;
  if (num_seqs == 0 || max_seqlen == 0 || max_seqlen > num_tokens) return QKRA_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(max_seqlen) * num_seqs < num_tokens) return QKRA_ERR_INVALID_ARGUMENT;
  if (static_cast<long long>(cache_capacity) < static_cast<long long>(max_cache_len) + max_seqlen)
    return QKRA_ERR_CAPACITY;
  if (!qkv || !q_norm_weight || !k_norm_weight || !positions || !cu_seqlens || !k_cache || !v_cache || !out)
    return QKRA_ERR_INVALID_ARGUMENT;
  const size_t need = prefill_workspace(cfg, num_tokens);
  if (workspace_bytes < need) return QKRA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return QKRA_ERR_INVALID_ARGUMENT;
  if (!aligned16(qkv) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(workspace))
    return QKRA_ERR_INVALID_ARGUMENT;

  const size_t es = elem_size(cfg->dtype);
  const size_t hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const Range r_qkv = range_of(qkv, num_tokens * (hq + 2 * hkv) * d * es);
  const Range r_out = range_of(out, num_tokens * hq * d * es);
  const size_t cache_bytes = paged ? pool_bytes(cfg, *paged) : static_cast<size_t>(num_seqs) * hkv * cache_capacity * d * es;
  const Range r_k = range_of(k_cache, cache_bytes), r_v = range_of(v_cache, cache_bytes);
  const Range r_ws = range_of(workspace, need);
  const Range r_wq = range_of(q_norm_weight, d * es), r_wk = range_of(k_norm_weight, d * es);
  const Range r_pos = range_of(positions, num_tokens * 4ull), r_cu = range_of(cu_seqlens, (num_seqs + 1ull) * 4);
  const Range r_len = range_of(cache_lens, cache_lens ? num_seqs * 4ull : 0);
  const Range r_tab = paged ? range_of(paged->table, table_bytes(num_seqs, *paged)) : Range{0, 0};
  for (Range w : {r_out, r_k, r_v, r_ws})
    for (Range r : {r_qkv, r_wq, r_wk, r_pos, r_cu, r_len, r_tab})
      if (overlap(w, r)) return QKRA_ERR_ALIASING;
  if (overlap(r_out, r_k) || overlap(r_out, r_v) || overlap(r_out, r_ws) || overlap(r_k, r_v) ||
      overlap(r_k, r_ws) || overlap(r_v, r_ws))
    return QKRA_ERR_ALIASING;

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  QkNormRopeArgs ka{};
  ka.qkv = qkv;
  ka.q_norm_weight = q_norm_weight;
  ka.k_norm_weight = k_norm_weight;
  ka.positions = positions;
  ka.seq_info = cu_seqlens;
  ka.slot_offsets = cache_lens;
  ka.decode_mode = 0;
  ka.num_rows = num_tokens;
  ka.num_seqs = num_seqs;
  ka.num_q_heads = cfg->num_q_heads;
  ka.num_kv_heads = cfg->num_kv_heads;
  ka.head_dim = cfg->head_dim;
  ka.dtype = cfg->dtype;
  ka.cache_capacity = cache_capacity;
  ka.rms_eps = cfg->rms_eps;
  ka.log2_rope_base = log2_of(cfg->rope_base);
  const bool fused_q = cfg->dtype == QKRA_BF16;
  ka.q_out = fused_q ? nullptr : workspace;
  ka.rope_table = fused_q ? static_cast<float*>(workspace) : nullptr;
  ka.k_cache = k_cache;
  ka.v_cache = v_cache;
  if (paged) ka.paged = *paged;
  // A bf16 prefill whose attention the fused step runs: kernel 1 goes out with the decode's, in one launch.
  const bool attn_deferred = defer && !paged && cfg->dtype == QKRA_BF16 && cache_lens == nullptr;
  hipError_t err = hipSuccess;
  if (attn_deferred) {
    defer->k1 = ka;
    defer->k1_set = true;
  } else {
    err = timed(kKernelQkNormRopePrefill, stream, [&] { return launch_qknorm_rope(ka, stream); });
    if (err != hipSuccess) return hip_status(err);
  }

  PrefillAttnArgs pa{};
  pa.q = workspace;
  pa.qkv = qkv;
  pa.q_norm_weight = q_norm_weight;
  pa.k_norm_weight = k_norm_weight;
  pa.rope_table = static_cast<const float*>(workspace);
  pa.rms_eps = cfg->rms_eps;
  pa.k_cache = k_cache;
  pa.v_cache = v_cache;
  pa.cu_seqlens = cu_seqlens;
  pa.past_lens = cache_lens;
  pa.out = out;
  pa.num_q_heads = cfg->num_q_heads;
  pa.num_kv_heads = cfg->num_kv_heads;
  pa.head_dim = cfg->head_dim;
  pa.cache_capacity = cache_capacity;
  pa.num_seqs = num_seqs;
  pa.max_seqlen = max_seqlen;
  pa.scale_log2 = softmax_scale_log2(cfg->head_dim);
  pa.tile_major = !cache_lens && num_seqs > 1 && static_cast<long long>(num_seqs) * max_seqlen == num_tokens;
  if (paged) pa.paged = *paged;
  // A plain bf16 prefill with the caller's weight bound launches only the softmax kernel it selects.
  const SoftmaxPath path = softmax_path(cfg, cache_lens);
  if (attn_deferred) {  // attention runs in the fused step
    // The fused launch is the unshifted kernel; only a bound selecting it spares the running-max launch.
    pa.single_path = path == SoftmaxPath::kUnshifted;
    defer->args = pa;
    defer->set = true;
    return QKRA_OK;
  }
  if (cfg->dtype == QKRA_BF16) {
    pa.single_path = path != SoftmaxPath::kBoth;
    if (path != SoftmaxPath::kShifted)
      err = timed(kKernelPrefillMfma, stream, [&] { return launch_prefill_attn_bf16(pa, true, stream); });
    if (err == hipSuccess && path != SoftmaxPath::kUnshifted)
      err = timed(kKernelPrefillMfmaShifted, stream, [&] { return launch_prefill_attn_bf16(pa, false, stream); });
  } else
    err = timed(kKernelPrefillFp32, stream, [&] { return launch_prefill_attn_fp32(pa, stream); });
  return hip_status(err);
}

}  // namespace

extern "C" {

QKRA_API int32_t qknorm_rope_attn_prefill(const qkra_config* cfg, const void* qkv, const void* q_norm_weight,
                                          const void* k_norm_weight, const int32_t* positions,
                                          const int32_t* cu_seqlens, int32_t num_tokens, int32_t num_seqs,
                                          int32_t max_seqlen, void* k_cache, void* v_cache,
                                          int32_t cache_capacity, void* out, void* workspace,
                                          size_t workspace_bytes, void* hip_stream) {
  return prefill_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, nullptr, num_tokens, num_seqs,
                      max_seqlen, 0, k_cache, v_cache, cache_capacity, out, workspace, workspace_bytes, hip_stream);
}

QKRA_API int32_t qknorm_rope_attn_prefill_append(const qkra_config* cfg, const void* qkv,
                                                 const void* q_norm_weight, const void* k_norm_weight,
                                                 const int32_t* positions, const int32_t* cu_seqlens,
                                                 const int32_t* cache_lens, int32_t num_tokens, int32_t num_seqs,
                                                 int32_t max_seqlen, int32_t max_cache_len, void* k_cache,
                                                 void* v_cache, int32_t cache_capacity, void* out,
                                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (num_tokens > 0 && !cache_lens) return QKRA_ERR_INVALID_ARGUMENT;
  return prefill_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens, num_tokens,
                      num_seqs, max_seqlen, max_cache_len, k_cache, v_cache, cache_capacity, out, workspace,
                      workspace_bytes, hip_stream);
}

namespace {

// The decode call.  validate_only: the argument checks alone (nothing is
// enqueued).  fused: a bf16 prefill whose attention runs in the same launch
// as the decode split (the fused step), then its running-max kernel.
int32_t decode_impl(const qkra_config* cfg, const void* qkv, const void* q_norm_weight, const void* k_norm_weight,
                    const int32_t* positions, const int32_t* cache_lens, int32_t num_seqs, int32_t max_cache_len,
                    void* k_cache, void* v_cache, int32_t cache_capacity, void* out, void* workspace,
                    size_t workspace_bytes, void* hip_stream, bool validate_only, const DeferredPrefill* fused,
                    const PagedTable* paged = nullptr) {
  const int32_t cs = check_config(cfg);
  if (cs != QKRA_OK) return cs;
  if (num_seqs < 0 || max_cache_len < 0 || cache_capacity < 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return QKRA_OK;
  if (static_cast<long long>(cache_capacity) < static_cast<long long>(max_cache_len) + 1) return QKRA_ERR_CAPACITY;
  if (!qkv || !q_norm_weight || !k_norm_weight || !positions || !cache_lens || !k_cache || !v_cache || !out)
    return QKRA_ERR_INVALID_ARGUMENT;
  if (cfg->dtype == QKRA_BF16) {  // the step plan counts in int32
    const long long steps = decode_units(cfg, num_seqs) * ((cache_capacity + kDecodeStepKeys - 1LL) / kDecodeStepKeys);
    if (steps + 2LL * kDecodeWaves * kDecodeMinStepsPerWave >= (1LL << 31)) return QKRA_ERR_UNSUPPORTED;
  }
  const size_t need = decode_workspace(cfg, num_seqs, max_cache_len);
  if (workspace_bytes < need) return QKRA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return QKRA_ERR_INVALID_ARGUMENT;
  if (!aligned16(qkv) || !aligned16(q_norm_weight) || !aligned16(k_norm_weight) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(workspace))
    return QKRA_ERR_INVALID_ARGUMENT;

  const size_t es = elem_size(cfg->dtype);
  const size_t hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
  const Range r_qkv = range_of(qkv, num_seqs * (hq + 2 * hkv) * d * es);
  const Range r_out = range_of(out, num_seqs * hq * d * es);
  const size_t cache_bytes = paged ? pool_bytes(cfg, *paged) : static_cast<size_t>(num_seqs) * hkv * cache_capacity * d * es;
  const Range r_k = range_of(k_cache, cache_bytes), r_v = range_of(v_cache, cache_bytes);
  const Range r_ws = range_of(workspace, need);
  const Range r_wq = range_of(q_norm_weight, d * es), r_wk = range_of(k_norm_weight, d * es);
  const Range r_pos = range_of(positions, num_seqs * 4ull), r_len = range_of(cache_lens, num_seqs * 4ull);
  const Range r_tab = paged ? range_of(paged->table, table_bytes(num_seqs, *paged)) : Range{0, 0};
  for (Range w : {r_out, r_k, r_v, r_ws})
    for (Range r : {r_qkv, r_wq, r_wk, r_pos, r_len, r_tab})
      if (overlap(w, r)) return QKRA_ERR_ALIASING;
  if (overlap(r_out, r_k) || overlap(r_out, r_v) || overlap(r_out, r_ws) || overlap(r_k, r_v) ||
      overlap(r_k, r_ws) || overlap(r_v, r_ws))
    return QKRA_ERR_ALIASING;
  if (validate_only) return QKRA_OK;

  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  QkNormRopeArgs ka{};
  ka.qkv = qkv;
  ka.q_norm_weight = q_norm_weight;
  ka.k_norm_weight = k_norm_weight;
  ka.positions = positions;
  ka.seq_info = cache_lens;
  ka.decode_mode = 1;
  ka.num_rows = num_seqs;
  ka.num_seqs = num_seqs;
  ka.num_q_heads = cfg->num_q_heads;
  ka.num_kv_heads = cfg->num_kv_heads;
  ka.head_dim = cfg->head_dim;
  ka.dtype = cfg->dtype;
  ka.cache_capacity = cache_capacity;
  ka.rms_eps = cfg->rms_eps;
  ka.log2_rope_base = log2_of(cfg->rope_base);
  ka.q_out = workspace;
  ka.k_cache = k_cache;
  ka.v_cache = v_cache;
  if (paged) ka.paged = *paged;
  char* ws = static_cast<char*>(workspace) + decode_q_bytes(cfg, num_seqs);
  if (cfg->dtype == QKRA_BF16) {  // kernel 1's launch also builds the split kernel's plan (one extra block)
    const int group = cfg->num_q_heads / cfg->num_kv_heads;
    ka.plan = reinterpret_cast<int32_t*>(ws);
    ka.plan_units = static_cast<int>(decode_units(cfg, num_seqs));
    ka.plan_nchunks = cfg->num_kv_heads * (group / decode_heads_per_wave(group));
  }
  hipError_t err;
  if (fused && fused->k1_set)  // the mixed step: the prefill's rows and these in one launch
    err = timed(kKernelQkNormRopePrefill, stream, [&] { return launch_qknorm_rope_pair(fused->k1, ka, stream); });
  else
    err = timed(kKernelQkNormRopeDecode, stream, [&] { return launch_qknorm_rope(ka, stream); });
  if (err != hipSuccess) return hip_status(err);

  DecodeAttnArgs da{};
  da.q = workspace;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.cache_lens = cache_lens;
  da.out = out;
  da.num_q_heads = cfg->num_q_heads;
  da.num_kv_heads = cfg->num_kv_heads;
  da.head_dim = cfg->head_dim;
  da.dtype = cfg->dtype;
  da.cache_capacity = cache_capacity;
  da.num_seqs = num_seqs;
  da.scale_log2 = softmax_scale_log2(cfg->head_dim);
  if (paged) da.paged = *paged;
  if (cfg->dtype == QKRA_BF16) {
    da.plan = reinterpret_cast<int32_t*>(ws);
    da.partials = reinterpret_cast<float*>(ws + decode_plan_bytes(cfg, num_seqs));
    da.num_units = static_cast<int>(decode_units(cfg, num_seqs));
    da.heads_per_wave = decode_heads_per_wave(cfg->num_q_heads / cfg->num_kv_heads);
    if (fused) {
      err = timed(kKernelFusedStep, stream, [&] { return launch_fused_step(fused->args, da, stream); });
      if (err != hipSuccess) return hip_status(err);
      // The running-max kernel takes the items the fused launch's unshifted prefill cannot; with the caller's
      // weight bound selecting the unshifted softmax there are none.
      if (!fused->args.single_path)
        err = timed(kKernelPrefillMfmaShifted, stream,
                    [&] { return launch_prefill_attn_bf16(fused->args, false, stream); });
    } else {
      err = timed(kKernelDecodeSplit, stream, [&] { return launch_decode_mfma(da, stream); });
    }
    if (err != hipSuccess) return hip_status(err);
    err = timed(kKernelDecodeCombine, stream, [&] { return launch_decode_mfma_combine(da, stream); });
    return hip_status(err);
  }
  da.partials = reinterpret_cast<float*>(ws);
  da.num_splits = decode_num_splits(max_cache_len);
  err = timed(kKernelDecodeSplit, stream, [&] { return launch_decode_split(da, stream); });
  if (err != hipSuccess) return hip_status(err);
  err = timed(kKernelDecodeCombine, stream, [&] { return launch_decode_combine(da, stream); });
  return hip_status(err);
}

}  // namespace

QKRA_API int32_t qknorm_rope_attn_decode(const qkra_config* cfg, const void* qkv, const void* q_norm_weight,
                                         const void* k_norm_weight, const int32_t* positions,
                                         const int32_t* cache_lens, int32_t num_seqs, int32_t max_cache_len,
                                         void* k_cache, void* v_cache, int32_t cache_capacity, void* out,
                                         void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, num_seqs, max_cache_len, k_cache,
                     v_cache, cache_capacity, out, workspace, workspace_bytes, hip_stream, false, nullptr);
}

QKRA_API int32_t qknorm_rope_attn_decode_paged(const qkra_config* cfg, const void* qkv, const void* q_norm_weight,
                                               const void* k_norm_weight, const int32_t* positions,
                                               const int32_t* cache_lens, int32_t num_seqs, int32_t max_cache_len,
                                               const qkra_paged_cache* cache, void* out, void* workspace,
                                               size_t workspace_bytes, void* hip_stream) {
  const int32_t cs = check_config(cfg);
  if (cs != QKRA_OK) return cs;
  if (num_seqs < 0 || max_cache_len < 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return QKRA_OK;
  PagedTable pt;
  int32_t capacity = 0;
  const int32_t st = paged_view(cache, num_seqs, &pt, &capacity);
  if (st != QKRA_OK) return st;
  return decode_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, num_seqs, max_cache_len,
                     cache->k_pool, cache->v_pool, capacity, out, workspace, workspace_bytes, hip_stream, false,
                     nullptr, &pt);
}

QKRA_API int32_t qknorm_rope_attn_prefill_append_paged(const qkra_config* cfg, const void* qkv,
                                                       const void* q_norm_weight, const void* k_norm_weight,
                                                       const int32_t* positions, const int32_t* cu_seqlens,
                                                       const int32_t* cache_lens, int32_t num_tokens,
                                                       int32_t num_seqs, int32_t max_seqlen, int32_t max_cache_len,
                                                       const qkra_paged_cache* cache, void* out, void* workspace,
                                                       size_t workspace_bytes, void* hip_stream) {
  const int32_t cs = check_config(cfg);
  if (cs != QKRA_OK) return cs;
  if (num_tokens < 0 || num_seqs < 0 || max_cache_len < 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return QKRA_OK;
  if (cache_lens == nullptr && max_cache_len != 0) return QKRA_ERR_INVALID_ARGUMENT;
  PagedTable pt;
  int32_t capacity = 0;
  const int32_t st = paged_view(cache, num_seqs, &pt, &capacity);
  if (st != QKRA_OK) return st;
  return prefill_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cu_seqlens, cache_lens, num_tokens, num_seqs,
                      max_seqlen, max_cache_len, cache->k_pool, cache->v_pool, capacity, out, workspace,
                      workspace_bytes, hip_stream, nullptr, &pt);
}

// ---- the decode entry point that allocates nothing ------------------------
// Its workspace is this file-scope device array: each GPU the library runs on
// holds its own copy (QKRA_NOALLOC_SCRATCH_BYTES) until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, taken once per device
// (with that device current) on the entry point's first call there.
static __device__ __align__(256) unsigned char scratch[QKRA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (QKRA_OK), or the HIP error.
int32_t device_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return hip_status(err);
  if (dev < 0 || dev >= kMaxDevices) return QKRA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return hip_status(err);
    if (p == nullptr) return QKRA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return QKRA_OK;
}
}  // namespace

QKRA_API int32_t qknorm_rope_attn_decode_noalloc(const qkra_config* cfg, const void* qkv, const void* q_norm_weight,
                                                 const void* k_norm_weight, const int32_t* positions,
                                                 const int32_t* cache_lens, int32_t num_seqs, int32_t max_cache_len,
                                                 void* k_cache, void* v_cache, int32_t cache_capacity, void* out,
                                                 void* hip_stream) {
  const int32_t cs = check_config(cfg);
  if (cs != QKRA_OK) return cs;
  if (num_seqs < 0 || max_cache_len < 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return QKRA_OK;
  // Sizes past the fixed scratch are refused before anything touches the GPU.
  if (qkra::decode_workspace(cfg, num_seqs, max_cache_len) > QKRA_NOALLOC_SCRATCH_BYTES) return QKRA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int32_t st = device_scratch(&ws);
  if (st != QKRA_OK) return st;
  // Nothing in the decode workspace needs to start at zero: every plan entry,
  // q~ row and partial record the kernels read is written earlier in the call.
  return decode_impl(cfg, qkv, q_norm_weight, k_norm_weight, positions, cache_lens, num_seqs, max_cache_len, k_cache,
                     v_cache, cache_capacity, out, ws, QKRA_NOALLOC_SCRATCH_BYTES, hip_stream, false, nullptr);
}

QKRA_API int32_t qknorm_rope_attn_mixed_step(
    const qkra_config* cfg, const void* q_norm_weight, const void* k_norm_weight,
    const void* prefill_qkv, const int32_t* prefill_positions, const int32_t* cu_seqlens, int32_t num_tokens,
    int32_t num_prefill_seqs, int32_t max_seqlen, void* prefill_k_cache, void* prefill_v_cache,
    int32_t prefill_cache_capacity, void* prefill_out, void* prefill_workspace, size_t prefill_workspace_bytes,
    const void* decode_qkv, const int32_t* decode_positions, const int32_t* cache_lens, int32_t num_decode_seqs,
    int32_t max_cache_len, void* decode_k_cache, void* decode_v_cache, int32_t decode_cache_capacity,
    void* decode_out, void* decode_workspace, size_t decode_workspace_bytes, void* hip_stream) {
  // Both halves' checks come first, so that nothing is enqueued for bad arguments.
  int32_t st = decode_impl(cfg, decode_qkv, q_norm_weight, k_norm_weight, decode_positions, cache_lens,
                           num_decode_seqs, max_cache_len, decode_k_cache, decode_v_cache, decode_cache_capacity,
                           decode_out, decode_workspace, decode_workspace_bytes, hip_stream, true, nullptr);
  if (st != QKRA_OK) return st;
  if (num_tokens < 0 || num_prefill_seqs < 0) return QKRA_ERR_INVALID_ARGUMENT;
  // The halves run at the same time: what one writes must not overlap anything the other touches.
  if (num_tokens > 0 && num_decode_seqs > 0) {
    const size_t es = elem_size(cfg->dtype);
    const size_t hq = cfg->num_q_heads, hkv = cfg->num_kv_heads, d = cfg->head_dim;
    const size_t pcache = static_cast<size_t>(num_prefill_seqs) * hkv * static_cast<size_t>(prefill_cache_capacity) * d * es;
    const size_t dcache = static_cast<size_t>(num_decode_seqs) * hkv * static_cast<size_t>(decode_cache_capacity) * d * es;
    // Each workspace counts with the bytes its half uses, as in that half's own checks (a caller may pass the
    // rest of one scratch arena as both workspaces).
    const size_t p_ws = std::min(qkra::prefill_workspace(cfg, num_tokens), prefill_workspace_bytes);
    const size_t d_ws = std::min(qkra::decode_workspace(cfg, num_decode_seqs, max_cache_len), decode_workspace_bytes);
    const Range p_w[] = {range_of(prefill_out, num_tokens * hq * d * es), range_of(prefill_k_cache, pcache),
                         range_of(prefill_v_cache, pcache), range_of(prefill_workspace, p_ws)};
    const Range d_w[] = {range_of(decode_out, num_decode_seqs * hq * d * es), range_of(decode_k_cache, dcache),
                         range_of(decode_v_cache, dcache), range_of(decode_workspace, d_ws)};
    const Range p_r[] = {range_of(prefill_qkv, num_tokens * (hq + 2 * hkv) * d * es),
                         range_of(prefill_positions, num_tokens * 4ull), range_of(cu_seqlens, (num_prefill_seqs + 1ull) * 4)};
    const Range d_r[] = {range_of(decode_qkv, num_decode_seqs * (hq + 2 * hkv) * d * es),
                         range_of(decode_positions, num_decode_seqs * 4ull), range_of(cache_lens, num_decode_seqs * 4ull)};
    for (const Range& w : p_w) {
      for (const Range& x : d_w)
        if (overlap(w, x)) return QKRA_ERR_ALIASING;
      for (const Range& x : d_r)
        if (overlap(w, x)) return QKRA_ERR_ALIASING;
    }
    for (const Range& w : d_w)
      for (const Range& x : p_r)
        if (overlap(w, x)) return QKRA_ERR_ALIASING;
  }
  const bool fuse = cfg->dtype == QKRA_BF16 && num_tokens > 0 && num_decode_seqs > 0 &&
                    fused_step_supported(cfg->head_dim, cfg->num_q_heads / cfg->num_kv_heads);
  DeferredPrefill deferred;
  st = prefill_impl(cfg, prefill_qkv, q_norm_weight, k_norm_weight, prefill_positions, cu_seqlens, nullptr, num_tokens,
                    num_prefill_seqs, max_seqlen, 0, prefill_k_cache, prefill_v_cache, prefill_cache_capacity,
                    prefill_out, prefill_workspace, prefill_workspace_bytes, hip_stream, fuse ? &deferred : nullptr);
  if (st != QKRA_OK) return st;
  return decode_impl(cfg, decode_qkv, q_norm_weight, k_norm_weight, decode_positions, cache_lens, num_decode_seqs,
                     max_cache_len, decode_k_cache, decode_v_cache, decode_cache_capacity, decode_out,
                     decode_workspace, decode_workspace_bytes, hip_stream, false, deferred.set ? &deferred : nullptr);
}

// ---- steps next to the attention layer ----------------------------------------

QKRA_API int32_t qknorm_rope_attn_fused_add_rmsnorm(int32_t dtype, float rms_eps, const void* x, void* residual,
                                                    int32_t has_residual, const void* weight, void* out,
                                                    int32_t num_tokens, int32_t hidden_size, void* hip_stream) {
  if (dtype != QKRA_BF16 && dtype != QKRA_FP32) return QKRA_ERR_UNSUPPORTED;
  if (!(rms_eps >= 0.0f) || !std::isfinite(rms_eps)) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_tokens < 0 || hidden_size <= 0 || hidden_size % 8 != 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (hidden_size > kMaxNormHidden) return QKRA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return QKRA_OK;
  if (!x || !residual || !weight || !out) return QKRA_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(residual) || !aligned16(weight) || !aligned16(out)) return QKRA_ERR_INVALID_ARGUMENT;
  const size_t rows = static_cast<size_t>(num_tokens) * hidden_size * elem_size(dtype);
  const Range r_x = range_of(x, rows), r_res = range_of(residual, rows), r_out = range_of(out, rows);
  const Range r_w = range_of(weight, static_cast<size_t>(hidden_size) * elem_size(dtype));
  const bool res_is_x = residual == x && !has_residual;
  if (out != x && overlap(r_out, r_x)) return QKRA_ERR_ALIASING;
  if (!res_is_x && overlap(r_res, r_x)) return QKRA_ERR_ALIASING;
  if (overlap(r_out, r_res) || overlap(r_out, r_w) || overlap(r_res, r_w)) return QKRA_ERR_ALIASING;
  AddRmsNormArgs a{};
  a.x = x;
  a.residual = residual;
  a.weight = weight;
  a.out = out;
  a.num_tokens = num_tokens;
  a.hidden_size = hidden_size;
  a.dtype = dtype;
  a.has_residual = has_residual ? 1 : 0;
  a.copy_residual = (!has_residual && !res_is_x) ? 1 : 0;
  a.rms_eps = rms_eps;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return hip_status(timed(kKernelAddRmsNorm, stream, [&] { return launch_fused_add_rmsnorm(a, stream); }));
}

QKRA_API int32_t qknorm_rope_attn_gather_last(int32_t dtype, const void* hidden, const int32_t* cu_seqlens,
                                              int32_t num_tokens, int32_t num_seqs, int32_t hidden_size, void* out,
                                              void* hip_stream) {
  if (dtype != QKRA_BF16 && dtype != QKRA_FP32) return QKRA_ERR_UNSUPPORTED;
  if (num_tokens < 0 || num_seqs < 0 || hidden_size <= 0) return QKRA_ERR_INVALID_ARGUMENT;
  const size_t row_bytes = static_cast<size_t>(hidden_size) * elem_size(dtype);
  if (row_bytes % 16 != 0 || row_bytes > (1u << 30)) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0) return QKRA_OK;
  if (!cu_seqlens || !out || (num_tokens > 0 && !hidden)) return QKRA_ERR_INVALID_ARGUMENT;
  if ((num_tokens > 0 && !aligned16(hidden)) || !aligned16(out) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
    return QKRA_ERR_INVALID_ARGUMENT;
  const Range r_out = range_of(out, num_seqs * row_bytes);
  if (overlap(r_out, range_of(hidden, num_tokens * row_bytes)) ||
      overlap(r_out, range_of(cu_seqlens, (num_seqs + 1ull) * 4)))
    return QKRA_ERR_ALIASING;
  GatherLastArgs a{};
  a.hidden = hidden;
  a.cu_seqlens = cu_seqlens;
  a.out = out;
  a.num_rows = num_tokens;
  a.num_seqs = num_seqs;
  a.hidden_size = hidden_size;
  a.dtype = dtype;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  return hip_status(timed(kKernelGatherLast, stream, [&] { return launch_gather_last(a, stream); }));
}

QKRA_API size_t qknorm_rope_attn_argmax_workspace_bytes(int32_t num_rows, int32_t vocab) {
  if (num_rows < 0 || vocab <= 0) return 0;
  const size_t recs = static_cast<size_t>(num_rows) * argmax_segments(std::max(num_rows, 1), vocab);
  return 2 * align_up(recs * 4);
}

QKRA_API int32_t qknorm_rope_attn_argmax(int32_t dtype, const void* logits, int32_t num_rows, int32_t vocab,
                                         int64_t row_stride, int32_t* out_index, void* workspace,
                                         size_t workspace_bytes, void* hip_stream) {
  if (dtype != QKRA_BF16 && dtype != QKRA_FP32) return QKRA_ERR_UNSUPPORTED;
  if (num_rows < 0 || vocab <= 0 || row_stride < vocab || row_stride % 8 != 0) return QKRA_ERR_INVALID_ARGUMENT;
  if (num_rows == 0) return QKRA_OK;
  if (!logits || !out_index) return QKRA_ERR_INVALID_ARGUMENT;
  const int segments = argmax_segments(num_rows, vocab);
  if (static_cast<long long>(num_rows) * segments >= (1LL << 31)) return QKRA_ERR_UNSUPPORTED;
  const size_t need = qknorm_rope_attn_argmax_workspace_bytes(num_rows, vocab);
  if (workspace_bytes < need) return QKRA_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return QKRA_ERR_INVALID_ARGUMENT;
  if (!aligned16(logits) || !aligned16(workspace) || (reinterpret_cast<uintptr_t>(out_index) & 3u))
    return QKRA_ERR_INVALID_ARGUMENT;
  const size_t es = elem_size(dtype);
  const Range r_in = range_of(logits, ((num_rows - 1) * static_cast<size_t>(row_stride) + vocab) * es);
  const Range r_idx = range_of(out_index, num_rows * 4ull), r_ws = range_of(workspace, need);
  if (overlap(r_idx, r_in) || overlap(r_ws, r_in) || overlap(r_idx, r_ws)) return QKRA_ERR_ALIASING;
  ArgmaxArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.num_rows = num_rows;
  a.vocab = vocab;
  a.dtype = dtype;
  a.segments = segments;
  a.part_v = static_cast<float*>(workspace);
  a.part_i = reinterpret_cast<int*>(static_cast<char*>(workspace) + need / 2);
  a.out = out_index;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t err = timed(kKernelArgmaxPartial, stream, [&] { return launch_argmax_partial(a, stream); });
  if (err != hipSuccess) return hip_status(err);
  return hip_status(timed(kKernelArgmaxFinal, stream, [&] { return launch_argmax_final(a, stream); }));
}

QKRA_API int32_t qknorm_rope_attn_set_kernel_timing(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  if (enable) {  // the pool is created once, here, and kept until the process ends
    for (; g_events_created < kTimingEvents; ++g_events_created) {
      hipEvent_t e = nullptr;
      const hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return hip_status(err);
      g_event_pool.push_back(e);
    }
  }
  g_timing_mask = static_cast<uint32_t>(enable);
  return QKRA_OK;
}

QKRA_API int32_t qknorm_rope_attn_read_kernel_timing(double* ms_total, int64_t* launches, int32_t max_kernels) {
  std::vector<TimingRecord> records;
  {
    std::lock_guard<std::mutex> lock(g_timing_mu);
    records.swap(g_timing_records);
  }
  for (int k = 0; k < max_kernels; ++k) {
    if (ms_total) ms_total[k] = 0.0;
    if (launches) launches[k] = 0;
  }
  int32_t status = kNumKernels;
  for (const TimingRecord& r : records) {
    float ms = 0.f;
    hipError_t err = hipEventSynchronize(r.stop);
    if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.start, r.stop);
    if (err != hipSuccess) {
      g_last_hip_error = static_cast<int32_t>(err);
      status = -QKRA_ERR_HIP;
    } else if (r.kernel < max_kernels) {
      if (ms_total) ms_total[r.kernel] += ms;
      if (launches) launches[r.kernel] += 1;
    }
  }
  std::lock_guard<std::mutex> lock(g_timing_mu);
  for (const TimingRecord& r : records) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  return status;
}

QKRA_API const char* qknorm_rope_attn_kernel_name(int32_t kernel_id) {
  switch (kernel_id) {
    case kKernelQkNormRopePrefill: return "qknorm_rope_kv_prefill";
    case kKernelQkNormRopeDecode: return "qknorm_rope_kv_decode";
    case kKernelPrefillMfma: return "prefill_attn_mfma_bf16";
    case kKernelPrefillMfmaShifted: return "prefill_attn_mfma_bf16_shifted";
    case kKernelFusedStep: return "fused_step_attn";
    case kKernelPrefillFp32: return "prefill_attn_fp32";
    case kKernelDecodeSplit: return "decode_attn_split";
    case kKernelDecodeCombine: return "decode_attn_combine";
    case kKernelAddRmsNorm: return "fused_add_rmsnorm";
    case kKernelGatherLast: return "gather_last";
    case kKernelArgmaxPartial: return "argmax_partial";
    case kKernelArgmaxFinal: return "argmax_final";
    default: return "unknown";
  }
}

}  // extern "C"
