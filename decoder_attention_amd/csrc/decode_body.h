// The work of one wavefront of the bf16 decode split (kernel 3a): its range
// of 32-key steps over the plan, with its K and V tiles at `ktile` and
// `vtile` (STEP rows of D + 8 elements each, in LDS).  Shared by the split
// kernel (decode_mfma.hip) and the decode role of the fused step kernel
// (prefill_mfma.hip).  The design notes are at the top of decode_mfma.hip.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace qkra {
namespace dbody {

constexpr int STEP = kDecodeStepKeys;  // keys per wavefront step
constexpr float TAU = 8.0f;            // lazy-rescale threshold (log2 units)

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(reinterpret_cast<__attribute__((address_space(3))) char*>(
          reinterpret_cast<uintptr_t>(p))));
}

// Max of a value over lanes l, l ^ 16, l ^ 32 and l ^ 48 (gfx950 row swaps).
__device__ __forceinline__ float quarter_max(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// ---- 3a: one wavefront per range of steps.
// kPaged: k_cache and v_cache are pools read through `paged` (a step's 32
// rows always lie in one page: pages hold a multiple of 32 slots).
template <int D, int GW, bool kPaged = false>
__device__ __forceinline__ void decode_wave(
    bf16* ktile, bf16* vtile, const int w,
    const bf16* __restrict__ q, const bf16* __restrict__ k_cache, const bf16* __restrict__ v_cache,
    const int32_t* __restrict__ cache_lens, const int32_t* __restrict__ plan, float* __restrict__ partials,
    int num_q_heads, int num_kv_heads, int cache_capacity, int chunks_per_kv, int num_units, float scale_log2,
    PagedTable paged = PagedTable{}) {
  constexpr int KS = D / 32;               // 32-d steps of the score product
  constexpr int DBLK = D / 16;             // 16-d blocks of the output
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int VLOADS = STEP * CPR / 64;  // 16-byte loads per lane per step, for K and for V
  constexpr int PREC = D + 4;              // floats per partial record: m, l, 2 pad, o[D]
  static_assert(GW <= 16, "at most 16 query heads per wavefront");
  // Per wavefront: one K tile and one V tile of STEP rows, each row padded by
  // 16 bytes, so that the A-operand reads of 16 K rows hit 16 distinct bank
  // quads and the transpose reads of 16 V rows cover every bank exactly twice
  // (the two-pass minimum for 512 bytes).
  constexpr int VROW = D + 8;              // elements per padded row
  constexpr int TILE = STEP * VROW;        // elements per tile

  const int lane = threadIdx.x & 63;
  // Plan entries and lengths are the same for every lane; readfirstlane keeps
  // them (and the buffer resources formed from them) in scalar registers even
  // where the compiler cannot use scalar loads for these pointers.
  const int total = __builtin_amdgcn_readfirstlane(plan[0]), per = __builtin_amdgcn_readfirstlane(plan[1]);
  const int32_t* S0 = plan + 2;
  const int first_unit = __builtin_amdgcn_readfirstlane(plan[3 + num_units + w]);
  if (first_unit < 0) return;  // idle wavefront (no barriers below)
  const int t0 = w * per;
  const int t1 = min(t0 + per, total);

  const int group = num_q_heads / num_kv_heads;
  const int nchunks = num_kv_heads * chunks_per_kv;
  const int l16 = lane & 15;  // query column / key row within a 16-key block
  const int lg = lane >> 4;   // lane group

  // Unit geometry (all wave-uniform).
  struct Unit {
    int s0, s1, nkeys, b, g, h0;
    const bf16* kb;  // contiguous caches: the unit's first row
    const bf16* vb;
  };
  auto unit_at = [&](int i) {
    Unit u;
    u.s0 = __builtin_amdgcn_readfirstlane(S0[i]);
    u.s1 = __builtin_amdgcn_readfirstlane(S0[i + 1]);
    u.b = i / nchunks;
    const int hc = i % nchunks;
    const int g = hc / chunks_per_kv;
    u.g = g;
    u.h0 = g * group + (hc % chunks_per_kv) * GW;
    u.nkeys = min(__builtin_amdgcn_readfirstlane(cache_lens[u.b]) + 1, cache_capacity);
    const size_t head_off = (static_cast<size_t>(u.b) * num_kv_heads + g) * cache_capacity * D;
    u.kb = k_cache + head_off;
    u.vb = v_cache + head_off;
    return u;
  };

  // Q^T (B operand): slot (step s, group lg, e) <-> d = 32*s + 8*lg + e.
  bf16x8 qf[KS];
  auto load_q = [&](const Unit& u) {
    const bool valid = l16 < GW;
    const bf16* src = q + (static_cast<size_t>(u.b) * num_q_heads + u.h0 + (valid ? l16 : 0)) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(src + 32 * s);
      if (!valid) v = bf16x8{};
      qf[s] = v;
    }
  };

  f32x4 o[DBLK];
  float m_run, l_run;
  auto reset = [&]() {
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = f32x4{};
    m_run = kNegInf;
    l_run = 0.f;
  };

  // One step of K and V rows, loaded lane-linearly (each instruction reads
  // 1 KB of contiguous rows, 16 bytes per lane) with buffer loads over the
  // unit's keys: keys at or past n_b, or any key when `live` is false, read as
  // zero without touching memory (their scores are masked and their
  // probabilities are zero).
  const uint32_t lin = static_cast<uint32_t>(16 * lane);
  u32x4 kst[VLOADS], vst[VLOADS];
  auto load_step = [&](const Unit& u, int t, bool live) {
    const bf16* kb = u.kb;
    const bf16* vb = u.vb;
    uint32_t range = live ? static_cast<uint32_t>(u.nkeys) * (D * 2) : 0u;
    uint32_t off = lin + static_cast<uint32_t>(t - u.s0) * (STEP * D * 2);
    if constexpr (kPaged) {  // the step's rows, from the page that holds them
      const int key0 = (t - u.s0) * STEP;
      const size_t row = paged_row<true>(paged, u.b, u.g, key0, num_kv_heads, D);
      kb = k_cache + row;
      vb = v_cache + row;
      range = live ? static_cast<uint32_t>(min(u.nkeys - key0, STEP)) * (D * 2) : 0u;
      off = lin;
    }
    const auto krs = buffer_rsrc(kb, range);
    const auto vrs = buffer_rsrc(vb, range);
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {  // 16-byte chunk 64*i + lane of the step's rows
      kst[i] = buffer_load16<true>(krs, off + 1024 * i);
      vst[i] = buffer_load16<true>(vrs, off + 1024 * i);
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int c = 64 * i + lane;
      const int at = (c / CPR) * VROW + (c % CPR) * 8;
      *reinterpret_cast<u32x4*>(ktile + at) = kst[i];
      *reinterpret_cast<u32x4*>(vtile + at) = vst[i];
    }
  };

  // The transpose read of lane group lg covers key rows 4*lg + j/4 (first
  // half) and 16 + 4*lg + j/4 (second half), j = lane % 16.
  const int r1 = 4 * lg + (l16 >> 2);
  const int r2 = r1 + 16;
  auto step = [&](int key0, int nkeys) {
    // ---- scores: A operand of key block kblk, step s = K[16*kblk + l16][32*s + 8*lg ..]
    bf16x8 kf[2][KS];
#pragma unroll
    for (int kblk = 0; kblk < 2; ++kblk)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        kf[kblk][s] = *reinterpret_cast<const bf16x8*>(ktile + (16 * kblk + l16) * VROW + 32 * s + 8 * lg);
    f32x4 sc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int kblk = 0; kblk < 2; ++kblk)
        sc[kblk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kblk][s], qf[s], sc[kblk], 0, 0, 0);
    // ---- V^T operands, read while the softmax runs
    bf16x8 vf[DBLK];
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      const int col = 16 * db + 4 * (l16 & 3);  // element column read by this lane
      const s16x4 a0 = lds_read_tr16(vtile + r1 * VROW + col);
      const s16x4 a1 = lds_read_tr16(vtile + r2 * VROW + col);
      vf[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // ---- softmax: register t of the B operand holds key 4*lg + t (t < 4) or 16 + 4*lg + t-4
    float x[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int key = key0 + (t < 4 ? 4 * lg + t : 16 + 4 * lg + t - 4);
      x[t] = key < nkeys ? sc[t >> 2][t & 3] : kNegInf;
    }
    float mloc = x[0];
#pragma unroll
    for (int t = 1; t < 8; ++t) mloc = fmaxf(mloc, x[t]);
    mloc *= scale_log2;
    if (__any(mloc > m_run + TAU)) {  // rare: raise the max of the queries that need it
      const float mt = quarter_max(mloc);
      const bool up = mt > m_run + TAU;
      const float alpha = up ? fast_exp2(m_run - mt) : 1.0f;
      if (up) m_run = mt;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
    }
    uint32_t wpk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(__builtin_fmaf(x[2 * e], scale_log2, -m_run));
      const float p1 = fast_exp2(__builtin_fmaf(x[2 * e + 1], scale_log2, -m_run));
      wpk[e] = pack_bf16x2(p0, p1);
      l_run = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(wpk[e]),
                                              bf16x2{static_cast<bf16>(1.0f), static_cast<bf16>(1.0f)}, l_run, false);
    }
    const bf16x8 pf = __builtin_bit_cast(bf16x8, u32x4{wpk[0], wpk[1], wpk[2], wpk[3]});
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DBLK; ++db) o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pf, o[db], 0, 0, 0);
  };

  // Partial record of unit i's portion: lane l holds d = 16*db + 4*lg + r of
  // query l%16; l is summed over the four lane groups of a query.  Slot i + w
  // is unique per (unit, wavefront) pair that meet.
  auto write_partial = [&](int i) {
    float l_tot = l_run + xor_shuffle(l_run, 16);
    l_tot += xor_shuffle(l_tot, 32);
    if (l16 < GW) {
      float* rec = partials + (static_cast<size_t>(i + w) * GW + l16) * PREC;
      if (lg == 0) *reinterpret_cast<f32x2*>(rec) = f32x2{m_run, l_tot};
#pragma unroll
      for (int db = 0; db < DBLK; ++db) *reinterpret_cast<f32x4*>(rec + 4 + 16 * db + 4 * lg) = o[db];
    }
  };

  // Flat loop over the wavefront's steps; the loads of step t + 1 (possibly
  // of the next unit) are in flight while step t is computed from the tiles.
  int ci = first_unit;  // unit of the step being computed
  Unit cu = unit_at(ci);
  int pi = ci;          // unit of the step being loaded
  Unit pu = cu;
  load_q(cu);
  reset();
  load_step(pu, t0, true);
  store_step();
  for (int t = t0; t < t1; ++t) {
    const int tn = t + 1;
    const bool more = tn < t1;
    if (more && tn == pu.s1) pu = unit_at(++pi);
    load_step(pu, more ? tn : pu.s0, more);
    step((t - cu.s0) * STEP, cu.nkeys);
    if (tn == cu.s1 || !more) {
      write_partial(ci);
      if (more) {
        ci = pi;
        cu = pu;
        load_q(cu);
        reset();
      }
    }
    store_step();  // the step above has read the tiles
  }
}

}  // namespace dbody
}  // namespace qkra
