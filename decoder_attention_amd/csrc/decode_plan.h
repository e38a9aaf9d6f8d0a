// The bf16 decode's step plan: which wavefront computes which keys.
//
// Units (request, KV head, chunk of GW query heads) are cut into steps of
// kDecodeStepKeys keys and laid end to end; the T steps are split evenly over
// kDecodeWaves wavefronts (at least kDecodeMinStepsPerWave each).  The plan is
// [T, per, S0[0..N], first_unit[0..W)] (int32): S0[i] is the first global step
// of unit i (S0[N] = T), per the steps per wavefront, first_unit[w] the unit
// holding step w*per (-1: an idle wavefront).  One workgroup builds it: kernel
// 1's decode launch runs it as one extra block beside the token blocks.
#pragma once

#include "launch.h"

namespace qkra {

// Steps of one request's units.  Consecutive units mostly share a request, so
// a thread reads each length once (a load per unit made the plan block slower
// than the token blocks beside it).
struct UnitSteps {
  const int32_t* cache_lens;
  int nchunks, cache_capacity;
  int b = -1, steps = 0;
  __device__ int operator()(int unit) {
    const int ub = unit / nchunks;
    if (ub != b) {
      b = ub;
      const int nkeys = min(cache_lens[ub] + 1, cache_capacity);
      steps = (nkeys + kDecodeStepKeys - 1) / kDecodeStepKeys;
    }
    return steps;
  }
};

// THREADS threads of one workgroup; s_scan is THREADS ints of LDS.
template <int THREADS>
__device__ void build_decode_plan(const int32_t* __restrict__ cache_lens, int32_t* __restrict__ plan, int num_units,
                                  int nchunks, int cache_capacity, int32_t* s_scan) {
  constexpr int num_waves = kDecodeWaves;
  const int tid = threadIdx.x;
  const int per_thread = (num_units + THREADS - 1) / THREADS;
  const int i0 = min(tid * per_thread, num_units);
  const int i1 = min(i0 + per_thread, num_units);
  UnitSteps unit_steps{cache_lens, nchunks, cache_capacity};
  int local = 0;
  for (int i = i0; i < i1; ++i) local += unit_steps(i);
  s_scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < THREADS; off <<= 1) {  // inclusive scan of the per-thread sums
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int32_t* S0 = plan + 2;
  int32_t* first = plan + 3 + num_units;
  const int total = s_scan[THREADS - 1];
  const int per = max((total + num_waves - 1) / num_waves, kDecodeMinStepsPerWave);
  // Each thread records the first steps of its units and, for every unit, the
  // wavefronts whose first step w*per falls inside it: w in
  // [ceil(S0_i / per), ceil((S0_i + steps_i) / per)).  No search, no barrier.
  int run = s_scan[tid] - local;
  for (int i = i0; i < i1; ++i) {
    const int steps = unit_steps(i);
    S0[i] = run;
    const long long wlo = (static_cast<long long>(run) + per - 1) / per;
    const long long whi = min((static_cast<long long>(run) + steps + per - 1) / per, static_cast<long long>(num_waves));
    for (long long w = wlo; w < whi; ++w) first[w] = i;
    run += steps;
  }
  if (tid == 0) {
    plan[0] = total;
    plan[1] = per;
    S0[num_units] = total;
  }
  for (int w = tid; w < num_waves; w += THREADS)  // wavefronts past the last step stay idle
    if (static_cast<long long>(w) * per >= total) first[w] = -1;
}

}  // namespace qkra
