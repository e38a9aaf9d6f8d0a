// Device-side helpers shared by the gfx950 kernels of the attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace qkra {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte / 8-byte integer vectors for raw loads and stores (HIP's
// uint4 is a struct whose copies go through memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();

// Raw 16-bit patterns <-> fp32 (bf16 is the upper half of an fp32).
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (round to nearest even, v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Reinterpret a 32-bit word as two bf16.  Takes the word by value: applying
// __builtin_bit_cast directly to an element of a native vector (v.y) reads
// element 0 with this compiler, so vector elements must pass through here.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane permute within rows of 16 lanes (DPP); CTRL is the dpp_ctrl encoding.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1.  Array indices
// inside f are compile-time constants from the start, so register arrays
// indexed there are split into scalars instead of being placed in memory.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(static_cast<F&&>(f), std::make_integer_sequence<int, N>{});
}

// Butterfly exchange across lanes (xor of the lane id) within a wavefront.
__device__ __forceinline__ float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Raw buffer resource over [base, base + bytes) (stride 0, 32-bit data format
// as gfx9-family untyped accesses require): a load at a byte offset >= bytes
// returns zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16-byte buffer load at a per-lane byte offset; NT marks it non-temporal.
template <bool NT>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, NT ? 2 : 0));
}

// 16 bytes per lane from a buffer straight into LDS (gfx950 buffer_load_dwordx4
// ... lds): lane i's piece lands at lds + 16 i bytes, so one instruction
// fills 1 KB of consecutive LDS.  An offset >= the resource's range writes
// zeros.  Counted by vmcnt, like any vector-memory load.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t offset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, offset, 0, 0, 0);
}

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt left at their maxima).
constexpr int kWaitVmcnt0 = 0x0F70;

}  // namespace qkra
