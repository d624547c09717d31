// device_common.h -- small gfx950 helpers shared by the dit_attn kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kBlock = 128;   // mask / fp8 scale block, in tokens
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, one L2 each

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero, which gives free bounds checks for ragged tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 positions away (lanes l and l^32 hold the two
// halves of one query row's keys in the 32x32 accumulator layout).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

// max(x[l], x[l ^ 32]) in every lane l, with one v_permlane32_swap: the
// swap of x with itself leaves x[l ^ 32] in the first result for the upper
// half of the lanes and in the second result for the lower half.
__device__ __forceinline__ float max_halves(float x) {
  const uint32_t xb = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const uint32_t other = (threadIdx.x & 32) ? r[0] : r[1];
  return fmaxf(x, __builtin_bit_cast(float, other));
}

// Work-group id -> logical tile id such that consecutive logical ids run on
// the same XCD.  Work-groups are dispatched round-robin over the XCDs, so
// physical id b lands on XCD b % 8; logical ids [x*per, (x+1)*per) are given
// to XCD x, keeping the query blocks of one (batch, head) -- which stream the
// same K/V -- inside one L2.
__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
  const int per = nwg / kXcds, rem = nwg % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair with one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + lo + hi of a packed bf16 pair (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x2(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

}  // namespace dit
