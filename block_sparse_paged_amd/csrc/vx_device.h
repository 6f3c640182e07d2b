// Device helpers shared by the libvx kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vx {

typedef uint16_t bf16_t;   // storage type of bfloat16 values

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- conversion
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (the compiler lowers the __bf16
// conversion to gfx950's hardware convert).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// Per-dtype view of a 16-byte vector: E elements, unpacked to fp32.
template <typename T> struct Vec16;

template <> struct Vec16<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};

template <> struct Vec16<bf16_t> {
  static constexpr int E = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
  }
  __device__ __forceinline__ static float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }
  __device__ __forceinline__ static bf16_t from_f32(float x) { return f32_to_bf16(x); }
};

// 2^x on the hardware exponential (v_exp_f32): results below the smallest
// normal float flush to 0, and 2^-inf is 0.  Softmax weights that small carry
// nothing, so the attention softmaxes use it instead of exp2f, whose
// subnormal range reduction costs three more instructions per call.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Online softmax with a lazy reference: the running output and denominator
// are rescaled only when some head's maximum logit (log2 units) rises more
// than this above the reference they share; below it the weights exp2(s -
// reference) stay under 2^kLazyRescale, and the final output o / l is the
// same softmax whatever the reference.
constexpr float kLazyRescale = 8.f;

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// ---------------------------------------------------------------- DPP
// Data-parallel-primitive lane moves (VALU, no LDS traffic).  Controls:
// quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), [2,3,0,1] = 0x4E (lane ^ 2),
// row_half_mirror = 0x141 (i <-> 7-i within 8), row_mirror = 0x140
// (i <-> 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W in {1, 2, 4, 8, 16}), every lane of
// the group receiving the total.
template <int W>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (W >= 2) x += dpp_mov<0xB1>(x);
  if constexpr (W >= 4) x += dpp_mov<0x4E>(x);
  if constexpr (W >= 8) x += dpp_mov<0x141>(x);
  if constexpr (W >= 16) x += dpp_mov<0x140>(x);
  return x;
}

// Sum over aligned groups of W lanes for any power of two W <= 64.
template <int W>
__device__ __forceinline__ float lane_group_sum(float x) {
  x = row_sum<(W < 16 ? W : 16)>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (W >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

// ---------------------------------------------------------------- reductions
// All-reduce over aligned groups of W consecutive lanes (W a power of two).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// All-reduce across the groups: lanes l, l^W, l^2W, ... (W a power of two).
template <int W>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
  for (int m = W; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int W>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
  for (int m = W; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// Integer DPP move; rows not in ROW_MASK and lanes whose source lies outside
// their row read 0.  Controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142
// (lane 15 of each row to the next row), row_bcast:31 = 0x143 (lane 31 to
// rows 2 and 3), plus the quad_perm / mirror controls above.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_int(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4, 8
// within each row of 16 lanes, then each row adds the totals of the rows
// below it through the two row broadcasts.
__device__ __forceinline__ int row_inclusive_scan(int x);

__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x = row_inclusive_scan(x);
  x += dpp_int<0x142, 0xA>(x);
  x += dpp_int<0x143, 0xC>(x);
  return x;
}

// Inclusive prefix sum within each row of 16 lanes.
__device__ __forceinline__ int row_inclusive_scan(int x) {
  x += dpp_int<0x111>(x);
  x += dpp_int<0x112>(x);
  x += dpp_int<0x114>(x);
  x += dpp_int<0x118>(x);
  return x;
}

}  // namespace vx
