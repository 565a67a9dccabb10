// Cross-lane sums without an LDS round trip, for gfx950 wave64.
#pragma once
#include <hip/hip_runtime.h>

namespace falcon {

// x of the lane a DPP control names within the lane's 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N = 1, 2, 4, 8 or 16 lanes: quad permutations, then
// the half-row and row mirrors, which pair the groups' halves as xor 4 and xor 8
// would (every lane of a group holds the same partial sum after each step).
template <int N>
__device__ __forceinline__ float lane_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "groups within a 16-lane row");
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// x plus the value of lane l ^ 16 (resp. l ^ 32), by the lane swaps of two
// registers a, b: v_permlane16_swap exchanges the odd 16-lane rows of a with the
// even rows of b, v_permlane32_swap the upper 32 lanes of a with the lower 32 of b.
// With a = b = x the two registers then hold the two partners' values in every
// lane.  Written out, so that the two copies are distinct registers; the nops
// cover the wait between a VALU write and the swap's read.  Call from code that
// every lane of the wave runs.
__device__ __forceinline__ float add_xor16(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float add_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return a + b;
}

// The same over N values: the lane swaps of four values at a time issued back to
// back between one pair of nops (the swaps of one block are independent).
__device__ __forceinline__ void add_xor16_4(float &x0, float &x1, float &x2, float &x3) {
  float a0 = x0, b0 = x0, a1 = x1, b1 = x1, a2 = x2, b2 = x2, a3 = x3, b3 = x3;
  asm volatile(
      "s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\tv_permlane16_swap_b32 %2, %3\n\t"
      "v_permlane16_swap_b32 %4, %5\n\tv_permlane16_swap_b32 %6, %7\n\ts_nop 1"
      : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
  x0 = a0 + b0;
  x1 = a1 + b1;
  x2 = a2 + b2;
  x3 = a3 + b3;
}
__device__ __forceinline__ void add_xor32_4(float &x0, float &x1, float &x2, float &x3) {
  float a0 = x0, b0 = x0, a1 = x1, b1 = x1, a2 = x2, b2 = x2, a3 = x3, b3 = x3;
  asm volatile(
      "s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\t"
      "v_permlane32_swap_b32 %4, %5\n\tv_permlane32_swap_b32 %6, %7\n\ts_nop 1"
      : "+v"(a0), "+v"(b0), "+v"(a1), "+v"(b1), "+v"(a2), "+v"(b2), "+v"(a3), "+v"(b3));
  x0 = a0 + b0;
  x1 = a1 + b1;
  x2 = a2 + b2;
  x3 = a3 + b3;
}
template <int N>
__device__ __forceinline__ void add_xor16_all(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i + 4 <= N; i += 4) add_xor16_4(x[i], x[i + 1], x[i + 2], x[i + 3]);
#pragma unroll
  for (int i = N - N % 4; i < N; ++i) x[i] = add_xor16(x[i]);
}
template <int N>
__device__ __forceinline__ void add_xor32_all(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i + 4 <= N; i += 4) add_xor32_4(x[i], x[i + 1], x[i + 2], x[i + 3]);
#pragma unroll
  for (int i = N - N % 4; i < N; ++i) x[i] = add_xor32(x[i]);
}

}  // namespace falcon
