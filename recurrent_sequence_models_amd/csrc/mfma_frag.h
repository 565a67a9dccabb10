// 16x16 MFMA fragments for gfx950 (CDNA4, wave64).
//
// Every 16x16 tile lives in one uniform per-lane layout of 4 values, with
// lane l = 16*g + c (g = l / 16 in 0..3, c = l % 16):
//
//   C-layout of M : lane holds M[4g + i][c],  i = 0..3     (accumulators, B operand)
//   A-layout of M : lane holds M[c][4g + i]                (= C-layout of M^T)
//
// mma16(D, a, b) adds A(16x16) * B(16x16) to D, with A given in A-layout and B
// in C-layout.  Because the result D comes out in C-layout, which is exactly
// the B-operand layout, a product can feed the next product without a trip
// through LDS; and the C-layout of M^T is the A-layout of M.
//
//  * bf16: one v_mfma_f32_16x16x32_bf16 whose upper four k-slots per lane are
//    zero (see below).
//  * fp32: four v_mfma_f32_16x16x4_f32, instruction i taking k = 4g + i.
// mma32 sums two k-blocks of 16.  For bf16 it is one v_mfma_f32_16x16x32_bf16
// whose 8 k-slots per lane are filled with the lane's 4 k of each block; the
// assignment of actual k to slots only has to be the same for A and B, which
// it is by construction.
//
// All bf16 products use the one 16x16x32 opcode, so every accumulation chain
// is a same-opcode chain.  A 16x16x16 bf16 MFMA accumulating onto the result
// of a directly preceding 16x16x32 one gave wrong output rows in the parity
// tests of these kernels; with the single opcode they pass.
#pragma once
#include <hip/hip_runtime.h>

namespace falcon {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

template <typename T> struct Op;
template <> struct Op<float> { typedef f4 frag; };
template <> struct Op<__bf16> { typedef bf4 frag; };

// Round-to-nearest-even fp32 -> bf16 as one vector conversion (two packed
// v_cvt_pk_bf16_f32), not four scalar conversions that then need repacking.
__device__ __forceinline__ bf4 to_op(const f4 &x, __bf16) { return __builtin_convertvector(x, bf4); }
__device__ __forceinline__ f4 to_op(const f4 &x, float) { return x; }
__device__ __forceinline__ f4 to_f4(const bf4 &x) { return f4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }
__device__ __forceinline__ f4 to_f4(const f4 &x) { return x; }

template <typename OpT>
__device__ __forceinline__ typename Op<OpT>::frag cvt(const f4 &x) { return to_op(x, OpT()); }

__device__ __forceinline__ void mma16(f4 &d, const bf4 &a, const bf4 &b) {
  const bf8 a8 = {a[0], a[1], a[2], a[3], (__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  const bf8 b8 = {b[0], b[1], b[2], b[3], (__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
  d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, d, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f4 &d, const f4 &a, const f4 &b) {
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], d, 0, 0, 0);
  d = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], d, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f4 &d, const bf4 &a0, const bf4 &a1, const bf4 &b0, const bf4 &b1) {
  bf8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  bf8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f4 &d, const f4 &a0, const f4 &a1, const f4 &b0, const f4 &b1) {
  mma16(d, a0, b0);
  mma16(d, a1, b1);
}

// Four consecutive operands from LDS (8-byte aligned for bf16, 16 for fp32).
__device__ __forceinline__ bf4 ld4(const __bf16 *p) { return *reinterpret_cast<const bf4 *>(p); }
__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }

// A-layout fragment of the 16x16 block at (r0, c0) of a row-major LDS matrix.
template <typename OpT>
__device__ __forceinline__ typename Op<OpT>::frag lda(const OpT *m, int ld, int r0, int c0, int lane) {
  return ld4(m + (r0 + (lane & 15)) * ld + c0 + 4 * (lane >> 4));
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// ---- Pairs of k-blocks --------------------------------------------------------
// A "pair" holds a lane's operands for two k-blocks of 16 (k = 4g+i of block 0 in
// `lo`, of block 1 in `hi`).  In LDS a pair is 8 consecutive elements when the k
// axis is stored permuted within groups of 32: logical k = 16h + 4g + i lives at
// position 8g + 4h + i (kperm), so one 16-byte read fills a 16x16x32 operand.
__device__ __forceinline__ int kperm(int k) { return (k & ~31) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3); }

template <typename T> struct Pair;
template <> struct Pair<__bf16> { bf8 v; };
template <> struct Pair<float> { f4 lo, hi; };

__device__ __forceinline__ Pair<__bf16> ldp(const __bf16 *p) { return {*reinterpret_cast<const bf8 *>(p)}; }
__device__ __forceinline__ Pair<float> ldp(const float *p) {
  return {*reinterpret_cast<const f4 *>(p), *reinterpret_cast<const f4 *>(p + 4)};
}
__device__ __forceinline__ Pair<__bf16> mkp(const bf4 &lo, const bf4 &hi) {
  return {bf8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}};
}
__device__ __forceinline__ Pair<float> mkp(const f4 &lo, const f4 &hi) { return {lo, hi}; }
__device__ __forceinline__ void mmap(f4 &d, const Pair<__bf16> &a, const Pair<__bf16> &b) {
  d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, d, 0, 0, 0);
}
__device__ __forceinline__ void mmap(f4 &d, const Pair<float> &a, const Pair<float> &b) {
  mma16(d, a.lo, b.lo);
  mma16(d, a.hi, b.hi);
}

// ---- Transposing LDS read (gfx950 ds_read_b64_tr_b16) ---------------------------
// Within each group of 16 lanes, lane j names 4 consecutive 16-bit elements of
// row j/4 (columns 4(j%4)..+3) of a 4x16 block; lane c receives column c of that
// block (its 4 rows).  Pointed at rows r0..r0+3 of a row-major matrix, it yields
// the A-layout fragment of the transposed 16x4 slice, or the C-layout fragment
// of a 4x16 slice, without a transposed copy in LDS.
__device__ __forceinline__ bf4 ldtr(const __bf16 *p) {
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(p));
  return __builtin_bit_cast(bf4, v);
}

}  // namespace falcon
