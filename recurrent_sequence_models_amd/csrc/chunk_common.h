// Device helpers shared by the chunked-forward kernels (fused and split):
// cross-lane reductions and scans, operand unpacking, the transposed operand
// read, and the per-wave tile assignment of the key-side products.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "mfma_frag.h"

namespace falcon {
namespace {

enum { V_F1 = 1, V_F1A = 2, V_F2 = 3, V_F2A = 4, V_F3 = 5, V_F3A = 6 };

// Hardware reciprocal square root / reciprocal (about 1 ulp); arguments are
// bounded away from zero and denormals by eps_phi and eps_eta.
__device__ __forceinline__ float safe_rsqrt(float s) { return s > 0.f ? __builtin_amdgcn_rsqf(s) : 0.f; }
__device__ __forceinline__ float fast_rcp(float s) { return __builtin_amdgcn_rcpf(s); }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

__device__ __forceinline__ void unpack(const uint4 &u, __bf16, float *out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(const uint4 &u, float, float *out) {
  out[0] = __uint_as_float(u.x); out[1] = __uint_as_float(u.y);
  out[2] = __uint_as_float(u.z); out[3] = __uint_as_float(u.w);
}

// `u` if `keep`, else zero, selected per component on values (a conditional
// expression on the uint4 objects themselves would select their addresses and
// force them into memory).
__device__ __forceinline__ uint4 keep_or_zero(bool keep, const uint4 &u) {
  return uint4{keep ? u.x : 0u, keep ? u.y : 0u, keep ? u.z : 0u, keep ? u.w : 0u};
}

// Completes this wave's outstanding LDS operations, so that values one lane wrote
// are visible to the other lanes of the same wave; also a compiler barrier.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Cross-lane moves inside a row of 16 lanes (DPP): no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_rows(float x) {  // lanes outside ROWMASK rows receive 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF, false));
}
// Sum over aligned groups of N consecutive lanes (N = 4, 8, 16, 32 or 64).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);                       // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                       // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp<0x111>(x);                      // row_shr:1 (lanes without a source add 0)
  x += dpp<0x112>(x);                      // row_shr:2
  x += dpp<0x114>(x);                      // row_shr:4
  x += dpp<0x118>(x);                      // row_shr:8
  x += dpp_rows<0x142, 0xA>(x);            // row_bcast:15 into rows 1 and 3
  x += dpp_rows<0x143, 0xC>(x);            // row_bcast:31 into rows 2 and 3
  return x;
}

// A-layout fragment of the transposed 16x16 block of a row-major matrix M:
// rows r0..r0+15 of M are the k axis, columns c0..c0+15 (given as the 4-column
// groups' physical offsets by `col4`) the M axis.  Lane (g, c) receives
// M[r0 + 4g + m][c0 + c], m = 0..3.
template <typename ColFn>
__device__ __forceinline__ bf4 ldT(const __bf16 *M, int ld, int r0, ColFn col4, int lane) {
  const int g = lane >> 4, j = lane & 15;
  return ldtr(M + (r0 + 4 * g + (j >> 2)) * ld + col4(j & 3));
}
template <typename ColFn>
__device__ __forceinline__ f4 ldT(const float *M, int ld, int r0, ColFn col4, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const int col = col4(c >> 2) + (c & 3);
  f4 r;
#pragma unroll
  for (int m = 0; m < 4; ++m) r[m] = M[(r0 + 4 * g + m) * ld + col];
  return r;
}

// Key-side tiles of one chunk, split over the four producer waves.  A wave
// gets the diagonal block `diag` (T_pp or A_pp, -1 if none) and up to four
// 16x16 tiles: Gram blocks A_pq (q < p) and score blocks P_pq (q <= p).  The
// tiles of a wave share few column blocks q, whose key rows are the left MFMA
// operand, and the diagonal block uses the same rows for both operands.
struct JobList {
  int diag, n;
  int isP[4], p[4], q[4];
};
constexpr JobList make_jobs(int nb, bool delta, int w) {
  JobList J{-1, 0, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  // (isP, p, q) triples per wave
  int t[4][4][3] = {};
  int n[4] = {0, 0, 0, 0};
  int dg[4] = {-1, -1, -1, -1};
  auto put = [&](int wv, int isP, int p, int q) { t[wv][n[wv]][0] = isP; t[wv][n[wv]][1] = p; t[wv][n[wv]][2] = q; ++n[wv]; };
  if (nb == 4) {
    if (delta) {
      dg[0] = 0; put(0, 0, 1, 0); put(0, 0, 2, 0); put(0, 0, 3, 0); put(0, 1, 0, 0);
      dg[1] = 3; put(1, 1, 1, 0); put(1, 1, 2, 0); put(1, 1, 3, 0); put(1, 1, 3, 3);
      dg[2] = 1; put(2, 0, 2, 1); put(2, 0, 3, 1); put(2, 1, 1, 1); put(2, 1, 2, 1);
      dg[3] = 2; put(3, 1, 3, 1); put(3, 0, 3, 2); put(3, 1, 2, 2); put(3, 1, 3, 2);
    } else {
      put(0, 1, 0, 0); put(0, 1, 1, 0); put(0, 1, 2, 0);
      put(1, 1, 3, 0); put(1, 1, 3, 3);
      put(2, 1, 1, 1); put(2, 1, 2, 1); put(2, 1, 3, 1);
      put(3, 1, 2, 2); put(3, 1, 3, 2);
    }
  } else if (nb == 2) {
    if (delta) {
      dg[0] = 0; put(0, 0, 1, 0);
      dg[1] = 1; put(1, 1, 1, 1);
      put(2, 1, 0, 0);
      put(3, 1, 1, 0);
    } else {
      put(0, 1, 0, 0); put(1, 1, 1, 0); put(2, 1, 1, 1);
    }
  } else {
    if (delta) dg[0] = 0;
    put(1, 1, 0, 0);
  }
  J.diag = dg[w];
  J.n = n[w];
  for (int j = 0; j < n[w]; ++j) {
    J.isP[j] = t[w][j][0];
    J.p[j] = t[w][j][1];
    J.q[j] = t[w][j][2];
  }
  return J;
}

// Score blocks with a window of bw pairs per step: the rows are the cs steps of a
// system (blocks of 16), the columns its 16*nb virtual rows (step r / bw).  Row
// block ps sees columns up to its last step, i.e. column blocks 0..score_qmax.
// With bw = 1 this is q <= ps.
constexpr int score_qmax(int ps, int nb, int cs, int bw) {
  const int smax = (16 * ps + 15 < cs - 1) ? 16 * ps + 15 : cs - 1;
  const int q = (smax * bw + bw - 1) / 16;
  return q < nb - 1 ? q : nb - 1;
}
// first fragment-pair slot of score-block row ps (pairs of column blocks)
constexpr int score_base(int ps, int nb, int cs, int bw) {
  int b = 0;
  for (int i = 0; i < ps; ++i) b += score_qmax(i, nb, cs, bw) / 2 + 1;
  return b;
}

// Tiles of a windowed system (nb <= 4 virtual-row blocks): one diagonal block per
// wave, then Gram and score tiles each to the least loaded wave.
constexpr JobList make_jobs_win(int nb, int cs, int bw, bool delta, int w) {
  JobList J{-1, 0, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  int t[4][4][3] = {};
  int n[4] = {0, 0, 0, 0}, load[4] = {0, 0, 0, 0};
  int dg[4] = {-1, -1, -1, -1};
  auto put = [&](int isP, int p, int q) {
    int k = 0;
    for (int i = 1; i < 4; ++i)
      if (load[i] < load[k]) k = i;
    t[k][n[k]][0] = isP; t[k][n[k]][1] = p; t[k][n[k]][2] = q;
    ++n[k];
    ++load[k];
  };
  if (delta) {
    for (int p = 0; p < nb; ++p) { dg[p] = p; load[p] = 1; }
    for (int p = 1; p < nb; ++p)
      for (int q = 0; q < p; ++q) put(0, p, q);
  }
  for (int ps = 0; ps < (cs + 15) / 16; ++ps)
    for (int q = 0; q <= score_qmax(ps, nb, cs, bw); ++q) put(1, ps, q);
  J.diag = dg[w];
  J.n = n[w];
  for (int j = 0; j < n[w]; ++j) {
    J.isP[j] = t[w][j][0];
    J.p[j] = t[w][j][1];
    J.q[j] = t[w][j][2];
  }
  return J;
}

}  // namespace
}  // namespace falcon
