// Segment-parallel (two-level) form of the chunked forward pass for sequences
// too few to fill the GPU ([P1] 三种等价形式: the chunk map S_C = S_0 M + N is
// affine in the incoming state, so maps compose; [P2] 三种视角).
//
// A sequence of T steps is cut into P segments of T/P steps.  Viewing the
// arrays [B, T, H, d] as [B*P, T/P, H, d] (a plain reshape) makes every segment
// a sequence of its own.  For every variant whose state map is shared by all
// rows of S (F1, F1A, F2A, F3, F3A; not F2, whose step differs per row), a
// segment maps its incoming state S_0 to S_0 M + N.  Then:
//   1. forward from S_0 = 0 on all segments at once          -> N
//   2. forward from S_0 = I                                   -> M + N
//   3. S_start[p] = S_start[p-1] M_{p-1} + N_{p-1}, p = 1..P-1 (this file)
//   4. forward from S_start on all segments at once           -> o and the final state
// Passes 1 and 2 write no outputs.  The key and window pairs entering each
// segment come straight from the inputs (this file), since they do not depend
// on the state.
#include "falcon_kernels.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

// The carried key (and window pairs) entering every segment: segment p > 0 takes
// x_prev = phi(k) of its previous step and the Bw-1 pairs before it; segment 0
// takes the caller's (zeros when there is none).  One wave per (b, p, h).
template <typename IT>
__global__ __launch_bounds__(64) void seg_boundary(SegArgs a) {
  const int id = blockIdx.x;  // ((b * P + p) * H + h)
  const int h = id % a.H, bp = id / a.H, p = bp % a.P, b = bp / a.P;
  const int lane = threadIdx.x;
  const int D = a.dk, DV = a.dv, W1 = a.window - 1;
  const int Ts = a.T / a.P;
  const size_t bh = (size_t)b * a.H + h;
  auto feature_row = [&](int tok, float *dst) {  // dst = phi(k[b, tok, h])
    const IT *kp = (const IT *)a.k + ((size_t)(b * a.T + tok) * a.H + h) * D;
    float v0 = lane < D ? (float)kp[lane] : 0.f;
    float v1 = lane + 64 < D ? (float)kp[lane + 64] : 0.f;
    float s = v0 * v0 + v1 * v1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
    const float inv = 1.f / sqrtf(s + a.eps_phi);
    if (lane < D) dst[lane] = v0 * inv;
    if (lane + 64 < D) dst[lane + 64] = v1 * inv;
  };
  float *xo = a.xseg + (size_t)id * D;
  if (p == 0) {
    for (int e = lane; e < D; e += 64) xo[e] = a.xprev0 ? a.xprev0[bh * D + e] : 0.f;
    for (int u = 0; u < W1; ++u) {
      for (int e = lane; e < D; e += 64) a.wxseg[((size_t)id * W1 + u) * D + e] = a.winx0 ? a.winx0[(bh * W1 + u) * D + e] : 0.f;
      for (int e = lane; e < DV; e += 64) a.wvseg[((size_t)id * W1 + u) * DV + e] = a.winv0 ? a.winv0[(bh * W1 + u) * DV + e] : 0.f;
    }
    return;
  }
  const int t0 = p * Ts;  // first step of the segment
  feature_row(t0 - 1, xo);
  for (int u = 0; u < W1; ++u) {  // pair of step j = t0 - W1 + u (j >= 1 since Ts >= Bw)
    const int j = t0 - W1 + u;
    feature_row(j - 1 + a.align, a.wxseg + ((size_t)id * W1 + u) * D);
    const IT *vp = (const IT *)a.v + ((size_t)(b * a.T + j) * a.H + h) * DV;
    for (int e = lane; e < DV; e += 64) a.wvseg[((size_t)id * W1 + u) * DV + e] = (float)vp[e];
  }
}

// S = I for every segment (the incoming state of pass 2).
__global__ __launch_bounds__(256) void seg_identity(float *S, int dv, int dk) {
  float *m = S + (size_t)blockIdx.x * dv * dk;
  for (int e = threadIdx.x; e < dv * dk; e += 256) m[e] = (e / dk == e % dk) ? 1.f : 0.f;
}

// S_start[b, 0] = the caller's S (or 0); S_start[b, p] = S_start[b, p-1] (MN - N)[p-1] + N[p-1].
// Workgroup (b, h, 16 value rows); rows of S are independent.  The segment maps
// do not depend on the chain, so each step's M = MN - N is read into registers
// (coalesced 16-byte loads) while the previous product runs, then staged in LDS;
// wave w computes key-column tiles w, w+4, ... of the slab on fp32 MFMA, and the
// slab stays in LDS as the left operand of the next product.
template <int D>
__global__ __launch_bounds__(256) void seg_combine(SegArgs a) {
  constexpr int LDS_ = D + 4;
  constexpr int NCT = D / 16;            // key-column tiles
  constexpr int NT = (NCT + 3) / 4;      // tiles per wave
  constexpr int NV = D * D / 4 / 256;    // 16-byte vectors of M per thread
  __shared__ __attribute__((aligned(16))) float sS[16 * LDS_];
  __shared__ __attribute__((aligned(16))) float sM[D * LDS_];
  const int nslab = a.dv / 16;
  const int slab = blockIdx.x % nslab, bh = blockIdx.x / nslab;
  const int h = bh % a.H, b = bh / a.H;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int r0 = 16 * slab;
  auto seg_off = [&](int p) { return ((size_t)(b * a.P + p) * a.H + h) * a.dv * D; };
  // start: the caller's S
  for (int e = tid; e < 16 * D; e += 256) {
    const int r = e / D, cidx = e % D;
    const float v = a.S0 ? a.S0[((size_t)bh * a.dv + r0 + r) * D + cidx] : 0.f;
    sS[r * LDS_ + cidx] = v;
    a.Sseg[seg_off(0) + (size_t)(r0 + r) * D + cidx] = v;
  }
  f4 mreg[NV];   // M of the next step, this thread's vectors
  f4 nreg[NT];   // N of the next step at this lane's output elements
  auto fetch = [&](int p) {   // the maps of segment p
    const float *N = a.Nseg + seg_off(p), *MN = a.MNseg + seg_off(p);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = 4 * (tid + 256 * j);
      mreg[j] = *reinterpret_cast<const f4 *>(MN + e) - *reinterpret_cast<const f4 *>(N + e);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int ct = w + 4 * j;
#pragma unroll
      for (int i = 0; i < 4; ++i) nreg[j][i] = ct < NCT ? N[(size_t)(r0 + 4 * g + i) * D + 16 * ct + cc] : 0.f;
    }
  };
  if (a.P > 1) fetch(0);
  for (int p = 1; p < a.P; ++p) {
    __syncthreads();   // the previous product is done with sM; the slab in sS is complete
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int e = 4 * (tid + 256 * j);
      *reinterpret_cast<f4 *>(sM + (e / D) * LDS_ + e % D) = mreg[j];
    }
    f4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = nreg[j];
    if (p + 1 < a.P) fetch(p);   // in flight during this step's product
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int ct = w + 4 * j;
      if (ct < NCT) {
#pragma unroll
        for (int kb = 0; kb < NCT; ++kb) {
          const f4 sa = *reinterpret_cast<const f4 *>(sS + cc * LDS_ + 16 * kb + 4 * g);  // S[c][16kb+4g+i]
          f4 mb;  // M[16kb+4g+i][16ct+c]
#pragma unroll
          for (int i = 0; i < 4; ++i) mb[i] = sM[(16 * kb + 4 * g + i) * LDS_ + 16 * ct + cc];
          mma16(acc[j], sa, mb);
        }
      }
    }
    __syncthreads();  // every wave is done reading the previous slab
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int ct = w + 4 * j;
      if (ct < NCT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * g + i;
          sS[r * LDS_ + 16 * ct + cc] = acc[j][i];
          a.Sseg[seg_off(p) + (size_t)(r0 + r) * D + 16 * ct + cc] = acc[j][i];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_seg_boundary(bool bf16, const SegArgs &a, hipStream_t st) {
  const unsigned n = (unsigned)a.B * a.P * a.H;
  if (bf16) hipLaunchKernelGGL((seg_boundary<__bf16>), dim3(n), dim3(64), 0, st, a);
  else hipLaunchKernelGGL((seg_boundary<float>), dim3(n), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_seg_identity(float *S, int nmat, int dv, int dk, hipStream_t st) {
  hipLaunchKernelGGL(seg_identity, dim3((unsigned)nmat), dim3(256), 0, st, S, dv, dk);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const SegArgs &a, hipStream_t st) {
  const unsigned n = (unsigned)a.B * a.H * (a.dv / 16);
  switch (a.dk) {
    case 32: hipLaunchKernelGGL((seg_combine<32>), dim3(n), dim3(256), 0, st, a); break;
    case 64: hipLaunchKernelGGL((seg_combine<64>), dim3(n), dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL((seg_combine<128>), dim3(n), dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace falcon
