// Chunked forward pass of Falcon-3 / 3A (a window of Bw pairs per step) on gfx950.
//
// Step definitions: [P1] Falcon家族 (sliding-window mini-batch of the last B pairs,
// residuals averaged) and [P2] 六个变体 (window average, not sum); the chunked
// evaluation follows [P1] 三种等价形式 form C / Figure 4-C and [P2] 三种视角.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// Step s writes Bw pairs j = s-Bw+1..s, each with weight w_s = eta_s / Bw and a
// residual against the same S_{s-1}.  A chunk of CS = C / Bw steps therefore
// has C "virtual rows" r = (s, j) (row r belongs to step s(r) = r / Bw and pair
// j(r) = s(r) - Bw + 1 + r % Bw).  Unrolling the recurrence over the chunk:
//   A[r][r'] = e^{L_{s(r)-1} - L_{s(r')}} <x_j(r), x_j(r')> w_{s(r')}   (s(r') < s(r))
//   (I + A) E = V_r - diag(e^{L_{s(r)-1}}) X_r S0^T        (E: one residual per row)
//   o_s      = e^{L_s} S0 q^_s + sum_{s(r) <= s} e^{L_s - L_{s(r)}} w_{s(r)} <x_j(r), q^_s> e_r
//   S^T_new  = e^{L_last} S0^T + X_r^T diag(e^{L_last - L_{s(r)}} w_{s(r)}) E
// with E = V_r (no solve) for Falcon-3A.  The solve is the same blocked WY
// solve as Falcon-1.  The C+Bw-1 distinct pair keys of a chunk sit in an LDS
// table; virtual rows are gathered from it per lane.  The last Bw-1 pairs of
// a chunk are carried to the next one in a small ring.
#include "falcon_kernels.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

enum { V_F1 = 1, V_F1A = 2, V_F3 = 5, V_F3A = 6 };

__device__ __forceinline__ void load_part(const __bf16 *p, float *out) {  // 8 values
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load_part(const float *p, float *out) {  // 4 values
  const float4 f = *reinterpret_cast<const float4 *>(p);
  out[0] = f.x; out[1] = f.y; out[2] = f.z; out[3] = f.w;
}

__device__ __forceinline__ float safe_rsqrt(float s) { return s > 0.f ? rsqrtf(s) : 0.f; }

template <int VAR, typename IT, int DK, int DV, int DVS, int C, int BW>
__global__ __launch_bounds__(DVS * 4) void chunk_fwd_window(FwdArgs a) {
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  constexpr int NW = DVS / 16, NT = NW * 64, NB = C / 16, NA = DK / 16;
  constexpr int CS = C / BW;                  // steps per WY system
  constexpr int CSP = CS < 16 ? 16 : CS;      // step rows padded to whole tiles
  constexpr int NBS = CSP / 16;
  constexpr int NP = CS + BW - 1;             // distinct pairs per system
  constexpr bool DELTA = (VAR == V_F3);
  constexpr int NSPLIT = DV / DVS;
  constexpr int LX = DK + 4, LT = C + 4, LV = DVS + 4, LO = DVS + 8;
  constexpr int VEC = 16 / sizeof(IT);
  static_assert(BW >= 2 && C % BW == 0, "window");

  __shared__ __attribute__((aligned(16))) OpT sKey[NP * LX];     // pair keys, oldest first
  __shared__ __attribute__((aligned(16))) OpT sXT[DK * LT];      // virtual-row keys, transposed
  __shared__ __attribute__((aligned(16))) OpT sQ[CSP * LX];
  __shared__ __attribute__((aligned(16))) OpT sA[DELTA ? C * LT : 4];
  __shared__ __attribute__((aligned(16))) OpT sP[CSP * LT];
  __shared__ __attribute__((aligned(16))) OpT sTb[DELTA ? NB * 16 * 20 : 4];
  __shared__ float sAd[DELTA ? NB * 16 * 17 : 1];
  __shared__ __attribute__((aligned(16))) float sPV[NP * LV];    // pair values of this slice
  __shared__ __attribute__((aligned(16))) IT sO[CSP * LO];
  __shared__ float sXn2[NP];
  __shared__ float sLc[CSP], sLm[CSP], sBeta[CSP];
  __shared__ __attribute__((aligned(16))) OpT sRingX[2][(BW - 1) * LX];
  __shared__ float sRingV[2][(BW - 1) * LV];
  __shared__ float sCarry[2][DK];
  __shared__ float sCarryN2[2];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int slice = blockIdx.x % NSPLIT, bh = blockIdx.x / NSPLIT;
  const int b = bh / a.H, h = bh % a.H;
  const int T = a.T, H = a.H;
  const int ch0 = slice * DVS;
  const int chW = ch0 + 16 * wv + cl;
  const int nsub = (T + CS - 1) / CS;

  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);

  auto tab = [](int r) { return r / BW + r % BW; };   // table row of virtual row r
  auto wstep = [&](int s) { return sBeta[s] / (a.eps_eta + sXn2[BW - 1 + s]) * (1.f / BW); };

  f4 sT[NA];
#pragma unroll
  for (int aa = 0; aa < NA; ++aa)
    sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * DV + chW) * DK + 16 * aa + 4 * g4)
                  : zero4();

  for (int e = tid; e < DK; e += NT) sCarry[0][e] = a.xprev0 ? a.xprev0[(size_t)bh * DK + e] : 0.f;
  for (int e = tid; e < (BW - 1) * DK; e += NT) {
    const int j = e / DK, d = e % DK;
    sRingX[0][j * LX + d] = (OpT)(a.winx0 ? a.winx0[((size_t)bh * (BW - 1) + j) * DK + d] : 0.f);
  }
  for (int e = tid; e < (BW - 1) * DVS; e += NT) {
    const int j = e / DVS, d = e % DVS;
    sRingV[0][j * LV + d] = a.winv0 ? a.winv0[((size_t)bh * (BW - 1) + j) * DV + ch0 + d] : 0.f;
  }
  for (int e = tid; e < CSP * LX; e += NT) sQ[e] = (OpT)0.f;
  __syncthreads();
  if (wv == 0) {
    float s = 0.f;
    for (int e = lane; e < DK; e += 64) s += sCarry[0][e] * sCarry[0][e];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sCarryN2[0] = s;
  }
  __syncthreads();

  for (int sc = 0; sc < nsub; ++sc) {
    const int s0 = sc * CS, cur = sc & 1, nxt = cur ^ 1;

    // ---- Phase A: pair table, queries, gates ---------------------------------
    for (int e = tid; e < (BW - 1) * DK; e += NT) {
      const int j = e / DK, d = e % DK;
      sKey[j * LX + d] = sRingX[cur][j * LX + d];
    }
    for (int e = tid; e < (BW - 1) * DVS; e += NT) {
      const int j = e / DVS, d = e % DVS;
      sPV[j * LV + d] = sRingV[cur][j * LV + d];
    }
    for (int e = tid; e < DK; e += NT) sKey[(BW - 1) * LX + e] = (OpT)sCarry[cur][e];
    if (tid == 0) sXn2[BW - 1] = sCarryN2[cur];
    {  // keys of steps s0..s0+CS-1: phi(k_t) is the key of pair t+1
      constexpr int TPR = DK / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < CS; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = s0 + r;
        float xv[VEC];
        if (r < CS && t < T) load_part(kp + ((size_t)(b * T + t) * H + h) * DK + part * VEC, xv);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xv[e] * xv[e];
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = safe_rsqrt(ss + a.eps_phi);
        if (r + 1 < CS) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sKey[(BW + r) * LX + part * VEC + e] = (OpT)(xv[e] * inv);
          if (part == 0) sXn2[BW + r] = ss * inv * inv;
        } else if (r + 1 == CS) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sCarry[nxt][part * VEC + e] = xv[e] * inv;
          if (part == 0) sCarryN2[nxt] = ss * inv * inv;
        }
      }
    }
    {  // queries
      constexpr int TPR = DK / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < CS; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = s0 + r;
        float xv[VEC];
        if (r < CS && t < T) load_part(qp + ((size_t)(b * T + t) * H + h) * DK + part * VEC, xv);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xv[e] * xv[e];
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = safe_rsqrt(ss + a.eps_phi);
        if (r < CS) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sQ[r * LX + part * VEC + e] = (OpT)(xv[e] * inv);
        }
      }
    }
    {  // values of the new pairs (pair s0 + r has value v_{s0+r})
      constexpr int TPR = DVS / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < CS; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = s0 + r;
        if (r < CS) {
          float xv[VEC];
          if (t < T) load_part(vp + ((size_t)(b * T + t) * H + h) * DV + ch0 + part * VEC, xv);
          else
#pragma unroll
            for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) sPV[(BW - 1 + r) * LV + part * VEC + e] = xv[e];
        }
      }
    }
    if (wv == 0) {  // gates of the CS steps
      const int t = s0 + lane;
      const bool ok = lane < CS && t < T;
      const float gg = ok ? fmaxf(a.g[(size_t)(b * T + t) * H + h], a.log_eps_gamma) : 0.f;
      float L = gg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(L, off);
        if (lane >= off) L += y;
      }
      if (lane < CSP) {
        sLc[lane] = L;
        sLm[lane] = L - gg;
        sBeta[lane] = ok ? a.beta[(size_t)(b * T + t) * H + h] : 0.f;
      }
    }
    __syncthreads();

    // ---- Phase B: carry ring, transposed virtual rows, Gram and score tiles --
    for (int e = tid; e < (BW - 1) * DK; e += NT) {
      const int j = e / DK, d = e % DK;
      sRingX[nxt][j * LX + d] = sKey[(CS + j) * LX + d];
    }
    for (int e = tid; e < (BW - 1) * DVS; e += NT) {
      const int j = e / DVS, d = e % DVS;
      sRingV[nxt][j * LV + d] = sPV[(CS + j) * LV + d];
    }
    for (int e = tid; e < DK * C; e += NT) {
      const int r = e % C, d = e / C;
      sXT[d * LT + r] = sKey[tab(r) * LX + d];
    }
    {
      constexpr int NPAIR = NB * (NB + 1) / 2;
      constexpr int NG = DELTA ? NPAIR : 0;
      constexpr int NJOB = NG + NBS * NB;
      for (int job = wv; job < NJOB; job += NW) {
        const bool isP = job >= NG;
        int p, q;
        if (!isP) {
          p = 0;
          while ((p + 1) * (p + 2) / 2 <= job) ++p;
          q = job - p * (p + 1) / 2;
        } else {
          p = (job - NG) / NB;     // step block
          q = (job - NG) % NB;     // virtual-row block
          if ((16 * q) / BW > 16 * p + 15) continue;   // every entry masked
        }
        const int krow = tab(16 * q + cl);
        f4 acc = zero4();
#pragma unroll
        for (int aa = 0; aa < NA; aa += 2) {
          const Frag b0 = ld4(sKey + krow * LX + 16 * aa + 4 * g4);
          const Frag b1 = ld4(sKey + krow * LX + 16 * aa + 16 + 4 * g4);
          if (isP) {
            mma32(acc, lda(sQ, LX, 16 * p, 16 * aa, lane), lda(sQ, LX, 16 * p, 16 * aa + 16, lane), b0, b1);
          } else {
            const int arow = tab(16 * p + cl);
            mma32(acc, ld4(sKey + arow * LX + 16 * aa + 4 * g4), ld4(sKey + arow * LX + 16 * aa + 16 + 4 * g4), b0, b1);
          }
        }
        const int col = 16 * q + cl, sc_ = col / BW;
        const float Lcol = sLc[sc_];
        const float wcol = wstep(sc_);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * p + 4 * g4 + i;
          if (isP) {
            const float val = (row < CS && sc_ <= row) ? acc[i] * __expf(sLc[row] - Lcol) * wcol : 0.f;
            sP[row * LT + col] = (OpT)val;
          } else {
            const int sr = row / BW;
            const float val = (sc_ < sr) ? acc[i] * __expf(sLm[sr] - Lcol) * wcol : 0.f;
            sA[row * LT + col] = (OpT)val;
            if (p == q) sAd[(p * 16 + 4 * g4 + i) * 17 + cl] = val;
          }
        }
      }
    }
    __syncthreads();

    // ---- Phase C: diagonal-block inverses (Falcon-3) -------------------------
    if (DELTA && wv == NW - 1) {
      const int p = lane >> 4, j = lane & 15;
      if (p < NB) {
        float col[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) col[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
          for (int i = kk + 1; i < 16; ++i) col[i] -= sAd[(p * 16 + i) * 17 + kk] * col[kk];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sTb[(p * 16 + i) * 20 + j] = (OpT)col[i];
      }
    }

    // ---- Phase D: state-dependent products -----------------------------------
    Frag Sb[NA];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) Sb[aa] = cvt<OpT>(sT[aa]);
    f4 QS[NBS], XS[NB];
#pragma unroll
    for (int p = 0; p < NBS; ++p) {
      QS[p] = zero4();
#pragma unroll
      for (int aa = 0; aa < NA; aa += 2)
        mma32(QS[p], lda(sQ, LX, 16 * p, 16 * aa, lane), lda(sQ, LX, 16 * p, 16 * aa + 16, lane), Sb[aa], Sb[aa + 1]);
    }
    if (DELTA) {
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        XS[p] = zero4();
        const int arow = tab(16 * p + cl);
#pragma unroll
        for (int aa = 0; aa < NA; aa += 2)
          mma32(XS[p], ld4(sKey + arow * LX + 16 * aa + 4 * g4), ld4(sKey + arow * LX + 16 * aa + 16 + 4 * g4),
                Sb[aa], Sb[aa + 1]);
      }
      __syncthreads();  // T_pp ready
    }

    Frag Eb[NB];
    f4 Ef[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 R;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * p + 4 * g4 + i;
        R[i] = sPV[tab(row) * LV + 16 * wv + cl];
        if (DELTA) R[i] -= __expf(sLm[row / BW]) * XS[p][i];
      }
      if (DELTA) {
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q < p; ++q) mma16(acc, lda(sA, LT, 16 * p, 16 * q, lane), Eb[q]);
        R -= acc;
        f4 E = zero4();
        mma16(E, lda(sTb, 20, 16 * p, 0, lane), cvt<OpT>(R));
        Ef[p] = E;
        Eb[p] = cvt<OpT>(E);
      } else {
        Ef[p] = R;
        Eb[p] = cvt<OpT>(R);
      }
    }

#pragma unroll
    for (int p = 0; p < NBS; ++p) {
      f4 O;
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] = __expf(sLc[16 * p + 4 * g4 + i]) * QS[p][i];
#pragma unroll
      for (int q = 0; q < NB; ++q)
        if ((16 * q) / BW <= 16 * p + 15) mma16(O, lda(sP, LT, 16 * p, 16 * q, lane), Eb[q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[(16 * p + 4 * g4 + i) * LO + 16 * wv + cl] = (IT)O[i];
    }

    {
      const float Llast = sLc[CS - 1];
      Frag CE[NB];
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        f4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = (16 * p + 4 * g4 + i) / BW;
          x[i] = __expf(Llast - sLc[s]) * wstep(s) * Ef[p][i];
        }
        CE[p] = cvt<OpT>(x);
      }
      const float lamtot = __expf(Llast);
#pragma unroll
      for (int aa = 0; aa < NA; ++aa) {
        f4 acc = sT[aa] * lamtot;
#pragma unroll
        for (int p = 0; p + 1 < NB; p += 2)
          mma32(acc, lda(sXT, LT, 16 * aa, 16 * p, lane), lda(sXT, LT, 16 * aa, 16 * p + 16, lane), CE[p], CE[p + 1]);
        if (NB & 1) mma16(acc, lda(sXT, LT, 16 * aa, 16 * (NB - 1), lane), CE[NB - 1]);
        sT[aa] = acc;
      }
      if (a.chunk_states && ((sc + 1) % BW == 0 || sc == nsub - 1)) {
        const int ci = sc / BW;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa)
          *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * a.nchunks + ci) * DV + chW) * DK + 16 * aa + 4 * g4) =
              sT[aa];
      }
    }
    __syncthreads();

    // ---- Phase E: store the outputs of the CS steps --------------------------
    {
      constexpr int TPR = DVS / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < CS; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = s0 + r;
        if (r < CS && t < T)
          *reinterpret_cast<uint4 *>(op + ((size_t)(b * T + t) * H + h) * DV + ch0 + part * VEC) =
              *reinterpret_cast<const uint4 *>(sO + r * LO + part * VEC);
      }
    }
  }

  if (a.S_out) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      *reinterpret_cast<f4 *>(a.S_out + ((size_t)bh * DV + chW) * DK + 16 * aa + 4 * g4) = sT[aa];
  }
}

template <int VAR, typename IT, int DK, int DV, int DVS, int C>
hipError_t by_window(int bw, const FwdArgs &a, hipStream_t s) {
  const int nblk = a.B * a.H * (DV / DVS);
#define FALCON_W(BW_)                                                                                     \
  if (bw == BW_) {                                                                                        \
    hipLaunchKernelGGL((chunk_fwd_window<VAR, IT, DK, DV, DVS, C, BW_>), dim3(nblk), dim3(DVS * 4), 0, s, a); \
    return hipGetLastError();                                                                             \
  }
  FALCON_W(2)
  FALCON_W(4)
  FALCON_W(8)
#undef FALCON_W
  return hipErrorInvalidValue;
}

template <int VAR, typename IT, int DK, int DV, int DVS>
hipError_t win_chunk(int chunk, int bw, const FwdArgs &a, hipStream_t s) {
  switch (chunk) {
    case 16: return by_window<VAR, IT, DK, DV, DVS, 16>(bw, a, s);
    case 32: return by_window<VAR, IT, DK, DV, DVS, 32>(bw, a, s);
    case 64: return by_window<VAR, IT, DK, DV, DVS, 64>(bw, a, s);
  }
  return hipErrorInvalidValue;
}

template <int VAR, typename IT>
hipError_t win_dims(int dk, int dv, int nsplit, int chunk, int bw, const FwdArgs &a, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  if (dk == 32 && nsplit == 1) return win_chunk<VAR, IT, 32, 32, 32>(chunk, bw, a, s);
  if (dk == 64 && nsplit == 1) return win_chunk<VAR, IT, 64, 64, 64>(chunk, bw, a, s);
  if constexpr (sizeof(IT) == 2) {
    if (dk == 128 && nsplit == 2) return win_chunk<VAR, IT, 128, 128, 64>(chunk, bw, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_fwd_rows(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                 const FwdArgs &a, hipStream_t s);

hipError_t launch_chunk_fwd_window(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                   const FwdArgs &a, hipStream_t s) {
  if (a.window == 1)  // a window of one pair is Falcon-1 / 1A
    return launch_chunk_fwd_rows(variant == V_F3 ? V_F1 : V_F1A, bf16, dk, dv, chunk, nsplit, a, s);
  if (variant == V_F3)
    return bf16 ? win_dims<V_F3, __bf16>(dk, dv, nsplit, chunk, a.window, a, s)
                : win_dims<V_F3, float>(dk, dv, nsplit, chunk, a.window, a, s);
  if (variant == V_F3A)
    return bf16 ? win_dims<V_F3A, __bf16>(dk, dv, nsplit, chunk, a.window, a, s)
                : win_dims<V_F3A, float>(dk, dv, nsplit, chunk, a.window, a, s);
  return hipErrorInvalidValue;
}

}  // namespace falcon
