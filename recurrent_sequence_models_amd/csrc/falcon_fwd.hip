// Chunked forward pass of Falcon-1 / 1A / 2 / 2A on gfx950.
//
// Chunked form: [P1] 三种等价形式 form C and Figure 4-C (per-chunk Gram and WY
// factors, triangular solve, cross-chunk state recurrence); [P2] 三种视角.
// Step definitions: [P1] Falcon家族, [P2] 六个变体 and 梯度下降 (NLMS);
// prefix alignment: [P1] 本质; decay floor: [P2] 正衰减钳制.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// One workgroup owns one sequence (b, h) and a slice of DVS value channels
// (rows of S); it walks the chunks in order and keeps its slice of S^T in
// registers, in fp32, for the whole sequence.  Per chunk of C steps with
// chunk-local inclusive log-decay sums L_i (L_{-1} = 0), x_i = phi(k_{i-1}),
// q^_i = phi(q_i) and incoming state S0:
//
//   A[i][j]  = e^{L_{i-1}-L_j} <x_i, x_j> w_j      (j < i; w_j = eta_j for F1, 1 for F2)
//   P[i][j]  = e^{L_i-L_j} <q^_i, x_j> w_j         (j <= i)
//   R        = V - diag(e^{L_{i-1}}) X S0^T
//   F1:  (I + A) E = R, solved in 16-row blocks: E_p = T_pp (R_p - sum_{q<p} A_pq E_q),
//        T_pp = (I + A_pp)^{-1} by forward substitution, the off-diagonal part on MFMA.
//   F2:  (I + A diag(eta_c)) e_c = r_c per value channel c; off-diagonal blocks on
//        MFMA with F = eta (.) E, the 16x16 diagonal blocks by per-channel substitution.
//   F1A/F2A: E = V (additive write, no solve).
//   O        = diag(e^{L_i}) Q^ S0^T + P E'            (E' = E, or eta (.) E per channel)
//   S^T_new  = e^{L_last} S0^T + X^T diag(e^{L_last-L_i}) E''   (E'' = eta E or eta (.) E)
//
// The rows of E are exactly the residuals v_t - S_{t-1} x_t of the recurrence.
// All products are 16x16 MFMA tiles (bf16 operands with fp32 accumulation for
// bf16 inputs; fp32 MFMA for fp32 inputs).  Steps past the end of the sequence
// are padded as identity steps (x = v = q = 0, beta = 0, g = 0).
#include "falcon_kernels.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

enum { V_F1 = 1, V_F1A = 2, V_F2 = 3, V_F2A = 4 };

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

template <int VAR, typename IT, int DK, int DV, int DVS, int C>
__global__ __launch_bounds__(DVS * 4) void chunk_fwd_rows(FwdArgs a) {
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  constexpr int NW = DVS / 16, NT = NW * 64, NB = C / 16, NA = DK / 16;
  constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2);
  constexpr int NSPLIT = DV / DVS;
  constexpr int LX = DK + 4, LT = C + 4, LV = DVS + 4, LO = DVS + 8;
  constexpr int VEC = 16 / sizeof(IT);
  static_assert(DV % DVS == 0 && DVS % 16 == 0 && C % 16 == 0 && DK % 32 == 0, "shape");

  __shared__ __attribute__((aligned(16))) OpT sX[C * LX];
  __shared__ __attribute__((aligned(16))) OpT sQ[C * LX];
  __shared__ __attribute__((aligned(16))) OpT sXT[DK * LT];
  __shared__ __attribute__((aligned(16))) OpT sA[DELTA ? C * LT : 4];
  __shared__ __attribute__((aligned(16))) OpT sP[C * LT];
  __shared__ __attribute__((aligned(16))) OpT sTb[VAR == V_F1 ? NB * 16 * 20 : 4];
  __shared__ float sAd[DELTA ? NB * 16 * 17 : 1];
  __shared__ __attribute__((aligned(16))) float sV[C * LV];
  __shared__ float sEV[PERCH ? C * LV : 1];
  __shared__ __attribute__((aligned(16))) IT sO[C * LO];
  __shared__ float sXn2[C], sLc[C], sLm[C], sBeta[C];
  __shared__ float sCarry[2][DK];
  __shared__ float sCarryN2[2];
  __shared__ float sScr[VAR == V_F2 ? NW * 16 * 17 : 1];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int slice = blockIdx.x % NSPLIT, bh = blockIdx.x / NSPLIT;
  const int b = bh / a.H, h = bh % a.H;
  const int T = a.T, H = a.H;
  const int ch0 = slice * DVS;
  const int chW = ch0 + 16 * wv + cl;  // value channel of this lane in C-layout tiles

  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);

  // S^T slice in C-layout: sT[aa][i] = S^T[16 aa + 4 g4 + i][chW] = S[chW][16 aa + 4 g4 + i]
  f4 sT[NA];
#pragma unroll
  for (int aa = 0; aa < NA; ++aa)
    sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * DV + chW) * DK + 16 * aa + 4 * g4)
                  : zero4();

  for (int e = tid; e < DK; e += NT) sCarry[0][e] = a.xprev0 ? a.xprev0[(size_t)bh * DK + e] : 0.f;
  __syncthreads();
  if (wv == 0) {
    float s = 0.f;
    for (int e = lane; e < DK; e += 64) s += sCarry[0][e] * sCarry[0][e];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sCarryN2[0] = s;
  }
  __syncthreads();

  for (int c = 0; c < a.nchunks; ++c) {
    const int c0 = c * C, cur = c & 1, nxt = cur ^ 1;

    // ---- Phase A: stage the chunk in LDS ------------------------------------
    for (int e = tid; e < DK; e += NT) {
      const float x = sCarry[cur][e];
      sX[e] = (OpT)x;
      sXT[e * LT] = (OpT)x;
    }
    if (tid == 0) sXn2[0] = sCarryN2[cur];
    {  // keys: phi(k_{c0+r}) is x of step r+1; the last one is carried to the next chunk
      constexpr int TPR = DK / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = c0 + r;
        float xv[VEC];
        if (r < C && t < T) load_part(kp + ((size_t)(b * T + t) * H + h) * DK + part * VEC, xv);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xv[e] * xv[e];
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = safe_rsqrt(ss + a.eps_phi);
        if (r + 1 < C) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const OpT xo = (OpT)(xv[e] * inv);
            sX[(r + 1) * LX + part * VEC + e] = xo;
            sXT[(part * VEC + e) * LT + r + 1] = xo;
          }
          if (part == 0) sXn2[r + 1] = ss * inv * inv;
        } else if (r + 1 == C) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sCarry[nxt][part * VEC + e] = xv[e] * inv;
          if (part == 0) sCarryN2[nxt] = ss * inv * inv;
        }
      }
    }
    {  // queries
      constexpr int TPR = DK / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = c0 + r;
        float xv[VEC];
        if (r < C && t < T) load_part(qp + ((size_t)(b * T + t) * H + h) * DK + part * VEC, xv);
        else
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) ss += xv[e] * xv[e];
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off);
        const float inv = safe_rsqrt(ss + a.eps_phi);
        if (r < C) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) sQ[r * LX + part * VEC + e] = (OpT)(xv[e] * inv);
        }
      }
    }
    {  // values of this slice (fp32 in LDS)
      constexpr int TPR = DVS / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = c0 + r;
        if (r < C) {
          float xv[VEC];
          if (t < T) load_part(vp + ((size_t)(b * T + t) * H + h) * DV + ch0 + part * VEC, xv);
          else
#pragma unroll
            for (int e = 0; e < VEC; ++e) xv[e] = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) sV[r * LV + part * VEC + e] = xv[e];
        }
      }
    }
    if (PERCH) {  // per-channel gains beta (fp32), turned into eta after the barrier
      constexpr int TPR = DVS / 4, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = c0 + r;
        if (r < C) {
          float xv[4] = {0.f, 0.f, 0.f, 0.f};
          if (t < T) load_part(a.beta + ((size_t)(b * T + t) * H + h) * DV + ch0 + part * 4, xv);
#pragma unroll
          for (int e = 0; e < 4; ++e) sEV[r * LV + part * 4 + e] = xv[e];
        }
      }
    }
    if (wv == 0) {  // gates: clamp in log space, chunk-local inclusive scan
      const int t = c0 + lane;
      const bool ok = lane < C && t < T;
      const float gg = ok ? fmaxf(a.g[(size_t)(b * T + t) * H + h], a.log_eps_gamma) : 0.f;
      float L = gg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(L, off);
        if (lane >= off) L += y;
      }
      if (lane < C) {
        sLc[lane] = L;
        sLm[lane] = L - gg;
        sBeta[lane] = (!PERCH && ok) ? a.beta[(size_t)(b * T + t) * H + h] : 0.f;
      }
    }
    __syncthreads();

    // ---- Phase B: key-side tiles (Gram with decay and step, scores) ----------
    {
      constexpr int NPAIR = NB * (NB + 1) / 2;
      constexpr int NJOB = (DELTA ? 2 : 1) * NPAIR;
      for (int job = wv; job < NJOB; job += NW) {
        const bool isP = job >= (DELTA ? NPAIR : 0);
        const int pj = isP ? job - (DELTA ? NPAIR : 0) : job;
        int p = 0;
        while ((p + 1) * (p + 2) / 2 <= pj) ++p;
        const int q = pj - p * (p + 1) / 2;
        const OpT *Am = isP ? sQ : sX;
        f4 acc = zero4();
#pragma unroll
        for (int aa = 0; aa < NA; aa += 2)
          mma32(acc, lda(Am, LX, 16 * p, 16 * aa, lane), lda(Am, LX, 16 * p, 16 * aa + 16, lane),
                lda(sX, LX, 16 * q, 16 * aa, lane), lda(sX, LX, 16 * q, 16 * aa + 16, lane));
        const int col = 16 * q + cl;
        const float Lcol = sLc[col];
        const float wcol = PERCH ? 1.f : sBeta[col] / (a.eps_eta + sXn2[col]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * p + 4 * g4 + i;
          if (isP) {
            const float val = (col <= row) ? acc[i] * __expf(sLc[row] - Lcol) * wcol : 0.f;
            sP[row * LT + col] = (OpT)val;
          } else if (DELTA) {
            const float val = (col < row) ? acc[i] * __expf(sLm[row] - Lcol) * wcol : 0.f;
            sA[row * LT + col] = (OpT)val;
            if (p == q) sAd[(p * 16 + 4 * g4 + i) * 17 + cl] = val;
          }
        }
      }
      if (PERCH) {
        for (int idx = tid; idx < C * DVS; idx += NT) {
          const int r = idx / DVS, cc = idx % DVS;
          sEV[r * LV + cc] = sEV[r * LV + cc] / (a.eps_eta + sXn2[r]);
        }
      }
    }
    __syncthreads();

    // ---- Phase C: diagonal-block inverses T_pp = (I + A_pp)^{-1} (F1) ---------
    if (VAR == V_F1 && wv == NW - 1) {
      const int p = lane >> 4, j = lane & 15;
      if (p < NB) {
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = (i == j) ? 1.f : 0.f;
#pragma unroll
          for (int kk = 0; kk < i; ++kk) s -= sAd[(p * 16 + i) * 17 + kk] * t[kk];
          t[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sTb[(p * 16 + i) * 20 + j] = (OpT)t[i];
      }
    }

    // ---- Phase D: the state-dependent products for this wave's 16 channels ---
    Frag Sb[NA];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) Sb[aa] = cvt<OpT>(sT[aa]);
    f4 QS[NB], XS[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      QS[p] = zero4();
      XS[p] = zero4();
#pragma unroll
      for (int aa = 0; aa < NA; aa += 2) {
        mma32(QS[p], lda(sQ, LX, 16 * p, 16 * aa, lane), lda(sQ, LX, 16 * p, 16 * aa + 16, lane), Sb[aa], Sb[aa + 1]);
        if (DELTA)
          mma32(XS[p], lda(sX, LX, 16 * p, 16 * aa, lane), lda(sX, LX, 16 * p, 16 * aa + 16, lane), Sb[aa], Sb[aa + 1]);
      }
    }
    if (VAR == V_F1) __syncthreads();  // T_pp ready

    Frag Eb[NB];  // operand form of E (F1/F1A) or eta (.) E (F2/F2A)
    f4 Ef[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 R;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * p + 4 * g4 + i;
        R[i] = sV[row * LV + 16 * wv + cl];
        if (DELTA) R[i] -= __expf(sLm[row]) * XS[p][i];
      }
      if (VAR == V_F1) {
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q < p; ++q) mma16(acc, lda(sA, LT, 16 * p, 16 * q, lane), Eb[q]);
        R -= acc;
        f4 E = zero4();
        mma16(E, lda(sTb, 20, 16 * p, 0, lane), cvt<OpT>(R));
        Ef[p] = E;
        Eb[p] = cvt<OpT>(E);
      } else if (VAR == V_F2) {
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q < p; ++q) mma16(acc, lda(sA, LT, 16 * p, 16 * q, lane), Eb[q]);
        R -= acc;
        float *scr = sScr + wv * 16 * 17;
#pragma unroll
        for (int i = 0; i < 4; ++i) scr[(4 * g4 + i) * 17 + cl] = R[i];
        __syncthreads();
        if (lane < 16) {  // lane = value channel: (I + A_pp diag(eta)) e = r by substitution
          float e[16], f[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float s = scr[i * 17 + lane];
#pragma unroll
            for (int kk = 0; kk < i; ++kk) s -= sAd[(p * 16 + i) * 17 + kk] * f[kk];
            e[i] = s;
            f[i] = sEV[(16 * p + i) * LV + 16 * wv + lane] * s;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) scr[i * 17 + lane] = f[i];
        }
        __syncthreads();
        f4 F;
#pragma unroll
        for (int i = 0; i < 4; ++i) F[i] = scr[(4 * g4 + i) * 17 + cl];
        Ef[p] = F;
        Eb[p] = cvt<OpT>(F);
      } else if (VAR == V_F1A) {
        Ef[p] = R;
        Eb[p] = cvt<OpT>(R);
      } else {  // F2A
        f4 F;
#pragma unroll
        for (int i = 0; i < 4; ++i) F[i] = sEV[(16 * p + 4 * g4 + i) * LV + 16 * wv + cl] * R[i];
        Ef[p] = F;
        Eb[p] = cvt<OpT>(F);
      }
    }

    // outputs o = e^{L} Q^ S0^T + P E'
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 O;
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] = __expf(sLc[16 * p + 4 * g4 + i]) * QS[p][i];
#pragma unroll
      for (int q = 0; q <= p; ++q) mma16(O, lda(sP, LT, 16 * p, 16 * q, lane), Eb[q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[(16 * p + 4 * g4 + i) * LO + 16 * wv + cl] = (IT)O[i];
    }

    // state: S^T <- e^{L_last} S^T + X^T diag(e^{L_last - L_i} w_i) E
    {
      const float Llast = sLc[C - 1];
      Frag CE[NB];
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        f4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * p + 4 * g4 + i;
          const float w = PERCH ? 1.f : sBeta[row] / (a.eps_eta + sXn2[row]);
          x[i] = __expf(Llast - sLc[row]) * w * Ef[p][i];
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
      if (a.chunk_states) {
#pragma unroll
        for (int aa = 0; aa < NA; ++aa)
          *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * a.nchunks + c) * DV + chW) * DK + 16 * aa + 4 * g4) =
              sT[aa];
      }
    }
    __syncthreads();

    // ---- Phase E: coalesced store of the chunk's outputs ----------------------
    {
      constexpr int TPR = DVS / VEC, RPP = NT / TPR;
#pragma unroll
      for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + tid / TPR, part = tid % TPR, t = c0 + r;
        if (r < C && t < T)
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
  if (a.write_tail && a.xprev_out && slice == 0 && wv == 0) {
    // x_prev = phi(k_{T-1})
    float s = 0.f, xv[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * j;
      if (e < DK) xv[j] = (float)kp[((size_t)(b * T + T - 1) * H + h) * DK + e];
      s += xv[j] * xv[j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    const float inv = safe_rsqrt(s + a.eps_phi);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * j;
      if (e < DK) a.xprev_out[(size_t)bh * DK + e] = xv[j] * inv;
    }
  }
}

// LDS bytes of chunk_fwd_rows (mirrors its __shared__ arrays).
template <int VAR, typename IT, int DK, int DVS, int C>
constexpr size_t rows_lds_bytes() {
  constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A), DELTA = (VAR == V_F1 || VAR == V_F2);
  constexpr size_t LX = DK + 4, LT = C + 4, LV = DVS + 4, LO = DVS + 8, NB = C / 16, NW = DVS / 16;
  return sizeof(IT) * (2 * C * LX + DK * LT + (DELTA ? C * LT : 4) + C * LT + (VAR == V_F1 ? NB * 320 : 4) + C * LO) +
         4 * ((DELTA ? NB * 272 : 1) + C * LV + (PERCH ? C * LV : 1) + 4 * C + 2 * DK + 2 + (VAR == V_F2 ? NW * 272 : 1));
}

template <int VAR, typename IT, int DK, int DV, int DVS, int C>
hipError_t launch_rows(const FwdArgs &a, hipStream_t s) {
  if constexpr (rows_lds_bytes<VAR, IT, DK, DVS, C>() + 1024 <= 160 * 1024) {
    const int nblk = a.B * a.H * (DV / DVS);
    hipLaunchKernelGGL((chunk_fwd_rows<VAR, IT, DK, DV, DVS, C>), dim3(nblk), dim3(DVS * 4), 0, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int VAR, typename IT, int DK, int DV, int DVS>
hipError_t by_chunk(int chunk, const FwdArgs &a, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_rows<VAR, IT, DK, DV, DVS, 16>(a, s);
    case 32: return launch_rows<VAR, IT, DK, DV, DVS, 32>(a, s);
    case 64: return launch_rows<VAR, IT, DK, DV, DVS, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int VAR, typename IT, int DK, int DV>
hipError_t by_split(int nsplit, int chunk, const FwdArgs &a, hipStream_t s) {
  switch (nsplit) {
    case 1: return by_chunk<VAR, IT, DK, DV, DV>(chunk, a, s);
    case 2: if constexpr (DV >= 32) return by_chunk<VAR, IT, DK, DV, DV / 2>(chunk, a, s); break;
    case 4: if constexpr (DV >= 64) return by_chunk<VAR, IT, DK, DV, DV / 4>(chunk, a, s); break;
    case 8: if constexpr (DV >= 128) return by_chunk<VAR, IT, DK, DV, DV / 8>(chunk, a, s); break;
  }
  return hipErrorInvalidValue;
}

template <int VAR, typename IT>
hipError_t by_dims(int dk, int dv, int nsplit, int chunk, const FwdArgs &a, hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (dk) {
    case 32: return by_split<VAR, IT, 32, 32>(nsplit, chunk, a, s);
    case 64: return by_split<VAR, IT, 64, 64>(nsplit, chunk, a, s);
    case 128:
      if constexpr (sizeof(IT) == 2) return by_split<VAR, IT, 128, 128>(nsplit, chunk, a, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_fwd_pipe_supported(int variant, bool bf16, int dk, int dv, int chunk);
hipError_t launch_chunk_fwd_pipe(int variant, bool bf16, int dk, int dv, int chunk, const FwdArgs &a,
                                 hipStream_t s);

hipError_t launch_chunk_fwd_rows(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                 const FwdArgs &a, hipStream_t s) {
  // the software-pipelined kernel takes whole sequences whenever its LDS footprint fits
  if (nsplit == 1 && chunk_fwd_pipe_supported(variant, bf16, dk, dv, chunk))
    return launch_chunk_fwd_pipe(variant, bf16, dk, dv, chunk, a, s);
#define FALCON_DISPATCH(VV)                                                         \
  return bf16 ? by_dims<VV, __bf16>(dk, dv, nsplit, chunk, a, s)                   \
              : by_dims<VV, float>(dk, dv, nsplit, chunk, a, s)
  switch (variant) {
    case V_F1: FALCON_DISPATCH(V_F1);
    case V_F1A: FALCON_DISPATCH(V_F1A);
    case V_F2: FALCON_DISPATCH(V_F2);
    case V_F2A: FALCON_DISPATCH(V_F2A);
  }
#undef FALCON_DISPATCH
  return hipErrorInvalidValue;
}

}  // namespace falcon
