// Software-pipelined chunked forward pass of Falcon-1 / 1A / 2 / 2A on gfx950.
//
// Same mathematics as the chunked form in falcon_fwd.hip ([P1] 三种等价形式
// form C and Figure 4-C: per-chunk Gram / WY factors, triangular solve and the
// cross-chunk state recurrence; [P2] 三种视角), organised so that only the
// state-dependent products sit on the serial chain.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// One workgroup per sequence (b, h), D/16 + 4 waves:
//   consumer waves (one per 16 value channels) keep S^T in registers and, for
//     chunk c, compute X S0^T, Q^ S0^T, the residuals E (blocked solve), the
//     outputs and the state update.  They read their values (and Falcon-2's
//     per-channel gains) straight from HBM in MFMA fragment layout, one chunk
//     ahead.
//   producer waves, in the same iteration, build the key-side tiles of chunk
//     c+1 (decayed Gram A with the step folded in, scores P, diagonal-block
//     inverses T_pp), stage the normalised keys/queries of chunk c+2 in LDS and
//     prefetch the raw inputs of chunk c+3 into registers.
// One workgroup barrier per chunk.  Input tiles are triple-buffered, key-side
// tiles double-buffered.  Every k axis an MFMA reduces over is stored permuted
// in LDS (kperm) so that one 16-byte read fills a 16x16x32 operand.
//
// Diagonal blocks: T_pp = (I + N)^{-1} with N strictly lower 16x16, and
// Falcon-2's per-channel systems (I + A_pp diag(eta_c)) e = r, are both solved
// by a block-Jacobi sweep over 4x4 sub-blocks: each lane group solves its own
// 4 rows exactly, and the coupling between sub-blocks (strictly block-lower,
// hence nilpotent) is one 16x16 MFMA per sweep; three sweeps are exact.
#include "falcon_kernels.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

enum { V_F1 = 1, V_F1A = 2, V_F2 = 3, V_F2A = 4 };

// gate arrays of an input slot
enum { G_LC = 0, G_LM, G_XN2, G_BETA, G_GAM, G_EL, G_ETA, G_CST, G_N };

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
__device__ __forceinline__ float safe_rsqrt(float s) { return s > 0.f ? rsqrtf(s) : 0.f; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

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

template <int VAR, typename IT, int D, int C>
struct Pipe {
  static constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  static constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2);
  static constexpr int NB = C / 16, NA = D / 16;
  static constexpr int NCW = D / 16, NPW = 4, NT = 64 * (NCW + NPW);
  static constexpr int NPT = 64 * NPW;                       // producer threads
  static constexpr int PADE = 16 / (int)sizeof(IT);          // elements in 16 bytes
  static constexpr int LX = D + PADE;                        // X, Q rows (k = dk, permuted)
  static constexpr int LT = C + PADE;                        // XT, Ao, P rows (k = chunk row)
  static constexpr int LTB = 16 + PADE;                      // T_pp / inner-block rows
  static constexpr int LO = 16 + PADE;                       // output staging rows
  static constexpr int VEC = PADE;
  static constexpr int TPR = D / VEC;                        // producer threads per input row
  static constexpr int RPP = NPT / TPR;                      // rows per producer pass
  static constexpr int NPASS = (C + RPP - 1) / RPP;
  static constexpr int NOFF = NB * (NB - 1) / 2, NPB = NB * (NB + 1) / 2;
  static constexpr size_t lds_bytes() {
    return sizeof(IT) * (3 * (2 * C * LX + D * LT) + 2 * (2 * C * LT + NB * 16 * LTB) + NCW * C * LO) +
           4 * (3 * G_N * C + 3 + (PERCH ? 2 * NB * 272 : 0) + (VAR == V_F1 ? NPW * 272 : 0) + 2 * D + 2);
  }
  static constexpr bool fits() { return lds_bytes() + 256 <= 160 * 1024; }
};

// position of chunk-row k in a row whose k axis is a chunk (permuted when C >= 32)
template <int C>
__device__ __forceinline__ int kc(int k) { return (C % 32 == 0) ? kperm(k) : k; }

template <int VAR, typename IT, int D, int C>
__global__ __launch_bounds__(64 * (D / 16 + 4)) void chunk_fwd_pipe(FwdArgs a) {
  using P = Pipe<VAR, IT, D, C>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = P::NB, NA = P::NA, NCW = P::NCW, NPW = P::NPW;
  constexpr int LX = P::LX, LT = P::LT, LTB = P::LTB, VEC = P::VEC, TPR = P::TPR, RPP = P::RPP, NPASS = P::NPASS;
  constexpr bool PERCH = P::PERCH, DELTA = P::DELTA;

  __shared__ __attribute__((aligned(16))) OpT sX[3][C * LX];      // x_i = phi(k_{i-1}), dk permuted
  __shared__ __attribute__((aligned(16))) OpT sQ[3][C * LX];      // q^_i, dk permuted
  __shared__ __attribute__((aligned(16))) OpT sXT[3][D * LT];     // X^T, chunk row permuted
  __shared__ __attribute__((aligned(16))) float sG[3][G_N * C];
  __shared__ float sLam[3];
  __shared__ __attribute__((aligned(16))) OpT sAo[2][C * LT];     // strictly-lower blocks of A (k permuted)
  __shared__ __attribute__((aligned(16))) OpT sP[2][C * LT];      // lower blocks of P (k permuted)
  __shared__ __attribute__((aligned(16))) OpT sTb[2][NB * 16 * LTB];  // F1: T_pp; F2: A_pp minus its 4x4 diagonal
  __shared__ float sAd2[PERCH ? 2 : 1][PERCH ? NB * 272 : 1];     // F2: diagonal blocks of A, fp32
  __shared__ float sAdT[VAR == V_F1 ? NPW : 1][VAR == V_F1 ? 272 : 1];  // F1: producer scratch
  __shared__ float sCarry[2][D];
  __shared__ float sCarryN2[2];
  __shared__ __attribute__((aligned(16))) IT sOst[NCW][C * P::LO];   // consumer output staging

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int T = a.T, H = a.H, NC = a.nchunks;
  const bool consumer = wv < NCW;
  const int pw = wv - NCW;                 // producer wave index
  const int ptid = tid - 64 * NCW;         // producer thread index
  const int chW = 16 * wv + cl;            // consumer lane's value channel

  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);

  // ================= producers =================
  uint4 rk[NPASS], rq[NPASS];              // raw key / query rows of one chunk
  float rg = 0.f, rb = 0.f;                // raw gate of row `lane` (producer wave NPW-1)

  auto prefetch = [&](int c) {             // global -> registers, chunk c
    const int c0 = c * C;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + ptid / TPR, part = ptid % TPR, t = c0 + r;
      const bool ok = r < C && t < T;
      const size_t row = ((size_t)(b * T + t) * H + h) * D + part * VEC;
      rk[ps] = ok ? *reinterpret_cast<const uint4 *>(kp + row) : uint4{0, 0, 0, 0};
      rq[ps] = ok ? *reinterpret_cast<const uint4 *>(qp + row) : uint4{0, 0, 0, 0};
    }
    if (pw == NPW - 1) {
      const int t = c0 + lane;
      const bool ok = lane < C && t < T;
      rg = ok ? a.g[(size_t)(b * T + t) * H + h] : 0.f;
      rb = (ok && !PERCH) ? a.beta[(size_t)(b * T + t) * H + h] : 0.f;
    }
  };

  // write 4 consecutive logical columns starting at k0 (multiple of 4) of a dk-permuted row
  auto put4 = [&](OpT *row, int k0, const float *v) {
    OpT *dst = row + kperm(k0);
    if constexpr (sizeof(OpT) == 2) {
      bf4 w;
      w[0] = (__bf16)v[0]; w[1] = (__bf16)v[1]; w[2] = (__bf16)v[2]; w[3] = (__bf16)v[3];
      *reinterpret_cast<bf4 *>(dst) = w;
    } else {
      *reinterpret_cast<f4 *>(dst) = f4{v[0], v[1], v[2], v[3]};
    }
  };

  auto stage = [&](int c) {                // registers -> normalised LDS tiles of chunk c
    const int s = c % 3;
    const int cin = (c + 1) & 1, cprev = c & 1;   // carry written for chunk c+1, read from chunk c-1
    OpT *X = sX[s], *Q = sQ[s], *XT = sXT[s];
    float *G = sG[s];
    for (int e = ptid; e < D; e += P::NPT) {
      const float x = sCarry[cprev][e];
      X[kperm(e)] = (OpT)x;
      XT[e * LT + kc<C>(0)] = (OpT)x;
    }
    if (ptid == 0) G[G_XN2 * C + 0] = sCarryN2[cprev];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + ptid / TPR, part = ptid % TPR;
      float xv[VEC], qv[VEC];
      unpack(rk[ps], IT(), xv);
      unpack(rq[ps], IT(), qv);
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) { sk += xv[e] * xv[e]; sq += qv[e] * qv[e]; }
      sk = group_sum<TPR>(sk);
      sq = group_sum<TPR>(sq);
      const float ik = safe_rsqrt(sk + a.eps_phi), iq = safe_rsqrt(sq + a.eps_phi);
#pragma unroll
      for (int e = 0; e < VEC; ++e) { xv[e] *= ik; qv[e] *= iq; }
      if (r + 1 < C) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) put4(X + (r + 1) * LX, part * VEC + e, xv + e);
#pragma unroll
        for (int e = 0; e < VEC; ++e) XT[(part * VEC + e) * LT + kc<C>(r + 1)] = (OpT)xv[e];
        if (part == 0) G[G_XN2 * C + r + 1] = sk * ik * ik;
      } else if (r + 1 == C) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) sCarry[cin][part * VEC + e] = xv[e];
        if (part == 0) sCarryN2[cin] = sk * ik * ik;
      }
      if (r < C) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) put4(Q + r * LX, part * VEC + e, qv + e);
      }
    }
    if (pw == NPW - 1) {   // clamp in log space, chunk-local inclusive scan
      const bool ok = lane < C && c * C + lane < T;
      const float g2 = ok ? fmaxf(rg, a.log_eps_gamma) : 0.f;
      const float L = wave_inclusive_scan(g2);
      if (lane < C) {
        G[G_LC * C + lane] = L;
        G[G_LM * C + lane] = L - g2;
        G[G_BETA * C + lane] = rb;
      }
    }
  };

  auto derive = [&](int c) {               // key-side tiles of chunk c (needs its staged inputs)
    const int s = c % 3, ds = c & 1;
    const OpT *X = sX[s], *Q = sQ[s];
    float *G = sG[s];
    auto wcol = [&](int col) { return PERCH ? 1.f : G[G_BETA * C + col] / (a.eps_eta + G[G_XN2 * C + col]); };
    auto gram = [&](const OpT *Am, int p, int q) {   // 16x16 block (p, q) of Am X^T
      f4 acc = zero4();
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2)
        mmap(acc, ldp(Am + (16 * p + cl) * LX + 32 * a2 + 8 * g4), ldp(X + (16 * q + cl) * LX + 32 * a2 + 8 * g4));
      return acc;
    };
    // diagonal Gram block pw (F1: T_pp; F2: A_pp)
    if (DELTA && pw < NB) {
      const int p = pw;
      const f4 acc = gram(X, p, p);
      const int col = 16 * p + cl;
      const float Lcol = G[G_LC * C + col], wc = wcol(col);
      const f4 Lmr = *reinterpret_cast<const f4 *>(G + G_LM * C + 16 * p + 4 * g4);
      f4 N;   // C-layout: N[4 g4 + i][cl] of the diagonal block (A with the step folded in for F1)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * __expf(Lmr[i] - Lcol) * wc;
        N[i] = (cl < 4 * g4 + i) ? v : 0.f;
      }
      const int r0 = 4 * g4;
      if (VAR == V_F1) {
        // T_pp = (I + N)^{-1}: T <- (I + N_d)^{-1} (I - N_o T), exact after 3 sweeps.
        float *Ad = sAdT[pw];
#pragma unroll
        for (int i = 0; i < 4; ++i) Ad[(r0 + i) * 17 + cl] = N[i];
        wave_lds_sync();
        f4 No;   // A-layout of N without its 4x4 diagonal sub-blocks: N[cl][4 g4 + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) No[i] = ((cl >> 2) == g4) ? 0.f : Ad[cl * 17 + r0 + i];
        const float n10 = Ad[(r0 + 1) * 17 + r0], n20 = Ad[(r0 + 2) * 17 + r0], n21 = Ad[(r0 + 2) * 17 + r0 + 1];
        const float n30 = Ad[(r0 + 3) * 17 + r0], n31 = Ad[(r0 + 3) * 17 + r0 + 1], n32 = Ad[(r0 + 3) * 17 + r0 + 2];
        f4 Z, Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Z[i] = (r0 + i == cl) ? 1.f : 0.f;
        auto local = [&](const f4 &z) {
          Y[0] = z[0];
          Y[1] = z[1] - n10 * Y[0];
          Y[2] = z[2] - n20 * Y[0] - n21 * Y[1];
          Y[3] = z[3] - n30 * Y[0] - n31 * Y[1] - n32 * Y[2];
        };
        local(Z);
#pragma unroll
        for (int it = 0; it < 3; ++it) {
          f4 cpl = zero4();
          mma16(cpl, No, Y);     // fp32 MFMA
          local(Z - cpl);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sTb[ds][(p * 16 + r0 + i) * LTB + cl] = (OpT)Y[i];
      } else {  // F2: full diagonal block (fp32) and its part outside the 4x4 diagonal sub-blocks
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sAd2[ds][p * 272 + (r0 + i) * 17 + cl] = N[i];
          sTb[ds][(p * 16 + r0 + i) * LTB + cl] = (OpT)((cl >> 2) == g4 ? 0.f : N[i]);
        }
      }
    }
    // off-diagonal A blocks and score blocks, a static round robin over producer waves
    constexpr int NG = DELTA ? P::NOFF : 0;
    constexpr int NJOB = NG + P::NPB;
#pragma unroll
    for (int jj = 0; jj < (NJOB + NPW - 1) / NPW; ++jj) {
      const int job = pw + jj * NPW;
      if (job < NJOB) {
        const bool isP = job >= NG;
        const int pj = isP ? job - NG : job;
        int p, q;
        if (isP) {
          p = 0;
          while ((p + 1) * (p + 2) / 2 <= pj) ++p;
          q = pj - p * (p + 1) / 2;
        } else {
          p = 1;
          while (p * (p + 1) / 2 <= pj) ++p;
          q = pj - p * (p - 1) / 2;
        }
        const f4 acc = gram(isP ? Q : X, p, q);
        const int col = 16 * q + cl;
        const float Lcol = G[G_LC * C + col], wc = wcol(col);
        // decay to the row: e^{L_i - L_j} for scores, e^{L_{i-1} - L_j} for the Gram
        const f4 Lr = *reinterpret_cast<const f4 *>(G + (isP ? G_LC : G_LM) * C + 16 * p + 4 * g4);
        OpT *dst = (isP ? sP[ds] : sAo[ds]) + kc<C>(col);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * p + 4 * g4 + i;
          const float v = acc[i] * __expf(Lr[i] - Lcol) * wc;
          dst[row * LT] = (OpT)((p > q || cl <= 4 * g4 + i) ? v : 0.f);   // Gram blocks have q < p
        }
      }
    }
    // per-row factors the consumers use
    if (pw == NPW - 1 && lane < C) {
      const float L = G[G_LC * C + lane], Lm = G[G_LM * C + lane];
      const float Llast = G[G_LC * C + C - 1];
      const float inv = 1.f / (a.eps_eta + G[G_XN2 * C + lane]);
      const float eta = PERCH ? inv : G[G_BETA * C + lane] * inv;
      G[G_GAM * C + lane] = __expf(Lm);
      G[G_EL * C + lane] = __expf(L);
      G[G_ETA * C + lane] = eta;
      G[G_CST * C + lane] = __expf(Llast - L) * (PERCH ? 1.f : eta);
      if (lane == 0) sLam[s] = __expf(Llast);
    }
  };

  // ================= consumers =================
  f4 sT[NA];                 // S^T of this wave's 16 channels, C-layout per dk block
  IT rv[NB][4];              // values of the next chunk, C-layout
  float rbeta[NB][4];        // F2/F2A: per-channel gains of the next chunk
  if (consumer) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) : zero4();
  }
  auto prefetch_v = [&](int c) {
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c * C + 16 * p + 4 * g4 + i;
        const size_t idx = ((size_t)(b * T + t) * H + h) * D + chW;
        rv[p][i] = (t < T) ? vp[idx] : (IT)0.f;
        if (PERCH) rbeta[p][i] = (t < T) ? a.beta[idx] : 0.f;
      }
  };

  auto consume = [&](int c) {
    const int s = c % 3, ds = c & 1, c0 = c * C;
    const OpT *X = sX[s], *Q = sQ[s], *XT = sXT[s];
    const float *G = sG[s];
    const OpT *Ao = sAo[ds], *Pm = sP[ds], *Tb = sTb[ds];
    Pr Sp[NA / 2];
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) Sp[a2] = mkp(cvt<OpT>(sT[2 * a2]), cvt<OpT>(sT[2 * a2 + 1]));
    f4 QS[NB], XS[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      QS[p] = zero4();
      XS[p] = zero4();
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2) {
        if (DELTA) mmap(XS[p], ldp(X + (16 * p + cl) * LX + 32 * a2 + 8 * g4), Sp[a2]);
        mmap(QS[p], ldp(Q + (16 * p + cl) * LX + 32 * a2 + 8 * g4), Sp[a2]);
      }
    }
    // A-layout operand of the 16x16 block (row block p, k block q) of a C x C tile
    auto blk1 = [&](const OpT *M, int p, int q) -> Frag {
      const int k0 = (C % 32 == 0) ? (32 * (q >> 1) + 8 * g4 + 4 * (q & 1)) : (16 * q + 4 * g4);
      return ld4(M + (16 * p + cl) * LT + k0);
    };
    auto blk2 = [&](const OpT *M, int p, int q) -> Pr {   // k blocks q, q+1 (q even)
      return ldp(M + (16 * p + cl) * LT + 32 * (q >> 1) + 8 * g4);
    };
    Frag Eb[NB];
    f4 Ef[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      const f4 gam = *reinterpret_cast<const f4 *>(G + G_GAM * C + 16 * p + 4 * g4);
      f4 R, eta4;
#pragma unroll
      for (int i = 0; i < 4; ++i) R[i] = to_f(rv[p][i]);
      if (DELTA) R -= gam * XS[p];
      if (PERCH) {
        const f4 inv = *reinterpret_cast<const f4 *>(G + G_ETA * C + 16 * p + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) eta4[i] = rbeta[p][i] * inv[i];
      }
      if (DELTA) {   // R -= sum_{q<p} A_pq E_q   (E_q = eta (.) E for F2)
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q + 1 < p; q += 2) mmap(acc, blk2(Ao, p, q), mkp(Eb[q], Eb[q + 1]));
        if (p & 1) mma16(acc, blk1(Ao, p, p - 1), Eb[p - 1]);
        R -= acc;
      }
      if (VAR == V_F1) {
        f4 E = zero4();
        mma16(E, ld4(Tb + (16 * p + cl) * LTB + 4 * g4), cvt<OpT>(R));
        Ef[p] = E;
        Eb[p] = cvt<OpT>(E);
      } else if (VAR == V_F2) {
        // rows 4g4..4g4+3 of block p: exact 4x4 solves, coupled by A_pp minus its 4x4 diagonal
        const float *Ad = sAd2[ds] + p * 272;
        const int r0 = 4 * g4;
        const float a10 = Ad[(r0 + 1) * 17 + r0], a20 = Ad[(r0 + 2) * 17 + r0], a21 = Ad[(r0 + 2) * 17 + r0 + 1];
        const float a30 = Ad[(r0 + 3) * 17 + r0], a31 = Ad[(r0 + 3) * 17 + r0 + 1], a32 = Ad[(r0 + 3) * 17 + r0 + 2];
        const Frag Ain = ld4(Tb + (16 * p + cl) * LTB + 4 * g4);
        f4 E, F;
        auto local = [&](const f4 &z) {
          E[0] = z[0];
          F[0] = eta4[0] * E[0];
          E[1] = z[1] - a10 * F[0];
          F[1] = eta4[1] * E[1];
          E[2] = z[2] - a20 * F[0] - a21 * F[1];
          F[2] = eta4[2] * E[2];
          E[3] = z[3] - a30 * F[0] - a31 * F[1] - a32 * F[2];
          F[3] = eta4[3] * E[3];
        };
        local(R);
#pragma unroll
        for (int it = 0; it < 3; ++it) {
          f4 cpl = zero4();
          mma16(cpl, Ain, cvt<OpT>(F));
          local(R - cpl);
        }
        Ef[p] = F;                 // eta (.) E feeds the state update and the outputs
        Eb[p] = cvt<OpT>(F);
      } else if (VAR == V_F1A) {
        Ef[p] = R;
        Eb[p] = cvt<OpT>(R);
      } else {
        const f4 F = eta4 * R;
        Ef[p] = F;
        Eb[p] = cvt<OpT>(F);
      }
    }
    // outputs o = e^{L} Q^ S0^T + P E'
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 O = *reinterpret_cast<const f4 *>(G + G_EL * C + 16 * p + 4 * g4) * QS[p];
#pragma unroll
      for (int q = 0; q + 1 <= p; q += 2) mmap(O, blk2(Pm, p, q), mkp(Eb[q], Eb[q + 1]));
      if (!(p & 1)) mma16(O, blk1(Pm, p, p), Eb[p]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sOst[wv][(16 * p + 4 * g4 + i) * P::LO + cl] = (IT)O[i];
    }
    wave_lds_sync();
    // each lane stores one step's 16 channels of this wave
#pragma unroll
    for (int r = lane; r < C; r += 64) {
      const int t = c0 + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 16 / VEC; ++j)
          *reinterpret_cast<uint4 *>(op + ((size_t)(b * T + t) * H + h) * D + 16 * wv + j * VEC) =
              *reinterpret_cast<const uint4 *>(&sOst[wv][r * P::LO + j * VEC]);
      }
    }
    // state: S^T <- e^{L_last} S^T + X^T diag(cst) E'
    Frag CE[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) CE[p] = cvt<OpT>(*reinterpret_cast<const f4 *>(G + G_CST * C + 16 * p + 4 * g4) * Ef[p]);
    const float lamtot = sLam[s];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) {
      f4 acc = sT[aa] * lamtot;
      if constexpr (NB == 1) {
        mma16(acc, ld4(XT + (16 * aa + cl) * LT + 4 * g4), CE[0]);
      } else {
#pragma unroll
        for (int p = 0; p < NB; p += 2)
          mmap(acc, ldp(XT + (16 * aa + cl) * LT + 32 * (p >> 1) + 8 * g4), mkp(CE[p], CE[p + 1]));
      }
      sT[aa] = acc;
    }
    if (a.chunk_states) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * NC + c) * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  };

  // ---------------- prologue ----------------
  if (!consumer) {
    // the carry slot read by chunk 0 is slot 0 (chunk -1's key = the incoming x_prev)
    for (int e = ptid; e < D; e += P::NPT) sCarry[0][e] = a.xprev0 ? a.xprev0[(size_t)bh * D + e] : 0.f;
    prefetch(0);
  } else {
    prefetch_v(0);
  }
  __syncthreads();
  if (pw == 0) {
    float s = 0.f;
    for (int e = lane; e < D; e += 64) s += sCarry[0][e] * sCarry[0][e];
    s = group_sum<64>(s);
    if (lane == 0) sCarryN2[0] = s;
  }
  __syncthreads();
  if (!consumer) {
    stage(0);
    if (NC > 1) prefetch(1);
  }
  __syncthreads();

  // ---------------- pipeline: iteration i derives chunk i, stages i+1, consumes i-1 ----------------
  for (int i = 0; i <= NC; ++i) {
    if (consumer) {
      if (i >= 1) {
        consume(i - 1);
        if (i < NC) prefetch_v(i);
      }
    } else {
      if (i + 1 < NC) {
        stage(i + 1);
        if (i + 2 < NC) prefetch(i + 2);
      }
      if (i < NC) derive(i);
    }
    __syncthreads();
  }

  if (consumer && a.S_out) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      *reinterpret_cast<f4 *>(a.S_out + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
  }
  if (a.write_tail && a.xprev_out && pw == 0) {
    float xv[2] = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * j;
      if (e < D) xv[j] = to_f(kp[((size_t)(b * T + T - 1) * H + h) * D + e]);
    }
    const float s = group_sum<64>(xv[0] * xv[0] + xv[1] * xv[1]);
    const float inv = safe_rsqrt(s + a.eps_phi);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = lane + 64 * j;
      if (e < D) a.xprev_out[(size_t)bh * D + e] = xv[j] * inv;
    }
  }
}

template <int VAR, typename IT, int D, int C>
hipError_t launch_pipe(const FwdArgs &a, hipStream_t s) {
  using P = Pipe<VAR, IT, D, C>;
  if constexpr (P::fits()) {
    hipLaunchKernelGGL((chunk_fwd_pipe<VAR, IT, D, C>), dim3(a.B * a.H), dim3(P::NT), 0, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int VAR, typename IT, int D>
bool pipe_fits_chunk(int chunk) {
  switch (chunk) {
    case 16: return Pipe<VAR, IT, D, 16>::fits();
    case 32: return Pipe<VAR, IT, D, 32>::fits();
    case 64: return Pipe<VAR, IT, D, 64>::fits();
  }
  return false;
}

template <int VAR, typename IT, int D>
hipError_t pipe_chunk(int chunk, const FwdArgs &a, hipStream_t s) {
  switch (chunk) {
    case 16: return launch_pipe<VAR, IT, D, 16>(a, s);
    case 32: return launch_pipe<VAR, IT, D, 32>(a, s);
    case 64: return launch_pipe<VAR, IT, D, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int VAR>
bool pipe_fits(bool bf16, int d, int chunk) {
  if (bf16) {
    if (d == 32) return pipe_fits_chunk<VAR, __bf16, 32>(chunk);
    if (d == 64) return pipe_fits_chunk<VAR, __bf16, 64>(chunk);
  } else {
    if (d == 32) return pipe_fits_chunk<VAR, float, 32>(chunk);
    if (d == 64) return pipe_fits_chunk<VAR, float, 64>(chunk);
  }
  return false;
}

template <int VAR>
hipError_t pipe_launch(bool bf16, int d, int chunk, const FwdArgs &a, hipStream_t s) {
  if (bf16) {
    if (d == 32) return pipe_chunk<VAR, __bf16, 32>(chunk, a, s);
    if (d == 64) return pipe_chunk<VAR, __bf16, 64>(chunk, a, s);
  } else {
    if (d == 32) return pipe_chunk<VAR, float, 32>(chunk, a, s);
    if (d == 64) return pipe_chunk<VAR, float, 64>(chunk, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool chunk_fwd_pipe_supported(int variant, bool bf16, int dk, int dv, int chunk) {
  if (dk != dv) return false;
  switch (variant) {
    case V_F1: return pipe_fits<V_F1>(bf16, dk, chunk);
    case V_F1A: return pipe_fits<V_F1A>(bf16, dk, chunk);
    case V_F2: return pipe_fits<V_F2>(bf16, dk, chunk);
    case V_F2A: return pipe_fits<V_F2A>(bf16, dk, chunk);
  }
  return false;
}

hipError_t launch_chunk_fwd_pipe(int variant, bool bf16, int dk, int dv, int chunk, const FwdArgs &a,
                                 hipStream_t s) {
  if (dk != dv) return hipErrorInvalidValue;
  switch (variant) {
    case V_F1: return pipe_launch<V_F1>(bf16, dk, chunk, a, s);
    case V_F1A: return pipe_launch<V_F1A>(bf16, dk, chunk, a, s);
    case V_F2: return pipe_launch<V_F2>(bf16, dk, chunk, a, s);
    case V_F2A: return pipe_launch<V_F2A>(bf16, dk, chunk, a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace falcon
