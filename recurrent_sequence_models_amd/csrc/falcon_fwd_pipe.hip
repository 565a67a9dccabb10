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
//     outputs and the state update;
//   producer waves, in the same iteration, build the key-side tiles of chunk
//     c+1 (decayed Gram A with the step folded in, scores P, diagonal-block
//     inverses T_pp), stage the raw keys / queries / values of chunk c+2 in LDS
//     and prefetch those of chunk c+3 into registers.
// One workgroup barrier per chunk.  Input tiles are triple-buffered, key-side
// tiles double-buffered.
//
// Operands are the raw (unnormalised) inputs: the feature map phi only scales
// rows, so its factors 1/sqrt(|k|^2 + eps) and 1/sqrt(|q|^2 + eps) are folded
// into the per-row decay / output / state factors and into the Gram and score
// tiles.  The producers compute the key-side tiles transposed, so each lane's
// MFMA result is exactly the consumer's A-operand fragment and is stored
// fragment-native (8 or 16 bytes per lane, no bank conflicts).  The consumers
// read X^T and the values in fragment layout with the transposing LDS read.
//
// Diagonal blocks: T_pp = (I + N)^{-1} (N strictly lower 16x16) and Falcon-2's
// per-channel systems (I + A_pp diag(eta_c)) e = r are solved by block-Jacobi
// sweeps over 4x4 sub-blocks: each lane group solves its own 4 rows or columns
// exactly, and the coupling between sub-blocks (strictly block-lower, hence
// nilpotent) is one 16x16 MFMA per sweep; three sweeps are exact.
#include "chunk_common.h"
#include "falcon_kernels.h"

namespace falcon {

namespace {

// per-row arrays of an input slot
enum {
  G_LC = 0,   // L_i, chunk-local inclusive log-decay sum
  G_LM,       // L_{i-1}
  G_IK,       // 1/sqrt(|k|^2 + eps) of the raw key in row i of X
  G_IQ,       // 1/sqrt(|q|^2 + eps)
  G_CF,       // column factor of the Gram and score tiles: IK_i * eta_i (F1/F1A) or IK_i (F2/F2A)
  G_ETA,      // eta_i (F1/F1A) or 1/(eps + |x_i|^2) (F2/F2A)
  G_GAM,      // e^{L_{i-1}} * IK_i           (consumers)
  G_EL,       // e^{L_i} * IQ_i               (consumers)
  G_CST,      // e^{L_last - L_i} * CF_i      (consumers)
  G_N
};

template <int VAR, typename IT, int D, int C>
struct Pipe {
  static constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  static constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2);
  static constexpr int NB = C / 16, NA = D / 16;
  static constexpr int SP = NB > 1 ? NB / 2 : 1;            // fragment pairs per tile row
  static constexpr int NCW = D / 16, NPW = 4, NT = 64 * (NCW + NPW);
  static constexpr int NPT = 64 * NPW;                       // producer threads
  static constexpr int PADE = 16 / (int)sizeof(IT);          // elements in 16 bytes
  static constexpr int LX = D + PADE;                        // X, Q rows (dk permuted), V rows
  static constexpr int LO = 16 + PADE;                       // output staging rows
  static constexpr int VEC = PADE;
  static constexpr int TPR = D / VEC;                        // producer threads per input row
  static constexpr int RPP = NPT / TPR;                      // rows per producer pass
  static constexpr int NPASS = (C + RPP - 1) / RPP;
  static constexpr int NOFF = NB * (NB - 1) / 2, NPB = NB * (NB + 1) / 2;
  static constexpr int FRAG = 64 * 8;                        // elements of one fragment pair
  static constexpr size_t lds_bytes() {
    return sizeof(IT) * (3 * 3 * C * LX + 2 * (2 * NB * SP * FRAG + NB * 64 * 4) + NCW * C * LO) +
           4 * (3 * G_N * C + 3 + (PERCH ? 2 * NB * 272 : 0) + 2 * D + 6);
  }
  static constexpr bool fits() { return lds_bytes() + 256 <= 160 * 1024; }
};

template <int VAR, typename IT, int D, int C>
__global__ __launch_bounds__(64 * (D / 16 + 4)) void chunk_fwd_pipe(FwdArgs a) {
  using P = Pipe<VAR, IT, D, C>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = P::NB, NA = P::NA, NCW = P::NCW, NPW = P::NPW, SP = P::SP;
  constexpr int LX = P::LX, VEC = P::VEC, TPR = P::TPR, RPP = P::RPP, NPASS = P::NPASS;
  constexpr bool PERCH = P::PERCH, DELTA = P::DELTA;

  __shared__ __attribute__((aligned(16))) OpT sX[3][C * LX];      // raw x_i = k_{i-1}, dk permuted
  __shared__ __attribute__((aligned(16))) OpT sQ[3][C * LX];      // raw q_i, dk permuted
  __shared__ __attribute__((aligned(16))) IT sV[3][C * LX];       // raw v_i, natural channel order
  __shared__ __attribute__((aligned(16))) float sG[3][G_N * C];
  __shared__ float sLam[3];
  __shared__ __attribute__((aligned(16))) OpT sAo[2][NB * SP * P::FRAG];  // A_pq (q < p), fragment pairs
  __shared__ __attribute__((aligned(16))) OpT sP[2][NB * SP * P::FRAG];   // P_pq (q <= p), fragment pairs
  __shared__ __attribute__((aligned(16))) OpT sTb[2][NB * 64 * 4];        // F1: T_pp; F2: A_pp off its 4x4 diagonal
  __shared__ float sAd2[PERCH ? 2 : 1][PERCH ? NB * 272 : 1];             // F2: diagonal blocks of A (C-layout)
  __shared__ __attribute__((aligned(16))) OpT sCarry[2][D];               // raw key carried to the next chunk
  __shared__ float sCarryF[2][3];                                         // its IK, CF, ETA
  __shared__ __attribute__((aligned(16))) IT sOst[NCW][C * P::LO];        // consumer output staging

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
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

  // fragment-native offset of tile (p, q) of a pair buffer; pairs are tiles (2s, 2s+1)
  auto fragoff = [&](int p, int q) { return ((p * SP + (q >> 1)) * 64 + lane) * 8 + (q & 1) * 4; };

  // ================= producers =================
  uint4 rk[NPASS], rq[NPASS], rv[NPASS];   // raw key / query / value rows of one chunk
  float rb1[NPASS];                        // beta of the row after (the step of x_{r+1} = phi(k_r))
  float rg = 0.f;                          // raw gate of row `lane` (producer wave NPW-1)

  // global -> registers, chunk c.  Rows past the end are clamped to the last
  // token (always in bounds) and zeroed when staged.
  auto prefetch = [&](int c) {
    const int c0 = c * C;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + ptid / TPR, part = ptid % TPR;
      const int t = min(c0 + r, T - 1);
      const size_t row = ((size_t)(b * T + t) * H + h) * D + part * VEC;
      rk[ps] = *reinterpret_cast<const uint4 *>(kp + row);
      rq[ps] = *reinterpret_cast<const uint4 *>(qp + row);
      rv[ps] = *reinterpret_cast<const uint4 *>(vp + row);
      if (!PERCH) rb1[ps] = a.beta[(size_t)(b * T + min(c0 + r + 1, T - 1)) * H + h];
    }
    if (pw == NPW - 1) rg = a.g[(size_t)(b * T + min(c0 + lane, T - 1)) * H + h];
  };

  // store VEC raw elements (one 16-byte vector) of logical columns k0..k0+VEC-1 in a dk-permuted row
  auto put_perm = [&](OpT *row, int k0, const uint4 &u) {
    if constexpr (sizeof(OpT) == 2) {   // 8 elements = two groups of 4, each contiguous after kperm
      *reinterpret_cast<uint2 *>(row + kperm(k0)) = uint2{u.x, u.y};
      *reinterpret_cast<uint2 *>(row + kperm(k0 + 4)) = uint2{u.z, u.w};
    } else {
      *reinterpret_cast<uint4 *>(row + kperm(k0)) = u;
    }
  };

  // registers -> raw LDS tiles of chunk c, with the per-row norms and step factors
  auto stage = [&](int c) {
    const int s = c % 3, c0 = c * C;
    const int cin = (c + 1) & 1, cprev = c & 1;   // carry written for chunk c+1, read from chunk c-1
    OpT *X = sX[s], *Q = sQ[s];
    IT *V = sV[s];
    float *G = sG[s];
    for (int e = ptid; e < D / 4; e += P::NPT)
      *reinterpret_cast<Frag *>(X + kperm(4 * e)) = *reinterpret_cast<const Frag *>(&sCarry[cprev][4 * e]);
    if (ptid == 0) {
      G[G_IK * C] = sCarryF[cprev][0];
      G[G_CF * C] = sCarryF[cprev][1];
      G[G_ETA * C] = sCarryF[cprev][2];
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int r = ps * RPP + ptid / TPR, part = ptid % TPR;
      const bool ok = c0 + r < T;
      const uint4 k4 = keep_or_zero(ok, rk[ps]), q4 = keep_or_zero(ok, rq[ps]), v4 = keep_or_zero(ok, rv[ps]);
      float xv[VEC], qv[VEC];
      unpack(k4, IT(), xv);
      unpack(q4, IT(), qv);
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) { sk += xv[e] * xv[e]; sq += qv[e] * qv[e]; }
      sk = group_sum<TPR>(sk);
      sq = group_sum<TPR>(sq);
      const float ik = safe_rsqrt(sk + a.eps_phi), iq = safe_rsqrt(sq + a.eps_phi);
      // key k_{c0+r} becomes x_{c0+r+1}: its step eta uses beta_{c0+r+1}
      const float inv = fast_rcp(a.eps_eta + sk * ik * ik);
      const float eta = PERCH ? inv : (c0 + r + 1 < T ? rb1[ps] : 0.f) * inv;
      const float cf = PERCH ? ik : ik * eta;
      if (r + 1 < C) {
        put_perm(X + (r + 1) * LX, part * VEC, k4);
        if (part == 0) {
          G[G_IK * C + r + 1] = ik;
          G[G_CF * C + r + 1] = cf;
          G[G_ETA * C + r + 1] = eta;
        }
      } else if (r + 1 == C) {
        *reinterpret_cast<uint4 *>(&sCarry[cin][part * VEC]) = k4;
        if (part == 0) {
          sCarryF[cin][0] = ik;
          sCarryF[cin][1] = cf;
          sCarryF[cin][2] = eta;
        }
      }
      if (r < C) {
        put_perm(Q + r * LX, part * VEC, q4);
        *reinterpret_cast<uint4 *>(V + r * LX + part * VEC) = v4;
        if (part == 0) G[G_IQ * C + r] = iq;
      }
    }
    if (pw == NPW - 1) {   // clamp in log space, chunk-local inclusive scan
      const bool ok = lane < C && c0 + lane < T;
      const float g2 = ok ? fmaxf(rg, a.log_eps_gamma) : 0.f;
      const float L = wave_inclusive_scan(g2);
      if (lane < C) {
        G[G_LC * C + lane] = L;
        G[G_LM * C + lane] = L - g2;
      }
    }
  };

  // key-side tiles of chunk c (needs its staged inputs)
  auto derive = [&](int c) {
    const int s = c % 3, ds = c & 1;
    const OpT *X = sX[s], *Q = sQ[s];
    float *G = sG[s];
    // A-operand fragments of rows 16 blk .. 16 blk + 15 of M (raw, dk permuted)
    auto rows16 = [&](const OpT *M, int blk, Pr (&out)[NA / 2]) {
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2) out[a2] = ldp(M + (16 * blk + cl) * LX + 32 * a2 + 8 * g4);
    };
    // lane (g, c) of the result: <Am_{4g+i}, Bm_c> for the two 16-row blocks
    auto tile = [&](const Pr (&Am)[NA / 2], const Pr (&Bm)[NA / 2]) {
      f4 acc = zero4();
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2) mmap(acc, Am[a2], Bm[a2]);
      return acc;
    };
    // Gram (isP = 0) or score (isP = 1) block (p, q), transposed: lane (g, c) holds
    // element (row 16p + c, col 16q + 4g + i), the consumers' A-operand fragment.
    auto finish = [&](const f4 &acc, int isP, int p, int q) {
      const f4 cf = *reinterpret_cast<const f4 *>(G + G_CF * C + 16 * q + 4 * g4);
      const f4 Lc4 = *reinterpret_cast<const f4 *>(G + G_LC * C + 16 * q + 4 * g4);
      const int row = 16 * p + cl;
      const float Lrow = G[(isP ? G_LC : G_LM) * C + row];
      const float rf = G[(isP ? G_IQ : G_IK) * C + row];
      f4 val;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * __expf(Lrow - Lc4[i]) * rf * cf[i];
        val[i] = (p > q || 4 * g4 + i <= cl) ? v : 0.f;
      }
      *reinterpret_cast<Frag *>(&(isP ? sP[ds] : sAo[ds])[fragoff(p, q)]) = cvt<OpT>(val);
    };
    // diagonal block p: F1 -> T_pp (A-layout), F2 -> A_pp (fp32, C-layout) and A_pp off its 4x4 diagonal
    auto diag = [&](const f4 &acc, int p) {   // acc: <x_{16p+4g+i}, x_{16p+c}> (symmetric)
      const int r0 = 4 * g4;
      const f4 cf4 = *reinterpret_cast<const f4 *>(G + G_CF * C + 16 * p + r0);
      const f4 ik4 = *reinterpret_cast<const f4 *>(G + G_IK * C + 16 * p + r0);
      const f4 Lc4 = *reinterpret_cast<const f4 *>(G + G_LC * C + 16 * p + r0);
      const f4 Lm4 = *reinterpret_cast<const f4 *>(G + G_LM * C + 16 * p + r0);
      const float Lc1 = G[G_LC * C + 16 * p + cl], Lm1 = G[G_LM * C + 16 * p + cl];
      const float ik1 = G[G_IK * C + 16 * p + cl], cf1 = G[G_CF * C + 16 * p + cl];
      f4 NA4, NC4;   // N[16p+c][16p+4g+i] (A-layout) and N[16p+4g+i][16p+c] (C-layout)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float va = acc[i] * __expf(Lm1 - Lc4[i]) * ik1 * cf4[i];
        const float vc = acc[i] * __expf(Lm4[i] - Lc1) * ik4[i] * cf1;
        NA4[i] = (r0 + i < cl) ? va : 0.f;
        NC4[i] = (cl < r0 + i) ? vc : 0.f;
      }
      if constexpr (VAR == V_F1) {
        // row-oriented: T (I + N) = I, so T <- (I - T N_o)(I + N_d)^{-1}, exact after 3 sweeps;
        // Y holds T in A-layout (row c, columns 4g..4g+3 of the block).
        // n_ab = N[4g+a][4g+b] sits in lane (g, 4g+a), entry b of NA4.
        const int src = 16 * g4 + r0;
        const float n10 = __shfl(NA4[0], src + 1), n20 = __shfl(NA4[0], src + 2), n21 = __shfl(NA4[1], src + 2);
        const float n30 = __shfl(NA4[0], src + 3), n31 = __shfl(NA4[1], src + 3), n32 = __shfl(NA4[2], src + 3);
        f4 NoC;   // C-layout of N without its 4x4 diagonal sub-blocks
#pragma unroll
        for (int i = 0; i < 4; ++i) NoC[i] = ((cl >> 2) == g4) ? 0.f : NC4[i];
        f4 Z, Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Z[i] = (r0 + i == cl) ? 1.f : 0.f;
        auto local = [&](const f4 &w) {     // t (I + N_gg) = w, t a row of 4
          Y[3] = w[3];
          Y[2] = w[2] - Y[3] * n32;
          Y[1] = w[1] - Y[2] * n21 - Y[3] * n31;
          Y[0] = w[0] - Y[1] * n10 - Y[2] * n20 - Y[3] * n30;
        };
        local(Z);
#pragma unroll
        for (int it = 0; it < 3; ++it) {
          f4 cpl = zero4();
          mma16(cpl, NoC, Y);   // fp32: C-layout of N_o^T Y^T = A-layout of Y N_o
          local(Z - cpl);
        }
        *reinterpret_cast<Frag *>(&sTb[ds][(p * 64 + lane) * 4]) = cvt<OpT>(Y);
      } else {
        f4 NoA;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sAd2[ds][p * 272 + (r0 + i) * 17 + cl] = NC4[i];
          NoA[i] = ((cl >> 2) == g4) ? 0.f : NA4[i];
        }
        *reinterpret_cast<Frag *>(&sTb[ds][(p * 64 + lane) * 4]) = cvt<OpT>(NoA);
      }
    };
    // per-row factors the consumers use
    auto rowfac = [&]() {
      if (lane < C) {
        const float L = G[G_LC * C + lane], Lm = G[G_LM * C + lane];
        const float Llast = G[G_LC * C + C - 1];
        G[G_GAM * C + lane] = __expf(Lm) * G[G_IK * C + lane];
        G[G_EL * C + lane] = __expf(L) * G[G_IQ * C + lane];
        G[G_CST * C + lane] = __expf(Llast - L) * G[G_CF * C + lane];
        if (lane == 0) sLam[s] = __expf(Llast);
      }
    };
    auto run = [&](auto wc) {
      constexpr int w = decltype(wc)::value;
      constexpr JobList J = make_jobs(NB, DELTA, w);
      constexpr int NJ = J.n > 0 ? J.n : 1;
      Pr Dop[NA / 2], Aop[NJ][NA / 2], Bop[NJ][NA / 2];
      if constexpr (J.diag >= 0) rows16(X, J.diag, Dop);
#pragma unroll
      for (int j = 0; j < J.n; ++j) {
        rows16(X, J.q[j], Aop[j]);
        rows16(J.isP[j] ? Q : X, J.p[j], Bop[j]);
      }
      f4 dacc, acc[NJ];
      if constexpr (J.diag >= 0) dacc = tile(Dop, Dop);
#pragma unroll
      for (int j = 0; j < J.n; ++j) acc[j] = tile(Aop[j], Bop[j]);
      if constexpr (J.diag >= 0) diag(dacc, J.diag);
#pragma unroll
      for (int j = 0; j < J.n; ++j) finish(acc[j], J.isP[j], J.p[j], J.q[j]);
      if constexpr (w == NPW - 1) rowfac();
    };
    if (pw == 0) run(std::integral_constant<int, 0>());
    else if (pw == 1) run(std::integral_constant<int, 1>());
    else if (pw == 2) run(std::integral_constant<int, 2>());
    else run(std::integral_constant<int, 3>());
  };

  // ================= consumers =================
  f4 sT[NA];                 // S^T of this wave's 16 channels, C-layout per dk block
  float rbeta[NB][4];        // F2/F2A: per-channel gains of the next chunk
  if (consumer) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) : zero4();
  }
  auto prefetch_beta = [&](int c) {
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c * C + 16 * p + 4 * g4 + i;
        rbeta[p][i] = (t < T) ? a.beta[((size_t)(b * T + t) * H + h) * D + chW] : 0.f;
      }
  };

  auto consume = [&](int c) {
    const int s = c % 3, ds = c & 1, c0 = c * C;
    const OpT *X = sX[s], *Q = sQ[s];
    const IT *V = sV[s];
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
    auto vcol = [&](int j4) { return 16 * wv + 4 * j4; };
    Frag Eb[NB];
    f4 Ef[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 R = to_f4(ldT(V, LX, 16 * p, vcol, lane));   // C-layout values of this wave's channels
      if (DELTA) R -= *reinterpret_cast<const f4 *>(G + G_GAM * C + 16 * p + 4 * g4) * XS[p];
      f4 eta4;
      if (PERCH) {
        const f4 inv = *reinterpret_cast<const f4 *>(G + G_ETA * C + 16 * p + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) eta4[i] = rbeta[p][i] * inv[i];
      }
      if (DELTA) {   // R -= sum_{q<p} A_pq E_q   (E_q = eta (.) E for F2)
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q + 1 < p; q += 2) mmap(acc, ldp(Ao + fragoff(p, q)), mkp(Eb[q], Eb[q + 1]));
        if (p & 1) mma16(acc, ld4(Ao + fragoff(p, p - 1)), Eb[p - 1]);
        R -= acc;
      }
      if constexpr (VAR == V_F1) {
        f4 E = zero4();
        mma16(E, ld4(Tb + (p * 64 + lane) * 4), cvt<OpT>(R));
        Ef[p] = E;
        Eb[p] = cvt<OpT>(E);
      } else if constexpr (VAR == V_F2) {
        // rows 4g4..4g4+3 of block p: exact 4x4 solves, coupled by A_pp minus its 4x4 diagonal
        const float *Ad = sAd2[ds] + p * 272;
        const int r0 = 4 * g4;
        const float a10 = Ad[(r0 + 1) * 17 + r0], a20 = Ad[(r0 + 2) * 17 + r0], a21 = Ad[(r0 + 2) * 17 + r0 + 1];
        const float a30 = Ad[(r0 + 3) * 17 + r0], a31 = Ad[(r0 + 3) * 17 + r0 + 1], a32 = Ad[(r0 + 3) * 17 + r0 + 2];
        const Frag Ain = ld4(Tb + (p * 64 + lane) * 4);
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
      } else if constexpr (VAR == V_F1A) {
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
      for (int q = 0; q + 1 <= p; q += 2) mmap(O, ldp(Pm + fragoff(p, q)), mkp(Eb[q], Eb[q + 1]));
      if (!(p & 1)) mma16(O, ld4(Pm + fragoff(p, p)), Eb[p]);
#pragma unroll
      for (int i = 0; i < 4; ++i) sOst[wv][(16 * p + 4 * g4 + i) * P::LO + cl] = (IT)O[i];
    }
    wave_lds_sync();
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
    // state: S^T <- e^{L_last} S^T + X~^T diag(cst) E'   (X~ raw keys; cst carries their norm)
    Frag CE[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) CE[p] = cvt<OpT>(*reinterpret_cast<const f4 *>(G + G_CST * C + 16 * p + 4 * g4) * Ef[p]);
    const float lamtot = sLam[s];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) {
      auto dkcol = [&](int j4) { return kperm(16 * aa + 4 * j4); };
      f4 acc = sT[aa] * lamtot;
      if constexpr (NB == 1) {
        mma16(acc, ldT(X, LX, 0, dkcol, lane), CE[0]);
      } else {
#pragma unroll
        for (int p = 0; p < NB; p += 2)
          mmap(acc, mkp(ldT(X, LX, 16 * p, dkcol, lane), ldT(X, LX, 16 * p + 16, dkcol, lane)), mkp(CE[p], CE[p + 1]));
      }
      sT[aa] = acc;
    }
    if (a.chunk_states) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * NC + c) * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  };

  // Each role runs its own loop, so neither keeps the other's loop-carried
  // registers live; both pass the same number of workgroup barriers (two in the
  // prologue, then one per iteration), which is what the barrier counts.
  if (consumer) {
    if (PERCH) prefetch_beta(0);
    __syncthreads();
    __syncthreads();
    // iteration i consumes chunk i-1 while the producers derive chunk i and stage i+1
    for (int i = 0; i <= NC; ++i) {
      if (i >= 1) {
        consume(i - 1);
        if (PERCH && i < NC) prefetch_beta(i);
      }
      __syncthreads();
    }
    if (a.S_out) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.S_out + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  } else {
    // chunk 0's first key is the incoming x_prev (already a feature: factor 1)
    for (int e = ptid; e < D; e += P::NPT) sCarry[0][e] = (OpT)(a.xprev0 ? a.xprev0[(size_t)bh * D + e] : 0.f);
    prefetch(0);
    if (pw == 0) {
      float s = 0.f;
      for (int e = lane; e < D; e += 64) {
        const float x = a.xprev0 ? a.xprev0[(size_t)bh * D + e] : 0.f;
        s += x * x;
      }
      s = group_sum<64>(s);
      if (lane == 0) {
        const float inv = fast_rcp(a.eps_eta + s);
        const float eta = PERCH ? inv : a.beta[(size_t)(b * T) * H + h] * inv;
        sCarryF[0][0] = 1.f;
        sCarryF[0][1] = PERCH ? 1.f : eta;
        sCarryF[0][2] = eta;
      }
    }
    __syncthreads();
    stage(0);
    if (NC > 1) prefetch(1);
    __syncthreads();
    for (int i = 0; i <= NC; ++i) {
      if (i + 1 < NC) {
        stage(i + 1);
        if (i + 2 < NC) prefetch(i + 2);
      }
      if (i < NC) derive(i);
      __syncthreads();
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
