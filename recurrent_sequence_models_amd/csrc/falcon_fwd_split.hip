// Chunk-parallel ("split") forward pass of Falcon-1 / 1A / 2 / 2A on gfx950.
//
// The chunked form ([P1] 三种等价形式 form C and Figure 4-C; [P2] 三种视角)
// separates what depends on the carried state from what does not:
//   * everything built from keys, queries and gates of one chunk -- the decayed
//     Gram blocks A_pq, the score blocks P_pq, the diagonal-block inverses T_pp
//     (F1) or the Falcon-2 diagonal blocks, and the per-row decay / norm / step
//     factors -- is independent across chunks;
//   * the residuals, outputs and the state update of chunk c need S at its start.
// The prep kernel runs one workgroup per chunk over the whole device and writes
// the first group, per chunk, as an "image": the exact LDS layout the scan
// reads.  The scan kernel runs one to eight workgroups per sequence (slices of
// the value channels): copy waves stream the key / query rows, the slice's
// values and the chunk image into double-buffered LDS one chunk ahead, and one
// consumer wave per 16 value channels carries S^T in registers.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// Image of one chunk (bytes, tiles in the input dtype, fragment pairs of 64
// lanes x 8 elements; slots hold only the tiles that exist):
//   A   : F2: A_pq, q < p         -- pair slot aslot_base(p) + q/2, half q&1
//   P   : P_pq, q <= p            -- pair slot pslot_base(p) + q/2, half q&1
//   T   : F1: the whole inverse T = (I + A)^{-1}, blocks T_pq, q <= p, laid out
//         like P; F2: A_pp without its 4x4 diagonal sub-blocks, one fragment each
//   AD  : F2 only, the 6 coefficients of each 4x4 diagonal sub-block (8 floats)
//   F   : per-row GAM, EL, CST, ETA (fp32, C each) and e^{L_last}
// With the whole T, Falcon-1's residuals of a chunk are E = T R with every
// block independent (no substitution across row blocks on the scan's path).
#include "chunk_common.h"
#include "falcon_kernels.h"

namespace falcon {

namespace {

// per-row arrays of the prep kernel
enum {
  R_LC = 0, R_LM, R_IK, R_IQ, R_CF, R_ETA,
  // separable decay factors around L_ref = L_last / 2 (used while |L_last| <= 160):
  R_EP,   // e^{L_i - L_ref} IQ_i       rows of score blocks
  R_EA,   // e^{L_{i-1} - L_ref} IK_i   rows of Gram blocks
  R_EC,   // e^{L_ref - L_j} CF_j       columns of both
  R_N
};
// per-row factors in the image (consumers)
enum {
  F_GAM = 0,  // e^{L_{i-1}} * IK_i
  F_EL,       // e^{L_i} * IQ_i
  F_CST,      // e^{L_last - L_i} * CF_i
  F_ETA,      // 1/(eps + |x_i|^2)  (Falcon-2 / 2A)
  F_N
};

constexpr int pslot_base(int p) {
  int b = 0;
  for (int i = 0; i < p; ++i) b += i / 2 + 1;
  return b;
}
constexpr int aslot_base(int p) {
  int b = 0;
  for (int i = 1; i < p; ++i) b += (i - 1) / 2 + 1;
  return b;
}

template <int VAR, typename IT, int D, int C>
struct Split {
  static constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  static constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2);
  static constexpr int NB = C / 16, NA = D / 16;
  static constexpr int FRAG = 64 * 8;                        // elements of one fragment pair
  static constexpr int SZ = (int)sizeof(IT);
  // Whole T = (I + A)^{-1} in the image for Falcon-1 (scan: E = T R, no substitution
  // across row blocks).  Off: on the 130M-layer shape it left the scan's time
  // unchanged and the fp32 inverse in LDS halved the prep kernel's occupancy.
  static constexpr bool TFULL = false;
  // Gram blocks go to the scan when it substitutes across row blocks (F2, or F1
  // with diagonal-block inverses only)
  static constexpr bool HAS_A = DELTA && !TFULL;
  static constexpr int NSP = pslot_base(NB), NSA = HAS_A ? aslot_base(NB) : 0;
  static constexpr int OFF_A = 0;
  static constexpr int OFF_P = OFF_A + NSA * FRAG * SZ;
  static constexpr int OFF_T = OFF_P + NSP * FRAG * SZ;
  static constexpr int OFF_AD = OFF_T + (TFULL ? NSP * FRAG * SZ : DELTA ? NB * 256 * SZ : 0);
  static constexpr int OFF_F = OFF_AD + (VAR == V_F2 ? NB * 32 * 4 : 0);
  static constexpr int IMG = ((OFF_F + (F_N * C + 4) * 4) + 15) / 16 * 16;
  static constexpr int NU = IMG / 16;                        // 16-byte units of the image
  // shared
  static constexpr int PADE = 16 / SZ, VEC = PADE;
  static constexpr int LX = D + PADE;                        // X, Q rows (dk permuted), V rows
  static constexpr int TPR = D / VEC;                        // threads per input row
  // prep kernel: 4 waves, one chunk
  static constexpr int NPW = 4, NPT = 256;
  static constexpr int RPP = NPT / TPR, NPASS = (C + RPP - 1) / RPP;
  static constexpr int LDT = C + 4;                          // fp32 rows of the prep's A and T
  static constexpr size_t prep_lds() { return (size_t)SZ * 2 * C * LX + 4 * R_N * C + (TFULL ? 8 * C * LDT : 0); }
  static size_t workspace(int bhc) { return (size_t)bhc * IMG; }
};

// The scan of one sequence is split over NS workgroups by value channel (rows
// of S evolve independently given the keys): each takes D/NS channels with
// one consumer wave per 16 of them, plus 8 copy waves that stage the shared
// key / query rows and chunk image and its own value columns.
template <int VAR, typename IT, int D, int C, int NS>
struct Scan {
  using S = Split<VAR, IT, D, C>;
  static constexpr int DS = D / NS;                          // value channels per workgroup
  static constexpr int NCW = DS / 16, NSW = 8, NT = 64 * (NCW + NSW), NST = 64 * NSW;
  static constexpr int LXV = DS + S::PADE;                   // V rows (this workgroup's channels)
  static constexpr int RPC = NST / S::TPR, NPK = (C + RPC - 1) / RPC;   // key / query rows per copy pass
  static constexpr int TPV = DS / S::VEC, RPV = NST / TPV, NPV = (C + RPV - 1) / RPV;
  static constexpr int NPI = (S::NU + NST - 1) / NST;
  static constexpr size_t lds() { return (size_t)S::SZ * 2 * (3 * C * S::LX + C * LXV) + 2 * (size_t)S::IMG; }
  static constexpr bool fits() {
    return DS >= 16 && D % NS == 0 && lds() + 256 <= 160 * 1024 && S::prep_lds() + 256 <= 64 * 1024;
  }
};

// fragment-native element offset of tile (.., q) in a pair buffer whose row of pairs starts at slot `base`
__device__ __forceinline__ int frag_off(int base, int q, int lane) { return ((base + (q >> 1)) * 64 + lane) * 8 + (q & 1) * 4; }

// store VEC raw elements (one 16-byte vector) of logical columns k0..k0+VEC-1 in a dk-permuted row
template <typename OpT>
__device__ __forceinline__ void put_perm(OpT *row, int k0, const uint4 &u) {
  if constexpr (sizeof(OpT) == 2) {   // 8 elements = two groups of 4, each contiguous after kperm
    *reinterpret_cast<uint2 *>(row + kperm(k0)) = uint2{u.x, u.y};
    *reinterpret_cast<uint2 *>(row + kperm(k0 + 4)) = uint2{u.z, u.w};
  } else {
    *reinterpret_cast<uint4 *>(row + kperm(k0)) = u;
  }
}

// VEC fp32 values of the carried feature x_prev, converted to the operand type
template <typename OpT, int VEC>
__device__ __forceinline__ uint4 pack_feature(const float *x, float &ss) {
  OpT tmp[VEC];
  ss = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    tmp[e] = (OpT)x[e];
    ss += x[e] * x[e];
  }
  return *reinterpret_cast<const uint4 *>(tmp);
}

// VEC raw values scaled by f, in the operand type (one 16-byte vector)
template <typename OpT, int VEC>
__device__ __forceinline__ uint4 scale_pack(const float *x, float f) {
  OpT tmp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) tmp[e] = (OpT)(x[e] * f);
  return *reinterpret_cast<const uint4 *>(tmp);
}

// ============================== prep kernel ==============================
template <int VAR, typename IT, int D, int C>
__global__ __launch_bounds__(256) void chunk_prep(FwdArgs a, unsigned char *ws) {
  using S = Split<VAR, IT, D, C>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = S::NB, NA = S::NA, LX = S::LX, VEC = S::VEC, TPR = S::TPR, RPP = S::RPP;
  constexpr bool PERCH = S::PERCH, DELTA = S::DELTA;

  __shared__ __attribute__((aligned(16))) OpT sX[C * LX];   // raw x_i = k_{i-1}, dk permuted
  __shared__ __attribute__((aligned(16))) OpT sQ[C * LX];   // raw q_i, dk permuted
  __shared__ __attribute__((aligned(16))) float sR[R_N * C];
  __shared__ __attribute__((aligned(16))) float sA64[S::TFULL ? C * S::LDT : 1];   // F1: fp32 A (off-diagonal blocks)
  __shared__ __attribute__((aligned(16))) float sT64[S::TFULL ? C * S::LDT : 1];   // F1: fp32 T (lower blocks)
  constexpr int LDT = S::LDT;

  const int tid = threadIdx.x, lane = tid & 63, pw = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int NC = a.nchunks, T = a.T, H = a.H;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC, b = bh / H, h = bh % H, c0 = c * C;
  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  unsigned char *img = ws + (size_t)blockIdx.x * S::IMG;
  OpT *gA = reinterpret_cast<OpT *>(img + S::OFF_A);
  OpT *gP = reinterpret_cast<OpT *>(img + S::OFF_P);
  OpT *gT = reinterpret_cast<OpT *>(img + S::OFF_T);
  float *gAd = reinterpret_cast<float *>(img + S::OFF_AD);
  float *gF = reinterpret_cast<float *>(img + S::OFF_F);

  // ---- rows: X row r holds k_{c0+r-1} (x_prev for the first row of the sequence), Q row r holds q_{c0+r}
#pragma unroll
  for (int ps = 0; ps < S::NPASS; ++ps) {
    const int r = ps * RPP + tid / TPR, part = tid % TPR;
    if (r < C) {
      const int tk = c0 + r - 1, tq = c0 + r;
      // loads use in-bounds (clamped) rows; rows outside the sequence are zeroed after the load
      const int tkc = min(max(tk, 0), T - 1), tqc = min(tq, T - 1);
      const uint4 kraw = *reinterpret_cast<const uint4 *>(kp + ((size_t)(b * T + tkc) * H + h) * D + part * VEC);
      const uint4 qraw = *reinterpret_cast<const uint4 *>(qp + ((size_t)(b * T + tqc) * H + h) * D + part * VEC);
      uint4 k4 = keep_or_zero(tk >= 0 && tk < T, kraw);
      const uint4 q4 = keep_or_zero(tq < T, qraw);
      float xv[VEC], qv[VEC];
      float sk = 0.f, sq = 0.f;
      if (tk < 0) {   // the carried feature phi(k_{-1}): fp32, already normalised
        float xf[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) xf[e] = a.xprev0 ? a.xprev0[(size_t)bh * D + part * VEC + e] : 0.f;
        k4 = pack_feature<OpT, VEC>(xf, sk);
      } else {
        unpack(k4, IT(), xv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sk += xv[e] * xv[e];
      }
      unpack(q4, IT(), qv);
#pragma unroll
      for (int e = 0; e < VEC; ++e) sq += qv[e] * qv[e];
      sk = group_sum<TPR>(sk);
      sq = group_sum<TPR>(sq);
      const float ik = tk < 0 ? 1.f : safe_rsqrt(sk + a.eps_phi);
      const float iq = safe_rsqrt(sq + a.eps_phi);
      const float inv = fast_rcp(a.eps_eta + sk * ik * ik);
      const float braw = PERCH ? 0.f : a.beta[(size_t)(b * T + tqc) * H + h];
      const float eta = PERCH ? inv : (tq < T ? braw : 0.f) * inv;
      put_perm(sX + r * LX, part * VEC, k4);
      put_perm(sQ + r * LX, part * VEC, q4);
      if (part == 0) {
        sR[R_IK * C + r] = ik;
        sR[R_IQ * C + r] = iq;
        sR[R_CF * C + r] = PERCH ? ik : ik * eta;
        sR[R_ETA * C + r] = eta;
      }
    }
  }
  if (pw == S::NPW - 1) {   // clamp in log space, chunk-local inclusive scan
    const bool ok = lane < C && c0 + lane < T;
    const float graw = a.g[(size_t)(b * T + min(c0 + lane, T - 1)) * H + h];
    const float g2 = ok ? fmaxf(graw, a.log_eps_gamma) : 0.f;
    const float L = wave_inclusive_scan(g2);
    if (lane < C) {
      sR[R_LC * C + lane] = L;
      sR[R_LM * C + lane] = L - g2;
    }
  }
  __syncthreads();
  // e^{L_i - L_j} = e^{L_i - L_ref} e^{L_ref - L_j}: each factor stays within
  // e^{+-80} while the chunk's total log-decay is >= -160, so both are normal
  // fp32 numbers and the product keeps fp32 relative accuracy; deeper decays
  // (a long run of floored steps) keep the per-element exponential.
  const float Llast = sR[R_LC * C + C - 1];
  const bool sep = Llast >= -160.f;
  if (sep && pw == 0 && lane < C) {
    const float Lref = 0.5f * Llast;
    sR[R_EP * C + lane] = __expf(sR[R_LC * C + lane] - Lref) * sR[R_IQ * C + lane];
    sR[R_EA * C + lane] = __expf(sR[R_LM * C + lane] - Lref) * sR[R_IK * C + lane];
    sR[R_EC * C + lane] = __expf(Lref - sR[R_LC * C + lane]) * sR[R_CF * C + lane];
  }
  __syncthreads();

  const OpT *X = sX, *Q = sQ;
  const float *G = sR;
  auto rows16 = [&](const OpT *M, int blk, Pr (&out)[NA / 2]) {
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) out[a2] = ldp(M + (16 * blk + cl) * LX + 32 * a2 + 8 * g4);
  };
  auto tile = [&](const Pr (&Am)[NA / 2], const Pr (&Bm)[NA / 2]) {
    f4 acc = zero4();
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) mmap(acc, Am[a2], Bm[a2]);
    return acc;
  };
  // Gram (isP = 0) or score (isP = 1) block (p, q), transposed: lane (g, c) holds
  // element (row 16p + c, col 16q + 4g + i), the consumers' A-operand fragment.
  auto finish = [&](const f4 &acc, int isP, int p, int q) {
    const int row = 16 * p + cl;
    f4 val;
    if (sep) {
      const f4 ec = *reinterpret_cast<const f4 *>(G + R_EC * C + 16 * q + 4 * g4);
      const float er = G[(isP ? R_EP : R_EA) * C + row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * er * ec[i];
        val[i] = (p > q || 4 * g4 + i <= cl) ? v : 0.f;
      }
    } else {
      const f4 cf = *reinterpret_cast<const f4 *>(G + R_CF * C + 16 * q + 4 * g4);
      const f4 Lc4 = *reinterpret_cast<const f4 *>(G + R_LC * C + 16 * q + 4 * g4);
      const float Lrow = G[(isP ? R_LC : R_LM) * C + row];
      const float rf = G[(isP ? R_IQ : R_IK) * C + row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * __expf(Lrow - Lc4[i]) * rf * cf[i];
        val[i] = (p > q || 4 * g4 + i <= cl) ? v : 0.f;
      }
    }
    if (S::TFULL && !isP) {   // F1 keeps A in fp32 for the inverse
#pragma unroll
      for (int i = 0; i < 4; ++i) sA64[(16 * p + cl) * LDT + 16 * q + 4 * g4 + i] = val[i];
      return;
    }
    OpT *dst = isP ? gP + frag_off(pslot_base(p), q, lane) : gA + frag_off(aslot_base(p), q, lane);
    *reinterpret_cast<Frag *>(dst) = cvt<OpT>(val);
  };
  // diagonal block p: F1 -> T_pp (A-layout); F2 -> the 4x4 diagonal coefficients and A_pp without them
  auto diag = [&](const f4 &acc, int p) {   // acc: <x_{16p+4g+i}, x_{16p+c}> (symmetric)
    const int r0 = 4 * g4;
    f4 NA4, NC4;   // N[16p+c][16p+4g+i] (A-layout) and N[16p+4g+i][16p+c] (C-layout)
    if (sep) {
      const f4 ea4 = *reinterpret_cast<const f4 *>(G + R_EA * C + 16 * p + r0);
      const f4 ec4 = *reinterpret_cast<const f4 *>(G + R_EC * C + 16 * p + r0);
      const float ea1 = G[R_EA * C + 16 * p + cl], ec1 = G[R_EC * C + 16 * p + cl];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        NA4[i] = (r0 + i < cl) ? acc[i] * ea1 * ec4[i] : 0.f;
        NC4[i] = (cl < r0 + i) ? acc[i] * ea4[i] * ec1 : 0.f;
      }
    } else {
      const f4 cf4 = *reinterpret_cast<const f4 *>(G + R_CF * C + 16 * p + r0);
      const f4 ik4 = *reinterpret_cast<const f4 *>(G + R_IK * C + 16 * p + r0);
      const f4 Lc4 = *reinterpret_cast<const f4 *>(G + R_LC * C + 16 * p + r0);
      const f4 Lm4 = *reinterpret_cast<const f4 *>(G + R_LM * C + 16 * p + r0);
      const float Lc1 = G[R_LC * C + 16 * p + cl], Lm1 = G[R_LM * C + 16 * p + cl];
      const float ik1 = G[R_IK * C + 16 * p + cl], cf1 = G[R_CF * C + 16 * p + cl];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float va = acc[i] * __expf(Lm1 - Lc4[i]) * ik1 * cf4[i];
        const float vc = acc[i] * __expf(Lm4[i] - Lc1) * ik4[i] * cf1;
        NA4[i] = (r0 + i < cl) ? va : 0.f;
        NC4[i] = (cl < r0 + i) ? vc : 0.f;
      }
    }
    if constexpr (VAR == V_F1) {
      // row-oriented block Jacobi: T (I + N) = I, so T <- (I - T N_o)(I + N_d)^{-1},
      // exact after 3 sweeps; Y holds T in A-layout (row c, columns 4g..4g+3).
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
      if constexpr (S::TFULL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sT64[(16 * p + cl) * LDT + 16 * p + 4 * g4 + i] = Y[i];
      } else {
        *reinterpret_cast<Frag *>(gT + (p * 64 + lane) * 4) = cvt<OpT>(Y);
      }
    } else {
      // lane (g, 4g+b) holds N[4g+a][4g+b] in NC4[a]; slots: 10 20 21 30 31 32
      if ((cl >> 2) == g4) {
        float *ad = gAd + (p * 4 + g4) * 8;
        const int bb = cl - r0;
        if (bb == 0) { ad[0] = NC4[1]; ad[1] = NC4[2]; ad[3] = NC4[3]; }
        if (bb == 1) { ad[2] = NC4[2]; ad[4] = NC4[3]; }
        if (bb == 2) ad[5] = NC4[3];
      }
      f4 NoA;
#pragma unroll
      for (int i = 0; i < 4; ++i) NoA[i] = ((cl >> 2) == g4) ? 0.f : NA4[i];
      *reinterpret_cast<Frag *>(gT + (p * 64 + lane) * 4) = cvt<OpT>(NoA);
    }
  };
  auto rowfac = [&]() {
    if (lane < C) {
      const float L = G[R_LC * C + lane], Lm = G[R_LM * C + lane];
      const float Llast = G[R_LC * C + C - 1];
      gF[F_GAM * C + lane] = __expf(Lm) * G[R_IK * C + lane];
      gF[F_EL * C + lane] = __expf(L) * G[R_IQ * C + lane];
      gF[F_CST * C + lane] = __expf(Llast - L) * G[R_CF * C + lane];
      gF[F_ETA * C + lane] = G[R_ETA * C + lane];
      if (lane == 0) gF[F_N * C] = __expf(Llast);
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
    if constexpr (w == S::NPW - 1) rowfac();
  };
  if (pw == 0) run(std::integral_constant<int, 0>());
  else if (pw == 1) run(std::integral_constant<int, 1>());
  else if (pw == 2) run(std::integral_constant<int, 2>());
  else run(std::integral_constant<int, 3>());

  if constexpr (S::TFULL) {
    // Off-diagonal blocks of T = (I + A)^{-1} by block forward substitution,
    // T_pq = -T_pp sum_{k=q}^{p-1} A_pk T_kq, one dependency level (p - q) at a
    // time, fp32 MFMA.  Level l has NB - l blocks; wave j takes block (q + l, q = j).
    for (int l = 1; l < NB; ++l) {
      __syncthreads();
      const int q = pw, p = q + l;
      if (p < NB) {
        f4 X = zero4();
        for (int k = q; k < p; ++k) {
          const f4 Apk = *reinterpret_cast<const f4 *>(&sA64[(16 * p + cl) * LDT + 16 * k + 4 * g4]);
          f4 Tkq;   // C-layout: T[16k+4g+i][16q+c]
#pragma unroll
          for (int i = 0; i < 4; ++i) Tkq[i] = sT64[(16 * k + 4 * g4 + i) * LDT + 16 * q + cl];
          mma16(X, Apk, Tkq);
        }
        const f4 Tpp = *reinterpret_cast<const f4 *>(&sT64[(16 * p + cl) * LDT + 16 * p + 4 * g4]);
        f4 Tpq = zero4();
        mma16(Tpq, Tpp, X);   // C-layout: rows 16p+4g+i, column 16q+c
#pragma unroll
        for (int i = 0; i < 4; ++i) sT64[(16 * p + 4 * g4 + i) * LDT + 16 * q + cl] = -Tpq[i];
      }
    }
    __syncthreads();
    // all blocks T_pq, q <= p, as A-layout fragments in the input dtype
    for (int j = pw; j < S::NB * (S::NB + 1) / 2; j += S::NPW) {
      int p = 0;
      while ((p + 1) * (p + 2) / 2 <= j) ++p;
      const int q = j - p * (p + 1) / 2;
      const f4 t = *reinterpret_cast<const f4 *>(&sT64[(16 * p + cl) * LDT + 16 * q + 4 * g4]);
      *reinterpret_cast<Frag *>(gT + frag_off(pslot_base(p), q, lane)) = cvt<OpT>(t);
    }
  }
}

// ============================== scan kernel ==============================
template <int VAR, typename IT, int D, int C, int NS>
__global__ __launch_bounds__(64 * (D / 16 / NS + 8)) void chunk_scan(FwdArgs a, const unsigned char *ws) {
  using S = Split<VAR, IT, D, C>;
  using Z = Scan<VAR, IT, D, C, NS>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = S::NB, NA = S::NA, NCW = Z::NCW, LX = S::LX, VEC = S::VEC, TPR = S::TPR, RPC = Z::RPC;
  constexpr int LXV = Z::LXV, TPV = Z::TPV, RPV = Z::RPV;
  constexpr bool PERCH = S::PERCH, DELTA = S::DELTA;

  // Operands with the per-row factors folded in (dk permuted), from x_i = k_{i-1} and q_i:
  __shared__ __attribute__((aligned(16))) OpT sXg[2][C * LX];  // GAM_i x_i   (residuals)
  __shared__ __attribute__((aligned(16))) OpT sXc[2][C * LX];  // CST_i x_i   (state update)
  __shared__ __attribute__((aligned(16))) OpT sQe[2][C * LX];  // EL_i q_i    (outputs)
  __shared__ __attribute__((aligned(16))) IT sV[2][C * LXV];   // raw v_i, this workgroup's channels
  __shared__ __attribute__((aligned(16))) unsigned char sImg[2][S::IMG];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  // workgroup -> (sequence, channel slice).  The NS slices of a sequence get ids
  // that are equal mod 8, i.e. the same XCD, so its L2 serves their shared reads.
  int bh, sp;
  if (NS > 1 && (a.B * a.H) % 8 == 0) {
    const int rest = blockIdx.x >> 3;
    sp = rest % NS;
    bh = (rest / NS) * 8 + (blockIdx.x & 7);
  } else {
    bh = blockIdx.x / NS;
    sp = blockIdx.x % NS;
  }
  const int b = bh / a.H, h = bh % a.H;
  const int T = a.T, H = a.H, NC = a.nchunks;
  const bool consumer = wv < NCW;
  const int ctid = tid - 64 * NCW;         // copy thread index
  const int chW = Z::DS * sp + 16 * wv + cl;   // consumer lane's value channel

  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);
  const unsigned char *wsq = ws + (size_t)bh * NC * S::IMG;

  // ================= copy waves =================
  // Two register sets: chunk c lands in set c & 1, two chunks ahead of its use,
  // so a load has two scan iterations to arrive.
  struct Regs {
    uint4 k[Z::NPK], q[Z::NPK], v[Z::NPV], img[Z::NPI];
    float fg[Z::NPK], fc[Z::NPK], fe[Z::NPK];   // GAM, CST of the row's x; EL of its q
  };
  Regs reg[2];
  auto prefetch = [&](int c, Regs &R) __attribute__((always_inline)) {    // global -> registers, chunk c (rows clamped in bounds)
    const int c0 = c * C;
#pragma unroll
    for (int ps = 0; ps < Z::NPV; ++ps) {
      const int r = min(ps * RPV + ctid / TPV, C - 1), part = ctid % TPV;
      const int tq = min(c0 + r, T - 1);
      R.v[ps] = *reinterpret_cast<const uint4 *>(vp + ((size_t)(b * T + tq) * H + h) * D + Z::DS * sp + part * VEC);
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPK; ++ps) {
      const int r = min(ps * RPC + ctid / TPR, C - 1), part = ctid % TPR;
      const int tk = min(max(c0 + r - 1, 0), T - 1), tq = min(c0 + r, T - 1);
      R.k[ps] = *reinterpret_cast<const uint4 *>(kp + ((size_t)(b * T + tk) * H + h) * D + part * VEC);
      R.q[ps] = *reinterpret_cast<const uint4 *>(qp + ((size_t)(b * T + tq) * H + h) * D + part * VEC);
      const float *Fg = reinterpret_cast<const float *>(wsq + (size_t)c * S::IMG + S::OFF_F);
      R.fg[ps] = Fg[F_GAM * C + r];
      R.fc[ps] = Fg[F_CST * C + r];
      R.fe[ps] = Fg[F_EL * C + r];
    }
    const uint4 *src = reinterpret_cast<const uint4 *>(wsq + (size_t)c * S::IMG);
#pragma unroll
    for (int j = 0; j < Z::NPI; ++j) R.img[j] = src[min(ctid + j * Z::NST, S::NU - 1)];
  };
  auto stage = [&](int c, const Regs &R) __attribute__((always_inline)) { // registers -> LDS slot c & 1
    const int s = c & 1, c0 = c * C;
#pragma unroll
    for (int ps = 0; ps < Z::NPV; ++ps) {
      const int r = ps * RPV + ctid / TPV, part = ctid % TPV;
      if (r < C) *reinterpret_cast<uint4 *>(sV[s] + r * LXV + part * VEC) = keep_or_zero(c0 + r < T, R.v[ps]);
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPK; ++ps) {
      const int r = ps * RPC + ctid / TPR, part = ctid % TPR;
      if (r < C) {
        float xv[VEC], qv[VEC];
        unpack(keep_or_zero(c0 + r - 1 < T, R.k[ps]), IT(), xv);
        if (c0 + r == 0) {   // first row of the sequence: the carried feature (fp32, IK = 1)
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = a.xprev0 ? a.xprev0[(size_t)bh * D + part * VEC + e] : 0.f;
        }
        const bool okq = c0 + r < T;
        unpack(keep_or_zero(okq, R.q[ps]), IT(), qv);
        put_perm(sXg[s] + r * LX, part * VEC, scale_pack<OpT, VEC>(xv, R.fg[ps]));
        put_perm(sXc[s] + r * LX, part * VEC, scale_pack<OpT, VEC>(xv, R.fc[ps]));
        put_perm(sQe[s] + r * LX, part * VEC, scale_pack<OpT, VEC>(qv, R.fe[ps]));
      }
    }
#pragma unroll
    for (int j = 0; j < Z::NPI; ++j) {
      const int u = ctid + j * Z::NST;
      if (u < S::NU) *reinterpret_cast<uint4 *>(sImg[s] + 16 * u) = R.img[j];
    }
  };

  // ================= consumers =================
  f4 sT[NA];                 // S^T of this wave's 16 channels, C-layout per dk block
  float rbeta[NB][4];        // F2/F2A: per-channel gains of the next chunk
  if (consumer) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) : zero4();
  }
  auto prefetch_beta = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c * C + 16 * p + 4 * g4 + i;   // zero past the end: padded rows must not write
        const float braw = a.beta[((size_t)(b * T + min(t, T - 1)) * H + h) * D + chW];
        rbeta[p][i] = t < T ? braw : 0.f;
      }
  };

  auto consume = [&](int c) __attribute__((always_inline)) {
    const int s = c & 1, c0 = c * C;
    const OpT *Xg = sXg[s], *Xc = sXc[s], *Qe = sQe[s];
    const IT *V = sV[s];
    const float *F = reinterpret_cast<const float *>(sImg[s] + S::OFF_F);
    const OpT *Ao = reinterpret_cast<const OpT *>(sImg[s] + S::OFF_A);
    const OpT *Pm = reinterpret_cast<const OpT *>(sImg[s] + S::OFF_P);
    const OpT *Tb = reinterpret_cast<const OpT *>(sImg[s] + S::OFF_T);
    Pr Sp[NA / 2];
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) Sp[a2] = mkp(cvt<OpT>(sT[2 * a2]), cvt<OpT>(sT[2 * a2 + 1]));
    // XS = diag(GAM) X S0^T: C-layout (token rows 16p+4g+i, channel c).
    // QSt = (diag(EL) Q^ S0^T)^T: C-layout with channel rows 16w+4g+i and token
    // column 16p+c (S fragments as the left operand).
    f4 QSt[NB], XS[NB];
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      QSt[p] = zero4();
      XS[p] = zero4();
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2) {
        const Pr qrow = ldp(Qe + (16 * p + cl) * LX + 32 * a2 + 8 * g4);
        if (DELTA) mmap(XS[p], ldp(Xg + (16 * p + cl) * LX + 32 * a2 + 8 * g4), Sp[a2]);
        mmap(QSt[p], Sp[a2], qrow);
      }
    }
    auto vcol = [&](int j4) { return 16 * wv + 4 * j4; };
    Frag Eb[NB];               // E' = E (F1), eta (.) E (F2), V (F1A), eta (.) V (F2A)
    if constexpr (VAR == V_F1 && S::TFULL) {
      // R = V - diag(GAM) X S0^T for every row block, then E = T R block by block
      Frag Rb[NB];
#pragma unroll
      for (int q = 0; q < NB; ++q)
        Rb[q] = cvt<OpT>(to_f4(ldT(V, LXV, 16 * q, vcol, lane)) - XS[q]);
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        f4 E = zero4();
#pragma unroll
        for (int q = 0; q + 1 <= p; q += 2) mmap(E, ldp(Tb + frag_off(pslot_base(p), q, lane)), mkp(Rb[q], Rb[q + 1]));
        if (!(p & 1)) mma16(E, ld4(Tb + frag_off(pslot_base(p), p, lane)), Rb[p]);
        Eb[p] = cvt<OpT>(E);
      }
    }
#pragma unroll
    for (int p = 0; p < NB && !(VAR == V_F1 && S::TFULL); ++p) {
      f4 R = to_f4(ldT(V, LXV, 16 * p, vcol, lane));  // C-layout values of this wave's channels
      if (DELTA) R -= XS[p];
      f4 eta4;
      if (PERCH) {
        const f4 inv = *reinterpret_cast<const f4 *>(F + F_ETA * C + 16 * p + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) eta4[i] = rbeta[p][i] * inv[i];
      }
      if (S::HAS_A) {   // R -= sum_{q<p} A_pq E_q   (E_q = eta (.) E for F2)
        f4 acc = zero4();
#pragma unroll
        for (int q = 0; q + 1 < p; q += 2) mmap(acc, ldp(Ao + frag_off(aslot_base(p), q, lane)), mkp(Eb[q], Eb[q + 1]));
        if (p & 1) mma16(acc, ld4(Ao + frag_off(aslot_base(p), p - 1, lane)), Eb[p - 1]);
        R -= acc;
      }
      if constexpr (VAR == V_F1) {
        f4 E = zero4();
        mma16(E, ld4(Tb + (p * 64 + lane) * 4), cvt<OpT>(R));
        Eb[p] = cvt<OpT>(E);
      } else if constexpr (VAR == V_F2) {
        // rows 4g4..4g4+3 of block p: exact 4x4 solves, coupled by A_pp minus its 4x4 diagonal
        const float *Ad = reinterpret_cast<const float *>(sImg[s] + S::OFF_AD) + (p * 4 + g4) * 8;
        const f4 c0v = *reinterpret_cast<const f4 *>(Ad), c1v = *reinterpret_cast<const f4 *>(Ad + 4);
        const float a10 = c0v[0], a20 = c0v[1], a21 = c0v[2], a30 = c0v[3], a31 = c1v[0], a32 = c1v[1];
        const Frag Ain = ld4(Tb + (p * 64 + lane) * 4);
        f4 E, Fv;
        auto local = [&](const f4 &zz) {
          E[0] = zz[0];
          Fv[0] = eta4[0] * E[0];
          E[1] = zz[1] - a10 * Fv[0];
          Fv[1] = eta4[1] * E[1];
          E[2] = zz[2] - a20 * Fv[0] - a21 * Fv[1];
          Fv[2] = eta4[2] * E[2];
          E[3] = zz[3] - a30 * Fv[0] - a31 * Fv[1] - a32 * Fv[2];
          Fv[3] = eta4[3] * E[3];
        };
        local(R);
#pragma unroll
        for (int it = 0; it < 3; ++it) {
          f4 cpl = zero4();
          mma16(cpl, Ain, cvt<OpT>(Fv));
          local(R - cpl);
        }
        Eb[p] = cvt<OpT>(Fv);      // eta (.) E feeds the state update and the outputs
      } else if constexpr (VAR == V_F1A) {
        Eb[p] = cvt<OpT>(R);
      } else {
        Eb[p] = cvt<OpT>(eta4 * R);
      }
    }
    // outputs, transposed: o^T = e^{L} (S0 Q^^T) + E'^T P^T.  The C-layout fragments of
    // E' are the left operands and the stored score fragments the right ones; lane
    // (g, c) ends with channels 16w+4g..16w+4g+3 of token 16p+c and stores them.
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 O = QSt[p];
#pragma unroll
      for (int q = 0; q + 1 <= p; q += 2) mmap(O, mkp(Eb[q], Eb[q + 1]), ldp(Pm + frag_off(pslot_base(p), q, lane)));
      if (!(p & 1)) mma16(O, Eb[p], ld4(Pm + frag_off(pslot_base(p), p, lane)));
      const int t = c0 + 16 * p + cl;
      if (t < T) *reinterpret_cast<Frag *>(op + ((size_t)(b * T + t) * H + h) * D + Z::DS * sp + 16 * wv + 4 * g4) = cvt<OpT>(O);
    }
    // state: S^T <- e^{L_last} S^T + (diag(CST) X)^T E'
    const Frag *CE = Eb;
    const float lamtot = F[F_N * C];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) {
      auto dkcol = [&](int j4) { return kperm(16 * aa + 4 * j4); };
      f4 acc = sT[aa] * lamtot;
      if constexpr (NB == 1) {
        mma16(acc, ldT(Xc, LX, 0, dkcol, lane), CE[0]);
      } else {
#pragma unroll
        for (int p = 0; p < NB; p += 2)
          mmap(acc, mkp(ldT(Xc, LX, 16 * p, dkcol, lane), ldT(Xc, LX, 16 * p + 16, dkcol, lane)), mkp(CE[p], CE[p + 1]));
      }
      sT[aa] = acc;
    }
    if (a.chunk_states) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * NC + c) * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  };

  // ---------------- scan: iteration i consumes chunk i and stages chunk i+1 ----------------
  // Each role runs its own loop, so neither keeps the other's loop-carried
  // registers live; both pass the same number of workgroup barriers (one per
  // chunk after a prologue barrier), which is what the barrier counts.
  if (consumer) {
    if (PERCH) prefetch_beta(0);
    __syncthreads();
    for (int i = 0; i < NC; ++i) {
      consume(i);
      if (PERCH && i + 1 < NC) prefetch_beta(i + 1);
      __syncthreads();
    }
    if (a.S_out) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.S_out + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  } else {
    prefetch(0, reg[0]);
    if (NC > 1) prefetch(1, reg[1]);
    stage(0, reg[0]);
    if (NC > 2) prefetch(2, reg[0]);
    __syncthreads();
    // the register sets are indexed with compile-time parity: two iterations per trip;
    // Rnext holds chunk i+1 and is refilled with chunk i+3
    auto copy_step = [&](int i, Regs &Rnext) __attribute__((always_inline)) {
      if (i + 1 < NC) {
        stage(i + 1, Rnext);
        if (i + 3 < NC) prefetch(i + 3, Rnext);
      }
    };
    for (int i = 0; i < NC; i += 2) {
      copy_step(i, reg[1]);
      __syncthreads();
      if (i + 1 < NC) {
        copy_step(i + 1, reg[0]);
        __syncthreads();
      }
    }
    if (a.write_tail && a.xprev_out && wv == NCW && sp == 0) {
      float xv[2] = {0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = lane + 64 * j;
        if (e < D) xv[j] = to_f(kp[((size_t)(b * T + T - 1) * H + h) * D + e]);
      }
      const float ss = group_sum<64>(xv[0] * xv[0] + xv[1] * xv[1]);
      const float inv = safe_rsqrt(ss + a.eps_phi);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = lane + 64 * j;
        if (e < D) a.xprev_out[(size_t)bh * D + e] = xv[j] * inv;
      }
    }
  }
}

// Channel splits built per shape: fp32 keeps whole sequences; bf16 takes 1 or
// 2 slices at d <= 64 and 2, 4 or 8 at d = 128 (whose values do not fit whole).
template <typename IT, int D>
constexpr bool ns_built(int ns) {
  if (sizeof(IT) == 4) return ns == 1;
  return D <= 64 ? (ns == 1 || ns == 2) : (ns == 2 || ns == 4 || ns == 8);
}
template <int VAR, typename IT, int D, int C, int NS>
constexpr bool scan_ok() { return ns_built<IT, D>(NS) && Scan<VAR, IT, D, C, NS>::fits(); }

// Smallest built split that fits and gives at least 128 scan workgroups (else
// the largest that fits); 0 when none fits.
template <int VAR, typename IT, int D, int C>
int pick_ns(int bh) {
  const bool ok[4] = {scan_ok<VAR, IT, D, C, 1>(), scan_ok<VAR, IT, D, C, 2>(), scan_ok<VAR, IT, D, C, 4>(),
                      scan_ok<VAR, IT, D, C, 8>()};
  int best = 0;
  for (int i = 0; i < 4; ++i) {
    if (!ok[i]) continue;
    best = 1 << i;
    if (bh * best >= 128) break;
  }
  return best;
}

template <int VAR, typename IT, int D, int C, int NS>
hipError_t launch_scan(const FwdArgs &a, const unsigned char *w, hipStream_t st) {
  if constexpr (scan_ok<VAR, IT, D, C, NS>()) {
    hipLaunchKernelGGL((chunk_scan<VAR, IT, D, C, NS>), dim3(a.B * a.H * NS), dim3(Scan<VAR, IT, D, C, NS>::NT), 0,
                       st, a, w);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

template <int VAR, typename IT, int D, int C>
hipError_t launch_split(const FwdArgs &a, void *ws, hipStream_t st) {
  const int ns = pick_ns<VAR, IT, D, C>(a.B * a.H);
  if (ns == 0) return hipErrorInvalidValue;
  unsigned char *w = static_cast<unsigned char *>(ws);
  hipLaunchKernelGGL((chunk_prep<VAR, IT, D, C>), dim3(a.B * a.H * a.nchunks), dim3(256), 0, st, a, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (ns) {
    case 1: return launch_scan<VAR, IT, D, C, 1>(a, w, st);
    case 2: return launch_scan<VAR, IT, D, C, 2>(a, w, st);
    case 4: return launch_scan<VAR, IT, D, C, 4>(a, w, st);
    case 8: return launch_scan<VAR, IT, D, C, 8>(a, w, st);
  }
  return hipErrorInvalidValue;
}

// Compile-time dispatch over (variant, dtype, d, chunk): `fn` receives the
// variant, a null pointer of the input type, d and the chunk as compile-time
// values.  Unlisted combinations return a value-initialised result, so callers
// check support before launching.
template <typename Fn>
auto dispatch_split(int variant, bool bf16, int d, int chunk, Fn &&fn) -> decltype(fn(std::integral_constant<int, V_F1>(), (float *)nullptr, std::integral_constant<int, 32>(), std::integral_constant<int, 16>())) {
  using R = decltype(fn(std::integral_constant<int, V_F1>(), (float *)nullptr, std::integral_constant<int, 32>(), std::integral_constant<int, 16>()));
  auto by_chunk = [&](auto v, auto *t, auto dd) -> R {
    switch (chunk) {
      case 16: return fn(v, t, dd, std::integral_constant<int, 16>());
      case 32: return fn(v, t, dd, std::integral_constant<int, 32>());
      case 64: return fn(v, t, dd, std::integral_constant<int, 64>());
    }
    return R();
  };
  auto by_d = [&](auto v, auto *t) -> R {
    if (d == 32) return by_chunk(v, t, std::integral_constant<int, 32>());
    if (d == 64) return by_chunk(v, t, std::integral_constant<int, 64>());
    if constexpr (sizeof(*t) == 2) {
      if (d == 128) return by_chunk(v, t, std::integral_constant<int, 128>());
    }
    return R();
  };
  auto by_type = [&](auto v) -> R {
    if (bf16) return by_d(v, (__bf16 *)nullptr);
    return by_d(v, (float *)nullptr);
  };
  switch (variant) {
    case V_F1: return by_type(std::integral_constant<int, V_F1>());
    case V_F1A: return by_type(std::integral_constant<int, V_F1A>());
    case V_F2: return by_type(std::integral_constant<int, V_F2>());
    case V_F2A: return by_type(std::integral_constant<int, V_F2A>());
  }
  return R();
}

}  // namespace

bool chunk_fwd_split_supported(int variant, bool bf16, int dk, int dv, int chunk) {
  if (dk != dv) return false;
  return dispatch_split(variant, bf16, dk, chunk, [](auto v, auto *t, auto dd, auto cc) -> bool {
    using IT = std::remove_pointer_t<decltype(t)>;
    return pick_ns<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value>(1) > 0;
  });
}

size_t chunk_fwd_split_workspace(int variant, bool bf16, int dk, int dv, int chunk, int bhc) {
  if (!chunk_fwd_split_supported(variant, bf16, dk, dv, chunk)) return 0;
  return dispatch_split(variant, bf16, dk, chunk, [bhc](auto v, auto *t, auto dd, auto cc) -> size_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return Split<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value>::workspace(bhc);
  });
}

hipError_t launch_chunk_fwd_split(int variant, bool bf16, int dk, int dv, int chunk, const FwdArgs &a, void *ws,
                                  hipStream_t st) {
  if (!chunk_fwd_split_supported(variant, bf16, dk, dv, chunk)) return hipErrorInvalidValue;
  const hipError_t r = dispatch_split(variant, bf16, dk, chunk, [&](auto v, auto *t, auto dd, auto cc) -> hipError_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return launch_split<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value>(a, ws, st);
  });
  return r;
}

}  // namespace falcon
