// Chunk-parallel ("split") forward pass of Falcon-1 / 1A / 2 / 2A / 3 / 3A on
// gfx950: the two kernels and their launch templates.  falcon_fwd_split.hip
// instantiates them with one pair per step, falcon_fwd_split_win.hip with the
// Falcon-3 windows.
//
// The chunked form ([P1] 三种等价形式 form C and Figure 4-C; [P2] 三种视角)
// separates what depends on the carried state from what does not:
//   * everything built from keys, queries and gates of one system of rows -- the
//     decayed Gram blocks A_pq, the score blocks P_pq, the diagonal-block
//     inverses T_pp (F1 / F3) or the Falcon-2 diagonal blocks, and the per-row
//     decay / norm / step factors -- is independent across systems;
//   * the residuals, outputs and the state update of a system need S at its start.
// The prep kernel runs one workgroup per system over the whole device and writes
// the first group, per system, as an "image": the exact LDS layout the scan
// reads.  The scan kernel runs one to eight workgroups per sequence (slices of
// the value channels): copy waves stream the key / query rows, the slice's
// values and the image into double-buffered LDS one system ahead, and one
// consumer wave per 16 value channels carries S^T in registers.
//
// Windows (Falcon-3 / 3A, [P1] Falcon家族, [P2] 六个变体): step s writes the Bw
// pairs j = s-Bw+1..s, each weighted w_s = eta_s / Bw and each with a residual
// against S_{s-1}.  A system then has C "virtual rows" r = (s, j), s = r / Bw,
// j = s - Bw + 1 + r % Bw, covering CS = C / Bw steps: Gram blocks run over
// virtual rows with the mask s(r') < s(r), score blocks over (step, virtual
// row) with s(r') <= s, and the state update over virtual rows.  Bw = 1 is the
// one-pair case (CS = C, r = s = j).  The public chunk (chunk_states cadence) is
// C steps, i.e. Bw systems.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// Image of one system (bytes, tiles in the input dtype, fragment pairs of 64
// lanes x 8 elements; slots hold only the tiles that exist):
//   A   : A_pq, q < p (F1 / F2 / F3)  -- pair slot aslot_base(p) + q/2, half q&1;
//         in the prep kernel's F1 / F3 images the blocks T_pq of T = (I + A)^{-1}
//         instead, with T_pp also in the free upper half of odd p's last slot
//   P   : P_pq (step block p, virtual-row block q <= qmax(p))
//                                      -- pair slot pbase(p) + q/2, half q&1
//   T   : F1 / F3: T_pp = (I + A_pp)^{-1} (the diagonal blocks of T); F2: A_pp without its 4x4 diagonal
//         sub-blocks; one fragment per diagonal block
//   AD  : F2 only, the 6 coefficients of each 4x4 diagonal sub-block (8 floats)
//   F   : per-row GAM, EL, CST, ETA (fp32, C each) and e^{L_last}
// After the images, one "carry" block per sequence holds the incoming x_prev
// (and window): the scan reads that copy, never the caller's incoming state,
// which the outgoing state may alias.
#pragma once
#include "chunk_common.h"
#include "falcon_kernels.h"

namespace falcon {

namespace {

// per-row arrays of the prep kernel (index: virtual row r, or step row s)
enum {
  R_LC = 0,  // L_{s(r)}            inclusive log-decay of the row's step
  R_LM,      // L_{s(r)-1}
  R_IK,      // 1/|k| of the row's key (1 for carried features)
  R_IQ,      // 1/|q_s|             step rows
  R_CF,      // IK_r w_{s(r)} (F1/F3), IK_r (F2/F2A), IK_r (F1A/F3A: w folded too)
  R_ETA,     // w_{s(r)}, or 1/(eps + |x_r|^2) for F2/F2A
  // separable decay factors around L_ref = L_last / 2 (used while L_last >= -160):
  R_EP,      // e^{L_s - L_ref} IQ_s      step rows of score blocks
  R_EA,      // e^{L_{s(r)-1} - L_ref} IK_r   rows of Gram blocks
  R_EC,      // e^{L_ref - L_{s(r)}} CF_r     columns of both
  // windows only:
  R_LQ,      // L_s                       step rows
  R_GQ,      // clamped log-decay of step s
  R_E2,      // |x_r|^2 of the normalised key
  R_BQ,      // beta_s
  R_N
};
// per-row factors in the image (consumers)
enum {
  F_GAM = 0,  // e^{L_{s(r)-1}} * IK_r        virtual rows
  F_EL,       // e^{L_s} * IQ_s               step rows
  F_CST,      // e^{L_last - L_{s(r)}} * CF_r virtual rows
  F_ETA,      // 1/(eps + |x_r|^2)  (Falcon-2 / 2A)
  F_N
};

constexpr int aslot_base(int p) {
  int b = 0;
  for (int i = 1; i < p; ++i) b += (i - 1) / 2 + 1;
  return b;
}

template <int VAR, typename IT, int D, int C, int BW>
struct Split {
  static_assert(16 % BW == 0 && C % 16 == 0, "steps must not straddle 16-row blocks");
  static constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  static constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2 || VAR == V_F3);
  static constexpr bool SDELTA = (VAR == V_F1 || VAR == V_F3);   // scalar step: T_pp per block
  static constexpr int NB = C / 16, NA = D / 16;
  static constexpr int CS = C / BW;                          // steps per system
  static constexpr int NBS = (CS + 15) / 16, CSP = 16 * NBS; // step rows, whole tiles
  static constexpr int RLQ = BW == 1 ? R_LC : R_LQ;          // L of a step row
  static constexpr int qmax(int ps) { return score_qmax(ps, NB, CS, BW); }
  static constexpr int pbase(int ps) { return score_base(ps, NB, CS, BW); }
  static constexpr int FRAG = 64 * 8;                        // elements of one fragment pair
  static constexpr int SZ = (int)sizeof(IT);
  static constexpr int NSP = pbase(NBS), NSA = DELTA ? aslot_base(NB) : 0;
  static constexpr int OFF_A = 0;
  static constexpr int OFF_P = OFF_A + NSA * FRAG * SZ;
  static constexpr int OFF_T = OFF_P + NSP * FRAG * SZ;
  static constexpr int OFF_AD = OFF_T + (DELTA ? NB * 256 * SZ : 0);
  static constexpr int OFF_F = OFF_AD + (VAR == V_F2 ? NB * 32 * 4 : 0);
  static constexpr int IMG = ((OFF_F + (F_N * C + 4) * 4) + 15) / 16 * 16;
  static constexpr int NU = IMG / 16;                        // 16-byte units of the image
  // carry block: x_prev [D], window keys [BW-1][D], window values [BW-1][D] (fp32)
  static constexpr int CARRY = ((2 * BW - 1) * D * 4 + 15) / 16 * 16;
  // shared
  static constexpr int PADE = 16 / SZ, VEC = PADE;
  static constexpr int LX = D + PADE;                        // X, Q rows (dk permuted), V rows
  static constexpr int TPR = D / VEC;                        // threads per input row
  // prep kernel: 4 waves, one system
  static constexpr int NPW = 4, NPT = 256;
  static constexpr int RPP = NPT / TPR, NPASS = (C + RPP - 1) / RPP;
  // the prep kernel of F1 / F3 also keeps the Gram blocks and T_pp in LDS to
  // complete the inverse of the system matrix (complete_inverse), over the rows
  static constexpr int LAT = SDELTA ? NSA * FRAG + NB * 256 : 1;
  static constexpr int PXQ = (C + CSP) * LX > LAT ? (C + CSP) * LX : LAT;   // rows X, Q (then the tiles)
  static constexpr size_t prep_lds() { return (size_t)SZ * PXQ + 4 * R_N * C; }
  __host__ __device__ static int nsys(int T) { return (T + CS - 1) / CS; }
  static size_t workspace(int bh, int T) { return (size_t)bh * nsys(T) * IMG + (size_t)bh * CARRY; }
  // Packed sequences (cu_seqlens): per head, sequence n's systems take image slots
  // from cu[n] / CS + n on, which leaves room for its nsys(cu[n+1] - cu[n]) systems
  // (floor(cu/CS) + ceil(T/CS) <= floor((cu + T)/CS) + 1), so the offsets follow from
  // cu alone; `slots` per head bounds them all.
  __host__ __device__ static int slot0(const int *cu, int n) { return cu[n] / CS + n; }
  __host__ __device__ static int slots(int N, int total) { return total / CS + N + 1; }
  static size_t workspace_varlen(int N, int H, int total) {
    return (size_t)H * slots(N, total) * IMG + (size_t)N * H * CARRY;
  }
};

// The scan of one sequence is split over NS workgroups by value channel (rows
// of S evolve independently given the keys).  A workgroup takes D/NS channels:
// per 16 of them one state wave (the chain S -> residuals -> S, system by system)
// and one output wave (the outputs of the previous system, from the S and E'
// fragments the state wave leaves in LDS), plus copy waves that stage the shared
// key / query rows and the slice's value columns.  Two-kernel form (ONE =
// false): 8 copy waves also stage the system image the prep kernel wrote.
// One-pass form (ONE = true): 4 derive waves build each image in LDS one system
// ahead (the prep kernel's tiles, from the staged rows), and 4 or 8 copy waves
// stage rows, their squared norms and the gates.
// Map form (MAPS = true, two-kernel only): the state at the end of each
// sequence and nothing else, for the segment-map passes of the two-level scan:
// no output waves, no query rows and no fragments handed to output waves, so
// wider channel slices fit.
template <int VAR, typename IT, int D, int C, int BW, int NS, bool ONE = false, bool MAPS = false>
struct Scan {
  static_assert(!(ONE && MAPS), "the map form is a two-kernel scan");
  using S = Split<VAR, IT, D, C, BW>;
  static constexpr int DS = D / NS;                          // value channels per workgroup
  // one-pass derive waves (8 measured slower than 4: every role shares the CU's SIMDs)
  static constexpr int NDW = ONE ? S::NPW : 0;
  // copy waves: 8 (two-kernel form: rows and images); one-pass form: 8 when the
  // workgroup has two state waves (1024 threads; the copy waves set the F1A period,
  // and F1 and F2A measured faster too), except Falcon-2, whose state waves need
  // more registers than 16 waves leave (156 VGPRs), else 4
  static constexpr int NCW = DS / 16, NSW = ONE ? (VAR != V_F2 && NCW == 2 ? 8 : 4) : 8;
  static constexpr int NOW = MAPS ? 0 : NCW;                 // output waves
  static constexpr int RG = BW == 1 ? R_EC + 1 : R_N;        // per-row arrays a derive wave uses
  static constexpr int NT = 64 * (NCW + NOW + NDW + NSW), NST = 64 * NSW;
  static constexpr int LXV = DS + S::PADE;                   // V rows (this workgroup's channels)
  static constexpr int RPC = NST / S::TPR, NPK = (C + RPC - 1) / RPC;   // key / query rows per copy pass
  static constexpr int TPV = DS / S::VEC, RPV = NST / TPV, NPV = (C + RPV - 1) / RPV;
  static constexpr int NPI = ONE ? 1 : (S::NU + NST - 1) / NST;
  // LDS slots: keys and values 2 (3 one-pass: derive waves read one system ahead),
  // queries 3 (4), images 3 (output waves lag one system); S and E' fragments 2
  static constexpr int NXS = ONE ? 3 : 2, NQS = MAPS ? 0 : ONE ? 4 : 3;
  static constexpr size_t lds() {
    return (size_t)S::SZ * (NXS * C * S::LX + NQS * S::CSP * S::LX + NXS * C * LXV) + 3 * (size_t)S::IMG +
           2 * (size_t)NOW * 64 * S::SZ * (8 * (S::NA / 2) + 4 * S::NB) +
           (ONE ? (size_t)4 * (3 * 4 * C + NDW * RG * C) : 0);
  }
  static constexpr bool fits() {
    return DS >= 16 && D % NS == 0 && C <= 64 && NT <= 1024 && lds() + 256 <= 160 * 1024 &&
           (ONE || S::prep_lds() + 256 <= 64 * 1024);
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

// VEC fp32 values of a carried feature, converted to the operand type
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

// sum of squares of one 16-byte vector of raw inputs (bf16: paired dot products)
__device__ __forceinline__ float sumsq(const uint4 &u, __bf16) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.x), __builtin_bit_cast(bf2, u.x), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.y), __builtin_bit_cast(bf2, u.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.z), __builtin_bit_cast(bf2, u.z), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, u.w), __builtin_bit_cast(bf2, u.w), s, false);
  return s;
}
__device__ __forceinline__ float sumsq(const uint4 &u, float) {
  const float a = __uint_as_float(u.x), b = __uint_as_float(u.y), c = __uint_as_float(u.z), d = __uint_as_float(u.w);
  return a * a + b * b + c * c + d * d;
}

// VEC raw values scaled by f, in the operand type (one 16-byte vector)
template <typename OpT, int VEC>
__device__ __forceinline__ uint4 scale_pack(const float *x, float f) {
  OpT tmp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) tmp[e] = (OpT)(x[e] * f);
  return *reinterpret_cast<const uint4 *>(tmp);
}

// Key-side tiles of one system from its raw rows X (virtual rows) and Q (step
// rows), dk permuted, and its per-row arrays G (R_* layout, C entries each):
// wave w of 4 computes its share of the Gram and score blocks and of the
// diagonal blocks, finishes them with the decay / norm / step factors and
// writes them, with the per-row factors (wave 3), into the image at img (global
// memory for the prep kernel, LDS for the one-pass kernel).
// The products need only the rows, so they are issued first; `rows()` then
// fills G (the one-pass kernel computes it there, while the products run) and
// returns the system's total log-decay L_last.  The finishing code is built
// twice, for separable (L_last >= -160) and per-element decay factors, so each
// version is one straight-line block in which the diagonal solve and the
// other tiles' finishing interleave.
template <int VAR, typename IT, int D, int C, int BW, bool LA = false, typename RowsFn>
__device__ __forceinline__ void derive_image(const IT *X, const IT *Q, const float *G, unsigned char *img, int w,
                                             int lane, RowsFn &&rows, IT *lat = nullptr) {
  using S = Split<VAR, IT, D, C, BW>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = S::NB, NA = S::NA, LX = S::LX, CS = S::CS, CSP = S::CSP, RLQ = S::RLQ;
  constexpr bool DELTA = S::DELTA;
  const int g4 = lane >> 4, cl = lane & 15;
  // LA: the Gram blocks and the diagonal-block inverses go to `lat` (LDS, the A
  // slots followed by the T fragments) for complete_inverse instead of the image;
  // it is written only after a workgroup barrier that follows the tile products
  // (all NPW waves call this once), so it may overlay the rows X and Q
  OpT *gA = LA ? lat : reinterpret_cast<OpT *>(img + S::OFF_A);
  OpT *gP = reinterpret_cast<OpT *>(img + S::OFF_P);
  OpT *gT = LA ? lat + S::NSA * S::FRAG : reinterpret_cast<OpT *>(img + S::OFF_T);
  float *gAd = reinterpret_cast<float *>(img + S::OFF_AD);
  float *gF = reinterpret_cast<float *>(img + S::OFF_F);
  (void)CS;
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
  // Gram (isP = 0, virtual rows 16p + c) or score (isP = 1, step rows 16p + c)
  // block (p, q), transposed: lane (g, c) holds element (row 16p + c, virtual-row
  // column 16q + 4g + i), the consumers' A-operand fragment.  Off-diagonal Gram
  // blocks are wholly visible (steps do not straddle blocks); score blocks see
  // the columns whose step is at most the row's.
  auto finish = [&](auto sepc, const f4 &acc, int isP, int p, int q) {
    const int row = 16 * p + cl;
    f4 val;
    if constexpr (decltype(sepc)::value) {
      const f4 ec = *reinterpret_cast<const f4 *>(G + R_EC * C + 16 * q + 4 * g4);
      const float er = G[(isP ? R_EP : R_EA) * C + row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * er * ec[i];
        val[i] = (!isP || (16 * q + 4 * g4 + i) / BW <= row) ? v : 0.f;
      }
    } else {
      const f4 cf = *reinterpret_cast<const f4 *>(G + R_CF * C + 16 * q + 4 * g4);
      const f4 Lc4 = *reinterpret_cast<const f4 *>(G + R_LC * C + 16 * q + 4 * g4);
      const float Lrow = G[(isP ? RLQ : R_LM) * C + row];
      const float rf = G[(isP ? R_IQ : R_IK) * C + row];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = acc[i] * __expf(Lrow - Lc4[i]) * rf * cf[i];
        val[i] = (!isP || (16 * q + 4 * g4 + i) / BW <= row) ? v : 0.f;
      }
    }
    OpT *dst = isP ? gP + frag_off(S::pbase(p), q, lane) : gA + frag_off(aslot_base(p), q, lane);
    *reinterpret_cast<Frag *>(dst) = cvt<OpT>(val);
  };
  // diagonal block p: F1/F3 -> T_pp (A-layout); F2 -> the 4x4 diagonal coefficients and A_pp without them
  auto diag = [&](auto sepc, const f4 &acc, int p) {   // acc: <x_{16p+4g+i}, x_{16p+c}> (symmetric)
    const int r0 = 4 * g4;
    f4 NA4, NC4;   // N[16p+c][16p+4g+i] (A-layout) and N[16p+4g+i][16p+c] (C-layout), strictly earlier steps
    if constexpr (decltype(sepc)::value) {
      const f4 ea4 = *reinterpret_cast<const f4 *>(G + R_EA * C + 16 * p + r0);
      const f4 ec4 = *reinterpret_cast<const f4 *>(G + R_EC * C + 16 * p + r0);
      const float ea1 = G[R_EA * C + 16 * p + cl], ec1 = G[R_EC * C + 16 * p + cl];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        NA4[i] = ((r0 + i) / BW < cl / BW) ? acc[i] * ea1 * ec4[i] : 0.f;
        NC4[i] = (cl / BW < (r0 + i) / BW) ? acc[i] * ea4[i] * ec1 : 0.f;
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
        NA4[i] = ((r0 + i) / BW < cl / BW) ? va : 0.f;
        NC4[i] = (cl / BW < (r0 + i) / BW) ? vc : 0.f;
      }
    }
    if constexpr (S::SDELTA) {
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
      // the sweeps run in the operand type: T_pp is stored in it, and a bf16
      // sweep is one MFMA instead of four fp32 ones on this serial chain
      const Frag NoCo = cvt<OpT>(NoC);
#pragma unroll
      for (int it = 0; it < 3; ++it) {
        f4 cpl = zero4();
        mma16(cpl, NoCo, cvt<OpT>(Y));   // C-layout of N_o^T Y^T = A-layout of Y N_o
        local(Z - cpl);
      }
      *reinterpret_cast<Frag *>(gT + (p * 64 + lane) * 4) = cvt<OpT>(Y);
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
  auto rowfac = [&](float Llast) {
    if (lane < C) {
      const float L = G[R_LC * C + lane], Lm = G[R_LM * C + lane];
      gF[F_GAM * C + lane] = __expf(Lm) * G[R_IK * C + lane];
      gF[F_EL * C + lane] = lane < CSP ? __expf(G[RLQ * C + lane]) * G[R_IQ * C + lane] : 0.f;
      gF[F_CST * C + lane] = __expf(Llast - L) * G[R_CF * C + lane];
      gF[F_ETA * C + lane] = G[R_ETA * C + lane];
      if (lane == 0) gF[F_N * C] = __expf(Llast);
    }
  };
  auto run = [&](auto wc) {
    constexpr int w = decltype(wc)::value;
    constexpr JobList J = BW == 1 ? make_jobs(NB, DELTA, w) : make_jobs_win(NB, CS, BW, DELTA, w);
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
    const float Llast = rows();
    // LA: `lat` may share LDS with the rows; every wave's products are done
    if constexpr (LA) __syncthreads();
    auto tail = [&](auto sepc) __attribute__((always_inline)) {
      if constexpr (J.diag >= 0) diag(sepc, dacc, J.diag);
#pragma unroll
      for (int j = 0; j < J.n; ++j) finish(sepc, acc[j], J.isP[j], J.p[j], J.q[j]);
      if constexpr (w == S::NPW - 1) rowfac(Llast);
    };
    if (Llast >= -160.f) tail(std::true_type());
    else tail(std::false_type());
  };
  if (w == 0) run(std::integral_constant<int, 0>());
  else if (w == 1) run(std::integral_constant<int, 1>());
  else if (w == 2) run(std::integral_constant<int, 2>());
  else run(std::integral_constant<int, 3>());
}

// Whole inverse of a system's matrix M = I + A (F1 / F3: A holds the decayed,
// step-weighted Gram blocks, so E = M^{-1} R is the WY solve of [P1] 三种等价形式
// form C), from the Gram blocks and the diagonal-block inverses T_pp that
// derive_image left in LDS (`lat`).  Block column q of T = M^{-1} follows by
// forward substitution down the column,
//   T_pq = -T_pp sum_{r=q}^{p-1} A_pr T_rq,   p > q,
// so wave q takes column q on its own, with no exchange between waves.  Each
// block is formed twice from the same operands: in C-layout (the right operand
// of the next block's products) and transposed, whose C-layout is the A-layout
// fragment the scan reads.  The image then holds T_pq in the A slots, and T_pp
// in T and, for odd p, in the free upper half of the slot of A_{p,p-1}, so that
// the scan forms E = T R with every product independent of the others.
template <int VAR, typename IT, int D, int C, int BW>
__device__ __forceinline__ void complete_inverse(const IT *lat, unsigned char *img, int w, int lane) {
  using S = Split<VAR, IT, D, C, BW>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  constexpr int NB = S::NB;
  const int g4 = lane >> 4, cl = lane & 15;
  const OpT *lA = lat, *lT = lat + S::NSA * S::FRAG;
  OpT *gA = reinterpret_cast<OpT *>(img + S::OFF_A);
  OpT *gT = reinterpret_cast<OpT *>(img + S::OFF_T);
  auto column = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const Frag tqq = ld4(lT + (q * 64 + lane) * 4);
    *reinterpret_cast<Frag *>(gT + (q * 64 + lane) * 4) = tqq;
    if constexpr (q & 1) *reinterpret_cast<Frag *>(gA + frag_off(aslot_base(q), q, lane)) = tqq;
    // C-layout of T_qq: element (4g+i, c) sits in lane 16(c/4) + 4g + i, entry c%4, of the A-layout
    f4 Tc[NB];
#pragma unroll
    for (int i = 0; i < 4; ++i) Tc[q][i] = (float)lT[(q * 64 + 16 * (cl >> 2) + 4 * g4 + i) * 4 + (cl & 3)];
#pragma unroll
    for (int p = q + 1; p < NB; ++p) {
      f4 sacc = zero4();   // sum_{r=q}^{p-1} A_pr T_rq, C-layout
#pragma unroll
      for (int r = q; r < p; ++r) mma16(sacc, ld4(lA + frag_off(aslot_base(p), r, lane)), cvt<OpT>(Tc[r]));
      const Frag sb = cvt<OpT>(sacc);
      const Frag tpp = ld4(lT + (p * 64 + lane) * 4);
      f4 tc = zero4(), tt = zero4();
      mma16(tc, tpp, sb);   // T_pp S: C-layout of -T_pq
      mma16(tt, sb, tpp);   // S^T T_pp^T: C-layout of -T_pq^T = A-layout of -T_pq
      Tc[p] = -tc;
      *reinterpret_cast<Frag *>(gA + frag_off(aslot_base(p), q, lane)) = cvt<OpT>(-tt);
    }
  };
  if (w == 0) column(std::integral_constant<int, 0>());
  if constexpr (NB > 1) if (w == 1) column(std::integral_constant<int, 1>());
  if constexpr (NB > 2) if (w == 2) column(std::integral_constant<int, 2>());
  if constexpr (NB > 3) if (w == 3) column(std::integral_constant<int, 3>());
}

// ============================== prep kernel ==============================
template <int VAR, typename IT, int D, int C, int BW>
__global__ __launch_bounds__(256) void chunk_prep(FwdArgs a, unsigned char *ws) {
  using S = Split<VAR, IT, D, C, BW>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = S::NB, NA = S::NA, LX = S::LX, VEC = S::VEC, TPR = S::TPR, RPP = S::RPP;
  constexpr int CS = S::CS, CSP = S::CSP, RLQ = S::RLQ;
  constexpr bool PERCH = S::PERCH, DELTA = S::DELTA;

  __shared__ __attribute__((aligned(16))) OpT sXQ[S::PXQ];
  OpT *const sX = sXQ;              // raw key of each virtual row, dk permuted
  OpT *const sQ = sXQ + C * LX;     // raw q of each step row, dk permuted
  __shared__ __attribute__((aligned(16))) float sR[R_N * C];

  const int tid = threadIdx.x, lane = tid & 63, pw = tid >> 6;
  const int g4 = lane >> 4, cl = lane & 15;
  const int H = a.H;
  // the workgroup's sequence b, head h and system c: one per system of a dense
  // [B, T] batch, or, for packed sequences, one per image slot of a head (slots
  // past the end of their sequence's systems have nothing to do)
  int T, b, h, c;
  long long tok0;
  unsigned char *img, *carry_base;
  if (a.cu) {
    const int SL = S::slots(a.B, a.T);
    h = blockIdx.x / SL;
    const int slot = blockIdx.x % SL;
    int lo = 0, hi = a.B - 1;   // the last sequence whose first slot is <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (S::slot0(a.cu, mid) <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    tok0 = a.cu[b];
    T = a.cu[b + 1] - a.cu[b];
    c = slot - S::slot0(a.cu, b);
    if (c >= S::nsys(T)) return;   // an unused slot (also every slot of an empty sequence)
    img = ws + (size_t)blockIdx.x * S::IMG;
    carry_base = ws + (size_t)H * SL * S::IMG;
  } else {
    T = a.T;
    const int NSYS = S::nsys(T), bhd = blockIdx.x / NSYS;
    c = blockIdx.x % NSYS;
    b = bhd / H;
    h = bhd % H;
    tok0 = (long long)b * T;
    img = ws + (size_t)blockIdx.x * S::IMG;
    carry_base = ws + (size_t)a.B * H * NSYS * S::IMG;
  }
  const int bh = b * H + h, c0 = c * CS;
  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);

  if (c == 0) {   // the sequence's carry block
    float *carry = reinterpret_cast<float *>(carry_base + (size_t)bh * S::CARRY);
    for (int e = tid; e < D; e += S::NPT) carry[e] = a.xprev0 ? a.xprev0[(size_t)bh * D + e] : 0.f;
    for (int e = tid; e < (BW - 1) * D; e += S::NPT) {
      carry[D + e] = a.winx0 ? a.winx0[(size_t)bh * (BW - 1) * D + e] : 0.f;
      carry[BW * D + e] = a.winv0 ? a.winv0[(size_t)bh * (BW - 1) * D + e] : 0.f;
    }
  }

  if constexpr (BW == 1) {
    // X row r holds k_{c0+r-1} (x_prev for the first row of the sequence; k_{c0+r}
    // with same-step pairs), Q row r holds q_{c0+r}
#pragma unroll
    for (int ps = 0; ps < S::NPASS; ++ps) {
      const int r = ps * RPP + tid / TPR, part = tid % TPR;
      if (r < C) {
        const int tk = c0 + r - 1 + a.align, tq = c0 + r;
        // loads use in-bounds (clamped) rows; rows outside the sequence are zeroed after the load
        const int tkc = min(max(tk, 0), T - 1), tqc = min(tq, T - 1);
        const uint4 kraw = *reinterpret_cast<const uint4 *>(kp + ((size_t)(tok0 + tkc) * H + h) * D + part * VEC);
        const uint4 qraw = *reinterpret_cast<const uint4 *>(qp + ((size_t)(tok0 + tqc) * H + h) * D + part * VEC);
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
        const float braw = PERCH ? 0.f : a.beta[(size_t)(tok0 + tqc) * H + h];
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
  } else {
    // virtual row r: step c0 + r/BW, pair j = step - BW + 1 + r%BW with key x_j = phi(k_{j-1})
    // (x_prev for j = 0, the carried window for j < 0); step row s holds q_{c0+s}
#pragma unroll
    for (int ps = 0; ps < S::NPASS; ++ps) {
      const int r = ps * RPP + tid / TPR, part = tid % TPR;
      if (r < C) {
        const int st = c0 + r / BW, j = st - BW + 1 + r % BW, tk = j - 1 + a.align;
        const int tkc = min(max(tk, 0), T - 1);
        const uint4 kraw = *reinterpret_cast<const uint4 *>(kp + ((size_t)(tok0 + tkc) * H + h) * D + part * VEC);
        uint4 k4 = keep_or_zero(tk >= 0 && st < T, kraw);
        float sk = 0.f;
        if (tk < 0 && st < T) {   // carried feature (fp32, already normalised): x_prev (j = 0) or window
          const float *src = j == 0 ? (a.xprev0 ? a.xprev0 + (size_t)bh * D : nullptr)
                                    : (a.winx0 ? a.winx0 + ((size_t)bh * (BW - 1) + j + BW - 1) * D : nullptr);
          float xf[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) xf[e] = src ? src[part * VEC + e] : 0.f;
          k4 = pack_feature<OpT, VEC>(xf, sk);
        } else {
          float xv[VEC];
          unpack(k4, IT(), xv);
#pragma unroll
          for (int e = 0; e < VEC; ++e) sk += xv[e] * xv[e];
        }
        sk = group_sum<TPR>(sk);
        const float ik = tk < 0 ? 1.f : safe_rsqrt(sk + a.eps_phi);
        put_perm(sX + r * LX, part * VEC, k4);
        if (part == 0) {
          sR[R_IK * C + r] = ik;
          sR[R_E2 * C + r] = sk * ik * ik;
        }
      }
      if (r < CSP) {
        const int tq = c0 + r;
        const bool okq = r < CS && tq < T;
        const int tqc = min(tq, T - 1);
        const uint4 qraw = *reinterpret_cast<const uint4 *>(qp + ((size_t)(tok0 + tqc) * H + h) * D + part * VEC);
        const uint4 q4 = keep_or_zero(okq, qraw);
        float qv[VEC], sq = 0.f;
        unpack(q4, IT(), qv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) sq += qv[e] * qv[e];
        sq = group_sum<TPR>(sq);
        put_perm(sQ + r * LX, part * VEC, q4);
        if (part == 0) {
          const float braw = a.beta[(size_t)(tok0 + tqc) * H + h];
          sR[R_IQ * C + r] = okq ? safe_rsqrt(sq + a.eps_phi) : 0.f;
          sR[R_BQ * C + r] = okq ? braw : 0.f;
        }
      }
    }
  }
  if (pw == S::NPW - 1) {   // clamp in log space, inclusive scan over the system's steps
    const bool ok = lane < CS && c0 + lane < T;
    const float graw = a.g[(size_t)(tok0 + min(c0 + lane, T - 1)) * H + h];
    const float g2 = ok ? fmaxf(graw, a.log_eps_gamma) : 0.f;
    const float L = wave_inclusive_scan(g2);
    if (BW == 1) {
      if (lane < C) {
        sR[R_LC * C + lane] = L;
        sR[R_LM * C + lane] = L - g2;
      }
    } else if (lane < CSP) {
      sR[R_LQ * C + lane] = L;
      sR[R_GQ * C + lane] = g2;
    }
  }
  __syncthreads();
  // e^{L_a - L_b} = e^{L_a - L_ref} e^{L_ref - L_b}: each factor stays within
  // e^{+-80} while the system's total log-decay is >= -160, so both are normal
  // fp32 numbers and the product keeps fp32 relative accuracy; deeper decays
  // (a long run of floored steps) keep the per-element exponential.
  const float Llast = sR[RLQ * C + CS - 1];
  const bool sep = Llast >= -160.f;
  const float Lref = 0.5f * Llast;
  if constexpr (BW == 1) {
    if (sep && pw == 0 && lane < C) {
      sR[R_EP * C + lane] = __expf(sR[R_LC * C + lane] - Lref) * sR[R_IQ * C + lane];
      sR[R_EA * C + lane] = __expf(sR[R_LM * C + lane] - Lref) * sR[R_IK * C + lane];
      sR[R_EC * C + lane] = __expf(Lref - sR[R_LC * C + lane]) * sR[R_CF * C + lane];
    }
  } else {
    if (tid < C) {   // virtual-row values from their step (the step's own pair is its newest row)
      const int r = tid, s = r / BW;
      const float Ls = sR[R_LQ * C + s], Lm = Ls - sR[R_GQ * C + s], ik = sR[R_IK * C + r];
      const float w = sR[R_BQ * C + s] * fast_rcp(a.eps_eta + sR[R_E2 * C + s * BW + BW - 1]) * (1.f / BW);
      const float cf = ik * w;
      sR[R_LC * C + r] = Ls;
      sR[R_LM * C + r] = Lm;
      sR[R_CF * C + r] = cf;
      sR[R_ETA * C + r] = w;
      if (sep) {
        sR[R_EA * C + r] = __expf(Lm - Lref) * ik;
        sR[R_EC * C + r] = __expf(Lref - Ls) * cf;
      }
    } else if (sep && tid >= 64 && tid < 64 + CSP) {
      const int s = tid - 64;
      sR[R_EP * C + s] = __expf(sR[R_LQ * C + s] - Lref) * sR[R_IQ * C + s];
    }
  }
  __syncthreads();

  if constexpr (S::SDELTA) {   // Gram blocks and T_pp of the system over the rows, then T
    derive_image<VAR, IT, D, C, BW, true>(sX, sQ, sR, img, pw, lane, [&]() { return Llast; }, sXQ);
    __syncthreads();
    complete_inverse<VAR, IT, D, C, BW>(sXQ, img, pw, lane);
  } else {
    derive_image<VAR, IT, D, C, BW>(sX, sQ, sR, img, pw, lane, [&]() { return Llast; });
  }
}

// ============================== scan kernel ==============================
template <int VAR, typename IT, int D, int C, int BW, int NS, bool ONE, bool MAPS>
__global__ __launch_bounds__((Scan<VAR, IT, D, C, BW, NS, ONE, MAPS>::NT)) void chunk_scan(FwdArgs a,
                                                                                          const unsigned char *ws) {
  using S = Split<VAR, IT, D, C, BW>;
  using Z = Scan<VAR, IT, D, C, BW, NS, ONE, MAPS>;
  using OpT = IT;
  using Frag = typename Op<OpT>::frag;
  using Pr = Pair<OpT>;
  constexpr int NB = S::NB, NA = S::NA, NCW = Z::NCW, LX = S::LX, VEC = S::VEC, TPR = S::TPR, RPC = Z::RPC;
  constexpr int LXV = Z::LXV, TPV = Z::TPV, RPV = Z::RPV;
  constexpr int CS = S::CS, CSP = S::CSP, NBS = S::NBS, NXS = Z::NXS, NDW = Z::NDW, NOW = Z::NOW;
  constexpr int NQS = Z::NQS > 0 ? Z::NQS : 1;   // query slots (one unused slot in the map form)
  constexpr bool PERCH = S::PERCH, DELTA = S::DELTA;
  constexpr bool FULLT = S::SDELTA && !ONE;   // the image holds the blocks of M^{-1} (complete_inverse)

  // Raw operands (dk permuted); the per-row factors are applied to the products,
  // so copy waves only move bytes and take few issue slots from the other waves:
  __shared__ __attribute__((aligned(16))) OpT sX[NXS][C * LX];     // key of each virtual row
  __shared__ __attribute__((aligned(16))) IT sV[NXS][C * LXV];     // raw v of each virtual row, this workgroup's channels
  __shared__ __attribute__((aligned(16))) OpT sQ[NQS][MAPS ? 8 : CSP * LX];   // q of each step row
  __shared__ __attribute__((aligned(16))) unsigned char sImg[3][S::IMG];
  // handed from each state wave to its output wave: S at the system's start, E'
  __shared__ Pr sSp[MAPS ? 1 : 2][MAPS ? 1 : NCW][NA / 2][MAPS ? 1 : 64];
  __shared__ Frag sEb[MAPS ? 1 : 2][MAPS ? 1 : NCW][NB][MAPS ? 1 : 64];
  // one-pass: squared norms of key / query rows, clamped log-decays and gains of
  // the steps (staged with the rows), and each derive wave's per-row arrays
  __shared__ float sNrm[ONE ? 3 : 1][2][ONE ? C : 1];
  __shared__ float sGB[ONE ? 3 : 1][2][ONE ? C : 1];
  __shared__ __attribute__((aligned(16))) float sG[ONE ? NDW : 1][ONE ? Z::RG * C : 1];

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
  // token range of the sequence: row b of a dense [B, T] batch, or the packed
  // tokens cu[b] .. cu[b+1] (one-pass form); an empty sequence is skipped whole
  const long long tok0 = a.cu ? (long long)a.cu[b] : (long long)b * a.T;
  const int T = a.cu ? a.cu[b + 1] - a.cu[b] : a.T;
  if (T <= 0) return;
  const int H = a.H, NC = a.nchunks, NSYS = S::nsys(T);
  const int role = wv < NCW ? 0 : wv < NCW + NOW ? 1 : wv < NCW + NOW + NDW ? 3 : 2;   // state, output, derive, copy
  const int cw = role == 1 ? wv - NCW : wv;                // channel group of a state / output wave
  const int dw = wv - NCW - NOW;                           // derive wave index
  const int ctid = tid - 64 * (NCW + NOW + NDW);           // copy thread index
  const int chW = Z::DS * sp + 16 * cw + cl;               // the lane's value channel

  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);
  // two-kernel form: this sequence's images (consecutive systems) and its carry
  // block, for a dense batch or packed sequences (image slots per head)
  const unsigned char *wsq = nullptr;
  const float *carry = nullptr;
  if constexpr (!ONE) {
    if (a.cu) {
      const int SL = S::slots(a.B, a.T);
      wsq = ws + ((size_t)h * SL + S::slot0(a.cu, b)) * S::IMG;
      carry = reinterpret_cast<const float *>(ws + (size_t)H * SL * S::IMG + (size_t)bh * S::CARRY);
    } else {
      wsq = ws + (size_t)bh * NSYS * S::IMG;
      carry = reinterpret_cast<const float *>(ws + (size_t)a.B * H * NSYS * S::IMG + (size_t)bh * S::CARRY);
    }
  }
  // carried features / window values: the prep kernel's copy (two-kernel form) or the
  // caller's incoming state (one-pass form; then the outgoing state is written by the
  // tail kernel when it may alias and other workgroups read it)
  auto carried_key = [&](int j, int e) -> float {   // element e of the key of pair j <= 0
    if constexpr (ONE) {
      const float *src = j == 0 ? a.xprev0 : a.winx0;
      return src ? src[(j == 0 ? (size_t)bh : (size_t)bh * (BW - 1) + j + BW - 1) * D + e] : 0.f;
    } else {
      return carry[(j == 0 ? 0 : (j + BW) * D) + e];
    }
  };
  auto carried_val = [&](int j, int ch) -> float {  // channel ch of the value of pair j < 0
    if constexpr (ONE) {
      return a.winv0 ? a.winv0[((size_t)bh * (BW - 1) + j + BW - 1) * D + ch] : 0.f;
    } else {
      return carry[(j + 2 * BW - 1) * D + ch];
    }
  };
  // step and pair index of virtual row r of the system starting at step c0
  auto step_of = [](int c0, int r) { return c0 + r / BW; };
  auto pair_of = [](int c0, int r) { return BW == 1 ? c0 + r : c0 + r / BW - BW + 1 + r % BW; };

  // ================= copy waves =================
  // Two register sets: system c lands in set c & 1, two systems ahead of its use,
  // so a load has two scan iterations to arrive.
  struct Regs {
    uint4 k[Z::NPK], q[Z::NPK], v[Z::NPV], img[Z::NPI];
    float g, bt;   // one-pass: log-decay and gain of step ctid
  };
  Regs reg[2];
  // A system is "interior" when every row's pair index is >= 1 and every step is
  // inside the sequence: its rows are then plain strided reads, with no clamps,
  // masks or carried features.
  auto interior = [&](int c) { return c * CS >= BW - a.align && (c + 1) * CS <= T; };
  const long long rstride = (long long)H * D;   // elements between consecutive tokens
  // One-pass form: interior systems load through buffer resources based at this
  // sequence's rows, with lane-constant byte offsets and the system's offset in an
  // SGPR, so a load needs no per-lane address arithmetic (-7 % VALU instructions,
  // -1 to -2 % time at the 130M-layer shape).  The two-kernel scan keeps plain
  // global loads: buffer loads measured 5-20 % slower there (at d = 128 most).
  // The range check of a buffer load sees the lane offset alone, which must
  // therefore be >= 0: the key and value resources start BW - 1 rows early, the
  // oldest pair a virtual row can name.  Used while every offset of the sequence
  // fits 31 bits.
  const bool bufok = ONE && (long long)(T + BW + 1) * rstride * S::SZ < 0x7fffffffLL;
  const long long tokv = tok0 - (BW - 1);         // value row of the oldest pair of system 0
  const long long tokb = tokv - 1 + a.align;      // its key row
  const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vp + tokv * rstride + (long long)h * D + Z::DS * sp), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(kp + tokb * rstride + (long long)h * D), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsq = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(qp + tok0 * rstride + (long long)h * D), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsg = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.g + tok0 * H + h), 0, 0x7fffffff, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.beta + (PERCH ? 0 : tok0 * H + h)), 0, 0x7fffffff, 0x00020000);
  int vofs_v[Z::NPV], vofs_k[Z::NPK], vofs_q[Z::NPK];
#pragma unroll
  for (int ps = 0; ps < Z::NPV; ++ps) {
    const int r = min(ps * RPV + ctid / TPV, C - 1), part = ctid % TPV;
    vofs_v[ps] = (int)(((pair_of(0, r) + BW - 1) * rstride + part * VEC) * S::SZ);
  }
#pragma unroll
  for (int ps = 0; ps < Z::NPK; ++ps) {
    const int r = min(ps * RPC + ctid / TPR, C - 1), part = ctid % TPR;
    vofs_k[ps] = (int)(((pair_of(0, r) + BW - 1) * rstride + part * VEC) * S::SZ);
    vofs_q[ps] = (int)((min(r, CS - 1) * rstride + part * VEC) * S::SZ);
  }
  const int vofs_g = min(ctid, CS - 1) * H * 4;
  auto prefetch = [&](int c, Regs &R) __attribute__((always_inline)) {    // global -> registers, system c (rows clamped in bounds)
    const int c0 = c * CS;
    if (ONE && bufok && interior(c)) {
      const int so = (int)(c0 * rstride * S::SZ);   // the system's first row
#pragma unroll
      for (int ps = 0; ps < Z::NPV; ++ps)
        R.v[ps] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsv, vofs_v[ps], so, 0));
#pragma unroll
      for (int ps = 0; ps < Z::NPK; ++ps) {
        R.k[ps] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsk, vofs_k[ps], so, 0));
        R.q[ps] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsq, vofs_q[ps], so, 0));
      }
      if constexpr (ONE) {
        const int sg = c0 * H * 4;
        R.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsg, vofs_g, sg, 0));
        R.bt = PERCH ? 0.f : __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, vofs_g, sg, 0));
      } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(wsq + (size_t)c * S::IMG);
#pragma unroll
        for (int j = 0; j < Z::NPI; ++j) R.img[j] = src[min(ctid + j * Z::NST, S::NU - 1)];
      }
      return;
    }
    if (interior(c)) {
      const long long base = (tok0 + c0) * rstride + (long long)h * D;   // token c0 of the sequence
#pragma unroll
      for (int ps = 0; ps < Z::NPV; ++ps) {
        const int r = min(ps * RPV + ctid / TPV, C - 1), part = ctid % TPV;
        R.v[ps] = *reinterpret_cast<const uint4 *>(vp + base + pair_of(0, r) * rstride + Z::DS * sp + part * VEC);
      }
#pragma unroll
      for (int ps = 0; ps < Z::NPK; ++ps) {
        const int r = min(ps * RPC + ctid / TPR, C - 1), part = ctid % TPR;
        R.k[ps] = *reinterpret_cast<const uint4 *>(kp + base + (pair_of(0, r) - 1 + a.align) * rstride + part * VEC);
        if constexpr (!MAPS) R.q[ps] = *reinterpret_cast<const uint4 *>(qp + base + min(r, CS - 1) * rstride + part * VEC);
      }
      if constexpr (ONE) {
        const size_t gi = ((size_t)(tok0 + c0 + min(ctid, CS - 1))) * H + h;
        R.g = a.g[gi];
        R.bt = PERCH ? 0.f : a.beta[gi];
      } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(wsq + (size_t)c * S::IMG);
#pragma unroll
        for (int j = 0; j < Z::NPI; ++j) R.img[j] = src[min(ctid + j * Z::NST, S::NU - 1)];
      }
      return;
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPV; ++ps) {
      const int r = min(ps * RPV + ctid / TPV, C - 1), part = ctid % TPV;
      const int tv = min(max(pair_of(c0, r), 0), T - 1);
      R.v[ps] = *reinterpret_cast<const uint4 *>(vp + ((size_t)(tok0 + tv) * H + h) * D + Z::DS * sp + part * VEC);
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPK; ++ps) {
      const int r = min(ps * RPC + ctid / TPR, C - 1), part = ctid % TPR;
      const int tk = min(max(pair_of(c0, r) - 1 + a.align, 0), T - 1), tq = min(c0 + r, T - 1);
      R.k[ps] = *reinterpret_cast<const uint4 *>(kp + ((size_t)(tok0 + tk) * H + h) * D + part * VEC);
      if constexpr (!MAPS) R.q[ps] = *reinterpret_cast<const uint4 *>(qp + ((size_t)(tok0 + tq) * H + h) * D + part * VEC);
    }
    if constexpr (ONE) {
      const int t = min(c0 + min(ctid, CSP - 1), T - 1);
      R.g = a.g[(size_t)(tok0 + t) * H + h];
      R.bt = PERCH ? 0.f : a.beta[(size_t)(tok0 + t) * H + h];
    } else {
      const uint4 *src = reinterpret_cast<const uint4 *>(wsq + (size_t)c * S::IMG);
#pragma unroll
      for (int j = 0; j < Z::NPI; ++j) R.img[j] = src[min(ctid + j * Z::NST, S::NU - 1)];
    }
  };
  auto stage = [&](int c, const Regs &R) __attribute__((always_inline)) { // registers -> LDS slots of system c
    const int s2 = c % NXS, s3 = c % NQS, si = c % 3, c0 = c * CS;
    if (interior(c)) {
#pragma unroll
      for (int ps = 0; ps < Z::NPV; ++ps) {
        const int r = ps * RPV + ctid / TPV, part = ctid % TPV;
        if (r < C) *reinterpret_cast<uint4 *>(sV[s2] + r * LXV + part * VEC) = R.v[ps];
      }
#pragma unroll
      for (int ps = 0; ps < Z::NPK; ++ps) {
        const int r = ps * RPC + ctid / TPR, part = ctid % TPR;
        if (r < C) {
          put_perm(sX[s2] + r * LX, part * VEC, R.k[ps]);
          if constexpr (ONE) {
            const float sk = group_sum<TPR>(sumsq(R.k[ps], IT()));
            if (part == 0) sNrm[si][0][r] = sk;
          }
          if (!MAPS && r < CSP) {
            const uint4 qq = CSP > CS ? keep_or_zero(r < CS, R.q[ps]) : R.q[ps];
            put_perm(sQ[s3] + r * LX, part * VEC, qq);
            if constexpr (ONE) {
              const float sq = group_sum<TPR>(sumsq(qq, IT()));
              if (part == 0) sNrm[si][1][r] = sq;
            }
          }
        }
      }
      if constexpr (ONE) {
        if (ctid < CSP) {
          const bool ok = ctid < CS;
          sGB[si][0][ctid] = ok ? fmaxf(R.g, a.log_eps_gamma) : 0.f;
          sGB[si][1][ctid] = ok ? R.bt : 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < Z::NPI; ++j) {
          const int u = ctid + j * Z::NST;
          if (u < S::NU) *reinterpret_cast<uint4 *>(sImg[si] + 16 * u) = R.img[j];
        }
      }
      return;
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPV; ++ps) {
      const int r = ps * RPV + ctid / TPV, part = ctid % TPV;
      if (r < C) {
        const int j = pair_of(c0, r);
        const bool live = step_of(c0, r) < T;
        uint4 vv = keep_or_zero(live && j >= 0, R.v[ps]);
        if (BW > 1 && live && j < 0) {   // a carried window value (fp32)
          float vf[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) vf[e] = carried_val(j, Z::DS * sp + part * VEC + e);
          vv = scale_pack<IT, VEC>(vf, 1.f);
        }
        *reinterpret_cast<uint4 *>(sV[s2] + r * LXV + part * VEC) = vv;
      }
    }
#pragma unroll
    for (int ps = 0; ps < Z::NPK; ++ps) {
      const int r = ps * RPC + ctid / TPR, part = ctid % TPR;
      if (r < C) {
        const int j = pair_of(c0, r);
        const bool live = step_of(c0, r) < T;
        const bool carried = j - 1 + a.align < 0;   // key before the sequence: x_prev (j = 0) or window
        uint4 kk = keep_or_zero(live && !carried, R.k[ps]);
        float sk = 0.f;   // one-pass: squared norm of the row, for the derive waves
        if (live && carried) {   // a carried feature (fp32, normalised)
          float xv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = carried_key(j, part * VEC + e);
          kk = scale_pack<OpT, VEC>(xv, 1.f);
          if constexpr (ONE) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) sk += xv[e] * xv[e];
          }
        } else if constexpr (ONE) {
          sk = sumsq(kk, IT());
        }
        put_perm(sX[s2] + r * LX, part * VEC, kk);
        if constexpr (ONE) {
          sk = group_sum<TPR>(sk);
          if (ctid % TPR == 0) sNrm[si][0][r] = sk;
        }
        if (!MAPS && r < CSP) {
          const uint4 qq = keep_or_zero(r < CS && c0 + r < T, R.q[ps]);
          put_perm(sQ[s3] + r * LX, part * VEC, qq);
          if constexpr (ONE) {
            const float sq = group_sum<TPR>(sumsq(qq, IT()));
            if (ctid % TPR == 0) sNrm[si][1][r] = sq;
          }
        }
      }
    }
    if constexpr (ONE) {
      if (ctid < CSP) {   // steps past the system or the sequence decay and write nothing
        const bool ok = ctid < CS && c0 + ctid < T;
        sGB[si][0][ctid] = ok ? fmaxf(R.g, a.log_eps_gamma) : 0.f;
        sGB[si][1][ctid] = ok ? R.bt : 0.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < Z::NPI; ++j) {
        const int u = ctid + j * Z::NST;
        if (u < S::NU) *reinterpret_cast<uint4 *>(sImg[si] + 16 * u) = R.img[j];
      }
    }
  };

  // ================= state waves =================
  f4 sT[NA];                 // S^T of this wave's 16 channels, C-layout per dk block
  float rbeta[NB][4];        // F2/F2A: per-channel gains of the next system
  if (role == 0) {
#pragma unroll
    for (int aa = 0; aa < NA; ++aa)
      sT[aa] = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) : zero4();
  }
  // raw gains (rows clamped in bounds); the mask for rows past the end is applied
  // where they are used, so nothing waits for these loads before the next system
  auto prefetch_beta = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < NB; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = c * CS + 16 * p + 4 * g4 + i;
        rbeta[p][i] = a.beta[((size_t)(tok0 + min(t, T - 1)) * H + h) * D + chW];
      }
  };

  auto consume = [&](int c) __attribute__((always_inline)) {
    const int s2 = c & 1, s3 = c % 3;
    const OpT *X = sX[c % NXS];
    const IT *V = sV[c % NXS];
    const float *F = reinterpret_cast<const float *>(sImg[s3] + S::OFF_F);
    const OpT *Ao = reinterpret_cast<const OpT *>(sImg[s3] + S::OFF_A);
    const OpT *Tb = reinterpret_cast<const OpT *>(sImg[s3] + S::OFF_T);
    Pr Sp[NA / 2];
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) {
      Sp[a2] = mkp(cvt<OpT>(sT[2 * a2]), cvt<OpT>(sT[2 * a2 + 1]));
      if constexpr (!MAPS) sSp[s2][cw][a2][lane] = Sp[a2];
    }
    // XS = diag(GAM) X S0^T: C-layout (virtual rows 16p+4g+i, channel c), the row
    // factor applied to the product
    f4 XS[NB];
    if constexpr (DELTA) {
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        XS[p] = zero4();
#pragma unroll
        for (int a2 = 0; a2 < NA / 2; ++a2) mmap(XS[p], ldp(X + (16 * p + cl) * LX + 32 * a2 + 8 * g4), Sp[a2]);
        XS[p] *= *reinterpret_cast<const f4 *>(F + F_GAM * C + 16 * p + 4 * g4);
      }
    }
    // state: S^T <- e^{L_last} S^T + X^T diag(CST) E', accumulated as row blocks finish
    const float lamtot = F[F_N * C];
#pragma unroll
    for (int aa = 0; aa < NA; ++aa) sT[aa] *= lamtot;
    auto vcol = [&](int j4) { return 16 * cw + 4 * j4; };
    Frag Eb[NB];               // E' = E (F1/F3), eta (.) E (F2), V (F1A/F3A), eta (.) V (F2A)
    Frag Ec[NB];               // diag(CST) E', the state update's right operand
    // F1 / F3 from a prep-made image: its A slots hold the blocks of T = M^{-1}
    // (complete_inverse), so E = T R needs every residual block first and then
    // no block waits for another
    Frag Rb[FULLT ? NB : 1];
    if constexpr (FULLT) {
#pragma unroll
      for (int p = 0; p < NB; ++p) Rb[p] = cvt<OpT>(to_f4(ldT(V, LXV, 16 * p, vcol, lane)) - XS[p]);
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) {
      f4 Ef;                   // E' in fp32
      if constexpr (FULLT) {
        Ef = zero4();
#pragma unroll
        for (int q = 0; q + 1 <= p; q += 2) mmap(Ef, ldp(Ao + frag_off(aslot_base(p), q, lane)), mkp(Rb[q], Rb[q + 1]));
        if (!(p & 1)) mma16(Ef, ld4(Tb + (p * 64 + lane) * 4), Rb[p]);
      } else {
        f4 R = to_f4(ldT(V, LXV, 16 * p, vcol, lane));  // C-layout values of this wave's channels
        if (DELTA) R -= XS[p];
        f4 eta4;
        if (PERCH) {
          const f4 inv = *reinterpret_cast<const f4 *>(F + F_ETA * C + 16 * p + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {   // zero past the end: padded rows must not write
            const int t = c * CS + 16 * p + 4 * g4 + i;
            eta4[i] = (t < T ? rbeta[p][i] : 0.f) * inv[i];
          }
        }
        if (DELTA) {   // R -= sum_{q<p} A_pq E_q   (E_q = eta (.) E for F2)
          f4 acc = zero4();
#pragma unroll
          for (int q = 0; q + 1 < p; q += 2) mmap(acc, ldp(Ao + frag_off(aslot_base(p), q, lane)), mkp(Eb[q], Eb[q + 1]));
          if (p & 1) mma16(acc, ld4(Ao + frag_off(aslot_base(p), p - 1, lane)), Eb[p - 1]);
          R -= acc;
        }
        if constexpr (S::SDELTA) {
          Ef = zero4();
          mma16(Ef, ld4(Tb + (p * 64 + lane) * 4), cvt<OpT>(R));
        } else if constexpr (VAR == V_F2) {
          // rows 4g4..4g4+3 of block p: exact 4x4 solves, coupled by A_pp minus its 4x4 diagonal
          const float *Ad = reinterpret_cast<const float *>(sImg[s3] + S::OFF_AD) + (p * 4 + g4) * 8;
          const f4 c0v = *reinterpret_cast<const f4 *>(Ad), c1v = *reinterpret_cast<const f4 *>(Ad + 4);
          const float a10 = c0v[0], a20 = c0v[1], a21 = c0v[2], a30 = c0v[3], a31 = c1v[0], a32 = c1v[1];
          const Frag Ain = ld4(Tb + (p * 64 + lane) * 4);
          f4 E;
          auto local = [&](const f4 &zz) {
            E[0] = zz[0];
            Ef[0] = eta4[0] * E[0];
            E[1] = zz[1] - a10 * Ef[0];
            Ef[1] = eta4[1] * E[1];
            E[2] = zz[2] - a20 * Ef[0] - a21 * Ef[1];
            Ef[2] = eta4[2] * E[2];
            E[3] = zz[3] - a30 * Ef[0] - a31 * Ef[1] - a32 * Ef[2];
            Ef[3] = eta4[3] * E[3];
          };
          local(R);
#pragma unroll
          for (int it = 0; it < 3; ++it) {
            f4 cpl = zero4();
            mma16(cpl, Ain, cvt<OpT>(Ef));
            local(R - cpl);
          }
        } else if constexpr (VAR == V_F2A) {
          Ef = eta4 * R;
        } else {
          Ef = R;
        }
      }
      Eb[p] = cvt<OpT>(Ef);
      if constexpr (!MAPS) sEb[s2][cw][p][lane] = Eb[p];
      Ec[p] = cvt<OpT>(Ef * *reinterpret_cast<const f4 *>(F + F_CST * C + 16 * p + 4 * g4));
      // a finished pair of row blocks (or the last, unpaired one) goes into the state
      if ((p & 1) || p == NB - 1) {
        const bool pair = p & 1;
        const int q0 = pair ? p - 1 : p;
#pragma unroll
        for (int aa = 0; aa < NA; ++aa) {
          auto dkcol = [&](int j4) { return kperm(16 * aa + 4 * j4); };
          if (pair)
            mmap(sT[aa], mkp(ldT(X, LX, 16 * q0, dkcol, lane), ldT(X, LX, 16 * p, dkcol, lane)), mkp(Ec[q0], Ec[p]));
          else
            mma16(sT[aa], ldT(X, LX, 16 * q0, dkcol, lane), Ec[q0]);
        }
      }
    }
    if (a.chunk_states && ((c + 1) % BW == 0 || c == NSYS - 1)) {   // every C steps
      const int ci = c / BW;
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.chunk_states + (((size_t)bh * NC + ci) * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  };

  // ================= output waves =================
  // outputs of system c, transposed: o^T = (diag(EL) Q^ S0^T)^T + E'^T P^T.  The
  // S fragments are the left operands of the first product; the C-layout
  // fragments of E' the left operands, the stored score fragments the right ones,
  // of the second.  Lane (g, c) ends with channels 16w+4g..16w+4g+3 of step 16p+c.
  auto output = [&](int c) __attribute__((always_inline)) {
    const int s2 = c & 1, s3 = c % 3, c0 = c * CS;
    const OpT *Q = sQ[c % NQS];
    const float *F = reinterpret_cast<const float *>(sImg[s3] + S::OFF_F);
    const OpT *Pm = reinterpret_cast<const OpT *>(sImg[s3] + S::OFF_P);
    Pr Sp[NA / 2];
    Frag Eb[NB];
#pragma unroll
    for (int a2 = 0; a2 < NA / 2; ++a2) Sp[a2] = sSp[s2][cw][a2][lane];
#pragma unroll
    for (int p = 0; p < NB; ++p) Eb[p] = sEb[s2][cw][p][lane];
#pragma unroll
    for (int ps = 0; ps < NBS; ++ps) {
      f4 O = zero4();
#pragma unroll
      for (int a2 = 0; a2 < NA / 2; ++a2) mmap(O, Sp[a2], ldp(Q + (16 * ps + cl) * LX + 32 * a2 + 8 * g4));
      O *= F[F_EL * C + 16 * ps + cl];
      const int qm = S::qmax(ps);
#pragma unroll
      for (int q = 0; q + 1 <= qm; q += 2) mmap(O, mkp(Eb[q], Eb[q + 1]), ldp(Pm + frag_off(S::pbase(ps), q, lane)));
      if (!(qm & 1)) mma16(O, Eb[qm], ld4(Pm + frag_off(S::pbase(ps), qm, lane)));
      const int srow = 16 * ps + cl, t = c0 + srow;
      if (op && srow < CS && t < T)  // no outputs when o is null (the segment-map passes)
        *reinterpret_cast<Frag *>(op + ((size_t)(tok0 + t) * H + h) * D + Z::DS * sp + 16 * cw + 4 * g4) = cvt<OpT>(O);
    }
  };

  // ================= derive waves (one-pass form) =================
  // The wave's share of the image tiles of system c; while its products run,
  // the per-row arrays (lane = row; each derive wave keeps its own copy) are
  // computed from the staged norms and gates, loaded first.
  auto derive = [&](int c) __attribute__((always_inline)) {
    const int si = c % 3, c0 = c * CS;
    float *G = sG[ONE ? dw : 0];
    const float *nk = sNrm[si][0], *nq = sNrm[si][1], *gg = sGB[si][0], *gb = sGB[si][1];
    const int lr = lane < C ? lane : 0;
    const float g2 = lane < CSP ? gg[lane] : 0.f;     // lane = step
    const float sk = nk[lr], sqn = lane < CSP ? nq[lane] : 0.f, gbl = lane < CSP ? gb[lane] : 0.f;
    auto rows = [&]() __attribute__((always_inline)) -> float {
      const float L = wave_inclusive_scan(g2);
      const float Llast = __shfl(L, CS - 1);
      const bool sep = Llast >= -160.f;
      const float Lref = 0.5f * Llast;
      if (lane >= C) {
        // rows past the system: no per-row entries
      } else if constexpr (BW == 1) {   // lane = row = step
        const bool carried = c0 + lane - 1 + a.align < 0;
        const float ik = carried ? 1.f : safe_rsqrt(sk + a.eps_phi);
        const float iq = safe_rsqrt(sqn + a.eps_phi);
        const float inv = fast_rcp(a.eps_eta + sk * ik * ik);
        const float eta = PERCH ? inv : gbl * inv;
        const float cf = PERCH ? ik : ik * eta;
        G[R_LC * C + lane] = L;
        G[R_LM * C + lane] = L - g2;
        G[R_IK * C + lane] = ik;
        G[R_IQ * C + lane] = iq;
        G[R_CF * C + lane] = cf;
        G[R_ETA * C + lane] = eta;
        if (sep) {
          G[R_EP * C + lane] = __expf(L - Lref) * iq;
          G[R_EA * C + lane] = __expf(L - g2 - Lref) * ik;
          G[R_EC * C + lane] = __expf(Lref - L) * cf;
        }
      } else {   // lane = virtual row r (step r / BW); step values come from lane = step
        const int st = lane / BW, j = c0 + st - BW + 1 + lane % BW;
        const float ik = j - 1 + a.align < 0 ? 1.f : safe_rsqrt(sk + a.eps_phi);
        const float e2 = sk * ik * ik;
        const float e2new = __shfl(e2, st * BW + BW - 1);   // the step's own (newest) pair
        const float Ls = __shfl(L, st), gs = __shfl(g2, st), bs = __shfl(gbl, st);
        const float w = bs * fast_rcp(a.eps_eta + e2new) * (1.f / BW);
        const float cf = ik * w;
        G[R_LC * C + lane] = Ls;
        G[R_LM * C + lane] = Ls - gs;
        G[R_IK * C + lane] = ik;
        G[R_CF * C + lane] = cf;
        G[R_ETA * C + lane] = w;
        if (sep) {
          G[R_EA * C + lane] = __expf(Ls - gs - Lref) * ik;
          G[R_EC * C + lane] = __expf(Lref - Ls) * cf;
        }
        if (lane < CSP) {
          const float iq = (lane < CS && c0 + lane < T) ? safe_rsqrt(sqn + a.eps_phi) : 0.f;
          G[R_IQ * C + lane] = iq;
          G[R_LQ * C + lane] = L;
          G[R_GQ * C + lane] = g2;
          if (sep) G[R_EP * C + lane] = __expf(L - Lref) * iq;
        }
      }
      wave_lds_sync();
      return Llast;
    };
    derive_image<VAR, IT, D, C, BW>(sX[c % NXS], sQ[c % NQS], G, sImg[si], dw, lane, rows);
  };

  // ---------------- scan: iteration i works on system i (state), i-1 (outputs), i+1 (staging) ----------------
  // Each role runs its own loop, so none keeps another's loop-carried registers
  // live; all pass the same number of workgroup barriers (a prologue barrier,
  // then one per iteration, NSYS + 1 iterations), which is what the barrier counts.
  // One-pass form: iteration k = -1..NSYS stages system k+2, derives k+1, runs the
  // state of k and the outputs of k-1, so every role passes NSYS + 3 barriers.
  constexpr int PRE = ONE ? 1 : 0;   // pipeline stages ahead of the state waves
  if (role == 0) {
    if (PERCH) prefetch_beta(0);
    __syncthreads();
    if (ONE) __syncthreads();
    for (int i = 0; i < NSYS; ++i) {
      consume(i);
      if (PERCH && i + 1 < NSYS) prefetch_beta(i + 1);
      __syncthreads();
    }
    __syncthreads();
    if (a.S_out) {
#pragma unroll
      for (int aa = 0; aa < NA; ++aa)
        *reinterpret_cast<f4 *>(a.S_out + ((size_t)bh * D + chW) * D + 16 * aa + 4 * g4) = sT[aa];
    }
  } else if (!MAPS && role == 1) {
    __syncthreads();
    if (ONE) __syncthreads();
    __syncthreads();
    for (int i = 1; i <= NSYS; ++i) {
      if (op) output(i - 1);   // the segment-map passes store no outputs and skip their products
      __syncthreads();
    }
  } else if (role == 3) {
    __syncthreads();
    for (int i = -1; i < NSYS - 1; ++i) {
      derive(i + 1);
      __syncthreads();
    }
    __syncthreads();
    __syncthreads();
  } else {
    prefetch(0, reg[0]);
    if (NSYS > 1) prefetch(1, reg[1]);
    stage(0, reg[0]);
    if (NSYS > 2) prefetch(2, reg[0]);
    __syncthreads();
    // the register sets are indexed with compile-time parity: two iterations per trip;
    // Rnext holds system i+1+PRE and is refilled with system i+3+PRE
    auto copy_step = [&](int i, Regs &Rnext) __attribute__((always_inline)) {
      if (i + 1 + PRE < NSYS) {
        stage(i + 1 + PRE, Rnext);
        if (i + 3 + PRE < NSYS) prefetch(i + 3 + PRE, Rnext);
      }
    };
    for (int i = -PRE; i < NSYS; i += 2) {
      copy_step(i, reg[1]);
      __syncthreads();
      if (i + 1 < NSYS) {
        copy_step(i + 1, reg[0]);
        __syncthreads();
      }
    }
    __syncthreads();
    if (a.write_tail) {
      // outgoing x_prev = phi(k_{T-1}) and, for windows, the last Bw-1 pairs
      // j = T-Bw+1..T-1 (keys phi(k_{j-1}), values v_j; carried ones for j <= 0)
      const int w8 = wv - NCW - NOW - NDW;
      // normalised key k_t (t >= 0) or carried key of pair j (t = j - 1 + align < 0) into dst[0..D)
      auto key_row = [&](int t, int j, float *dst) {
        float xv[2] = {0.f, 0.f};
        if (t >= 0) {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int e = lane + 64 * m;
            if (e < D) xv[m] = to_f(kp[((size_t)(tok0 + t) * H + h) * D + e]);
          }
          const float inv = safe_rsqrt(group_sum<64>(xv[0] * xv[0] + xv[1] * xv[1]) + a.eps_phi);
          xv[0] *= inv;
          xv[1] *= inv;
        } else {
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const int e = lane + 64 * m;
            if (e < D) xv[m] = carried_key(j, e);
          }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int e = lane + 64 * m;
          if (e < D) dst[e] = xv[m];
        }
      };
      for (int u = w8; u < BW; u += Z::NSW) {   // window pairs 0..BW-2, then x_prev
        if (u == BW - 1) {
          if (sp == 0 && a.xprev_out) key_row(T - 1, 0, a.xprev_out + (size_t)bh * D);
        } else {
          const int j = T - BW + 1 + u;
          if (sp == 0 && a.winx_out) key_row(j - 1 + a.align, j, a.winx_out + ((size_t)bh * (BW - 1) + u) * D);
          if (a.winv_out) {
            for (int e = lane; e < Z::DS; e += 64) {
              const int ch = Z::DS * sp + e;
              a.winv_out[((size_t)bh * (BW - 1) + u) * D + ch] =
                  j >= 0 ? to_f(vp[((size_t)(tok0 + j) * H + h) * D + ch]) : carried_val(j, ch);
            }
          }
        }
      }
    }
  }
}

// Channel splits built per shape: fp32 keeps whole sequences; bf16 takes 1 or
// 2 slices at d <= 64 and 2, 4 or 8 at d = 128 (whose values do not fit whole).
// The map form takes whole sequences, or 2 slices at d = 128.
template <typename IT, int D>
constexpr bool ns_built(int ns, bool maps = false, bool one = false) {
  if (maps) return sizeof(IT) == 2 && D == 128 ? (ns == 1 || ns == 2) : ns == 1;
  if (sizeof(IT) == 4) return ns == 1;
  if (D == 64 && !one && ns == 4) return true;   // two-kernel form: one state wave per workgroup
  return D <= 64 ? (ns == 1 || ns == 2) : (ns == 2 || ns == 4 || ns == 8);
}
template <int VAR, typename IT, int D, int C, int BW, int NS, bool ONE = false, bool MAPS = false>
constexpr bool scan_ok() {
  return ns_built<IT, D>(NS, MAPS, ONE) && Scan<VAR, IT, D, C, BW, NS, ONE, MAPS>::fits();
}

// Smallest built split that fits and gives at least 128 scan workgroups (else
// the largest that fits); 0 when none fits.
template <int VAR, typename IT, int D, int C, int BW, bool ONE = false>
int pick_ns(int bh) {
  const bool ok[4] = {scan_ok<VAR, IT, D, C, BW, 1, ONE>(), scan_ok<VAR, IT, D, C, BW, 2, ONE>(),
                      scan_ok<VAR, IT, D, C, BW, 4, ONE>(), scan_ok<VAR, IT, D, C, BW, 8, ONE>()};
  int best = 0;
  for (int i = 0; i < 4; ++i) {
    if (!ok[i]) continue;
    best = 1 << i;
    if (bh * best >= 128) break;
  }
  return best;
}

// Map form: the smallest split that fits and gives at least 256 workgroups (one
// per compute unit; these scans are chain-bound), else the largest; 0 if none.
template <int VAR, typename IT, int D, int C, int BW>
int pick_ns_maps(int bh) {
  if constexpr (VAR == V_F2) {   // per-channel steps: no single segment map
    return 0;
  } else {
    const bool ok[2] = {scan_ok<VAR, IT, D, C, BW, 1, false, true>(), scan_ok<VAR, IT, D, C, BW, 2, false, true>()};
    int best = 0;
    for (int i = 0; i < 2; ++i) {
      if (!ok[i]) continue;
      best = 1 << i;
      if (bh * best >= 256) break;
    }
    return best;
  }
}

template <int VAR, typename IT, int D, int C, int BW, int NS, bool ONE = false, bool MAPS = false>
hipError_t launch_scan(const FwdArgs &a, const unsigned char *w, hipStream_t st) {
  if constexpr (scan_ok<VAR, IT, D, C, BW, NS, ONE, MAPS>()) {
    hipLaunchKernelGGL((chunk_scan<VAR, IT, D, C, BW, NS, ONE, MAPS>), dim3(a.B * a.H * NS),
                       dim3(Scan<VAR, IT, D, C, BW, NS, ONE, MAPS>::NT), 0, st, a, w);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// One-pass form: a single launch, no workspace.
template <int VAR, typename IT, int D, int C, int BW>
hipError_t launch_onepass(const FwdArgs &a, hipStream_t st) {
  switch (pick_ns<VAR, IT, D, C, BW, true>(a.B * a.H)) {
    case 1: return launch_scan<VAR, IT, D, C, BW, 1, true>(a, nullptr, st);
    case 2: return launch_scan<VAR, IT, D, C, BW, 2, true>(a, nullptr, st);
    case 4: return launch_scan<VAR, IT, D, C, BW, 4, true>(a, nullptr, st);
    case 8: return launch_scan<VAR, IT, D, C, BW, 8, true>(a, nullptr, st);
  }
  return hipErrorInvalidValue;
}

template <int VAR, typename IT, int D, int C, int BW>
hipError_t launch_split(const FwdArgs &a, void *ws, hipStream_t st) {
  const int ns = pick_ns<VAR, IT, D, C, BW>(a.B * a.H);
  if (ns == 0) return hipErrorInvalidValue;
  using Sp = Split<VAR, IT, D, C, BW>;
  unsigned char *w = static_cast<unsigned char *>(ws);
  // packed sequences: one prep workgroup per image slot of each head (a.T is the total token count)
  const long long nprep = a.cu ? (long long)a.H * Sp::slots(a.B, a.T) : (long long)a.B * a.H * Sp::nsys(a.T);
  if (!a.reuse_images) {   // the images depend on keys, queries and gates only, not on S0
    hipLaunchKernelGGL((chunk_prep<VAR, IT, D, C, BW>), dim3((unsigned)nprep), dim3(256), 0, st, a, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.maps_only) {   // the end state alone, on the map form where it is built
    switch (pick_ns_maps<VAR, IT, D, C, BW>(a.B * a.H)) {
      case 1: return launch_scan<VAR, IT, D, C, BW, 1, false, true>(a, w, st);
      case 2: return launch_scan<VAR, IT, D, C, BW, 2, false, true>(a, w, st);
    }
  }
  switch (ns) {
    case 1: return launch_scan<VAR, IT, D, C, BW, 1>(a, w, st);
    case 2: return launch_scan<VAR, IT, D, C, BW, 2>(a, w, st);
    case 4: return launch_scan<VAR, IT, D, C, BW, 4>(a, w, st);
    case 8: return launch_scan<VAR, IT, D, C, BW, 8>(a, w, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace
}  // namespace falcon
