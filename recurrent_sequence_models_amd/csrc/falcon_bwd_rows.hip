// Backward pass in the recurrent form for the shapes the chunk-parallel backward
// (falcon_bwd.hip) does not build: windows of B_w pairs (Falcon-3 / 3A) and head
// dims 32 and 128, for every variant.
//
// Rows of S evolve independently given the keys, in the step ([P1] 三种等价形式:
// the recurrent form is the step itself) and in its adjoint.  For value row i:
//   forward   S_t[i] = lam_t S_{t-1}[i] + w_t sum_j e_j[i] x_j,
//             e_j[i] = v_j[i] - S_{t-1}[i].x_j (F1 / F2 / F3) or v_j[i] (additive),
//   adjoint   G[i]  += do_t[i] qh_t,   u_j[i] = G[i].x_j,
//             G[i]   = lam_t G[i] - w_t sum_j u_j[i] x_j   (additive: lam_t G[i]),
// over the pairs j = t-B_w+1..t of step t, with w_t = eta_t / B_w (eta_t[i] for
// F2 / F2A, whose window is one pair) and G the gradient at S_t.  Only the
// gradients of what all rows share sum over rows:
//   dqh_t = sum_i do_t[i] S_t[i],    dlam_t = sum_i G[i].S_{t-1}[i],
//   dx_j += w_t sum_i (e_j[i] G[i] - u_j[i] S_{t-1}[i])   (second term F1/F2/F3),
//   d eta: sum_i sum_j e_j[i] u_j[i] (scalar step) or per row (F2 / F2A),
// while dv_j[i] = sum over the steps using pair j of w_t u_j[i] stays in its row.
//
// bwd_rows: one workgroup per (sequence, 16 value rows), LP = 16 or 32 lanes per
// row with D/LP columns per lane (4 or 8 waves).  The forward pass's per-chunk states are
// the checkpoints: the chunks run in reverse, each one first forward, keeping the
// state every SUB steps in LDS, then stretch by stretch backward: the stretch's
// SUB states are recomputed into registers and the adjoint steps run in reverse.
// Every step's row sums are reduced over the workgroup's 16 rows (lane swaps
// within a wave, then LDS over the waves) and written to the workspace, one record
// per workgroup, so the result does not depend on scheduling.
// bwd_rows_finish: one wave per token adds the records of the D/16 workgroups of
// its sequence and takes the gradients through eta's norm, the decay clamp and
// the feature map phi (adjoint s (d - u^ (u^.d)) of u^ = u s, s = 1/sqrt(|u|^2 + eps)).
#include "chunk_common.h"
#include "falcon_kernels.h"
#include "lane_ops.h"

namespace falcon {

namespace {

constexpr int RROWS = 16;             // value rows per workgroup

// A value row is spread over LP = 16 or 32 lanes (D / LP columns each): 16 rows
// per workgroup of 4 or 8 waves (one or two per SIMD).
template <int LP>
struct RowLanes {
  static constexpr int RPW = 64 / LP;          // rows per wave
  static constexpr int NW = RROWS / RPW;       // waves per workgroup
  static constexpr int NT = 64 * NW;           // threads per workgroup
};

template <int D, int LP>
struct RowGeom {
  static constexpr int E = D / LP;                // columns per lane
  static constexpr int SUB = D == 128 ? 8 : 16;   // steps whose states stay in registers (a stretch)
  static constexpr int STG = D == 128 ? 32 : 64;  // steps whose inputs are staged in LDS at once (a unit)
  static constexpr int MAXCK = STG / SUB;         // stretches per unit
  static constexpr int MAXNU = 64 / STG;          // units per forward chunk (chunk <= 64)
};

// Workspace records (floats): per workgroup slice sl of a sequence, for every
// token the row sums dqh (D), dx of the pair with the token's index (D), and
// (dlam, d eta sum); then the carried window pairs' dx.
struct RowWs {
  float *q, *x, *s, *w;
};
__host__ __device__ inline RowWs row_ws(float *base, int B, int H, int T, int D, int BW) {
  const size_t bth = (size_t)B * T * H, nsl = (size_t)D / RROWS;
  RowWs p;
  p.q = base;
  p.x = p.q + nsl * bth * D;
  p.s = p.x + nsl * bth * D;
  p.w = p.s + nsl * bth * 2;
  return p;
}
inline size_t row_ws_floats(int B, int H, int T, int D, int BW) {
  const size_t bth = (size_t)B * T * H, nsl = (size_t)D / RROWS;
  return nsl * (bth * (2 * (size_t)D + 2) + (size_t)B * H * (BW - 1) * D);
}

// Sum over the LP lanes of a row: DPP butterflies within each 16-lane row of the
// wave, then (LP = 32) the lane swap of the two halves; no LDS trip.  Every lane
// of the wave must run these.
template <int LP>
__device__ __forceinline__ float rsumL(float x) {
  x = lane_sum<16>(x);
  if constexpr (LP == 32) x = add_xor16(x);
  return x;
}
template <int LP, int N>
__device__ __forceinline__ void rsumL_all(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = lane_sum<16>(x[i]);
  if constexpr (LP == 32) add_xor16_all(x);
}
// Sum over the 64 / LP rows of a wave.
template <int LP>
__device__ __forceinline__ float rsumW(float x) {
  if constexpr (LP == 16) x = add_xor16(x);
  return add_xor32(x);
}
template <int LP, int N>
__device__ __forceinline__ void rsumW_all(float (&x)[N]) {
  if constexpr (LP == 16) add_xor16_all(x);
  add_xor32_all(x);
}

template <typename IT, int E>
__device__ __forceinline__ void load_cols(const IT *p, float (&v)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = (float)p[e];
}

template <int VAR, typename IT, int D, int BW, int LP>
__global__ __launch_bounds__(RowLanes<LP>::NT) void bwd_rows(BwdArgs a) {
  using Gm = RowGeom<D, LP>;
  constexpr int LPR = LP, RPW = RowLanes<LP>::RPW, NWR = RowLanes<LP>::NW, RNT = RowLanes<LP>::NT;
  constexpr int E = Gm::E, SUB = Gm::SUB, STG = Gm::STG, NP = STG + BW - 1;
  constexpr bool DELTA = VAR == V_F1 || VAR == V_F2 || VAR == V_F3;
  constexpr bool PERCH = VAR == V_F2 || VAR == V_F2A;
  static_assert(SUB % BW == 0, "a stretch holds whole windows");
  static_assert(!PERCH || BW == 1, "per-channel steps have one pair per step");

  // one unit of up to STG steps u0 ..: the keys of its pairs u0-BW+1 .., its queries,
  // the rows' values and do, and the per-step factors
  __shared__ __attribute__((aligned(16))) float sK[NP * D];
  __shared__ __attribute__((aligned(16))) float sQ[STG * D];
  __shared__ float sV[NP * RROWS];
  __shared__ float sDO[STG * RROWS];
  __shared__ float sW[STG * (PERCH ? RROWS : 1)];                   // w_t (per row for F2 / F2A)
  __shared__ float sLam[STG], sEn[STG];                             // lam_t, eps_eta + |x_t|^2
  __shared__ __attribute__((aligned(16))) float sCk[Gm::MAXCK * RNT * E];   // state at each stretch start of the unit
  __shared__ __attribute__((aligned(16))) float sUS[Gm::MAXNU * RNT * E];   // state at each unit start of the chunk
  __shared__ __attribute__((aligned(16))) float sRq[NWR * SUB * D], sRx[NWR * SUB * D];   // per-wave row sums
  __shared__ float sRs[NWR * SUB * 2];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int rr = RPW * w + lane / LPR;    // row of the workgroup
  const int p = lane % LPR, c0 = p * E;   // this lane's columns c0 .. c0+E-1
  constexpr int NSL = D / RROWS;
  const int n_seq = blockIdx.x / NSL, sl = blockIdx.x % NSL;
  const int b = n_seq / a.H, h = n_seq % a.H, T = a.T, H = a.H;
  const int ch = sl * RROWS + rr;         // value channel of this row
  const size_t bth = (size_t)a.B * T * H;
  const RowWs ws = row_ws(a.ws, a.B, H, T, D, BW);
  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  const IT *dop = static_cast<const IT *>(a.dO);
  auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

  // The inputs of the unit of steps u0 .. u0+n-1 into LDS (steps past T are
  // identity steps: no pair written, no output read).  Every global read of the
  // unit is issued in one pass; one barrier.
  auto stage = [&](int u0, int n) {
    // rows of LPR lanes; the loop bounds are wave-uniform (rsumL needs the whole
    // wave), rows past the end load nothing and store nothing
    for (int rb = RPW * w; rb < n + BW - 1; rb += RNT / LPR) {   // pair keys
      const int r = rb + lane / LPR;
      const bool row_ok = r < n + BW - 1;
      const int j = u0 - BW + 1 + r;                          // pair index; pairs j < 0 are the carried window
      const int kt = j - 1 + a.align;                         // token of the pair's raw key
      const int i = r - (BW - 1);                             // the step whose newest pair this is
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
      bool raw = false;
      if (row_ok && j < T) {
        if (j < 0) {
          if (a.winx0) load_cols<float, E>(a.winx0 + ((size_t)n_seq * (BW - 1) + j + BW - 1) * D + c0, x);
        } else if (kt < 0) {
          if (a.xprev0) load_cols<float, E>(a.xprev0 + (size_t)n_seq * D + c0, x);
        } else {
          load_cols<IT, E>(kp + tok(kt) * D + c0, x);
          raw = true;
        }
      }
      // the step's gain, read with its key: 16 channels (one per lane) for F2 / F2A
      float beta = 0.f;
      if (row_ok && i >= 0 && j < T && (!PERCH || p < RROWS))
        beta = PERCH ? a.beta[tok(j) * D + sl * RROWS + p] : a.beta[tok(j)];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x[e] * x[e];
      ss = rsumL<LP>(ss);
      if (!row_ok) continue;
      const float sc = raw ? 1.f / sqrtf(ss + a.eps_phi) : 1.f;
#pragma unroll
      for (int e = 0; e < E; ++e) sK[r * D + c0 + e] = x[e] * sc;
      if (i >= 0) {
        const float en = a.eps_eta + ss * sc * sc;
        if (p == 0) sEn[i] = en;
        if (PERCH) {
          if (p < RROWS) sW[i * RROWS + p] = beta / en;
        }
        else if (p == 0) sW[i] = beta / en * (1.f / BW);
      }
    }
    for (int rb = RPW * w; rb < n; rb += RNT / LPR) {  // queries
      const int r = rb + lane / LPR;
      const int t = u0 + r;
      float x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = 0.f;
      if (r < n && t < T) load_cols<IT, E>(qp + tok(t) * D + c0, x);
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x[e] * x[e];
      ss = rsumL<LP>(ss);
      if (r >= n) continue;
      const float sc = 1.f / sqrtf(ss + a.eps_phi);
#pragma unroll
      for (int e = 0; e < E; ++e) sQ[r * D + c0 + e] = x[e] * sc;
    }
    for (int e = tid; e < (n + BW - 1) * RROWS; e += RNT) {   // the rows' values of every staged pair
      const int r = e / RROWS, c = sl * RROWS + e % RROWS, j = u0 - BW + 1 + r;
      float v = 0.f;
      if (j >= 0 && j < T) v = (float)vp[tok(j) * D + c];
      else if (j < 0 && a.winv0) v = a.winv0[((size_t)n_seq * (BW - 1) + j + BW - 1) * D + c];
      sV[e] = v;
    }
    for (int e = tid; e < n * RROWS; e += RNT) {
      const int t = u0 + e / RROWS;
      sDO[e] = t < T ? (float)dop[tok(t) * D + sl * RROWS + e % RROWS] : 0.f;
    }
    for (int i = tid; i < n; i += RNT) {
      const int t = u0 + i;
      sLam[i] = t < T ? __expf(fmaxf(a.g[tok(t)], a.log_eps_gamma)) : 1.f;
    }
    __syncthreads();
  };
  auto wstep = [&](int i) { return PERCH ? sW[i * RROWS + rr] : sW[i]; };

  // One forward step on this lane's columns of S: step i of the staged unit.
  auto fwd = [&](const float (&S)[E], float (&Sn)[E], int i) __attribute__((always_inline)) {
    const float lam = sLam[i], wt = wstep(i);
    float eb[BW];
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      float d = 0.f;
      if (DELTA) {
#pragma unroll
        for (int e = 0; e < E; ++e) d += S[e] * sK[(i + bb) * D + c0 + e];
      }
      eb[bb] = d;
    }
    if (DELTA) rsumL_all<LP>(eb);
#pragma unroll
    for (int bb = 0; bb < BW; ++bb) {
      eb[bb] = wt * (sV[(i + bb) * RROWS + rr] - eb[bb]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float s = lam * S[e];
#pragma unroll
      for (int bb = 0; bb < BW; ++bb) s += eb[bb] * sK[(i + bb) * D + c0 + e];
      Sn[e] = s;
    }
  };

  float G[E];
  if (a.dST) load_cols<float, E>(a.dST + ((size_t)n_seq * D + ch) * D + c0, G);
  else {
#pragma unroll
    for (int e = 0; e < E; ++e) G[e] = 0.f;
  }
  // running sums of the pairs still receiving contributions, by pair index mod BW
  float dxa[BW][E], dva[BW];
#pragma unroll
  for (int s = 0; s < BW; ++s) {
    dva[s] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) dxa[s][e] = 0.f;
  }

  const int K = a.cs_step;                  // the forward's chunk: 16, 32 or 64 steps
  const int U = K < STG ? K : STG;          // steps per unit
  const int NCK = (T + K - 1) / K, NU = K / U, NSU = U / SUB;
  for (int c = NCK - 1; c >= 0; --c) {
    // the state entering chunk c: the forward's end state of chunk c-1, or the initial state
    float S[E];
    const float *ck = c ? a.chunk_states + (((size_t)n_seq * a.cs_nc + c - 1) * D + ch) * D + c0
                        : (a.S0 ? a.S0 + ((size_t)n_seq * D + ch) * D + c0 : nullptr);
    if (ck) load_cols<float, E>(ck, S);
    else {
#pragma unroll
      for (int e = 0; e < E; ++e) S[e] = 0.f;
    }
    for (int u = 0; u < NU; ++u) {          // forward to each unit's start (own elements only)
#pragma unroll
      for (int e = 0; e < E; ++e) sUS[(u * RNT + tid) * E + e] = S[e];
      if (u + 1 == NU) break;
      stage(c * K + u * U, U);
      for (int i = 0; i < U; ++i) {
        float Sn[E];
        fwd(S, Sn, i);
#pragma unroll
        for (int e = 0; e < E; ++e) S[e] = Sn[e];
      }
      __syncthreads();   // the next stage overwrites the inputs
    }
    for (int u = NU - 1; u >= 0; --u) {
      const int u0 = c * K + u * U;
      stage(u0, U);
#pragma unroll
      for (int e = 0; e < E; ++e) S[e] = sUS[(u * RNT + tid) * E + e];
      for (int st = 0; st < NSU; ++st) {    // forward through the unit, keeping each stretch's start
#pragma unroll
        for (int e = 0; e < E; ++e) sCk[(st * RNT + tid) * E + e] = S[e];
        if (st + 1 == NSU) break;
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          float Sn[E];
          fwd(S, Sn, st * SUB + i);
#pragma unroll
          for (int e = 0; e < E; ++e) S[e] = Sn[e];
        }
      }
      for (int st = NSU - 1; st >= 0; --st) {
        const int b0 = st * SUB, s0 = u0 + b0;   // the stretch within the unit, and its first step
        float hs[SUB + 1][E];   // hs[i] = S_{s0+i-1}
#pragma unroll
        for (int e = 0; e < E; ++e) hs[0][e] = sCk[(st * RNT + tid) * E + e];
#pragma unroll
        for (int i = 0; i < SUB; ++i) fwd(hs[i], hs[i + 1], b0 + i);
#pragma unroll
        for (int i = SUB - 1; i >= 0; --i) {
          const int t = s0 + i, iu = b0 + i;
          const float dot = sDO[iu * RROWS + rr], lam = sLam[iu], wt = wstep(iu);
          float qv[E];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            G[e] += dot * sQ[iu * D + c0 + e];
            qv[e] = dot * hs[i + 1][e];
          }
          // row dot products: G.S_{t-1}, G.x_j and S_{t-1}.x_j
          float dl = 0.f, u[BW], dd[BW];
#pragma unroll
          for (int bb = 0; bb < BW; ++bb) u[bb] = dd[bb] = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) {
            dl += G[e] * hs[i][e];
#pragma unroll
            for (int bb = 0; bb < BW; ++bb) {
              const float xk = sK[(iu + bb) * D + c0 + e];
              u[bb] += G[e] * xk;
              if (DELTA) dd[bb] += hs[i][e] * xk;
            }
          }
          {   // the row sums of this step, reduced together
            constexpr int NR = 1 + (DELTA ? 2 : 1) * BW;
            float red[NR];
            red[0] = dl;
#pragma unroll
            for (int bb = 0; bb < BW; ++bb) {
              red[1 + bb] = u[bb];
              if constexpr (DELTA) red[1 + BW + bb] = dd[bb];
            }
            rsumL_all<LP>(red);
            dl = red[0];
#pragma unroll
            for (int bb = 0; bb < BW; ++bb) {
              u[bb] = red[1 + bb];
              if constexpr (DELTA) dd[bb] = red[1 + BW + bb];
            }
          }
          float deta = 0.f;
#pragma unroll
          for (int bb = 0; bb < BW; ++bb) {
            const float ev = sV[(iu + bb) * RROWS + rr] - (DELTA ? dd[bb] : 0.f);
            deta += ev * u[bb];
            const int slot = (i + 1 + bb) % BW;   // pair t-BW+1+bb; s0 is a multiple of BW
            dva[slot] += wt * u[bb];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              dxa[slot][e] += wt * ev * G[e];
              if (DELTA) dxa[slot][e] -= wt * u[bb] * hs[i][e];
            }
          }
#pragma unroll
          for (int e = 0; e < E; ++e) {
            float gn = lam * G[e];
            if (DELTA) {
#pragma unroll
              for (int bb = 0; bb < BW; ++bb) gn -= wt * u[bb] * sK[(iu + bb) * D + c0 + e];
            }
            G[e] = gn;
          }
          // pair t has all its contributions: its value gradient, and its dx into the row sums
          const int sl_t = (i + BW) % BW;
          if (p == 0 && t < T) {
            a.dv[tok(t) * D + ch] = dva[sl_t];
            if (PERCH) a.dbeta[tok(t) * D + ch] = deta / sEn[iu];
          }
          dva[sl_t] = 0.f;
          float es = PERCH ? deta * wt : deta;   // F2 / F2A: sum over rows of d eta_i eta_i
          {   // over the wave's rows, reduced together
            float red[2 + 2 * E];
            red[0] = es;
            red[1] = dl;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              red[2 + e] = qv[e];
              red[2 + E + e] = dxa[sl_t][e];
            }
            rsumW_all<LP>(red);
            es = red[0];
            dl = red[1];
#pragma unroll
            for (int e = 0; e < E; ++e) {
              qv[e] = red[2 + e];
              dxa[sl_t][e] = red[2 + E + e];
            }
          }
          if (lane < LPR) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              sRq[(w * SUB + i) * D + c0 + e] = qv[e];
              sRx[(w * SUB + i) * D + c0 + e] = dxa[sl_t][e];
            }
            if (p == 0) {
              sRs[(w * SUB + i) * 2] = dl;
              sRs[(w * SUB + i) * 2 + 1] = es;
            }
          }
#pragma unroll
          for (int e = 0; e < E; ++e) dxa[sl_t][e] = 0.f;
        }
        __syncthreads();
        // the stretch's row sums over the four waves, one record per workgroup
        for (int e = tid; e < SUB * D; e += RNT) {
          const int i = e / D, col = e % D, t = s0 + i;
          if (t < T) {
            const size_t o = ((size_t)sl * bth + tok(t)) * D + col;
            float sq = 0.f, sx = 0.f;
#pragma unroll
            for (int v = 0; v < NWR; ++v) {   // fixed order over the waves
              sq += sRq[(v * SUB + i) * D + col];
              sx += sRx[(v * SUB + i) * D + col];
            }
            ws.q[o] = sq;
            ws.x[o] = sx;
          }
        }
        if (tid < SUB * 2) {
          const int i = tid >> 1, t = s0 + i;
          if (t < T) {
            float ss = 0.f;
#pragma unroll
            for (int v = 0; v < NWR; ++v) ss += sRs[(v * SUB + i) * 2 + (tid & 1)];
            ws.s[((size_t)sl * bth + tok(t)) * 2 + (tid & 1)] = ss;
          }
        }
        __syncthreads();   // the next stretch writes its row sums
      }
    }
  }
  // the gradient at the initial state, and the carried window pairs (j = -BW+1 .. -1)
  if (a.dS0) {
#pragma unroll
    for (int e = 0; e < E; ++e) a.dS0[((size_t)n_seq * D + ch) * D + c0 + e] = G[e];
  }
  if constexpr (BW > 1) {
    __syncthreads();
#pragma unroll
    for (int j = -BW + 1; j < 0; ++j) {
      const int s = (j + BW) % BW;
      if (p == 0 && a.dwinv0) a.dwinv0[((size_t)n_seq * (BW - 1) + j + BW - 1) * D + ch] = dva[s];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = rsumW<LP>(dxa[s][e]);
        if (lane < LPR) sRx[(w * SUB + j + BW - 1) * D + c0 + e] = x;
      }
    }
    __syncthreads();
    for (int e = tid; e < (BW - 1) * D; e += RNT) {
      const int jj = e / D, col = e % D;
      float sx = 0.f;
#pragma unroll
      for (int v = 0; v < NWR; ++v) sx += sRx[(v * SUB + jj) * D + col];
      ws.w[(((size_t)sl * a.B * H + n_seq) * (BW - 1) + jj) * D + col] = sx;
    }
  }
}

// Sum over a wave.
__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// One wave per token (b, t, h), then one per carried window pair of each sequence.
template <int VAR, typename IT, int D, int BW>
__global__ __launch_bounds__(256) void bwd_rows_finish(BwdArgs a) {
  constexpr int EL = D > 64 ? D / 64 : 1;   // columns per lane
  constexpr bool PERCH = VAR == V_F2 || VAR == V_F2A;
  constexpr int NSL = D / RROWS;
  const int lane = threadIdx.x & 63;
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int T = a.T, H = a.H;
  const size_t bth = (size_t)a.B * T * H;
  const RowWs ws = row_ws(a.ws, a.B, H, T, D, BW);
  if (wid >= (long long)bth) {   // the carried window: dx of pairs j < 0 (given as features)
    if constexpr (BW > 1) {
      const long long idx = wid - (long long)bth;   // (n, slot)
      if (idx >= (long long)a.B * H * (BW - 1) || !a.dwinx0) return;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int col = lane + 64 * e;
        if (col >= D) continue;
        float s = 0.f;
        for (int sl = 0; sl < NSL; ++sl) s += ws.w[((size_t)sl * a.B * H * (BW - 1) + idx) * D + col];
        a.dwinx0[idx * D + col] = s;
      }
    }
    return;
  }
  const size_t tk = (size_t)wid;   // ((b T + t) H + h)
  const int h = (int)(tk % H);
  const int t = (int)((tk / H) % T);
  const int b = (int)(tk / ((size_t)H * T));
  const int n = b * H + h;
  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  float dqh[EL], dx[EL], q[EL], x[EL];
  float dl = 0.f, de = 0.f;
  for (int sl = 0; sl < NSL; ++sl) {
    dl += ws.s[((size_t)sl * bth + tk) * 2];
    de += ws.s[((size_t)sl * bth + tk) * 2 + 1];
  }
  // the key of pair t: raw k_{t-1+align}, or the carried x_prev (prefix pairing, t = 0)
  const int kt = t - 1 + a.align;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const int col = lane + 64 * e;
    dqh[e] = dx[e] = q[e] = x[e] = 0.f;
    if (col < D) {
      for (int sl = 0; sl < NSL; ++sl) {
        dqh[e] += ws.q[((size_t)sl * bth + tk) * D + col];
        dx[e] += ws.x[((size_t)sl * bth + tk) * D + col];
      }
      q[e] = (float)qp[tk * D + col];
      if (kt >= 0) x[e] = (float)kp[(((size_t)b * T + kt) * H + h) * D + col];
      else if (a.xprev0) x[e] = a.xprev0[(size_t)n * D + col];
    }
  }
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    sq += q[e] * q[e];
    sk += x[e] * x[e];
  }
  sq = wsum(sq);
  sk = wsum(sk);
  const float iq = 1.f / sqrtf(sq + a.eps_phi);
  const float ik = kt >= 0 ? 1.f / sqrtf(sk + a.eps_phi) : 1.f;   // carried features are used as given
  const float en = a.eps_eta + sk * ik * ik;
  // eta's norm term and the gain gradient
  float coef;
  if (PERCH) {
    coef = -2.f * de / en;   // de = sum_i d eta_i eta_i
  } else {
    const float deta = de * (1.f / BW);
    const float eta = a.beta[tk] / en;
    if (lane == 0) a.dbeta[tk] = deta / en;
    coef = -2.f * deta * eta / en;
  }
  if (lane == 0) {
    const float g = a.g[tk];
    a.dg[tk] = g > a.log_eps_gamma ? dl * __expf(g) : 0.f;
  }
  float dq1 = 0.f, dk1 = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    q[e] *= iq;
    x[e] *= ik;
    dx[e] += coef * x[e];
    dq1 += q[e] * dqh[e];
    dk1 += x[e] * dx[e];
  }
  dq1 = wsum(dq1);
  dk1 = wsum(dk1);
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const int col = lane + 64 * e;
    if (col >= D) continue;
    a.dq[tk * D + col] = iq * (dqh[e] - q[e] * dq1);
    if (kt >= 0) a.dk[(((size_t)b * T + kt) * H + h) * D + col] = ik * (dx[e] - x[e] * dk1);
    else if (a.dxprev0) a.dxprev0[(size_t)n * D + col] = dx[e];
    // the prefix pairing gives k_{T-1} no pair: its gradient is 0; the same-step
    // pairing does not read the carried x_prev
    if (!a.align && t == T - 1) a.dk[tk * D + col] = 0.f;
    if (a.align && t == 0 && a.dxprev0) a.dxprev0[(size_t)n * D + col] = 0.f;
  }
}

// Lanes per value row: 32 (two waves per SIMD, D / 32 columns per lane), except
// for windows of residual pairs (Falcon-3 with Bw > 1), whose steps reduce 2 Bw + 1
// row sums and B_w more per recomputed step: there the swaps between the 16-lane
// halves cost more than the second wave per SIMD gains (window 4: 16 lanes 4.6 ms,
// 32 lanes 5.3 ms; F3A window 4 and Falcon-1 at d = 128 are 14-19 % faster on 32),
// and at Bw = 8 the registers of 32 would spill.
template <int VAR, int D, int BW>
constexpr int rows_lanes() {
  return (VAR == V_F3 && BW > 1) ? 16 : 32;
}

template <int VAR, typename IT, int D, int BW>
hipError_t launch_rows_t(const BwdArgs &a, hipStream_t st) {
  constexpr int LP = rows_lanes<VAR, D, BW>();
  hipLaunchKernelGGL((bwd_rows<VAR, IT, D, BW, LP>), dim3((unsigned)(a.B * a.H * (D / RROWS))),
                     dim3(RowLanes<LP>::NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long waves = (long long)a.B * a.T * a.H + (long long)a.B * a.H * (BW - 1);
  hipLaunchKernelGGL((bwd_rows_finish<VAR, IT, D, BW>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename IT, int D>
hipError_t launch_rows_d(int variant, int window, const BwdArgs &a, hipStream_t st) {
  switch (variant) {
    case V_F1: return launch_rows_t<V_F1, IT, D, 1>(a, st);
    case V_F1A: return launch_rows_t<V_F1A, IT, D, 1>(a, st);
    case V_F2: return launch_rows_t<V_F2, IT, D, 1>(a, st);
    case V_F2A: return launch_rows_t<V_F2A, IT, D, 1>(a, st);
    case V_F3:
      switch (window) {
        case 1: return launch_rows_t<V_F1, IT, D, 1>(a, st);   // one pair: Falcon-1
        case 2: return launch_rows_t<V_F3, IT, D, 2>(a, st);
        case 4: return launch_rows_t<V_F3, IT, D, 4>(a, st);
        case 8: return launch_rows_t<V_F3, IT, D, 8>(a, st);
      }
      break;
    case V_F3A:
      switch (window) {
        case 1: return launch_rows_t<V_F1A, IT, D, 1>(a, st);
        case 2: return launch_rows_t<V_F3A, IT, D, 2>(a, st);
        case 4: return launch_rows_t<V_F3A, IT, D, 4>(a, st);
        case 8: return launch_rows_t<V_F3A, IT, D, 8>(a, st);
      }
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool rows_bwd_supported(int variant, bool bf16, int dk, int dv, int chunk, int window) {
  if (dk != dv || !(dk == 32 || dk == 64 || (dk == 128 && bf16))) return false;
  if (!(chunk == 16 || chunk == 32 || chunk == 64)) return false;
  if (variant < V_F1 || variant > V_F3A) return false;
  if (variant == V_F3 || variant == V_F3A) return window == 1 || window == 2 || window == 4 || window == 8;
  return window == 1;
}

size_t rows_bwd_workspace(int variant, int B, int H, int T, int d, int window) {
  const int bw = (variant == V_F3 || variant == V_F3A) ? window : 1;
  return row_ws_floats(B, H, T, d, bw) * sizeof(float);
}

hipError_t launch_rows_bwd(int variant, bool bf16, int d, int window, const BwdArgs &a, hipStream_t st) {
  if (bf16) {
    if (d == 32) return launch_rows_d<__bf16, 32>(variant, window, a, st);
    if (d == 64) return launch_rows_d<__bf16, 64>(variant, window, a, st);
    if (d == 128) return launch_rows_d<__bf16, 128>(variant, window, a, st);
  } else {
    if (d == 32) return launch_rows_d<float, 32>(variant, window, a, st);
    if (d == 64) return launch_rows_d<float, 64>(variant, window, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace falcon
