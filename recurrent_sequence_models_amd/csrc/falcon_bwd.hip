// Backward pass of the chunk-parallel form for Falcon-1 / 1A (scalar NLMS step,
// one pair per step), Falcon-2 and Falcon-2A (per-value-channel steps), d_k = d_v
// = 64, chunks of 64 steps.
//
// Falcon-2A writes diag(beta_t) v_t x_t^T / (eps_eta + |x_t|^2): it is Falcon-1A
// with values beta (.) v and a unit gain ([P1] Falcon家族: only the step becomes a
// vector over value channels).  So it runs the Falcon-1A kernels with those
// values and eta_t = 1 / (eps_eta + |x_t|^2), and the gradient of the values dE
// gives dv = beta (.) dE and the per-channel gain gradient dbeta = v (.) dE.
//
// It differentiates the scalar <do, o> + <dS_T, S_T> with respect to q, k, v,
// beta, the log-decay g and the incoming state, reading the per-chunk states the
// forward pass wrote ([P1] 三种等价形式 form C / Figure 4-C: the chunked form is
// the one a training framework runs, so it is the one differentiated here).
//
// Chunk-local notation (steps i = 0..63 of a chunk, rows past T are identity
// steps: x = q = v = 0, eta = 0, log-decay 0):
//   L_i = sum_{s<=i} l_s with l = max(g, log eps_gamma); Lm_i = L_{i-1} (Lm_0 = 0)
//   A = strict-tril(X X^T o e^{Lm_i - L_j}),  P = tril(Qh X^T o e^{L_i - L_j})
//   M = I + A diag(eta),  R = V - diag(e^{Lm}) X S0^T,  E = M^-1 R  (F1A: E = V)
//   O = diag(e^L) Qh S0^T + P diag(eta) E,   S_C = e^{L_C} S0 + E^T diag(b) X,
//   b_i = eta_i e^{L_C - L_i}.
// With G the gradient at the chunk's end state, the gradient at its start is
//   G0 = e^{L_C} G - (G X^T) diag(b) W + do^T (diag(e^L) Qh - P diag(eta) W),
//   W = M^-1 diag(e^{Lm}) X   (F1A: W = 0),
// a reverse recurrence of the same shape as the forward state recurrence.
//
// Three launches (mfma_frag.h fragment layouts).  The per-chunk kernels run their
// products on bf16 MFMA with fp32 accumulation for bf16 inputs (every operand is
// rounded to bf16 once, as in the forward pass) and on fp32 MFMA for fp32 inputs;
// the reverse-time scans carry G in fp32:
//   bwd_prep   one workgroup per chunk: the chunk's transition of the reverse
//              recurrence, M = e^{L_C} I - X^T diag(b) W (so G0 = G M + Z), and
//              Z = do^T (diag(e^L) Qh - P diag(eta) W) into the workspace.
//   bwd_scan   one workgroup per sequence, one compute wave per 16 value
//              channels (rows of G are independent) and four loader waves,
//              chunks in reverse: writes G at every chunk end and the gradient
//              of the initial S (Falcon-1A / 2A: bwd_scan_add, elementwise).
//   bwd_chunk  one workgroup per chunk: recomputes A, P, E from the chunk's
//              incoming state and takes the adjoint of every product above.
//
// Layout of a workgroup: C x 64 matrices whose columns are value or key channels
// are held by waves in 16-column tiles, so a triangular solve along the chunk
// runs inside a wave (or a pair of waves) with few barriers; C x C matrices are
// computed in 16x16 tiles spread over the waves and staged in LDS.  LDS rows
// have a pitch of 68 floats,
// which makes both the 16-byte row reads and the 4-byte column reads of the
// fragment loads free of bank conflicts.
#include "falcon_kernels.h"
#include "lane_ops.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

constexpr int D = 64;    // d_k = d_v
constexpr int C = 64;    // steps per chunk
constexpr int LD = 68;   // LDS pitch of a 64-wide matrix (floats)
constexpr int MAT = C * LD;

// ---- fragments (lane l = 16g + c) ---------------------------------------------
// A-layout of the 16x16 block at (r0, k0) of row-major M: M[r0 + c][k0 + 4g + i].
__device__ __forceinline__ f4 a_rm(const float *m, int ld, int r0, int k0, int lane) {
  return *reinterpret_cast<const f4 *>(m + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4));
}
// A-layout of the block at (r0, k0) of M^T: M[k0 + 4g + i][r0 + c].
__device__ __forceinline__ f4 a_tr(const float *m, int ld, int r0, int k0, int lane) {
  const float *p = m + (k0 + 4 * (lane >> 4)) * ld + r0 + (lane & 15);
  return f4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}
// C-layout (B operand) of the block at (k0, c0) of M: M[k0 + 4g + i][c0 + c].
__device__ __forceinline__ f4 b_rm(const float *m, int ld, int k0, int c0, int lane) {
  return a_tr(m, ld, c0, k0, lane);
}
// C-layout of the block at (k0, c0) of M^T: M[c0 + c][k0 + 4g + i].
__device__ __forceinline__ f4 b_tr(const float *m, int ld, int k0, int c0, int lane) {
  return a_rm(m, ld, c0, k0, lane);
}
// Store a C-layout tile into the block at (r0, c0) of row-major M.
__device__ __forceinline__ void st_c(float *m, int ld, int r0, int c0, int lane, const f4 &v) {
  float *p = m + (r0 + 4 * (lane >> 4)) * ld + c0 + (lane & 15);
  p[0] = v[0];
  p[ld] = v[1];
  p[2 * ld] = v[2];
  p[3 * ld] = v[3];
}

// One 16x16x16 product of fp32 fragments, d += a b: four fp32 MFMAs, or (BF, for
// bf16 inputs) both operands rounded to bf16 on one bf16 MFMA with fp32
// accumulation.  The reverse-time scans stay on fp32 MFMA.
template <bool BF>
__device__ __forceinline__ void mmx(f4 &d, const f4 &a, const f4 &b) {
  if constexpr (BF) mma16(d, to_op(a, __bf16()), to_op(b, __bf16()));
  else mma16(d, a, b);
}

// Sum over the 16 lanes that share a row of a C-layout tile.
__device__ __forceinline__ float sum16(float x) { return lane_sum<16>(x); }
// Sum over the 4 lane groups that share a column of a C-layout tile.
__device__ __forceinline__ float sum4g(float x) { return add_xor32(add_xor16(x)); }
__device__ __forceinline__ float sum64(float x) { return sum4g(sum16(x)); }

// The chunk's rows in LDS: keys x_i (features), queries qh_i and the per-row
// scalars.  With NTH threads, thread (row r = tid / NP, part p = tid % NP) takes
// 64 / NP channels, NP = NTH / 64.
struct RowScalars {
  float L[C], Lm[C], eta[C], en[C];  // L_i, L_{i-1}, eta_i, eps_eta + |x_i|^2
  float ik[C], iq[C];                // 1/|k| of row i's key (0 unless it is one) and 1/|q_i| (0 past T)
};

template <int NP>
__device__ __forceinline__ float sum_parts(float x) { return lane_sum<NP>(x); }

template <typename IT, int E>
__device__ __forceinline__ void load_e(const IT *p, float (&v)[E]) {
#pragma unroll
  for (int j = 0; j < E; ++j) v[j] = (float)p[j];
}

// One thread's share of a chunk's key and query rows and of its per-row gain and
// log-decay, read from global memory ahead of their use (fetch_rows), so that a
// kernel can issue these loads together with its others before waiting on any.
template <int NTH>
struct Rows {
  static constexpr int NP = NTH / 64, E = 64 / NP;
  float x[E], q[E], beta, g;
};

template <typename IT, int NTH>
__device__ void fetch_rows(const BwdArgs &a, int n, int c, Rows<NTH> &R) {
  constexpr int NP = NTH / 64, E = 64 / NP;
  const int tid = threadIdx.x, r = tid / NP, p = tid % NP;
  const int b = n / a.H, h = n % a.H;
  const int t = c * C + r;
  const int kt = t - 1 + a.align;  // key index of the pair written at step t
  const bool live = t < a.T;
#pragma unroll
  for (int j = 0; j < E; ++j) R.x[j] = R.q[j] = 0.f;
  const bool key_row = live && kt >= 0;
  if (key_row) load_e<IT, E>((const IT *)a.k + ((size_t)(b * a.T + kt) * a.H + h) * D + E * p, R.x);
  else if (live && a.xprev0) load_e<float, E>(a.xprev0 + (size_t)n * D + E * p, R.x);  // the carried feature
  if (live) load_e<IT, E>((const IT *)a.q + ((size_t)(b * a.T + t) * a.H + h) * D + E * p, R.q);
  const size_t gi = (size_t)(b * a.T + t) * a.H + h;
  R.beta = (live && p == 0) ? a.beta[gi] : 0.f;
  R.g = (live && p == 0) ? a.g[gi] : 0.f;
}

// The rows into LDS: normalised keys X and queries Qh, and the per-row scalars
// (the log-decays summed along the chunk).  Ends with a barrier.
template <int NTH, bool UNIT = false>   // UNIT: eta = 1 / (eps_eta + |x|^2) (Falcon-2A)
__device__ void stage_rows(const BwdArgs &a, int c, Rows<NTH> &R, float *sX, float *sQ, RowScalars &rs) {
  constexpr int NP = NTH / 64, E = 64 / NP;
  const int tid = threadIdx.x, r = tid / NP, p = tid % NP, lane = tid & 63;
  const int t = c * C + r;
  const int kt = t - 1 + a.align;
  const bool live = t < a.T;
  const bool key_row = live && kt >= 0;
  float sx = 0.f, sq = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    sx += R.x[j] * R.x[j];
    sq += R.q[j] * R.q[j];
  }
  sx = sum_parts<NP>(sx);
  sq = sum_parts<NP>(sq);
  const float ix = key_row ? 1.f / sqrtf(sx + a.eps_phi) : 1.f;
  const float iq = 1.f / sqrtf(sq + a.eps_phi);
  float e = 0.f;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    R.x[j] *= ix;
    R.q[j] = live ? R.q[j] * iq : 0.f;
    e += R.x[j] * R.x[j];
  }
  e = sum_parts<NP>(e);
#pragma unroll
  for (int j = 0; j < E; j += 4) {
    *reinterpret_cast<f4 *>(sX + r * LD + E * p + j) = f4{R.x[j], R.x[j + 1], R.x[j + 2], R.x[j + 3]};
    *reinterpret_cast<f4 *>(sQ + r * LD + E * p + j) = f4{R.q[j], R.q[j + 1], R.q[j + 2], R.q[j + 3]};
  }
  if (p == 0) {
    const float en = a.eps_eta + e;
    rs.en[r] = en;
    rs.ik[r] = key_row ? ix : 0.f;
    rs.iq[r] = live ? iq : 0.f;
    rs.eta[r] = live ? (UNIT ? 1.f : R.beta) / en : 0.f;
    rs.L[r] = live ? fmaxf(R.g, a.log_eps_gamma) : 0.f;  // log-decay, summed below
  }
  __syncthreads();
  if (tid < 64) {  // inclusive prefix sum of the log-decays along the chunk
    float l = rs.L[lane];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(l, o);
      if (lane >= o) l += y;
    }
    const float lm = __shfl_up(l, 1);
    rs.L[lane] = l;
    rs.Lm[lane] = lane ? lm : 0.f;
  }
  __syncthreads();
}

template <typename IT, int NTH, bool UNIT = false>
__device__ void load_rows(const BwdArgs &a, int n, int c, float *sX, float *sQ, RowScalars &rs) {
  Rows<NTH> R;
  fetch_rows<IT, NTH>(a, n, c, R);
  stage_rows<NTH, UNIT>(a, c, R, sX, sQ, rs);
}

// One 16x16 tile (rt, ct <= rt) of A (skipped for F1A) and P into LDS, with
// their masks (strict / causal) and decays.
template <bool ADD, bool BF>
__device__ void gram_tile(const float *sX, const float *sQ, float *sA, float *sP, const RowScalars &rs, int rt,
                          int ct, int lane) {
  const int g = lane >> 4, cc = lane & 15;
  f4 pa = zero4(), pp = zero4();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f4 xb = b_tr(sX, LD, 16 * kb, 16 * ct, lane);
    if (!ADD) mmx<BF>(pa, a_rm(sX, LD, 16 * rt, 16 * kb, lane), xb);
    mmx<BF>(pp, a_rm(sQ, LD, 16 * rt, 16 * kb, lane), xb);
  }
  const int col = 16 * ct + cc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    pa[i] = col < row ? __expf(rs.Lm[row] - rs.L[col]) * pa[i] : 0.f;
    pp[i] = col <= row ? __expf(rs.L[row] - rs.L[col]) * pp[i] : 0.f;
  }
  if (!ADD) st_c(sA, LD, 16 * rt, 16 * ct, lane, pa);
  st_c(sP, LD, 16 * rt, 16 * ct, lane, pp);
}

// The 10 tiles on or below the diagonal of a 4x4 tiling, in row order (tiles above
// the diagonal are never read).
__device__ __forceinline__ void lower_tile(int k, int &rt, int &ct) {
  rt = k < 1 ? 0 : k < 3 ? 1 : k < 6 ? 2 : 3;
  ct = k - rt * (rt + 1) / 2;
}
// Diagonal block b of a chunk solve, for the 16 columns of one wave (value or
// key channels; C-layout: lane (g, c) holds rows 16b+4g..16b+4g+3 of column c),
// with steps eta per row and column (the same for every column but Falcon-2's):
//   lower (UPPER = false): y = (I + A_bb diag(eta))^-1 r,
//   upper (UPPER = true):  y = (I + diag(eta) A_bb^T)^-1 r.
// Each lane solves its own 4 rows exactly with the 6 coefficients of its 4x4
// diagonal sub-block; the coupling between the four row groups (A_bb without
// those sub-blocks) is strictly block-triangular, so three sweeps of it on MFMA
// make the solution exact.
template <bool UPPER, bool BF>
__device__ __forceinline__ f4 pc_diag(const f4 &r, const f4 &et, const float *sA, int b, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const float *Ag = sA + (16 * b + 4 * g) * LD + 16 * b + 4 * g;   // this row group's 4x4 sub-block
  const float a10 = Ag[LD], a20 = Ag[2 * LD], a21 = Ag[2 * LD + 1];
  const float a30 = Ag[3 * LD], a31 = Ag[3 * LD + 1], a32 = Ag[3 * LD + 2];
  f4 an = UPPER ? a_tr(sA, LD, 16 * b, 16 * b, lane) : a_rm(sA, LD, 16 * b, 16 * b, lane);
  if ((c >> 2) == g) an = zero4();   // A-layout row c lies in group c / 4
  auto local = [&](const f4 &z) {
    f4 y;
    if constexpr (UPPER) {
      y[3] = z[3];
      y[2] = z[2] - et[2] * (a32 * y[3]);
      y[1] = z[1] - et[1] * (a21 * y[2] + a31 * y[3]);
      y[0] = z[0] - et[0] * (a10 * y[1] + a20 * y[2] + a30 * y[3]);
    } else {
      y[0] = z[0];
      y[1] = z[1] - a10 * (et[0] * y[0]);
      y[2] = z[2] - a20 * (et[0] * y[0]) - a21 * (et[1] * y[1]);
      y[3] = z[3] - a30 * (et[0] * y[0]) - a31 * (et[1] * y[1]) - a32 * (et[2] * y[2]);
    }
    return y;
  };
  f4 y = local(r);
#pragma unroll
  for (int it = 0; it < 3; ++it) {
    f4 cpl = zero4();
    if constexpr (UPPER) {
      mmx<BF>(cpl, an, y);
      y = local(r - et * cpl);
    } else {
      mmx<BF>(cpl, an, et * y);
      y = local(r - cpl);
    }
  }
  return y;
}

// Y <- M^-1 Y for one 16-column tile held by a wave (blocked forward substitution).
template <bool BF>
__device__ void solve_lower(f4 (&y)[4], const float *sA, const RowScalars &rs, int lane) {
  const int g = lane >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f4 s = zero4();
#pragma unroll
    for (int bp = 0; bp < b; ++bp) {
      f4 af = a_rm(sA, LD, 16 * b, 16 * bp, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] *= rs.eta[16 * bp + 4 * g + i];
      mmx<BF>(s, af, y[bp]);
    }
    const float *eb = rs.eta + 16 * b + 4 * g;
    const f4 et = {eb[0], eb[1], eb[2], eb[3]};
    y[b] = pc_diag<false, BF>(y[b] - s, et, sA, b, lane);
  }
}

// Y <- M^-T Y (blocked backward substitution).
template <bool BF>
__device__ void solve_upper(f4 (&y)[4], const float *sA, const RowScalars &rs, int lane) {
  const int g = lane >> 4, cc = lane & 15;
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    f4 s = zero4();
#pragma unroll
    for (int bp = b + 1; bp < 4; ++bp) {
      f4 af = a_tr(sA, LD, 16 * b, 16 * bp, lane);
      af *= rs.eta[16 * b + cc];
      mmx<BF>(s, af, y[bp]);
    }
    const float *eb = rs.eta + 16 * b + 4 * g;
    const f4 et = {eb[0], eb[1], eb[2], eb[3]};
    y[b] = pc_diag<true, BF>(y[b] - s, et, sA, b, lane);
  }
}

// This thread's share of rows 0..63 of a [C][64] input-typed array (rows past
// `rows_live` are zero), as fp32, and its store into LDS.
template <int NTH>
struct RowShare {
  static constexpr int NP = NTH / 64, E = 64 / NP;
  float v[E];
  template <typename IT>
  __device__ void load(const IT *base, size_t row_stride, int rows_live) {
    const int r = threadIdx.x / NP, p = threadIdx.x % NP;
    if (r < rows_live) load_e<IT, E>(base + (size_t)r * row_stride + E * p, v);
    else {
#pragma unroll
      for (int j = 0; j < E; ++j) v[j] = 0.f;
    }
  }
  __device__ void store(float *dst) const {
    const int r = threadIdx.x / NP, p = threadIdx.x % NP;
#pragma unroll
    for (int j = 0; j < E; j += 4)
      *reinterpret_cast<f4 *>(dst + r * LD + E * p + j) = f4{v[j], v[j + 1], v[j + 2], v[j + 3]};
  }
};

// Workspace arrays of one chunk.
// Workspace arrays of one chunk: the transition M = e^{L_C} I - X^T diag(b) W of
// the reverse recurrence, stored as the A-operand fragments of its transpose
// (fp32 inputs: fragment (kt, kb) of M^T at ((4 kt + kb) 64 + lane) 4 floats;
// bf16 inputs: the pairs (kt, kb / 2) of Mh at ((2 kt + kb / 2) 64 + lane) 8 +
// (kb & 1) 4 bf16 elements, Ml 4096 elements later), the injected
// gradient Z and the gradient G at the chunk's end (row-major, value rows), and
// the chunk's decay e^{L_C}.
struct WsPtr {
  float *M, *Z, *G, *dec;
};
__device__ __forceinline__ WsPtr ws_of(const BwdArgs &a, size_t chunk_id) {
  const size_t nch = (size_t)a.B * a.H * a.NC;
  float *base = a.ws;
  WsPtr p;
  p.M = base + chunk_id * D * D;
  p.Z = base + nch * D * D + chunk_id * D * D;
  p.G = base + 2 * nch * D * D + chunk_id * D * D;
  p.dec = base + 3 * nch * D * D + chunk_id;
  return p;
}

// ---- bwd_prep -------------------------------------------------------------------
// 256 threads.  LDS: X, Qh (then do), A, P and the diagonal-block inverses, so
// two workgroups share a compute unit.
template <typename IT, bool ADD>
__global__ __launch_bounds__(256) void bwd_prep(BwdArgs a) {
  constexpr bool BF = std::is_same_v<IT, __bf16>;   // bf16 inputs: products on bf16 MFMA
  __shared__ __attribute__((aligned(16))) float sX[MAT], sQ[MAT], sA[ADD ? 4 : MAT], sP[ADD ? 4 : MAT];
  __shared__ RowScalars rs;
  const int n = blockIdx.x / a.NC, c = blockIdx.x % a.NC;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
  const int b = n / a.H, h = n % a.H;
  const int live = min(C, a.T - c * C);
  RowShare<256> dO;
  dO.load((const IT *)a.dO + ((size_t)(b * a.T + c * C) * a.H + h) * D, (size_t)a.H * D, live);
  load_rows<IT, 256>(a, n, c, sX, sQ, rs);  // ends with a barrier
  const WsPtr ws = ws_of(a, blockIdx.x);
  const float LC = rs.L[C - 1];

  f4 qe[4];  // diag(e^L) Qh - P diag(eta) W, column tile w (key channels)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    qe[rt] = b_rm(sQ, LD, 16 * rt, 16 * w, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) qe[rt][i] *= __expf(rs.L[16 * rt + 4 * g + i]);
  }
  if (!ADD) {
    for (int k = w; k < 10; k += 4) {
      int rt, ct;
      lower_tile(k, rt, ct);
      gram_tile<false, BF>(sX, sQ, sA, sP, rs, rt, ct, lane);
    }
  }
  __syncthreads();  // sQ is read: it takes do from here on
  dO.store(sQ);
  if (!ADD) {
    f4 W[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      W[rt] = b_rm(sX, LD, 16 * rt, 16 * w, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i) W[rt][i] *= __expf(rs.Lm[16 * rt + 4 * g + i]);
    }
    solve_lower<BF>(W, sA, rs, lane);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f4 s = zero4();
#pragma unroll
      for (int kb = 0; kb <= rt; ++kb) {
        f4 af = a_rm(sP, LD, 16 * rt, 16 * kb, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] *= rs.eta[16 * kb + 4 * g + i];
        mmx<BF>(s, af, W[kb]);
      }
      qe[rt] -= s;
    }
    // M = e^{L_C} I - X^T diag(b) W, b_i = eta_i e^{L_C - L_i}: key rows 16kt.., key columns 16w..,
    // which is the A-operand fragment (w, kt) of M^T; for bf16 inputs stored as
    // its two bf16 parts for the scan's split products
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * g + i;
        W[rt][i] *= rs.eta[row] * __expf(LC - rs.L[row]);
      }
    }
    const float dec = __expf(LC);
    // bf16 inputs: X^T diag(b) W as three bf16 products of the split parts (x = xh + xl,
    // xh = bf16(x), xl = bf16(x - xh)), Xl Wh + Xh Wl + Xh Wh, exact to a relative 2^-16
    // (the dropped Xl Wl and the rounding of the low parts); fp32 inputs: fp32 MFMA
    bf4 wh[4], wl[4];
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        wh[kb] = to_op(W[kb], __bf16());
        wl[kb] = to_op(W[kb] - to_f4(wh[kb]), __bf16());
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f4 m = zero4();
      if constexpr (BF) {
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const f4 x0 = a_tr(sX, LD, 16 * kt, 32 * kp, lane), x1 = a_tr(sX, LD, 16 * kt, 32 * kp + 16, lane);
          const bf4 xh0 = to_op(x0, __bf16()), xh1 = to_op(x1, __bf16());
          const bf4 xl0 = to_op(x0 - to_f4(xh0), __bf16()), xl1 = to_op(x1 - to_f4(xh1), __bf16());
          mma32(m, xl0, xl1, wh[2 * kp], wh[2 * kp + 1]);
          mma32(m, xh0, xh1, wl[2 * kp], wl[2 * kp + 1]);
          mma32(m, xh0, xh1, wh[2 * kp], wh[2 * kp + 1]);
        }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) mma16(m, a_tr(sX, LD, 16 * kt, 16 * kb, lane), W[kb]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) m[i] = (16 * kt + 4 * g + i == 16 * w + cc ? dec : 0.f) - m[i];
      if constexpr (BF) {   // Mh then Ml, each as k-block pairs (w, kt / 2) of bf16
        const bf4 mh = to_op(m, __bf16()), ml = to_op(m - to_f4(mh), __bf16());
        __bf16 *dst = reinterpret_cast<__bf16 *>(ws.M) + ((2 * w + kt / 2) * 64 + lane) * 8 + (kt & 1) * 4;
        *reinterpret_cast<bf4 *>(dst) = mh;
        *reinterpret_cast<bf4 *>(dst + 8 * 64 * 8) = ml;
      } else {
        *reinterpret_cast<f4 *>(ws.M + ((4 * w + kt) * 64 + lane) * 4) = m;
      }
    }
  }
  __syncthreads();  // every thread's rows of do are in sQ
  // Z = do^T qe: value-channel rows, key-channel column tile w.
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f4 z = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mmx<BF>(z, a_tr(sQ, LD, 16 * rt, 16 * kb, lane), qe[kb]);
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.Z[(16 * rt + 4 * g + i) * D + 16 * w + cc] = z[i];
  }
  if (threadIdx.x == 0) *ws.dec = __expf(LC);
}

// ---- bwd_scan -------------------------------------------------------------------
// Falcon-1: workgroup = one sequence.  Compute wave w (0..3) carries the rows
// 16w..16w+15 of G (value channels; rows of G evolve independently) transposed,
// as four C-layout tiles of G^T (key rows 16kt.., value columns).  Per chunk, in
// reverse,
//   G^T <- M^T G^T + Z^T,
// so each product's result is the next chunk's right operand and no lane
// exchange is needed.  Loader waves (4..7) copy each chunk's M fragments and Z
// into a ring of LDS slots, NR - 1 chunks ahead of the compute waves, with their
// own global reads a further KL chunks ahead in registers; the compute waves read
// only LDS, so their chain never waits on memory.  One barrier per chunk.
// fp32 inputs: fp32 MFMA.  bf16 inputs (BF): M arrives split as Mh + Ml (two
// bf16 parts, Mh = bf16(M), Ml = bf16(M - Mh)) and G is split the same way each
// chunk; G M = Gh Mh + Gh Ml + Gl Mh up to a relative 2^-16 (the dropped Gl Ml
// and the rounding of the low parts), on bf16 MFMA with fp32 accumulation.
constexpr int SCAN_NR = 4;                       // LDS ring slots
constexpr int SCAN_ZP = 68;                      // LDS pitch of Z's rows (floats)
constexpr int SCAN_SLOT = D * D + D * SCAN_ZP;   // floats: M fragments, then Z

template <bool BF>
__global__ __launch_bounds__(512) void bwd_scan(BwdArgs a) {
  constexpr int NR = SCAN_NR, KL = 4;
  __shared__ __attribute__((aligned(16))) float ring[NR * SCAN_SLOT];
  const int n = blockIdx.x;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
  const int NC = a.NC;
  if (w >= 4) {
    // ---- loader waves: chunk NC-1-j goes to slot j % NR, written in iteration j - (NR-1)
    const int t = threadIdx.x - 256;
    f4 r[KL][8];
    auto load = [&](int j, f4 (&dst)[8]) {   // chunk NC-1-j, clamped: the last loads are spare
      const WsPtr ws = ws_of(a, (size_t)n * NC + max(NC - 1 - j, 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = *reinterpret_cast<const f4 *>(ws.M + (q * 256 + t) * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[4 + q] = *reinterpret_cast<const f4 *>(ws.Z + (q * 256 + t) * 4);
    };
    auto put = [&](int j, const f4 (&src)[8]) {
      float *slot = ring + (j % NR) * SCAN_SLOT;
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<f4 *>(slot + (q * 256 + t) * 4) = src[q];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = (q * 256 + t) * 4;   // Z[e / 64][e % 64 ..]
        *reinterpret_cast<f4 *>(slot + D * D + (e >> 6) * SCAN_ZP + (e & 63)) = src[4 + q];
      }
    };
    // register set k holds chunk NC-1-j for j = k (mod KL)
#pragma unroll
    for (int k = 0; k < KL; ++k) load(k, r[k]);
    // prologue: slots of chunks j = 0..NR-2
    int j = 0;
#pragma unroll
    for (int k = 0; k < NR - 1; ++k, ++j) {
      put(j, r[k % KL]);
      load(j + KL, r[k % KL]);
    }
    __syncthreads();
    // iteration i writes chunk jj = i + NR - 1 from register set jj % KL (i is a
    // multiple of KL at the top of the unrolled body)
    int i = 0;
    for (; i + KL <= NC; i += KL) {
#pragma unroll
      for (int k = 0; k < KL; ++k) {
        const int jj = i + k + NR - 1;
        put(jj, r[(k + NR - 1) % KL]);
        load(jj + KL, r[(k + NR - 1) % KL]);
        __syncthreads();
      }
    }
#pragma unroll
    for (int k = 0; k < KL - 1; ++k) {
      if (i + k < NC) {
        const int jj = i + k + NR - 1;
        put(jj, r[(k + NR - 1) % KL]);
        __syncthreads();
      }
    }
    return;
  }
  // ---- compute waves
  // lane (g, cc) of tile kt holds G[16w + cc][16kt + 4g + i], i = 0..3
  const size_t row = (size_t)(16 * w + cc) * D + 4 * g;   // + 16 kt
  f4 G[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
    G[kt] = a.dST ? *reinterpret_cast<const f4 *>(a.dST + (size_t)n * D * D + row + 16 * kt) : zero4();
  __syncthreads();   // the loaders' prologue
  for (int i = 0; i < NC; ++i) {
    const int c = NC - 1 - i;
    const float *slot = ring + (i % NR) * SCAN_SLOT;
    float *gout = ws_of(a, (size_t)n * NC + c).G;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) *reinterpret_cast<f4 *>(gout + row + 16 * kt) = G[kt];  // at the end of chunk c
    f4 Gn[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      Gn[kt] = *reinterpret_cast<const f4 *>(slot + D * D + (16 * w + cc) * SCAN_ZP + 16 * kt + 4 * g);
    if constexpr (BF) {
      const bf8 *mh = reinterpret_cast<const bf8 *>(slot), *ml = mh + 8 * 64;
      bf8 gh[2], gl[2];
#pragma unroll
      for (int kbp = 0; kbp < 2; ++kbp) {
        const bf4 h0 = to_op(G[2 * kbp], __bf16()), h1 = to_op(G[2 * kbp + 1], __bf16());
        const bf4 l0 = to_op(G[2 * kbp] - to_f4(h0), __bf16()), l1 = to_op(G[2 * kbp + 1] - to_f4(h1), __bf16());
        gh[kbp] = bf8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        gl[kbp] = bf8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int kbp = 0; kbp < 2; ++kbp) {
          const int j = 2 * kt + kbp;
          Gn[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ml[j * 64 + lane], gh[kbp], Gn[kt], 0, 0, 0);
          Gn[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh[j * 64 + lane], gl[kbp], Gn[kt], 0, 0, 0);
          Gn[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh[j * 64 + lane], gh[kbp], Gn[kt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          mma16(Gn[kt], *reinterpret_cast<const f4 *>(slot + ((4 * kt + kb) * 64 + lane) * 4), G[kb]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) G[kt] = Gn[kt];
    __syncthreads();   // slot i % NR is free for the loaders
  }
  if (a.dS0) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) *reinterpret_cast<f4 *>(a.dS0 + (size_t)n * D * D + row + 16 * kt) = G[kt];
  }
}

// Falcon-1A / 2A: G <- e^{L_C} G + Z elementwise.  Four workgroups per sequence,
// one 16-byte column group of G per thread; a ring of the next PF chunks' Z and
// decay is in flight (slot j holds chunk c - j; the loop body has no branch).
__global__ __launch_bounds__(256) void bwd_scan_add(BwdArgs a) {
  constexpr int PF = 8;
  const int n = blockIdx.x >> 2;
  const size_t e = ((size_t)(blockIdx.x & 3) * 256 + threadIdx.x) * 4;
  f4 G = a.dST ? *reinterpret_cast<const f4 *>(a.dST + (size_t)n * D * D + e) : zero4();
  f4 z[PF];
  float dc[PF];
  auto fetch = [&](int c, int j) {   // c clamped to 0: the ring's last loads are spare
    const WsPtr ws = ws_of(a, (size_t)n * a.NC + max(c, 0));
    z[j] = *reinterpret_cast<const f4 *>(ws.Z + e);
    dc[j] = *ws.dec;
  };
  auto step = [&](int c, int j) {
    *reinterpret_cast<f4 *>(ws_of(a, (size_t)n * a.NC + c).G + e) = G;   // at the end of chunk c
    G = dc[j] * G + z[j];
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) fetch(a.NC - 1 - j, j);
  int c = a.NC - 1;
  for (; c >= PF - 1; c -= PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      step(c - j, j);
      fetch(c - j - PF, j);
    }
  }
#pragma unroll
  for (int j = 0; j < PF - 1; ++j)
    if (j <= c) step(c - j, j);
  if (a.dS0) *reinterpret_cast<f4 *>(a.dS0 + (size_t)n * D * D + e) = G;
}

// ---- bwd_chunk ------------------------------------------------------------------
// 1024 threads = 16 waves (four per SIMD).  Wave w owns the 16x16 tile (rt, ct) =
// (w / 4, w % 4) of every C x 64 matrix.  The triangular solves run on four
// solver waves, one per column tile, which read the right-hand side from LDS and
// write the solution back (two barriers per solve).  The 10 lower tiles of the
// C x C products go to waves 0..9.  Per-wave partial sums of the row gradients
// (dL, d eta) are added in a fixed order at the end, so results are deterministic.
constexpr int NTC = 1024;
constexpr int NWC = NTC / 64;

// Adjoint of one lower tile (rt, ct) of A and P: from t = dR E^T and u = do E^T,
// the tile's contributions to dL and d eta, and dAG = dA o Gamma, dPD = dP o D in
// place of A and P.
template <bool ADD, bool BF>
__device__ void adjoint_tile(float *sA, float *sP, const float *sG, const float *sO, const float *sE,
                             const RowScalars &rs, float *pLw, float *pEw, int rt, int ct, int lane) {
  const int g = lane >> 4, cc = lane & 15;
  f4 t = zero4(), u = zero4();
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f4 eb = b_tr(sE, LD, 16 * kb, 16 * ct, lane);
    if (!ADD) mmx<BF>(t, a_rm(sG, LD, 16 * rt, 16 * kb, lane), eb);
    mmx<BF>(u, a_rm(sO, LD, 16 * rt, 16 * kb, lane), eb);
  }
  const int col = 16 * ct + cc;
  const float etac = rs.eta[col];
  float colL = 0.f, colE = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    float rowL = 0.f, rowLm = 0.f;
    if (!ADD) {
      const float Aij = sA[row * LD + col];
      const float dM = col < row ? -t[i] : 0.f;
      colE += Aij * dM;  // d eta_j += A_ij dM_ij
      const float dA = dM * etac;
      const float H = dA * Aij;
      rowLm += H;
      colL -= H;
      sA[row * LD + col] = col < row ? dA * __expf(rs.Lm[row] - rs.L[col]) : 0.f;
    }
    const float dP = col <= row ? u[i] * etac : 0.f;
    const float HP = dP * sP[row * LD + col];
    rowL += HP;
    colL -= HP;
    sP[row * LD + col] = col <= row ? dP * __expf(rs.L[row] - rs.L[col]) : 0.f;
    rowL = sum16(rowL);
    rowLm = sum16(rowLm);
    if (cc == 0) {
      pLw[row] += rowL;
      if (row > 0) pLw[row - 1] += rowLm;
    }
  }
  colL = sum4g(colL);
  colE = sum4g(colE);
  if (g == 0) {
    pLw[col] += colL;
    pEw[col] += colE;
  }
}

// The gradients of the rows' features taken through the feature map phi: dq_t
// from dQh (sO) for t < T, and dk of the key row r carries from dX (sE), plus the
// carried x_prev's gradient.  With u^ = u / sqrt(|u|^2 + eps) the normalised row
// (sQ, sX) and s = 1 / sqrt(|u|^2 + eps) (rs.iq, rs.ik), the adjoint of
// phi is s (d - u^ (u^ . d)), so nothing is read back from memory.  1024 threads,
// one chunk.
__device__ void through_phi(const BwdArgs &a, int n, int c, size_t row0, int b, int h, const float *sO,
                            const float *sE, const float *sX, const float *sQ, const RowScalars &rs) {
  const int tid = threadIdx.x;
  constexpr int NP = NTC / 64, EE = 64 / NP;
  const int r = tid / NP, p = tid % NP;
  const int t = c * C + r;
  float u[EE], d[EE];
#pragma unroll
  for (int j = 0; j < EE; ++j) {
    u[j] = sQ[r * LD + EE * p + j];
    d[j] = sO[r * LD + EE * p + j];
  }
  float dot = 0.f;
#pragma unroll
  for (int j = 0; j < EE; ++j) dot += u[j] * d[j];
  dot = sum_parts<NP>(dot);
  if (t < a.T) {
    const float s = rs.iq[r];
    float *dst = a.dq + (row0 + (size_t)r * a.H) * D + EE * p;
#pragma unroll
    for (int j = 0; j < EE; j += 4)
      *reinterpret_cast<f4 *>(dst + j) = f4{s * (d[j] - u[j] * dot), s * (d[j + 1] - u[j + 1] * dot),
                                            s * (d[j + 2] - u[j + 2] * dot), s * (d[j + 3] - u[j + 3] * dot)};
  }
  // key of row r: k_{t-1+align}; under the prefix pairing the row at t == T
  // carries k_{T-1}, whose gradient is 0 (that row's dX is 0; rs.ik is 0 there).
  const int kt = t - 1 + a.align;
  const bool key_row = kt >= 0 && kt < a.T && t <= a.T - a.align;
#pragma unroll
  for (int j = 0; j < EE; ++j) {
    u[j] = sX[r * LD + EE * p + j];
    d[j] = sE[r * LD + EE * p + j];
  }
  dot = 0.f;
#pragma unroll
  for (int j = 0; j < EE; ++j) dot += u[j] * d[j];
  dot = sum_parts<NP>(dot);
  if (key_row) {
    const float s = rs.ik[r];
    float *dst = a.dk + ((size_t)(b * a.T + kt) * a.H + h) * D + EE * p;
#pragma unroll
    for (int j = 0; j < EE; j += 4)
      *reinterpret_cast<f4 *>(dst + j) = f4{s * (d[j] - u[j] * dot), s * (d[j + 1] - u[j + 1] * dot),
                                            s * (d[j + 2] - u[j + 2] * dot), s * (d[j + 3] - u[j + 3] * dot)};
  }
  if (t == 0 && a.dxprev0) {  // the carried x_prev is row 0's key (prefix); unread under same-step pairs
    float *dst = a.dxprev0 + (size_t)n * D + EE * p;
#pragma unroll
    for (int j = 0; j < EE; ++j) dst[j] = a.align ? 0.f : d[j];
  }
  // Prefix pairing with T a multiple of C: k_{T-1} has no row here; its gradient is 0.
  if (!a.align && c == a.NC - 1 && a.T % C == 0 && r == 0) {
    float *dst = a.dk + ((size_t)(b * a.T + a.T - 1) * a.H + h) * D + EE * p;
#pragma unroll
    for (int j = 0; j < EE; j += 4) *reinterpret_cast<f4 *>(dst + j) = zero4();
  }
}

template <typename IT, bool ADD, bool PC = false>   // PC: Falcon-2A (ADD, per-channel gains)
__global__ __launch_bounds__(NTC) void bwd_chunk(BwdArgs a) {
  constexpr bool BF = std::is_same_v<IT, __bf16>;   // bf16 inputs: products on bf16 MFMA
  __shared__ __attribute__((aligned(16))) float sX[MAT], sQ[MAT], sS[MAT], sG[MAT], sA[ADD ? 4 : MAT], sP[MAT],
      sE[MAT], sO[MAT];
  __shared__ RowScalars rs;
  __shared__ float pL[NWC][C], pE[NWC][C], pC[NWC], sCoef[C];
  const int n = blockIdx.x / a.NC, c = blockIdx.x % a.NC;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int ct = w & 3, rt = w >> 2;  // this wave's tile of the C x 64 matrices
  const int b = n / a.H, h = n % a.H;
  const int live = min(C, a.T - c * C);
  const size_t row0 = (size_t)(b * a.T + c * C) * a.H + h;  // (b, t0, h)
  const WsPtr ws = ws_of(a, blockIdx.x);

  // Phase 0: the rows, do, the incoming state S0, the end-state gradient G and v.
  // Every global read is issued before the first is used, so they share one
  // round trip.
  Rows<NTC> rows;
  fetch_rows<IT, NTC>(a, n, c, rows);
  f4 V, Vraw, Bch;   // Falcon-2A: the value beta (.) v, and v and beta themselves
  {
    RowShare<NTC> rO;
    rO.load((const IT *)a.dO + row0 * D, (size_t)a.H * D, live);
    const float *S0 = c ? a.chunk_states + ((size_t)n * a.cs_nc + (size_t)c * (C / a.cs_step) - 1) * D * D
                        : (a.S0 ? a.S0 + (size_t)n * D * D : nullptr);
    const int r = tid >> 4, p = tid & 15;
    const f4 s0v = S0 ? *reinterpret_cast<const f4 *>(S0 + r * D + 4 * p) : zero4();
    const f4 gv = *reinterpret_cast<const f4 *>(ws.G + r * D + 4 * p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      const size_t e = (row0 + (size_t)row * a.H) * D + 16 * ct + cc;
      Vraw[i] = row < live ? (float)((const IT *)a.v)[e] : 0.f;
      Bch[i] = (PC && row < live) ? a.beta[e] : 0.f;
      V[i] = PC ? Bch[i] * Vraw[i] : Vraw[i];
    }
    *reinterpret_cast<f4 *>(sS + r * LD + 4 * p) = s0v;
    *reinterpret_cast<f4 *>(sG + r * LD + 4 * p) = gv;
    rO.store(sO);
    pL[w][lane] = 0.f;
    pE[w][lane] = 0.f;
  }
  stage_rows<NTC, PC>(a, c, rows, sX, sQ, rs);  // ends with a barrier
  const float LC = rs.L[C - 1];
  float lc = 0.f;  // this lane's share of dL_C
  {
    const int r = tid >> 4, p = tid & 15;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += sG[r * LD + 4 * p + j] * sS[r * LD + 4 * p + j];
    lc += __expf(LC) * s;  // e^{L_C} <G, S0>
  }

  // Phase 1: A and P tiles; R = V - diag(e^Lm) X S0^T; dQh from the first read term; Y = X G^T.
  if (w < 10) {
    int tr, tc;
    lower_tile(w, tr, tc);
    gram_tile<ADD, BF>(sX, sQ, sA, sP, rs, tr, tc, lane);
  }
  f4 E, dQ, Y;
  {
    f4 xs = zero4(), dq = zero4(), y = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f4 xa = a_rm(sX, LD, 16 * rt, 16 * kb, lane);
      if (!ADD) mmx<BF>(xs, xa, b_tr(sS, LD, 16 * kb, 16 * ct, lane));
      mmx<BF>(y, xa, b_tr(sG, LD, 16 * kb, 16 * ct, lane));
      mmx<BF>(dq, a_rm(sO, LD, 16 * rt, 16 * kb, lane), b_rm(sS, LD, 16 * kb, 16 * ct, lane));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      E[i] = ADD ? V[i] : V[i] - __expf(rs.Lm[row]) * xs[i];
      dQ[i] = __expf(rs.L[row]) * dq[i];
      const float part = sum16(sQ[row * LD + 16 * ct + cc] * dQ[i]);  // qh_i . dQh_i
      if (cc == 0) pL[w][row] += part;
    }
    Y = y;
  }

  // Phase 2-3: E = M^-1 R on the solver waves (one per column tile).
  st_c(sE, LD, 16 * rt, 16 * ct, lane, E);  // R (F1A: E = V)
  __syncthreads();  // A, P and R are complete
  if (!ADD) {
    if (w < 4) {
      f4 y4[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) y4[bb] = b_rm(sE, LD, 16 * bb, 16 * w, lane);
      solve_lower<BF>(y4, sA, rs, lane);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) st_c(sE, LD, 16 * bb, 16 * w, lane, y4[bb]);
    }
    __syncthreads();
    E = b_rm(sE, LD, 16 * rt, 16 * ct, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // db_i = E_i . (G x_i): into d eta_i, dL_i and dL_C
    const int row = 16 * rt + 4 * g + i;
    const float db = sum16(E[i] * Y[i]);
    const float f = __expf(LC - rs.L[row]);
    if (cc == 0) {
      pE[w][row] += db * f;
      pL[w][row] -= db * rs.eta[row] * f;
      lc += db * rs.eta[row] * f;
    }
  }

  // Phase 4: Z = P^T do; dE = diag(b) Y + diag(eta) Z; dX = diag(b) E G.
  f4 dE, dX;
  {
    f4 z = zero4(), u = zero4();
    for (int kb = rt; kb < 4; ++kb) mmx<BF>(z, a_tr(sP, LD, 16 * rt, 16 * kb, lane), b_rm(sO, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mmx<BF>(u, a_rm(sE, LD, 16 * rt, 16 * kb, lane), b_rm(sG, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      const float bb = rs.eta[row] * __expf(LC - rs.L[row]);
      dE[i] = bb * Y[i] + rs.eta[row] * z[i];
      dX[i] = bb * u[i];
      const float de = sum16(z[i] * E[i]);
      if (cc == 0) pE[w][row] += de;
    }
  }

  // Phase 5: dR = M^-T dE (= dv) on the solver waves; F1A: dv = dE.
  if (!ADD) {
    __syncthreads();  // every wave is done reading G
    st_c(sG, LD, 16 * rt, 16 * ct, lane, dE);
    __syncthreads();
    if (w < 4) {
      f4 y4[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) y4[bb] = b_rm(sG, LD, 16 * bb, 16 * w, lane);
      solve_upper<BF>(y4, sA, rs, lane);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) st_c(sG, LD, 16 * bb, 16 * w, lane, y4[bb]);  // sG now holds dR
    }
    __syncthreads();
    dE = b_rm(sG, LD, 16 * rt, 16 * ct, lane);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    const size_t e = (row0 + (size_t)row * a.H) * D + 16 * ct + cc;
    if (row < live) {
      a.dv[e] = PC ? Bch[i] * dE[i] : dE[i];
      if (PC) a.dbeta[e] = Vraw[i] * dE[i];   // per-channel gains: d beta = v (.) dE
    }
  }

  // Phase 6: dR S0 (into dX and dL_{i-1}); the C x C adjoints.
  if (!ADD) {
    f4 s = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mmx<BF>(s, a_rm(sG, LD, 16 * rt, 16 * kb, lane), b_rm(sS, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      const float am = __expf(rs.Lm[row]);
      dX[i] -= am * s[i];
      const float part = sum16(sX[row * LD + 16 * ct + cc] * s[i]);
      if (cc == 0 && row > 0) pL[w][row - 1] -= am * part;
    }
  }
  if (w < 10) {
    int tr, tc;
    lower_tile(w, tr, tc);
    adjoint_tile<ADD, BF>(sA, sP, sG, sO, sE, rs, pL[w], pE[w], tr, tc, lane);
  }
  __syncthreads();

  // Phase 7: dQh += dPD X; dX += dPD^T Qh + dAG X + dAG^T X.
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f4 xb = b_rm(sX, LD, 16 * kb, 16 * ct, lane);
    if (kb <= rt) {
      mmx<BF>(dQ, a_rm(sP, LD, 16 * rt, 16 * kb, lane), xb);
      if (!ADD) mmx<BF>(dX, a_rm(sA, LD, 16 * rt, 16 * kb, lane), xb);
    }
    if (kb >= rt) {
      mmx<BF>(dX, a_tr(sP, LD, 16 * rt, 16 * kb, lane), b_rm(sQ, LD, 16 * kb, 16 * ct, lane));
      if (!ADD) mmx<BF>(dX, a_tr(sA, LD, 16 * rt, 16 * kb, lane), xb);
    }
  }
  lc = sum64(lc);
  if (lane == 0) pC[w] = lc;
  __syncthreads();

  // Phase 8: per-row totals; dL -> d(log-decay) by a reverse sum; beta and the |x|^2 term.
  if (w == 0) {
    const int i = lane;
    float de = 0.f, dl = 0.f;
#pragma unroll
    for (int v = 0; v < NWC; ++v) {
      de += pE[v][i];
      dl += pL[v][i];
    }
    if (i == C - 1) {
#pragma unroll
      for (int v = 0; v < NWC; ++v) dl += pC[v];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(dl, o);
      if (i + o < 64) dl += y;
    }
    if (i < live) {
      const size_t gi = row0 + (size_t)i * a.H;
      if (!PC) a.dbeta[gi] = de / rs.en[i];   // Falcon-2A writes its per-channel d beta above
      a.dg[gi] = a.g[gi] > a.log_eps_gamma ? dl : 0.f;
    }
    sCoef[i] = -2.f * de * rs.eta[i] / rs.en[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    dX[i] += sCoef[row] * sX[row * LD + 16 * ct + cc];
  }
  st_c(sO, LD, 16 * rt, 16 * ct, lane, dQ);
  st_c(sE, LD, 16 * rt, 16 * ct, lane, dX);
  __syncthreads();

  through_phi(a, n, c, row0, b, h, sO, sE, sX, sQ, rs);
}

// ================= Falcon-2: per-value-channel steps =================
// Falcon-2 gives every value channel (row of S) its own step eta_ch, so each
// channel has its own chunk matrix M_ch = I + A diag(eta_ch) ([P1] Falcon家族;
// the per-channel solve the forward pass also runs).  With F = eta (.) E and
// c_i = e^{L_C - L_i}, the chunk's adjoint is
//   Y = X G^T, Z = P^T do, dF = diag(c) Y + Z, dE = eta (.) dF,
//   dR[:, ch] = M_ch^-T dE[:, ch]                 (a per-channel transposed solve)
//   d eta = E (.) (dF - A^T dR),  dA = -strict-tril(dR F^T),  dP = tril(do F^T),
//   dv = dR,  G0 = e^{L_C} G + do^T diag(e^L) Qh - dR^T diag(e^{Lm}) X,
// the same as Falcon-1 with the solves per channel and F in place of diag(eta) E.
// In the reverse recurrence dR splits into M^-T (eta (.) diag(c) X G^T), which
// needs G and is solved inside the scan, and M^-T (eta (.) Z), which does not:
// the prep kernel folds it into Zc = do^T diag(e^L) Qh - (e^{Lm} (.) M^-T(eta (.) Z))^T X.

// Workspace arrays of one chunk (Falcon-2).
struct WsF2 {
  float *X, *A, *Zc, *G, *ETA, *RV, *dec;
};
__device__ __forceinline__ WsF2 ws_f2(const BwdArgs &a, size_t chunk_id) {
  const size_t nch = (size_t)a.B * a.H * a.NC;
  float *base = a.ws;
  WsF2 p;
  p.X = base + chunk_id * C * D;
  p.A = base + nch * C * D + chunk_id * C * C;
  p.Zc = base + nch * (C * D + C * C) + chunk_id * D * D;
  p.G = base + nch * (C * D + C * C + D * D) + chunk_id * D * D;
  p.ETA = base + nch * (C * D + C * C + 2 * D * D) + chunk_id * C * D;
  p.RV = base + nch * (2 * C * D + C * C + 2 * D * D) + chunk_id * 2 * C;   // c_i, e^{Lm_i}
  p.dec = base + nch * (2 * C * D + C * C + 2 * D * D + 2 * C) + chunk_id;
  return p;
}

constexpr int SP = 17;                 // pitch of the scan's C x 16 arrays (one 16-channel slice)

// Y <- M_ch^-1 Y for the 16 channels of one wave (forward substitution).
template <bool BF>
__device__ void solve_lower_pc(f4 (&y)[4], const f4 (&et)[4], const float *sA, int lane) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f4 s = zero4();
#pragma unroll
    for (int bp = 0; bp < b; ++bp) mmx<BF>(s, a_rm(sA, LD, 16 * b, 16 * bp, lane), et[bp] * y[bp]);
    y[b] = pc_diag<false, BF>(y[b] - s, et[b], sA, b, lane);
  }
}

// Y <- M_ch^-T Y for the 16 channels of one wave (backward substitution).
template <bool BF>
__device__ void solve_upper_pc(f4 (&y)[4], const f4 (&et)[4], const float *sA, int lane) {
#pragma unroll
  for (int b = 3; b >= 0; --b) {
    f4 s = zero4();
#pragma unroll
    for (int bp = b + 1; bp < 4; ++bp) mmx<BF>(s, a_tr(sA, LD, 16 * b, 16 * bp, lane), y[bp]);
    y[b] = pc_diag<true, BF>(y[b] - et[b] * s, et[b], sA, b, lane);
  }
}

// Gains beta[t][ch] of the C-layout tile (rows 16rt + 4g + i, channels 16ct + c);
// zero past the sequence.  steps_of turns them into eta = beta / (eps_eta + |x|^2).
__device__ __forceinline__ f4 beta_tile(const BwdArgs &a, size_t row0, int live, int rt, int ct, int lane) {
  const int g = lane >> 4, cc = lane & 15;
  f4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    e[i] = row < live ? a.beta[(row0 + (size_t)row * a.H) * D + 16 * ct + cc] : 0.f;
  }
  return e;
}
__device__ __forceinline__ f4 steps_of(const f4 &beta, const RowScalars &rs, int rt, int lane) {
  const float *er = rs.eta + 16 * rt + 4 * (lane >> 4);
  return f4{beta[0] * er[0], beta[1] * er[1], beta[2] * er[2], beta[3] * er[3]};
}

// Steps eta[i][ch] = beta[t][ch] / (eps_eta + |x_i|^2) of the C-layout tile
// (rows 16rt + 4g + i, channels 16ct + c); zero past the sequence.
__device__ __forceinline__ f4 eta_tile(const BwdArgs &a, size_t row0, int live, const RowScalars &rs, int rt, int ct,
                                       int lane) {
  const int g = lane >> 4, cc = lane & 15;
  f4 e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    e[i] = row < live ? a.beta[(row0 + (size_t)row * a.H) * D + 16 * ct + cc] * rs.eta[row] : 0.f;
  }
  return e;
}

// ---- bwd_prep_f2 ------------------------------------------------------------------
// 256 threads; wave w takes value channels 16w..16w+15 for the solve and key
// columns 16w..16w+15 for Zc.  Writes X, A, Zc, eta, (c, e^{Lm}) and e^{L_C}.
template <typename IT>
__global__ __launch_bounds__(256) void bwd_prep_f2(BwdArgs a) {
  constexpr bool BF = std::is_same_v<IT, __bf16>;   // bf16 inputs: products on bf16 MFMA
  // LDS: X, Qh (then do), A and P (then D): 70.7 KB, two workgroups per compute unit
  __shared__ __attribute__((aligned(16))) float sX[MAT], sQ[MAT], sA[MAT], sP[MAT];
  float *const sD = sP;
  __shared__ RowScalars rs;
  const int n = blockIdx.x / a.NC, c = blockIdx.x % a.NC;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
  const int b = n / a.H, h = n % a.H;
  const int live = min(C, a.T - c * C);
  const size_t row0 = (size_t)(b * a.T + c * C) * a.H + h;
  RowShare<256> dO;
  dO.load((const IT *)a.dO + row0 * D, (size_t)a.H * D, live);
  load_rows<IT, 256, true>(a, n, c, sX, sQ, rs);  // rs.eta = 1 / (eps_eta + |x|^2); ends with a barrier
  const WsF2 ws = ws_f2(a, blockIdx.x);
  const float LC = rs.L[C - 1];

  f4 qe[4];  // diag(e^L) Qh, key column tile w
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    qe[rt] = b_rm(sQ, LD, 16 * rt, 16 * w, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) qe[rt][i] *= __expf(rs.L[16 * rt + 4 * g + i]);
  }
  for (int k = w; k < 10; k += 4) {
    int rt, ct;
    lower_tile(k, rt, ct);
    gram_tile<false, BF>(sX, sQ, sA, sP, rs, rt, ct, lane);
  }
  __syncthreads();  // A, P complete; sQ is read: it takes do from here on
  dO.store(sQ);
  __syncthreads();
  // B = eta (.) P^T do for value channels 16w.., then M^-T B per channel
  f4 y[4], et[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f4 z = zero4();
    for (int kb = rt; kb < 4; ++kb) mmx<BF>(z, a_tr(sP, LD, 16 * rt, 16 * kb, lane), b_rm(sQ, LD, 16 * kb, 16 * w, lane));
    et[rt] = eta_tile(a, row0, live, rs, rt, w, lane);
    y[rt] = et[rt] * z;
  }
  solve_upper_pc<BF>(y, et, sA, lane);
  __syncthreads();  // every wave is done reading P: D takes its place
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f4 d = y[rt];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] *= __expf(rs.Lm[16 * rt + 4 * g + i]);
    st_c(sD, LD, 16 * rt, 16 * w, lane, d);   // e^{Lm} (.) M^-T (eta (.) Z)
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.ETA[(16 * rt + 4 * g + i) * D + 16 * w + cc] = et[rt][i];
  }
  __syncthreads();
  // Zc = do^T diag(e^L) Qh - D^T X: value-channel rows, key-column tile w
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f4 z = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      mmx<BF>(z, a_tr(sQ, LD, 16 * rt, 16 * kb, lane), qe[kb]);
      mmx<BF>(z, -a_tr(sD, LD, 16 * rt, 16 * kb, lane), b_rm(sX, LD, 16 * kb, 16 * w, lane));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.Zc[(16 * rt + 4 * g + i) * D + 16 * w + cc] = z[i];
  }
  {
    const int r = threadIdx.x >> 2, p = threadIdx.x & 3;
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      *reinterpret_cast<f4 *>(ws.X + r * D + 16 * p + j) = *reinterpret_cast<const f4 *>(sX + r * LD + 16 * p + j);
      *reinterpret_cast<f4 *>(ws.A + r * C + 16 * p + j) = *reinterpret_cast<const f4 *>(sA + r * LD + 16 * p + j);
    }
  }
  if (threadIdx.x < C) {
    const int i = threadIdx.x;
    ws.RV[i] = __expf(LC - rs.L[i]);
    ws.RV[C + i] = __expf(rs.Lm[i]);
  }
  if (threadIdx.x == 0) *ws.dec = __expf(LC);
}

// ---- bwd_scan_f2 -------------------------------------------------------------------
// Workgroup (sequence n, value rows 16s..16s+15), chunks in reverse; wave w holds
// key columns 16w..16w+15 of G.  Per chunk: Y^T = G X^T, B = eta (.) c (.) Y, the
// per-channel solve dR = M^-T B on wave 0, then G <- e^{L_C} G - (e^{Lm} (.) dR)^T X + Zc.
// The next chunk's X, A, steps, row factors and Zc are fetched into registers
// while the current chunk is reduced.  G and its two products stay on fp32 MFMA;
// BF (bf16 inputs) puts the solve's coupling sweeps on bf16 MFMA, as in bwd_chunk_f2.
template <bool BF>
__global__ __launch_bounds__(256) void bwd_scan_f2(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sX[MAT], sA[MAT], sG[16 * LD], sB[C * SP], sE[C * SP];
  __shared__ float sRV[2 * C];
  const int n = blockIdx.x >> 2, s = blockIdx.x & 3;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, cc = lane & 15;
  const int tid = threadIdx.x, r = tid >> 2, p = tid & 3;
  const size_t tile = (size_t)(16 * s + 4 * g) * D + 16 * w + cc;  // + i * D
  f4 G = zero4();
  if (a.dST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) G[i] = a.dST[(size_t)n * D * D + tile + i * D];
  }
  f4 nx[4], na[4], nz;
  float ne[4], nrv, ndec;
  auto fetch = [&](int c) {
    const WsF2 ws = ws_f2(a, (size_t)n * a.NC + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      nx[j] = *reinterpret_cast<const f4 *>(ws.X + r * D + 16 * p + 4 * j);
      na[j] = *reinterpret_cast<const f4 *>(ws.A + r * C + 16 * p + 4 * j);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;   // C x 16 steps of this slice's channels
      ne[j] = ws.ETA[(e >> 4) * D + 16 * s + (e & 15)];
    }
    nrv = tid < 2 * C ? ws.RV[tid] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) nz[i] = ws.Zc[tile + i * D];
    ndec = *ws.dec;
  };
  fetch(a.NC - 1);
  for (int c = a.NC - 1; c >= 0; --c) {
    const WsF2 ws = ws_f2(a, (size_t)n * a.NC + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) ws.G[tile + i * D] = G[i];  // gradient at the end of chunk c
    __syncthreads();  // the previous chunk's readers are done
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *reinterpret_cast<f4 *>(sX + r * LD + 16 * p + 4 * j) = nx[j];
      *reinterpret_cast<f4 *>(sA + r * LD + 16 * p + 4 * j) = na[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j;
      sE[(e >> 4) * SP + (e & 15)] = ne[j];
    }
    if (tid < 2 * C) sRV[tid] = nrv;
    const f4 Zc = nz;
    const float dec = ndec;
    st_c(sG, LD, 0, 16 * w, lane, G);
    __syncthreads();
    if (c > 0) fetch(c - 1);   // in flight during this chunk's products
    {  // (G X^T) tile: channels 16s.., chunk rows 16w..; B = eta (.) c (.) Y into sB [row][channel]
      f4 y = zero4();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) mma16(y, a_rm(sG, LD, 0, 16 * kb, lane), b_tr(sX, LD, 16 * kb, 16 * w, lane));
      const int row = 16 * w + cc;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 4 * g + i;
        sB[row * SP + ch] = sE[row * SP + ch] * sRV[row] * y[i];
      }
    }
    __syncthreads();
    if (w == 0) {  // dR = M^-T B for the 16 channels; e^{Lm} (.) dR back into sB
      f4 yy[4], et[4];
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        yy[bb] = b_rm(sB, SP, 16 * bb, 0, lane);
        et[bb] = b_rm(sE, SP, 16 * bb, 0, lane);
      }
      solve_upper_pc<BF>(yy, et, sA, lane);
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) yy[bb][i] *= sRV[C + 16 * bb + 4 * g + i];
        st_c(sB, SP, 16 * bb, 0, lane, yy[bb]);
      }
    }
    __syncthreads();
    f4 u = zero4();  // (e^{Lm} (.) dR)^T X: channels 16s.., key columns 16w..
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mma16(u, a_tr(sB, SP, 0, 16 * kb, lane), b_rm(sX, LD, 16 * kb, 16 * w, lane));
    G = dec * G - u + Zc;
  }
  if (a.dS0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a.dS0[(size_t)n * D * D + tile + i * D] = G[i];
  }
}

// ---- bwd_chunk_f2 ------------------------------------------------------------------
// 16 waves, wave w owns tile (rt, ct) = (w / 4, w % 4) of every C x 64 matrix; the
// per-channel solves run on waves 0..3 (one 16-channel column tile each).
template <typename IT>
__global__ __launch_bounds__(NTC) void bwd_chunk_f2(BwdArgs a) {
  constexpr bool BF = std::is_same_v<IT, __bf16>;   // bf16 inputs: products on bf16 MFMA
  __shared__ __attribute__((aligned(16))) float sX[MAT], sQ[MAT], sS[MAT], sG[MAT], sA[MAT], sP[MAT], sE[MAT],
      sO[MAT];
  __shared__ RowScalars rs;
  __shared__ float pL[NWC][C], pE[NWC][C], pC[NWC], sCoef[C];
  const int n = blockIdx.x / a.NC, c = blockIdx.x % a.NC;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, cc = lane & 15;
  const int ct = w & 3, rt = w >> 2;
  const int b = n / a.H, h = n % a.H;
  const int live = min(C, a.T - c * C);
  const size_t row0 = (size_t)(b * a.T + c * C) * a.H + h;
  const WsF2 ws = ws_f2(a, blockIdx.x);

  // Phase 0: the rows, the gains, do, the incoming state S0, the end-state
  // gradient G and v.  Every global read is issued before the first is used.
  Rows<NTC> R;
  fetch_rows<IT, NTC>(a, n, c, R);
  f4 ET = beta_tile(a, row0, live, rt, ct, lane);   // this tile's gains (steps below)
  f4 e4[4];   // solver waves: the gains, then the steps, of their column tile
  if (w < 4) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) e4[bb] = beta_tile(a, row0, live, bb, w, lane);
  }
  f4 V;
  {
    RowShare<NTC> rO;
    rO.load((const IT *)a.dO + row0 * D, (size_t)a.H * D, live);
    const float *S0 = c ? a.chunk_states + ((size_t)n * a.cs_nc + (size_t)c * (C / a.cs_step) - 1) * D * D
                        : (a.S0 ? a.S0 + (size_t)n * D * D : nullptr);
    const int r = tid >> 4, p = tid & 15;
    const f4 s0v = S0 ? *reinterpret_cast<const f4 *>(S0 + r * D + 4 * p) : zero4();
    const f4 gv = *reinterpret_cast<const f4 *>(ws.G + r * D + 4 * p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      V[i] = row < live ? (float)((const IT *)a.v)[(row0 + (size_t)row * a.H) * D + 16 * ct + cc] : 0.f;
    }
    *reinterpret_cast<f4 *>(sS + r * LD + 4 * p) = s0v;
    *reinterpret_cast<f4 *>(sG + r * LD + 4 * p) = gv;
    rO.store(sO);
    pL[w][lane] = 0.f;
    pE[w][lane] = 0.f;
  }
  stage_rows<NTC, true>(a, c, R, sX, sQ, rs);  // rs.eta = 1 / (eps_eta + |x|^2); ends with a barrier
  ET = steps_of(ET, rs, rt, lane);
  if (w < 4) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) e4[bb] = steps_of(e4[bb], rs, bb, lane);
  }
  const float LC = rs.L[C - 1];
  float lc = 0.f;
  {
    const int r = tid >> 4, p = tid & 15;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += sG[r * LD + 4 * p + j] * sS[r * LD + 4 * p + j];
    lc += __expf(LC) * s;  // e^{L_C} <G, S0>
  }

  // Phase 1: A and P tiles; R = V - diag(e^Lm) X S0^T; dQh from the first read term; Y = X G^T.
  if (w < 10) {
    int tr, tc;
    lower_tile(w, tr, tc);
    gram_tile<false, BF>(sX, sQ, sA, sP, rs, tr, tc, lane);
  }
  f4 E, dQ, Y;
  {
    f4 xs = zero4(), dq = zero4(), y = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f4 xa = a_rm(sX, LD, 16 * rt, 16 * kb, lane);
      mmx<BF>(xs, xa, b_tr(sS, LD, 16 * kb, 16 * ct, lane));
      mmx<BF>(y, xa, b_tr(sG, LD, 16 * kb, 16 * ct, lane));
      mmx<BF>(dq, a_rm(sO, LD, 16 * rt, 16 * kb, lane), b_rm(sS, LD, 16 * kb, 16 * ct, lane));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      E[i] = V[i] - __expf(rs.Lm[row]) * xs[i];
      dQ[i] = __expf(rs.L[row]) * dq[i];
      const float part = sum16(sQ[row * LD + 16 * ct + cc] * dQ[i]);  // qh_i . dQh_i
      if (cc == 0) pL[w][row] += part;
    }
    Y = y;
  }

  // Phase 2-3: E[:, ch] = M_ch^-1 R[:, ch] on waves 0..3 (one per column tile).
  st_c(sE, LD, 16 * rt, 16 * ct, lane, E);  // R
  __syncthreads();                           // A, P and R are complete
  if (w < 4) {
    f4 y4[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) y4[bb] = b_rm(sE, LD, 16 * bb, 16 * w, lane);
    solve_lower_pc<BF>(y4, e4, sA, lane);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) st_c(sE, LD, 16 * bb, 16 * w, lane, y4[bb]);
  }
  __syncthreads();
  E = b_rm(sE, LD, 16 * rt, 16 * ct, lane);
  const f4 F = ET * E;   // eta (.) E

  // Phase 4: Z = P^T do; dF = c (.) Y + Z; d eta = E (.) dF; dE = eta (.) dF; dX = c (.) F G.
  f4 dE, dX, deta;
  {
    f4 z = zero4();
    for (int kb = rt; kb < 4; ++kb) mmx<BF>(z, a_tr(sP, LD, 16 * rt, 16 * kb, lane), b_rm(sO, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      const float cf = __expf(LC - rs.L[row]);
      const float fy = F[i] * Y[i] * cf;   // the c_i term of S_C: into dL_i and dL_C
      const float part = sum16(fy);
      if (cc == 0) {
        pL[w][row] -= part;
        lc += part;
      }
      const float dF = cf * Y[i] + z[i];
      deta[i] = E[i] * dF;
      dE[i] = ET[i] * dF;
    }
  }
  __syncthreads();                           // every wave has read E from sE
  st_c(sE, LD, 16 * rt, 16 * ct, lane, F);   // sE holds F from here on
  __syncthreads();
  {
    f4 u = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mmx<BF>(u, a_rm(sE, LD, 16 * rt, 16 * kb, lane), b_rm(sG, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) dX[i] = __expf(LC - rs.L[16 * rt + 4 * g + i]) * u[i];
  }

  // Phase 5: dR = M_ch^-T dE on waves 0..3 (= dv).
  __syncthreads();  // every wave is done reading G
  st_c(sG, LD, 16 * rt, 16 * ct, lane, dE);
  __syncthreads();
  if (w < 4) {
    f4 y4[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) y4[bb] = b_rm(sG, LD, 16 * bb, 16 * w, lane);
    solve_upper_pc<BF>(y4, e4, sA, lane);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) st_c(sG, LD, 16 * bb, 16 * w, lane, y4[bb]);  // sG now holds dR
  }
  __syncthreads();
  const f4 dR = b_rm(sG, LD, 16 * rt, 16 * ct, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    if (row < live) a.dv[(row0 + (size_t)row * a.H) * D + 16 * ct + cc] = dR[i];
  }

  // Phase 6: dR S0 (into dX and dL_{i-1}); d eta -= E (.) A^T dR; the C x C adjoints.
  {
    f4 s = zero4(), t2 = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) mmx<BF>(s, a_rm(sG, LD, 16 * rt, 16 * kb, lane), b_rm(sS, LD, 16 * kb, 16 * ct, lane));
    for (int kb = rt; kb < 4; ++kb) mmx<BF>(t2, a_tr(sA, LD, 16 * rt, 16 * kb, lane), b_rm(sG, LD, 16 * kb, 16 * ct, lane));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      const float am = __expf(rs.Lm[row]);
      dX[i] -= am * s[i];
      const float part = sum16(sX[row * LD + 16 * ct + cc] * s[i]);
      if (cc == 0 && row > 0) pL[w][row - 1] -= am * part;
      deta[i] -= E[i] * t2[i];
    }
  }
  __syncthreads();  // every wave has read A (A^T dR): the adjoint tiles overwrite it
  if (w < 10) {   // dA = -strict-tril(dR F^T), dP = tril(do F^T), with their decays
    int tr, tc;
    lower_tile(w, tr, tc);
    const int tg = lane >> 4, tcc = lane & 15;
    f4 t = zero4(), u = zero4();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const f4 fb = b_tr(sE, LD, 16 * kb, 16 * tc, lane);
      mmx<BF>(t, a_rm(sG, LD, 16 * tr, 16 * kb, lane), fb);
      mmx<BF>(u, a_rm(sO, LD, 16 * tr, 16 * kb, lane), fb);
    }
    const int col = 16 * tc + tcc;
    float colL = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tr + 4 * tg + i;
      float rowL = 0.f, rowLm = 0.f;
      const float Aij = sA[row * LD + col];
      const float dA = col < row ? -t[i] : 0.f;
      const float H = dA * Aij;
      rowLm += H;
      colL -= H;
      sA[row * LD + col] = col < row ? dA * __expf(rs.Lm[row] - rs.L[col]) : 0.f;
      const float dP = col <= row ? u[i] : 0.f;
      const float HP = dP * sP[row * LD + col];
      rowL += HP;
      colL -= HP;
      sP[row * LD + col] = col <= row ? dP * __expf(rs.L[row] - rs.L[col]) : 0.f;
      rowL = sum16(rowL);
      rowLm = sum16(rowLm);
      if (tcc == 0) {
        pL[w][row] += rowL;
        if (row > 0) pL[w][row - 1] += rowLm;
      }
    }
    colL = sum4g(colL);
    if (tg == 0) pL[w][col] += colL;
  }
  {  // d beta = d eta / (eps + |x|^2); sum over this tile's channels of d eta (.) eta, for |x|^2
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * g + i;
      if (row < live) a.dbeta[(row0 + (size_t)row * a.H) * D + 16 * ct + cc] = deta[i] * rs.eta[row];
      const float part = sum16(deta[i] * ET[i]);
      if (cc == 0) pE[w][row] += part;
    }
  }
  __syncthreads();

  // Phase 7: dQh += dPD X; dX += dPD^T Qh + dAG X + dAG^T X.
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f4 xb = b_rm(sX, LD, 16 * kb, 16 * ct, lane);
    if (kb <= rt) {
      mmx<BF>(dQ, a_rm(sP, LD, 16 * rt, 16 * kb, lane), xb);
      mmx<BF>(dX, a_rm(sA, LD, 16 * rt, 16 * kb, lane), xb);
    }
    if (kb >= rt) {
      mmx<BF>(dX, a_tr(sP, LD, 16 * rt, 16 * kb, lane), b_rm(sQ, LD, 16 * kb, 16 * ct, lane));
      mmx<BF>(dX, a_tr(sA, LD, 16 * rt, 16 * kb, lane), xb);
    }
  }
  lc = sum64(lc);
  if (lane == 0) pC[w] = lc;
  __syncthreads();

  // Phase 8: per-row totals; dL -> d(log-decay) by a reverse sum; the |x|^2 term.
  if (w == 0) {
    const int i = lane;
    float de = 0.f, dl = 0.f;
#pragma unroll
    for (int v = 0; v < NWC; ++v) {
      de += pE[v][i];
      dl += pL[v][i];
    }
    if (i == C - 1) {
#pragma unroll
      for (int v = 0; v < NWC; ++v) dl += pC[v];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(dl, o);
      if (i + o < 64) dl += y;
    }
    if (i < live) {
      const size_t gi = row0 + (size_t)i * a.H;
      a.dg[gi] = a.g[gi] > a.log_eps_gamma ? dl : 0.f;
    }
    sCoef[i] = -2.f * de * rs.eta[i];   // -2 sum_ch d eta eta / (eps + |x|^2)
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * rt + 4 * g + i;
    dX[i] += sCoef[row] * sX[row * LD + 16 * ct + cc];
  }
  st_c(sO, LD, 16 * rt, 16 * ct, lane, dQ);
  st_c(sE, LD, 16 * rt, 16 * ct, lane, dX);
  __syncthreads();
  through_phi(a, n, c, row0, b, h, sO, sE, sX, sQ, rs);
}

template <typename IT, bool ADD, bool PC = false>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t st) {
  const unsigned nch = (unsigned)a.B * a.H * a.NC;
  hipLaunchKernelGGL((bwd_prep<IT, ADD>), dim3(nch), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ADD) hipLaunchKernelGGL(bwd_scan_add, dim3((unsigned)a.B * a.H * 4), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((bwd_scan<std::is_same_v<IT, __bf16>>), dim3((unsigned)a.B * a.H), dim3(512), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk<IT, ADD, PC>), dim3(nch), dim3(NTC), 0, st, a);
  return hipGetLastError();
}

template <typename IT>
hipError_t launch_bwd_f2(const BwdArgs &a, hipStream_t st) {
  const unsigned nch = (unsigned)a.B * a.H * a.NC;
  hipLaunchKernelGGL((bwd_prep_f2<IT>), dim3(nch), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_scan_f2<std::is_same_v<IT, __bf16>>), dim3((unsigned)a.B * a.H * 4), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chunk_f2<IT>), dim3(nch), dim3(NTC), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// The kernels work in chunks of 64 steps whatever the forward's chunk: the
// gradient does not depend on the chunking, and a forward at chunk 16 or 32
// wrote the state at every 64-step boundary among its per-chunk states.
bool chunk_bwd_supported(int variant, int dk, int dv, int chunk, int window) {
  return variant >= 1 && variant <= 4 && dk == D && dv == D && (chunk == 16 || chunk == 32 || chunk == C) &&
         window == 1;
}

size_t chunk_bwd_workspace(int variant, int B, int H, int T) {
  const size_t nch = (size_t)B * H * ((T + C - 1) / C);
  if (variant == 3)   // Falcon-2: keys, A, Zc, G, eta, (c, e^{Lm}) and the decay per chunk
    return nch * (2 * C * D + C * C + 2 * D * D + 2 * C + 1) * sizeof(float);
  return (3 * nch * D * D + nch) * sizeof(float);
}

hipError_t launch_chunk_bwd(int variant, bool bf16, const BwdArgs &a, hipStream_t st) {
  if (variant == 3) return bf16 ? launch_bwd_f2<__bf16>(a, st) : launch_bwd_f2<float>(a, st);
  if (variant == 4) return bf16 ? launch_bwd_t<__bf16, true, true>(a, st) : launch_bwd_t<float, true, true>(a, st);
  const bool add = variant == 2;
  if (bf16) return add ? launch_bwd_t<__bf16, true>(a, st) : launch_bwd_t<__bf16, false>(a, st);
  return add ? launch_bwd_t<float, true>(a, st) : launch_bwd_t<float, false>(a, st);
}

}  // namespace falcon
