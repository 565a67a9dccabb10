// Falcon-3A with a window of 2, 4 or 8 pairs, head dim 64, chunks of 64 steps:
// the banded-weight chunk form.  The window-averaged additive write is [P1]
// Falcon家族 (window average); the chunked form it rearranges is [P1] 三种等价形式
// (form C).
//
// Falcon-3A never reads S in its write, so each step adds a fixed rank-B_w term
// and S is a decayed sum of them.  Inside a chunk, with L_s the cumulative
// clamped log-decay of its steps 0..s and eta_u = beta_u / (eps_eta + |x_u|^2) / B_w,
// pair j (local index, -B_w+1 <= j <= 63; negative j are the previous chunk's last
// pairs or the carried window) is written at the steps u = max(j, 0) .. j + B_w - 1,
// so with m = min(j + B_w - 1, s)
//
//   omega(s, j) = sum_{u = max(j,0)}^{m} e^{L_s - L_u} eta_u = e^{L_s - L_m} P_j(m),
//   P_j(u) = lambda_u P_j(u - 1) + eta_u,
//
//   o_s     = e^{L_s} S_c q_s + sum_j omega(s, j) <x_j, q_s> v_j,
//   S_{c+1} = e^{L_63} S_c + U_c,   U_c = sum_j omega(63, j) v_j x_j^T.
//
// Every factor e^{L_s - L_m} has m <= s, so no weight grows without bound under
// deep decay.  Three kernels:
//   band_state  (one workgroup per chunk)     U_c and the chunk's decay e^{L_63};
//   band_scan   (four per sequence)           S_c = state entering chunk c, written
//                                             over U_c; S_T, chunk states, x_prev, window;
//   band_out    (one workgroup per chunk)     the outputs from S_c and the chunk's pairs.
// The products run on MFMA 16x16 tiles; the halo (up to 7 earlier pairs) is one
// extra block of 16 pair rows, zero above the window.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "chunk_common.h"
#include "falcon_kernels.h"

namespace falcon {
namespace {

constexpr int BD = 64;              // head dim (keys and values)
constexpr int BC = 64;              // steps per chunk
constexpr int BHALO = 16;           // pair rows ahead of the chunk's own (the window's reach, padded)
constexpr int BNR = BC + BHALO;     // pair rows held per chunk
constexpr int BNT = 256;            // threads of band_state / band_out
// per-sequence copy of the carried state: x_prev, then up to 7 window keys and 7 values
constexpr int CARRY = 1024, CX = 0, CWX = 64, CWV = 64 + 7 * 64;

template <typename IT> constexpr int band_ld() { return BD + 16 / (int)sizeof(IT); }   // 72 (bf16), 68 (fp32)

struct BandWs {
  float *U;       // [BH][NC][d*d] row-major: U_c (band_state), then S_c entering chunk c (band_scan)
  float *dec;     // [BH][NC]: e^{L_63} of chunk c
  float *carry;   // [BH][CARRY]: the call's incoming x_prev and window
};

__host__ __device__ inline size_t band_dec_floats(size_t bhnc) { return (bhnc + 63) & ~size_t(63); }

__host__ __device__ inline BandWs band_ws(void *ws, int bh, int nc) {
  float *p = static_cast<float *>(ws);
  const size_t bhnc = (size_t)bh * nc;
  return BandWs{p, p + bhnc * BD * BD, p + bhnc * BD * BD + band_dec_floats(bhnc)};
}

__device__ inline size_t row_of(const FwdArgs &a, int b, int t, int h) { return ((size_t)b * a.T + t) * a.H + h; }

// 16 consecutive elements as fp32
__device__ inline void load16(const __bf16 *p, float *o) {
  const uint4 *u = reinterpret_cast<const uint4 *>(p);
  unpack(u[0], __bf16(), o);
  unpack(u[1], __bf16(), o + 8);
}
__device__ inline void load16(const float *p, float *o) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f4 v = reinterpret_cast<const f4 *>(p)[j];
    o[4 * j] = v[0]; o[4 * j + 1] = v[1]; o[4 * j + 2] = v[2]; o[4 * j + 3] = v[3];
  }
}
__device__ inline void zero16(float *o) {
#pragma unroll
  for (int j = 0; j < 16; ++j) o[j] = 0.f;
}
// 16 values into LDS in the operand type (16-byte aligned destination)
__device__ inline void store16(__bf16 *p, const float *x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) *reinterpret_cast<bf4 *>(p + 4 * j) = to_op(f4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]}, __bf16());
}
__device__ inline void store16(float *p, const float *x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) reinterpret_cast<f4 *>(p)[j] = f4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}

// 16 elements as raw 16-byte words, converted after the loads of a phase are all issued
template <typename IT> struct Raw16 { uint4 u[sizeof(IT) * 16 / 16]; };
template <typename IT>
__device__ inline Raw16<IT> fetch16(const IT *p) {
  Raw16<IT> r;
#pragma unroll
  for (int j = 0; j < (int)(sizeof(IT) * 16 / 16); ++j) r.u[j] = reinterpret_cast<const uint4 *>(p)[j];
  return r;
}
template <typename IT>
__device__ inline void unpack16(const Raw16<IT> &r, float *o) {
  constexpr int PER = 16 / (int)sizeof(IT);
#pragma unroll
  for (int j = 0; j < (int)(sizeof(IT) * 16 / 16); ++j) unpack(r.u[j], IT(), o + PER * j);
}

// One chunk's pair rows, queries and step scalars in LDS.
template <typename IT>
struct alignas(16) BandTile {
  static constexpr int LD = band_ld<IT>();
  IT X[BNR * LD];      // keys of pairs j = row - 16 (band_out: then their values)
  float L[BC];         // cumulative clamped log-decay
  float lam[BC];       // lambda_s
  float eta[BC];       // eta_s (already divided by the window)
  float P[BNR * 8];    // P_j(m) at [row][m - j]
  float w[BNR];        // band_state: omega(63, j)
};

// Every global row a thread needs for one chunk, loaded before any is used: the
// pair rows tid / 4 and tid / 4 + 64 (keys and values), the query row tid / 4, and
// the step scalars.  Pair row r is step t = t0 + r - 16; quarter qd of each row.
template <typename IT>
struct ChunkFetch {
  Raw16<IT> k[2], v[2], q;
  float beta[2], g;
};

template <typename IT, bool QUERIES>
__device__ void fetch_chunk(ChunkFetch<IT> &f, const FwdArgs &a, int b, int h, int t0, int n) {
  const int tid = threadIdx.x, qd = tid & 3;
  const IT *K = static_cast<const IT *>(a.k), *V = static_cast<const IT *>(a.v);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 2) + 64 * i, t = t0 + r - BHALO;
    if (r >= BNR) break;   // wave-uniform
    if (t < a.T && t >= (a.align == 0 ? 1 : 0))
      f.k[i] = fetch16(K + row_of(a, b, a.align == 0 ? t - 1 : t, h) * BD + 16 * qd);
    if (t >= 0 && t < a.T) f.v[i] = fetch16(V + row_of(a, b, t, h) * BD + 16 * qd);
    if (r >= BHALO && r - BHALO < n && qd == 0) f.beta[i] = a.beta[row_of(a, b, t, h)];
  }
  if (QUERIES && (tid >> 2) < n) f.q = fetch16(static_cast<const IT *>(a.q) + row_of(a, b, t0 + (tid >> 2), h) * BD + 16 * qd);
  if (tid < n) f.g = a.g[row_of(a, b, t0 + tid, h)];
}

// Pair keys into LDS with eta and the decays.  A key is the carried window for
// t < 0, the incoming x_prev for the first step under prefix pairs, phi of a key
// row otherwise, zero outside -Hw..T-1; eta_s uses |x_s|^2 of the same key.
template <typename IT>
__device__ void keys_to_lds(BandTile<IT> &s, const ChunkFetch<IT> &f, const FwdArgs &a, int t0, int n, int Hw,
                            const float *cxp, const float *cwx) {
  const int tid = threadIdx.x, qd = tid & 3;
  const float inv_w = 1.f / (float)a.window;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 2) + 64 * i, t = t0 + r - BHALO;
    if (r >= BNR) break;   // wave-uniform
    float x[16];
    bool norm = false;
    if (t < -Hw || t >= a.T) {
      zero16(x);
    } else if (t < 0) {
      if (cwx) load16(cwx + (Hw + t) * BD + 16 * qd, x); else zero16(x);
    } else if (a.align == 0 && t == 0) {
      if (cxp) load16(cxp + 16 * qd, x); else zero16(x);
    } else {
      unpack16(f.k[i], x);
      norm = true;
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += x[j] * x[j];
    ss = group_sum<4>(ss);
    if (norm) {
      const float rs = safe_rsqrt(ss + a.eps_phi);
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] *= rs;
      ss *= rs * rs;
    }
    store16(s.X + r * BandTile<IT>::LD + 16 * qd, x);
    if (r >= BHALO && qd == 0) {
      const int st = r - BHALO;
      s.eta[st] = st < n ? f.beta[i] / (a.eps_eta + ss) * inv_w : 0.f;
    }
  }
  if (tid < 64) {
    const float lg = tid < n ? fmaxf(f.g, a.log_eps_gamma) : 0.f;
    s.L[tid] = wave_inclusive_scan(lg);
    s.lam[tid] = __expf(lg);
  }
}

// Pair row i of this thread's values as fp32 (carried window for t < 0).
template <typename IT>
__device__ void value_row(const ChunkFetch<IT> &f, int i, const FwdArgs &a, int t, int Hw, const float *cwv, float *x) {
  const int qd = threadIdx.x & 3;
  if (t < -Hw || t >= a.T) zero16(x);
  else if (t < 0) { if (cwv) load16(cwv + (Hw + t) * BD + 16 * qd, x); else zero16(x); }
  else unpack16(f.v[i], x);
}

// P_j(m) for every pair row (band_out), or only omega(n - 1, j) (band_state).
template <typename IT, bool TABLE>
__device__ void weights(BandTile<IT> &s, int n, int Hw) {
  const int r = threadIdx.x;
  if (r >= BNR) return;
  const int j = r - BHALO;
  if (j < -Hw || j >= n) {
    if (!TABLE) s.w[r] = 0.f;
    return;
  }
  const int m1 = min(j + Hw, n - 1);
  float p = 0.f;
  for (int m = max(j, 0); m <= m1; ++m) {
    p = s.lam[m] * p + s.eta[m];
    if (TABLE) s.P[r * 8 + (m - j)] = p;
  }
  if (!TABLE) s.w[r] = __expf(s.L[n - 1] - s.L[m1]) * p;
}

// ---- band_state: U_c = sum_j omega(63, j) v_j x_j^T --------------------------------
template <typename IT>
__global__ __launch_bounds__(BNT) void band_state(FwdArgs a, BandWs ws) {
  constexpr int LD = BandTile<IT>::LD;
  __shared__ BandTile<IT> s;
  __shared__ alignas(16) IT Vs[BNR * LD];   // values scaled by omega(63, j)
  const int nc = a.nchunks, seq = blockIdx.x / nc, c = blockIdx.x % nc;
  const int b = seq / a.H, h = seq % a.H, Hw = a.window - 1;
  const int t0 = c * BC, n = min(BC, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, cc = lane & 15;

  if (c == 0) {   // the carried state, for band_out and the tails (the caller may update it in place)
    float *cy = ws.carry + (size_t)seq * CARRY;
    for (int i = tid; i < BD; i += BNT) cy[CX + i] = a.xprev0 ? a.xprev0[(size_t)seq * BD + i] : 0.f;
    for (int i = tid; i < Hw * BD; i += BNT) {
      cy[CWX + i] = a.winx0 ? a.winx0[(size_t)seq * Hw * BD + i] : 0.f;
      cy[CWV + i] = a.winv0 ? a.winv0[(size_t)seq * Hw * BD + i] : 0.f;
    }
  }
  const float *cxp = a.xprev0 ? a.xprev0 + (size_t)seq * BD : nullptr;
  const float *cwx = a.winx0 ? a.winx0 + (size_t)seq * Hw * BD : nullptr;
  const float *cwv = a.winv0 ? a.winv0 + (size_t)seq * Hw * BD : nullptr;
  ChunkFetch<IT> f;
  fetch_chunk<IT, false>(f, a, b, h, t0, n);
  keys_to_lds<IT>(s, f, a, t0, n, Hw, cxp, cwx);
  __syncthreads();
  weights<IT, false>(s, n, Hw);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 2) + 64 * i;
    if (r >= BNR) break;   // wave-uniform
    float x[16];
    value_row<IT>(f, i, a, t0 + r - BHALO, Hw, cwv, x);
    const float om = s.w[r];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] *= om;
    store16(Vs + r * LD + 16 * (tid & 3), x);
  }
  __syncthreads();

  // wave w: U^T tiles of value channels 16w.. (so a lane holds four consecutive
  // key channels of one row of U), all four key-channel blocks
  f4 u[4] = {zero4(), zero4(), zero4(), zero4()};
  typename Op<IT>::frag bv[5];
#pragma unroll
  for (int q = 0; q < BNR / 16; ++q) bv[q] = ldT(Vs, LD, 16 * q, [&](int i) { return 16 * w + 4 * i; }, lane);
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    auto xa = [&](int q) { return ldT(s.X, LD, 16 * q, [&](int i) { return 16 * bb + 4 * i; }, lane); };
    mma32(u[bb], xa(0), xa(1), bv[0], bv[1]);
    mma32(u[bb], xa(2), xa(3), bv[2], bv[3]);
    mma16(u[bb], xa(4), bv[4]);
  }
  float *U = ws.U + ((size_t)seq * nc + c) * BD * BD + (16 * w + cc) * BD + 4 * g;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) *reinterpret_cast<f4 *>(U + 16 * bb) = u[bb];
  if (tid == 0) ws.dec[(size_t)seq * nc + c] = __expf(s.L[n - 1]);
}

// ---- band_scan: S_c entering every chunk, the final state and the tails ------------
template <typename IT>
__global__ __launch_bounds__(256) void band_scan(FwdArgs a, BandWs ws) {
  constexpr int PF = 8;
  const int nc = a.nchunks, seq = blockIdx.x >> 2;
  const size_t e = ((size_t)(blockIdx.x & 3) * 256 + threadIdx.x) * 4;
  const size_t base = (size_t)seq * nc;
  f4 S = a.S0 ? *reinterpret_cast<const f4 *>(a.S0 + (size_t)seq * BD * BD + e) : zero4();
  f4 u[PF];
  float dc[PF];
  auto fetch = [&](int c, int j) {   // c clamped: the ring's last loads are spare
    c = min(c, nc - 1);
    u[j] = *reinterpret_cast<const f4 *>(ws.U + (base + c) * BD * BD + e);
    dc[j] = ws.dec[base + c];
  };
  auto step = [&](int c, int j) {
    *reinterpret_cast<f4 *>(ws.U + (base + c) * BD * BD + e) = S;   // entering chunk c
    S = dc[j] * S + u[j];
    if (a.chunk_states) *reinterpret_cast<f4 *>(a.chunk_states + (base + c) * BD * BD + e) = S;
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) fetch(j, j);
  int c = 0;
  for (; c + PF <= nc; c += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      step(c + j, j);
      fetch(c + j + PF, j);
    }
  }
#pragma unroll
  for (int j = 0; j < PF - 1; ++j)
    if (c + j < nc) step(c + j, j);
  if (a.S_out) *reinterpret_cast<f4 *>(a.S_out + (size_t)seq * BD * BD + e) = S;

  // x_prev = phi(k_{T-1}) and the last Bw - 1 pairs (from the carried copy where t < 0)
  if ((blockIdx.x & 3) != 0 || !a.write_tail) return;
  const int Hw = a.window - 1, b = seq / a.H, h = seq % a.H, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const float *cy = ws.carry + (size_t)seq * CARRY;
  const IT *K = static_cast<const IT *>(a.k), *Vv = static_cast<const IT *>(a.v);
  for (int i = wv; i <= Hw; i += 4) {   // wave-uniform
    float x = 0.f, v = 0.f;
    bool norm = false;
    if (i == Hw) {
      x = to_f(K[row_of(a, b, a.T - 1, h) * BD + lane]);
      norm = true;
    } else {
      const int t = a.T - Hw + i;
      if (t < 0) {
        x = cy[CWX + (Hw + t) * BD + lane];
        v = cy[CWV + (Hw + t) * BD + lane];
      } else {
        v = to_f(Vv[row_of(a, b, t, h) * BD + lane]);
        if (a.align == 0 && t == 0) {
          x = cy[CX + lane];
        } else {
          x = to_f(K[row_of(a, b, a.align == 0 ? t - 1 : t, h) * BD + lane]);
          norm = true;
        }
      }
    }
    const float ss = group_sum<64>(x * x);
    if (norm) x *= safe_rsqrt(ss + a.eps_phi);
    if (i == Hw) {
      if (a.xprev_out) a.xprev_out[(size_t)seq * BD + lane] = x;
    } else {
      if (a.winx_out) a.winx_out[((size_t)seq * Hw + i) * BD + lane] = x;
      if (a.winv_out) a.winv_out[((size_t)seq * Hw + i) * BD + lane] = v;
    }
  }
}

// ---- band_out: o_s = e^{L_s} S_c q_s + sum_j omega(s, j) <x_j, q_s> v_j --------------
// Score tiles (pair block q, step block p), q = 0 the halo, q <= p + 1: 14 of them,
// numbered p-major from base(p) = p (p + 3) / 2.
__device__ inline int tile_p(int k) { return k >= 9 ? 3 : k >= 5 ? 2 : k >= 2 ? 1 : 0; }
constexpr int NTILE = 14;

template <typename IT>
__global__ __launch_bounds__(BNT) void band_out(FwdArgs a, BandWs ws) {
  constexpr int LD = BandTile<IT>::LD;
  using Frag = typename Op<IT>::frag;
  __shared__ BandTile<IT> s;
  __shared__ alignas(16) IT Q[BC * LD];
  __shared__ Frag Wt[NTILE * 64];   // weighted score tiles as B-operand fragments, one per lane
  const int nc = a.nchunks, seq = blockIdx.x / nc, c = blockIdx.x % nc;
  const int b = seq / a.H, h = seq % a.H, Hw = a.window - 1;
  const int t0 = c * BC, n = min(BC, a.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, cc = lane & 15, qd = tid & 3;
  const float *cy = ws.carry + (size_t)seq * CARRY;

  // wave w owns value channels 16w..16w+15: its rows of S_c, fetched first
  const float *Sc = ws.U + ((size_t)seq * nc + c) * BD * BD + (16 * w + cc) * BD + 4 * g;
  f4 sv[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) sv[kb] = *reinterpret_cast<const f4 *>(Sc + 16 * kb);

  ChunkFetch<IT> f;
  fetch_chunk<IT, true>(f, a, b, h, t0, n);
  keys_to_lds<IT>(s, f, a, t0, n, Hw, cy + CX, cy + CWX);
  {
    const int r = tid >> 2;   // query rows: one per group of four lanes
    float x[16];
    if (r < n) unpack16(f.q, x);
    else zero16(x);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += x[j] * x[j];
    const float rs = safe_rsqrt(group_sum<4>(ss) + a.eps_phi);
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] *= rs;
    store16(Q + r * LD + 16 * qd, x);
  }
  __syncthreads();
  weights<IT, true>(s, n, Hw);
  __syncthreads();

  for (int k = w; k < NTILE; k += 4) {   // wave-uniform
    const int p = tile_p(k), q = k - p * (p + 3) / 2, st = 16 * p + cc;
    f4 sc = zero4();   // <x_j, q_s> at j = 16q - 16 + 4g + i, s = st
    const IT *xr = s.X + (16 * q + cc) * LD + 4 * g, *qr = Q + st * LD + 4 * g;
#pragma unroll
    for (int kb = 0; kb < 4; kb += 2) mma32(sc, ld4(xr + 16 * kb), ld4(xr + 16 * kb + 16), ld4(qr + 16 * kb), ld4(qr + 16 * kb + 16));
    f4 wt;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * q + 4 * g + i, j = r - BHALO;
      float om = 0.f;
      if (j >= -Hw && j <= st && st < n) {
        const int m = min(j + Hw, st);
        om = __expf(s.L[st] - s.L[m]) * s.P[r * 8 + (m - j)];
      }
      wt[i] = sc[i] * om;
    }
    Wt[k * 64 + lane] = cvt<IT>(wt);
  }
  __syncthreads();
  // the keys are no longer needed: the values take their place
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = (tid >> 2) + 64 * i;
    if (r >= BNR) break;   // wave-uniform
    const int t = t0 + r - BHALO;
    if (t >= 0 && t < a.T) {   // input rows go in as they are
#pragma unroll
      for (int j = 0; j < (int)(sizeof(IT) * 16 / 16); ++j)
        reinterpret_cast<uint4 *>(s.X + r * LD + 16 * qd)[j] = f.v[i].u[j];
    } else {
      float x[16];
      value_row<IT>(f, i, a, t, Hw, cy + CWV, x);
      store16(s.X + r * LD + 16 * qd, x);
    }
  }
  __syncthreads();

  Frag vf[5];   // V^T blocks (channels 16w.., pair block q)
#pragma unroll
  for (int q = 0; q < 5; ++q) vf[q] = ldT(s.X, LD, 16 * q, [&](int i) { return 16 * w + 4 * i; }, lane);
  Frag sh[4], sl[4];   // S_c rows; bf16: high and low parts, about 16 bits of S in the product
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    sh[kb] = cvt<IT>(sv[kb]);
    if constexpr (std::is_same_v<IT, __bf16>) sl[kb] = cvt<IT>(sv[kb] - to_f4(sh[kb]));
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int st = 16 * p + cc;
    f4 o = zero4();
    const Frag *wp = Wt + (p * (p + 3) / 2) * 64 + lane;
#pragma unroll
    for (int q = 0; q + 1 <= p + 1; q += 2) mma32(o, vf[q], vf[q + 1], wp[64 * q], wp[64 * q + 64]);
    if (p % 2 == 1) mma16(o, vf[p + 1], wp[64 * (p + 1)]);   // odd count p + 2 of pair blocks: the last one
    f4 in = zero4();
    Frag qf[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) qf[kb] = ld4(Q + st * LD + 16 * kb + 4 * g);
#pragma unroll
    for (int kb = 0; kb < 4; kb += 2) {
      mma32(in, sh[kb], sh[kb + 1], qf[kb], qf[kb + 1]);
      if constexpr (std::is_same_v<IT, __bf16>) mma32(in, sl[kb], sl[kb + 1], qf[kb], qf[kb + 1]);
    }
    if (st < n) {
      o += __expf(s.L[st]) * in;
      *reinterpret_cast<Frag *>(static_cast<IT *>(a.o) + row_of(a, b, t0 + st, h) * BD + 16 * w + 4 * g) = cvt<IT>(o);
    }
  }
}

template <typename IT>
hipError_t launch_band(const FwdArgs &a, void *wsp, hipStream_t st) {
  const int bh = a.B * a.H;
  const BandWs ws = band_ws(wsp, bh, a.nchunks);
  const unsigned nb = (unsigned)bh * a.nchunks;
  hipLaunchKernelGGL(band_state<IT>, dim3(nb), dim3(BNT), 0, st, a, ws);
  hipLaunchKernelGGL(band_scan<IT>, dim3((unsigned)bh * 4), dim3(256), 0, st, a, ws);
  hipLaunchKernelGGL(band_out<IT>, dim3(nb), dim3(BNT), 0, st, a, ws);
  return hipGetLastError();
}

}  // namespace

bool chunk_fwd_band_supported(int variant, int dk, int dv, int chunk, int window) {
  return variant == V_F3A && dk == BD && dv == BD && chunk == BC && (window == 2 || window == 4 || window == 8);
}

size_t chunk_fwd_band_workspace(int bh, int T) {
  const size_t nc = (size_t)(T + BC - 1) / BC, bhnc = (size_t)bh * nc;
  return (bhnc * BD * BD + band_dec_floats(bhnc) + (size_t)bh * CARRY) * sizeof(float);
}

hipError_t launch_chunk_fwd_band(bool bf16, const FwdArgs &a, void *ws, hipStream_t st) {
  if (a.nchunks < 1 || a.cu || a.maps_only || a.reuse_images ||
      !chunk_fwd_band_supported(V_F3A, BD, BD, BC, a.window))
    return hipErrorInvalidValue;
  return bf16 ? launch_band<__bf16>(a, ws, st) : launch_band<float>(a, ws, st);
}

}  // namespace falcon
