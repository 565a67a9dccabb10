// Single-token recurrent step of Falcon fast-weight attention on gfx950
// (recurrent form: [P1] 三种等价形式 form A; [P2] 三种视角), and the small
// kernel that writes the carried key / window of a chunked call.
// ([P1] = zhouql-dev.github.io "把状态更新写成一条学习规则：Falcon 家族重新对齐
// fast-weight 记忆"; [P2] = 59188saintaubert.com "给记忆装一个“及时纠错”的开关：
// Falcon让循环模型学会边写边改".)
//
// The step is row-local: for value channel i, with x = x_prev (= phi(k_{t-1})),
// q^ = phi(q_t), lam = max(e^g, eps_gamma), eta = beta / (eps_eta + |x|^2) and the
// window pairs (x_j, v_j) (just (x, v_t) unless Falcon-3):
//   e_ij  = v_j[i] - s_i . x_j           (regression family; v_j[i] for the A variants)
//   s_i  <- lam s_i + (eta_i / Bw) sum_j e_ij x_j
//   o_i   = lam (s_i . q^) + (eta_i / Bw) sum_j e_ij (x_j . q^)    (= s_i_new . q^)
// so each row of S is read once and written once, in place: the kernel is a
// single HBM stream over the state.
#include "falcon_kernels.h"
#include "mfma_frag.h"

namespace falcon {

namespace {

enum { V_F1 = 1, V_F1A = 2, V_F2 = 3, V_F2A = 4, V_F3 = 5, V_F3A = 6 };
constexpr int MAXW = 8;

__device__ __forceinline__ float ld1(const __bf16 *p) { return (float)*p; }
__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ void st1(__bf16 *p, float x) { *p = (__bf16)x; }
__device__ __forceinline__ void st1(float *p, float x) { *p = x; }

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {  // x + x of the lane CTRL names (DPP, no LDS trip)
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Sum over the LPR (4..64) lanes of one row, in every lane of it: butterflies
// inside groups of 4, 8 and 16 lanes by DPP (quad permutations, half-row and
// row mirrors), across 16-lane rows by lane shuffles.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(LPR >= 4 && LPR <= 64 && (LPR & (LPR - 1)) == 0, "row of 4..64 lanes");
  x = dpp_add<0xB1>(x);                                // quad_perm [1,0,3,2]
  x = dpp_add<0x4E>(x);                                // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x = dpp_add<0x141>(x);       // row_half_mirror
  if constexpr (LPR >= 16) x = dpp_add<0x140>(x);      // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  if constexpr (LPR >= 64) x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float dot4(const f4 &a, const f4 &b) {
  return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}

// BW: the window size (compile time, so a window holds only the registers it uses;
// 1 for every variant but Falcon-3 / 3A).
template <int VAR, typename IT, int DK, int DV, int BW>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
  constexpr int LPR = DK / 4;          // lanes per row of S (float4 per lane)
  constexpr int RPW = 64 / LPR;        // rows per wave pass
  constexpr bool PERCH = (VAR == V_F2 || VAR == V_F2A);
  constexpr bool WIN = (VAR == V_F3 || VAR == V_F3A);
  constexpr bool DELTA = (VAR == V_F1 || VAR == V_F2 || VAR == V_F3);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int part = lane % LPR, rsub = lane / LPR;
  const int bh = blockIdx.x;
  const IT *qp = static_cast<const IT *>(a.q);
  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  IT *op = static_cast<IT *>(a.o);

  // per-sequence scalars, computed redundantly by every row group
  f4 qv, kv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    qv[e] = ld1(qp + (size_t)bh * DK + 4 * part + e);
    kv[e] = ld1(kp + (size_t)bh * DK + 4 * part + e);
  }
  const float kn = row_sum<LPR>(dot4(kv, kv));
  const f4 xk = kv * (kn + a.eps_phi > 0.f ? rsqrtf(kn + a.eps_phi) : 0.f);   // phi(k_t)
  // the key of this step's pair: the carried phi(k_{t-1}), or phi(k_t) with same-step pairs
  const f4 x = a.align ? xk : *reinterpret_cast<const f4 *>(a.xprev + (size_t)bh * DK + 4 * part);
  const float qn = row_sum<LPR>(dot4(qv, qv));
  const f4 qh = qv * (qn + a.eps_phi > 0.f ? rsqrtf(qn + a.eps_phi) : 0.f);
  const float xn2 = row_sum<LPR>(dot4(x, x));
  const float xq = row_sum<LPR>(dot4(x, qh));
  const float lam = __expf(fmaxf(a.g[bh], a.log_eps_gamma));
  const float etas = PERCH ? 0.f : a.beta[bh] / (a.eps_eta + xn2);
  const float inv_e = 1.f / (a.eps_eta + xn2);

  // Falcon-3: the window's values are staged in LDS once per sequence (one
  // coalesced read), so the per-row loop reads them without a global load whose
  // address the compiler cannot separate from the state rows it stores.
  constexpr int NW = BW > 1 ? BW - 1 : 1;   // window slots held (1 when unused)
  __shared__ float swv[NW][DV];
  if (WIN && BW > 1) {
    for (int i = tid; i < (BW - 1) * DV; i += 256) swv[i / DV][i % DV] = a.winv[(size_t)bh * (BW - 1) * DV + i];
    __syncthreads();
  }
  f4 wx[NW];
  float wxq[NW];
  if (WIN && BW > 1) {
#pragma unroll
    for (int j = 0; j < BW - 1; ++j) {
      wx[j] = *reinterpret_cast<const f4 *>(a.winx + ((size_t)bh * (BW - 1) + j) * DK + 4 * part);
      wxq[j] = row_sum<LPR>(dot4(wx[j], qh));
    }
  }

  // All of this workgroup's state rows are read up front (one 16-byte vector per
  // lane and pass), so every load of the stream is in flight at once; then each
  // pass reduces, updates and writes its rows.
  constexpr int NP = (DV + 4 * RPW - 1) / (4 * RPW);   // passes of 4 waves x RPW rows
  f4 srow[NP];
  float vrow[NP], brow[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * 4 * RPW + wv * RPW + rsub;
    const bool ok = row < DV;  // uniform per row group
    srow[p] = ok ? *reinterpret_cast<const f4 *>(a.S + ((size_t)bh * DV + row) * DK + 4 * part) : zero4();
    vrow[p] = ok ? ld1(vp + (size_t)bh * DV + row) : 0.f;
    brow[p] = (PERCH && ok) ? a.beta[(size_t)bh * DV + row] : 0.f;
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int row = p * 4 * RPW + wv * RPW + rsub;
    const bool ok = row < DV;
    const f4 s = srow[p];
    const float vi = vrow[p];
    const float eta = PERCH ? brow[p] * inv_e : etas;
    const float sq = row_sum<LPR>(dot4(s, qh));
    float o;
    f4 snew = s * lam;
    if (!WIN) {
      const float e = DELTA ? vi - row_sum<LPR>(dot4(s, x)) : vi;
      snew += x * (eta * e);
      o = lam * sq + eta * e * xq;
    } else {
      const float w = eta / (float)BW;
      float acc_o = 0.f;
#pragma unroll
      for (int j = 0; j < BW - 1; ++j) {
        const float vj = ok ? swv[j][row] : 0.f;
        const float e = DELTA ? vj - row_sum<LPR>(dot4(s, wx[j])) : vj;
        snew += wx[j] * (w * e);
        acc_o += e * wxq[j];
      }
      const float e = DELTA ? vi - row_sum<LPR>(dot4(s, x)) : vi;
      snew += x * (w * e);
      acc_o += e * xq;
      o = lam * sq + w * acc_o;
    }
    if (ok) {
      *reinterpret_cast<f4 *>(a.S + ((size_t)bh * DV + row) * DK + 4 * part) = snew;
      if (part == 0) st1(op + (size_t)bh * DV + row, o);
    }
  }

  // every lane has read x_prev and the window; now they may be replaced
  __syncthreads();
  if (wv == 0 && rsub == 0) {
    const f4 xn = xk;
    if (WIN && BW > 1) {
      // shift the window: drop the oldest pair, append (x, v)
#pragma unroll
      for (int j = 0; j < BW - 2; ++j)
        *reinterpret_cast<f4 *>(a.winx + ((size_t)bh * (BW - 1) + j) * DK + 4 * part) = wx[j + 1];
      *reinterpret_cast<f4 *>(a.winx + ((size_t)bh * (BW - 1) + BW - 2) * DK + 4 * part) = x;
    }
    *reinterpret_cast<f4 *>(a.xprev + (size_t)bh * DK + 4 * part) = xn;
  }
  if (WIN && BW > 1) {
    // value window, shifted from the staged copy: drop the oldest value, append v_t
    for (int i = tid; i < (BW - 1) * DV; i += 256) {
      const int j = i / DV, row = i % DV;
      a.winv[(size_t)bh * (BW - 1) * DV + i] = j + 1 < BW - 1 ? swv[j + 1][row] : ld1(vp + (size_t)bh * DV + row);
    }
  }
}

// x_prev = phi(k_{T-1}) and, for a window, the last Bw-1 pairs (x_s, v_s),
// s = T-Bw+1..T-1, where x_s = phi(k_{s-1}) for s >= 1, x_0 = the incoming x_prev
// and s < 0 are pairs of the incoming window.  One workgroup per sequence;
// every old value it needs is read before anything is written, so the
// outputs may alias the incoming state.
template <typename IT, int DK, int DV>
__global__ __launch_bounds__(256) void tail_kernel(FwdArgs a) {
  const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
  const int tid = threadIdx.x;
  // token range: row b of a dense batch, or the packed tokens cu[b] .. cu[b+1]
  const long long tok0 = a.cu ? (long long)a.cu[b] : (long long)b * a.T;
  const int T = a.cu ? a.cu[b + 1] - a.cu[b] : a.T, H = a.H, BW = a.window;
  if (T <= 0) return;   // empty packed sequence: skipped

  const IT *kp = static_cast<const IT *>(a.k);
  const IT *vp = static_cast<const IT *>(a.v);
  __shared__ float sx[MAXW][DK];   // new window keys, then x_prev
  __shared__ float sv[MAXW][DV];
  __shared__ float snorm[MAXW];
  // slot j = 0..BW-2 is pair s = T - BW + 1 + j, whose key is k_{s-1+align} (carried
  // when that index is negative: x_prev for s = 0, the window for s < 0); slot BW-1
  // is phi(k_{T-1})
  auto key_index = [&](int j) { return j == BW - 1 ? T - 1 : T - BW + j + a.align; };
  for (int j = 0; j < BW; ++j) {
    const int s = T - BW + 1 + j, t = key_index(j);
    for (int e = tid; e < DK; e += 256) {
      float x;
      if (t >= 0) x = ld1(kp + ((size_t)(tok0 + t) * H + h) * DK + e);
      else if (s == 0) x = a.xprev0 ? a.xprev0[(size_t)bh * DK + e] : 0.f;
      else x = a.winx0 ? a.winx0[((size_t)bh * (BW - 1) + (BW - 1 + s)) * DK + e] : 0.f;
      sx[j][e] = x;
    }
    if (j < BW - 1) {
      for (int e = tid; e < DV; e += 256) {
        float v;
        if (s >= 0) v = ld1(vp + ((size_t)(tok0 + s) * H + h) * DV + e);
        else v = a.winv0 ? a.winv0[((size_t)bh * (BW - 1) + (BW - 1 + s)) * DV + e] : 0.f;
        sv[j][e] = v;
      }
    }
  }
  __syncthreads();
  for (int j = tid >> 6; j < BW; j += 4) {   // wave w normalises slots w, w+4 when they came from a key
    const int lane = tid & 63;
    float ss = 0.f;
    for (int e = lane; e < DK; e += 64) ss += sx[j][e] * sx[j][e];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) snorm[j] = (key_index(j) >= 0) ? (ss + a.eps_phi > 0.f ? rsqrtf(ss + a.eps_phi) : 0.f) : 1.f;
  }
  __syncthreads();
  for (int e = tid; e < DK; e += 256) a.xprev_out[(size_t)bh * DK + e] = sx[BW - 1][e] * snorm[BW - 1];
  if (BW > 1 && a.winx_out) {
    for (int j = 0; j < BW - 1; ++j) {
      for (int e = tid; e < DK; e += 256)
        a.winx_out[((size_t)bh * (BW - 1) + j) * DK + e] = sx[j][e] * snorm[j];
      for (int e = tid; e < DV; e += 256) a.winv_out[((size_t)bh * (BW - 1) + j) * DV + e] = sv[j][e];
    }
  }
}

template <int VAR, typename IT, int BW>
hipError_t step_dims(int dk, int dv, const StepArgs &a, hipStream_t s) {
  const int nblk = a.B * a.H;
#define FALCON_STEP(DK_, DV_)                                                                  \
  if (dk == DK_ && dv == DV_) {                                                                \
    hipLaunchKernelGGL((step_kernel<VAR, IT, DK_, DV_, BW>), dim3(nblk), dim3(256), 0, s, a);  \
    return hipGetLastError();                                                                  \
  }
  FALCON_STEP(32, 32)
  FALCON_STEP(64, 64)
  FALCON_STEP(128, 128)
#undef FALCON_STEP
  return hipErrorInvalidValue;
}

template <typename IT>
hipError_t tail_dims(int dk, int dv, const FwdArgs &a, hipStream_t s) {
  const int nblk = a.B * a.H;
#define FALCON_TAIL(DK_, DV_)                                                             \
  if (dk == DK_ && dv == DV_) {                                                           \
    hipLaunchKernelGGL((tail_kernel<IT, DK_, DV_>), dim3(nblk), dim3(256), 0, s, a);      \
    return hipGetLastError();                                                             \
  }
  FALCON_TAIL(32, 32)
  FALCON_TAIL(64, 64)
  FALCON_TAIL(128, 128)
#undef FALCON_TAIL
  return hipErrorInvalidValue;
}

template <int VAR>
hipError_t step_window(bool bf16, int dk, int dv, const StepArgs &a, hipStream_t s) {
#define FALCON_W(W_) \
  case W_: return bf16 ? step_dims<VAR, __bf16, W_>(dk, dv, a, s) : step_dims<VAR, float, W_>(dk, dv, a, s)
  switch (a.window) {
    FALCON_W(1); FALCON_W(2); FALCON_W(3); FALCON_W(4); FALCON_W(5); FALCON_W(6); FALCON_W(7); FALCON_W(8);
  }
#undef FALCON_W
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_step(int variant, bool bf16, int dk, int dv, const StepArgs &a, hipStream_t s) {
#define FALCON_V(VV) return bf16 ? step_dims<VV, __bf16, 1>(dk, dv, a, s) : step_dims<VV, float, 1>(dk, dv, a, s)
  switch (variant) {
    case V_F1: FALCON_V(V_F1);
    case V_F1A: FALCON_V(V_F1A);
    case V_F2: FALCON_V(V_F2);
    case V_F2A: FALCON_V(V_F2A);
    case V_F3: return step_window<V_F3>(bf16, dk, dv, a, s);
    case V_F3A: return step_window<V_F3A>(bf16, dk, dv, a, s);
  }
#undef FALCON_V
  return hipErrorInvalidValue;
}

hipError_t launch_tail(int variant, bool bf16, int dk, int dv, const FwdArgs &a, hipStream_t s) {
  (void)variant;
  return bf16 ? tail_dims<__bf16>(dk, dv, a, s) : tail_dims<float>(dk, dv, a, s);
}

}  // namespace falcon
