// Internal launch interface between the C ABI (falcon_abi.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace falcon {

// Everything a forward launch needs, already validated by the host.
struct FwdArgs {
  const void *q, *k, *v;         // [B,T,H,dk|dv] in the input dtype
  const float *beta;             // [B,T,H] or [B,T,H,dv]
  const float *g;                // [B,T,H] log-decay (unclamped)
  const float *S0;               // [B,H,dv,dk] or null (zeros)
  const float *xprev0;           // [B,H,dk] or null (zeros)
  const float *winx0, *winv0;    // [B,H,Bw-1,dk|dv] or null (zeros)
  float *S_out;                  // [B,H,dv,dk] or null
  float *xprev_out;              // [B,H,dk] or null (written by the kernel only when write_tail)
  float *winx_out, *winv_out;    // [B,H,Bw-1,dk|dv] or null
  void *o;                       // [B,T,H,dv]
  float *chunk_states;           // [B,H,NC,dv,dk] or null
  const int *cu;                 // packed sequences: [B+1] token offsets (q, k, v, o are [cu[B], H, d]), or null
  int B, T, H, nchunks, window;
  int align;                     // 0: pair (phi(k_{t-1}), v_t); 1: pair (phi(k_t), v_t)
  float log_eps_gamma, eps_phi, eps_eta;
  int write_tail;                // 1: the main kernel writes x_prev / window itself
  int reuse_images;              // two-kernel path: the workspace already holds this call's images
  int maps_only;                 // two-kernel path: only S_out is wanted (no o, x_prev or window)
};

struct StepArgs {
  const void *q, *k, *v;
  const float *beta, *g;
  float *S, *xprev, *winx, *winv;
  void *o;
  int B, H, window;
  int align;                     // 0: pair (x_prev, v_t); 1: pair (phi(k_t), v_t)
  float log_eps_gamma, eps_phi, eps_eta;
};

// Everything a backward pass needs, already validated by the host: the
// chunk-parallel kernels (falcon_bwd.hip: F1 / F1A / F2 / F2A, d = 64) or the
// recurrent-form kernels (falcon_bwd_rows.hip: every variant, d = 32 / 64 / 128).
struct BwdArgs {
  const void *q, *k, *v, *dO;    // [B,T,H,d] in the input dtype
  const float *beta, *g;         // [B,T,H] (F2 / F2A: beta [B,T,H,d])
  const float *S0, *xprev0;      // incoming S [B,H,d,d] and x_prev [B,H,d], or null (zeros)
  const float *winx0, *winv0;    // incoming window [B,H,Bw-1,d], or null (zeros)
  const float *chunk_states;     // [B,H,cs_nc,d,d]: S at the end of every forward chunk
  const float *dST;              // [B,H,d,d] gradient w.r.t. S_T, or null (zero)
  float *dq, *dk, *dv;           // [B,T,H,d] fp32
  float *dbeta, *dg;             // [B,T,H] fp32 (F2 / F2A: dbeta [B,T,H,d])
  float *dS0, *dxprev0;          // [B,H,d,d], [B,H,d] or null
  float *dwinx0, *dwinv0;        // [B,H,Bw-1,d] or null
  float *ws;                     // the backward workspace
  int B, T, H, NC;               // NC: chunks of 64 steps (chunk-parallel kernels)
  int cs_nc, cs_step;            // chunk_states holds cs_nc states per sequence, one every cs_step
                                 // steps (the forward's chunk: 16, 32 or 64); the chunk-parallel
                                 // kernels read those at 64-step boundaries
  int align;
  float log_eps_gamma, eps_phi, eps_eta;
};

// The segment-parallel forward: per-segment carried keys / windows and the
// composition of the segments' state maps.
struct SegArgs {
  const void *k, *v;                          // [B,T,H,d] in the input dtype
  const float *S0, *xprev0, *winx0, *winv0;   // the caller's incoming state, or null (zeros)
  float *xseg, *wxseg, *wvseg;                // [B*P,H,dk], [B*P,H,Bw-1,dk|dv]: entering each segment
  const float *Nseg, *MNseg;                  // [B*P,H,dv,dk]: segment end states from S0 = 0 and S0 = I
  float *Sseg;                                // [B*P,H,dv,dk]: the state entering each segment
  int B, T, H, P, dk, dv, window, align;
  float eps_phi;
};

// Return hipSuccess or the launch error.  `variant` is falcon_variant_t,
// `bf16` selects the input dtype.  Unsupported combinations return
// hipErrorInvalidValue (the host validates first, so this is a safety net).
hipError_t launch_chunk_fwd(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                            const FwdArgs &a, hipStream_t stream);
hipError_t launch_tail(int variant, bool bf16, int dk, int dv, const FwdArgs &a, hipStream_t stream);
hipError_t launch_step(int variant, bool bf16, int dk, int dv, const StepArgs &a, hipStream_t stream);

bool chunk_bwd_supported(int variant, int dk, int dv, int chunk, int window);
size_t chunk_bwd_workspace(int variant, int B, int H, int T);
hipError_t launch_chunk_bwd(int variant, bool bf16, const BwdArgs &a, hipStream_t stream);
bool rows_bwd_supported(int variant, bool bf16, int dk, int dv, int chunk, int window);
size_t rows_bwd_workspace(int variant, int B, int H, int T, int d, int window);
hipError_t launch_rows_bwd(int variant, bool bf16, int d, int window, const BwdArgs &a, hipStream_t stream);

hipError_t launch_seg_boundary(bool bf16, const SegArgs &a, hipStream_t stream);
hipError_t launch_seg_identity(float *S, int nmat, int dv, int dk, hipStream_t stream);
hipError_t launch_seg_combine(const SegArgs &a, hipStream_t stream);

// The per-shape d_v split of the forward kernel (channels per workgroup = dv / nsplit).
int choose_nsplit(int variant, bool bf16, int dk, int dv, int chunk, int batch_heads);

}  // namespace falcon
