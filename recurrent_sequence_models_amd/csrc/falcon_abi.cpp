// C ABI of the Falcon fast-weight attention library (declared in include/falcon.h).
//
// Host side only: every argument is validated here before the first HIP call,
// so an invalid call returns a status without touching the device.  The
// kernels live in falcon_fwd.hip, falcon_fwd3.hip and falcon_step.hip.
#include "falcon.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "falcon_kernels.h"

namespace {

using falcon::BwdArgs;
using falcon::FwdArgs;
using falcon::StepArgs;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool windowed(int v) { return v == FALCON_3 || v == FALCON_3A; }
bool per_channel(int v) { return v == FALCON_2 || v == FALCON_2A; }
bool finite(float x) { return std::isfinite(x); }

// Shape checks shared by both entry points.  `step` skips seqlen/chunk.
int check_shape(const falcon_shape_t *s, bool step) {
  if (!s) return FALCON_ERR_INVALID_ARG;
  if (s->variant < FALCON_1 || s->variant > FALCON_3A) return FALCON_ERR_INVALID_ARG;
  if (s->dtype != FALCON_F32 && s->dtype != FALCON_BF16) return FALCON_ERR_INVALID_ARG;
  if (s->batch < 1 || s->heads < 1 || s->dk < 1 || s->dv < 1) return FALCON_ERR_INVALID_ARG;
  if (!step && (s->seqlen < 1 || s->chunk < 1)) return FALCON_ERR_INVALID_ARG;
  if (!finite(s->eps_gamma) || !finite(s->eps_phi) || !finite(s->eps_eta)) return FALCON_ERR_INVALID_ARG;
  if (!(s->eps_gamma > 0.f && s->eps_gamma <= 1.f)) return FALCON_ERR_INVALID_ARG;
  if (s->eps_phi < 0.f || !(s->eps_eta > 0.f)) return FALCON_ERR_INVALID_ARG;
  if (s->window < 1) return FALCON_ERR_INVALID_ARG;
  if (s->align != FALCON_ALIGN_PREFIX && s->align != FALCON_ALIGN_SAME) return FALCON_ERR_INVALID_ARG;
  if (!windowed(s->variant) && s->window != 1) return FALCON_ERR_INVALID_ARG;
  if (windowed(s->variant) && s->window > 8) return FALCON_ERR_UNSUPPORTED;
  if (s->dk != s->dv) return FALCON_ERR_UNSUPPORTED;
  if (s->dk != 32 && s->dk != 64 && s->dk != 128) return FALCON_ERR_UNSUPPORTED;
  if (!step) {
    if (s->chunk != 16 && s->chunk != 32 && s->chunk != 64) return FALCON_ERR_UNSUPPORTED;
    if (s->dtype == FALCON_F32 && s->dk > 64) return FALCON_ERR_UNSUPPORTED;
    if (windowed(s->variant) && 64 % s->window != 0) return FALCON_ERR_UNSUPPORTED;
    if ((int64_t)s->batch * s->seqlen > INT32_MAX) return FALCON_ERR_UNSUPPORTED;
  }
  if ((int64_t)s->batch * s->heads > INT32_MAX / 2) return FALCON_ERR_UNSUPPORTED;
  return FALCON_OK;
}

int check_state(const falcon_state_t *st, const falcon_shape_t *s) {
  if (!st->S || !st->x_prev) return FALCON_ERR_INVALID_ARG;
  if (!aligned16(st->S) || !aligned16(st->x_prev)) return FALCON_ERR_INVALID_ARG;
  if (windowed(s->variant) && s->window > 1) {
    if (!st->win_x || !st->win_v) return FALCON_ERR_INVALID_ARG;
    if (!aligned16(st->win_x) || !aligned16(st->win_v)) return FALCON_ERR_INVALID_ARG;
  }
  return FALCON_OK;
}

int check_io(const void *q, const void *k, const void *v, const float *beta, const float *g, const void *o) {
  if (!q || !k || !v || !beta || !g || !o) return FALCON_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(beta))
    return FALCON_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(g) & 3u) != 0) return FALCON_ERR_INVALID_ARG;
  return FALCON_OK;
}

// Whether the one-pass kernel writes the outgoing x_prev / window itself (1) or
// leaves it to the tail kernel (0).  The copy waves that write it run after the
// kernel's last barrier, while other workgroups of the sequence (ns > 1 channel
// slices) may still read the incoming state, and, for a window, the copy waves
// of one workgroup read carried pairs (sequences shorter than the window) that
// their neighbours overwrite.  So an outgoing state that aliases the incoming one
// goes through the tail kernel, which reads everything before it writes, unless
// a single workgroup per sequence writes only x_prev (which it never reads then:
// x_prev = phi(k_{T-1}) comes from the inputs).
int onepass_writes_tail(const falcon_state_t *init, const falcon_state_t *final_state, bool win, int ns) {
  if (!final_state) return 0;
  const bool alias = init && (init->x_prev == final_state->x_prev ||
                              (win && (init->win_x == final_state->win_x || init->win_v == final_state->win_v)));
  if (!alias) return 1;
  return (ns == 1 && !win) ? 1 : 0;
}

}  // namespace

namespace falcon {
hipError_t static_scratch(void **out);   // falcon_static.hip
hipError_t launch_chunk_fwd_rows(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                 const FwdArgs &a, hipStream_t s);
hipError_t launch_chunk_fwd_window(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                                   const FwdArgs &a, hipStream_t s);
bool chunk_fwd_pipe_supported(int variant, bool bf16, int dk, int dv, int chunk);
bool chunk_fwd_split_supported(int variant, bool bf16, int dk, int dv, int chunk, int window);
size_t chunk_fwd_split_workspace(int variant, bool bf16, int dk, int dv, int chunk, int window, int bh, int T);
size_t chunk_fwd_split_workspace_varlen(int variant, bool bf16, int dk, int dv, int chunk, int window, int N, int H,
                                        int total);
hipError_t launch_chunk_fwd_split(int variant, bool bf16, int dk, int dv, int chunk, int window, const FwdArgs &a,
                                  void *ws, hipStream_t s);
int chunk_fwd_onepass_ns(int variant, bool bf16, int dk, int dv, int chunk, int window, int bh);
bool chunk_fwd_band_supported(int variant, int dk, int dv, int chunk, int window);   // falcon_fwd_band.hip
size_t chunk_fwd_band_workspace(int bh, int T);
hipError_t launch_chunk_fwd_band(bool bf16, const FwdArgs &a, void *ws, hipStream_t s);
hipError_t launch_chunk_fwd_onepass(int variant, bool bf16, int dk, int dv, int chunk, int window, const FwdArgs &a,
                                    hipStream_t s);

int choose_nsplit(int variant, bool bf16, int dk, int dv, int chunk, int batch_heads) {
  int n = 1;
  // whole sequences per workgroup on the software-pipelined kernel when it fits
  if (!windowed(variant) && chunk_fwd_pipe_supported(variant, bf16, dk, dv, chunk)) return 1;
  // Falcon-3: one workgroup takes up to 64 value channels.
  if (windowed(variant)) return dv == 128 ? 2 : 1;
  // F2 keeps per-channel steps in LDS: at 128 channels a workgroup takes 64 of them.
  if (per_channel(variant) && dv == 128) n = 2;
  // Few sequences: split the value channels over more workgroups (rows of S are
  // independent given the keys), so more compute units take part.
  while (batch_heads * n < 128 && dv / (2 * n) >= 16 && n < 8) n *= 2;
  return n;
}

hipError_t launch_chunk_fwd(int variant, bool bf16, int dk, int dv, int chunk, int nsplit,
                            const FwdArgs &a, hipStream_t s) {
  if (windowed(variant)) return launch_chunk_fwd_window(variant, bf16, dk, dv, chunk, nsplit, a, s);
  return launch_chunk_fwd_rows(variant, bf16, dk, dv, chunk, nsplit, a, s);
}
}  // namespace falcon

extern "C" {

int falcon_abi_version(void) { return FALCON_ABI_VERSION; }

const char *falcon_status_string(int status) {
  switch (status) {
    case FALCON_OK: return "FALCON_OK";
    case FALCON_ERR_INVALID_ARG: return "FALCON_ERR_INVALID_ARG: invalid argument";
    case FALCON_ERR_UNSUPPORTED: return "FALCON_ERR_UNSUPPORTED: valid but unsupported shape or option";
    case FALCON_ERR_WORKSPACE: return "FALCON_ERR_WORKSPACE: workspace too small";
    case FALCON_ERR_HIP: return "FALCON_ERR_HIP: HIP launch or runtime error";
  }
  return "unknown falcon status";
}

size_t falcon_chunk_fwd_workspace(const falcon_shape_t *shape) {
  if (check_shape(shape, false) != FALCON_OK) return 0;
  // one image per system of rows (at least one step each) must have an int index
  const int64_t bhs = (int64_t)shape->batch * shape->heads * shape->seqlen;
  if (bhs > INT32_MAX) return 0;
  const size_t split = falcon::chunk_fwd_split_workspace(shape->variant, shape->dtype == FALCON_BF16, shape->dk,
                                                        shape->dv, shape->chunk, shape->window,
                                                        shape->batch * shape->heads, shape->seqlen);
  // Falcon-3A windows at d = 64, chunk 64 run the banded-weight kernels (fp32 and bf16 inputs); the
  // size covers both paths
  if (falcon::chunk_fwd_band_supported(shape->variant, shape->dk, shape->dv, shape->chunk, shape->window))
    return std::max(split, falcon::chunk_fwd_band_workspace(shape->batch * shape->heads, shape->seqlen));
  return split;
}

int falcon_chunk_fwd(const falcon_shape_t *s, const void *q, const void *k, const void *v,
                     const float *beta, const float *log_lambda, const falcon_state_t *init,
                     falcon_state_t *final_state, void *o, float *chunk_states, void *workspace,
                     size_t workspace_bytes, void *stream) {
  int st = check_shape(s, false);
  if (st != FALCON_OK) return st;
  if ((st = check_io(q, k, v, beta, log_lambda, o)) != FALCON_OK) return st;
  if (init && (st = check_state(init, s)) != FALCON_OK) return st;
  if (final_state && (st = check_state(final_state, s)) != FALCON_OK) return st;
  if (chunk_states && !aligned16(chunk_states)) return FALCON_ERR_INVALID_ARG;
  const size_t ws_need = falcon_chunk_fwd_workspace(s);
  const bool split = workspace != nullptr && ws_need > 0;
  if (split && workspace_bytes < ws_need) return FALCON_ERR_WORKSPACE;
  if (split && !aligned16(workspace)) return FALCON_ERR_INVALID_ARG;

  const bool bf16 = s->dtype == FALCON_BF16;
  const bool win = windowed(s->variant) && s->window > 1;
  const int nsplit = falcon::choose_nsplit(s->variant, bf16, s->dk, s->dv, s->chunk, s->batch * s->heads);
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = log_lambda;
  a.S0 = init ? init->S : nullptr;
  a.xprev0 = init ? init->x_prev : nullptr;
  a.winx0 = (init && win) ? init->win_x : nullptr;
  a.winv0 = (init && win) ? init->win_v : nullptr;
  a.S_out = final_state ? final_state->S : nullptr;
  a.xprev_out = final_state ? final_state->x_prev : nullptr;
  a.winx_out = (final_state && win) ? final_state->win_x : nullptr;
  a.winv_out = (final_state && win) ? final_state->win_v : nullptr;
  a.o = o;
  a.chunk_states = chunk_states;
  a.B = s->batch; a.T = s->seqlen; a.H = s->heads;
  a.nchunks = (s->seqlen + s->chunk - 1) / s->chunk;
  a.window = windowed(s->variant) ? s->window : 1;
  a.align = s->align;
  a.log_eps_gamma = std::log(s->eps_gamma);
  a.eps_phi = s->eps_phi;
  a.eps_eta = s->eps_eta;
  // The main kernel writes x_prev (and the window) itself when that cannot race
  // with another workgroup still reading the incoming state: on the split path
  // (its scan reads a copy the prep kernel made), with one workgroup per
  // sequence, or when the two buffers are distinct.  Otherwise a tail kernel does.
  const bool xprev_alias = init && final_state && init->x_prev == final_state->x_prev;
  a.write_tail = (final_state && (split || (!win && (nsplit == 1 || !xprev_alias)))) ? 1 : 0;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  // Without a workspace: the one-pass kernel where it is built for the shape.
  const int onepass = split ? 0 : falcon::chunk_fwd_onepass_ns(s->variant, bf16, s->dk, s->dv, s->chunk, a.window,
                                                                s->batch * s->heads);
  if (onepass) {
    a.write_tail = onepass_writes_tail(init, final_state, win, onepass);
    if (falcon::launch_chunk_fwd_onepass(s->variant, bf16, s->dk, s->dv, s->chunk, a.window, a, hs) != hipSuccess)
      return FALCON_ERR_HIP;
    if (final_state && !a.write_tail) {
      if (falcon::launch_tail(s->variant, bf16, s->dk, s->dv, a, hs) != hipSuccess) return FALCON_ERR_HIP;
    }
    return FALCON_OK;
  }
  // same-step pairs run only on the chunk-parallel kernels
  if (!split && s->align != FALCON_ALIGN_PREFIX) return FALCON_ERR_UNSUPPORTED;
  if (split && falcon::chunk_fwd_band_supported(s->variant, s->dk, s->dv, s->chunk, a.window))
    return falcon::launch_chunk_fwd_band(bf16, a, workspace, hs) == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
  if (split) {   // prep over all systems, then the scan workgroups of each sequence
    return falcon::launch_chunk_fwd_split(s->variant, bf16, s->dk, s->dv, s->chunk, a.window, a, workspace, hs) ==
                   hipSuccess
               ? FALCON_OK
               : FALCON_ERR_HIP;
  }
  if (falcon::launch_chunk_fwd(s->variant, bf16, s->dk, s->dv, s->chunk, nsplit, a, hs) != hipSuccess)
    return FALCON_ERR_HIP;
  if (final_state && !a.write_tail) {
    if (falcon::launch_tail(s->variant, bf16, s->dk, s->dv, a, hs) != hipSuccess) return FALCON_ERR_HIP;
  }
  return FALCON_OK;
}

int falcon_chunk_fwd_static(const falcon_shape_t *s, const void *q, const void *k, const void *v,
                            const float *beta, const float *log_lambda, const falcon_state_t *init,
                            falcon_state_t *final_state, void *o, float *chunk_states, void *stream) {
  int st = check_shape(s, false);
  if (st != FALCON_OK) return st;
  if ((st = check_io(q, k, v, beta, log_lambda, o)) != FALCON_OK) return st;
  if (init && (st = check_state(init, s)) != FALCON_OK) return st;
  if (final_state && (st = check_state(final_state, s)) != FALCON_OK) return st;
  if (chunk_states && !aligned16(chunk_states)) return FALCON_ERR_INVALID_ARG;
  const size_t need = falcon_chunk_fwd_workspace(s);
  if (need == 0) return FALCON_ERR_UNSUPPORTED;
  if (need > FALCON_STATIC_SCRATCH_BYTES) return FALCON_ERR_WORKSPACE;
  void *scratch = nullptr;   // this device's copy of the library's scratch array
  if (falcon::static_scratch(&scratch) != hipSuccess || !scratch) return FALCON_ERR_HIP;
  return falcon_chunk_fwd(s, q, k, v, beta, log_lambda, init, final_state, o, chunk_states, scratch, need, stream);
}

size_t falcon_chunk_fwd_varlen_workspace(const falcon_shape_t *s) {
  if (check_shape(s, false) != FALCON_OK) return 0;
  // image slots per head must have int indices
  if ((int64_t)s->heads * ((int64_t)s->seqlen + s->batch + 1) > INT32_MAX) return 0;
  return falcon::chunk_fwd_split_workspace_varlen(s->variant, s->dtype == FALCON_BF16, s->dk, s->dv, s->chunk,
                                                  s->window, s->batch, s->heads, s->seqlen);
}

int falcon_chunk_fwd_varlen(const falcon_shape_t *s, const int32_t *cu_seqlens, const void *q, const void *k,
                            const void *v, const float *beta, const float *log_lambda, const falcon_state_t *init,
                            falcon_state_t *final_state, void *o, void *workspace, size_t workspace_bytes,
                            void *stream) {
  int st = check_shape(s, false);
  if (st != FALCON_OK) return st;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return FALCON_ERR_INVALID_ARG;
  if ((st = check_io(q, k, v, beta, log_lambda, o)) != FALCON_OK) return st;
  if (init && (st = check_state(init, s)) != FALCON_OK) return st;
  if (final_state && (st = check_state(final_state, s)) != FALCON_OK) return st;
  const bool bf16 = s->dtype == FALCON_BF16;
  const bool win = windowed(s->variant) && s->window > 1;
  const int window = windowed(s->variant) ? s->window : 1;
  const size_t ws_need = falcon_chunk_fwd_varlen_workspace(s);
  const bool split = workspace != nullptr && ws_need > 0;
  if (split && workspace_bytes < ws_need) return FALCON_ERR_WORKSPACE;
  if (split && !aligned16(workspace)) return FALCON_ERR_INVALID_ARG;
  const int ns =
      split ? 0 : falcon::chunk_fwd_onepass_ns(s->variant, bf16, s->dk, s->dv, s->chunk, window, s->batch * s->heads);
  if (!split && ns == 0) return ws_need > 0 ? FALCON_ERR_WORKSPACE : FALCON_ERR_UNSUPPORTED;
  FwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = log_lambda;
  a.S0 = init ? init->S : nullptr;
  a.xprev0 = init ? init->x_prev : nullptr;
  a.winx0 = (init && win) ? init->win_x : nullptr;
  a.winv0 = (init && win) ? init->win_v : nullptr;
  a.S_out = final_state ? final_state->S : nullptr;
  a.xprev_out = final_state ? final_state->x_prev : nullptr;
  a.winx_out = (final_state && win) ? final_state->win_x : nullptr;
  a.winv_out = (final_state && win) ? final_state->win_v : nullptr;
  a.o = o;
  a.chunk_states = nullptr;
  a.cu = cu_seqlens;
  a.B = s->batch; a.T = s->seqlen; a.H = s->heads;
  a.nchunks = 1;
  a.window = window;
  a.align = s->align;
  a.log_eps_gamma = std::log(s->eps_gamma);
  a.eps_phi = s->eps_phi;
  a.eps_eta = s->eps_eta;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (split) {   // prep over every image slot, then the scan workgroups of each sequence; the scan
                 // reads the prep's copy of the incoming x_prev / window, so it writes the outgoing ones
    a.write_tail = final_state ? 1 : 0;
    return falcon::launch_chunk_fwd_split(s->variant, bf16, s->dk, s->dv, s->chunk, window, a, workspace, hs) ==
                   hipSuccess
               ? FALCON_OK
               : FALCON_ERR_HIP;
  }
  a.write_tail = onepass_writes_tail(init, final_state, win, ns);
  if (falcon::launch_chunk_fwd_onepass(s->variant, bf16, s->dk, s->dv, s->chunk, window, a, hs) != hipSuccess)
    return FALCON_ERR_HIP;
  if (final_state && !a.write_tail) {
    if (falcon::launch_tail(s->variant, bf16, s->dk, s->dv, a, hs) != hipSuccess) return FALCON_ERR_HIP;
  }
  return FALCON_OK;
}

int falcon_recurrent_step(const falcon_shape_t *s, const void *q, const void *k, const void *v,
                          const float *beta, const float *log_lambda, falcon_state_t *state, void *o,
                          void *stream) {
  int st = check_shape(s, true);
  if (st != FALCON_OK) return st;
  if ((st = check_io(q, k, v, beta, log_lambda, o)) != FALCON_OK) return st;
  if (!state) return FALCON_ERR_INVALID_ARG;
  if ((st = check_state(state, s)) != FALCON_OK) return st;
  const bool win = windowed(s->variant) && s->window > 1;
  StepArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = log_lambda;
  a.S = state->S; a.xprev = state->x_prev;
  a.winx = win ? state->win_x : nullptr;
  a.winv = win ? state->win_v : nullptr;
  a.o = o;
  a.B = s->batch; a.H = s->heads;
  a.window = windowed(s->variant) ? s->window : 1;
  a.align = s->align;
  a.log_eps_gamma = std::log(s->eps_gamma);
  a.eps_phi = s->eps_phi;
  a.eps_eta = s->eps_eta;
  if (falcon::launch_step(s->variant, s->dtype == FALCON_BF16, s->dk, s->dv, a,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return FALCON_ERR_HIP;
  return FALCON_OK;
}

}  // extern "C"

namespace {

// The chunk-parallel backward where it is built (F1 / F1A / F2 / F2A, and
// F3 / F3A with one pair, which are F1 / F1A; d = 64), else the recurrent-form
// one (every variant and window, d = 32 / 64 / 128).
int bwd_variant(const falcon_shape_t *s) {
  if (windowed(s->variant) && s->window == 1) return s->variant == FALCON_3 ? FALCON_1 : FALCON_1A;
  return s->variant;
}
bool bwd_chunk_parallel(const falcon_shape_t *s) {
  return falcon::chunk_bwd_supported(bwd_variant(s), s->dk, s->dv, s->chunk, windowed(s->variant) ? s->window : 1);
}
bool bwd_rows(const falcon_shape_t *s) {
  return falcon::rows_bwd_supported(s->variant, s->dtype == FALCON_BF16, s->dk, s->dv, s->chunk,
                                    windowed(s->variant) ? s->window : 1);
}
size_t bwd_workspace(const falcon_shape_t *s) {
  if (bwd_chunk_parallel(s)) return falcon::chunk_bwd_workspace(bwd_variant(s), s->batch, s->heads, s->seqlen);
  if (bwd_rows(s))
    return falcon::rows_bwd_workspace(s->variant, s->batch, s->heads, s->seqlen, s->dk,
                                      windowed(s->variant) ? s->window : 1);
  return 0;
}

}  // namespace

extern "C" {

size_t falcon_chunk_bwd_workspace(const falcon_shape_t *s) {
  if (check_shape(s, false) != FALCON_OK) return 0;
  return bwd_workspace(s);
}

int falcon_chunk_bwd(const falcon_shape_t *s, const void *q, const void *k, const void *v, const float *beta,
                     const float *log_lambda, const falcon_state_t *init, const float *chunk_states,
                     const void *d_o, const float *d_final_S, float *dq, float *dk, float *dv, float *dbeta,
                     float *dg, falcon_state_t *d_init, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape(s, false);
  if (st != FALCON_OK) return st;
  if ((st = check_io(q, k, v, beta, log_lambda, d_o)) != FALCON_OK) return st;
  if (!chunk_states || !dq || !dk || !dv || !dbeta || !dg || !workspace) return FALCON_ERR_INVALID_ARG;
  if (!aligned16(chunk_states) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FALCON_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(dbeta) & 3u) != 0 || (reinterpret_cast<uintptr_t>(dg) & 3u) != 0)
    return FALCON_ERR_INVALID_ARG;
  if (d_final_S && !aligned16(d_final_S)) return FALCON_ERR_INVALID_ARG;
  if (init && (st = check_state(init, s)) != FALCON_OK) return st;
  if (d_init && (st = check_state(d_init, s)) != FALCON_OK) return st;
  const bool wy = bwd_chunk_parallel(s);
  if (!wy && !bwd_rows(s)) return FALCON_ERR_UNSUPPORTED;
  if (workspace_bytes < bwd_workspace(s)) return FALCON_ERR_WORKSPACE;
  const bool win = windowed(s->variant) && s->window > 1;
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dO = d_o; a.beta = beta; a.g = log_lambda;
  a.S0 = init ? init->S : nullptr;
  a.xprev0 = init ? init->x_prev : nullptr;
  a.winx0 = init && win ? init->win_x : nullptr;
  a.winv0 = init && win ? init->win_v : nullptr;
  a.chunk_states = chunk_states;
  a.dST = d_final_S;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dg = dg;
  a.dS0 = d_init ? d_init->S : nullptr;
  a.dxprev0 = d_init ? d_init->x_prev : nullptr;
  a.dwinx0 = d_init && win ? d_init->win_x : nullptr;
  a.dwinv0 = d_init && win ? d_init->win_v : nullptr;
  a.ws = static_cast<float *>(workspace);
  a.B = s->batch; a.T = s->seqlen; a.H = s->heads;
  a.NC = (s->seqlen + 63) / 64;                        // the kernels' chunks of 64 steps
  a.cs_nc = (s->seqlen + s->chunk - 1) / s->chunk;      // the forward's per-chunk states
  a.cs_step = s->chunk;
  a.align = s->align;
  a.log_eps_gamma = std::log(s->eps_gamma);
  a.eps_phi = s->eps_phi;
  a.eps_eta = s->eps_eta;
  const hipError_t e =
      wy ? falcon::launch_chunk_bwd(bwd_variant(s), s->dtype == FALCON_BF16, a, static_cast<hipStream_t>(stream))
         : falcon::launch_rows_bwd(s->variant, s->dtype == FALCON_BF16, s->dk, win ? s->window : 1, a,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FALCON_OK : FALCON_ERR_HIP;
}

}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of the segment-parallel workspace: the two-kernel path's scratch
// for B*P sequences of T/P steps, then the per-segment state arrays.
struct SegLayout {
  size_t split, S, N, MN, x, wx, wv, Sf, xf, wxf, wvf, total;
};

bool seg_layout(const falcon_shape_t *s, int nseg, SegLayout &L) {
  if (check_shape(s, false) != FALCON_OK || nseg < 1 || s->seqlen % nseg != 0) return false;
  if (s->variant == FALCON_2) return false;  // F2: a different state map for every row of S
  const int Ts = s->seqlen / nseg;
  const int window = windowed(s->variant) ? s->window : 1;
  if (Ts < window) return false;
  const int64_t bph = (int64_t)s->batch * nseg * s->heads;
  if (bph * Ts > INT32_MAX || bph > INT32_MAX / 2) return false;
  const size_t split = falcon::chunk_fwd_split_workspace(s->variant, s->dtype == FALCON_BF16, s->dk, s->dv, s->chunk,
                                                         s->window, (int)bph, Ts);
  if (split == 0) return false;
  const size_t mat = (size_t)bph * s->dv * s->dk * 4, vec = (size_t)bph * s->dk * 4;
  const size_t wx = (size_t)bph * (window - 1) * s->dk * 4, wv = (size_t)bph * (window - 1) * s->dv * 4;
  size_t off = 0;
  auto take = [&](size_t n) { const size_t o = off; off = align256(off + n); return o; };
  L.split = take(split);
  L.S = take(mat);
  L.N = take(mat);
  L.MN = take(mat);
  L.x = take(vec);
  L.wx = take(wx);
  L.wv = take(wv);
  L.Sf = take(mat);
  L.xf = take(vec);
  L.wxf = take(wx);
  L.wvf = take(wv);
  L.total = off;
  return true;
}

}  // namespace

extern "C" {

size_t falcon_chunk_fwd_segmented_workspace(const falcon_shape_t *s, int32_t nseg) {
  SegLayout L;
  return seg_layout(s, nseg, L) ? L.total : 0;
}

int falcon_chunk_fwd_segmented(const falcon_shape_t *s, int32_t nseg, const void *q, const void *k, const void *v,
                               const float *beta, const float *log_lambda, const falcon_state_t *init,
                               falcon_state_t *final_state, void *o, void *workspace, size_t workspace_bytes,
                               void *stream) {
  int st = check_shape(s, false);
  if (st != FALCON_OK) return st;
  if ((st = check_io(q, k, v, beta, log_lambda, o)) != FALCON_OK) return st;
  if (init && (st = check_state(init, s)) != FALCON_OK) return st;
  if (final_state && (st = check_state(final_state, s)) != FALCON_OK) return st;
  if (nseg < 1 || s->seqlen % nseg != 0) return FALCON_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return FALCON_ERR_INVALID_ARG;
  SegLayout L;
  if (!seg_layout(s, nseg, L)) return FALCON_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return FALCON_ERR_WORKSPACE;
  unsigned char *ws = static_cast<unsigned char *>(workspace);
  auto F = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
  const bool bf16 = s->dtype == FALCON_BF16;
  const bool win = windowed(s->variant) && s->window > 1;
  const int window = windowed(s->variant) ? s->window : 1;
  const int P = nseg, Ts = s->seqlen / nseg;
  hipStream_t hs = static_cast<hipStream_t>(stream);

  falcon::SegArgs g{};
  g.k = k; g.v = v;
  g.S0 = init ? init->S : nullptr;
  g.xprev0 = init ? init->x_prev : nullptr;
  g.winx0 = (init && win) ? init->win_x : nullptr;
  g.winv0 = (init && win) ? init->win_v : nullptr;
  g.xseg = F(L.x); g.wxseg = F(L.wx); g.wvseg = F(L.wv);
  g.Nseg = F(L.N); g.MNseg = F(L.MN); g.Sseg = F(L.S);
  g.B = s->batch; g.T = s->seqlen; g.H = s->heads; g.P = P;
  g.dk = s->dk; g.dv = s->dv; g.window = window; g.align = s->align;
  g.eps_phi = s->eps_phi;

  // One forward over all B*P segments, each a sequence of Ts steps (the arrays
  // [B,T,H,d] read as [B*P,Ts,H,d]).
  // The three passes share one set of images (they depend on the inputs, not on
  // S0): the first pass builds them, the later ones only scan.
  bool images = false;
  auto forward = [&](const float *S0, float *S_out, float *x_out, float *wx_out, float *wv_out, void *out) {
    FwdArgs a{};
    a.reuse_images = images ? 1 : 0;
    a.maps_only = out ? 0 : 1;   // the map passes want the end states alone
    images = true;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = log_lambda;
    a.S0 = S0;
    a.xprev0 = F(L.x);
    a.winx0 = win ? F(L.wx) : nullptr;
    a.winv0 = win ? F(L.wv) : nullptr;
    a.S_out = S_out; a.xprev_out = x_out; a.winx_out = wx_out; a.winv_out = wv_out;
    a.o = out;
    a.chunk_states = nullptr;
    a.B = s->batch * P; a.T = Ts; a.H = s->heads;
    a.nchunks = (Ts + s->chunk - 1) / s->chunk;
    a.window = window;
    a.align = s->align;
    a.log_eps_gamma = std::log(s->eps_gamma);
    a.eps_phi = s->eps_phi;
    a.eps_eta = s->eps_eta;
    a.write_tail = 1;
    return falcon::launch_chunk_fwd_split(s->variant, bf16, s->dk, s->dv, s->chunk, window, a, ws + L.split, hs);
  };
  if (falcon::launch_seg_boundary(bf16, g, hs) != hipSuccess) return FALCON_ERR_HIP;
  if (P > 1) {
    if (forward(nullptr, F(L.N), nullptr, nullptr, nullptr, nullptr) != hipSuccess) return FALCON_ERR_HIP;
    if (falcon::launch_seg_identity(F(L.S), s->batch * P * s->heads, s->dv, s->dk, hs) != hipSuccess)
      return FALCON_ERR_HIP;
    if (forward(F(L.S), F(L.MN), nullptr, nullptr, nullptr, nullptr) != hipSuccess) return FALCON_ERR_HIP;
    if (falcon::launch_seg_combine(g, hs) != hipSuccess) return FALCON_ERR_HIP;
  } else if (init) {
    if (hipMemcpyAsync(F(L.S), init->S, (size_t)s->batch * s->heads * s->dv * s->dk * 4, hipMemcpyDeviceToDevice,
                       hs) != hipSuccess)
      return FALCON_ERR_HIP;
  }
  const float *S_in = (P > 1 || init) ? F(L.S) : nullptr;
  if (forward(S_in, F(L.Sf), F(L.xf), win ? F(L.wxf) : nullptr, win ? F(L.wvf) : nullptr, o) != hipSuccess)
    return FALCON_ERR_HIP;
  if (final_state) {  // the last segment's final state is the sequence's
    const size_t H = s->heads;
    auto copy_last = [&](void *dst, const float *src, size_t per_bh) {
      const size_t row = H * per_bh * 4;
      return hipMemcpy2DAsync(dst, row, src + (size_t)(P - 1) * H * per_bh, (size_t)P * row, row, s->batch,
                              hipMemcpyDeviceToDevice, hs);
    };
    if (copy_last(final_state->S, F(L.Sf), (size_t)s->dv * s->dk) != hipSuccess) return FALCON_ERR_HIP;
    if (copy_last(final_state->x_prev, F(L.xf), (size_t)s->dk) != hipSuccess) return FALCON_ERR_HIP;
    if (win) {
      if (copy_last(final_state->win_x, F(L.wxf), (size_t)(window - 1) * s->dk) != hipSuccess) return FALCON_ERR_HIP;
      if (copy_last(final_state->win_v, F(L.wvf), (size_t)(window - 1) * s->dv) != hipSuccess) return FALCON_ERR_HIP;
    }
  }
  return FALCON_OK;
}

}  // extern "C"
