// Launch side of the chunk-parallel forward pass (kernels in split_impl.h):
// the one-pair variants Falcon-1 / 1A / 2 / 2A (and Falcon-3 / 3A with a
// window of one pair, which are Falcon-1 / 1A), and the entry points that
// route windows of 2, 4 or 8 pairs to falcon_fwd_split_win.hip.
#include "split_impl.h"

namespace falcon {

bool chunk_fwd_split_win_supported(int variant, bool bf16, int d, int chunk, int window);
size_t chunk_fwd_split_win_workspace(int variant, bool bf16, int d, int chunk, int window, int bh, int T);
size_t chunk_fwd_split_win_workspace_varlen(int variant, bool bf16, int d, int chunk, int window, int N, int H,
                                            int total);
hipError_t launch_chunk_fwd_split_win(int variant, bool bf16, int d, int chunk, int window, const FwdArgs &a,
                                      void *ws, hipStream_t st);
int chunk_fwd_onepass_win_ns(int variant, bool bf16, int d, int chunk, int window, int bh);
hipError_t launch_chunk_fwd_onepass_win(int variant, bool bf16, int d, int chunk, int window, const FwdArgs &a,
                                        hipStream_t st);

namespace {

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

// a window of one pair is the one-pair variant
int one_pair(int variant) { return variant == V_F3 ? V_F1 : variant == V_F3A ? V_F1A : variant; }

}  // namespace

bool chunk_fwd_split_supported(int variant, bool bf16, int dk, int dv, int chunk, int window) {
  if (dk != dv) return false;
  if (window > 1) return chunk_fwd_split_win_supported(variant, bf16, dk, chunk, window);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [](auto v, auto *t, auto dd, auto cc) -> bool {
    using IT = std::remove_pointer_t<decltype(t)>;
    return pick_ns<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1>(1) > 0;
  });
}

size_t chunk_fwd_split_workspace(int variant, bool bf16, int dk, int dv, int chunk, int window, int bh, int T) {
  if (!chunk_fwd_split_supported(variant, bf16, dk, dv, chunk, window)) return 0;
  if (window > 1) return chunk_fwd_split_win_workspace(variant, bf16, dk, chunk, window, bh, T);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [bh, T](auto v, auto *t, auto dd, auto cc) -> size_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return Split<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1>::workspace(bh, T);
  });
}

// Scratch of the two-kernel path for N packed sequences of `total` tokens over H heads.
size_t chunk_fwd_split_workspace_varlen(int variant, bool bf16, int dk, int dv, int chunk, int window, int N, int H,
                                        int total) {
  if (!chunk_fwd_split_supported(variant, bf16, dk, dv, chunk, window)) return 0;
  if (window > 1) return chunk_fwd_split_win_workspace_varlen(variant, bf16, dk, chunk, window, N, H, total);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [N, H, total](auto v, auto *t, auto dd, auto cc) -> size_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return Split<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1>::workspace_varlen(N, H, total);
  });
}

hipError_t launch_chunk_fwd_split(int variant, bool bf16, int dk, int dv, int chunk, int window, const FwdArgs &a,
                                  void *ws, hipStream_t st) {
  if (!chunk_fwd_split_supported(variant, bf16, dk, dv, chunk, window)) return hipErrorInvalidValue;
  if (window > 1) return launch_chunk_fwd_split_win(variant, bf16, dk, chunk, window, a, ws, st);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [&](auto v, auto *t, auto dd, auto cc) -> hipError_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return launch_split<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1>(a, ws, st);
  });
}

// One-pass form (no workspace): channel split it would use for bh sequences, 0 if not built.
int chunk_fwd_onepass_ns(int variant, bool bf16, int dk, int dv, int chunk, int window, int bh) {
  if (dk != dv) return 0;
  if (window > 1) return chunk_fwd_onepass_win_ns(variant, bf16, dk, chunk, window, bh);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [bh](auto v, auto *t, auto dd, auto cc) -> int {
    using IT = std::remove_pointer_t<decltype(t)>;
    return pick_ns<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1, true>(bh);
  });
}

hipError_t launch_chunk_fwd_onepass(int variant, bool bf16, int dk, int dv, int chunk, int window, const FwdArgs &a,
                                    hipStream_t st) {
  if (chunk_fwd_onepass_ns(variant, bf16, dk, dv, chunk, window, a.B * a.H) == 0) return hipErrorInvalidValue;
  if (window > 1) return launch_chunk_fwd_onepass_win(variant, bf16, dk, chunk, window, a, st);
  return dispatch_split(one_pair(variant), bf16, dk, chunk, [&](auto v, auto *t, auto dd, auto cc) -> hipError_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return launch_onepass<decltype(v)::value, IT, decltype(dd)::value, decltype(cc)::value, 1>(a, st);
  });
}

}  // namespace falcon
